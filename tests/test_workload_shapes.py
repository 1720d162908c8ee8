"""The synthetic FLUX-12B tensor set that stands in for the model (shapes
only, no weights) against the sizes the pages state: the block counts and the
~12B total of the TorchTitan FLUX post, and the share of small tensors that
the storage policy of sd-scripts PR #2187 keeps in fp32."""
import synth
from figures import page_figure


def test_flux_set_has_the_stated_blocks_and_size():
    fig = page_figure("flux_model_size")
    shapes = synth.WORKLOADS["flux_dev_12b"]()
    blocks = {kind: {s.name.split(".")[1] for s in shapes if s.name.startswith(kind + ".")}
              for kind in ("double_blocks", "single_blocks")}
    assert len(blocks["double_blocks"]) == fig["double_blocks"]
    assert len(blocks["single_blocks"]) == fig["single_blocks"]
    total = synth.total_params(shapes)
    assert total == 11_901_408_320
    assert abs(total / fig["approx_params"] - 1) < fig["relative_tolerance"]


def test_small_tensor_share_matches_the_policy_statement():
    fig = page_figure("small_tensor_share")
    shapes = synth.WORKLOADS["flux_dev_12b"]()
    small = sum(1 for s in shapes if s.numel <= fig["max_elements"])
    lo, hi = fig["accepted_range"]
    assert small == 275 and len(shapes) == 780
    assert lo <= small / len(shapes) <= hi


def test_double_block_set_is_one_double_block():
    one = synth.WORKLOADS["flux_double_block"]()
    full = synth.WORKLOADS["flux_dev_12b"]()
    first = [s for s in full if s.name.startswith("double_blocks.0.")]
    assert sorted(s.numel for s in one) == sorted(s.numel for s in first)
    assert synth.total_params(one) == 339_831_296
