"""Parameter-set shapes and input recipes for the synthetic workloads.

Shapes follow the public FLUX.1 transformer layout named on the TorchTitan
FLUX forum post ("FLUX is Here: Experience Diffusion Model Training on
TorchTitan", FSDP section: 19 + 38 transformer blocks, hidden 3072) with the
~12B total given there; the block counts are read as 19 double-stream and 38
single-stream blocks, the only assignment that gives ~12B parameters. Linear
weights are stored [out_features, in_features], row-major.

No optimizer arithmetic lives here.
"""
from dataclasses import dataclass

H = 3072          # hidden size
MLP = 4 * H       # 12288
HEAD = 128        # per-head q/k RMSNorm width

# synthetic stream ids (see synth.h): weights, residual bits, gradients
STREAM_HI = 0
STREAM_LO = 1
STREAM_GRAD = 2

SIGMA_W = 0.02
SIGMA_G = 1e-3


@dataclass(frozen=True)
class Shape:
    name: str
    rows: int      # 0 for 1-D tensors
    cols: int      # 0 for 1-D tensors
    numel: int

    @property
    def is_2d(self):
        return self.rows > 0


def _lin(name, out_f, in_f, bias=True):
    out = [Shape(name + ".weight", out_f, in_f, out_f * in_f)]
    if bias:
        out.append(Shape(name + ".bias", 0, 0, out_f))
    return out


def _vec(name, n):
    return [Shape(name, 0, 0, n)]


def double_block(prefix="double"):
    """One double-stream block: image and text streams, 24 tensors."""
    t = []
    for s in ("img", "txt"):
        p = f"{prefix}.{s}"
        t += _lin(p + "_mod.lin", 6 * H, H)
        t += _lin(p + "_attn.qkv", 3 * H, H)
        t += _vec(p + "_attn.norm.query_norm.scale", HEAD)
        t += _vec(p + "_attn.norm.key_norm.scale", HEAD)
        t += _lin(p + "_attn.proj", H, H)
        t += _lin(p + "_mlp.0", MLP, H)
        t += _lin(p + "_mlp.2", H, MLP)
    return t


def single_block(prefix="single"):
    """One single-stream block: fused qkv+mlp in, fused attn+mlp out, 8 tensors."""
    t = []
    t += _lin(prefix + ".linear1", 3 * H + MLP, H)
    t += _lin(prefix + ".linear2", H, H + MLP)
    t += _vec(prefix + ".norm.query_norm.scale", HEAD)
    t += _vec(prefix + ".norm.key_norm.scale", HEAD)
    t += _lin(prefix + ".modulation.lin", 3 * H, H)
    return t


def embedders_and_final():
    t = []
    t += _lin("img_in", H, 64)
    t += _lin("time_in.in_layer", H, 256)
    t += _lin("time_in.out_layer", H, H)
    t += _lin("vector_in.in_layer", H, 768)
    t += _lin("vector_in.out_layer", H, H)
    t += _lin("guidance_in.in_layer", H, 256)
    t += _lin("guidance_in.out_layer", H, H)
    t += _lin("txt_in", H, 4096)
    t += _lin("final_layer.adaLN_modulation.1", 2 * H, H)
    t += _lin("final_layer.linear", 64, H)
    return t


def single_tensor_1024x3072():
    """A single [1024, 3072] weight (3,145,728 parameters)."""
    return [Shape("w", 1024, 3072, 1024 * 3072)]


def flux_double_block_set():
    """One FLUX double-stream block's parameters (339,831,296)."""
    return double_block("double_blocks.0")


def flux_dev_set():
    """The full FLUX-dev-shaped parameter set (11,901,408,320 parameters, 780 tensors)."""
    t = embedders_and_final()
    for i in range(19):
        t += double_block(f"double_blocks.{i}")
    for i in range(38):
        t += single_block(f"single_blocks.{i}")
    return t


WORKLOADS = {
    "single_1024x3072": single_tensor_1024x3072,
    "flux_double_block": flux_double_block_set,
    "flux_dev_12b": flux_dev_set,
}


def total_params(shapes):
    return sum(s.numel for s in shapes)
