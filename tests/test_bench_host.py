"""Host checks of bench.py's measurement bookkeeping (no GPU): the algorithmic
byte counts behind its roofline figures, and the kernel-source hash that
decides whether a committed counter summary still describes the kernels."""
import bench


def test_step_bytes_per_format():
    """Read hi, lo, grad, m, v and write hi, lo, m, v: 18 B per element, plus
    two scales read and written (16 B) per 256-block, a partial block counted
    whole; the storage formats change only their own streams."""
    import precision_state_amd as ps   # here, not at collection: only when the test runs
    assert bench.step_bytes(256) == 18 * 256 + 16
    assert bench.step_bytes(257) == 18 * 257 + 2 * 16
    assert bench.step_bytes(256, 0, residual=False) == 14 * 256 + 16          # stochastic rounding
    assert bench.step_bytes(100, ps.TENSOR_FP32_MOMENTS) == (8 + 2 + 16) * 100  # m, v fp32 read + written
    assert bench.step_bytes(100, ps.TENSOR_F24_MOMENTS) == (8 + 2 + 12) * 100   # 3 B each way per moment
    assert bench.step_bytes(100, ps.TENSOR_FP32_PARAM | ps.TENSOR_FP32_MOMENTS) == (8 + 4 + 16) * 100


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* a block\n comment */ }\n"
    b = "int f(int x) {\n\n  return 2 * x;   }  // other words\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("2 * x", "3 * x"))


def test_counter_summary_follows_the_code_not_its_comments(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k(float* p) { p[0] = 1.0f; }  // v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash(["k.hip"])
    (tmp_path / "profiles" / "s.txt").write_text(
        f"# a header line: ignored\nhbm_bytes_per_step: 123\nkernel_source_sha256: {h}\n")
    assert bench.read_counter_summary("s.txt", "hbm_bytes_per_step", ["k.hip"]) == 123.0
    src.write_text("/* the same kernel, commented */\n__global__ void k(float* p) {\n  p[0] = 1.0f;\n}\n")
    assert bench.read_counter_summary("s.txt", "hbm_bytes_per_step", ["k.hip"]) == 123.0
    src.write_text("__global__ void k(float* p) { p[0] = 2.0f; }\n")
    assert bench.read_counter_summary("s.txt", "hbm_bytes_per_step", ["k.hip"]) is None
    assert bench.read_counter_summary("missing.txt", "hbm_bytes_per_step", ["k.hip"]) is None
