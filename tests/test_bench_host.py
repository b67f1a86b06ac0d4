"""Host-side logic of bench.py, CPU only: the roofline arithmetic against the per-unit figures
derived by hand for the measured workloads, and the source digest that keeps stored HBM
traffic counters tied to the code they were measured on."""
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _tree(tmp_path):
    d = tmp_path / "delta_rule_linear_chunked_amd" / "csrc"
    d.mkdir(parents=True)
    for f in bench.PREFILL_SOURCES:
        shutil.copy(os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc", f), d / f)
    return d


def test_digest_ignores_comments_and_sees_code(tmp_path, monkeypatch):
    d = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_digest()
    src = (d / "prefill.hip").read_text()
    assert "constexpr int LDT = 68;" in src
    (d / "prefill.hip").write_text("// a new comment line\n" + src.replace("\n", "\n   ", 3) + "\n/* trailing\n block */\n")
    assert bench.kernel_source_digest() == base
    (d / "prefill.hip").write_text(src.replace("constexpr int LDT = 68;", "constexpr int LDT = 72;"))
    assert bench.kernel_source_digest() != base


def test_prefill_roofline_arithmetic():
    # KDA, bf16 q/k/v, d = 128: (2 d_k + d_v) * 2 + 4 d_k (alpha) + 4 (beta) + 4 d_v (o) bytes
    # per token-head, plus S0 and S_T; the useful work of the chunked form at C = 64 is
    # 140,438 FLOP per token-head (triangular A, P, T, W, U counts, the three state products
    # and P delta)
    B, T, H, D = 4, 4096, 16, 128
    nbytes, flops = bench.prefill_work(B, T, H, D, D)
    assert (2 * D + D) * 2 + 4 * D + 4 + 4 * D == 1796
    assert nbytes == B * T * H * 1796 + 2 * B * H * D * D * 4 == 479_199_232
    assert flops == B * T * H * 140_438
    # bf16 decay pre-activations (the fused preparation's input) halve alpha's bytes
    assert bench.prefill_work(B, T, H, D, D, alpha_bytes=2)[0] == nbytes - B * T * H * 2 * D


def test_decode_roofline_arithmetic():
    # per head-step: the fp32 state read and written (8 d_k d_v bytes) plus the token's q, k, v
    # (bf16), alpha (fp32), beta and o (fp32): 132,868 bytes at d = 128; 512 x 32 heads per step
    per_head = 8 * 128 * 128 + (2 * 128 + 128) * 2 + 4 * 128 + 4 + 4 * 128
    assert per_head == 132_868
    assert bench.decode_bytes(512, 32, 128, 128) == 512 * 32 * per_head == 2_176_909_312


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr, (r.returncode, r.stderr)
    assert r.stdout == ""  # no JSON line
