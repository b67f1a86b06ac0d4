"""bench.py reports stored HBM traffic counters only while the prefill sources match the ones
they were measured on: comments and whitespace may change, code may not. CPU only."""
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
    for f in ("prefill.hip", "common.hpp"):
        shutil.copy(os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc", f), d / f)
    return d


def test_digest_ignores_comments_and_sees_code(tmp_path, monkeypatch):
    d = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_digest()
    src = (d / "prefill.hip").read_text()
    (d / "prefill.hip").write_text("// a new comment line\n" + src.replace("\n", "\n   ", 3) + "\n/* trailing\n block */\n")
    assert bench.kernel_source_digest() == base
    (d / "prefill.hip").write_text(src.replace("constexpr int CH = 64;", "constexpr int CH = 32;"))
    assert bench.kernel_source_digest() != base
