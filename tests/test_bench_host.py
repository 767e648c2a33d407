"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _reader(edit=None):
    def read(f):
        t = open(os.path.join(ROOT, "sparse_moe_transformer_gemm_amd", "csrc", f)).read()
        return edit(f, t) if edit else t
    return read


def test_traffic_hash_ignores_comments_not_code():
    base = bench.traffic_sources_hash(_reader())
    assert base == bench.traffic_sources_hash()
    # comments and white space only: same hash
    commented = bench.traffic_sources_hash(
        _reader(lambda f, t: t.replace("\n", "  // note\n", 3) + "\n/* block\n comment */\n" if f == "ffn.hip" else t))
    assert commented == base
    # a changed constant: another hash
    changed = bench.traffic_sources_hash(
        _reader(lambda f, t: t.replace("kPrefWaves = 8", "kPrefWaves = 4") if f == "ffn.hip" else t))
    assert changed != base

