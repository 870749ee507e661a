"""Host-side logic of bench.py: the metric's FLOP count, the algorithmic
bytes behind the roofline figure, and the lookup of committed HBM traffic.

The expected FLOP and byte counts are the per-configuration figures of the
scope table, computed there from the shapes alone (4 B H N^2 d, halved when
causal; Q, K, V, O at 2 bytes per element and an fp32 LSE per row; K and V
rows past a sequence's valid length not counted), so a slip in bench.py's
formulas (a missing factor, a dropped LSE term, counting padded keys) fails
here rather than in a number nobody re-derives.
"""
import os

import numpy as np
import pytest

import attn_inputs as ai
import bench

METRIC_FLOPS = {
    "single_head": 524_288,
    "reranker": 5_033_164_800,
    "prefill": 137_438_953_472,
    "peaky": 137_438_953_472,
    "long_context": 8_796_093_022_208,
}

ALGORITHMIC_BYTES = {
    "single_head": 16_640,
    "prefill": 134_742_016,
    "peaky": 135_266_304,
    "long_context": 1_077_936_128,
}


@pytest.mark.parametrize("name", sorted(METRIC_FLOPS))
def test_metric_flops(name):
    assert bench.metric_flops(ai.WORKLOADS[name]) == METRIC_FLOPS[name]


@pytest.mark.parametrize("name", sorted(ALGORITHMIC_BYTES))
def test_algorithmic_bytes_dense(name):
    assert bench.algorithmic_bytes(ai.WORKLOADS[name]) == ALGORITHMIC_BYTES[name]


def test_algorithmic_bytes_reranker_counts_valid_keys_only():
    w = ai.WORKLOADS["reranker"]
    kl = ai.generate(w)["key_len"]
    # Q, O and LSE of every row, plus K and V of the valid rows of 12 heads
    assert bench.algorithmic_bytes(w, kl) == 20_275_200 + 1_536 * int(np.sum(kl))
    # all keys valid: the dense figure
    assert bench.algorithmic_bytes(w, None) == 20_275_200 + 1_536 * 50 * 256


@pytest.mark.parametrize("name,f_alg", [("prefill", 137_472_507_904), ("long_context", 8_796_361_457_664)])
def test_causal_visible_pairs_include_the_diagonal(name, f_alg):
    w = ai.WORKLOADS[name]
    assert 4 * w.d * bench.visible_pairs(w) == f_alg


def test_visible_per_query_end_aligned_causal():
    # 3 query rows against 5 keys: the last row sees all 5, the first 3
    w = ai.Workload("t", 1, 1, 5, 32, ai.F16, True, False, Nq=3, seed=1)
    assert bench.visible_per_query(w, 5).tolist() == [3, 4, 5]
    assert bench.visible_per_query(w, 4).tolist() == [3, 4, 4]
    # more query rows than keys: the first rows see nothing
    w2 = ai.Workload("t", 1, 1, 2, 32, ai.F16, True, False, Nq=4, seed=1)
    assert bench.visible_per_query(w2, 2).tolist() == [0, 0, 1, 2]


def test_read_traffic_needs_the_current_source_digest(tmp_path, monkeypatch):
    digest = bench.source_digest()
    assert len(digest) == 16 and int(digest, 16) >= 0
    f = tmp_path / "traffic.txt"
    f.write_text(
        "header line\n"
        f"traffic kernel=k_a workload=w_a source_sha256_16={digest} hbm_bytes_per_launch=1234 read_bytes=1000 write_bytes=234\n"
        "traffic kernel=k_b workload=w_b source_sha256_16=0000000000000000 hbm_bytes_per_launch=99 read_bytes=9 write_bytes=90\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("k_a", "w_a") == 1234
    assert bench.read_traffic("k_a", "w_b") is None       # other workload
    assert bench.read_traffic("k_b", "w_b") is None       # taken on other sources
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_traffic("k_a", "w_a") is None


def test_code_only_drops_comments_and_keeps_code():
    src = ('#include "a.h"  // the header\n'
           '/* a block\n   over lines */\n'
           'int x = 1;   \n'
           '\n'
           'const char *s = "// kept /* too */";  // gone\n'
           "char c = '/'; int y = 2 / 3; /* inline */ int z;\n")
    assert bench.code_only(src) == ('#include "a.h"\n'
                                    'int x = 1;\n'
                                    'const char *s = "// kept /* too */";\n'
                                    "char c = '/'; int y = 2 / 3;  int z;")
    # a comment alone does not change the code, an edit of the code does
    assert bench.code_only(src.replace("// the header", "// another")) == bench.code_only(src)
    assert bench.code_only(src.replace("x = 1", "x = 2")) != bench.code_only(src)


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int f() { return 1; }  // one\n")
    b.write_text("/* two */ int g;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a), str(b)])
    d0 = bench.source_digest()
    a.write_text("// a note\nint f() { return 1; }\n")
    assert bench.source_digest() == d0
    a.write_text("int f() { return 2; }\n")
    assert bench.source_digest() != d0


def test_kernel_sources_exist():
    import re
    for path in bench.KERNEL_SOURCES:
        assert os.path.exists(path), path
        # code_only reads ' and " as literal delimiters: digit separators
        # and raw strings would confuse it
        text = open(path, encoding="utf-8").read()
        assert not re.search(r"[0-9]'[0-9]", text) and 'R"(' not in text, path


def test_input_sets_evict_the_caches_within_bounds():
    # enough copies that the others move more than the eviction target
    # between two uses of one copy; at least 16 for small sets, at most 4096
    big = 200 << 20
    n = bench.input_sets(big)
    assert (n - 1) * big >= bench.ROTATE_EVICT_BYTES and n >= 2
    assert bench.input_sets(32 << 20) == max(bench.ROTATE_MIN_SETS_SMALL,
                                            1 + bench.ROTATE_EVICT_BYTES // (32 << 20))
    assert bench.input_sets(1 << 20) == 513          # 512 MiB of other copies
    assert bench.input_sets(16 << 10) == bench.ROTATE_MAX_SETS
    assert bench.input_sets(1) == bench.ROTATE_MAX_SETS
    assert bench.input_sets(4 << 30) == 2
