"""The work counts behind every throughput the bench reports (no GPU).

bench.py turns times into TFLOP/s with 4·d·hq × (visible query-key pairs),
counted per step with a binary search over each shard's key positions, and
into GB/s with the decode partial's visible tokens and the merge's byte
formula. These tests build small workloads on the CPU (the library's own
partition and placement calls) and check those counts against the oracle's
one-query-at-a-time count and against closed forms.
"""
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def env():
    import context_partial_attention_amd as cpa

    if not os.path.exists(cpa.library_path()):
        pytest.fail("libcpattn.so is not built (python -m context_partial_attention_amd.build)")
    cpa.load_library()
    import bench
    from context_partial_attention_amd import harness
    from context_partial_attention_amd import workloads as wl

    return bench, harness, wl


PASS_KV = [
    ("cp2_r0", dict(lengths=(300, 517, 1000), batch=3, len_range=(), cp=2, rank=0)),
    ("cp4_r1", dict(lengths=(777, 64, 2), batch=3, len_range=(), cp=4, rank=1)),
    ("cp8_r5_tiny", dict(lengths=(3, 0, 17, 250, 1), batch=5, len_range=(), cp=8, rank=5)),
]


@pytest.mark.parametrize("name,changes", PASS_KV, ids=[p[0] for p in PASS_KV])
def test_pass_kv_pair_counts(env, name, changes):
    bench, harness, wl = env
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, hq=2, hkv=1, d=64, **changes)
    inp = harness.build(w, device="cpu")
    qp, cu = inp["q_positions_host"], inp["cu_q_host"]
    total = 0
    for i, st in enumerate(inp["steps"]):
        want = oracle.visible_pairs(qp, cu, st["k_positions_host"], st["cu_k_host"])
        assert bench.pass_kv_pairs(inp, i) == want
        total += want
    # the cp shards partition every sequence's keys, so the steps together see
    # exactly the causal pairs of the rank's queries against the whole sequence
    full = [np.arange(L) for L in inp["lens"]]
    cu_full = np.concatenate([[0], np.cumsum([len(f) for f in full])])
    assert total == oracle.visible_pairs(qp, cu, np.concatenate(full) if full else np.zeros(0, int), cu_full)


def test_pass_kv_pairs_closed_form(env):
    # one sequence with 2cp | L: every rank's steps together see L(L+1)/(2cp) pairs
    bench, harness, wl = env
    L, cp = 1024, 4
    for r in range(cp):
        w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name="cf", lengths=(L,), batch=1, len_range=(),
                      cp=cp, rank=r, hq=2, hkv=1, d=64)
        inp = harness.build(w, device="cpu")
        assert sum(bench.pass_kv_pairs(inp, i) for i in range(cp)) == L * (L + 1) // (2 * cp)


PAGED = [
    ("passq_cp4", dict(kind="pass_q", batch=2, cached=1000, new=300, cp=4, rank=0, interleave=8)),
    ("passq_cp3_il5", dict(kind="pass_q", batch=3, cached=513, new=130, cp=3, rank=0, interleave=5)),
    ("decode_cp2", dict(kind="decode", batch=16, len_range=(1, 3000), lengths=(), cp=2, rank=0, interleave=8)),
]


@pytest.mark.parametrize("name,changes", PAGED, ids=[p[0] for p in PAGED])
def test_paged_pair_counts(env, name, changes):
    bench, harness, wl = env
    base = "allgather_decode_cp2" if changes["kind"] == "decode" else "chunked_prefill_passq_cp4"
    w = wl.scaled(wl.WORKLOADS[base], name=name, hq=2, hkv=1, d=64, **changes)
    inp = harness.build(w, device="cpu")
    qp, cu = inp["q_positions_host"], inp["cu_q_host"]
    total = 0
    for r, rk in enumerate(inp["ranks"]):
        want = oracle.visible_pairs(qp, cu, rk["local_to_global_host"], rk["cu_local_host"])
        assert bench.paged_pairs(inp, r) == want
        total += want
    # round-robin placement deals every cached and new token to exactly one rank
    lens = inp["lens"]
    full = np.concatenate([np.arange(L) for L in lens])
    cu_full = np.concatenate([[0], np.cumsum(lens)])
    assert total == oracle.visible_pairs(qp, cu, full, cu_full)
    if w.kind == "decode":
        # one query at L - 1 per sequence: its pairs are the rank's local tokens
        r0 = inp["ranks"][w.rank]
        assert bench.paged_pairs(inp, w.rank) == int(np.sum(r0["local_lens_host"]))


def test_merge_bytes_formula(env):
    bench, _, wl = env
    w = wl.WORKLOADS["qwen2.5_3b_cp2_rank0"]
    rows, parts = 1000 * w.hq, 2
    # each part: fp32 O (4 d bytes) and one fp32 LSE per row; out: bf16 O and fp32 LSE
    assert bench.merge_bytes(w, rows, parts, 2) == parts * rows * (4 * w.d + 4) + rows * (2 * w.d + 4)


def test_source_digest_ignores_comments_only(env):
    """The counter summaries stay valid across comment edits of the kernel
    source, and go stale on any code change."""
    bench = env[0]
    src = "int a; // one\n/* two\n three */ int b;\n\n  // four\nint c;  \n"
    assert bench._code_only(src) == "int a;\n int b;\nint c;"
    assert bench._code_only(src.replace("// one", "// ONE")) == bench._code_only(src)
    assert bench._code_only(src.replace("int c;", "int c = 1;")) != bench._code_only(src)
