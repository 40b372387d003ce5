"""GPU parity: every entry point of libcpattn.so against the fp64 CPU oracle.

Small cases compare every output element. The full-size workloads run in the
launch configuration the benchmark times, into outputs filled with NaN first;
every row is checked for properties that hold at any size, and the oracle is
compared with every element (Qwen2.5-3B-shaped prefill, decode) or with
sampled rows (128K prefill, chunked prefill). The bar:
max |dO| <= 2e-2 and max |dLSE| <= 1e-3 for bf16 inputs with fp32
accumulation, rows with no visible key exactly (O = 0, LSE = -inf), no NaN.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from parity_util import (assert_close, expected_pass_kv, expected_round_robin, f64, sample_rows)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def cpa(gpu):
    import context_partial_attention_amd as cpa

    cpa.load_library()
    return cpa


@pytest.fixture(scope="module")
def wl():
    from context_partial_attention_amd import workloads

    return workloads


@pytest.fixture(scope="module")
def harness():
    from context_partial_attention_amd import harness

    return harness


def _check_schedule(harness, w, rows=None, pool_fill=0.0, seed=0):
    """Runs a workload's whole schedule on the GPU and compares every partial
    and the merge with the oracle on `rows` (all rows when None)."""
    inp = harness.build(w, device="cuda", pool_fill=pool_fill)
    run = harness.Runner(inp)
    run.step()
    torch.cuda.synchronize()
    if w.kind == "pass_kv":
        rows_, parts, merged = expected_pass_kv(inp, rows)
    else:
        rows_, parts, merged = expected_round_robin(inp, rows)
    ridx = torch.as_tensor(rows_, device="cuda")
    errs = []
    for s, (o_ref, l_ref) in enumerate(parts):
        errs.append(assert_close(f64(run.o_parts[s][ridx]), f64(run.lse_parts[s][ridx]), o_ref, l_ref,
                                 f"{w.name} partial {s}"))
    errs.append(assert_close(f64(run.o[ridx]), f64(run.lse[ridx]), merged[0], merged[1], f"{w.name} merged"))
    return inp, run, errs


# ----------------------------------------------------------------- tiny fp32 workload, every element


def test_tiny_prefill_cp2_fp32_all_elements(cpa, wl, harness):
    w = wl.WORKLOADS["tiny_prefill_cp2"]
    _say(f"case {w.name}")
    inp, run, errs = _check_schedule(harness, w)
    # fp32 inputs: the merged result must also equal full causal attention of the sequence
    q = f64(inp["draws"][0][0])
    k = f64(inp["draws"][0][1])
    v = f64(inp["draws"][0][2])
    fo, fl = oracle.full_causal_attn(q, k, v, w.scale, rows=inp["q_positions_host"])
    assert_close(f64(run.o), f64(run.lse), fo, fl, "tiny merged vs full attention", o_tol=1e-4, lse_tol=1e-5)
    # chunk-0 queries see nothing of rank 1's shard in step 2
    assert np.all(np.isneginf(f64(run.lse_parts[1])[:64]))


# ----------------------------------------------------------------- small bf16 variants, every element


SMALL = [
    # name, kind, changes
    ("passkv_ragged_cp2_r0", dict(kind="pass_kv", lengths=(300, 517, 1000), batch=3, len_range=(), cp=2, rank=0)),
    ("passkv_ragged_cp2_r1", dict(kind="pass_kv", lengths=(300, 517, 1000), batch=3, len_range=(), cp=2, rank=1)),
    ("passkv_cp4_r3_d64_g1", dict(kind="pass_kv", lengths=(777,), batch=1, len_range=(), cp=4, rank=3, hq=4, hkv=4,
                                  d=64)),
    ("passkv_tiny_chunks", dict(kind="pass_kv", lengths=(3, 1, 0, 9, 130), batch=5, len_range=(), cp=4, rank=2)),
    ("passq_cp4_small", dict(kind="pass_q", batch=2, cached=1000, new=300, cp=4, rank=0, interleave=8)),
    ("passq_cp3_il5_d64", dict(kind="pass_q", batch=3, cached=513, new=130, cp=3, rank=0, interleave=5, d=64,
                               hq=8, hkv=1)),
    # a local shard of 75000 keys (4688 blocks): a long block table, read one entry per wave and tile
    ("passq_long_cache", dict(kind="pass_q", batch=1, cached=150000, new=70, cp=2, rank=1,
                                           interleave=8, hq=4, hkv=2, d=64)),
    # odd GQA group: the paged prefill runs on the one-head-per-workgroup kernel
    ("passq_cp2_g3", dict(kind="pass_q", batch=2, cached=700, new=150, cp=2, rank=1, interleave=4, hq=6, hkv=2)),
    ("decode_cp2_small", dict(kind="decode", batch=16, len_range=(1, 3000), lengths=(), cp=2, rank=0,
                              interleave=8)),
    ("decode_cp4_d64_g8", dict(kind="decode", batch=9, len_range=(1, 700), lengths=(), cp=4, rank=0, interleave=3,
                               d=64, hq=16, hkv=2)),
    # enough sequences for the decode kernel's longer splits (2048 and 1024 local tokens; the split
    # size is checked through the workspace size), several splits per sequence with ragged ends
    ("decode_512seqs_split2048", dict(kind="decode", batch=512, len_range=(1, 6000), lengths=(), cp=2, rank=1,
                                      interleave=8)),
    ("decode_400seqs_split1024", dict(kind="decode", batch=400, len_range=(1, 6000), lengths=(), cp=2, rank=0,
                                      interleave=8, hq=8, hkv=2)),
    # no context parallelism (cp = 1): the rank holds every token, one step, nothing to merge with
    ("passkv_cp1_whole", dict(kind="pass_kv", lengths=(700, 130, 1), batch=3, len_range=(), cp=1, rank=0)),
    ("passq_cp1_whole", dict(kind="pass_q", batch=2, cached=500, new=200, cp=1, rank=0, interleave=8)),
    ("decode_cp1_whole", dict(kind="decode", batch=8, len_range=(1, 2000), lengths=(), cp=1, rank=0, interleave=8)),
    # one 200K-token context and a short one: 196 splits of 512 local tokens for the long one
    ("decode_long_200k_split512", dict(kind="decode", batch=2, lengths=(200000, 37), len_range=(), cp=2, rank=1,
                                       interleave=8)),
]


@pytest.mark.parametrize("name,changes", SMALL, ids=[s[0] for s in SMALL])
def test_small_bf16_all_elements(cpa, wl, harness, name, changes):
    base = {"pass_kv": "qwen2.5_3b_cp2_rank0", "pass_q": "chunked_prefill_passq_cp4",
            "decode": "allgather_decode_cp2"}[changes["kind"]]
    w = wl.scaled(wl.WORKLOADS[base], name=name, seed=100 + len(name), **changes)
    _say(f"case {name}")
    # NaN in every unused cache slot: any read of one would show up in the results
    inp, _, _ = _check_schedule(harness, w, pool_fill=float("nan"))
    if "_split" in name:
        split = int(name.rsplit("split", 1)[1])
        max_blocks = inp["ranks"][w.rank]["block_table"].shape[1]
        need = cpa.partial_attn_paged_workspace(w.batch, 1, max_blocks, 16, w.hq, w.d)
        n_splits = need // (w.batch * w.hq * (w.d + 1) * 4)
        assert max_blocks * 16 > split and n_splits == -(-max_blocks * 16 // split), (max_blocks, n_splits)


FOLD_CASES = [
    # sequences shorter than one interleave group: the other rank has no key for them (LSE -inf)
    ("decode_fold_cp2_short", dict(kind="decode", batch=7, lengths=(1, 5, 8, 9, 17, 100, 3000), len_range=(), cp=2,
                                   rank=0, interleave=8)),
    ("decode_fold_cp4_d64_g8", dict(kind="decode", batch=9, len_range=(1, 700), lengths=(), cp=4, rank=2,
                                    interleave=3, d=64, hq=16, hkv=2)),
    # pass-Q: a 3-token cache, so the first new queries see keys on rank 0 only
    ("passq_fold_cp4_short", dict(kind="pass_q", batch=2, cached=3, new=140, cp=4, rank=0, interleave=8)),
    ("passq_fold_cp3_il5_d64", dict(kind="pass_q", batch=3, cached=513, new=130, cp=3, rank=1, interleave=5, d=64,
                                    hq=8, hkv=1)),
]


@pytest.mark.parametrize("name,changes", FOLD_CASES, ids=[c[0] for c in FOLD_CASES])
def test_rank_fold_all_elements(cpa, wl, harness, name, changes):
    """The other ranks' partials folded into the rank's own paged launches
    (decode: its merge kernel; pass-Q: the prefill epilogue): every element
    against the oracle's merge of all ranks, within 1e-5 of the separate merge
    of the same partials, the rank's own partial bit-identical to the plain
    call, received rows with LSE -inf never read (their O is NaN), bf16 parts,
    no parts at all, and the most parts the call takes."""
    base = "allgather_decode_cp2" if changes["kind"] == "decode" else "chunked_prefill_passq_cp4"
    w = wl.scaled(wl.WORKLOADS[base], name=name, seed=300 + len(name), **changes)
    _say(f"case {name}")
    nan = float("nan")
    inp = harness.build(w, device="cuda", pool_fill=nan)
    run = harness.Runner(inp, merged_dtype=torch.float32)
    run.poison()
    r = w.rank
    others = [i for i in range(w.cp) if i != r]
    for i in range(w.cp):
        run.partial(i)
    run.merge()
    torch.cuda.synchronize()
    sep_o, sep_l = run.o.clone(), run.lse.clone()
    own_o, own_l = run.o_parts[r].clone(), run.lse_parts[r].clone()
    _, parts, merged = expected_round_robin(inp, None)
    n_empty = 0
    for i in others:
        empty = torch.isneginf(run.lse_parts[i])
        n_empty += int(empty.sum())
        run.o_parts[i][empty] = nan
    if name.endswith("short"):
        assert n_empty > 0
    for t in (run.o, run.lse, run.o_parts[r], run.lse_parts[r]):
        t.fill_(nan)
    run.rank_fold()
    torch.cuda.synchronize()
    assert torch.equal(run.o_parts[r], own_o) and torch.equal(run.lse_parts[r], own_l)
    e = assert_close(f64(run.o), f64(run.lse), merged[0], merged[1], f"{name} folded")
    _say(f"  folded: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")
    np.testing.assert_allclose(f64(run.o), f64(sep_o), rtol=0, atol=1e-5)
    np.testing.assert_allclose(f64(run.lse), f64(sep_l), rtol=0, atol=1e-5)

    # parts received in bf16, result in bf16
    rk = inp["ranks"][r]
    args = (inp["q"], inp["q_pos"], inp["cu_q"], rk["k_cache"], rk["v_cache"], rk["block_table"],
            rk["local_kv_lens"], w.cp, r, w.interleave, inp["max_q"], w.scale)
    bparts = [run.o_parts[i].bfloat16() for i in others]
    own_b = torch.full_like(bparts[0], nan)
    ob, lb = cpa.partial_attn_paged_merged(*args, bparts, [run.lse_parts[i] for i in others],
                                           out_dtype=torch.bfloat16, own_out=own_b)
    torch.cuda.synchronize()
    assert torch.equal(own_b, own_o.bfloat16())
    # (the received rows holding NaN have LSE -inf, hence weight 0: zeros stand in for them)
    ref_o, ref_l = oracle.lse_merge([f64(own_o)] + [np.nan_to_num(f64(b), nan=0.0) for b in bparts],
                                    [f64(own_l)] + [f64(run.lse_parts[i]) for i in others])
    assert_close(f64(ob), f64(lb), ref_o, ref_l, f"{name} bf16 parts")

    # no received parts: the plain decode call's result, bit for bit
    o0, l0 = cpa.partial_attn_paged_merged(*args, [], [])
    torch.cuda.synchronize()
    assert torch.equal(o0, own_o) and torch.equal(l0, own_l)

    # the most parts the call takes (15): random partials beside the received ones, some rows empty
    g = torch.Generator(device="cuda").manual_seed(17)
    extra = 15 - len(others)
    xo = [torch.randn(own_o.shape, device="cuda", generator=g) for _ in range(extra)]
    xl = [torch.randn(own_l.shape, device="cuda", generator=g) * 4 for _ in range(extra)]
    for t in xl:
        t[torch.rand(t.shape, device="cuda", generator=g) < 0.2] = float("-inf")
    po = [run.o_parts[i] for i in others] + xo
    pl = [run.lse_parts[i] for i in others] + xl
    om, lm = cpa.partial_attn_paged_merged(*args, po, pl)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge([f64(own_o)] + [np.nan_to_num(f64(t), nan=0.0) for t in po],
                                    [f64(own_l)] + [f64(t) for t in pl])
    assert_close(f64(om), f64(lm), ref_o, ref_l, f"{name} 15 parts")


def test_rank_fold_odd_group_prefill_unsupported(cpa, wl, harness):
    """Pass-Q prefill with an odd GQA group runs on the one-head kernel, which
    has no fold: refused (compute the partial and merge instead)."""
    w = wl.scaled(wl.WORKLOADS["chunked_prefill_passq_cp4"], name="fold_g3", batch=1, cached=100, new=40, cp=2,
                  rank=0, interleave=4, hq=6, hkv=2)
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    with pytest.raises(cpa.CpaError) as err:
        run.rank_fold()
    assert err.value.status == -2


def test_small_bf16_output_and_no_mask(cpa, wl, harness):
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name="nomask", lengths=(400, 129), batch=2, len_range=())
    _say("case bf16 output + no mask")
    inp = harness.build(w, device="cuda")
    st = inp["steps"][1]
    o, l = cpa.partial_attn(inp["q"], inp["q_pos"], inp["cu_q"], st["k"], st["v"], st["k_pos"], st["cu_k"],
                            inp["max_q"], w.scale, causal=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    mine = oracle.zigzag_partition(inp["lens"], w.cp, w.rank)
    src = oracle.zigzag_partition(inp["lens"], w.cp, (w.rank - 1) % w.cp)
    q_all = torch.cat([d[0] for d in inp["draws"]])
    k_all = torch.cat([d[1] for d in inp["draws"]])
    v_all = torch.cat([d[2] for d in inp["draws"]])
    q = f64(q_all[torch.as_tensor(mine["src_index"], device="cuda")])
    k = f64(k_all[torch.as_tensor(src["src_index"], device="cuda")])
    v = f64(v_all[torch.as_tensor(src["src_index"], device="cuda")])
    ro, rl = oracle.partial_attn(q, mine["positions"], mine["cu_seqlens"], k, v, src["positions"],
                                 src["cu_seqlens"], w.scale, causal=False)
    assert_close(f64(o), f64(l), ro, rl, "no-mask bf16-out")
    # the batched call with its launch order (whose entries carry each unit's
    # key-tile count) gives the same bits as the single call without a mask
    ws = torch.empty(cpa.partial_attn_multi_workspace(1, 2, inp["max_q"]), dtype=torch.uint8, device="cuda")
    (om,), (lm,) = cpa.partial_attn_multi(inp["q"], inp["q_pos"], inp["cu_q"], [st["k"]], [st["v"]], [st["k_pos"]],
                                          [st["cu_k"]], inp["max_q"], w.scale, causal=False,
                                          out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(om, o) and torch.equal(lm, l), "no-mask batched launch differs from the single call"


MULTI = [
    ("cp4_r1_ragged", dict(lengths=(300, 517, 1000), batch=3, len_range=(), cp=4, rank=1)),
    ("cp3_r2_d64_g1", dict(lengths=(777, 64), batch=2, len_range=(), cp=3, rank=2, hq=4, hkv=4, d=64)),
    ("cp2_r0_fp32", dict(lengths=(200, 90), batch=2, len_range=(), cp=2, rank=0, dtype=torch.float32)),
    ("cp2_r1_d64_g4", dict(lengths=(600, 129), batch=2, len_range=(), cp=2, rank=1, hq=8, hkv=2, d=64)),
    # eight shards (the most one launch takes), sequences shorter than 2cp: empty chunks and shards
    ("cp8_r5_tiny", dict(lengths=(3, 0, 17, 250, 1), batch=5, len_range=(), cp=8, rank=5)),
    # GQA group of 6: three head pairs per KV head
    ("cp2_r0_g6", dict(lengths=(450, 1200), batch=2, len_range=(), cp=2, rank=0, hq=12, hkv=2)),
]


@pytest.mark.parametrize("name,changes", MULTI, ids=[m[0] for m in MULTI])
def test_multi_shard_launch_equals_separate_calls(cpa, wl, harness, name, changes):
    """Every pass-KV step in one batched launch gives, shard by shard, exactly
    the bits of the separate per-step calls, and both match the oracle."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, seed=300 + len(name), **changes)
    _say(f"case multi {name}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    for i in range(w.cp):
        run.partial(i)
    torch.cuda.synchronize()
    sep = [(o.clone(), l.clone()) for o, l in zip(run.o_parts, run.lse_parts)]
    for ordered in (False, True):  # fixed order, then heaviest-tile-first order
        for o, l in zip(run.o_parts, run.lse_parts):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        run.partials_batched(ordered=ordered)
        torch.cuda.synchronize()
        for s, (o, l) in enumerate(sep):
            assert torch.equal(run.o_parts[s], o), f"{name} shard {s} ordered={ordered}: O differs from separate call"
            assert torch.equal(run.lse_parts[s], l), f"{name} shard {s} ordered={ordered}: LSE differs"
    rows, parts, _ = expected_pass_kv(inp, None)
    tol = dict(o_tol=1e-4, lse_tol=1e-5) if changes.get("dtype") == torch.float32 else {}
    for s, (o_ref, l_ref) in enumerate(parts):
        assert_close(f64(run.o_parts[s]), f64(run.lse_parts[s]), o_ref, l_ref, f"multi {name} shard {s}", **tol)


# many short sequences: 2000 and 2200 (shard, sequence) segments, 6000 and
# 6600 units for the ordering pre-pass; a few sequences of a few thousand
# tokens, a short launch against its heaviest unit (ordered heaviest first);
# two long sequences, a long launch (ordered shard-major)
PREPASS = [
    ("seqs_1000_cp2_r0", dict(batch=1000, len_range=(1, 700), lengths=(), cp=2, rank=0, hq=4, hkv=2, d=64)),
    ("seqs_1100_cp2_r1", dict(batch=1100, len_range=(1, 700), lengths=(), cp=2, rank=1, hq=4, hkv=2, d=64)),
    ("few_heaviest_first_cp2_r0", dict(batch=4, lengths=(2453, 3682, 4327, 6706), len_range=(), cp=2, rank=0)),
    ("long_shard_major_cp2_r1", dict(batch=2, lengths=(100000, 70001), len_range=(), cp=2, rank=1, hq=16, hkv=2,
                                     d=64)),
]


@pytest.mark.parametrize("name,changes", PREPASS, ids=[m[0] for m in PREPASS])
def test_ordering_prepass_segments(cpa, wl, harness, name, changes):
    """The launch order and per-unit key-tile counts from the pre-pass give
    the bits of the separate per-step calls, which search the key positions
    themselves."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, seed=700 + len(name), **changes)
    _say(f"case prepass {name}")
    inp = harness.build(w, device="cuda")
    n_units = -(-inp["max_q"] // 128) * w.batch * w.cp
    assert n_units <= 8192, "the units must fit the pre-pass"
    run = harness.Runner(inp)
    assert run.workspace is not None
    for i in range(w.cp):
        run.partial(i)
    torch.cuda.synchronize()
    sep = [(o.clone(), l.clone()) for o, l in zip(run.o_parts, run.lse_parts)]
    for o, l in zip(run.o_parts, run.lse_parts):
        o.fill_(float("nan"))
        l.fill_(float("nan"))
    run.partials_batched(ordered=True)
    torch.cuda.synchronize()
    for s, (o, l) in enumerate(sep):
        assert torch.equal(run.o_parts[s], o), f"{name} shard {s}: O differs from the separate call"
        assert torch.equal(run.lse_parts[s], l), f"{name} shard {s}: LSE differs from the separate call"
    # the order itself (the workspace starts with one entry per unit: the unit index in the low 13
    # bits, its visible key-tile count above): a permutation of the units, heaviest first (counts
    # from 4095 tiles up rank as equal), or, when each CU's share of the launch's key tiles is at
    # least 12 times the heaviest unit's, shard-major with the heaviest first within each shard
    # (counts from 511 up rank as equal)
    e = run.workspace[: 4 * n_units].view(torch.int32).cpu().numpy().astype(np.int64)
    unit, work = e & 8191, e >> 13
    assert np.array_equal(np.sort(unit), np.arange(n_units))
    shard = unit % w.cp
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    shard_major = int(work.sum()) * w.hkv * (w.hq // w.hkv // 2) >= 12 * int(work.max()) * n_cus
    if name.startswith("long"):
        assert shard_major and work.max() > 511
    if name.startswith("few"):
        assert not shard_major
    if shard_major:
        assert np.all(np.diff(shard) >= 0), "shard-major"
        for sh in range(w.cp):
            assert np.all(np.diff(np.minimum(work[shard == sh], 511)) <= 0), f"shard {sh}: heaviest first"
    else:
        assert np.all(np.diff(np.minimum(work, 4095)) <= 0), "heaviest first"


MERGED = [
    ("cp2_r0_ragged", dict(lengths=(300, 517, 1000), batch=3, len_range=(), cp=2, rank=0)),
    ("cp4_r2_d64_g4", dict(lengths=(777, 64, 2), batch=3, len_range=(), cp=4, rank=2, hq=8, hkv=2, d=64)),
    ("cp8_r3_tiny", dict(lengths=(3, 0, 17, 250, 1), batch=5, len_range=(), cp=8, rank=3)),
]


@pytest.mark.parametrize("name,changes", MERGED, ids=[m[0] for m in MERGED])
def test_merged_walk_all_elements(cpa, wl, harness, name, changes):
    """The one-walk merged result equals the oracle's merge of the step
    partials (every element), and the GPU's partials + merge to rounding."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, seed=500 + len(name), **changes)
    _say(f"case merged {name}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    for out_dtype in (torch.float32, torch.bfloat16):
        o = torch.full_like(run.o, float("nan"), dtype=out_dtype)
        lse = torch.full_like(run.lse, float("nan"))
        run.merged_walk(out=o, lse=lse)
        torch.cuda.synchronize()
        _, _, merged = expected_pass_kv(inp, None)
        assert_close(f64(o), f64(lse), merged[0], merged[1], f"merged walk {name} {out_dtype}")
    run.step()  # partials + separate merge
    torch.cuda.synchronize()
    o32 = torch.empty_like(run.o, dtype=torch.float32)
    l32 = torch.empty_like(run.lse)
    run.merged_walk(out=o32, lse=l32)
    torch.cuda.synchronize()
    assert_close(f64(o32), f64(l32), f64(run.o), f64(run.lse), f"merged walk vs partials + merge {name}")


# full-size workloads whose every output element is compared with the oracle
# (the rest are compared on sampled rows plus properties of every row)
ALL_ROWS = ("qwen2.5_3b_cp2_rank0", "allgather_decode_cp2")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen2.5_3b_cp2_rank0", "llama3_8b_128k_cp4_rank1"])
def test_fused_merge_full_size(cpa, wl, harness, name):
    """The one-walk merge and the running merge at full size, into outputs
    filled with NaN first (so every row must have been written): every row of
    the Qwen2.5-3B-shaped workload, sampled rows of the 128K one."""
    w = wl.WORKLOADS[name]
    _say(f"case merged full-size {name}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    run.poison()
    run.merged_walk()
    torch.cuda.synchronize()
    assert not torch.isnan(run.o).any() and torch.isfinite(run.lse).all()
    vmax = max(float(d[2].float().abs().max()) for d in inp["draws"])
    assert float(run.o.float().abs().max()) <= vmax * (1 + 2 ** -8) + 1e-3
    rows = None if name in ALL_ROWS else sample_rows(inp["cu_q_host"], inp["q_positions_host"], n_random=48,
                                                      seed=w.seed)
    rows_, _, merged = expected_pass_kv(inp, rows)
    ridx = torch.as_tensor(rows_, device="cuda")
    e = assert_close(f64(run.o[ridx]), f64(run.lse[ridx]), merged[0], merged[1], f"{name} merged walk")
    _say(f"  merged walk: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} over {len(rows_)} rows")
    # the same shards folded in one at a time (running merge), bf16 output at the last step
    run.poison()
    run.ring_accumulate()
    torch.cuda.synchronize()
    assert not torch.isnan(run.o).any() and torch.isfinite(run.lse).all()
    e = assert_close(f64(run.o[ridx]), f64(run.lse[ridx]), merged[0], merged[1], f"{name} ring accumulate")
    _say(f"  ring accumulate: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} over {len(rows_)} rows")


def test_merged_walk_without_mask(cpa, wl, harness):
    """No mask: every query sees every key of every shard; the one-walk merge
    equals the oracle's merge of the unmasked partials."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name="merged_nomask", lengths=(333, 700), batch=2,
                  len_range=(), cp=4, rank=1)
    _say("case merged walk, no mask")
    inp = harness.build(w, device="cuda")
    st = inp["steps"]
    o, l = cpa.partial_attn_merged(inp["q"], inp["q_pos"], inp["cu_q"], [s["k"] for s in st], [s["v"] for s in st],
                                   [s["k_pos"] for s in st], [s["cu_k"] for s in st], inp["max_q"], w.scale,
                                   causal=False)
    torch.cuda.synchronize()
    lens = inp["lens"]
    mine = oracle.zigzag_partition(lens, w.cp, w.rank)
    q_all = torch.cat([d[0] for d in inp["draws"]])
    k_all = torch.cat([d[1] for d in inp["draws"]])
    v_all = torch.cat([d[2] for d in inp["draws"]])
    q = f64(q_all[torch.as_tensor(mine["src_index"], device="cuda")])
    parts = []
    for s in range(w.cp):
        src = oracle.zigzag_partition(lens, w.cp, (w.rank - s) % w.cp)
        idx = torch.as_tensor(src["src_index"], device="cuda")
        parts.append(oracle.partial_attn(q, mine["positions"], mine["cu_seqlens"], f64(k_all[idx]), f64(v_all[idx]),
                                         src["positions"], src["cu_seqlens"], w.scale, causal=False))
    mo, ml = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert_close(f64(o), f64(l), mo, ml, "merged walk without mask")


def test_merged_walk_unsupported_cases(cpa, wl, harness):
    """An odd GQA group or fp32 inputs are refused (compute partials + merge instead)."""
    for name, changes in (("odd", dict(hq=3, hkv=1)), ("fp32", dict(dtype=torch.float32))):
        w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, lengths=(100,), batch=1, len_range=(),
                      **changes)
        inp = harness.build(w, device="cuda")
        run = harness.Runner(inp)
        with pytest.raises(cpa.CpaError) as err:
            run.merged_walk()
        assert err.value.status == -2


@pytest.mark.parametrize("name,changes", MERGED, ids=[m[0] for m in MERGED])
def test_ring_accumulate_all_elements(cpa, wl, harness, name, changes):
    """Running merge: the shards folded in one at a time into (O, LSE) equal
    the oracle's merged result, both as the ring runs them (the own shard as
    a plain partial, the others folded in) and folded into an empty
    accumulator (LSE -inf, O NaN: an empty row's O is never read)."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, seed=600 + len(name), **changes)
    _say(f"case ring {name}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    _, _, merged = expected_pass_kv(inp, None)
    run.poison()
    run.ring_accumulate()
    torch.cuda.synchronize()
    assert_close(f64(run.o), f64(run.lse), merged[0], merged[1], f"ring {name} (bf16 out)")
    assert_close(f64(run.o_parts[0]), f64(run.lse_parts[0]), merged[0], merged[1], f"ring {name} (fp32 acc)")
    # every shard folded into an empty accumulator
    st = inp["steps"]
    accs = []
    for ws in (None, run.workspace):  # index order, then heaviest-first order: the same bits
        o_acc = torch.full_like(run.o_parts[0], float("nan"))
        lse_acc = torch.full_like(run.lse_parts[0], float("-inf"))
        for s in st:
            cpa.partial_attn_accumulate(inp["q"], inp["q_pos"], inp["cu_q"], s["k"], s["v"], s["k_pos"], s["cu_k"],
                                        inp["max_q"], w.scale, o_acc, lse_acc, workspace=ws)
        torch.cuda.synchronize()
        accs.append((o_acc, lse_acc))
    o_acc, lse_acc = accs[0]
    assert_close(f64(o_acc), f64(lse_acc), merged[0], merged[1], f"ring {name} from an empty accumulator")
    assert torch.equal(accs[1][0], o_acc) and torch.equal(accs[1][1], lse_acc)


GRAPH_CASES = [
    ("pass_kv", "qwen2.5_3b_cp2_rank0", dict(lengths=(300, 517, 1000), batch=3, len_range=(), cp=2, rank=1)),
    ("pass_q", "chunked_prefill_passq_cp4", dict(batch=2, cached=1000, new=300, cp=4, rank=0, interleave=8)),
    ("decode", "allgather_decode_cp2", dict(batch=16, len_range=(1, 3000), lengths=(), cp=2, rank=0, interleave=8)),
]


@pytest.mark.parametrize("kind,base,changes", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_graph_replay_matches_eager(cpa, wl, harness, kind, base, changes):
    """The step captured in a HIP graph: three replays, each after other eager
    work on the same buffers, each bit-identical to the eager step."""
    w = wl.scaled(wl.WORKLOADS[base], name=f"graph_{kind}", seed=700 + len(kind), kind=kind, **changes)
    _say(f"case graph {kind}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    cases = [(run.step, lambda: [run.o, run.lse] + run.o_parts + run.lse_parts)]
    if kind == "pass_kv":
        cases.append((run.merged_walk, lambda: [run.o, run.lse]))
    for fn, outputs in cases:
        fn()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outputs()]
        graph = run.capture(fn)
        for rep in range(3):
            for t in outputs():
                t.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(outputs(), ref)):
                assert torch.equal(a, b), f"{kind} {fn.__name__} replay {rep}: output {i} differs from eager"
            # eager work on the same buffers between replays
            run.partial(0)
            run.merge()
            torch.cuda.synchronize()


def test_invariants_ones_and_zero_keys(cpa, wl, harness):
    """V = 1 gives O = 1 on every row that sees a key; K = 0 gives
    LSE = ln(#visible keys) exactly enough to check the mask counts."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name="inv", lengths=(1000, 333), batch=2, len_range=())
    _say("case invariants")
    inp = harness.build(w, device="cuda")
    st = inp["steps"][0]
    ones = torch.ones_like(st["v"])
    zeros = torch.zeros_like(st["k"])
    o, l = cpa.partial_attn(inp["q"], inp["q_pos"], inp["cu_q"], st["k"], ones, st["k_pos"], st["cu_k"],
                            inp["max_q"], w.scale)
    o2, l2 = cpa.partial_attn(inp["q"], inp["q_pos"], inp["cu_q"], zeros, st["v"], st["k_pos"], st["cu_k"],
                              inp["max_q"], w.scale)
    torch.cuda.synchronize()
    fin = torch.isfinite(l)
    # P enters the P.V product rounded to bf16 (relative error <= 2^-9 per weight)
    # while the normaliser sums fp32 P, so O = 1 holds to within 2^-9 / (1 - 2^-9).
    assert float(torch.abs(o[fin] - 1).max()) <= 2.0 ** -8
    qp, cu = inp["q_positions_host"], inp["cu_q_host"]
    kp, cuk = st["k_positions_host"], st["cu_k_host"]
    counts = np.zeros(len(qp))
    for b in range(len(cu) - 1):
        counts[cu[b]:cu[b + 1]] = np.searchsorted(kp[cuk[b]:cuk[b + 1]], qp[cu[b]:cu[b + 1]], side="right")
    want = np.where(counts > 0, np.log(np.maximum(counts, 1)), -np.inf)
    got = f64(l2)
    for h in range(w.hq):
        np.testing.assert_array_equal(np.isneginf(got[:, h]), np.isneginf(want))
        fin = np.isfinite(want)
        assert np.max(np.abs(got[fin, h] - want[fin])) < 1e-5


def test_merge_identity_and_empty_part(cpa):
    _say("case merge identity")
    g = torch.Generator(device="cuda").manual_seed(7)
    o = torch.randn((1000, 8, 128), generator=g, device="cuda")
    l = torch.randn((1000, 8), generator=g, device="cuda")
    mo, ml = cpa.lse_merge([o], [l])
    torch.cuda.synchronize()
    assert torch.allclose(mo, o, atol=1e-5) and torch.allclose(ml, l, atol=1e-5)
    mo, ml = cpa.lse_merge([torch.zeros_like(o), o], [torch.full_like(l, -math.inf), l])
    torch.cuda.synchronize()
    assert torch.allclose(mo, o, atol=1e-5) and torch.allclose(ml, l, atol=1e-5)
    e = torch.full_like(l, -math.inf)
    mo, ml = cpa.lse_merge([torch.zeros_like(o)] * 3, [e] * 3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(ml)) and torch.all(mo == 0)


@pytest.mark.parametrize("n_parts,d", [(1, 64), (3, 128), (16, 64), (5, 128)])
def test_merge_random_parts_vs_oracle(cpa, n_parts, d):
    _say(f"case merge n={n_parts} d={d}")
    g = torch.Generator(device="cuda").manual_seed(n_parts * 100 + d)
    rows = 777
    os_ = [torch.randn((rows, d), generator=g, device="cuda") for _ in range(n_parts)]
    ls_ = [torch.randn((rows,), generator=g, device="cuda") * 5 for _ in range(n_parts)]
    ls_[0][::7] = -math.inf
    for dt in (torch.float32, torch.bfloat16):
        parts_o = [x.to(dt) for x in os_]
        mo, ml = cpa.lse_merge(parts_o, ls_, out_dtype=dt)
        torch.cuda.synchronize()
        ro, rl = oracle.lse_merge([f64(x) for x in parts_o], [f64(x) for x in ls_])
        assert_close(f64(mo), f64(ml), ro, rl, f"merge {dt}")


# ----------------------------------------------------------------- the five full-size workloads


def _row_properties(inp, run):
    """Properties every row must satisfy at any size: no NaN, merged LSE finite
    (every query sees at least one key overall), and |O| <= max |V| since O is
    a convex combination of value rows."""
    for t in [run.o, run.lse] + run.o_parts + run.lse_parts:
        assert not torch.isnan(t).any()
    assert torch.isfinite(run.lse).all()
    vmax = max(float(d[2].float().abs().max()) for d in inp["draws"])
    assert float(run.o.float().abs().max()) <= vmax * (1 + 2 ** -8) + 1e-3
    for o in run.o_parts:
        assert float(o.abs().max()) <= vmax * (1 + 2 ** -8) + 1e-3


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen2.5_3b_cp2_rank0", "llama3_8b_128k_cp4_rank1", "chunked_prefill_passq_cp4",
                                  "allgather_decode_cp2"])
def test_full_size_workload(cpa, wl, harness, name):
    """A workload at full size in the launch configuration the benchmark times,
    into outputs filled with NaN first: every row is checked for the
    properties that hold at any size (so an unwritten row fails), every
    element of the Qwen2.5-3B-shaped and decode workloads is compared with the
    oracle, and sampled rows of the other two."""
    w = wl.WORKLOADS[name]
    _say(f"case full-size {name}")
    inp = harness.build(w, device="cuda")
    run = harness.Runner(inp)
    run.poison()
    run.step()
    torch.cuda.synchronize()
    _row_properties(inp, run)
    cu, pos = inp["cu_q_host"], inp["q_positions_host"]
    rows = None if name in ALL_ROWS else sample_rows(cu, pos, n_random=192, seed=w.seed)
    if w.kind == "pass_kv":
        rows_, parts, merged = expected_pass_kv(inp, rows)
        # exact -inf pattern on every row of every step, from positions alone
        for s, st in enumerate(inp["steps"]):
            kp, cuk = st["k_positions_host"], st["cu_k_host"]
            got = f64(run.lse_parts[s])
            for b in range(len(cu) - 1):
                qa, qe = cu[b], cu[b + 1]
                first = kp[cuk[b]] if cuk[b + 1] > cuk[b] else np.iinfo(np.int64).max
                empty = pos[qa:qe] < first
                np.testing.assert_array_equal(np.isneginf(got[qa:qe]).all(axis=1), empty)
    else:
        rows_, parts, merged = expected_round_robin(inp, rows)
    ridx = torch.as_tensor(rows_, device="cuda")
    for s, (o_ref, l_ref) in enumerate(parts):
        e = assert_close(f64(run.o_parts[s][ridx]), f64(run.lse_parts[s][ridx]), o_ref, l_ref, f"{name} part {s}")
        _say(f"  part {s}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} over {len(rows_)} rows")
    e = assert_close(f64(run.o[ridx]), f64(run.lse[ridx]), merged[0], merged[1], f"{name} merged")
    _say(f"  merged: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} over {len(rows_)} of {len(pos)} rows")


def test_launch_past_the_sort_capacity(cpa, wl, harness):
    """More (query tile, sequence, shard) units than the launch-order pre-pass
    sorts (8192: here 4100 short sequences x 2 shards): the workspace query
    reports 0 bytes and the batched launch runs in index order, searching each
    unit's key range itself. Every element of both partials and of the merge
    against the oracle, into NaN-filled outputs."""
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name="many_short", batch=4100, len_range=(3, 40),
                  lengths=(), seed=77)
    _say("case many_short (8200 tile units)")
    inp = harness.build(w, device="cuda")
    units = -(-inp["max_q"] // 128) * len(inp["lens"]) * w.cp
    assert units > 8192
    assert cpa.partial_attn_multi_workspace(w.cp, len(inp["lens"]), inp["max_q"]) == 0
    run = harness.Runner(inp)
    assert run.workspace is None
    run.poison()
    run.step()
    torch.cuda.synchronize()
    _, parts, merged = expected_pass_kv(inp, None)
    for s, (o_ref, l_ref) in enumerate(parts):
        assert_close(f64(run.o_parts[s]), f64(run.lse_parts[s]), o_ref, l_ref, f"many_short partial {s}")
    assert_close(f64(run.o), f64(run.lse), merged[0], merged[1], "many_short merged")
