"""The no-allocation batched call (cpa_partial_attn_multi_noalloc) against the
call it varies (cpa_partial_attn_multi with a caller workspace): same kernels,
same launch order, so every output must match bit for bit. Two calls in a
row, the second on a smaller input, then the first again: whatever the shared
scratch keeps from an earlier call must not reach a later one."""
import sys

import pytest
import torch

from parity_util import assert_close, expected_pass_kv, f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    ("cp4_r1_ragged", dict(lengths=(300, 517, 1000), batch=3, len_range=(), cp=4, rank=1)),
    ("cp2_r0_small", dict(lengths=(100, 37), batch=2, len_range=(), cp=2, rank=0)),
]


def _inputs(wl, harness, name, changes):
    w = wl.scaled(wl.WORKLOADS["qwen2.5_3b_cp2_rank0"], name=name, seed=900 + len(name), **changes)
    inp = harness.build(w, device="cuda")
    return w, inp, harness.Runner(inp)


def _noalloc(cpa, w, inp, run):
    st = inp["steps"]
    for o, l in zip(run.o_parts, run.lse_parts):
        o.fill_(float("nan"))
        l.fill_(float("nan"))
    torch.cuda.synchronize()
    cpa.partial_attn_multi_noalloc(inp["q"], inp["q_pos"], inp["cu_q"], [s["k"] for s in st], [s["v"] for s in st],
                                   [s["k_pos"] for s in st], [s["cu_k"] for s in st], inp["max_q"], w.scale,
                                   run.o_parts, run.lse_parts)
    torch.cuda.synchronize()
    return [(o.clone(), l.clone()) for o, l in zip(run.o_parts, run.lse_parts)]


def _with_workspace(w, run):
    assert run.workspace is not None
    for o, l in zip(run.o_parts, run.lse_parts):
        o.fill_(float("nan"))
        l.fill_(float("nan"))
    run.partials_batched(ordered=True)
    torch.cuda.synchronize()
    return [(o.clone(), l.clone()) for o, l in zip(run.o_parts, run.lse_parts)]


def test_noalloc_matches_workspace_call(gpu):
    import context_partial_attention_amd as cpa
    from context_partial_attention_amd import harness
    from context_partial_attention_amd import workloads as wl

    cpa.load_library()
    runs = [_inputs(wl, harness, n, c) for n, c in CASES]
    for i in (0, 1, 0):  # the second call is the smaller input; then the first again
        w, inp, run = runs[i]
        _say(f"case no-alloc {CASES[i][0]}")
        got = _noalloc(cpa, w, inp, run)
        want = _with_workspace(w, run)
        for s, ((go, gl), (wo, wlse)) in enumerate(zip(got, want)):
            assert torch.equal(go, wo), f"{CASES[i][0]} shard {s}: O differs from the workspace call"
            assert torch.equal(gl, wlse), f"{CASES[i][0]} shard {s}: LSE differs from the workspace call"
        rows, parts, _ = expected_pass_kv(inp, None)
        for s, (o_ref, l_ref) in enumerate(parts):
            assert_close(f64(got[s][0]), f64(got[s][1]), o_ref, l_ref, f"no-alloc {CASES[i][0]} shard {s}")


def test_noalloc_rejects_sizes_beyond_its_scratch(gpu):
    import context_partial_attention_amd as cpa
    from context_partial_attention_amd import harness
    from context_partial_attention_amd import workloads as wl

    w, inp, run = _inputs(wl, harness, *CASES[1])
    st = inp["steps"]
    # 8193 query tiles of 128 rows claimed for each of 2 sequences and 2 shards:
    # refused on the host before any launch
    with pytest.raises(cpa.CpaError) as err:
        cpa.partial_attn_multi_noalloc(inp["q"], inp["q_pos"], inp["cu_q"], [s["k"] for s in st],
                                       [s["v"] for s in st], [s["k_pos"] for s in st], [s["cu_k"] for s in st],
                                       8193 * 128, w.scale, run.o_parts, run.lse_parts)
    assert err.value.status == -3 and "8192" in str(err.value)
