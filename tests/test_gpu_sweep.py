"""GPU parity over a seeded sweep of small configurations.

Each case draws its own shape (schedule, CP size and rank, head counts and
GQA group, head dim, sequence count and lengths, interleave, cache length)
from a fixed seed, runs the schedule the benchmark runs (pass-KV: the batched
launch and the merge, plus the fused walk and the ring where supported;
pass-Q and decode: the other ranks' partials and the rank's own launch with
them folded in) into NaN-filled outputs, and compares every element with the
oracle. Lengths include ones shorter than a tile, a chunk or an interleave
group, so partial tiles, empty shards and query tiles that straddle the two
zigzag chunks of a rank all occur.
"""
import numpy as np
import pytest
import torch

from parity_util import assert_close, expected_pass_kv, expected_round_robin, f64

pytestmark = pytest.mark.gpu


def _draw_case(i: int) -> tuple:
    rng = np.random.default_rng(9000 + i)
    kind = ("pass_kv", "pass_q", "decode")[i % 3]
    cp = int(rng.choice([1, 2, 3, 4]))
    rank = int(rng.integers(0, cp))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([64, 128]))
    ch = dict(kind=kind, cp=cp, rank=rank, hq=hkv * g, hkv=hkv, d=d, dtype=torch.bfloat16)
    if kind == "pass_kv":
        n = int(rng.integers(1, 5))
        lens = tuple(int(x) for x in rng.integers(1, 900, size=n))
        ch.update(batch=n, lengths=lens, len_range=())
    elif kind == "pass_q":
        ch.update(batch=int(rng.integers(1, 3)), cached=int(rng.integers(0, 1200)), new=int(rng.integers(2, 300)),
                  interleave=int(rng.choice([1, 3, 8, 16])))
    else:
        n = int(rng.integers(1, 12))
        ch.update(batch=n, len_range=(1, int(rng.integers(2, 2500))), lengths=(),
                  interleave=int(rng.choice([1, 3, 8, 16])))
    return f"sweep{i:02d}_{kind}_cp{cp}r{rank}_g{g}_d{d}", ch


CASES = [_draw_case(i) for i in range(60)]
BASE = {"pass_kv": "qwen2.5_3b_cp2_rank0", "pass_q": "chunked_prefill_passq_cp4", "decode": "allgather_decode_cp2"}


@pytest.mark.parametrize("name,changes", CASES, ids=[c[0] for c in CASES])
def test_sweep_all_elements(name, changes):
    import context_partial_attention_amd as cpa
    from context_partial_attention_amd import harness, workloads as wl

    cpa.load_library()
    w = wl.scaled(wl.WORKLOADS[BASE[changes["kind"]]], name=name, seed=4000 + int(name[5:7]), **changes)
    print(f"case {name}: {changes}", flush=True)
    inp = harness.build(w, device="cuda", pool_fill=float("nan"))
    run = harness.Runner(inp)
    run.poison()
    run.step()
    torch.cuda.synchronize()
    if w.kind == "pass_kv":
        _, parts, merged = expected_pass_kv(inp, None)
    else:
        _, parts, merged = expected_round_robin(inp, None)
    for s, (o_ref, l_ref) in enumerate(parts):
        assert_close(f64(run.o_parts[s]), f64(run.lse_parts[s]), o_ref, l_ref, f"{name} partial {s}")
    assert_close(f64(run.o), f64(run.lse), merged[0], merged[1], f"{name} merged")
    if w.kind == "pass_kv" and w.hq // w.hkv % 2 == 0:
        # the fused walk and the ring give the same merged result
        for fn in (run.merged_walk, run.ring_accumulate):
            run.o.fill_(float("nan"))
            run.lse.fill_(float("nan"))
            fn()
            torch.cuda.synchronize()
            assert_close(f64(run.o), f64(run.lse), merged[0], merged[1], f"{name} {fn.__name__}")
