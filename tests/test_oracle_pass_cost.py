"""Pins of oracle.pass_cost (per-step transfer against compute for the two
exchange schemes), each from something other than the function itself:
brute-force pair counts, the full-prefill closed form of the crossover, the
pages' two cases, and exact scaling laws."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("q_lens,kv_lens", [([7], [7]), ([5, 3], [40, 3]), ([1], [9]), ([0, 4], [6, 4])])
def test_pairs_equal_brute_force_count(q_lens, kv_lens):
    # visible_pairs counts, one query at a time, the keys with position <= the
    # query's position: the causal set the step computes
    want = 0
    for ql, kl in zip(q_lens, kv_lens):
        qp = np.arange(kl - ql, kl)
        want += oracle.visible_pairs(qp, [0, ql], np.arange(kl), [0, kl])
    r = oracle.pass_cost(q_lens, kv_lens, hq=8, hkv=2, d=64, elem_bytes=2, cp=2, link_bytes_per_s=1e11,
                         mfma_flops_per_s=1e15)
    assert r["pairs"] == want


def test_full_prefill_pairs_closed_form():
    L = 1000
    r = oracle.pass_cost([L], [L], hq=32, hkv=8, d=128, elem_bytes=2, cp=4, link_bytes_per_s=1.53e11,
                         mfma_flops_per_s=1.25e15)
    assert r["pairs"] == L * (L + 1) // 2


@pytest.mark.parametrize("cp,hq,hkv,eb", [(4, 32, 8, 2), (2, 16, 2, 2), (8, 64, 8, 1)])
def test_full_prefill_kv_transfer_hidden_past_closed_form_length(cp, hq, hkv, eb):
    # full prefill of length L: the KV shard of a step is 2*hkv*d*eb*L/cp bytes and
    # the step computes 4*d*hq*L(L+1)/2/cp^2 FLOP, so the transfer hides iff
    # L + 1 >= cp*hkv*eb*mfma/(hq*link), independent of d
    link, mfma = 1e11, 1e15
    thr = cp * hkv * eb * mfma / (hq * link)  # an integer for these sizes
    L0 = int(round(thr)) - 1  # the tie; check one away on either side
    for d in (64, 128):
        lo = oracle.pass_cost([L0 - 1], [L0 - 1], hq, hkv, d, eb, cp, link, mfma)
        hi = oracle.pass_cost([L0 + 1], [L0 + 1], hq, hkv, d, eb, cp, link, mfma)
        assert not lo["kv_hidden"] and hi["kv_hidden"]


def test_the_pages_two_cases():
    # full prefill with groups of more than two query heads per KV head passes KV,
    # and at 128K tokens the KV transfer of a step hides under its compute
    full = oracle.pass_cost([131072], [131072], hq=32, hkv=8, d=128, elem_bytes=2, cp=4,
                            link_bytes_per_s=1.53e11, mfma_flops_per_s=1.25e15)
    assert full["pass_kv"] and full["kv_hidden"]
    # chunked prefill with a cache far longer than the new tokens passes Q, and the
    # Q shard is the cheaper transfer
    chunk = oracle.pass_cost([4096, 4096], [69632, 69632], hq=16, hkv=2, d=128, elem_bytes=2, cp=4,
                             link_bytes_per_s=1.53e11, mfma_flops_per_s=1.25e15)
    assert not chunk["pass_kv"] and chunk["q_transfer_s"] < chunk["kv_transfer_s"] and chunk["q_hidden"]
    # bytes per step: one rank's shard (8192 new tokens and 139264 context tokens over 4 ranks)
    assert chunk["q_step_bytes"] == 8192 * 16 * 128 * 2 / 4
    assert chunk["kv_step_bytes"] == 139264 * 2 * 2 * 128 * 2 / 4


def test_scaling_laws():
    base = dict(q_lens=[300, 70], kv_lens=[2000, 70], hq=16, hkv=2, d=128, elem_bytes=2, cp=2)
    r = oracle.pass_cost(**base, link_bytes_per_s=1e11, mfma_flops_per_s=1e15)
    r2 = oracle.pass_cost(**base, link_bytes_per_s=1e11, mfma_flops_per_s=2e15)
    r3 = oracle.pass_cost(**base, link_bytes_per_s=4e11, mfma_flops_per_s=4e15)
    assert r2["step_compute_s"] == r["step_compute_s"] / 2  # a power of two: exact
    assert r2["kv_transfer_s"] == r["kv_transfer_s"]
    assert (r3["kv_hidden"], r3["q_hidden"]) == (r["kv_hidden"], r["q_hidden"])
    # four times the ranks: each step moves a quarter of the shard bytes, computes a sixteenth
    r4 = oracle.pass_cost(**{**base, "cp": 8}, link_bytes_per_s=1e11, mfma_flops_per_s=1e15)
    assert r4["kv_step_bytes"] == r["kv_step_bytes"] / 4 and r4["step_flops"] == r["step_flops"] / 16


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pass_cost([5], [4], 8, 2, 64, 2, 2, 1e11, 1e15)  # more new tokens than context
    with pytest.raises(ValueError):
        oracle.pass_cost([5], [5], 8, 2, 64, 2, 0, 1e11, 1e15)
    with pytest.raises(ValueError):
        oracle.pass_cost([5], [5], 8, 2, 64, 2, 2, 0.0, 1e15)
