"""Pins for the oracle's floating-point work: attention, partial attention, merge.

Every check compares the oracle with something independent of it: a
pure-Python brute force with math.fsum, torch's scaled_dot_product_attention
in fp64 on the CPU, scipy's logsumexp, hand-derived closed forms, and
invariants of the method (merging partials over any split of the keys gives
full attention).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute_force(q, k, v, scale):
    """Causal GQA attention with Python loops and math.fsum."""
    L, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o = np.zeros((L, hq, d))
    lse = np.zeros((L, hq))
    for h in range(hq):
        kv = h // g
        for i in range(L):
            s = [scale * math.fsum(q[i, h, x] * k[j, kv, x] for x in range(d)) for j in range(i + 1)]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            lse[i, h] = m + math.log(z)
            for x in range(d):
                o[i, h, x] = math.fsum(math.exp(s[j] - lse[i, h]) * v[j, kv, x] for j in range(i + 1))
    return o, lse


@pytest.mark.parametrize("L,hq,hkv,d", [(1, 1, 1, 1), (7, 2, 1, 3), (12, 4, 2, 5), (24, 3, 3, 4)])
def test_full_attn_brute_force(L, hq, hkv, d):
    q, k, v = _rand((L, hq, d), 1), _rand((L, hkv, d), 2), _rand((L, hkv, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.full_causal_attn(q, k, v, scale)
    bo, blse = _brute_force(q, k, v, scale)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,hq,hkv,d", [(50, 8, 2, 64), (33, 4, 4, 16), (70, 16, 2, 8)])
def test_full_attn_vs_torch_sdpa_fp64(L, hq, hkv, d):
    q, k, v = _rand((L, hq, d), 4), _rand((L, hkv, d), 5), _rand((L, hkv, d), 6)
    scale = 1 / math.sqrt(d)
    o, _ = oracle.full_causal_attn(q, k, v, scale)
    g = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)  # [H, L, D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    L, hq, hkv, d = 40, 4, 2, 8
    q, k, v = _rand((L, hq, d), 7), _rand((L, hkv, d), 8), _rand((L, hkv, d), 9)
    scale = 0.3
    _, lse = oracle.full_causal_attn(q, k, v, scale)
    for h in range(hq):
        s = scale * q[:, h, :] @ k[:, h // 2, :].T
        s[np.triu_indices(L, 1)] = -np.inf
        np.testing.assert_allclose(lse[:, h], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    # With V = identity (one-hot per key), O is the softmax row itself.
    L, d = 20, 20
    q = _rand((L, 1, 6), 10)
    k = _rand((L, 1, 6), 11)
    v = np.eye(L)[:, None, :]
    o, _ = oracle.full_causal_attn(q, k, v, 0.5)
    p = o[:, 0, :]
    np.testing.assert_allclose(p.sum(axis=1), np.ones(L), rtol=0, atol=1e-13)
    assert np.all(p >= 0)
    assert np.all(p[np.triu_indices(L, 1)] == 0)


def test_hand_worked_two_keys():
    # q0 = (1, 0), q1 = (0, 1), k0 = (1, 0), k1 = (0, 1), v0 = (1, 2), v1 = (3, 4), scale 1.
    # Row 0 sees key 0 only: s = 1, LSE = 1, O = v0.
    # Row 1 sees both: s = (0, 1), LSE = ln(1 + e), O = (v0 + e v1) / (1 + e).
    q = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])
    o, lse = oracle.full_causal_attn(q, k, v, 1.0)
    e = math.e
    assert lse[0, 0] == pytest.approx(1.0, abs=1e-15)
    np.testing.assert_allclose(o[0, 0], [1.0, 2.0], atol=1e-15)
    assert lse[1, 0] == pytest.approx(math.log(1 + e), abs=1e-15)
    np.testing.assert_allclose(o[1, 0], [(1 + 3 * e) / (1 + e), (2 + 4 * e) / (1 + e)], atol=1e-15)


# ------------------------------------------------------------ partial attention


def test_partial_equals_full_when_shard_is_whole_sequence():
    L, hq, hkv, d = 37, 4, 2, 8
    q, k, v = _rand((L, hq, d), 12), _rand((L, hkv, d), 13), _rand((L, hkv, d), 14)
    pos = np.arange(L)
    o, lse = oracle.partial_attn(q, pos, [0, L], k, v, pos, [0, L], 0.25)
    fo, flse = oracle.full_causal_attn(q, k, v, 0.25)
    np.testing.assert_array_equal(o, fo)
    np.testing.assert_array_equal(lse, flse)


def test_partial_zero_keys_closed_form():
    # K = 0 makes every visible score 0: LSE = ln(#visible), O = mean of visible V.
    rng = np.random.default_rng(15)
    q_pos = np.sort(rng.choice(200, size=30, replace=False))
    k_pos = np.sort(rng.choice(200, size=40, replace=False))
    q = _rand((30, 4, 6), 16)
    k = np.zeros((40, 2, 6))
    v = _rand((40, 2, 6), 17)
    o, lse = oracle.partial_attn(q, q_pos, [0, 30], k, v, k_pos, [0, 40], 1.0)
    for i, p in enumerate(q_pos):
        n = int(np.sum(k_pos <= p))
        for h in range(4):
            if n == 0:
                assert lse[i, h] == -np.inf and np.all(o[i, h] == 0)
            else:
                assert lse[i, h] == pytest.approx(math.log(n), abs=1e-14)
                np.testing.assert_allclose(o[i, h], v[k_pos <= p, h // 2].mean(axis=0), atol=1e-14)


def test_partial_ones_values():
    q, k = _rand((9, 2, 4), 18), _rand((11, 1, 4), 19)
    v = np.ones((11, 1, 4))
    q_pos = np.arange(20, 29)
    k_pos = np.arange(15, 37, 2)
    o, lse = oracle.partial_attn(q, q_pos, [0, 9], k, v, k_pos, [0, 11], 0.5)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    assert np.all(np.isfinite(lse))


def test_partial_empty_rows_and_empty_shard():
    q = _rand((4, 2, 4), 20)
    k, v = _rand((3, 1, 4), 21), _rand((3, 1, 4), 22)
    o, lse = oracle.partial_attn(q, [0, 1, 2, 3], [0, 4], k, v, [10, 11, 12], [0, 3], 1.0)
    assert np.all(lse == -np.inf) and np.all(o == 0)
    o, lse = oracle.partial_attn(q, [0, 1, 2, 3], [0, 4], k[:0], v[:0], [], [0, 0], 1.0)
    assert np.all(lse == -np.inf) and np.all(o == 0)


def test_partial_no_mask_sees_whole_shard():
    q, k, v = _rand((5, 2, 4), 23), _rand((6, 2, 4), 24), _rand((6, 2, 4), 25)
    o, lse = oracle.partial_attn(q, np.zeros(5), [0, 5], k, v, np.arange(100, 106), [0, 6], 1.0, causal=False)
    for h in range(2):
        s = q[:, h] @ k[:, h].T
        np.testing.assert_allclose(lse[:, h], logsumexp(s, axis=1), atol=1e-13)


def test_partial_varlen_sequences_do_not_mix():
    lens = [5, 9]
    q = _rand((14, 2, 4), 26)
    k, v = _rand((14, 1, 4), 27), _rand((14, 1, 4), 28)
    pos = np.concatenate([np.arange(5), np.arange(9)])
    o, lse = oracle.partial_attn(q, pos, [0, 5, 14], k, v, pos, [0, 5, 14], 0.7)
    o0, l0 = oracle.full_causal_attn(q[:5], k[:5], v[:5], 0.7)
    o1, l1 = oracle.full_causal_attn(q[5:], k[5:], v[5:], 0.7)
    np.testing.assert_array_equal(o, np.concatenate([o0, o1]))
    np.testing.assert_array_equal(lse, np.concatenate([l0, l1]))


def test_partial_rows_subset():
    q, k, v = _rand((20, 2, 4), 29), _rand((20, 1, 4), 30), _rand((20, 1, 4), 31)
    pos = np.arange(20)
    o, lse = oracle.partial_attn(q, pos, [0, 20], k, v, pos, [0, 20], 1.0)
    rows = np.array([3, 17, 0])
    so, slse = oracle.partial_attn(q, pos, [0, 20], k, v, pos, [0, 20], 1.0, rows=rows)
    np.testing.assert_array_equal(so, o[rows])
    np.testing.assert_array_equal(slse, lse[rows])


# ------------------------------------------------------------------- merge


def test_merge_over_random_key_splits_equals_full():
    rng = np.random.default_rng(32)
    L, hq, hkv, d = 60, 4, 2, 8
    q, k, v = _rand((L, hq, d), 33), _rand((L, hkv, d), 34), _rand((L, hkv, d), 35)
    pos = np.arange(L)
    fo, flse = oracle.full_causal_attn(q, k, v, 0.4)
    for trial in range(6):
        nparts = int(rng.integers(1, 6))
        owner = rng.integers(0, nparts, size=L)
        if trial == 0:
            owner[:] = 0  # all keys in part 0, the others empty
        if trial == 1:
            owner[:] = 1 % nparts
            owner[7] = 0  # a one-token shard
        os_, ls_ = [], []
        for s in range(nparts):
            kp = pos[owner == s]
            o, l = oracle.partial_attn(q, pos, [0, L], k[owner == s], v[owner == s], kp, [0, len(kp)], 0.4)
            os_.append(o)
            ls_.append(l)
        mo, ml = oracle.lse_merge(os_, ls_)
        np.testing.assert_allclose(mo, fo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, flse, rtol=0, atol=1e-12)


def test_merge_identity_and_ignored_empty_part():
    o, l = _rand((10, 3, 4), 36), _rand((10, 3), 37)
    mo, ml = oracle.lse_merge([o], [l])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, l, atol=1e-15)
    mo, ml = oracle.lse_merge([np.zeros_like(o), o], [np.full_like(l, -np.inf), l])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, l, atol=1e-15)


def test_merge_all_empty_rows():
    o = np.zeros((3, 2, 4))
    l = np.full((3, 2), -np.inf)
    mo, ml = oracle.lse_merge([o, o, o], [l, l, l])
    assert np.all(ml == -np.inf) and np.all(mo == 0)


def test_merge_equal_lse_closed_form():
    a, b = _rand((5, 4), 38), _rand((5, 4), 39)
    l = _rand((5,), 40)
    mo, ml = oracle.lse_merge([a, b], [l, l])
    np.testing.assert_allclose(ml, l + math.log(2), atol=1e-14)
    np.testing.assert_allclose(mo, (a + b) / 2, atol=1e-14)


def test_merge_permutation_invariant():
    os_ = [_rand((6, 3), 41 + i) for i in range(4)]
    ls_ = [_rand((6,), 51 + i) * 3 for i in range(4)]
    mo, ml = oracle.lse_merge(os_, ls_)
    perm = [2, 0, 3, 1]
    po, pl = oracle.lse_merge([os_[i] for i in perm], [ls_[i] for i in perm])
    np.testing.assert_allclose(po, mo, atol=1e-14)
    np.testing.assert_allclose(pl, ml, atol=1e-14)


# ---------------------------------------------------------- whole schedules


@pytest.mark.parametrize("L,cp,rank", [(256, 2, 0), (256, 2, 1), (203, 3, 2), (64, 4, 1), (5, 4, 3)])
def test_pass_kv_schedule_reproduces_full_attention(L, cp, rank):
    hq, hkv, d = 4, 2, 8
    q, k, v = _rand((L, hq, d), 60), _rand((L, hkv, d), 61), _rand((L, hkv, d), 62)
    mine = oracle.zigzag_partition([L], cp, rank)
    qp = mine["positions"]
    os_, ls_ = [], []
    for s in range(cp):
        src = (rank - s) % cp
        kp = oracle.zigzag_partition([L], cp, src)["positions"]
        o, l = oracle.partial_attn(q[qp], qp, [0, len(qp)], k[kp], v[kp], kp, [0, len(kp)], 0.3)
        os_.append(o)
        ls_.append(l)
    mo, ml = oracle.lse_merge(os_, ls_)
    fo, fl = oracle.full_causal_attn(q, k, v, 0.3, rows=qp)
    np.testing.assert_allclose(mo, fo, atol=1e-12)
    np.testing.assert_allclose(ml, fl, atol=1e-12)


@pytest.mark.parametrize("cp,I", [(4, 8), (2, 8), (3, 2)])
def test_round_robin_partials_reproduce_full_attention(cp, I):
    # pass-Q over a round-robin cache (new queries at the end of the sequence)
    # and allgather decode (one query at L-1) both merge one partial per rank.
    L, n_new, hq, hkv, d = 150, 20, 4, 1, 8
    q, k, v = _rand((L, hq, d), 63), _rand((L, hkv, d), 64), _rand((L, hkv, d), 65)
    for qrows in (np.arange(L - n_new, L), np.array([L - 1])):
        os_, ls_ = [], []
        for r in range(cp):
            kp = oracle.rr_placement([L], cp, r, I)["local_to_global"]
            o, l = oracle.partial_attn(q[qrows], qrows, [0, len(qrows)], k[kp], v[kp], kp, [0, len(kp)], 0.2)
            os_.append(o)
            ls_.append(l)
        mo, ml = oracle.lse_merge(os_, ls_)
        fo, fl = oracle.full_causal_attn(q, k, v, 0.2, rows=qrows)
        np.testing.assert_allclose(mo, fo, atol=1e-12)
        np.testing.assert_allclose(ml, fl, atol=1e-12)
