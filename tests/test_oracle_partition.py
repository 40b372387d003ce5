"""Pins for the oracle's integer work: zigzag partition and round-robin placement.

Each test checks the oracle against something other than itself: a library
routine (numpy.array_split), brute-force enumeration, a closed form derived
by hand, or the workload statements kept in tests/golden/.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("L", [0, 1, 3, 7, 8, 64, 255, 256, 1000, 2051, 8195])
@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_chunk_sizes_match_array_split(L, cp):
    want = [len(c) for c in np.array_split(np.arange(L), 2 * cp)]
    assert oracle.zigzag_chunk_sizes(L, cp) == want


def test_chunk_sizes_worked_value():
    assert oracle.zigzag_chunk_sizes(2051, 4) == [257, 257, 257, 256, 256, 256, 256, 256]


def test_zigzag_ownership_golden():
    with open(os.path.join(GOLDEN, "zigzag_ownership.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        part = oracle.zigzag_partition([c["L"]], c["cp"], c["rank"])
        sizes = np.diff(part["chunk_bounds"][0])
        assert set(sizes.tolist()) == {c["chunk_size"]}
        want = np.concatenate([np.arange(a, b) for a, b in c["position_runs"]])
        np.testing.assert_array_equal(part["positions"], want)
        bounds = part["chunk_bounds"][0]
        owned = [int(np.searchsorted(bounds, p, side="right") - 1) for p in (want[0], want[-1])]
        assert owned == c["owned_chunks"]


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_zigzag_covers_every_token_once(cp):
    rng = np.random.default_rng(cp)
    lens = rng.integers(0, 300, size=5).tolist() + [1, 2 * cp - 1]
    seen = np.zeros(sum(lens), dtype=np.int64)
    for r in range(cp):
        part = oracle.zigzag_partition(lens, cp, r)
        seen[part["src_index"]] += 1
        # positions ascend within each sequence and map back to src_index
        cu = part["cu_seqlens"]
        starts = np.concatenate([[0], np.cumsum(lens)])
        for b in range(len(lens)):
            p = part["positions"][cu[b]:cu[b + 1]]
            assert np.all(np.diff(p) > 0)
            np.testing.assert_array_equal(part["src_index"][cu[b]:cu[b + 1]], starts[b] + p)
    assert np.all(seen == 1)


@pytest.mark.parametrize("L,cp", [(256, 2), (64, 4), (96, 3), (16, 8), (2048, 2)])
def test_balance_closed_form_when_divisible(L, cp):
    # Closed form (derived by hand): with 2cp | L and chunk size c = L/(2cp),
    # chunk i's rows see i*c + a + 1 keys, so chunks r and 2cp-1-r together
    # see (2cp-1)c^2 + c(c+1) = L(L+1)/(2cp) pairs, the same for every rank.
    want = L * (L + 1) // (2 * cp)
    for r in range(cp):
        part = oracle.zigzag_partition([L], cp, r)
        pos = part["positions"]
        full = np.arange(L)
        got = oracle.visible_pairs(pos, [0, len(pos)], full, [0, L])
        assert got == want


def test_balance_worked_values():
    assert 256 * 257 // 4 == 16448
    assert 131072 * 131073 // 8 == 2_147_500_032
    # not balanced when 2cp does not divide L: L=2050, cp=2
    got = []
    for r in range(2):
        pos = oracle.zigzag_partition([2050], 2, r)["positions"]
        got.append(oracle.visible_pairs(pos, [0, len(pos)], np.arange(2050), [0, 2050]))
    assert got == [1_050_625, 1_051_650]


def test_partition_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.zigzag_partition([10], 2, 2)
    with pytest.raises(ValueError):
        oracle.zigzag_partition([10], 0, 0)


# ---------------------------------------------------------------- placement


def _local_len_closed_form(L, cp, r, I):
    # Derived by hand: each full cycle of I*cp positions gives I tokens to
    # every rank; the leftover L mod (I*cp) positions fill rank 0's group
    # first, then rank 1's, and so on.
    return (L // (I * cp)) * I + min(max(L % (I * cp) - r * I, 0), I)


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("I", [1, 2, 8, 16])
def test_placement_brute_force(cp, I):
    rng = np.random.default_rng(cp * 100 + I)
    for L in list(rng.integers(0, 500, size=6)) + [I * cp, I * cp + 1]:
        L = int(L)
        owner = np.zeros(L, dtype=np.int64)
        counts = np.zeros(cp, dtype=np.int64)
        local_seen = [[] for _ in range(cp)]
        # brute force: deal groups of I positions to ranks in turn
        for t in range(L):
            r = (t // I) % cp
            owner[t] = r
            local_seen[r].append(t)
            counts[r] += 1
        np.testing.assert_array_equal(oracle.rr_rank(np.arange(L), cp, I), owner)
        for r in range(cp):
            assert oracle.rr_local_len(L, cp, r, I) == counts[r] == _local_len_closed_form(L, cp, r, I)
            pl = oracle.rr_placement([L], cp, r, I)
            np.testing.assert_array_equal(pl["local_to_global"], np.array(local_seen[r], dtype=np.int64))
            l = np.arange(counts[r])
            t = oracle.rr_global_index(l, r, cp, I)
            np.testing.assert_array_equal(oracle.rr_local_index(t, cp, I), l)
            np.testing.assert_array_equal(oracle.rr_rank(t, cp, I), np.full(len(l), r))


def test_placement_golden_counts():
    with open(os.path.join(GOLDEN, "rr_placement_counts.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = [oracle.rr_local_len(c["L"], c["cp"], r, c["interleave"]) for r in range(c["cp"])]
        assert got == c["local_lens"], c


@pytest.mark.parametrize("I", [1, 4, 8, 16])
def test_half_of_computed_tokens_at_cp2(I):
    # The utility page's review fixes a cp=2 test to expect each request to
    # keep N // 2 of its computed tokens on a rank; with round-robin groups
    # of I this holds whenever 2*I divides N.
    for N in (2 * I, 10 * I, 64 * I):
        pl = oracle.rr_placement([N, 2 * N], 2, 0, I)
        assert pl["local_lens"].tolist() == [N // 2, N]


def test_placement_packs_sequences():
    lens = [5, 0, 33, 17]
    pl = oracle.rr_placement(lens, 3, 1, 4)
    assert pl["cu_local"].tolist() == np.concatenate([[0], np.cumsum(pl["local_lens"])]).tolist()
    for b, L in enumerate(lens):
        seg = pl["local_to_global"][pl["cu_local"][b]:pl["cu_local"][b + 1]]
        assert np.all(seg < L)
        assert np.all(np.diff(seg) > 0)


# ----------------------------------------------------------------- choice of the exchanged shard


def test_choose_pass_follows_the_pages_statements():
    """[PASSKV], Purpose: full prefill passes KV when a KV head serves more than
    two query heads; chunked prefill with a much longer cache passes Q."""
    # full prefill, GQA groups of 8 (the Qwen2.5-3B and Llama-3-8B shapes): pass KV
    assert oracle.choose_pass([4096, 2048], [4096, 2048], hq=16, hkv=2, d=128)["pass_kv"]
    assert oracle.choose_pass([131072], [131072], hq=32, hkv=8, d=128)["pass_kv"]
    # full prefill without grouping (MHA, one query head per KV head): pass Q
    assert not oracle.choose_pass([4096], [4096], hq=32, hkv=32, d=128)["pass_kv"]
    # chunked prefill, 4096 new tokens on a 65536-token cache, groups of 8: pass Q
    assert not oracle.choose_pass([4096, 4096], [69632, 69632], hq=16, hkv=2, d=128)["pass_kv"]


@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
def test_choose_pass_full_prefill_boundary_is_group_of_two(g):
    """With kv_lens == q_lens the rule reduces to hq / hkv > 2 (closed form),
    whatever the lengths, head dim or element size."""
    rng = np.random.default_rng(g)
    lens = rng.integers(1, 5000, size=5)
    for d, eb in ((64, 2), (128, 2), (128, 4)):
        r = oracle.choose_pass(lens, lens, hq=4 * g, hkv=4, d=d, elem_bytes=eb)
        assert r["pass_kv"] == (g > 2)
        assert r["kv_bytes"] == 2 * 4 * d * eb * int(lens.sum())
        assert r["q_bytes"] == 4 * g * d * eb * int(lens.sum())


def test_choose_pass_crossover_in_cache_length():
    """Chunked prefill: with q new tokens and group g, pass KV holds exactly while
    the context is shorter than g*q/2 tokens (brute force over lengths)."""
    for g, q in ((8, 100), (4, 37), (2, 64)):
        for ctx in range(q, g * q):
            assert oracle.choose_pass([q], [ctx], hq=2 * g, hkv=2, d=64)["pass_kv"] == (2 * ctx < g * q)
