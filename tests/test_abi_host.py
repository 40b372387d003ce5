"""C-ABI checks that need no GPU: the library loads, exports every function
include/cpattn.h declares, its host integer calls match the oracle bit for
bit, and bad arguments come back as error statuses (before any GPU access).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cpa():
    import context_partial_attention_amd as cpa

    if not os.path.exists(cpa.library_path()):
        pytest.fail("libcpattn.so is not built (python -m context_partial_attention_amd.build)")
    cpa.load_library()
    return cpa


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "cpattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cpa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ["cpa_cp_partition", "cpa_rr_placement", "cpa_partial_attn", "cpa_partial_attn_paged",
                 "cpa_partial_attn_paged_workspace", "cpa_lse_merge", "cpa_last_error"]:
        assert want in names


def test_library_exports_every_declared_symbol(cpa):
    lib = ctypes.CDLL(cpa.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_cp_partition_matches_oracle(cpa, cp):
    rng = np.random.default_rng(cp)
    lens = [0, 1, 2 * cp - 1, 2 * cp] + rng.integers(0, 5000, size=6).tolist() + [8195, 2051]
    for r in range(cp):
        got = cpa.cp_partition(lens, cp, r)
        want = oracle.zigzag_partition(lens, cp, r)
        for key in ("chunk_bounds", "cu_seqlens", "positions", "src_index"):
            np.testing.assert_array_equal(got[key], want[key].astype(np.int32), err_msg=key)


@pytest.mark.parametrize("cp,I", [(1, 1), (2, 8), (3, 2), (4, 8), (4, 16), (8, 1)])
def test_rr_placement_matches_oracle(cpa, cp, I):
    rng = np.random.default_rng(cp * 10 + I)
    lens = [0, 1, I, I * cp, I * cp + 1] + rng.integers(0, 3000, size=6).tolist()
    for r in range(cp):
        got = cpa.rr_placement(lens, cp, r, I)
        want = oracle.rr_placement(lens, cp, r, I)
        np.testing.assert_array_equal(got["local_lens"], want["local_lens"].astype(np.int32))
        np.testing.assert_array_equal(got["local_to_global"], want["local_to_global"].astype(np.int32))


def test_workload_sized_placement(cpa):
    # the chunked-prefill layout: 69632 tokens over 4 ranks, interleave 8
    for r in range(4):
        got = cpa.rr_placement([69632, 69632], 4, r, 8)
        assert got["local_lens"].tolist() == [17408, 17408]
        want = oracle.rr_placement([69632], 4, r, 8)["local_to_global"].astype(np.int32)
        np.testing.assert_array_equal(got["local_to_global"][:17408], want)


def test_partition_large_sequence(cpa):
    got = cpa.cp_partition([131072], 4, 1)
    assert got["positions"][0] == 16384 and got["positions"][16383] == 32767
    assert got["positions"][16384] == 98304 and got["positions"][-1] == 114687


def _status(fn, *args):
    return fn(*args)


def test_host_error_statuses(cpa):
    lib = cpa.load_library()
    n = ctypes.c_int64(0)
    lens = (ctypes.c_int32 * 2)(10, 20)
    # rank out of range, cp < 1, NULL n_out, negative length, capacity too small
    assert lib.cpa_cp_partition(2, lens, 2, 2, None, None, None, None, 0, ctypes.byref(n)) == -1
    assert b"rank" in lib.cpa_last_error()
    assert lib.cpa_cp_partition(2, lens, 0, 0, None, None, None, None, 0, ctypes.byref(n)) == -1
    assert lib.cpa_cp_partition(2, lens, 2, 0, None, None, None, None, 0, None) == -1
    bad = (ctypes.c_int32 * 1)(-5)
    assert lib.cpa_cp_partition(1, bad, 2, 0, None, None, None, None, 0, ctypes.byref(n)) == -1
    small = (ctypes.c_int32 * 4)()
    assert lib.cpa_cp_partition(2, lens, 2, 0, None, None, small, None, 4, ctypes.byref(n)) == -3
    assert n.value == 15
    loc = (ctypes.c_int32 * 2)()
    assert lib.cpa_rr_placement(2, lens, 2, 0, 0, loc, None, 0, ctypes.byref(n)) == -1  # interleave 0
    assert lib.cpa_rr_placement(2, lens, 2, 0, 8, loc, small, 4, ctypes.byref(n)) == -3
    # rank 0 at cp=2, I=8 holds positions 0-7 of L=10 and 0-7, 16-19 of L=20: 8 + 12 tokens
    assert lib.cpa_rr_placement(2, lens, 2, 0, 8, loc, None, 0, ctypes.byref(n)) == 0 and n.value == 20
    assert list(loc) == [8, 12]


def test_device_call_validation_before_gpu(cpa):
    """Argument errors are reported without touching a GPU (none is present here)."""
    lib = cpa.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # hq not a multiple of hkv
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 6, 4, 128, 0, 0.1, 1, fake, 1,
                                fake, None) == -1
    # unsupported head dim
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, 2, 96, 0, 0.1, 1, fake, 1,
                                fake, None) == -2
    # fp32 input with bf16 output
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, 2, 64, 1, 0.1, 1, fake, 0,
                                fake, None) == -2
    # bad scale, bad mask
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, 2, 64, 0, -1.0, 1, fake, 1,
                                fake, None) == -1
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, 2, 64, 0, 0.1, 7, fake, 1,
                                fake, None) == -1
    # NULL output pointer
    assert lib.cpa_partial_attn(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, 2, 64, 0, 0.1, 1, None, 1,
                                fake, None) == -1
    # paged: cp_rank >= cp_size, interleave 0, block size 32, workspace too small for decode
    args = dict(bs=16, cp=2, rank=0, il=8, maxq=4, ws=None, wsb=0)

    def paged(bs=16, cp=2, rank=0, il=8, maxq=4, ws=None, wsb=0, dtype=0):
        return lib.cpa_partial_attn_paged(fake, fake, fake, fake, fake, fake, 8, fake, bs, cp, rank, il, 2, maxq,
                                          8, 2, 128, dtype, 0.1, 1, fake, 1, fake, ws, wsb, None)

    assert paged(**{**args, "rank": 2}) == -1
    assert paged(**{**args, "il": 0}) == -1
    assert paged(**{**args, "bs": 32}) == -2
    assert paged(**{**args, "maxq": 1}) == -3
    assert paged(dtype=1) == -2
    need = ctypes.c_size_t(0)
    assert lib.cpa_partial_attn_paged_workspace(2, 1, 8, 16, 8, 128, ctypes.byref(need)) == 0
    assert need.value == 2 * 8 * 1 * 129 * 4
    # decode splits: 2048 local tokens while that leaves >= 1024 (sequence, split) pairs at the
    # longest length, else 1024, else 512
    for seqs, blocks, split in [(256, 1024, 2048), (128, 1024, 2048), (100, 1024, 1024), (60, 1024, 512),
                                (16, 8192, 2048), (1, 10, 512), (512, 188, 2048), (400, 188, 1024)]:
        assert lib.cpa_partial_attn_paged_workspace(seqs, 1, blocks, 16, 32, 128, ctypes.byref(need)) == 0
        assert need.value == seqs * 32 * -(-blocks * 16 // split) * 129 * 4, (seqs, blocks, split)
    assert lib.cpa_partial_attn_paged_workspace(2, 7, 8, 16, 8, 128, ctypes.byref(need)) == 0 and need.value == 0
    # merge: too many parts, bad d
    ptrs = (ctypes.c_void_p * 17)(*([0x1000] * 17))
    assert lib.cpa_lse_merge(17, ptrs, ptrs, 1, 10, 128, fake, 1, fake, None) == -1
    assert lib.cpa_lse_merge(2, ptrs, ptrs, 1, 10, 80, fake, 1, fake, None) == -2
    assert lib.cpa_lse_merge(0, ptrs, ptrs, 1, 10, 128, fake, 1, fake, None) == -1


def test_multi_shard_call_validation_before_gpu(cpa):
    lib = cpa.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    arr = (ctypes.c_void_p * 9)(*([0x1000] * 9))

    def multi(n, k=arr, mask=1, hkv=2, d=128):
        return lib.cpa_partial_attn_multi(n, fake, fake, fake, k, arr, arr, arr, 1, 4, 8, hkv, d, 0, 0.1, mask, arr,
                                          1, arr, None, 0, None)

    assert multi(0) == -1  # no shard
    assert multi(9) == -1  # more than 8 shards
    assert multi(2, k=None) == -1  # NULL pointer array
    assert multi(2, hkv=3) == -1  # hq not a multiple of hkv
    assert multi(2, d=96) == -2  # unsupported head dim
    n = ctypes.c_size_t(7)
    assert lib.cpa_partial_attn_multi_workspace(2, 4, 3700, ctypes.byref(n)) == 0
    assert n.value >= 29 * 4 * 2 * 4 and n.value % 256 == 0  # one int per (query tile, sequence, shard)
    assert lib.cpa_partial_attn_multi_workspace(2, 4, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.cpa_partial_attn_multi_workspace(9, 4, 100, ctypes.byref(n)) == -1
    # the ordering pre-pass sorts at most 8192 (query tile, sequence, shard) units; past that the
    # launch runs in index order and asks for no workspace
    assert lib.cpa_partial_attn_multi_workspace(8, 64, 2048, ctypes.byref(n)) == 0 and n.value == 8192 * 4
    assert lib.cpa_partial_attn_multi_workspace(8, 64, 2049, ctypes.byref(n)) == 0 and n.value == 0


def test_merged_call_validation_before_gpu(cpa):
    lib = cpa.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    arr = (ctypes.c_void_p * 9)(*([0x1000] * 9))

    def merged(n, k=arr, hkv=2, d=128, dt=0, odt=1):
        return lib.cpa_partial_attn_merged(n, fake, fake, fake, k, arr, arr, arr, 1, 4, 8, hkv, d, dt, 0.1, 1, fake,
                                           odt, fake, None, 0, None)

    assert merged(0) == -1 and merged(9) == -1  # shard count out of range
    assert merged(2, k=None) == -1  # NULL pointer array
    assert merged(2, hkv=3) == -1  # hq not a multiple of hkv
    assert merged(2, d=96) == -2  # unsupported head dim
    assert merged(2, hkv=8) == -2  # GQA group of 1: no merged walk
    assert merged(2, dt=1) == -2  # fp32 inputs: no merged walk


def test_paged_merged_call_validation_before_gpu(cpa):
    lib = cpa.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    arr = (ctypes.c_void_p * 16)(*([0x1000] * 16))

    def call(maxq=1, n=1, parts=arr, pdt=0, ws=fake, wsb=1 << 20, bs=16, rank=0):
        return lib.cpa_partial_attn_paged_merged(fake, fake, fake, fake, fake, fake, 8, fake, bs, 2, rank, 8, 2, maxq,
                                                 8, 2, 128, 0, 0.1, 1, n, parts, parts, pdt, None, None, fake, 0,
                                                 fake, ws, wsb, None)

    assert call(n=16) == -1 and call(n=-1) == -1  # part count out of range
    assert call(parts=None) == -1  # NULL part arrays
    assert call(pdt=5) == -1  # bad part dtype
    assert call(ws=None, wsb=0) == -3  # decode workspace missing
    assert call(bs=32) == -2 and call(rank=2) == -1  # the paged checks


def test_choose_pass_matches_oracle(cpa):
    """Host choice of the exchanged shard: bit-exact against the oracle on
    random batches, and the pages' two cases."""
    import oracle

    rng = np.random.default_rng(11)
    for _ in range(200):
        nb = int(rng.integers(0, 6))
        q = rng.integers(0, 9000, size=nb)
        kv = q + rng.integers(0, 70000, size=nb)
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.integers(1, 9))
        d, eb = int(rng.choice([64, 128])), int(rng.choice([1, 2, 4]))
        assert cpa.choose_pass(q, kv, hq, hkv, d, eb) == oracle.choose_pass(q, kv, hq, hkv, d, eb)
    assert cpa.choose_pass([6706], [6706], 16, 2, 128)["pass_kv"]  # full prefill, groups of 8
    assert not cpa.choose_pass([4096, 4096], [69632, 69632], 16, 2, 128)["pass_kv"]  # chunked, long cache


def test_choose_pass_errors(cpa):
    lib = cpa.load_library()
    pk = ctypes.c_int32(7)
    lens = (ctypes.c_int32 * 2)(5, -1)
    assert lib.cpa_choose_pass(2, lens, lens, 8, 2, 64, 2, ctypes.byref(pk), None, None) == -1  # negative length
    assert lib.cpa_choose_pass(1, None, lens, 8, 2, 64, 2, ctypes.byref(pk), None, None) == -1  # NULL array
    assert lib.cpa_choose_pass(1, lens, lens, 8, 0, 64, 2, ctypes.byref(pk), None, None) == -1  # hkv 0
    assert lib.cpa_choose_pass(0, None, None, 8, 2, 64, 2, None, None, None) == -1  # NULL result
    assert lib.cpa_choose_pass(0, None, None, 8, 2, 64, 2, ctypes.byref(pk), None, None) == 0 and pk.value == 0


def test_accumulate_call_validation_before_gpu(cpa):
    lib = cpa.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first

    def acc(o_acc=fake, lse_acc=fake, hkv=2, dt=0):
        return lib.cpa_partial_attn_accumulate(fake, fake, fake, fake, fake, fake, fake, 1, 4, 8, hkv, 128, dt, 0.1,
                                               1, o_acc, lse_acc, None, 0, None, 0, None)

    assert acc(o_acc=None) == -1 and acc(lse_acc=None) == -1  # NULL accumulator
    assert acc(hkv=3) == -1  # hq not a multiple of hkv
    assert acc(hkv=8) == -2  # GQA group of 1: not supported
    assert acc(dt=1) == -2  # fp32 inputs: not supported


def test_pass_cost_matches_oracle(cpa):
    """cpa_pass_cost against oracle.pass_cost: integers and flags bit-exact,
    the per-step figures to the last bit of a double (both sides compute the
    same correctly rounded quotients of exact integers)."""
    rng = np.random.default_rng(11)
    cases = [([131072], [131072], 32, 8, 128, 2, 4), ([4096, 4096], [69632, 69632], 16, 2, 128, 2, 4),
             ([1], [1], 8, 2, 64, 2, 2), ([0, 0], [5, 0], 4, 4, 64, 1, 3)]
    for _ in range(20):
        n = int(rng.integers(1, 5))
        kv = rng.integers(0, 20000, size=n)
        q = np.minimum(kv, rng.integers(0, 5000, size=n))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 8]))
        cases.append((q.tolist(), kv.tolist(), g * hkv, hkv, int(rng.choice([64, 128])), int(rng.choice([1, 2])),
                      int(rng.integers(1, 9))))
    for q, kv, hq, hkv, d, eb, cp in cases:
        for link, mfma in ((1.53e11, 1.25e15), (1e9, 1e12), (3e11, 7e14)):
            got = cpa.pass_cost(q, kv, hq, hkv, d, eb, cp, link, mfma)
            want = oracle.pass_cost(q, kv, hq, hkv, d, eb, cp, link, mfma)
            for key, val in want.items():
                assert got[key] == val, (key, got[key], val, q, kv, hq, hkv, d, eb, cp)


def test_pass_cost_errors(cpa):
    lib = cpa.load_library()
    r = cpa.binding.PassCost()
    lens = (ctypes.c_int32 * 1)(5)
    small = (ctypes.c_int32 * 1)(4)
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 2, 1e11, 1e15, None) == -1  # NULL out
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 0, 1e11, 1e15, ctypes.byref(r)) == -1  # cp 0
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 2, 0.0, 1e15, ctypes.byref(r)) == -1  # zero rate
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 2, float("nan"), 1e15, ctypes.byref(r)) == -1
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 2, 1e11, float("inf"), ctypes.byref(r)) == -1
    assert lib.cpa_pass_cost(1, lens, small, 8, 2, 64, 2, 2, 1e11, 1e15, ctypes.byref(r)) == -1  # q > kv
    assert lib.cpa_pass_cost(1, lens, lens, 8, 2, 64, 2, 2, 1e11, 1e15, ctypes.byref(r)) == 0
    assert r.pairs == 15
