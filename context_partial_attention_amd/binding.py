"""ctypes binding of libcpattn.so: argument marshalling only.

Names follow the C ABI (include/cpattn.h) without the `cpa_` prefix. Device
entry points take torch tensors (for their device pointers), enqueue on the
current torch stream and return without synchronising.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

BF16, F32 = 0, 1
MASK_NONE, MASK_CAUSAL = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcpattn.so")
_lib = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_f32 = ctypes.c_float
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class CpaError(RuntimeError):
    """A libcpattn call returned a negative status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libcpattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m context_partial_attention_amd.build`"
        )
    lib = ctypes.CDLL(_LIB_PATH)
    lib.cpa_last_error.restype = ctypes.c_char_p
    lib.cpa_last_error.argtypes = []
    lib.cpa_cp_partition.restype = _i32
    lib.cpa_cp_partition.argtypes = [_i32, _i32p, _i32, _i32, _i32p, _i32p, _i32p, _i32p, _i64, _i64p]
    lib.cpa_rr_placement.restype = _i32
    lib.cpa_rr_placement.argtypes = [_i32, _i32p, _i32, _i32, _i32, _i32p, _i32p, _i64, _i64p]
    lib.cpa_choose_pass.restype = _i32
    lib.cpa_choose_pass.argtypes = [_i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32p, _i64p, _i64p]
    lib.cpa_partial_attn.restype = _i32
    lib.cpa_partial_attn.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                     _p, _i32, _p, _p]
    lib.cpa_partial_attn_multi_workspace.restype = _i32
    lib.cpa_partial_attn_multi_workspace.argtypes = [_i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.cpa_partial_attn_multi.restype = _i32
    lib.cpa_partial_attn_multi.argtypes = [_i32, _p, _p, _p, ctypes.POINTER(_p), ctypes.POINTER(_p),
                                           ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i32, _i32, _i32, _i32,
                                           _i32, _f32, _i32, ctypes.POINTER(_p), _i32, ctypes.POINTER(_p), _p,
                                           ctypes.c_size_t, _p]
    lib.cpa_partial_attn_merged.restype = _i32
    lib.cpa_partial_attn_merged.argtypes = [_i32, _p, _p, _p, ctypes.POINTER(_p), ctypes.POINTER(_p),
                                            ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _i32, _p, _i32, _p, _p, ctypes.c_size_t, _p]
    lib.cpa_partial_attn_accumulate.restype = _i32
    lib.cpa_partial_attn_accumulate.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                _i32, _p, _p, _p, _i32, _p]
    lib.cpa_partial_attn_paged_workspace.restype = _i32
    lib.cpa_partial_attn_paged_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.cpa_partial_attn_paged.restype = _i32
    lib.cpa_partial_attn_paged.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _f32, _i32, _p, _i32, _p, _p, ctypes.c_size_t,
                                           _p]
    lib.cpa_lse_merge.restype = _i32
    lib.cpa_lse_merge.argtypes = [_i32, ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i64, _i32, _p, _i32, _p, _p]
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = load_library().cpa_last_error().decode(errors="replace")
        raise CpaError(fn, status, msg)


def _i32_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_i32p)


# ----------------------------------------------------------------- host calls


def cp_partition(seq_lens, cp_size: int, rank: int) -> dict:
    """Zigzag shard of `rank`: chunk_bounds, cu_seqlens, positions, src_index (int32)."""
    lib = load_library()
    lens = _i32_array(seq_lens)
    nseq = len(lens)
    n = ctypes.c_int64(0)
    bounds = np.zeros((nseq, 2 * cp_size + 1), dtype=np.int32) if cp_size >= 1 else None
    cu = np.zeros(nseq + 1, dtype=np.int32)
    _check("cpa_cp_partition", lib.cpa_cp_partition(nseq, _ptr(lens), cp_size, rank, _ptr(bounds), _ptr(cu),
                                                    None, None, 0, ctypes.byref(n)))
    pos = np.zeros(n.value, dtype=np.int32)
    src = np.zeros(n.value, dtype=np.int32)
    _check("cpa_cp_partition", lib.cpa_cp_partition(nseq, _ptr(lens), cp_size, rank, _ptr(bounds), _ptr(cu),
                                                    _ptr(pos), _ptr(src), n.value, ctypes.byref(n)))
    return {"chunk_bounds": bounds, "cu_seqlens": cu, "positions": pos, "src_index": src}


def rr_placement(seq_lens, cp_size: int, rank: int, interleave: int) -> dict:
    """Round-robin placement of `rank`: local_lens, cu_local, local_to_global (int32)."""
    lib = load_library()
    lens = _i32_array(seq_lens)
    nseq = len(lens)
    n = ctypes.c_int64(0)
    local = np.zeros(nseq, dtype=np.int32)
    _check("cpa_rr_placement", lib.cpa_rr_placement(nseq, _ptr(lens), cp_size, rank, interleave, _ptr(local),
                                                    None, 0, ctypes.byref(n)))
    l2g = np.zeros(n.value, dtype=np.int32)
    _check("cpa_rr_placement", lib.cpa_rr_placement(nseq, _ptr(lens), cp_size, rank, interleave, _ptr(local),
                                                    _ptr(l2g), n.value, ctypes.byref(n)))
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(local)
    return {"local_lens": local, "cu_local": cu, "local_to_global": l2g}


def choose_pass(q_lens, kv_lens, hq: int, hkv: int, d: int, elem_bytes: int = 2) -> dict:
    """Pass KV or pass Q for a prefill batch: {"pass_kv", "kv_bytes", "q_bytes"}."""
    lib = load_library()
    ql, kl = _i32_array(q_lens), _i32_array(kv_lens)
    if len(ql) != len(kl):
        raise ValueError("q_lens and kv_lens need one entry per sequence")
    pk = ctypes.c_int32(0)
    kvb, qb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("cpa_choose_pass", lib.cpa_choose_pass(len(ql), _ptr(ql), _ptr(kl), hq, hkv, d, elem_bytes,
                                                  ctypes.byref(pk), ctypes.byref(kvb), ctypes.byref(qb)))
    return {"pass_kv": bool(pk.value), "kv_bytes": kvb.value, "q_bytes": qb.value}


# --------------------------------------------------------------- device calls


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def partial_attn(q, q_pos, cu_q, k, v, k_pos, cu_k, max_q: int, scale: float, causal: bool = True,
                 out=None, lse=None, out_dtype=None, stream=None):
    """One pass-KV step: q [Tq,hq,d] against contiguous k, v [Tk,hkv,d]. Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = q.shape
    hkv = k.shape[1]
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    num_seqs = cu_q.numel() - 1
    lib = load_library()
    _check("cpa_partial_attn", lib.cpa_partial_attn(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k, "k"), _dev(v, "v"), _dev(k_pos, "k_pos"),
        _dev(cu_k, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
        _stream(stream)))
    return out, lse


def partial_attn_multi_workspace(n_shards: int, num_seqs: int, max_q: int) -> int:
    """Bytes of the launch-order workspace of partial_attn_multi (0: none used)."""
    n = ctypes.c_size_t(0)
    _check("cpa_partial_attn_multi_workspace",
           load_library().cpa_partial_attn_multi_workspace(n_shards, num_seqs, int(max_q), ctypes.byref(n)))
    return n.value


def partial_attn_multi(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, max_q: int, scale: float, causal: bool = True,
                       outs=None, lses=None, out_dtype=None, workspace=None, stream=None):
    """Several pass-KV steps at once: q against each resident shard (ks[i], vs[i], k_poss[i], cu_ks[i]).
    `workspace` (a uint8 GPU tensor of partial_attn_multi_workspace() bytes, or None) enables the
    heaviest-tile-first launch order. Returns the lists (outs, lses), one partial per shard."""
    torch = _torch()
    tq, hq, d = q.shape
    n = len(ks)
    hkv = ks[0].shape[1]
    out_dtype = out_dtype or torch.float32
    if outs is None:
        outs = [torch.empty((tq, hq, d), dtype=out_dtype, device=q.device) for _ in range(n)]
    if lses is None:
        lses = [torch.empty((tq, hq), dtype=torch.float32, device=q.device) for _ in range(n)]
    if not (len(vs) == len(k_poss) == len(cu_ks) == len(outs) == len(lses) == n):
        raise ValueError("every per-shard list needs one entry per shard")
    arr = lambda ts, name: (_p * n)(*[_dev(t, name) for t in ts])  # noqa: E731
    num_seqs = cu_q.numel() - 1
    _check("cpa_partial_attn_multi", load_library().cpa_partial_attn_multi(
        n, _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), arr(ks, "k"), arr(vs, "v"), arr(k_poss, "k_pos"),
        arr(cu_ks, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, arr(outs, "out"), _dtype_code(outs[0]), arr(lses, "lse"),
        _dev(workspace, "workspace"), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return outs, lses


def partial_attn_merged(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, max_q: int, scale: float, causal: bool = True,
                        out=None, lse=None, out_dtype=None, workspace=None, stream=None):
    """The merged pass-KV result over resident shards (ks[i], vs[i], k_poss[i], cu_ks[i]) in one walk.
    `workspace` as for partial_attn_multi. Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = q.shape
    n = len(ks)
    hkv = ks[0].shape[1]
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    if not (len(vs) == len(k_poss) == len(cu_ks) == n):
        raise ValueError("every per-shard list needs one entry per shard")
    arr = lambda ts, name: (_p * n)(*[_dev(t, name) for t in ts])  # noqa: E731
    num_seqs = cu_q.numel() - 1
    _check("cpa_partial_attn_merged", load_library().cpa_partial_attn_merged(
        n, _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), arr(ks, "k"), arr(vs, "v"), arr(k_poss, "k_pos"),
        arr(cu_ks, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
        _dev(workspace, "workspace"), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out, lse


def partial_attn_accumulate(q, q_pos, cu_q, k, v, k_pos, cu_k, max_q: int, scale: float, o_acc, lse_acc,
                            causal: bool = True, out=None, stream=None):
    """One pass-KV step folded into the running (o_acc, lse_acc) (fp32, in place); `out`, if given,
    also receives the merged O (bf16 or fp32). Returns (o_acc, lse_acc)."""
    tq, hq, d = q.shape
    hkv = k.shape[1]
    num_seqs = cu_q.numel() - 1
    _check("cpa_partial_attn_accumulate", load_library().cpa_partial_attn_accumulate(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k, "k"), _dev(v, "v"), _dev(k_pos, "k_pos"),
        _dev(cu_k, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc"), _dev(out, "out"),
        F32 if out is None else _dtype_code(out), _stream(stream)))
    return o_acc, lse_acc


def partial_attn_paged_workspace(num_seqs: int, max_q: int, max_blocks: int, block_size: int, hq: int,
                                 d: int) -> int:
    n = ctypes.c_size_t(0)
    _check("cpa_partial_attn_paged_workspace", load_library().cpa_partial_attn_paged_workspace(
        num_seqs, max_q, max_blocks, block_size, hq, d, ctypes.byref(n)))
    return n.value


def partial_attn_paged(q, q_pos, cu_q, k_cache, v_cache, block_table, local_kv_lens, cp_size: int, cp_rank: int,
                       interleave: int, max_q: int, scale: float, causal: bool = True, out=None, lse=None,
                       out_dtype=None, workspace=None, stream=None):
    """Q against one rank's paged round-robin KV shard (k/v cache [blocks,hkv,16,d]). Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = q.shape
    hkv, block_size = k_cache.shape[1], k_cache.shape[2]
    num_seqs = cu_q.numel() - 1
    max_blocks = block_table.shape[1]
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    need = partial_attn_paged_workspace(num_seqs, int(max_q), max_blocks, block_size, hq, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check("cpa_partial_attn_paged", lib.cpa_partial_attn_paged(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), max_blocks, _dev(local_kv_lens, "local_kv_lens"), block_size, cp_size,
        cp_rank, interleave, num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
        _dev(workspace, "workspace"), ws_bytes, _stream(stream)))
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse_out=None, out_dtype=None, stream=None):
    """Exact merge of partials o_parts[s] [..., d], lse_parts[s] [...]. Returns (o, lse)."""
    torch = _torch()
    n = len(o_parts)
    if n != len(lse_parts) or n == 0:
        raise ValueError("need the same, non-zero number of O and LSE parts")
    o0 = o_parts[0]
    d = o0.shape[-1]
    rows = o0.numel() // d
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(o0.shape, dtype=out_dtype, device=o0.device)
    if lse_out is None:
        lse_out = torch.empty(o0.shape[:-1], dtype=torch.float32, device=o0.device)
    for o, l in zip(o_parts, lse_parts):
        if o.numel() != rows * d or l.numel() != rows or o.dtype != o0.dtype or l.dtype != torch.float32:
            raise ValueError("every part must have the same shape and dtype; LSE parts are float32")
    optrs = (_p * n)(*[_dev(o, "o_part") for o in o_parts])
    lptrs = (_p * n)(*[_dev(l, "lse_part") for l in lse_parts])
    _check("cpa_lse_merge", load_library().cpa_lse_merge(
        n, optrs, lptrs, _dtype_code(o0), rows, d, _dev(out, "out"), _dtype_code(out), _dev(lse_out, "lse_out"),
        _stream(stream)))
    return out, lse_out
