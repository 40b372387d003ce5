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


class PassCost(ctypes.Structure):
    """cpa_pass_cost_t."""

    _fields_ = [("pass_kv", _i32), ("kv_hidden", _i32), ("q_hidden", _i32), ("kv_bytes", _i64),
                ("q_bytes", _i64), ("pairs", _i64), ("kv_step_bytes", ctypes.c_double),
                ("q_step_bytes", ctypes.c_double), ("step_flops", ctypes.c_double),
                ("kv_transfer_s", ctypes.c_double), ("q_transfer_s", ctypes.c_double),
                ("step_compute_s", ctypes.c_double)]


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
    lib.cpa_pass_cost.restype = _i32
    lib.cpa_pass_cost.argtypes = [_i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, ctypes.c_double,
                                  ctypes.c_double, ctypes.POINTER(PassCost)]
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
    lib.cpa_partial_attn_multi_noalloc.restype = _i32
    lib.cpa_partial_attn_multi_noalloc.argtypes = [_i32, _p, _p, _p, ctypes.POINTER(_p), ctypes.POINTER(_p),
                                                   ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _f32, _i32, ctypes.POINTER(_p), _i32,
                                                   ctypes.POINTER(_p), _p]
    lib.cpa_partial_attn_merged.restype = _i32
    lib.cpa_partial_attn_merged.argtypes = [_i32, _p, _p, _p, ctypes.POINTER(_p), ctypes.POINTER(_p),
                                            ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _i32, _p, _i32, _p, _p, ctypes.c_size_t, _p]
    lib.cpa_partial_attn_accumulate.restype = _i32
    lib.cpa_partial_attn_accumulate.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                _i32, _p, _p, _p, _i32, _p, ctypes.c_size_t, _p]
    lib.cpa_partial_attn_paged_workspace.restype = _i32
    lib.cpa_partial_attn_paged_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.cpa_partial_attn_paged.restype = _i32
    lib.cpa_partial_attn_paged.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _f32, _i32, _p, _i32, _p, _p, ctypes.c_size_t,
                                           _p]
    lib.cpa_partial_attn_paged_merged.restype = _i32
    lib.cpa_partial_attn_paged_merged.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, ctypes.POINTER(_p),
                                                  ctypes.POINTER(_p), _i32, _p, _p, _p, _i32, _p, _p,
                                                  ctypes.c_size_t, _p]
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


def pass_cost(q_lens, kv_lens, hq: int, hkv: int, d: int, elem_bytes: int, cp_size: int,
              link_bytes_per_s: float, mfma_flops_per_s: float) -> dict:
    """Per-step transfer and compute of pass-KV and pass-Q for a prefill batch
    (every field of cpa_pass_cost_t; the flags as bools)."""
    lib = load_library()
    ql, kl = _i32_array(q_lens), _i32_array(kv_lens)
    if len(ql) != len(kl):
        raise ValueError("q_lens and kv_lens need one entry per sequence")
    r = PassCost()
    _check("cpa_pass_cost", lib.cpa_pass_cost(len(ql), _ptr(ql), _ptr(kl), hq, hkv, d, elem_bytes, cp_size,
                                              float(link_bytes_per_s), float(mfma_flops_per_s), ctypes.byref(r)))
    out = {name: getattr(r, name) for name, _ in PassCost._fields_}
    for flag in ("pass_kv", "kv_hidden", "q_hidden"):
        out[flag] = bool(out[flag])
    return out


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


# Shape and dtype checks of the device arguments. The library sees only
# pointers and sizes, so it cannot tell a mis-sized or mis-typed tensor from a
# good one; these run before any pointer is passed (and before the GPU check,
# so they also hold for tensors on the CPU). Values stored in device memory
# (offsets, positions, block-table entries) are not read here.


def _shape(t, name: str, shape: tuple, dtypes):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} has dtype {str(t.dtype).replace('torch.', '')}, expected {want}")
    del torch


def _same_device(*named):
    devs = {(n, t.device) for n, t in named if t is not None}
    if len({d for _, d in devs}) > 1:
        raise ValueError("tensors are on different devices: " + ", ".join(f"{n}={d}" for n, d in sorted(devs)))


def _check_q(q):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError(f"q must be [tokens, hq, d], got shape {tuple(q.shape)}")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q has dtype {q.dtype}, expected bfloat16 or float32")
    return q.shape


def _check_kv(q, k, v, kname: str = "k", vname: str = "v"):
    tq, hq, d = q.shape
    if k.dim() != 3 or k.shape[2] != d:
        raise ValueError(f"{kname} must be [tokens, hkv, {d}], got shape {tuple(k.shape)}")
    hkv = k.shape[1]
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"{kname}: hq ({hq}) must be a multiple of hkv ({hkv})")
    _shape(k, kname, k.shape, q.dtype)
    _shape(v, vname, k.shape, q.dtype)
    return hkv


def _check_seq_index(q, q_pos, cu_q, causal: bool):
    torch = _torch()
    tq = q.shape[0]
    if cu_q is None or cu_q.dim() != 1 or cu_q.numel() < 1:
        raise ValueError("cu_q must be a 1-D int32 tensor of num_seqs + 1 offsets")
    _shape(cu_q, "cu_q", cu_q.shape, torch.int32)
    if causal or q_pos is not None:
        _shape(q_pos, "q_pos", (tq,), torch.int32)
    return cu_q.numel() - 1


def _check_outputs(q, out, lse, name_o: str = "out", name_lse: str = "lse"):
    torch = _torch()
    tq, hq, d = q.shape
    _shape(out, name_o, (tq, hq, d), (torch.float32, torch.bfloat16))
    _shape(lse, name_lse, (tq, hq), torch.float32)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def partial_attn(q, q_pos, cu_q, k, v, k_pos, cu_k, max_q: int, scale: float, causal: bool = True,
                 out=None, lse=None, out_dtype=None, stream=None):
    """One pass-KV step: q [Tq,hq,d] against contiguous k, v [Tk,hkv,d]. Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    hkv = _check_kv(q, k, v)
    num_seqs = _check_seq_index(q, q_pos, cu_q, causal)
    _shape(cu_k, "cu_k", (num_seqs + 1,), torch.int32)
    if causal or k_pos is not None:
        _shape(k_pos, "k_pos", (k.shape[0],), torch.int32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_outputs(q, out, lse)
    _same_device(("q", q), ("q_pos", q_pos), ("cu_q", cu_q), ("k", k), ("v", v), ("k_pos", k_pos), ("cu_k", cu_k),
                 ("out", out), ("lse", lse))
    lib = load_library()
    _check("cpa_partial_attn", lib.cpa_partial_attn(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k, "k"), _dev(v, "v"), _dev(k_pos, "k_pos"),
        _dev(cu_k, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
        _stream(stream)))
    return out, lse


def _check_shards(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, causal: bool):
    """Shapes and dtypes of the per-shard lists of the batched calls."""
    torch = _torch()
    if len(ks) < 1:
        raise ValueError("need at least one KV shard")
    if not (len(vs) == len(k_poss) == len(cu_ks) == len(ks)):
        raise ValueError("every per-shard list needs one entry per shard")
    num_seqs = _check_seq_index(q, q_pos, cu_q, causal)
    hkv = None
    for i in range(len(ks)):
        h = _check_kv(q, ks[i], vs[i], f"ks[{i}]", f"vs[{i}]")
        if hkv is not None and h != hkv:
            raise ValueError("every shard needs the same number of KV heads")
        hkv = h
        _shape(cu_ks[i], f"cu_ks[{i}]", (num_seqs + 1,), torch.int32)
        if causal or k_poss[i] is not None:
            _shape(k_poss[i], f"k_poss[{i}]", (ks[i].shape[0],), torch.int32)
        _same_device(("q", q), ("q_pos", q_pos), ("cu_q", cu_q), (f"ks[{i}]", ks[i]), (f"vs[{i}]", vs[i]),
                     (f"k_poss[{i}]", k_poss[i]), (f"cu_ks[{i}]", cu_ks[i]))
    return hkv, num_seqs


def _check_workspace(workspace):
    torch = _torch()
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.dim() != 1):
        raise ValueError("workspace must be a 1-D uint8 tensor")


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
    tq, hq, d = _check_q(q)
    n = len(ks)
    out_dtype = out_dtype or torch.float32
    if outs is None:
        outs = [torch.empty((tq, hq, d), dtype=out_dtype, device=q.device) for _ in range(n)]
    if lses is None:
        lses = [torch.empty((tq, hq), dtype=torch.float32, device=q.device) for _ in range(n)]
    if not (len(vs) == len(k_poss) == len(cu_ks) == len(outs) == len(lses) == n):
        raise ValueError("every per-shard list needs one entry per shard")
    hkv, num_seqs = _check_shards(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, causal)
    for i in range(n):
        _check_outputs(q, outs[i], lses[i], f"outs[{i}]", f"lses[{i}]")
        if outs[i].dtype != outs[0].dtype:
            raise ValueError("every partial output needs the same dtype")
    _check_workspace(workspace)
    _same_device(("q", q), ("workspace", workspace), *[(f"outs[{i}]", t) for i, t in enumerate(outs)],
                 *[(f"lses[{i}]", t) for i, t in enumerate(lses)])
    arr = lambda ts, name: (_p * n)(*[_dev(t, name) for t in ts])  # noqa: E731
    _check("cpa_partial_attn_multi", load_library().cpa_partial_attn_multi(
        n, _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), arr(ks, "k"), arr(vs, "v"), arr(k_poss, "k_pos"),
        arr(cu_ks, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, arr(outs, "out"), _dtype_code(outs[0]), arr(lses, "lse"),
        _dev(workspace, "workspace"), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return outs, lses


def partial_attn_multi_noalloc(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, max_q: int, scale: float, outs, lses,
                               causal: bool = True, stream=None):
    """partial_attn_multi without any allocation: the launch order lives in the
    library's own device scratch (at most 8192 tile units). The caller passes
    every output (outs[i], lses[i]). Returns (outs, lses)."""
    tq, hq, d = _check_q(q)
    n = len(ks)
    if outs is None or lses is None or len(outs) != n or len(lses) != n:
        raise ValueError("the no-allocation call needs one caller-allocated output and LSE per shard")
    hkv, num_seqs = _check_shards(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, causal)
    for i in range(n):
        _check_outputs(q, outs[i], lses[i], f"outs[{i}]", f"lses[{i}]")
        if outs[i].dtype != outs[0].dtype:
            raise ValueError("every partial output needs the same dtype")
    _same_device(("q", q), *[(f"outs[{i}]", t) for i, t in enumerate(outs)],
                 *[(f"lses[{i}]", t) for i, t in enumerate(lses)])
    arr = lambda ts, name: (_p * n)(*[_dev(t, name) for t in ts])  # noqa: E731
    _check("cpa_partial_attn_multi_noalloc", load_library().cpa_partial_attn_multi_noalloc(
        n, _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), arr(ks, "k"), arr(vs, "v"), arr(k_poss, "k_pos"),
        arr(cu_ks, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, arr(outs, "out"), _dtype_code(outs[0]), arr(lses, "lse"),
        _stream(stream)))
    return outs, lses


def partial_attn_merged(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, max_q: int, scale: float, causal: bool = True,
                        out=None, lse=None, out_dtype=None, workspace=None, stream=None):
    """The merged pass-KV result over resident shards (ks[i], vs[i], k_poss[i], cu_ks[i]) in one walk.
    `workspace` as for partial_attn_multi. Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    n = len(ks)
    hkv, num_seqs = _check_shards(q, q_pos, cu_q, ks, vs, k_poss, cu_ks, causal)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_outputs(q, out, lse)
    _check_workspace(workspace)
    _same_device(("q", q), ("out", out), ("lse", lse), ("workspace", workspace))
    arr = lambda ts, name: (_p * n)(*[_dev(t, name) for t in ts])  # noqa: E731
    _check("cpa_partial_attn_merged", load_library().cpa_partial_attn_merged(
        n, _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), arr(ks, "k"), arr(vs, "v"), arr(k_poss, "k_pos"),
        arr(cu_ks, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
        _dev(workspace, "workspace"), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out, lse


def partial_attn_accumulate(q, q_pos, cu_q, k, v, k_pos, cu_k, max_q: int, scale: float, o_acc, lse_acc,
                            causal: bool = True, out=None, workspace=None, stream=None):
    """One pass-KV step folded into the running (o_acc, lse_acc) (fp32, in place); `out`, if given,
    also receives the merged O (bf16 or fp32). `workspace` (a uint8 GPU tensor of at least
    partial_attn_multi_workspace(1, ...) bytes, or None) enables the heaviest-first launch order.
    Returns (o_acc, lse_acc)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    hkv = _check_kv(q, k, v)
    num_seqs = _check_seq_index(q, q_pos, cu_q, causal)
    _shape(cu_k, "cu_k", (num_seqs + 1,), torch.int32)
    if causal or k_pos is not None:
        _shape(k_pos, "k_pos", (k.shape[0],), torch.int32)
    _shape(o_acc, "o_acc", (tq, hq, d), torch.float32)
    _shape(lse_acc, "lse_acc", (tq, hq), torch.float32)
    if out is not None:
        _shape(out, "out", (tq, hq, d), (torch.float32, torch.bfloat16))
    _check_workspace(workspace)
    _same_device(("q", q), ("q_pos", q_pos), ("cu_q", cu_q), ("k", k), ("v", v), ("k_pos", k_pos), ("cu_k", cu_k),
                 ("o_acc", o_acc), ("lse_acc", lse_acc), ("out", out), ("workspace", workspace))
    _check("cpa_partial_attn_accumulate", load_library().cpa_partial_attn_accumulate(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k, "k"), _dev(v, "v"), _dev(k_pos, "k_pos"),
        _dev(cu_k, "cu_k"), num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, _dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc"), _dev(out, "out"),
        F32 if out is None else _dtype_code(out), _dev(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return o_acc, lse_acc


def partial_attn_paged_workspace(num_seqs: int, max_q: int, max_blocks: int, block_size: int, hq: int,
                                 d: int) -> int:
    n = ctypes.c_size_t(0)
    _check("cpa_partial_attn_paged_workspace", load_library().cpa_partial_attn_paged_workspace(
        num_seqs, max_q, max_blocks, block_size, hq, d, ctypes.byref(n)))
    return n.value


def _check_paged(q, q_pos, cu_q, k_cache, v_cache, block_table, local_kv_lens, causal):
    """Validates the paged-shard arguments; returns (num_seqs, hkv, block_size, max_blocks)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    if k_cache.dim() != 4 or k_cache.shape[3] != d:
        raise ValueError(f"k_cache must be [blocks, hkv, block_size, {d}], got shape {tuple(k_cache.shape)}")
    hkv, block_size = k_cache.shape[1], k_cache.shape[2]
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"k_cache: hq ({hq}) must be a multiple of hkv ({hkv})")
    _shape(k_cache, "k_cache", k_cache.shape, q.dtype)
    _shape(v_cache, "v_cache", k_cache.shape, q.dtype)
    num_seqs = _check_seq_index(q, q_pos, cu_q, causal)
    if block_table is None or block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError(f"block_table must be [num_seqs={num_seqs}, max_blocks] int32")
    _shape(block_table, "block_table", block_table.shape, torch.int32)
    _shape(local_kv_lens, "local_kv_lens", (num_seqs,), torch.int32)
    return num_seqs, hkv, block_size, block_table.shape[1]


def partial_attn_paged(q, q_pos, cu_q, k_cache, v_cache, block_table, local_kv_lens, cp_size: int, cp_rank: int,
                       interleave: int, max_q: int, scale: float, causal: bool = True, out=None, lse=None,
                       out_dtype=None, workspace=None, stream=None):
    """Q against one rank's paged round-robin KV shard (k/v cache [blocks,hkv,16,d]). Returns (o, lse)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    num_seqs, hkv, block_size, max_blocks = _check_paged(q, q_pos, cu_q, k_cache, v_cache, block_table,
                                                         local_kv_lens, causal)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_outputs(q, out, lse)
    _check_workspace(workspace)
    _same_device(("q", q), ("q_pos", q_pos), ("cu_q", cu_q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_table", block_table), ("local_kv_lens", local_kv_lens), ("out", out), ("lse", lse),
                 ("workspace", workspace))
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


def partial_attn_paged_merged(q, q_pos, cu_q, k_cache, v_cache, block_table, local_kv_lens, cp_size: int,
                              cp_rank: int, interleave: int, max_q: int, scale: float, o_parts, lse_parts,
                              causal: bool = True, out=None, lse=None, out_dtype=None, own_out=None, own_lse=None,
                              workspace=None, stream=None):
    """This rank's partial against its paged shard (decode, or pass-Q prefill
    with an even GQA group), merged in the same call with the other ranks'
    partials o_parts[j] [Tq,hq,d], lse_parts[j] [Tq,hq]. own_out / own_lse
    (optional) receive this rank's own partial in the parts' dtype. Returns
    (o, lse)."""
    torch = _torch()
    tq, hq, d = _check_q(q)
    num_seqs, hkv, block_size, max_blocks = _check_paged(q, q_pos, cu_q, k_cache, v_cache, block_table,
                                                         local_kv_lens, causal)
    n = len(o_parts)
    if n != len(lse_parts) or n > 15:
        raise ValueError("need the same number (at most 15) of O and LSE parts")
    part_dtype = o_parts[0].dtype if n else (own_out.dtype if own_out is not None else torch.float32)
    if part_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"O parts have dtype {part_dtype}, expected float32 or bfloat16")
    for j in range(n):
        _shape(o_parts[j], f"o_parts[{j}]", (tq, hq, d), part_dtype)
        _shape(lse_parts[j], f"lse_parts[{j}]", (tq, hq), torch.float32)
    if own_out is not None:
        _shape(own_out, "own_out", (tq, hq, d), part_dtype)
    if own_lse is not None:
        _shape(own_lse, "own_lse", (tq, hq), torch.float32)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_outputs(q, out, lse)
    _check_workspace(workspace)
    _same_device(("q", q), ("q_pos", q_pos), ("cu_q", cu_q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_table", block_table), ("local_kv_lens", local_kv_lens), ("out", out), ("lse", lse),
                 ("workspace", workspace), ("own_out", own_out), ("own_lse", own_lse),
                 *[(f"o_parts[{j}]", t) for j, t in enumerate(o_parts)],
                 *[(f"lse_parts[{j}]", t) for j, t in enumerate(lse_parts)])
    need = partial_attn_paged_workspace(num_seqs, int(max_q), max_blocks, block_size, hq, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    optrs = (_p * max(n, 1))(*[_dev(o, "o_part") for o in o_parts])
    lptrs = (_p * max(n, 1))(*[_dev(t, "lse_part") for t in lse_parts])
    lib = load_library()
    _check("cpa_partial_attn_paged_merged", lib.cpa_partial_attn_paged_merged(
        _dev(q, "q"), _dev(q_pos, "q_pos"), _dev(cu_q, "cu_q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), max_blocks, _dev(local_kv_lens, "local_kv_lens"), block_size, cp_size,
        cp_rank, interleave, num_seqs, int(max_q), hq, hkv, d, _dtype_code(q), float(scale),
        MASK_CAUSAL if causal else MASK_NONE, n, optrs, lptrs,
        BF16 if part_dtype == torch.bfloat16 else F32,
        None if own_out is None else _dev(own_out, "own_out"), None if own_lse is None else _dev(own_lse, "own_lse"),
        _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"), _dev(workspace, "workspace"), ws_bytes,
        _stream(stream)))
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
    if o0.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"O parts have dtype {o0.dtype}, expected float32 or bfloat16")
    for o, l in zip(o_parts, lse_parts):
        if tuple(o.shape) != tuple(o0.shape) or l.numel() != rows or o.dtype != o0.dtype or l.dtype != torch.float32:
            raise ValueError("every part must have the same shape and dtype; LSE parts are float32")
    _shape(out, "out", tuple(o0.shape), (torch.float32, torch.bfloat16))
    if lse_out.numel() != rows or lse_out.dtype != torch.float32:
        raise ValueError(f"lse_out must hold {rows} float32 values")
    _same_device(*[(f"o_parts[{i}]", t) for i, t in enumerate(o_parts)],
                 *[(f"lse_parts[{i}]", t) for i, t in enumerate(lse_parts)], ("out", out), ("lse_out", lse_out))
    optrs = (_p * n)(*[_dev(o, "o_part") for o in o_parts])
    lptrs = (_p * n)(*[_dev(l, "lse_part") for l in lse_parts])
    _check("cpa_lse_merge", load_library().cpa_lse_merge(
        n, optrs, lptrs, _dtype_code(o0), rows, d, _dev(out, "out"), _dtype_code(out), _dev(lse_out, "lse_out"),
        _stream(stream)))
    return out, lse_out
