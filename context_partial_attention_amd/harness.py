"""Device-side setup and step runners for the five workloads (HIP path only).

Builds the inputs one CP rank holds, through the library's own host calls
(cp_partition, rr_placement) plus torch gathers and scatters for the data
movement, and runs the hot path of each schedule:

  pass_kv  one partial per KV shard (the rank's own shard first, then ranks
           r-1, r-2, ... mod cp), then the cp-way merge
  pass_q   one partial of all new queries per rank's paged round-robin shard
           (every rank's pool resident in this GPU's memory)
  decode   one partial per rank's paged round-robin shard for the single query
           of every sequence
  (paged)  the rank's own partial is merged with the other ranks' (resident)
           partials inside its own launches (pass-Q: the prefill kernel's
           epilogue; decode: the decode merge kernel)

The CPU oracle never sees anything built here except the raw draws of
workloads.draw_sequence, which both sides share.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as cpa
from .workloads import Workload, block_permutation, draw_sequence, query_rows, seq_lengths


def _i32(x, device):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def build(w: Workload, device="cuda", keep_full: bool = True, pool_fill: float = 0.0) -> dict:
    """Draws the workload on `device` and lays out what the rank computes on.

    pool_fill is written into every paged-cache slot before the tokens are
    scattered in (NaN makes any read of an unused slot visible in results).
    """
    lens = seq_lengths(w)
    draws = []
    for b, L in enumerate(lens):
        draws.append(draw_sequence(w, b, L, query_rows(w, L), device=device))
    out = {"workload": w, "lens": lens, "device": device}
    if keep_full:
        out["draws"] = draws
    if w.kind == "pass_kv":
        _build_pass_kv(w, lens, draws, device, out)
    else:
        _build_paged(w, lens, draws, device, out, pool_fill)
    return out


def _build_pass_kv(w, lens, draws, device, out):
    q_full = torch.cat([d[0] for d in draws])
    k_full = torch.cat([d[1] for d in draws])
    v_full = torch.cat([d[2] for d in draws])
    mine = cpa.cp_partition(lens, w.cp, w.rank)
    src = torch.as_tensor(mine["src_index"].astype(np.int64), device=device)
    out["q"] = q_full.index_select(0, src).contiguous()
    out["q_pos"] = _i32(mine["positions"], device)
    out["cu_q"] = _i32(mine["cu_seqlens"], device)
    out["q_positions_host"] = mine["positions"]
    out["cu_q_host"] = mine["cu_seqlens"]
    out["max_q"] = int(np.max(np.diff(mine["cu_seqlens"]))) if len(lens) else 0
    steps = []
    for s in range(w.cp):
        r = (w.rank - s) % w.cp
        part = cpa.cp_partition(lens, w.cp, r)
        sidx = torch.as_tensor(part["src_index"].astype(np.int64), device=device)
        steps.append({
            "src_rank": r,
            "k": k_full.index_select(0, sidx).contiguous(),
            "v": v_full.index_select(0, sidx).contiguous(),
            "k_pos": _i32(part["positions"], device),
            "cu_k": _i32(part["cu_seqlens"], device),
            "k_positions_host": part["positions"],
            "cu_k_host": part["cu_seqlens"],
        })
    out["steps"] = steps


def _build_paged(w, lens, draws, device, out, pool_fill):
    bs = w.block_size
    if w.kind == "pass_q":
        qpos = [np.arange(L - w.new, L) for L in lens]
    else:
        qpos = [np.array([L - 1]) for L in lens]
    out["q"] = torch.cat([d[0] for d in draws]).contiguous()
    qp = np.concatenate(qpos).astype(np.int32)
    out["q_pos"] = _i32(qp, device)
    cu = np.concatenate([[0], np.cumsum([len(p) for p in qpos])]).astype(np.int32)
    out["cu_q"] = _i32(cu, device)
    out["q_positions_host"] = qp
    out["cu_q_host"] = cu
    out["max_q"] = int(max(len(p) for p in qpos))
    ranks = []
    for r in range(w.cp):
        pl = cpa.rr_placement(lens, w.cp, r, w.interleave)
        local = pl["local_lens"].astype(np.int64)
        nblk = (local + bs - 1) // bs
        max_blocks = int(nblk.max()) if len(nblk) else 0
        total = int(nblk.sum())
        perm = block_permutation(w, total, r).numpy()
        table = np.zeros((len(lens), max_blocks), dtype=np.int32)
        off = 0
        for b in range(len(lens)):
            table[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += nblk[b]
        kc = torch.full((total, w.hkv, bs, w.d), pool_fill, dtype=w.dtype, device=device)
        vc = torch.full((total, w.hkv, bs, w.d), pool_fill, dtype=w.dtype, device=device)
        tab_dev = torch.as_tensor(table, device=device)
        for b in range(len(lens)):
            a, e = int(pl["cu_local"][b]), int(pl["cu_local"][b + 1])
            t = torch.as_tensor(pl["local_to_global"][a:e].astype(np.int64), device=device)
            slots = torch.arange(e - a, device=device)
            blk = tab_dev[b].long()[slots // bs]
            kc[blk, :, slots % bs, :] = draws[b][1].index_select(0, t)
            vc[blk, :, slots % bs, :] = draws[b][2].index_select(0, t)
        ranks.append({
            "rank": r,
            "k_cache": kc,
            "v_cache": vc,
            "block_table": tab_dev,
            "local_kv_lens": _i32(pl["local_lens"], device),
            "local_lens_host": pl["local_lens"],
            "local_to_global_host": pl["local_to_global"],
            "cu_local_host": pl["cu_local"],
        })
    out["ranks"] = ranks


class Runner:
    """Preallocated outputs and the step of one workload's hot path."""

    def __init__(self, inp: dict, merged_dtype=None):
        self.inp = inp
        w = inp["workload"]
        self.w = w
        dev = inp["q"].device
        tq = inp["q"].shape[0]
        n_parts = w.cp
        self.merged_dtype = merged_dtype or w.dtype
        self.o_parts = [torch.empty((tq, w.hq, w.d), dtype=torch.float32, device=dev) for _ in range(n_parts)]
        self.lse_parts = [torch.empty((tq, w.hq), dtype=torch.float32, device=dev) for _ in range(n_parts)]
        self.o = torch.empty((tq, w.hq, w.d), dtype=self.merged_dtype, device=dev)
        self.lse = torch.empty((tq, w.hq), dtype=torch.float32, device=dev)
        self.workspace = None
        if w.kind == "pass_kv":
            need = cpa.partial_attn_multi_workspace(w.cp, len(inp["lens"]), inp["max_q"])
            if need:
                self.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        else:
            need = max(
                cpa.partial_attn_paged_workspace(len(inp["lens"]), inp["max_q"], r["block_table"].shape[1],
                                                 w.block_size, w.hq, w.d)
                for r in inp["ranks"]
            )
            if need:
                self.workspace = torch.empty(need, dtype=torch.uint8, device=dev)

    def outputs(self) -> list:
        """Every output buffer of the step (partials, merged O and LSE)."""
        return [self.o, self.lse] + self.o_parts + self.lse_parts

    def poison(self):
        """Fills every output with NaN, so that a row no kernel writes shows up
        as NaN in the results."""
        for t in self.outputs():
            t.fill_(float("nan"))

    def partial(self, i: int, stream=None):
        """Partial i of the schedule (pass-KV step i, or rank i's paged shard)."""
        inp, w = self.inp, self.w
        if w.kind == "pass_kv":
            st = inp["steps"][i]
            cpa.partial_attn(inp["q"], inp["q_pos"], inp["cu_q"], st["k"], st["v"], st["k_pos"], st["cu_k"],
                             inp["max_q"], w.scale, True, out=self.o_parts[i], lse=self.lse_parts[i], stream=stream)
        else:
            rk = inp["ranks"][i]
            cpa.partial_attn_paged(inp["q"], inp["q_pos"], inp["cu_q"], rk["k_cache"], rk["v_cache"],
                                   rk["block_table"], rk["local_kv_lens"], w.cp, rk["rank"], w.interleave,
                                   inp["max_q"], w.scale, True, out=self.o_parts[i], lse=self.lse_parts[i],
                                   workspace=self.workspace, stream=stream)

    def partials_batched(self, stream=None, ordered=True):
        """Every pass-KV step of the rank in one launch (all shards resident),
        heaviest tiles first unless `ordered` is False."""
        inp, w = self.inp, self.w
        st = inp["steps"]
        cpa.partial_attn_multi(inp["q"], inp["q_pos"], inp["cu_q"], [s["k"] for s in st], [s["v"] for s in st],
                               [s["k_pos"] for s in st], [s["cu_k"] for s in st], inp["max_q"], w.scale, True,
                               outs=self.o_parts, lses=self.lse_parts,
                               workspace=self.workspace if ordered else None, stream=stream)

    def merged_walk(self, stream=None, out=None, lse=None):
        """The merged pass-KV result in one walk over all resident shards
        (writes self.o and self.lse unless other outputs are given)."""
        inp, w = self.inp, self.w
        st = inp["steps"]
        cpa.partial_attn_merged(inp["q"], inp["q_pos"], inp["cu_q"], [s["k"] for s in st], [s["v"] for s in st],
                                [s["k_pos"] for s in st], [s["cu_k"] for s in st], inp["max_q"], w.scale, True,
                                out=self.o if out is None else out, lse=self.lse if lse is None else lse,
                                workspace=self.workspace, stream=stream)

    def ring_accumulate(self, stream=None, out=None):
        """The pass-KV steps as a ring would run them: one shard at a time. The
        rank's own shard (step 0) is a plain partial into (o_parts[0],
        lse_parts[0]) (fp32); every later shard is folded into that running
        (O, LSE) as it arrives. `out` (or self.o) receives the merged O at the
        last step, self.lse the LSE."""
        inp, w = self.inp, self.w
        o_acc, lse_acc = self.o_parts[0], self.lse_parts[0]
        for i, st in enumerate(inp["steps"]):
            last = i == len(inp["steps"]) - 1
            if i == 0:  # heaviest-first order through the one-shard batched call
                cpa.partial_attn_multi(inp["q"], inp["q_pos"], inp["cu_q"], [st["k"]], [st["v"]], [st["k_pos"]],
                                       [st["cu_k"]], inp["max_q"], w.scale, True, outs=[o_acc], lses=[lse_acc],
                                       workspace=self.workspace, stream=stream)
                if last:  # a single shard: the partial is the result
                    (self.o if out is None else out).copy_(o_acc)
                continue
            cpa.partial_attn_accumulate(inp["q"], inp["q_pos"], inp["cu_q"], st["k"], st["v"], st["k_pos"],
                                        st["cu_k"], inp["max_q"], w.scale, o_acc, lse_acc,
                                        out=(self.o if out is None else out) if last else None,
                                        workspace=self.workspace, stream=stream)
        self.lse.copy_(lse_acc)

    def capture(self, fn=None):
        """Captures one call of `fn` (default: step) into a HIP graph and returns
        it. Every kernel of the path is a plain launch on the current stream
        (no memsets, no allocations), so replays repeat the eager results."""
        fn = fn or self.step
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        return graph

    def rank_fold(self, stream=None, own=True):
        """Paged schedules (decode, pass-Q): the rank's own partial against its
        paged shard, merged in the same call with the other ranks' partials
        already in o_parts / lse_parts (self.o, self.lse receive the result).
        With `own`, the rank's own partial is also written to its o_parts /
        lse_parts entry."""
        inp, w = self.inp, self.w
        r = w.rank
        others = [i for i in range(w.cp) if i != r]
        rk = inp["ranks"][r]
        cpa.partial_attn_paged_merged(inp["q"], inp["q_pos"], inp["cu_q"], rk["k_cache"], rk["v_cache"],
                                      rk["block_table"], rk["local_kv_lens"], w.cp, rk["rank"], w.interleave,
                                      inp["max_q"], w.scale, [self.o_parts[i] for i in others],
                                      [self.lse_parts[i] for i in others], True, out=self.o, lse=self.lse,
                                      own_out=self.o_parts[r] if own else None,
                                      own_lse=self.lse_parts[r] if own else None, workspace=self.workspace,
                                      stream=stream)

    def merge(self, stream=None):
        cpa.lse_merge(self.o_parts, self.lse_parts, out=self.o, lse_out=self.lse, stream=stream)

    def step(self, stream=None):
        """The rank's whole share: every partial, then the merge. Pass-KV steps
        run as one batched launch (their shards are all resident), followed by
        the merge; the paged schedules (decode, pass-Q) compute the other
        ranks' partials (as they would arrive), then the rank's own partial
        with the merge folded in."""
        if self.w.kind == "pass_kv":
            self.partials_batched(stream)
            self.merge(stream)
            return
        if not self.fold_supported():  # odd GQA group in prefill: no fold
            for i in range(self.w.cp):
                self.partial(i, stream)
            self.merge(stream)
            return
        for i in range(self.w.cp):
            if i != self.w.rank:
                self.partial(i, stream)
        self.rank_fold(stream)

    def fold_supported(self) -> bool:
        """Whether the rank's own paged launch can fold the other ranks'
        partials in (decode always; prefill with an even GQA group)."""
        w = self.w
        return w.kind == "decode" or (w.kind == "pass_q" and (w.hq // w.hkv) % 2 == 0)
