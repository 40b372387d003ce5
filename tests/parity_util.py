"""Oracle-side expectations and comparison helpers for the GPU parity tests.

Expected values come only from oracle/ applied to the raw seeded draws of
workloads.draw_sequence (the one thing both sides share). Partitions,
placements, gathers and positions are rebuilt here with the oracle's own
functions, independently of the library and its harness.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

O_TOL = 2e-2    # max |O_gpu - O_oracle| for bf16 inputs with fp32 accumulation
LSE_TOL = 1e-3  # max |LSE_gpu - LSE_oracle|


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _cat(ts):
    return torch.cat(ts) if len(ts) > 1 else ts[0]


def expected_pass_kv(inp: dict, rows=None):
    """Oracle partials (one per step, own shard first) and merged result for
    the packed rows `rows` of the rank's zigzag query shard."""
    w, lens, draws = inp["workload"], inp["lens"], inp["draws"]
    mine = oracle.zigzag_partition(lens, w.cp, w.rank)
    n = len(mine["positions"])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    q_all = _cat([d[0] for d in draws])
    k_all = _cat([d[1] for d in draws])
    v_all = _cat([d[2] for d in draws])
    src = torch.as_tensor(mine["src_index"][rows], device=q_all.device)
    q_sel = f64(q_all.index_select(0, src))
    qpos = mine["positions"][rows]
    seq_of_row = np.searchsorted(mine["cu_seqlens"], rows, side="right") - 1
    # regroup the selected rows as their own packed batch (sorted by sequence)
    cu_sel = np.searchsorted(seq_of_row, np.arange(len(lens) + 1), side="left")
    parts = []
    for s in range(w.cp):
        r = (w.rank - s) % w.cp
        kp = oracle.zigzag_partition(lens, w.cp, r)
        kidx = torch.as_tensor(kp["src_index"], device=k_all.device)
        k = f64(k_all.index_select(0, kidx))
        v = f64(v_all.index_select(0, kidx))
        parts.append(oracle.partial_attn(q_sel, qpos, cu_sel, k, v, kp["positions"], kp["cu_seqlens"], w.scale))
        print(f"    oracle: step {s} done ({len(rows)} rows)", flush=True)
    merged = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    return rows, parts, merged


def expected_round_robin(inp: dict, rows=None):
    """Oracle partials (one per rank, rank 0 first) and merged result for the
    packed query rows `rows` of a pass-Q or decode workload."""
    w, lens, draws = inp["workload"], inp["lens"], inp["draws"]
    nq = [d[0].shape[0] for d in draws]
    cu = np.concatenate([[0], np.cumsum(nq)])
    rows = np.arange(cu[-1]) if rows is None else np.asarray(rows)
    seq_of_row = np.searchsorted(cu, rows, side="right") - 1
    parts_o = [np.zeros((len(rows), w.hq, w.d)) for _ in range(w.cp)]
    parts_l = [np.zeros((len(rows), w.hq)) for _ in range(w.cp)]
    for i, b in enumerate(np.unique(seq_of_row)):
        if i % 32 == 31:
            print(f"    oracle: {i + 1} sequences done", flush=True)
        sel = np.nonzero(seq_of_row == b)[0]
        local_rows = rows[sel] - cu[b]
        L = lens[b]
        qpos = (L - nq[b]) + local_rows
        q = f64(draws[b][0][torch.as_tensor(local_rows, device=draws[b][0].device)])
        for r in range(w.cp):
            l2g = oracle.rr_placement([L], w.cp, r, w.interleave)["local_to_global"]
            idx = torch.as_tensor(l2g, device=draws[b][1].device)
            k = f64(draws[b][1].index_select(0, idx))
            v = f64(draws[b][2].index_select(0, idx))
            o, l = oracle.partial_attn(q, qpos, [0, len(sel)], k, v, l2g, [0, len(l2g)], w.scale)
            parts_o[r][sel] = o
            parts_l[r][sel] = l
    parts = list(zip(parts_o, parts_l))
    merged = oracle.lse_merge(parts_o, parts_l)
    return rows, parts, merged


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, what: str, o_tol=O_TOL, lse_tol=LSE_TOL):
    """Parity bar: no NaN; -inf rows exactly -inf with O exactly 0; elsewhere
    max-abs error within the tolerances."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    empty = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse_gpu), empty, err_msg=f"{what}: -inf rows differ")
    assert np.all(o_gpu[empty] == 0), f"{what}: O of empty rows is not 0"
    fin = ~empty
    if fin.any():
        lerr = np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))
        oerr = np.max(np.abs(o_gpu[fin] - o_ref[fin]))
        assert lerr <= lse_tol, f"{what}: max |dLSE| = {lerr:.3g} > {lse_tol}"
        assert oerr <= o_tol, f"{what}: max |dO| = {oerr:.3g} > {o_tol}"
        return float(oerr), float(lerr)
    return 0.0, 0.0


def sample_rows(cu: np.ndarray, positions: np.ndarray, n_random: int, seed: int, tile: int = 128) -> np.ndarray:
    """Rows worth checking in a big packed shard: each sequence's first and
    last rows, rows around jumps in position (zigzag chunk boundaries), rows
    around kernel tile boundaries, plus random rows."""
    rng = np.random.default_rng(seed)
    picks = set()
    n = int(cu[-1])
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        if e <= a:
            continue
        picks.update([a, e - 1])
        p = positions[a:e]
        jumps = np.nonzero(np.diff(p) != 1)[0]
        for j in jumps[:8]:
            picks.update([a + j, a + j + 1])
        for t in range(a + tile, e, tile * max(1, (e - a) // (tile * 6))):
            picks.update([t - 1, t])
    picks.update(rng.integers(0, max(1, n), size=n_random).tolist())
    return np.array(sorted(x for x in picks if 0 <= x < n), dtype=np.int64)
