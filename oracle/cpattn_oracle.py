"""Plain CPU oracle, fp64, for partial causal GQA attention under context parallelism.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module. It shares no code
with the HIP library and imports nothing from it.

Sources: three vLLM pull-request pages.
  [PCP-GQA]  "[Feature] Support Prefill Context Parallel (PCP) for GQA flashinfer"
             (vLLM PR 28723): Purpose; Test Plan (the interleave-size flag).
  [PASSKV]   "Add utility functions to enable pass-kv prefill and allgather decode"
             (vLLM PR 26059): Purpose (sequence dependency of attention, exchanging
             Q or KV shards, partial attention, round-robin KV for decode); the
             review's suggested test fix for per-rank token counts.
  [PCP-BASE] "[Feature] Prefill Context Parallel (PCP) basic support" (vLLM PR 28718):
             Purpose (splitting the sequence dimension at prefill, block tables
             extended for CP); review summary (the interleave size shared by
             prefill and decode CP).

The pages give no formulas. Each function below states the plain mathematical
definition it implements and the reading taken where the pages are silent.
Every function is pinned by the CPU tests (brute force, closed forms, library
routines, invariants); none is marked "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Sequence partitioning (integer work)
# ----------------------------------------------------------------------------


def zigzag_chunk_sizes(L: int, cp: int) -> list[int]:
    """Sizes of the 2*cp chunks a length-L sequence is cut into.

    [PCP-GQA]/[PCP-BASE] Purpose: prefill CP splits the sequence dimension
    across ranks. Reading taken for the split: 2*cp contiguous chunks in
    position order; when 2*cp does not divide L the first L mod 2*cp chunks
    hold one extra token (no padding, so shapes stay exact).
    """
    n = 2 * cp
    return [L // n + (1 if c < L % n else 0) for c in range(n)]


def zigzag_partition(seq_lens, cp: int, rank: int) -> dict:
    """The query/KV shard that rank `rank` holds under the zigzag split.

    Rank r owns chunk r and chunk 2*cp-1-r (the load-balanced pairing: an
    early, cheap chunk with a late, expensive one under the causal mask).
    Tokens of a shard are kept in ascending global position; shards of a
    batch are packed sequence after sequence.

    Returns int64 arrays:
      chunk_bounds [B, 2cp+1]  chunk start positions within each sequence, then L
      cu_seqlens   [B+1]       shard offsets into the packed shard
      positions    [n]         global position (within its sequence) of each shard token
      src_index    [n]         index of the token in the packed unsharded batch
    """
    if cp < 1 or not (0 <= rank < cp):
        raise ValueError("need cp >= 1 and 0 <= rank < cp")
    n = 2 * cp
    bounds, cu, pos, src = [], [0], [], []
    seq_start = 0
    for L in seq_lens:
        L = int(L)
        if L < 0:
            raise ValueError("negative sequence length")
        sizes = zigzag_chunk_sizes(L, cp)
        b = [0]
        for s in sizes:
            b.append(b[-1] + s)
        bounds.append(b)
        own = []
        for c in (rank, n - 1 - rank):
            own.extend(range(b[c], b[c + 1]))
        pos.extend(own)
        src.extend(seq_start + p for p in own)
        cu.append(cu[-1] + len(own))
        seq_start += L
    return {
        "chunk_bounds": np.array(bounds, dtype=np.int64).reshape(len(seq_lens), n + 1),
        "cu_seqlens": np.array(cu, dtype=np.int64),
        "positions": np.array(pos, dtype=np.int64),
        "src_index": np.array(src, dtype=np.int64),
    }


def rr_rank(t, cp: int, interleave: int):
    """Rank that stores the KV of global position t under round-robin placement.

    [PASSKV] Purpose: for decode the KV is stored on the CP ranks in a
    round-robin manner; [PCP-GQA] Test Plan and [PCP-BASE] review summary: the
    placement has an interleave size. Reading taken: positions [0, I) go to
    rank 0, the next I to rank 1, and so on cyclically.
    """
    return (np.asarray(t) // interleave) % cp


def rr_local_index(t, cp: int, interleave: int):
    """Index of global position t within its rank's local KV sequence.

    A rank's local tokens are its positions in ascending order; each full
    cycle of cp*I positions contributes I local tokens to every rank.
    """
    t = np.asarray(t)
    return (t // (interleave * cp)) * interleave + t % interleave


def rr_global_index(local, rank: int, cp: int, interleave: int):
    """Global position of local index `local` on rank `rank` (inverse map)."""
    local = np.asarray(local)
    return ((local // interleave) * cp + rank) * interleave + local % interleave


def rr_local_len(L: int, cp: int, rank: int, interleave: int) -> int:
    """Number of positions in [0, L) that rank `rank` stores: by enumeration."""
    return int(np.count_nonzero(rr_rank(np.arange(int(L)), cp, interleave) == rank))


def rr_placement(seq_lens, cp: int, rank: int, interleave: int) -> dict:
    """Local lengths and the local -> global position map for one rank.

    For each sequence, every position t in [0, L) with rr_rank(t) == rank is
    stored at local slot rr_local_index(t). Returns int64 arrays:
      local_lens      [B]
      cu_local        [B+1]
      local_to_global [sum(local_lens)]  packed sequence after sequence
    """
    if cp < 1 or not (0 <= rank < cp) or interleave < 1:
        raise ValueError("need cp >= 1, 0 <= rank < cp, interleave >= 1")
    lens, maps = [], []
    for L in seq_lens:
        t = np.arange(int(L))
        mine = t[rr_rank(t, cp, interleave) == rank]
        slot = rr_local_index(mine, cp, interleave)
        m = np.full(len(mine), -1, dtype=np.int64)
        m[slot] = mine  # raises if a slot falls outside [0, len): caught by tests
        lens.append(len(mine))
        maps.append(m)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    l2g = np.concatenate(maps).astype(np.int64) if maps else np.zeros(0, np.int64)
    return {"local_lens": np.array(lens, dtype=np.int64), "cu_local": cu, "local_to_global": l2g}


# ----------------------------------------------------------------------------
# Attention (floating-point work), fp64
# ----------------------------------------------------------------------------


def attend(q, k, v, visible, scale: float):
    """Masked softmax attention for one head, straight from the definition.

    q [m, D], k [n, D], v [n, D], visible [m, n] bool.
      s_ij   = scale * <q_i, k_j>                 for visible (i, j)
      LSE_i  = log sum_{j visible} exp(s_ij)      (natural log; max-shifted)
      O_i    = sum_{j visible} exp(s_ij - LSE_i) v_j
    A row that sees no key gets O_i = 0 and LSE_i = -inf.
    [PASSKV] Purpose: each token attends to all previous tokens of its
    sequence; a partial attention is the same computation over a subset of
    the keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    visible = np.asarray(visible, dtype=bool)
    m_rows, d = q.shape[0], v.shape[1]
    o = np.zeros((m_rows, d), dtype=np.float64)
    lse = np.full(m_rows, -np.inf, dtype=np.float64)
    if k.shape[0] == 0 or m_rows == 0:
        return o, lse
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    has = visible.any(axis=1)
    if not has.any():
        return o, lse
    s = s[has]
    mx = s.max(axis=1, keepdims=True)
    lse_h = mx[:, 0] + np.log(np.exp(s - mx).sum(axis=1))
    w = np.exp(s - lse_h[:, None])
    o[has] = w @ v
    lse[has] = lse_h
    return o, lse


def _row_blocks(m: int, n: int, budget_elems: int = 1 << 23):
    step = max(1, budget_elems // max(1, n))
    for a in range(0, m, step):
        yield a, min(m, a + step)


def full_causal_attn(q, k, v, scale: float, rows=None):
    """Full causal GQA attention of one unsharded sequence, for chosen rows.

    q [L, Hq, D]; k, v [L, Hkv, D]; query head h reads KV head h // (Hq/Hkv)
    (contiguous head groups: the plain reading of GQA). Query i sees keys
    j <= i. `rows` selects query positions (default: all). Returns O
    [len(rows), Hq, D] and LSE [len(rows), Hq]. This is the result the
    partial-and-merge method must reproduce.
    """
    q = np.asarray(q)
    L = q.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = np.arange(L)
    return _attn_by_positions(q[rows], rows, k, v, pos, scale, causal=True)


def _attn_by_positions(q, q_pos, k, v, k_pos, scale, causal):
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    hq, hkv = q.shape[1], k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    m_rows, d = q.shape[0], v.shape[2]
    o = np.zeros((m_rows, hq, d), dtype=np.float64)
    lse = np.full((m_rows, hq), -np.inf, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    for h in range(hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        for a, b in _row_blocks(m_rows, k.shape[0]):
            if causal:
                vis = k_pos[None, :] <= q_pos[a:b, None]
            else:
                vis = np.ones((b - a, k.shape[0]), dtype=bool)
            o[a:b, h], lse[a:b, h] = attend(q[a:b, h, :], kh, vh, vis, scale)
    return o, lse


def partial_attn(q, q_pos, cu_q, k, v, k_pos, cu_k, scale: float, causal: bool = True, rows=None):
    """Partial attention of a packed Q shard against one packed KV shard.

    q [Tq, Hq, D] with global positions q_pos [Tq]; k, v [Tk, Hkv, D] with
    global positions k_pos [Tk]; cu_q/cu_k [B+1] delimit the sequences. Query
    i of sequence b attends to the keys of sequence b with k_pos <= q_pos
    (causal in global positions; `causal=False` lets it see the whole shard).
    This is the per-step computation of pass-KV and pass-Q prefill and of
    allgather decode ([PASSKV] Purpose). `rows` optionally restricts the
    packed query rows computed. Returns O [rows, Hq, D], LSE [rows, Hq].
    """
    q = np.asarray(q)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    tq = q.shape[0]
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    seq_of_row = np.searchsorted(cu_q, rows, side="right") - 1
    hq, d = q.shape[1], np.asarray(v).shape[2]
    o = np.zeros((len(rows), hq, d), dtype=np.float64)
    lse = np.full((len(rows), hq), -np.inf, dtype=np.float64)
    for b in np.unique(seq_of_row):
        sel = np.nonzero(seq_of_row == b)[0]
        r = rows[sel]
        ka, kb = cu_k[b], cu_k[b + 1]
        o[sel], lse[sel] = _attn_by_positions(
            q[r], q_pos[r], np.asarray(k)[ka:kb], np.asarray(v)[ka:kb], k_pos[ka:kb], scale, causal
        )
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Exact merge of partial results over disjoint key sets.

    For each row with partials (O_s, LSE_s), s = 0..n-1:
      M   = max_s LSE_s;  if M = -inf the row is (0, -inf)
      LSE = M + log sum_s exp(LSE_s - M)
      O   = sum_s exp(LSE_s - LSE) O_s
    Because the key sets are disjoint, sum over the union equals the sum of
    the per-part sums, so this reproduces attention over the union exactly.
    Partials are taken in the order given (ascending source rank).
    o_parts: sequence of [..., D]; lse_parts: sequence of [...].
    """
    o_parts = [np.asarray(o, dtype=np.float64) for o in o_parts]
    lse_parts = [np.asarray(x, dtype=np.float64) for x in lse_parts]
    if not o_parts:
        raise ValueError("need at least one partial")
    lse_stack = np.stack(lse_parts)  # [n, ...]
    mx = lse_stack.max(axis=0)
    finite = np.isfinite(mx)
    safe_mx = np.where(finite, mx, 0.0)
    tot = np.exp(lse_stack - safe_mx).sum(axis=0)
    lse = np.where(finite, safe_mx + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.zeros_like(o_parts[0])
    for o_s, l_s in zip(o_parts, lse_parts):
        w = np.where(finite, np.exp(l_s - np.where(finite, lse, 0.0)), 0.0)
        o = o + w[..., None] * o_s
    return o, lse


def visible_pairs(q_pos, cu_q, k_pos, cu_k, causal: bool = True) -> int:
    """Number of (query, key) pairs a partial attention computes: for each
    query, the keys of its sequence with k_pos <= q_pos (all of them when not
    causal). Counted one query at a time."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    total = 0
    for b in range(len(cu_q) - 1):
        kp = k_pos[cu_k[b]:cu_k[b + 1]]
        for p in q_pos[cu_q[b]:cu_q[b + 1]]:
            total += int(np.count_nonzero(kp <= p)) if causal else len(kp)
    return total


# ----------------------------------------------------------------------------
# Choice of the exchanged shard (host policy)
# ----------------------------------------------------------------------------


def choose_pass(q_lens, kv_lens, hq: int, hkv: int, d: int, elem_bytes: int = 2) -> dict:
    """Pass KV or pass Q for a prefill batch ([PASSKV], Purpose: the choice
    follows the relative sizes of the Q and KV tensors; full prefill prefers
    passing KV because a KV head usually serves more than two query heads,
    chunked prefill with a cache much longer than the new tokens prefers
    passing Q).

    Reading: compare the bytes each scheme moves around the ring for the
    batch, K plus V of every context token (2 * hkv * d per token) against Q
    of every new token (hq * d per token); pass KV iff strictly fewer bytes.
    For full prefill (kv_lens == q_lens) this is hq / hkv > 2, the pages'
    statement. q_lens: new tokens per sequence; kv_lens: context tokens per
    sequence (cached + new).
    """
    t_q = int(sum(int(x) for x in q_lens))
    t_kv = int(sum(int(x) for x in kv_lens))
    kv_bytes = 2 * hkv * d * elem_bytes * t_kv
    q_bytes = hq * d * elem_bytes * t_q
    return {"pass_kv": kv_bytes < q_bytes, "kv_bytes": kv_bytes, "q_bytes": q_bytes}


def pass_cost(q_lens, kv_lens, hq: int, hkv: int, d: int, elem_bytes: int, cp: int,
              link_bytes_per_s: float, mfma_flops_per_s: float) -> dict:
    """Per-step cost of the two exchange schemes for a prefill batch.

    [PASSKV], Purpose: the exchanged shard is chosen from the relative sizes
    of Q and KV, and the partial-attention compute of a step is what hides
    the transfer of the next shard. Readings taken:
      * a rank's work is 1/cp of the batch's (zigzag and round-robin shards
        balance it) and a step is 1/cp of a rank's work, so a step computes
        4 * d * hq * pairs / cp^2 FLOP, where pairs counts the (new token,
        context key) pairs the causal mask lets through: new token i of a
        sequence with c cached tokens sits at position c + i and sees c + i + 1
        keys;
      * a step moves one rank's shard over one link: K+V of T_kv / cp context
        tokens under pass-KV, Q of T_q / cp new tokens under pass-Q;
      * a transfer is hidden when it takes no longer than the step's compute
        at the given MFMA rate.
    The choice itself is `choose_pass` (fewer bytes moved). q_lens: new tokens
    per sequence; kv_lens: context tokens per sequence (cached + new).
    """
    if cp < 1 or link_bytes_per_s <= 0 or mfma_flops_per_s <= 0:
        raise ValueError("need cp >= 1 and positive rates")
    choice = choose_pass(q_lens, kv_lens, hq, hkv, d, elem_bytes)
    pairs = 0
    for ql, kl in zip(q_lens, kv_lens):
        ql, kl = int(ql), int(kl)
        if ql > kl:
            raise ValueError("a sequence has more new tokens than context tokens")
        cached = kl - ql
        for i in range(ql):  # one new token at a time
            pairs += cached + i + 1
    step_flops = 4 * d * hq * pairs / (cp * cp)
    kv_step = choice["kv_bytes"] / cp
    q_step = choice["q_bytes"] / cp
    t_compute = step_flops / mfma_flops_per_s
    t_kv = kv_step / link_bytes_per_s
    t_q = q_step / link_bytes_per_s
    return {
        "pass_kv": choice["pass_kv"],
        "kv_bytes": choice["kv_bytes"],
        "q_bytes": choice["q_bytes"],
        "pairs": pairs,
        "kv_step_bytes": kv_step,
        "q_step_bytes": q_step,
        "step_flops": step_flops,
        "kv_transfer_s": t_kv,
        "q_transfer_s": t_q,
        "step_compute_s": t_compute,
        "kv_hidden": t_kv <= t_compute,
        "q_hidden": t_q <= t_compute,
    }
