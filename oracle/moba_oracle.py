"""Plain fp64 CPU oracle for the MoBA prefill forward.

TEST INFRASTRUCTURE ONLY.  This file is the checker that the HIP kernels are
compared against.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the product path never does, and it shares
no code, table or helper with the HIP sources.

Sources (cited by page title and section):
  report  -- the deep-dive report page on "MoBA: Mixture of Block Attention
             for Long-Context LLMs" (arXiv 2502.13189).
  course  -- the course page "Paper: MoBA (Moonshot)" (module F26).
  blog    -- the blog page on getting the MoonshotAI/MoBA code to run.

What MoBA computes, per query row (b, t, h), written out step by step in the
order the report gives it:
  1. report §2.1: cut the length-S context into n = S/B blocks of B keys;
     block i (0-indexed here) holds positions [iB, (i+1)B).  A block is the
     unit of choice: a chosen block is attended in full, an unchosen one not
     at all.  S not divisible by B is an error (blog §1.1: the original code
     asserts), so no padding is defined.
  2. report §2.2 and the course summary: summarise each block by the mean of
     its keys, mu_i = mean(K[block i]); the gate score is s_i = <q, mu_i>.
     No router parameters and no scaling are involved.
  3. report §2.3: causality.  Blocks that lie in the query's future get score
     -inf (never routed to); the query's own block j = floor(t/B) is always
     chosen; inside the own block a causal mask applies.
  4. report §2.2: hard top-k gating (g_i in {0, 1}) over the admissible
     blocks; the output is softmax attention over the union of the chosen
     blocks' positions.
Readings where the pages leave a step open (each listed in the design notes):
  * top-k counts the forced own block: own block + (k-1) best past blocks.
    Pinned by the report's sparsity figures (3 of 16 blocks -> 81.25 %,
    3 of 64 and 12 of 256 -> 95.31 %; report summary and §3.3).
  * when fewer than k-1 past blocks exist, all of them are chosen; topk >= n
    is allowed and gives dense causal attention (course summary: with every
    block chosen MoBA is exactly dense attention).
  * ties in the gate go to the lower block index.
  * the attention logits carry the usual 1/sqrt(D) factor (the report prints
    the softmax without it; MoBA has to reduce to standard attention).
  * grouped-query attention: query head h reads KV head floor(h / (Hq/Hkv)),
    and routes with its own q (course exercise: per-head routing).
  * non-causal mode (causal = False): no future mask, no forced block, plain
    top-k over all n blocks, no mask inside blocks.

Decode (decode_rows): one new query per sequence, at position t = L - 1 of
a cache of L keys and values, is routed and attended exactly as prefill row t
(the pages leave sparse decode open, report §6.3; this is the plainest
reading): its own block j = t // B is cut at t, the past blocks 0..j-1 are
complete and ranked by their mean keys.

Gate variant (report §1.3 and §5: Quest is placed in the family as MoBA with
small blocks and min/max pooling of the block's keys):
  * gate = "minmax": block i is summarised by the element-wise minimum lo_i
    and maximum hi_i of its keys; its score is the largest value q.k can take
    for any k inside that box, sum_d max(q_d lo_id, q_d hi_id).  This is the
    plainest score that uses both summaries; it bounds every q.k_s of the
    block from above.  Causal rules, forced block and top-k are unchanged.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Step 1 and 2: blocks and their mean keys (report §2.1, §2.2)
# ----------------------------------------------------------------------------
def num_blocks(seqlen: int, block_size: int) -> int:
    """n = S / B (report §2.1).  Non-divisible lengths are rejected, as the
    original code does (blog §1.1)."""
    if block_size <= 0 or seqlen % block_size != 0:
        raise ValueError(f"seqlen {seqlen} is not a multiple of block_size {block_size}")
    return seqlen // block_size


def block_means(k: np.ndarray, block_size: int) -> np.ndarray:
    """mu[b, hk, i, :] = mean of K[b, iB:(i+1)B, hk, :]  (report §2.2).

    k: [batch, S, Hkv, D] (any float dtype; values are taken exactly).
    Returns fp64 [batch, Hkv, n, D].  Computed block by block so the 1M
    workload does not need an fp64 copy of all of K at once."""
    b, S, Hkv, D = k.shape
    n = num_blocks(S, block_size)
    mu = np.empty((b, Hkv, n, D), dtype=np.float64)
    for bb in range(b):
        for i in range(n):
            blk = np.asarray(k[bb, i * block_size:(i + 1) * block_size], dtype=np.float64)  # [B, Hkv, D]
            mu[bb, :, i, :] = blk.mean(axis=0)
    return mu


def block_minmax(k: np.ndarray, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Element-wise minimum and maximum of each block's keys (the min/max
    pooling of the Quest-style gate, report §1.3): lo, hi [batch, Hkv, n, D]
    fp64 (exact: they are input values)."""
    b, S, Hkv, D = k.shape
    n = num_blocks(S, block_size)
    lo = np.empty((b, Hkv, n, D), dtype=np.float64)
    hi = np.empty((b, Hkv, n, D), dtype=np.float64)
    for bb in range(b):
        for i in range(n):
            blk = np.asarray(k[bb, i * block_size:(i + 1) * block_size], dtype=np.float64)  # [B, Hkv, D]
            lo[bb, :, i, :] = blk.min(axis=0)
            hi[bb, :, i, :] = blk.max(axis=0)
    return lo, hi


# ----------------------------------------------------------------------------
# Step 3 and 4: gate scores, causal rules, top-k (report §2.2, §2.3)
# ----------------------------------------------------------------------------
def gate_scores(q_row: np.ndarray, mu_head: np.ndarray) -> np.ndarray:
    """s_i = <q, mu_i> for every block i  (report §2.2).  mu_head: [n, D]."""
    return mu_head @ np.asarray(q_row, dtype=np.float64)


def gate_scores_minmax(q_row: np.ndarray, lo_head: np.ndarray, hi_head: np.ndarray) -> np.ndarray:
    """s_i = sum_d max(q_d lo_id, q_d hi_id): the largest q.k over the box
    [lo_i, hi_i] (the Quest-style gate's score).  lo_head, hi_head: [n, D]."""
    q64 = np.asarray(q_row, dtype=np.float64)
    return np.maximum(lo_head * q64, hi_head * q64).sum(axis=1)


def select_blocks(scores: np.ndarray, j: int, topk: int, causal: bool) -> List[int]:
    """The chosen block indices, ascending.

    causal (report §2.3): blocks after the own block j are excluded (score
    -inf), block j is always kept and fills one of the k slots; the other
    min(k-1, j) slots go to the highest-scoring past blocks 0..j-1, ties to
    the lower index.
    non-causal: the top min(k, n) of all n blocks, ties to the lower index.
    """
    n = len(scores)
    if topk < 1:
        raise ValueError("topk must be >= 1")
    if causal:
        past = list(range(j))
        m = min(topk - 1, j)
        # sort by (-score, index): a stable descending order
        ranked = sorted(past, key=lambda i: (-float(scores[i]), i))
        chosen = ranked[:m] + [j]
    else:
        ranked = sorted(range(n), key=lambda i: (-float(scores[i]), i))
        chosen = ranked[:min(topk, n)]
    return sorted(chosen)


def key_ranges(sel: Sequence[int], t: int, block_size: int, causal: bool) -> List[Tuple[int, int]]:
    """The chosen blocks' positions as [start, end) ranges, ascending (report
    §2.2); the own block is cut at the query itself (report §2.3, causal mask
    in-block)."""
    B = block_size
    j = t // B
    return [(i * B, t + 1 if (causal and i == j) else (i + 1) * B) for i in sorted(sel)]


def key_positions(sel: Sequence[int], t: int, block_size: int, causal: bool) -> np.ndarray:
    """Union of the chosen blocks' positions, ascending (key_ranges)."""
    parts = [np.arange(a, e) for a, e in key_ranges(sel, t, block_size, causal)]
    return np.concatenate(parts) if parts else np.zeros((0,), dtype=np.int64)


# ----------------------------------------------------------------------------
# Step 4: softmax attention over the union (report §2.2)
# ----------------------------------------------------------------------------
def _attend_blocks(q64: np.ndarray, k_head: np.ndarray, v_head: np.ndarray,
                   sel: Sequence[int], t: int, B: int, causal: bool, scale: float) -> np.ndarray:
    """o = softmax(scale * q.K[keys]^T) V[keys] over keys = key_positions(sel,
    t, B, causal), fp64 with the maximum subtracted (report §2.2: softmax
    attention over the union of the chosen blocks).  The chosen blocks are
    read as contiguous slices in ascending key order (no gathered copy of K),
    which keeps the 1M rows affordable."""
    logit_parts, v_parts = [], []
    for a, e in key_ranges(sel, t, B, causal):
        logit_parts.append((k_head[a:e] @ q64) * scale)
        v_parts.append(v_head[a:e])
    logits = np.concatenate(logit_parts)
    m = logits.max()
    p = np.exp(logits - m)
    acc = np.zeros(q64.shape[0], dtype=np.float64)
    off = 0
    for vp in v_parts:
        acc += p[off:off + vp.shape[0]] @ vp
        off += vp.shape[0]
    return acc / p.sum()


# ----------------------------------------------------------------------------
# Whole forward
# ----------------------------------------------------------------------------
def _check_shapes(q, k, v, block_size, topk):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, seqlen, heads, head_dim]")
    b, S, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[1] != S or k.shape[3] != D:
        raise ValueError("k and v must be [batch, seqlen, kv_heads, head_dim] matching q")
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if topk < 1:
        raise ValueError("topk must be >= 1")
    num_blocks(S, block_size)
    return b, S, Hq, Hkv, D


def moba_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_size: int,
                 topk: int, causal: bool = True, gate: str = "mean") -> Tuple[np.ndarray, np.ndarray]:
    """Full MoBA forward on small inputs.

    Returns out [batch, S, Hq, D] fp64 and sel_idx [batch, Hq, S, topk] int32
    (chosen blocks ascending, padded with -1)."""
    b, S, Hq, Hkv, D = _check_shapes(q, k, v, block_size, topk)
    rows = [(bb, t, h) for bb in range(b) for h in range(Hq) for t in range(S)]
    res = moba_rows(q, k, v, block_size, topk, causal, rows, gate=gate)
    out = np.zeros((b, S, Hq, D), dtype=np.float64)
    sel_idx = np.full((b, Hq, S, topk), -1, dtype=np.int32)
    for r, (bb, t, h) in enumerate(rows):
        out[bb, t, h] = res.out[r]
        sel_idx[bb, h, t] = res.sel[r]
    return out, sel_idx


# ----------------------------------------------------------------------------
# Backward: gradients of the forward with the gate's choice held fixed
# ----------------------------------------------------------------------------
def moba_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, block_size: int,
                  topk: int, causal: bool = True,
                  sel_idx: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """dq, dk, dv of sum(dout * out) and the row log-sum-exp, fp64, small inputs.

    The gate is a hard top-k with no parameters (report §2.2): it only picks
    which keys each row attends, and no gradient flows through the choice.
    With the chosen key set K_t of row t fixed, the row is plain softmax
    attention, so (the report trains models with MoBA, §3.3 and §3.4, but
    prints no backward; the plainest reading is the gradient of the attention
    over K_t):
      p_s = exp(scale q.k_s - lse),  lse = log sum_{s in K_t} exp(scale q.k_s)
      dv_s += p_s dout,   dp_s = dout . v_s,   delta = dout . out
      ds_s = p_s (dp_s - delta)
      dq = scale sum_s ds_s k_s,   dk_s += scale ds_s q.
    sel_idx (as moba_forward returns it) fixes the choice; by default the
    oracle's own gate makes it.  Returns dq [b, S, Hq, D], dk, dv [b, S,
    Hkv, D] and lse [b, Hq, S] (natural log)."""
    b, S, Hq, Hkv, D = _check_shapes(q, k, v, block_size, topk)
    g = Hq // Hkv
    B = block_size
    scale = 1.0 / math.sqrt(D)
    if sel_idx is None:
        _, sel_idx = moba_forward(q, k, v, B, topk, causal)
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    do64 = np.asarray(dout, dtype=np.float64)
    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    lse = np.zeros((b, Hq, S))
    for bb in range(b):
        for h in range(Hq):
            hk = h // g
            for t in range(S):
                sel = [int(i) for i in sel_idx[bb, h, t] if i >= 0]
                # the row's keys as the contiguous ranges of the chosen
                # blocks in ascending order
                ranges = key_ranges(sel, t, B, causal)
                kk = np.concatenate([k64[bb, a:e, hk] for a, e in ranges])
                vv = np.concatenate([v64[bb, a:e, hk] for a, e in ranges])
                logits = (kk @ q64[bb, t, h]) * scale
                m = logits.max()
                z = np.exp(logits - m).sum()
                lse[bb, h, t] = m + math.log(z)
                p = np.exp(logits - lse[bb, h, t])
                o = p @ vv
                dp = vv @ do64[bb, t, h]
                ds = p * (dp - do64[bb, t, h] @ o)
                dq[bb, t, h] = scale * (ds @ kk)
                off = 0
                for a, e in ranges:
                    dk[bb, a:e, hk] += scale * np.outer(ds[off:off + e - a], q64[bb, t, h])
                    dv[bb, a:e, hk] += np.outer(p[off:off + e - a], do64[bb, t, h])
                    off += e - a
    return dq, dk, dv, lse


def backward_dq_rows(q, k, v, dout, block_size: int, causal: bool,
                     rows: Sequence[Tuple[int, int, int]],
                     sels: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """dq and lse of single rows (b, t, h) with their chosen blocks given:
    the same per-row formulas as moba_backward, for checking sampled rows of
    large inputs (dq of a row depends on that row alone).  Arrays may be any
    type with numpy indexing (a KV head is converted per row)."""
    D = q.shape[3]
    g = q.shape[2] // k.shape[2]
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    order = sorted(range(len(rows)), key=lambda r: (rows[r][0], rows[r][2] // g, r))
    cur = None
    for r in order:
        (bb, t, h), sel = rows[r], sels[r]
        hk = h // g
        if cur != (bb, hk):  # each (batch, KV head) converted once
            cur = (bb, hk)
            k_head = np.asarray(k[bb, :, hk, :], dtype=np.float64)
            v_head = np.asarray(v[bb, :, hk, :], dtype=np.float64)
        keys = key_positions([int(i) for i in sel if i >= 0], t, block_size, causal)
        kk = k_head[keys]
        vv = v_head[keys]
        q64 = np.asarray(q[bb, t, h], dtype=np.float64)
        do64 = np.asarray(dout[bb, t, h], dtype=np.float64)
        logits = (kk @ q64) * scale
        m = logits.max()
        lse[r] = m + math.log(np.exp(logits - m).sum())
        p = np.exp(logits - lse[r])
        ds = p * (vv @ do64 - do64 @ (p @ vv))
        dq[r] = scale * (ds @ kk)
    return dq, lse


def backward_row_stats(q, k, v, dout, block_size: int, causal: bool,
                       rows: Sequence[Tuple[int, int, int]], sels: Sequence[Sequence[int]]) -> dict:
    """Per row (b, t, h) with its chosen blocks given: the row's log-sum-exp
    of the scaled logits (natural log) and delta = dout . out over all of its
    keys, the two row quantities every key's gradient needs (the same
    formulas as moba_backward).  Returns {(b, t, h): (lse, delta)}."""
    D = q.shape[3]
    g = q.shape[2] // k.shape[2]
    B = block_size
    scale = 1.0 / math.sqrt(D)
    out = {}
    order = sorted(range(len(rows)), key=lambda r: (rows[r][0], rows[r][2] // g, r))
    cur = None
    for r in order:
        bb, t, h = rows[r]
        hk = h // g
        if cur != (bb, hk):  # each (batch, KV head) converted once
            cur = (bb, hk)
            k_head = np.asarray(k[bb, :, hk, :], dtype=np.float64)
            v_head = np.asarray(v[bb, :, hk, :], dtype=np.float64)
        q64 = np.asarray(q[bb, t, h], dtype=np.float64)
        do64 = np.asarray(dout[bb, t, h], dtype=np.float64)
        sel = sorted(int(c) for c in sels[r] if c >= 0)
        o = _attend_blocks(q64, k_head, v_head, sel, t, B, causal, scale)
        # the log-sum-exp over the same keys, block by block in ascending order
        logits = np.concatenate([(k_head[a:e] @ q64) * scale for a, e in key_ranges(sel, t, B, causal)])
        m = logits.max()
        out[(bb, t, h)] = (m + math.log(np.exp(logits - m).sum()), float(do64 @ o))
    return out


def attending_rows(sel_idx, block_size: int, causal: bool, b: int, s: int, hk: int, g: int):
    """The rows (b, t, h) of KV head hk that attend key position s: the key's
    block is in the row's selection and, in the row's own block, s <= t
    (report §2.3)."""
    B = block_size
    i = s // B
    rows = []
    for h in range(hk * g, (hk + 1) * g):
        for t in np.nonzero((np.asarray(sel_idx[b, h]) == i).any(axis=1))[0].tolist():
            if causal and t // B == i and t < s:
                continue
            rows.append((b, t, h))
    return rows


def backward_dkdv_keys(q, k, v, dout, block_size: int, causal: bool,
                       keys: Sequence[Tuple[int, int, int]], sel_idx,
                       row_stats: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """dk and dv of single keys (b, s, hk) with every row's chosen blocks
    given by sel_idx [b, Hq, S, topk]: the same formulas as moba_backward,
    summed over the rows that attend key s (attending_rows), for checking
    sampled keys of large inputs:
      dv_s = sum p_s dout,  dk_s = scale sum p_s (dout . v_s - delta) q.
    Each row's (lse, delta) comes from backward_row_stats (computed here for
    the rows `row_stats` lacks).  Arrays may be any type with numpy indexing."""
    b, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    scale = 1.0 / math.sqrt(D)
    stats = dict(row_stats or {})
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for x, (bb, s_pos, hk) in enumerate(keys):
        rows = attending_rows(sel_idx, block_size, causal, bb, s_pos, hk, g)
        need = [r for r in rows if r not in stats]
        if need:
            stats.update(backward_row_stats(q, k, v, dout, block_size, causal, need,
                                            [sel_idx[r[0], r[2], r[1]] for r in need]))
        k_s = np.asarray(k[bb, s_pos, hk], dtype=np.float64)
        v_s = np.asarray(v[bb, s_pos, hk], dtype=np.float64)
        for (_, t, h) in rows:
            q64 = np.asarray(q[bb, t, h], dtype=np.float64)
            do64 = np.asarray(dout[bb, t, h], dtype=np.float64)
            lse, delta = stats[(bb, t, h)]
            p = math.exp(float(k_s @ q64) * scale - lse)
            dk[x] += scale * p * (float(v_s @ do64) - delta) * q64
            dv[x] += p * do64
    return dk, dv


# ----------------------------------------------------------------------------
# Decode: one new query per sequence against a cache of its keys and values
# ----------------------------------------------------------------------------
def decode_rows(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, lens: Sequence[int],
                block_size: int, topk: int, keep_scores: bool = False,
                rows: Optional[Sequence[Tuple[int, int]]] = None,
                given_sel: Optional[Sequence[Sequence[int]]] = None) -> "RowResult":
    """Decode-time MoBA: for sequence b with L = lens[b] cached positions (the
    new token's own key and value included), the new query q[b, h] sits at
    position t = L - 1 and is routed exactly as prefill row t would be
    (report §2.2 and §2.3): own block j = t // B (its keys jB..t), the top
    min(k-1, j) of the complete past blocks 0..j-1 by <q, mean key>, ties to
    the lower index, softmax over the union.  The pages evaluate MoBA with
    full attention during generation (report §4.4, §5.1) and name sparse
    decode as future work (report §6.3) without fixing its rule; this is the
    prefill rule applied to the last row.

    q: [batch, Hq, D]; k_cache, v_cache: [batch, Lmax, Hkv, D].  `rows`
    lists the (b, h) pairs to evaluate (default: all, b-major); `given_sel`,
    if set, replaces the gate's choice per row (checking an output under
    another valid top-k set after a near tie)."""
    b, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    B = block_size
    scale = 1.0 / math.sqrt(D)
    if rows is None:
        rows = [(bb, h) for bb in range(b) for h in range(Hq)]
    rows = list(rows)
    res = RowResult(len(rows), D, topk)
    order = sorted(range(len(rows)), key=lambda r: (rows[r][0], rows[r][1] // g, r))
    cur = None
    for r in order:
        bb, h = rows[r]
        L = int(lens[bb])
        if not 1 <= L <= k_cache.shape[1]:
            raise ValueError(f"cache length {L} outside [1, {k_cache.shape[1]}]")
        t = L - 1
        j = t // B
        hk = h // g
        if cur != (bb, hk):
            cur = (bb, hk)
            k_head = np.asarray(k_cache[bb, :L, hk, :], dtype=np.float64)
            v_head = np.asarray(v_cache[bb, :L, hk, :], dtype=np.float64)
            mu = k_head[:j * B].reshape(j, B, D).mean(axis=1)  # the complete past blocks
            absk = np.abs(k_head[:j * B]).reshape(j, B, D).mean(axis=1)
        q64 = np.asarray(q[bb, h], dtype=np.float64)
        scores = mu @ q64
        if given_sel is None:
            sel = select_blocks(np.concatenate([scores, [0.0]]), j, topk, True)
        else:
            sel = sorted(int(i) for i in given_sel[r] if i >= 0)
        res.out[r] = _attend_blocks(q64, k_head, v_head, sel, t, B, True, scale)
        res.sel[r, :len(sel)] = sel
        if keep_scores:
            res.scores[r] = scores
        m = min(topk - 1, j)
        if 0 < m < j:
            ranked = sorted(range(j), key=lambda i: (-float(scores[i]), i))
            res.gap[r] = float(scores[ranked[m - 1]] - scores[ranked[m]])
            res.boundary[r] = (scores[ranked[m - 1]], scores[ranked[m]])
        res.score_eps[r] = score_error_bound(q64, mu, absk, B) if j else 0.0
    return res


class RowResult:
    """Per-row oracle results: out [R, D], sel [R, topk] (-1 padded); for the
    gate check, the fp64 gap between the last chosen and the first unchosen
    candidate score and those two scores (`boundary`); and `score_eps`, a
    worst-case bound on the error of any one of the row's scores when it is
    formed in fp32 in any order (score_error_bound)."""

    def __init__(self, R: int, D: int, topk: int):
        self.out = np.zeros((R, D), dtype=np.float64)
        self.sel = np.full((R, topk), -1, dtype=np.int32)
        self.gap = np.full((R,), np.inf)
        self.boundary = np.zeros((R, 2))
        self.score_eps = np.zeros((R,))
        self.scores: List[Optional[np.ndarray]] = [None] * R


def moba_rows(q, k, v, block_size: int, topk: int, causal: bool,
              rows: Sequence[Tuple[int, int, int]], mu: Optional[np.ndarray] = None,
              given_sel: Optional[Sequence[Sequence[int]]] = None,
              keep_scores: bool = False, gate: str = "mean",
              minmax: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> RowResult:
    """MoBA forward for the listed rows (b, t, h) only.

    gate: "mean" (report §2.2) or "minmax" (the Quest-style variant, see the
    header).  `mu` (block_means of k) or `minmax` (block_minmax of k) may be
    passed in to avoid recomputing them.
    `given_sel`, if set, replaces the gate's choice for each row (used to check
    a row's output under another valid top-k set after a near tie).
    q, k, v can be any array type with numpy indexing (torch CPU tensors are
    converted per head)."""
    b, S, Hq, Hkv, D = _check_shapes(q, k, v, block_size, topk)
    B = block_size
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    if gate not in ("mean", "minmax"):
        raise ValueError("gate must be 'mean' or 'minmax'")
    if gate == "mean" and mu is None:
        mu = block_means(k, B)
    if gate == "minmax" and minmax is None:
        minmax = block_minmax(k, B)
    absk = None
    res = RowResult(len(rows), D, topk)
    # group rows by (batch, kv head) so each head's K/V is converted once
    order = sorted(range(len(rows)), key=lambda r: (rows[r][0], rows[r][2] // g, r))
    cur = None
    for r in order:
        bb, t, h = rows[r]
        hk = h // g
        if cur != (bb, hk):
            cur = (bb, hk)
            k_head = np.asarray(k[bb, :, hk, :], dtype=np.float64)
            v_head = np.asarray(v[bb, :, hk, :], dtype=np.float64)
            absk = np.abs(k_head).reshape(S // B, B, D).mean(axis=1)  # [n, D] mean |K| per block
        q64 = np.asarray(q[bb, t, h], dtype=np.float64)
        j = t // B
        if gate == "mean":
            scores = gate_scores(q64, mu[bb, hk])
        else:
            scores = gate_scores_minmax(q64, minmax[0][bb, hk], minmax[1][bb, hk])
        if given_sel is None:
            sel = select_blocks(scores, j, topk, causal)
        else:
            sel = sorted(int(i) for i in given_sel[r] if i >= 0)
        res.out[r] = _attend_blocks(q64, k_head, v_head, sel, t, B, causal, scale)
        res.sel[r, :len(sel)] = sel
        if keep_scores:
            res.scores[r] = scores
        # gate margin and fp32 error bound (used by the near-tie protocol)
        cand = list(range(j)) if causal else list(range(len(scores)))
        m = min(topk - 1, j) if causal else min(topk, len(scores))
        if 0 < m < len(cand):
            ranked = sorted(cand, key=lambda i: (-float(scores[i]), i))
            res.gap[r] = float(scores[ranked[m - 1]] - scores[ranked[m]])
            res.boundary[r] = (scores[ranked[m - 1]], scores[ranked[m]])
        if gate == "mean":
            res.score_eps[r] = score_error_bound(q64, mu[bb, hk], absk, B)
        else:
            res.score_eps[r] = score_error_bound_minmax(q64, minmax[0][bb, hk], minmax[1][bb, hk])
    return res


def near_tie_rows(res: "RowResult", rel: float = 1e-4,
                  abs_tol: Optional[np.ndarray] = None) -> np.ndarray:
    """Rows whose gate decision is a near tie: the fp64 gap between the last
    chosen and the first unchosen candidate score is at most `rel` times the
    larger of their magnitudes (the parity rule for the gate: selections must
    agree exactly except at such gaps; two exactly zero scores count too).  `abs_tol` (per row), if given, also
    counts gaps at or below it."""
    tie = res.gap <= rel * near_tie_scale(res)
    if abs_tol is not None:
        tie = tie | (res.gap <= np.asarray(abs_tol, dtype=np.float64))
    return tie


def near_tie_scale(res: "RowResult") -> np.ndarray:
    """Per row, the larger magnitude of the two boundary scores (the last
    chosen and the first unchosen), the scale of the relative gap."""
    return np.max(np.abs(res.boundary), axis=1)


# ----------------------------------------------------------------------------
# Near-tie protocol (test infrastructure for comparing an fp32 gate)
# ----------------------------------------------------------------------------
# The GPU ranks fp32 scores and this oracle ranks exact (fp64) ones.  The gate
# check therefore forgives a differing selection only where the fp64 gap at
# the top-k boundary is below 1e-4 of the scores' magnitude (near_tie_rows);
# the bounds below state how far an fp32 score can be from the exact one at
# worst, whatever the summation order (Higham, "Accuracy and Stability of
# Numerical Algorithms", section 3.1: gamma_n bounds n successive roundings).
def _gamma(n: int, u: float = 2.0 ** -24) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32 unit roundoff u."""
    return n * u / (1.0 - n * u)


def score_error_bound(q64: np.ndarray, mu_head: np.ndarray, absk_mean: np.ndarray, B: int) -> float:
    """An upper bound, over all blocks of this row, on |fp32 score - exact
    score| when the block mean is summed and the dot product is formed in fp32
    in any order: gamma_{3D+1} * sum|q_d mu_d| (the dot product, allowing the
    mean to be split into three exact bf16 parts) plus
    gamma_{B+2} * sum |q_d| mean|K_d| (the mean's sum and its division)."""
    D = q64.shape[0]
    dot = _gamma(3 * D + 1) * (np.abs(mu_head) @ np.abs(q64))
    mean = _gamma(B + 2) * (absk_mean @ np.abs(q64))
    return float(np.max(dot + mean))


def score_error_bound_minmax(q64: np.ndarray, lo_head: np.ndarray, hi_head: np.ndarray) -> float:
    """An upper bound, over all blocks of this row, on |fp32 score - exact
    score| for the min/max gate when the score is formed in fp32 in any order
    from exact products (q_d times the chosen bound, or the bf16 split
    q+ . hi + q- . lo over 2 D terms): gamma_{2D+1} * sum_d |q_d| max(|lo_d|, |hi_d|)."""
    D = q64.shape[0]
    mag = np.maximum(np.abs(lo_head), np.abs(hi_head)) @ np.abs(q64)
    return float(np.max(_gamma(2 * D + 1) * mag))


def valid_topk_set(scores: np.ndarray, chosen_past: Iterable[int], j: int, m: int, tol: float) -> bool:
    """Whether `chosen_past` is a top-m set of the candidate scores 0..j-1 up
    to `tol`: it has m distinct candidates and no unchosen candidate beats any
    chosen one by more than `tol`."""
    chosen = sorted(set(int(i) for i in chosen_past))
    if len(chosen) != m or any(i < 0 or i >= j for i in chosen):
        return False
    rest = [i for i in range(j) if i not in set(chosen)]
    if not rest or not chosen:
        return True
    return max(scores[i] for i in rest) <= min(scores[i] for i in chosen) + tol


def count_selected_keys(seqlen: int, block_size: int, topk: int, causal: bool) -> int:
    """Keys attended by one query head summed over all positions, from the
    selection rule alone (the gate picks exactly min(k-1, j) past blocks)."""
    B = block_size
    n = num_blocks(seqlen, B)
    total = 0
    for t in range(seqlen):
        j = t // B
        if causal:
            total += min(topk - 1, j) * B + (t - j * B + 1)
        else:
            total += min(topk, n) * B
    return total
