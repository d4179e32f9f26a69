"""Float64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Every function
works on float64 NumPy arrays holding the exact values the GPU receives
(bf16 or fp32 inputs widened without rounding); it shares no code with the
HIP kernels.

Layout: q, o, do are [B, H, Nq, d]; k, v are [B, H, Nk, d]; lse is
[B, H, Nq]; lengths is a length-B integer array of key lengths (or None for
"all Nk keys valid").  Usually Nq == Nk == N.  Packed batches (the *_packed
routines) hold the sequences back to back, head-major: q, o, do are
[H, total_q, d], k, v are [H, total_k, d], lse is [H, total_q], and sequence
b owns query rows cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1].

Semantics (the plain definition the tiled method reaches exactly):
  s_ij = scale * q_i . k_j,
  visible(i, j) = j < L_b and (not causal or j <= i + Nk - Nq);
  for a row with a non-empty visible set V_i:
      m_i = max_{j in V_i} s_ij,  l_i = sum_{j in V_i} exp(s_ij - m_i),
      O_i = sum_{j in V_i} exp(s_ij - m_i) v_j / l_i,  LSE_i = m_i + ln l_i;
  for a row with nothing visible: O_i = 0, LSE_i = -inf.
The pages define the causal mask for square problems (j <= i).  With Nq !=
Nk the queries are read as the last Nq positions of a sequence of Nk
("bottom-right" alignment: the last query sees every key), which keeps the
square case unchanged and makes one query against a cache see all of it.

Citations are to the three source pages:
  [clozo]  "What is FlashAttention?" (interview.clozo.ai)
  [deep]   "FlashAttention" (deepconcepts.dev)
  [infra]  "Explain FlashAttention and why it is IO-aware"
           (aiinfrainterviews.com)
"""

from __future__ import annotations


import numpy as np

__all__ = [
    "visible_mask",
    "scaled_scores",
    "attention_materialised",
    "attention_rows",
    "online_row",
    "attention_online",
    "attention_backward",
    "finite_difference_grads",
    "merge_states",
    "attention_decode",
    "attention_packed",
    "attention_backward_packed",
]


# ---------------------------------------------------------------------------
# Masks and scores
# ---------------------------------------------------------------------------

def _clamp_length(length, n):
    """Key length of one sequence, clamped to [0, n] (None means n)."""
    if length is None:
        return n
    return int(min(max(int(length), 0), n))


def visible_mask(rows, n_keys, causal, length=None, keys=None, offset=0):
    """Boolean [len(rows), len(keys)] mask of visible (query, key) pairs.

    `keys` are absolute key positions (default: all n_keys of them); query
    row i sits at sequence position i + offset (offset = Nk - Nq).
    Positions are absolute sequence positions, never tile-local ones
    ([infra] "Executable recurrence, with an empty-state policy": the causal
    mask uses global query and key positions across tile boundaries).  The
    key-length mask hides keys j >= L_b; query rows are not masked.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    keys = (np.arange(n_keys, dtype=np.int64) if keys is None
            else np.asarray(keys, dtype=np.int64).reshape(-1))
    vis = np.broadcast_to(keys[None, :] < _clamp_length(length, n_keys),
                          (rows.size, keys.size)).copy()
    if causal:
        vis &= keys[None, :] <= rows[:, None] + int(offset)
    return vis


def scaled_scores(q_rows, k, scale):
    """s = scale * q K^T for a block of query rows of one head.

    [infra] "Keep only the state needed for the final weighted average":
    scores are the query-key products times the scale, plus the mask.
    """
    return float(scale) * (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T)


# ---------------------------------------------------------------------------
# Route A: materialised stable softmax (the plain definition)
# ---------------------------------------------------------------------------

def _rows_materialised(q_rows, rows, k, v, scale, causal, length, offset=0):
    """O and LSE for the given absolute query rows of one head.

    Stable softmax with the row maximum subtracted before exponentiation
    ([deep] "Why it is allowed to be exact": subtracting the maximum keeps
    exp representable without changing the ratio).
    """
    s = scaled_scores(q_rows, k, scale)
    vis = visible_mask(rows, k.shape[0], causal, length, offset=offset)
    s = np.where(vis, s, -np.inf)
    nonempty = vis.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    o = np.zeros((q_rows.shape[0], v.shape[1]), np.float64)
    o[nonempty] = (p[nonempty] @ v) / l[nonempty, None]
    lse = np.full(q_rows.shape[0], -np.inf)
    lse[nonempty] = m[nonempty] + np.log(l[nonempty])
    return o, lse


def attention_materialised(q, k, v, scale, causal=False, lengths=None, row_block=512):
    """Route A: exact attention by materialising each score row block.

    This is the three-pass standard attention ([clozo] "Step 1: Why standard
    attention is memory-bound"), done on the CPU in float64, blocked over
    query rows only to bound host memory.  Returns (o, lse).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, N, d = q.shape
    offset = k.shape[2] - N
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        length = None if lengths is None else lengths[b]
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = _rows_materialised(
                    q[b, h, rows], rows, k[b, h], v[b, h], scale, causal, length, offset)
    return o, lse


def attention_rows(q_head, k_head, v_head, rows, scale, causal=False, length=None):
    """Route A restricted to selected absolute query rows of one head.

    Used to check sampled outputs of full-size problems row by row.
    """
    rows = np.asarray(rows, dtype=np.int64)
    offset = np.asarray(k_head).shape[0] - np.asarray(q_head).shape[0]
    return _rows_materialised(np.asarray(q_head, np.float64)[rows], rows,
                              np.asarray(k_head, np.float64),
                              np.asarray(v_head, np.float64),
                              scale, causal, length, offset)


# ---------------------------------------------------------------------------
# Route B: the online recurrence
# ---------------------------------------------------------------------------

def _fold_chunk(m, l, o, s, v, *, subtract_max=True, rescale=True):
    """Fold one chunk of keys into the running state of a set of rows.

    The state update of [infra] "Keep only the state needed for the final
    weighted average" (and [deep] "Why it is allowed to be exact"), for R
    rows at once: m (R,) running maxima, l (R,) running sums of exponentials
    relative to m, o (R, dv) value sums on the same scale; s (R, c) the
    chunk's scaled scores with -inf at keys a row does not see, v (c, dv)
    the chunk's value rows.  A row that sees no key of the chunk keeps its
    state (its factor is 1 and nothing is added), so -inf - (-inf) is never
    formed ([infra] "Executable recurrence, with an empty-state policy").

    `subtract_max` / `rescale` = False plant the two classic mistakes for the
    negative tests: the reference stays 0 instead of the running maximum, or
    the old sums are not multiplied by exp(m_old - m_new).

    Returns (m, l, o, factor, seen): the new state, the factor the old sums
    were multiplied by, and which rows saw a key in this chunk.
    """
    dt = l.dtype.type
    seen = np.any(~np.isneginf(s), axis=1)
    if subtract_max:
        ref = np.maximum(m, np.max(s, axis=1, initial=-np.inf))
    else:
        ref = np.zeros_like(m)
    ref = np.where(seen, ref, m)
    was_empty = np.isneginf(m)
    safe_gap = np.where(seen & ~was_empty, m - ref, dt(0.0))
    if rescale:
        factor = np.where(was_empty, dt(0.0), np.exp(safe_gap))
    else:
        factor = np.ones_like(l)
    factor = np.where(seen, factor, dt(1.0))
    safe_ref = np.where(seen, ref, dt(0.0))
    w = np.where(np.isneginf(s), dt(0.0), np.exp(s - safe_ref[:, None]))
    o_new = factor[:, None] * o + (w @ v).astype(o.dtype)
    l_new = factor * l + w.sum(axis=1, dtype=l.dtype)
    return ref.astype(m.dtype), l_new, o_new, factor, seen


def online_row(scores, values, tile=2, *, dtype=np.float64,
               subtract_max=True, rescale=True, return_state=False):
    """Online softmax-weighted average of value rows for ONE query.

    The single-row case of the state update `_fold_chunk` (the same update
    `attention_online` applies to every row of a head), run over consecutive
    chunks of `tile` scores; the result is o / l, or zeros when no score was
    visible ([infra] "Executable recurrence, with an empty-state policy").

    `scores` are already scaled and masked (-inf for masked keys).  The
    inputs must be well formed as that page requires: a positive integer
    tile, a 1-D score vector with one entry per row of a 2-D value matrix,
    scores finite or -inf, values finite.

    `subtract_max` and `rescale` exist ONLY so that negative tests can plant
    the two classic mistakes ([deep] "Why it is allowed to be exact": drop
    the rescale and the answer is wrong; drop the maximum subtraction and a
    x30 magnitude overflows float32).  `dtype` selects the working precision
    (float64 by default; float32 for the overflow demonstration).

    Returns the output vector, or (output, trace) with return_state=True,
    where trace lists (m, factor, l, o) after every chunk that held a visible
    score.
    """
    if type(tile) is not int or tile < 1:
        raise ValueError("tile must be a positive int")
    s_row = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim != 2 or s_row.shape != (vals.shape[0],):
        raise ValueError("need exactly one score per value row")
    if np.isnan(s_row).any() or (s_row == np.inf).any():
        raise ValueError("scores must be finite or -inf")
    if not np.isfinite(vals).all():
        raise ValueError("values must be finite")

    dt = np.dtype(dtype).type
    s_row = s_row.astype(dtype)
    vals = vals.astype(dtype)
    m = np.full(1, -np.inf, dtype)
    l = np.zeros(1, dtype)
    o = np.zeros((1, vals.shape[1]), dtype)
    trace = []
    n = s_row.shape[0]
    with np.errstate(over="ignore", invalid="ignore"):
        for c0 in range(0, n, tile):
            c1 = min(n, c0 + tile)
            m, l, o, factor, seen = _fold_chunk(
                m, l, o, s_row[None, c0:c1], vals[c0:c1],
                subtract_max=subtract_max, rescale=rescale)
            if seen[0]:
                trace.append((float(m[0]), float(factor[0]), float(l[0]),
                              o[0].astype(np.float64).copy()))
        out = o[0] / l[0] if l[0] != dt(0.0) else np.zeros_like(o[0])
    if return_state:
        return out.astype(np.float64), trace
    return out.astype(np.float64)


def attention_online(q, k, v, scale, causal=False, lengths=None, tile=64,
                     return_state=False):
    """Route B: the online recurrence over key chunks of width `tile`.

    Vectorised over all query rows of a head; each chunk is folded into the
    per-row state (m, l, o) by `_fold_chunk` ([infra] "Keep only the state
    needed for the final weighted average"; [deep] "Why it is allowed to be
    exact": rescale both sums by exp(m_old - m_new), divide by l after the
    last chunk).  Rows for which a chunk is fully masked keep their state
    ([infra] "Executable recurrence, with an empty-state policy").  Shares
    no code with route A beyond the mask and score helpers.

    Returns (o, lse) or, with return_state=True, (o, lse, m, l).
    """
    if type(tile) is not int or tile < 1:
        raise ValueError("tile must be a positive int")
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, N, v.shape[3]))
    LSE = np.empty((B, H, N))
    M = np.empty((B, H, N))
    L = np.empty((B, H, N))
    rows = np.arange(N)
    for b in range(B):
        length = None if lengths is None else lengths[b]
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            o = np.zeros((N, v.shape[3]))
            for j0 in range(0, Nk, tile):
                keys = np.arange(j0, min(Nk, j0 + tile))
                vis = visible_mask(rows, Nk, causal, length, keys=keys, offset=Nk - N)
                live = vis.any(axis=1)            # rows with something visible here
                if not live.any():
                    continue
                s = np.where(vis[live], scaled_scores(q[b, h, live], k[b, h, keys], scale),
                             -np.inf)
                m[live], l[live], o[live], _, _ = _fold_chunk(m[live], l[live], o[live], s,
                                                             v[b, h, keys])
            done = l > 0
            O[b, h, done] = o[done] / l[done, None]
            LSE[b, h] = np.where(done, m + np.log(np.where(done, l, 1.0)), -np.inf)
            M[b, h] = m
            L[b, h] = l
    if return_state:
        return O, LSE, M, L
    return O, LSE


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def attention_backward(q, k, v, o, do, lse, scale, causal=False, lengths=None,
                       row_block=512):
    """Exact gradients of the scalar <dO, O> with respect to Q, K and V.

    The pages fix only that the backward rebuilds S and P from Q, K, V and
    the saved output and per-row statistics ([clozo] "Step 4: The backward
    pass recomputes instead of storing"; [deep] "What it does not do").  The
    formulas are the textbook softmax Jacobian, pinned by finite differences:
        P_ij = exp(s_ij - LSE_i) on visible pairs, 0 elsewhere;
        dV = P^T dO;  dP = dO V^T;  D_i = sum_t dO_it O_it;
        dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
    Rows with nothing visible (LSE = -inf) contribute nothing.
    Returns (dq, dk, dv).
    """
    q, k, v, o, do = (np.asarray(t, np.float64) for t in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        length = None if lengths is None else lengths[b]
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                s = scaled_scores(q[b, h, rows], k[b, h], scale)
                vis = visible_mask(rows, k.shape[2], causal, length, offset=k.shape[2] - N)
                row_lse = lse[b, h, rows]
                ok = vis & np.isfinite(row_lse)[:, None]
                p = np.where(ok, np.exp(np.where(ok, s - row_lse[:, None], 0.0)), 0.0)
                g = do[b, h, rows]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                D = np.sum(g * o[b, h, rows], axis=1)
                ds = p * (dp - D[:, None])
                dq[b, h, rows] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv


def finite_difference_grads(q, k, v, do, scale, causal=False, lengths=None, eps=1e-6):
    """Central finite differences of <dO, O(q, k, v)> for every input element.

    Brute-force check of attention_backward on tiny inputs; the forward used
    is route A.  Cost is 2 * (#elements) forward passes.
    """
    q, k, v, do = (np.array(t, np.float64) for t in (q, k, v, do))

    def loss(qq, kk, vv):
        o, _ = attention_materialised(qq, kk, vv, scale, causal, lengths)
        return float(np.sum(o * do))

    grads = []
    for which in range(3):
        base = [q, k, v]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            g[idx] = (loss(*plus) - loss(*minus)) / (2.0 * eps)
        grads.append(g)
    return tuple(grads)


# ---------------------------------------------------------------------------
# Decoding against a key/value cache, split over the key dimension
# ---------------------------------------------------------------------------

def merge_states(o_parts, lse_parts):
    """Combine partial results of one softmax row computed over disjoint key sets.

    [deep] "What it does not do": at decode time the useful parallelism is
    across the sequence dimension (flash-decoding).  Each part s covers its own
    keys and yields the normalised partial output o_s and
    lse_s = ln sum_{j in s} exp(s_j).  Writing lse_s = m_s + ln l_s, this is the
    rescale-and-add step of the online recurrence ([clozo] "Step 2";
    [infra] "Keep only the state needed for the final weighted average")
    applied to whole parts:
        LSE = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - LSE) o_s.
    The largest lse is subtracted before exponentiating.  Parts with
    lse_s = -inf (no visible key) contribute nothing; when every part is empty
    O = 0 and LSE = -inf (the empty-row policy of [infra] "Executable
    recurrence, with an empty-state policy").

    o_parts: [..., S, d]; lse_parts: [..., S].  Returns (O [..., d], LSE [...]).
    """
    o = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    nonempty = np.isfinite(m)
    m_safe = np.where(nonempty, m, 0.0)
    w = np.where(np.isneginf(lse), 0.0, np.exp(lse - m_safe))
    total = w.sum(axis=-1, keepdims=True)
    total_safe = np.where(nonempty, total, 1.0)
    out = (w[..., None] * o).sum(axis=-2) / total_safe
    out = np.where(nonempty, out, 0.0)
    lse_out = np.where(nonempty, m_safe + np.log(total_safe), -np.inf)
    return out, lse_out[..., 0]


def attention_decode(q, k, v, scale, lengths=None, chunk=None):
    """One new query row per (batch, head) against a key/value cache.

    q: [B, H, d]; k, v: [B, H, N, d] (cache of capacity N); the query attends
    to every cached key j < L_b ([deep] "What it does not do": a decode step
    has a single query row and reads the whole cache, one score per key).
    chunk=None computes the plain definition (one materialised score row);
    chunk=C splits the keys into parts [0, C), [C, 2C), ..., computes each
    part's (o_s, lse_s) by the plain definition on its own keys, and combines
    them with merge_states.  Returns (O [B, H, d], LSE [B, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = k.shape
    o = np.zeros((B, H, v.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = _clamp_length(None if lengths is None else lengths[b], N)
        bounds = [(0, L)] if chunk is None else [(c0, min(c0 + chunk, L))
                                                 for c0 in range(0, max(L, 1), chunk)]
        for h in range(H):
            parts_o, parts_lse = [], []
            for c0, c1 in bounds:
                if c1 <= c0:
                    parts_o.append(np.zeros(v.shape[3]))
                    parts_lse.append(-np.inf)
                    continue
                s = scale * (k[b, h, c0:c1] @ q[b, h])
                m = s.max()
                e = np.exp(s - m)
                parts_o.append(e @ v[b, h, c0:c1] / e.sum())
                parts_lse.append(m + np.log(e.sum()))
            o[b, h], lse[b, h] = merge_states(np.array(parts_o), np.array(parts_lse))
    return o, lse


# ---------------------------------------------------------------------------
# Packed batches
# ---------------------------------------------------------------------------
#
# The pages treat one sequence at a time; a packed batch is read as a set of
# independent problems of that definition, one per sequence (its own Nq_b
# queries, its own Nk_b keys, the causal offset Nk_b - Nq_b of its own).
# Rows that belong to no sequence are left at O = 0, LSE = -inf and zero
# gradients.

def _packed_spans(cu):
    cu = np.asarray(cu, dtype=np.int64).reshape(-1)
    return [(int(cu[b]), int(cu[b + 1])) for b in range(cu.size - 1)]


def attention_packed(q, k, v, cu_q, cu_k, scale, causal=False):
    """Forward over a packed batch: each sequence is one problem of the plain
    definition (attention_materialised on its rows).  Returns (O, LSE)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    H, total_q, _ = q.shape
    o = np.zeros((H, total_q, v.shape[2]))
    lse = np.full((H, total_q), -np.inf)
    for (q0, q1), (k0, k1) in zip(_packed_spans(cu_q), _packed_spans(cu_k)):
        if q1 <= q0:
            continue
        ob, lb = attention_materialised(q[None, :, q0:q1], k[None, :, k0:k1],
                                        v[None, :, k0:k1], scale, causal)
        o[:, q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def attention_backward_packed(q, k, v, o, do, lse, cu_q, cu_k, scale, causal=False):
    """Gradients over a packed batch, one attention_backward per sequence.
    Returns (dq, dk, dv) in the packed layout."""
    q, k, v, o, do = (np.asarray(t, np.float64) for t in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for (q0, q1), (k0, k1) in zip(_packed_spans(cu_q), _packed_spans(cu_k)):
        if q1 <= q0 or k1 <= k0:
            continue
        g = attention_backward(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1],
                               o[None, :, q0:q1], do[None, :, q0:q1], lse[None, :, q0:q1],
                               scale, causal)
        dq[:, q0:q1] = g[0][0]
        dk[:, k0:k1] = g[1][0]
        dv[:, k0:k1] = g[2][0]
    return dq, dk, dv
