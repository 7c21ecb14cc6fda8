"""CPU oracle for exact attention, forward and backward, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module: only the tests, the package's smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

Contents
--------
``dense_fwd``    the materialised definition: scores, masked row softmax, P V.
``online_fwd``   the tiled Q-block-outer / key-block-inner forward with the
                 running (max m, denominator l, unnormalised numerator a) row
                 state, written from the online-softmax description.
``dense_bwd``    the textbook gradient of softmax attention, recomputing P
                 from Q, K and the log-sum-exp.
``transfer_ledger``  the element-transfer count of the explorer's declared
                 dense and tiled schedules.
``online_fwd_kv_outer``  the original key/value-outer loop order with the
                 normalised in-place output update.
``loop_order_ledger``  element transfers of the query-outer and the
                 key/value-outer orders, causal skipping included.

Conventions shared by all functions (readings of the pages where they are
silent; each is also listed with the design notes):

* Tensors are [..., N, d] arrays (any leading batch/head axes); every head is
  independent.  Arithmetic is float64 whatever the input dtype.
* Scores are ``scale * q_i . k_j``; the scale multiplies the raw dot product
  before the maximum is taken.
* Causal: key j is visible to query i iff j <= i (lower-triangular mask with
  -inf fill, as in nanoGPT's manual attention quoted on "FlashAttention -- the
  same attention, made memory-aware", section 00).
* Sliding window (``window`` = W, causal only): key j is visible to query i iff
  i - W < j <= i, the W most recent keys including the query's own position.
  This is a further key set whose blocks can be skipped like the causal
  upper triangle ("Flash Attention: IO-Aware Exact Attention", section
  "Storage, arithmetic and IO are separate quantities", on skipped blocks
  changing which pairs are computed); the window's definition is a reading,
  not a page fact.
* Block-sparse mask (``block_mask``, blocks of ``block`` = 64 queries by 64
  keys): key j is visible to query i iff block_mask[..., i // 64, j // 64] is
  nonzero, and-ed with the causal mask when that is on.  The pages name
  masks that skip whole blocks only as a change of which pairs are computed
  ("Flash Attention: IO-Aware Exact Attention", section "Storage, arithmetic
  and IO are separate quantities"); the block size and the layout
  [..., ceil(N / 64), ceil(N / 64)] (leading axes broadcast over batch and
  head) are a reading.  A row that sees no key at all has O = 0 and
  LSE = -inf (an empty sum), also a reading.
* The saved per-row statistic is the natural-log log-sum-exp of the scaled,
  masked scores: LSE_i = m_i + ln(l_i).
"""
from __future__ import annotations

import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_window(causal, window):
    if window is not None:
        if not causal:
            raise ValueError("a sliding window is defined for causal attention only")
        if int(window) < 1:
            raise ValueError("window must be >= 1")


BLOCK = 64  # block-sparse mask granularity (queries and keys)


def _scores(q, k, scale, causal, rows=None, window=None, block_mask=None):
    """Scaled scores S[..., i, j] = scale * q_i . k_j with the causal (and
    sliding-window, or block-sparse) mask applied.

    ``rows`` optionally restricts the queries to the given indices (the
    definition is per row, so a subset of rows is the same computation).
    """
    _check_window(causal, window)
    q = _as64(q)
    k = _as64(k)
    qi = q if rows is None else q[..., rows, :]
    s = (qi @ np.swapaxes(k, -1, -2)) * float(scale)
    n_k = k.shape[-2]
    r = np.arange(q.shape[-2]) if rows is None else np.asarray(rows)
    j = np.arange(n_k)
    if causal:
        visible = j[None, :] <= r[:, None]
        if window is not None:
            visible = visible & (j[None, :] > r[:, None] - int(window))
        s = np.where(visible, s, -np.inf)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        n_qb, n_kb = -(-q.shape[-2] // BLOCK), -(-n_k // BLOCK)
        if bm.shape[-2:] != (n_qb, n_kb):
            raise ValueError(f"block_mask must end in ({n_qb}, {n_kb}), got {bm.shape}")
        # visible[..., i, j] = bm[..., i // 64, j // 64]
        rows_of = np.take(bm, r // BLOCK, axis=-2)
        visible = np.take(rows_of, j // BLOCK, axis=-1)
        s = np.where(visible, s, -np.inf)
    return s


def dense_fwd(q, k, v, causal=False, scale=None, rows=None, window=None, block_mask=None):
    """Materialised attention O = softmax(scale * Q K^T) V and its row LSE.

    Follows the dense three-step path ("Flash Attention: IO-Aware Exact
    Attention", section "Why intermediate matrices cost memory traffic"): form
    every score S, normalise each row of S by its own max and sum to get P, then
    multiply P by V.  The same steps are nanoGPT's manual attention on
    "FlashAttention -- the same attention, made memory-aware", section 00.

    Returns ``(o, lse)`` with o [..., R, d_v] and lse [..., R] in float64, where R
    is N or ``len(rows)``.
    """
    q = _as64(q)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = _scores(q, k, scale, causal, rows, window, block_mask)
    m = s.max(axis=-1, keepdims=True)
    seen = np.isfinite(m)                      # rows with at least one visible key
    e = np.exp(s - np.where(seen, m, 0.0))     # hidden keys: exp(-inf) = 0
    ell = e.sum(axis=-1, keepdims=True)
    p = np.where(seen, e / np.where(seen, ell, 1.0), 0.0)
    o = p @ _as64(v)
    with np.errstate(divide="ignore"):
        lse = np.where(seen[..., 0], m[..., 0] + np.log(ell[..., 0]), -np.inf)
    return o, lse


def dense_probs(q, k, causal=False, scale=None, window=None, block_mask=None):
    """The normalised probability matrix P of the dense path (for row-sum checks);
    rows with no visible key are all zero."""
    q = _as64(q)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = _scores(q, k, scale, causal, window=window, block_mask=block_mask)
    m = s.max(axis=-1, keepdims=True)
    seen = np.isfinite(m)
    e = np.exp(s - np.where(seen, m, 0.0))
    return np.where(seen, e / np.where(seen, e.sum(axis=-1, keepdims=True), 1.0), 0.0)


def _tile_summary(t, v_tile):
    """Summary of one tile for each row: its largest score m_t, the sum
    l_t = sum_j exp(t_j - m_t) and the d_v-wide a_t = sum_j exp(t_j - m_t) v_j.
    A row whose scores in the tile are all -inf (masked) has m_t = -inf,
    l_t = 0 and a_t = 0: the summary of no key."""
    m_t = t.max(axis=1)
    seen = np.isfinite(m_t)
    e = np.where(seen[:, None], np.exp(t - np.where(seen, m_t, 0.0)[:, None]), 0.0)
    return m_t, e.sum(axis=1), e @ v_tile


def _merge(first, second):
    """Combine the summaries of two disjoint key sets into the summary of
    their union: both are moved to the larger maximum before they are added,
    a summary of no key (m = -inf) weighing 0.  The operation is associative
    and commutative, so the result does not depend on how the keys were
    grouped into tiles or in what order the tiles came."""
    m1, l1, a1 = first
    m2, l2, a2 = second
    m = np.maximum(m1, m2)
    ref = np.where(np.isfinite(m), m, 0.0)
    w1 = np.where(np.isfinite(m1), np.exp(m1 - ref), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(m2 - ref), 0.0)
    return m, w1 * l1 + w2 * l2, w1[:, None] * a1 + w2[:, None] * a2


def online_fwd(q, k, v, causal=False, scale=None, query_block=2, key_block=2, trace=None,
               window=None):
    """Tiled forward with the online softmax, one head at a time.

    Loop order: query blocks outside, key/value blocks inside; each query block
    keeps its row state resident while every key tile passes ("Flash Attention:
    IO-Aware Exact Attention", section "Loop order changes which data is
    reloaded").  The row state is a running maximum ``m``, a denominator ``l``
    and a d_v-wide unnormalised numerator ``a`` (section "Online softmax makes
    tiling exact" of the same page; its displayed formulas did not survive
    extraction, and this is the reading that the page's own CPU check, the
    two-block worked example on Road to Intelligence "FlashAttention", section
    "The trick that makes tiling possible", and section 03 of "FlashAttention
    -- the same attention, made memory-aware" agree on).

    Here the state is the merge (``_merge``) of the summaries (``_tile_summary``)
    of the tiles seen so far: a row starts from the summary of no key
    (m = -inf, l = 0, a = 0), and each tile's summary is merged into it.  The
    merge moves both sides to the new maximum m' = max(m, m_t): the old state
    is scaled by alpha = exp(m - m') (zero while no key was seen), the tile's
    by exp(m_t - m'), which is the page's update l' = alpha l + sum_j p_j,
    a' = alpha a + sum_j p_j V_tile[j] with p_j = exp(t_j - m').  At the end
    O = a / l (one division, the unnormalised FlashAttention-2 form) and
    LSE = m + ln l.

    Masked keys (causal j > i, or j <= i - window) have t_j = -inf and
    contribute nothing; a row all of whose keys so far are masked keeps the
    summary of no key.  Tail tiles are simply shorter (keys beyond N do not
    exist); tiles larger than N are allowed.

    ``trace``, when a list, receives one dict per (query block, key tile) with
    copies of the state after that tile: keys ``row0``, ``col0``, ``m``, ``l``, ``a``.
    """
    _check_window(causal, window)
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    lead = q.shape[:-2]
    n_q, n_k = q.shape[-2], k.shape[-2]
    dv = v.shape[-1]
    qf = q.reshape((-1, n_q, q.shape[-1]))
    kf = k.reshape((-1, n_k, k.shape[-1]))
    vf = v.reshape((-1, n_k, dv))
    out = np.empty((qf.shape[0], n_q, dv))
    lse = np.empty((qf.shape[0], n_q))
    for h in range(qf.shape[0]):
        for row0 in range(0, n_q, query_block):
            rows = np.arange(row0, min(n_q, row0 + query_block))
            query = qf[h, rows]
            state = (np.full(len(rows), -np.inf), np.zeros(len(rows)), np.zeros((len(rows), dv)))
            for col0 in range(0, n_k, key_block):
                cols = np.arange(col0, min(n_k, col0 + key_block))
                t = (query @ kf[h, cols].T) * scale
                if causal:
                    t = np.where(cols[None, :] <= rows[:, None], t, -np.inf)
                if window is not None:
                    t = np.where(cols[None, :] > rows[:, None] - int(window), t, -np.inf)
                state = _merge(state, _tile_summary(t, vf[h, cols]))
                if trace is not None:
                    m, ell, a = state
                    trace.append({"head": h, "row0": row0, "col0": col0,
                                  "m": m.copy(), "l": ell.copy(), "a": a.copy()})
            m, ell, a = state
            out[h, rows] = a / ell[:, None]
            lse[h, rows] = m + np.log(ell)
    return out.reshape(lead + (n_q, dv)), lse.reshape(lead + (n_q,))


def online_fwd_kv_outer(q, k, v, causal=False, scale=None, query_block=2, key_block=2):
    """Tiled forward in the original loop order: key/value tiles outside,
    query blocks inside, with a normalised output updated in place.

    "FlashAttention -- the same attention, made memory-aware", section 04
    gives the loop nest (one K/V tile loaded, then every query tile visited
    under it) and section 03 the merge of one tile into a query block's running
    answer; "Flash Attention: IO-Aware Exact Attention", section "Loop order
    changes which data is reloaded", names this the original algorithm, which
    reloads Q and the row state for every K/V block.  For a query block with
    state (O, m, l) and a tile of scores t and values V_tile:

        m_t = max_j t_j,   P = exp(t - m_t),   l_t = sum_j P_j
        m' = max(m, m_t)
        l' = exp(m - m') l + exp(m_t - m') l_t
        O' = (l exp(m - m') O + exp(m_t - m') P V_tile) / l'

    State starts at O = 0, m = -inf, l = 0 (the exp of -inf is 0); rows whose
    keys are all masked in a tile leave their state unchanged.  Returns (O, LSE)
    with LSE = m + ln l, as ``dense_fwd``.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    lead = q.shape[:-2]
    n_q, n_k = q.shape[-2], k.shape[-2]
    dv = v.shape[-1]
    qf = q.reshape((-1, n_q, q.shape[-1]))
    kf = k.reshape((-1, n_k, k.shape[-1]))
    vf = v.reshape((-1, n_k, dv))
    out = np.zeros((qf.shape[0], n_q, dv))
    m = np.full((qf.shape[0], n_q), -np.inf)
    ell = np.zeros((qf.shape[0], n_q))
    for h in range(qf.shape[0]):
        for col0 in range(0, n_k, key_block):              # outer: key/value tiles
            cols = np.arange(col0, min(n_k, col0 + key_block))
            for row0 in range(0, n_q, query_block):        # inner: query tiles
                rows = np.arange(row0, min(n_q, row0 + query_block))
                t = (qf[h, rows] @ kf[h, cols].T) * scale
                if causal:
                    t = np.where(cols[None, :] <= rows[:, None], t, -np.inf)
                m_t = t.max(axis=1)
                hit = np.isfinite(m_t)                     # rows with a visible key here
                if not hit.any():
                    continue
                r = rows[hit]
                t, m_t = t[hit], m_t[hit]
                p = np.exp(t - m_t[:, None])
                l_t = p.sum(axis=1)
                m_old, l_old = m[h, r], ell[h, r]
                m_new = np.maximum(m_old, m_t)
                keep = np.where(np.isfinite(m_old), np.exp(m_old - m_new), 0.0)
                take = np.exp(m_t - m_new)
                l_new = keep * l_old + take * l_t
                out[h, r] = ((l_old * keep)[:, None] * out[h, r]
                             + take[:, None] * (p @ vf[h, cols])) / l_new[:, None]
                m[h, r], ell[h, r] = m_new, l_new
    lse = m + np.log(ell)
    return out.reshape(lead + (n_q, dv)), lse.reshape(lead + (n_q,))


def loop_order_ledger(n, d, dv, query_block, key_block, order, causal=False):
    """Element transfers between device memory and the chip for one head under
    the two loop orders, counted by walking the loops ("Flash Attention:
    IO-Aware Exact Attention", section "Loop order changes which data is
    reloaded"; its counts assume the working set fits on chip and exclude
    caches, as here).

    ``order="q_outer"``: a query block is read once, its output block and
    per-row statistic (one LSE value) written once; every K and V tile it can
    see is read once per query block.
    ``order="kv_outer"``: every K and V tile is read once; for every (tile,
    query block) pair with a visible key the query block is read, the row
    state (output block and two statistics per row, m and l) is read unless
    this is the block's first visit, and the state is written back.

    Causal skips the (query block, key tile) pairs in which no key is visible.
    Returns a dict of element counts per transfer and their ``total``.
    """
    if order not in ("q_outer", "kv_outer"):
        raise ValueError("order must be 'q_outer' or 'kv_outer'")
    c = {"Q_read": 0, "K_read": 0, "V_read": 0, "O_read": 0, "O_write": 0,
         "stat_read": 0, "stat_write": 0}
    blocks = [(r0, min(n, r0 + query_block)) for r0 in range(0, n, query_block)]
    tiles = [(c0, min(n, c0 + key_block)) for c0 in range(0, n, key_block)]

    def visible(b, t):
        return (not causal) or t[0] <= b[1] - 1   # first key <= last row

    if order == "q_outer":
        for b in blocks:
            rows = b[1] - b[0]
            c["Q_read"] += rows * d
            for t in tiles:
                if visible(b, t):
                    c["K_read"] += (t[1] - t[0]) * d
                    c["V_read"] += (t[1] - t[0]) * dv
            c["O_write"] += rows * dv
            c["stat_write"] += rows
    else:
        seen = set()
        for t in tiles:
            c["K_read"] += (t[1] - t[0]) * d
            c["V_read"] += (t[1] - t[0]) * dv
            for b in blocks:
                if not visible(b, t):
                    continue
                rows = b[1] - b[0]
                c["Q_read"] += rows * d
                if b in seen:
                    c["O_read"] += rows * dv
                    c["stat_read"] += 2 * rows
                seen.add(b)
                c["O_write"] += rows * dv
                c["stat_write"] += 2 * rows
    c["total"] = sum(c.values())
    return c


def dense_bwd(q, k, v, do, causal=False, scale=None, window=None, block_mask=None):
    """Gradients of L = sum(O * dO) for O = softmax(scale * Q K^T) V.

    The pages state only that the backward pass recomputes the score and
    probability tiles from Q, K, V and the saved normalisation statistics
    instead of storing them ("Flash Attention: IO-Aware Exact Attention",
    section "Storage, arithmetic and IO are separate quantities"; Road to
    Intelligence "FlashAttention", section "The trick that makes tiling
    possible").  The gradient itself is the textbook one of a row softmax
    followed by a matrix product, written out here without autograd:

        P    = exp(S - LSE)                 (recomputed)
        dV   = P^T dO
        dP   = dO V^T
        D_i  = sum_c dO_ic O_ic             (= sum_j P_ij dP_ij)
        dS   = P * (dP - D)
        dQ   = scale * dS K
        dK   = scale * dS^T Q

    Returns ``(dq, dk, dv, o, lse)`` in float64.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    o, lse = dense_fwd(q, k, v, causal, scale, window=window, block_mask=block_mask)
    s = _scores(q, k, scale, causal, window=window, block_mask=block_mask)
    seen = np.isfinite(lse)[..., None]         # a row with no visible key has P = 0
    p = np.where(seen, np.exp(s - np.where(seen, lse[..., None], 0.0)), 0.0)
    kt = np.swapaxes
    dv = kt(p, -1, -2) @ do
    dp = do @ kt(v, -1, -2)
    D = (do * o).sum(axis=-1, keepdims=True)
    ds = p * (dp - D)
    dq = scale * (ds @ k)
    dk = scale * (kt(ds, -1, -2) @ q)
    return dq, dk, dv, o, lse


def sampled_bwd(q, k, v, do, causal=False, scale=None, rows=(), cols=(), chunk=1024):
    """The gradients of dense_bwd for one head ([N, d] arrays, d_v for v and
    do), restricted to the listed query rows (dQ) and key columns (dK, dV), for
    sequences whose N x N matrices do not fit in memory.

    Same definitions as dense_bwd: P = exp(S - LSE), dP = dO V^T,
    D_i = sum_c dO_ic O_ic, dS = P * (dP - D), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO.  Every query row enters dK and dV of a key,
    so the rows are visited in chunks: each chunk forms its scores against all
    keys, its LSE, O and D, adds its share of dK and dV of the listed keys, and
    gives dQ of the listed rows it holds.  Returns ``(dq, dk, dv)`` in float64,
    shaped [len(rows), d], [len(cols), d], [len(cols), d_v].
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    n = q.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    dq = np.zeros((len(rows), q.shape[1]))
    dk = np.zeros((len(cols), k.shape[1]))
    dv = np.zeros((len(cols), v.shape[1]))
    for r0 in range(0, n, chunk):
        r = np.arange(r0, min(n, r0 + chunk))
        s = _scores(q, k, scale, causal, rows=r)           # [c, N]
        m = s.max(axis=-1, keepdims=True)
        lse = m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True))
        p = np.exp(s - lse)
        o = p @ v
        D = (do[r] * o).sum(axis=-1, keepdims=True)
        # the listed keys: dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij q_i
        pc = p[:, cols]
        dsc = pc * (do[r] @ v[cols].T - D)
        dv += pc.T @ do[r]
        dk += scale * (dsc.T @ q[r])
        # the listed rows in this chunk: dQ_i = scale sum_j dS_ij k_j
        mine = np.nonzero((rows >= r0) & (rows < r0 + len(r)))[0]
        if len(mine):
            loc = rows[mine] - r0
            ds = p[loc] * (do[rows[mine]] @ v.T - D[loc])
            dq[mine] = scale * (ds @ k)
    return dq, dk, dv


def transfer_ledger(n, d, dv, query_block, key_block):
    """Count element transfers of the explorer's declared dense and tiled schedules.

    Both schedules keep one query block resident and stream every key/value
    tile past it ("Flash Attention: IO-Aware Exact Attention", section "Loop
    order changes which data is reloaded"): a query block is read once, every
    K and V tile is read once per query block, the output block is written
    once.  The dense schedule additionally writes each score tile to HBM, reads
    it back for the softmax, writes the probability tile and reads it back for
    the product with V.  The walk below visits the tiles in loop order and adds
    up the elements each step moves; caches and spills are not modelled.
    """
    tiled = {"Q_read": 0, "K_read": 0, "V_read": 0, "O_write": 0}
    extra = {"S_write": 0, "S_read": 0, "P_write": 0, "P_read": 0}
    for row0 in range(0, n, query_block):
        rows = min(n, row0 + query_block) - row0
        tiled["Q_read"] += rows * d
        for col0 in range(0, n, key_block):
            cols = min(n, col0 + key_block) - col0
            tiled["K_read"] += cols * d
            tiled["V_read"] += cols * dv
            extra["S_write"] += rows * cols
            extra["S_read"] += rows * cols
            extra["P_write"] += rows * cols
            extra["P_read"] += rows * cols
        tiled["O_write"] += rows * dv
    dense = dict(tiled, **extra)
    return {"tiled": tiled, "dense": dense,
            "tiled_total": sum(tiled.values()), "dense_total": sum(dense.values())}
