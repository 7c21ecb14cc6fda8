"""Whole-output comparison of large GPU results with the float64 dense oracle.

The full-size workloads are too large for one dense N x N float64 matrix of
every head at once (B=1, H=16, N=8192 needs 8 GiB), so the oracle is run head
by head on blocks of rows.  The definition is per row, so a block of rows is
the same computation (``oracle.dense_fwd(rows=...)``).  Every row of every head
is compared; the error statistics are accumulated over the whole tensor and
printed once per tensor.  Test helper only (no GPU code here).
"""
from __future__ import annotations

import concurrent.futures
import os
import sys
import threading

import numpy as np

import oracle


class ErrStats:
    """Running max abs error, squared-error sums and failure count of one tensor."""

    def __init__(self, name, atol, rtol):
        self.name, self.atol, self.rtol = name, atol, rtol
        self.lock = threading.Lock()
        self.max_abs = 0.0
        self.sq_err = 0.0
        self.sq_ref = 0.0
        self.n = 0
        self.fails = 0
        self.first_fail = None

    def add(self, got, ref, where):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (self.name, got.shape, ref.shape)
        # exact matches (including equal infinities) have zero error
        same = (got == ref)
        err = np.where(same, 0.0, np.abs(got - ref))
        bad = ~(err <= self.atol + self.rtol * np.abs(ref))
        fin = np.isfinite(ref)
        max_abs = float(err.max()) if err.size else 0.0
        sq_err = float(np.sum(np.where(fin, err, 0.0) ** 2))
        sq_ref = float(np.sum(np.where(fin, ref, 0.0) ** 2))
        nb = int(bad.sum())
        first = None
        if nb:
            idx = np.argwhere(bad)[0]
            first = (where, tuple(int(i) for i in idx), float(got[tuple(idx)]), float(ref[tuple(idx)]))
        with self.lock:
            self.max_abs = max(self.max_abs, max_abs)
            self.sq_err += sq_err
            self.sq_ref += sq_ref
            self.n += err.size
            if first is not None and self.first_fail is None:
                self.first_fail = first
            self.fails += nb

    def report(self, label="", floor=1e-300):
        """Print the statistics, assert no element failed, return the relative
        RMS error (the reference RMS taken as at least ``floor``)."""
        rel_rms = float(np.sqrt(self.sq_err / max(self.n, 1)) /
                        max(np.sqrt(self.sq_ref / max(self.n, 1)), floor))
        print(f"    {label}{self.name}: {self.n} elements, max_abs={self.max_abs:.3e} "
              f"rel_rms={rel_rms:.3e} fails={self.fails}", flush=True)
        sys.stdout.flush()
        assert self.fails == 0, (f"{label}{self.name}: {self.fails} of {self.n} elements out of "
                                 f"tolerance; first at {self.first_fail}")
        return rel_rms


def workers():
    """Threads for the per-head oracle work (numpy releases the GIL in its
    large array operations; BLAS threads add to these)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def for_each_head(B, H, fn):
    """Run fn(b, h) for every head on a thread pool; re-raises the first error."""
    with concurrent.futures.ThreadPoolExecutor(workers()) as ex:
        for f in [ex.submit(fn, b, h) for b in range(B) for h in range(H)]:
            f.result()


def _mask_of(block_mask, b, h):
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm[b if bm.shape[0] > 1 else 0, h if bm.shape[1] > 1 else 0]


def compare_fwd_all_rows(o, lse, x, causal, scale, tol, lse_tol, window=None, block_mask=None,
                         v=None, chunk=2048, label=""):
    """Compare o [B, H, N, d_v] and lse [B, H, N] (or None) with dense_fwd on
    every row of every head; tol and lse_tol are (atol, rtol).  ``v`` overrides
    x["v"] (values of another width)."""
    q, k = x["q"], x["k"]
    v = x["v"] if v is None else v
    B, H, N = q.shape[:3]
    so = ErrStats("O", *tol)
    sl = ErrStats("LSE", *lse_tol) if lse is not None else None

    def one_head(b, h):
        bm = _mask_of(block_mask, b, h)
        for r0 in range(0, N, chunk):
            rows = np.arange(r0, min(N, r0 + chunk))
            ro, rl = oracle.dense_fwd(q[b, h], k[b, h], v[b, h], causal=causal, scale=scale,
                                      rows=rows, window=window, block_mask=bm)
            so.add(o[b, h, rows], ro, (b, h, r0))
            if sl is not None:
                sl.add(lse[b, h, rows], rl, (b, h, r0))

    for_each_head(B, H, one_head)
    so.report(label)
    if sl is not None:
        sl.report(label)
    assert np.isfinite(o).all()


def compare_bwd_all_heads(grads, x, causal, scale, tol, rel_rms_max, heads=None, window=None,
                          block_mask=None, label=""):
    """Compare GPU gradients (dq, dk, dv as [B, H, N, .] arrays) with dense_bwd
    on every head (or the listed (b, h) heads); tol is (atol, rtol), and the
    relative RMS error of each tensor, per head and over all of them, must stay
    below rel_rms_max (references that vanish, e.g. the gradients of a single
    key, are measured against an RMS floor of 1e-3)."""
    B, H = x["q"].shape[:2]
    stats = [ErrStats(n, *tol) for n in ("dQ", "dK", "dV")]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = {}

    def one_head(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        bm = _mask_of(block_mask, b, h)
        ref = oracle.dense_bwd(x["q"][sl], x["k"][sl], x["v"][sl], x["do"][sl], causal=causal,
                               scale=scale, window=window,
                               block_mask=None if bm is None else bm[None, None])[:3]
        for st, g, r in zip(stats, grads, ref):
            st.add(g[sl], r, (b, h))
            e = np.asarray(g[sl], np.float64) - r
            rel = float(np.sqrt(np.mean(e ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-3))
            with st.lock:
                if rel > worst.get(st.name, (0.0, None))[0]:
                    worst[st.name] = (rel, (b, h))

    with concurrent.futures.ThreadPoolExecutor(workers()) as ex:
        for f in [ex.submit(one_head, b, h) for b, h in heads]:
            f.result()
    for st in stats:
        rel = st.report(label, floor=1e-3)
        assert rel < rel_rms_max, f"{label}{st.name}: relative RMS error {rel:.3e}"
        w_rel, w_head = worst.get(st.name, (0.0, None))
        print(f"    {label}{st.name}: worst head {w_head} rel_rms={w_rel:.3e}", flush=True)
        assert w_rel < rel_rms_max, f"{label}{st.name}: relative RMS error {w_rel:.3e} on head {w_head}"
