"""GPU parity at the sizes the kernels' loops and grids reach.

* One head of N = 65536 (d = 128, bf16), causal and unmasked: O and LSE on
  sampled rows -- the first and last rows, rows on both sides of the 32-row
  wave, 256-row workgroup and 64-key tile edges, and seeded random rows --
  against ``oracle.dense_fwd`` on those rows (the definition is per row).
* The backward of one causal head of N = 32768 (d = 128, bf16): dQ on
  sampled rows and dK, dV on sampled key columns against
  ``oracle.sampled_bwd``, and two identities over all keys: every row of dS
  sums to zero, so sum_j dK_j = 0, and every row of P sums to one, so
  sum_j dV_j = sum_i dO_i.
* A grid of 2048 heads (B = 64, H = 32, N = 256, d = 64, bf16, causal): the
  forward on every row of every head and the backward on every head.

Tolerances as elsewhere: |err| <= 2e-2 + 1e-2 |ref| on O, dQ, dK, dV and
1e-4 + 1e-5 |ref| on the fp32 LSE.
"""
import sys

import numpy as np
import pytest

import oracle
import whole_output
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "lse": (1e-4, 1e-5)}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_12_amd as m
    m.lib()
    return m


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    atol, rtol = TOL[tol]
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    log(f"    {name}: max_abs={err.max():.3e} fails={int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance, max abs {err.max():.3e}"


def edge_rows(n, seed, extra=24):
    """First and last rows, both sides of every 32/64/256 edge in the first
    and last 1024 rows and in the middle, and seeded random rows."""
    rows = {0, 1, n - 2, n - 1}
    for base in (0, n // 2, n - 1024):
        for e in range(base, min(n, base + 1024), 32):
            rows.update((max(0, e - 1), e))
    rows.update(np.random.default_rng(seed).integers(0, n, extra).tolist())
    return np.array(sorted(rows))


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16).contiguous()


@pytest.mark.parametrize("causal", [True, False])
def test_forward_longest_head(fa, causal):
    n, d = 65536, 128
    log(f"case limits fwd N={n} d={d} causal={causal}")
    x = workloads.random_inputs(1, 1, n, d, "bf16", seed=6553)
    q, k, v = (to_dev(x[m]) for m in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    rows = edge_rows(n, 6554)
    o, lse = o[0, 0, rows].float().cpu().numpy(), lse[0, 0, rows].cpu().numpy()
    ro, rl = oracle.dense_fwd(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], causal=causal, rows=rows)
    compare(f"O ({len(rows)} rows)", o, ro, "bf16")
    compare(f"LSE ({len(rows)} rows)", lse, rl, "lse")
    assert np.isfinite(o).all()


def test_backward_long_head(fa):
    n, d = 32768, 128
    log(f"case limits bwd N={n} d={d} causal")
    x = workloads.random_inputs(1, 1, n, d, "bf16", seed=3276, with_do=True)
    q, k, v, do = (to_dev(x[m]) for m in ("q", "k", "v", "do"))
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = (t[0, 0].float().cpu().numpy() for t in (dq, dk, dv))
    rows = edge_rows(n, 3277, extra=8)[::4]
    cols = edge_rows(n, 3278, extra=8)[::4]
    rq, rk, rv = oracle.sampled_bwd(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["do"][0, 0], causal=True,
                                    rows=rows, cols=cols)
    compare(f"dQ ({len(rows)} rows)", dq[rows], rq, "bf16")
    compare(f"dK ({len(cols)} keys)", dk[cols], rk, "bf16")
    compare(f"dV ({len(cols)} keys)", dv[cols], rv, "bf16")
    # Identities over every key.  Each gradient carries its own rounding
    # (about 2.4e-3 of its RMS, from the bf16 operands and output), so a sum
    # over N keys may drift by about sqrt(N) times that; a key block that is
    # dropped or counted twice moves it by about sqrt(128) RMS.
    bound = lambda g: 0.01 * np.sqrt(n) * np.sqrt(np.mean(g.astype(np.float64) ** 2))
    sk = np.abs(dk.astype(np.float64).sum(axis=0))
    log(f"    sum_j dK_j: max {sk.max():.3e} (bound {bound(dk):.3e})")
    assert sk.max() <= bound(dk)
    sv = np.abs(dv.astype(np.float64).sum(axis=0) - x["do"][0, 0].astype(np.float64).sum(axis=0))
    log(f"    sum_j dV_j - sum_i dO_i: max {sv.max():.3e} (bound {bound(dv):.3e})")
    assert sv.max() <= bound(dv)


def test_widest_grid(fa):
    B, H, n, d = 64, 32, 256, 64
    log(f"case limits grid B={B} H={H} N={n} d={d} causal")
    x = workloads.random_inputs(B, H, n, d, "bf16", seed=2048, with_do=True)
    q, k, v, do = (to_dev(x[m]) for m in ("q", "k", "v", "do"))
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), x, True, d ** -0.5,
                                      TOL["bf16"], TOL["lse"], label="grid ")
    grads = tuple(t.float().cpu().numpy() for t in (dq, dk, dv))
    whole_output.compare_bwd_all_heads(grads, x, True, d ** -0.5, TOL["bf16"], 2e-2, label="grid ")
