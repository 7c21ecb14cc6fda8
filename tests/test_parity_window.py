"""GPU parity of the causal sliding window (attn_fwd_window, attn_bwd_window).

Key j is visible to query i iff i - W < j <= i.  The HIP path is compared
element by element with the float64 oracle (``oracle.dense_fwd`` /
``oracle.dense_bwd`` with ``window=W``) on the same dtype-rounded inputs.
Tolerances as for the plain calls: fp32 max |err| <= 1e-5 on O and LSE;
fp16/bf16 |err| <= 2e-2 + 1e-2 |ref| on O, dQ, dK, dV and 1e-4 + 1e-5 |ref| on
the fp32 LSE.  Window sizes cover 1 (each query sees only itself), values
below, at and across the 32-key block and 64-key tile edges, and W >= N.
"""
import sys

import numpy as np
import pytest

import oracle
import whole_output
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
TOL = {"fp32": (1e-5, 0.0), "fp16": (2e-2, 1e-2), "bf16": (2e-2, 1e-2), "lse": (1e-4, 1e-5)}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_12_amd as m
    m.lib()
    return m


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DT[dtype]).contiguous()


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


def fwd_case(fa, x, dtype, w, rows=None):
    q, k, v = (to_dev(x[n], dtype) for n in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=True, window=w)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=True, window=w, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    compare("O", o, ro, dtype)
    compare("LSE", lse, rl, "fp32" if dtype == "fp32" else "lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 96, 128])
def test_window_fwd_sweep(fa, dtype, d):
    for i, (n, w) in enumerate([(1, 1), (31, 1), (64, 17), (257, 32), (257, 33), (600, 64),
                                (600, 65), (1000, 100), (1000, 256), (777, 300), (300, 299), (300, 300),
                                (300, 5000)]):
        seed = 7000 + 13 * n + w + d
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case window fwd dtype={dtype} d={d} B,H={bh} N={n} W={w} seed={seed}")
        fwd_case(fa, workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed), dtype, w)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_window_fwd_sweep_d256(fa, dtype):
    """Head dim 256 (its own kernel: 32-key blocks, one wave per SIMD): waves
    whose window starts after the workgroup's first block form their first
    scores from the resident tile; one sharp fp16/bf16 case (scores of std 9)
    moves the lazy reference at those starts."""
    cases = [(1, 1), (31, 1), (64, 17), (257, 32), (257, 33), (600, 64), (600, 65), (1000, 100),
             (777, 300), (300, 5000)]
    for i, (n, w) in enumerate(cases):
        seed = 7050 + 13 * n + w
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case window fwd dtype={dtype} d=256 B,H={bh} N={n} W={w} seed={seed}")
        fwd_case(fa, workloads.random_inputs(bh[0], bh[1], n, 256, dtype, seed), dtype, w)
    log(f"case window fwd dtype={dtype} d=256 sharp N=700 W=150")
    fwd_case(fa, workloads.random_inputs(1, 2, 700, 256, dtype, 7099, qk_std=3.0, v_dist="uniform"),
             dtype, 150)


def fwd_all_rows(fa, x, w, label):
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=True, window=w)
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), x, True,
                                      1.0 / np.sqrt(x["q"].shape[-1]), TOL["bf16"], TOL["lse"],
                                      window=w, label=label)


def test_window_fwd_long_all_rows(fa):
    n, w = 4099, 1000
    log(f"case window fwd long N={n} W={w}")
    x = workloads.random_inputs(1, 4, n, 128, "bf16", seed=7100)
    fwd_all_rows(fa, x, w, f"N={n} W={w} ")


def test_window_bench_workload_all_rows(fa):
    """The benchmarked window workload at full size (B=1, H=16, N=8192, d=128,
    W=1024, bf16), in the launch the benchmark times, every row of every head."""
    w = workloads.WORKLOADS["long_window_bf16"]
    log(f"case window bench workload {w.name} N={w.N} W={w.window}")
    x = workloads.make_inputs(w)
    fwd_all_rows(fa, x, w.window, f"{w.name} ")


def test_window_at_least_n_equals_causal(fa):
    x = workloads.random_inputs(1, 3, 333, 128, "bf16", seed=7200)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    ref = fa.attn_fwd(q, k, v, causal=True)
    for w in (333, 334, 10**9):
        got = fa.attn_fwd(q, k, v, causal=True, window=w)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), w


def test_window_needle(fa):
    """A much higher score just outside a row's window must not leak in."""
    n, d, w = 256, 64, 48
    rng = np.random.default_rng(7300)
    q = rng.standard_normal((1, 1, n, d)) * 0.1
    k = rng.standard_normal((1, 1, n, d)) * 0.1
    v = rng.standard_normal((1, 1, n, d))
    for i in range(w, n):
        k[0, 0, i - w] = q[0, 0, i] * 40.0  # the key one step outside row i's window
    x = {"q": workloads.round_to_dtype(q, "bf16"), "k": workloads.round_to_dtype(k, "bf16"),
         "v": workloads.round_to_dtype(v, "bf16")}
    log(f"case window needle N={n} W={w}")
    fwd_case(fa, x, "bf16", w)


def bwd_case(fa, x, dtype, w):
    q, k, v, do = (to_dev(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.attn_fwd(q, k, v, causal=True, window=w)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True, window=w)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=True, window=w)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, g.float().cpu().numpy(), r, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_window_bwd_sweep(fa, dtype, d):
    for i, (n, w) in enumerate([(1, 1), (65, 1), (65, 33), (300, 64), (300, 100), (777, 129),
                                (777, 300), (500, 500)]):
        seed = 7400 + 11 * n + w + d
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case window bwd dtype={dtype} d={d} B,H={bh} N={n} W={w} seed={seed}")
        bwd_case(fa, workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed, with_do=True), dtype, w)
