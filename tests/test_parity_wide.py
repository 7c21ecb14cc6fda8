"""GPU parity at head dim 256 (attn_fwd, attn_bwd and their strided calls).

The HIP result is compared element by element with the float64 oracle
(``oracle.dense_fwd``, ``oracle.dense_bwd``) on the same dtype-rounded inputs: O, dQ, dK, dV within
2e-2 + 1e-2 |ref|, the fp32 LSE within 1e-4 + 1e-5 |ref|.  Lengths cover one
row, ragged tails of the 64-key tiles and the 128-query blocks, several
blocks, negative and zero scales, sharp rows whose maximum moves late, and a
[B, N, H, d] view.
"""
import sys

import numpy as np
import pytest

import oracle
import whole_output
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}
TOL = {"o": (2e-2, 1e-2), "lse": (1e-4, 1e-5)}
D = 256


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


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DT[dtype]).contiguous()


def run(fa, x, dtype, causal, scale=None, rows=None):
    q, k, v = (dev(x[n], dtype) for n in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    compare("O", o, ro, "o")
    compare("LSE", lse, rl, "lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_sweep(fa, dtype, causal):
    for i, n in enumerate([1, 31, 64, 65, 127, 128, 129, 257, 300, 777]):
        seed = 12000 + 7 * n + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case wide dtype={dtype} causal={causal} B,H={bh} N={n} seed={seed}")
        run(fa, workloads.random_inputs(bh[0], bh[1], n, D, dtype, seed), dtype, causal)


def test_wide_scales_and_sharp_rows(fa):
    """Negative and zero scale; sharp rows (q, k ~ N(0, 9)) whose maximum moves
    far past the first block's, which raises the lazy reference."""
    x = workloads.random_inputs(1, 2, 333, D, "bf16", 12100)
    for scale in (-0.2, 0.0, 0.5):
        log(f"case wide scale={scale}")
        run(fa, x, "bf16", True, scale=scale)
    for dtype in ("fp16", "bf16"):
        xs = workloads.random_inputs(1, 2, 600, D, dtype, 12101, qk_std=3.0)
        log(f"case wide sharp {dtype} N=600")
        run(fa, xs, dtype, False)
        run(fa, xs, dtype, True)


def test_wide_bshd_view(fa):
    """q, k, v as [B, H, N, d] views of [B, N, H, d] memory (the strided call)."""
    b, h, n = 2, 3, 300
    x = workloads.random_inputs(b, h, n, D, "bf16", 12200)
    q, k, v = (dev(x[m].transpose(0, 2, 1, 3), "bf16").transpose(1, 2) for m in "qkv")
    assert not q.is_contiguous()
    log("case wide bshd")
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=True)
    compare("O", o.float().cpu().numpy(), ro, "o")
    compare("LSE", lse.cpu().numpy(), rl, "lse")


def test_wide_long_head_all_rows(fa):
    """A long head (B=1, H=16, N=8192, d=256, causal, bf16), every row of every
    head."""
    n = 8192
    x = workloads.random_inputs(1, 16, n, D, "bf16", 12300)
    log("case wide long head")
    q, k, v = (dev(x[m], "bf16") for m in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), x, True,
                                      1.0 / np.sqrt(D), TOL["o"], TOL["lse"], label="d=256 ")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_backward_sweep(fa, dtype, causal):
    """dQ, dK, dV at d = 256 against ``oracle.dense_bwd`` (same tolerance)."""
    for i, n in enumerate([1, 31, 65, 129, 300, 777]):
        seed = 12400 + 7 * n + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case wide bwd dtype={dtype} causal={causal} B,H={bh} N={n} seed={seed}")
        x = workloads.random_inputs(bh[0], bh[1], n, D, dtype, seed, with_do=True)
        q, k, v, do = (dev(x[m], dtype) for m in ("q", "k", "v", "do"))
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            compare(name, g.float().cpu().numpy(), r, "o")


def test_wide_backward_scales_and_bshd(fa):
    """Negative and zero scale, and [B, N, H, d] views (the strided call)."""
    x = workloads.random_inputs(1, 2, 333, D, "bf16", 12500, with_do=True)
    q, k, v, do = (dev(x[m], "bf16") for m in ("q", "k", "v", "do"))
    for scale in (-0.2, 0.0):
        log(f"case wide bwd scale={scale}")
        o, lse = fa.attn_fwd(q, k, v, causal=True, scale=scale)
        dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=True, scale=scale)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            compare(name, g.float().cpu().numpy(), r, "o")
    b, h, n = 2, 2, 300
    x = workloads.random_inputs(b, h, n, D, "bf16", 12501, with_do=True)
    q, k, v, do = (dev(x[m].transpose(0, 2, 1, 3), "bf16").transpose(1, 2) for m in ("q", "k", "v", "do"))
    log("case wide bwd bshd")
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=True)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, g.float().cpu().numpy(), r, "o")
