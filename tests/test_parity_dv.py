"""GPU parity with values of another width (attn_fwd_dv, attn_bwd_dv).

q and k are [B, H, N, d], v, o and dout [B, H, N, dv] with d and dv in
{64, 96, 128, 256}, d != dv: the six pairs below 256 (MFMA kernels and the
fp32 path) and the six with a 256-wide side (the d = 256 kernels, bf16 and
fp16).  The HIP results are compared element by element with
the float64 oracle (``oracle.dense_fwd`` and ``oracle.dense_bwd``, which take v
of any width) on the same dtype-rounded inputs: O, dQ, dK, dV within
2e-2 + 1e-2 |ref| (fp16/bf16) or 1e-5 (fp32), the fp32 LSE within
1e-4 + 1e-5 |ref|.
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
PAIRS = [(128, 64), (64, 128), (128, 96), (96, 128), (96, 64), (64, 96)]
PAIRS_256 = [(256, 64), (256, 96), (256, 128), (64, 256), (96, 256), (128, 256)]


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


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d,dv", PAIRS)
@pytest.mark.parametrize("causal", [False, True])
def test_dv_forward_sweep(fa, dtype, d, dv, causal):
    for i, n in enumerate([1, 31, 65, 257, 300, 777]):
        seed = 9950 + n + d + dv + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case dv fwd dtype={dtype} d={d} dv={dv} causal={causal} B,H={bh} N={n} seed={seed}")
        xq = workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed)
        xv = workloads.random_inputs(bh[0], bh[1], n, dv, dtype, seed + 1)
        q, k = (torch.from_numpy(xq[m]).to("cuda").to(TORCH_DT[dtype]).contiguous() for m in "qk")
        v = torch.from_numpy(xv["v"]).to("cuda").to(TORCH_DT[dtype]).contiguous()
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        assert tuple(o.shape) == (bh[0], bh[1], n, dv)
        torch.cuda.synchronize()
        ro, rl = oracle.dense_fwd(xq["q"], xq["k"], xv["v"], causal=causal)
        compare("O", o.float().cpu().numpy(), ro, dtype)
        compare("LSE", lse.cpu().numpy(), rl, "fp32" if dtype == "fp32" else "lse")


def test_dv_long_head_all_rows(fa):
    """A long head (B=1, H=4, N=4099, d=128, dv=64, causal), every row."""
    n = 4099
    xq = workloads.random_inputs(1, 4, n, 128, "bf16", 9990)
    xv = workloads.random_inputs(1, 4, n, 64, "bf16", 9991)
    q, k = (torch.from_numpy(xq[m]).to("cuda").to(torch.bfloat16).contiguous() for m in "qk")
    v = torch.from_numpy(xv["v"]).to("cuda").to(torch.bfloat16).contiguous()
    log("case dv long head")
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), xq, True,
                                      1.0 / np.sqrt(128), TOL["bf16"], TOL["lse"], v=xv["v"],
                                      label="d=128 dv=64 ")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d,dv", PAIRS)
@pytest.mark.parametrize("causal", [False, True])
def test_dv_backward_sweep(fa, dtype, d, dv, causal):
    for i, n in enumerate([1, 31, 65, 257, 300, 777]):
        seed = 9850 + n + d + dv + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case dv bwd dtype={dtype} d={d} dv={dv} causal={causal} B,H={bh} N={n} seed={seed}")
        xq = workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed)
        xv = workloads.random_inputs(bh[0], bh[1], n, dv, dtype, seed + 1, with_do=True)
        dev = lambda x: torch.from_numpy(x).to("cuda").to(TORCH_DT[dtype]).contiguous()
        q, k, v, do = dev(xq["q"]), dev(xq["k"]), dev(xv["v"]), dev(xv["do"])
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        dq, dk, dvg = fa.attn_bwd(q, k, v, o, lse, do, causal=causal)
        assert dq.shape == q.shape and dk.shape == k.shape and dvg.shape == v.shape
        torch.cuda.synchronize()
        rq, rk, rv, _, _ = oracle.dense_bwd(xq["q"], xq["k"], xv["v"], xv["do"], causal=causal)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dvg, rv)):
            compare(name, g.float().cpu().numpy(), r, dtype)


def test_dv_backward_long_head(fa):
    """A longer head (B=1, H=2, N=2113, causal, bf16) for every pair."""
    n = 2113
    for d, dv in PAIRS:
        xq = workloads.random_inputs(1, 2, n, d, "bf16", 9993 + d)
        xv = workloads.random_inputs(1, 2, n, dv, "bf16", 9994 + dv, with_do=True)
        dev = lambda x: torch.from_numpy(x).to("cuda").to(torch.bfloat16).contiguous()
        q, k, v, do = dev(xq["q"]), dev(xq["k"]), dev(xv["v"]), dev(xv["do"])
        log(f"case dv bwd long head d={d} dv={dv}")
        o, lse = fa.attn_fwd(q, k, v, causal=True)
        dq, dk, dvg = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        rq, rk, rv, _, _ = oracle.dense_bwd(xq["q"], xq["k"], xv["v"], xv["do"], causal=True)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dvg, rv)):
            compare(name, g.float().cpu().numpy(), r, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d,dv", PAIRS_256)
@pytest.mark.parametrize("causal", [False, True])
def test_dv_256_forward_backward_sweep(fa, dtype, d, dv, causal):
    """Pairs with a 256-wide side: forward (O, LSE) and backward (dQ, dK, dV)."""
    for i, n in enumerate([1, 31, 65, 300, 777]):
        seed = 9750 + n + d + 3 * dv + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case dv256 dtype={dtype} d={d} dv={dv} causal={causal} B,H={bh} N={n} seed={seed}")
        xq = workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed)
        xv = workloads.random_inputs(bh[0], bh[1], n, dv, dtype, seed + 1, with_do=True)
        dev = lambda x: torch.from_numpy(x).to("cuda").to(TORCH_DT[dtype]).contiguous()
        q, k, v, do = dev(xq["q"]), dev(xq["k"]), dev(xv["v"]), dev(xv["do"])
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        assert tuple(o.shape) == (bh[0], bh[1], n, dv)
        dq, dk, dvg = fa.attn_bwd(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle.dense_fwd(xq["q"], xq["k"], xv["v"], causal=causal)
        compare("O", o.float().cpu().numpy(), ro, dtype)
        compare("LSE", lse.cpu().numpy(), rl, "lse")
        rq, rk, rv, _, _ = oracle.dense_bwd(xq["q"], xq["k"], xv["v"], xv["do"], causal=causal)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dvg, rv)):
            compare(name, g.float().cpu().numpy(), r, dtype)


def test_dv_256_long_head(fa):
    """B=1, H=2, N=2113, causal, bf16: (256, 128) and (128, 256), forward on
    every row and backward."""
    n = 2113
    for d, dv in ((256, 128), (128, 256)):
        xq = workloads.random_inputs(1, 2, n, d, "bf16", 9700 + d)
        xv = workloads.random_inputs(1, 2, n, dv, "bf16", 9701 + dv, with_do=True)
        dev = lambda x: torch.from_numpy(x).to("cuda").to(torch.bfloat16).contiguous()
        q, k, v, do = dev(xq["q"]), dev(xq["k"]), dev(xv["v"]), dev(xv["do"])
        log(f"case dv256 long head d={d} dv={dv}")
        o, lse = fa.attn_fwd(q, k, v, causal=True)
        dq, dk, dvg = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), xq, True,
                                          1.0 / np.sqrt(d), TOL["bf16"], TOL["lse"], v=xv["v"],
                                          label=f"d={d} dv={dv} ")
        rq, rk, rv, _, _ = oracle.dense_bwd(xq["q"], xq["k"], xv["v"], xv["do"], causal=True)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dvg, rv)):
            compare(name, g.float().cpu().numpy(), r, "bf16")
