"""GPU parity of strided views (attn_fwd_strided, attn_bwd_strided).

The binding passes torch's strides to the *_strided calls whenever a tensor is
not contiguous, so these tests hand it transposed ([B, N, H, d] memory),
packed ([B, N, 3, H, d] memory) and broadcast (one k/v head for all query
heads) views and compare element by element with the float64 oracle on the
same numbers (O, dQ, dK, dV within 2e-2 + 1e-2 |ref| for fp16/bf16, 1e-5 for
fp32; the fp32 LSE within 1e-4 + 1e-5 |ref|).
"""
import sys

import numpy as np
import pytest

import oracle
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


def bshd(x, dtype):
    """A [B, H, N, d] view of a contiguous [B, N, H, d] device tensor holding x."""
    t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to("cuda").to(TORCH_DT[dtype])
    v = t.transpose(1, 2)
    assert not v.is_contiguous() or x.shape[1] == 1 or x.shape[2] == 1
    return v


def host(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bshd_forward(fa, dtype, d, causal):
    for n, (b, h) in [(1, (1, 3)), (65, (2, 3)), (300, (1, 4)), (777, (2, 2))]:
        seed = 9000 + n + d + 3 * int(causal)
        log(f"case bshd fwd dtype={dtype} d={d} causal={causal} B,H={b, h} N={n} seed={seed}")
        x = workloads.random_inputs(b, h, n, d, dtype, seed)
        q, k, v = (bshd(x[m], dtype) for m in "qkv")
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        assert o.stride() == q.stride()  # the output keeps the [B, N, H, d] layout
        torch.cuda.synchronize()
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
        compare("O", host(o), ro, dtype)
        compare("LSE", lse.cpu().numpy(), rl, "fp32" if dtype == "fp32" else "lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_packed_qkv_forward(fa, dtype):
    """q, k, v sliced from one [B, N, 3, H, d] tensor; o dense."""
    b, h, n, d = 2, 3, 333, 128
    x = workloads.random_inputs(b, h, n, d, dtype, 9100)
    packed = np.stack([x[m].transpose(0, 2, 1, 3) for m in "qkv"], axis=2)  # [B, N, 3, H, d]
    t = torch.from_numpy(np.ascontiguousarray(packed)).to("cuda").to(TORCH_DT[dtype])
    q, k, v = (t[:, :, i].transpose(1, 2) for i in range(3))
    out = torch.empty((b, h, n, d), dtype=TORCH_DT[dtype], device="cuda")
    log(f"case packed qkv dtype={dtype}")
    o, lse = fa.attn_fwd(q, k, v, causal=True, out=out)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=True)
    compare("O", host(o), ro, dtype)
    compare("LSE", lse.cpu().numpy(), rl, "lse")


@pytest.mark.parametrize("d", [64, 96, 128])
def test_multi_query_forward(fa, d):
    """One k and one v head shared by all query heads (head stride 0)."""
    b, h, n = 2, 4, 300
    xq = workloads.random_inputs(b, h, n, d, "bf16", 9200 + d)
    xkv = workloads.random_inputs(b, 1, n, d, "bf16", 9300 + d)
    q = torch.from_numpy(xq["q"]).to("cuda").to(torch.bfloat16)
    k1, v1 = (torch.from_numpy(xkv[m]).to("cuda").to(torch.bfloat16) for m in "kv")
    k, v = k1.expand(b, h, n, d), v1.expand(b, h, n, d)
    assert k.stride(1) == 0
    log(f"case multi-query d={d}")
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    kb = np.broadcast_to(xkv["k"], (b, h, n, d))
    vb = np.broadcast_to(xkv["v"], (b, h, n, d))
    ro, rl = oracle.dense_fwd(xq["q"], kb, vb, causal=True)
    compare("O", host(o), ro, "bf16")
    compare("LSE", lse.cpu().numpy(), rl, "lse")


def test_dense_strides_match_the_plain_call_bitwise(fa):
    """The strided call with the dense strides runs the same kernels."""
    b, h, n, d = 1, 2, 257, 128
    x = workloads.random_inputs(b, h, n, d, "bf16", 9400)
    q, k, v = (torch.from_numpy(x[m]).to("cuda").to(torch.bfloat16).contiguous() for m in "qkv")
    o1, l1 = fa.attn_fwd(q, k, v, causal=True)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    dense = (h * n * d, n * d, d)
    st = fa.attn_fwd_strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                 b, h, n, d, dense, dense, dense, fa.MASK_CAUSAL, 1 / np.sqrt(d),
                                 fa.BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bshd_backward(fa, dtype, d, causal):
    for n, (b, h) in [(1, (1, 2)), (65, (2, 2)), (300, (1, 3)), (777, (1, 2))]:
        seed = 9500 + n + d + 5 * int(causal)
        log(f"case bshd bwd dtype={dtype} d={d} causal={causal} B,H={b, h} N={n} seed={seed}")
        x = workloads.random_inputs(b, h, n, d, dtype, seed, with_do=True)
        q, k, v, do = (bshd(x[m], dtype) for m in ("q", "k", "v", "do"))
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=causal)
        assert dq.stride() == q.stride()
        torch.cuda.synchronize()
        rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal)
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            compare(name, host(g), r, dtype)
