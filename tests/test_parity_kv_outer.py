"""GPU parity of the key/value-outer forward (attn_fwd_kv_outer).

The original loop order ("Flash Attention: IO-Aware Exact Attention", section
"Loop order changes which data is reloaded"; the normalised per-tile update of
"FlashAttention -- the same attention, made memory-aware", section 03) reaches
the same exact attention, so the HIP result is compared element by element with
the float64 dense oracle on the same dtype-rounded inputs: O within
2e-2 + 1e-2 |ref|, the fp32 LSE within 1e-4 + 1e-5 |ref|.
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


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DT[dtype]).contiguous()


def compare(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    atol, rtol = TOL[tol]
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    log(f"    {name}: max_abs={err.max():.3e} fails={int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance, max abs {err.max():.3e}"


def run_case(fa, x, dtype, causal, scale=None, rows=None):
    q, k, v = (to_dev(x[n], dtype) for n in "qkv")
    o, lse = fa.attn_fwd_kv_outer(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    compare("O", o, ro, "o")
    compare("LSE", lse, rl, "lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_kv_outer_sweep(fa, dtype, d, causal):
    for i, n in enumerate([1, 31, 64, 65, 257, 300, 777]):
        seed = 8000 + 7 * n + d + int(causal)
        bh = (1, 2) if i % 2 else (2, 1)
        log(f"case kv_outer dtype={dtype} d={d} causal={causal} B,H={bh} N={n} seed={seed}")
        run_case(fa, workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed), dtype, causal)


def test_kv_outer_scales_and_sharp_rows(fa):
    """Negative and zero scale; sharp fp16 rows (q, k ~ N(0, 9)) that move the
    running maximum in many tiles."""
    x = workloads.random_inputs(1, 2, 333, 128, "bf16", seed=8100)
    for scale in (-0.2, 0.0, 0.5):
        log(f"case kv_outer scale={scale}")
        run_case(fa, x, "bf16", True, scale=scale)
    w = workloads.WORKLOADS["ragged_sharp_fp16"]
    xs = workloads.make_inputs(w, B=1, H=2, N=600, seed=8101)
    log("case kv_outer sharp fp16 N=600")
    run_case(fa, xs, "fp16", False)


def test_kv_outer_bench_workload_all_rows(fa):
    """The long causal head (B=1, H=16, N=8192, d=128, bf16), every row of every
    head against the oracle, and the whole output against the query-outer
    kernel."""
    w = workloads.WORKLOADS["long_causal_bf16"]
    x = workloads.make_inputs(w)
    log(f"case kv_outer bench workload {w.name}")
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    o, lse = fa.attn_fwd_kv_outer(q, k, v, causal=True)
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), x, True, w.scale,
                                      TOL["o"], TOL["lse"], label=f"{w.name} kv_outer ")
    o1, l1 = fa.attn_fwd_kv_outer(q, k, v, causal=True)
    o2, l2 = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    # two roundings of the same exact result: bf16 output half-ulps apart at most a few
    d_o = (o1.float() - o2.float()).abs().max().item()
    d_l = (l1 - l2).abs().max().item()
    log(f"    kv_outer vs attn_fwd: max |dO|={d_o:.3e} max |dLSE|={d_l:.3e}")
    assert d_o <= 2e-2 and d_l <= 1e-3
