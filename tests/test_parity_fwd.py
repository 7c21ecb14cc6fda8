"""GPU parity of the forward pass against the float64 CPU oracle.

Every case draws seeded inputs (``workloads``), runs the HIP path through the C
ABI, runs the oracle on the same dtype-rounded values and compares element by
element.  Tolerances: fp32 max |err| <= 1e-5 on O and LSE; fp16/bf16
|err| <= 2e-2 + 1e-2 |ref| on O.  The LSE is an fp32 output computed from the
rounded inputs in fp32 whatever the input type, so for fp16/bf16 inputs it is
held to |err| <= 1e-4 + 1e-5 |ref| (fp32 score sums, exp2 and a row sum of up
to 8192 fp32 probabilities).  Full-size workloads compare every row of every
head, the dense oracle running head by head on blocks of rows.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import whole_output
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
TOL = {"fp32": (1e-5, 0.0), "fp16": (2e-2, 1e-2), "bf16": (2e-2, 1e-2)}
# LSE of fp16/bf16 inputs: computed in fp32 from the rounded inputs
LSE_TOL = {"fp32": "fp32", "fp16": "lse", "bf16": "lse"}
TOL["lse"] = (1e-4, 1e-5)


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


def compare(name, got, ref, dtype):
    """Assert |got - ref| <= atol + rtol |ref| everywhere; print error statistics."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    rel_rms = float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300))
    log(f"    {name}: max_abs={err.max():.3e} rel_rms={rel_rms:.3e} fails={int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance, max abs {err.max():.3e}"
    return err.max(), rel_rms


def run_fwd(fa, x, dtype, causal, scale=None, return_lse=True):
    q, k, v = (to_dev(x[n], dtype) for n in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=causal, scale=scale, return_lse=return_lse)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), None if lse is None else lse.cpu().numpy())


def sample_rows(N, n_random=24, seed=0):
    rows = {0, 1, 31, 32, 63, 64, 65, 127, 128, 129, N // 2, N - 65, N - 64, N - 2, N - 1}
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, N, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


# ------------------------------------------------------------------ the five workloads

def test_tiny_fp32_full(fa):
    w = workloads.WORKLOADS["tiny_fp32_full"]
    log(f"case {w}")
    x = workloads.make_inputs(w)
    o, lse = run_fwd(fa, x, w.dtype, w.causal)
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale)
    compare("O", o, ro, "fp32")
    compare("LSE", lse, rl, LSE_TOL["fp32"])


def test_gpt2s_causal_bf16_full(fa):
    w = workloads.WORKLOADS["gpt2s_causal_bf16"]
    log(f"case {w}")
    x = workloads.make_inputs(w)
    o, lse = run_fwd(fa, x, w.dtype, w.causal)
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=True, scale=w.scale)
    compare("O", o, ro, w.dtype)
    compare("LSE", lse, rl, LSE_TOL[w.dtype])


@pytest.mark.parametrize("name", ["long_causal_bf16", "ragged_sharp_fp16", "fwd_bwd_causal_bf16"])
def test_large_workload_all_rows(fa, name):
    """The three full-size forward workloads, every row of every head."""
    w = workloads.WORKLOADS[name]
    log(f"case {w}")
    x = workloads.make_inputs(w)
    o, lse = run_fwd(fa, x, w.dtype, w.causal)
    whole_output.compare_fwd_all_rows(o, lse, x, w.causal, w.scale, TOL[w.dtype],
                                      TOL[LSE_TOL[w.dtype]], label=f"{name} ")
    assert np.isfinite(lse).all()


# ------------------------------------------------------------------ sweep

SWEEP_N = [1, 2, 15, 63, 64, 65, 127, 128, 129, 200, 257, 288, 289, 543, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep(fa, dtype, d, causal):
    for i, n in enumerate(SWEEP_N):
        bh = (1, 3) if i % 2 else (1, 1)
        seed = 1000 + 17 * n + d + (7 if causal else 0)
        log(f"case sweep dtype={dtype} d={d} causal={causal} B,H={bh} N={n} seed={seed}")
        x = workloads.random_inputs(bh[0], bh[1], n, d, dtype, seed)
        o, lse = run_fwd(fa, x, dtype, causal)
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
        compare("O", o, ro, dtype)
        compare("LSE", lse, rl, LSE_TOL[dtype])


# ------------------------------------------------------------------ structured inputs

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1000, 64), (4097, 128)])
def test_needles(fa, dtype, causal, n, d):
    """Near one-hot rows: a dropped tile or a leaky mask moves O by about |V|."""
    log(f"case needles dtype={dtype} causal={causal} N={n} d={d}")
    x = workloads.needle_inputs(1, 2, n, d, dtype, seed=n + d, causal=causal)
    o, lse = run_fwd(fa, x, dtype, causal)
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
    compare("O", o, ro, dtype)
    compare("LSE", lse, rl, LSE_TOL[dtype])
    # these rows are nearly one-hot, so the output is held much tighter than the tolerance
    assert np.abs(o - ro).max() < 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.9])
def test_scale_sign_and_zero(fa, dtype, scale):
    log(f"case scale={scale} dtype={dtype}")
    x = workloads.random_inputs(1, 2, 300, 64, dtype, seed=77)
    for causal in (False, True):
        o, lse = run_fwd(fa, x, dtype, causal, scale=scale)
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal, scale=scale)
        compare("O", o, ro, dtype)
        compare("LSE", lse, rl, LSE_TOL[dtype])


def test_sharp_rows_rescaling(fa):
    """Scores with std 9 and an increasing trend: the row max jumps in most tiles."""
    log("case sharp rows")
    n, d = 777, 128
    x = workloads.random_inputs(1, 2, n, d, "fp16", seed=5, qk_std=3.0, v_dist="uniform")
    ramp = np.linspace(0, 2, n, dtype=np.float32)[None, None, :, None]
    x["k"] = workloads.round_to_dtype(x["k"] + ramp, "fp16")
    for causal in (False, True):
        o, lse = run_fwd(fa, x, "fp16", causal)
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
        compare("O", o, ro, "fp16")
        compare("LSE", lse, rl, LSE_TOL["fp16"])


@pytest.mark.parametrize("d", [64, 128])
def test_sharp_rows_fp32(fa, d):
    """fp32 inputs with scores of std 9 and an increasing trend, held to 1e-5
    (two heads: the row-per-wave kernel, whose running maximum moves block by
    block)."""
    n = 777
    log(f"case sharp rows fp32 d={d} N={n}")
    x = workloads.random_inputs(1, 2, n, d, "fp32", seed=70 + d, qk_std=3.0, v_dist="uniform")
    ramp = np.linspace(0, 2, n, dtype=np.float32)[None, None, :, None]
    x["k"] = (x["k"] + ramp).astype(np.float32)
    for causal in (False, True):
        o, lse = run_fwd(fa, x, "fp32", causal)
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
        compare("O", o, ro, "fp32")
        compare("LSE", lse, rl, LSE_TOL["fp32"])


@pytest.mark.parametrize("kind", ["plain", "causal", "window", "sparse", "dv", "strided"])
def test_fp32_tiled_kernel(fa, kind):
    """fp32 launches that fill the GPU with 64-row workgroups (B*H*ceil(N/64) >= 256:
    here 20 heads of N = 777) run the tiled fp32 kernel, whose rows' keys are split
    over four waves and merged; smaller launches run the row-per-wave kernel, which
    the sweeps cover.  Sharp rows (q, k ~ N(0, 9)) with a ramp on the keys, so the
    waves' running maxima differ widely before the merge; every head is compared."""
    n, h = 777, 20
    d, dv = (128, 64) if kind == "dv" else (64, 64)
    log(f"case fp32 tiled kernel kind={kind} H={h} N={n} d={d} dv={dv}")
    x = workloads.random_inputs(1, h, n, d, "fp32", seed=4321, qk_std=3.0, v_dist="uniform")
    ramp = np.linspace(0, 2, n, dtype=np.float32)[None, None, :, None]
    x["k"] = (x["k"] + ramp).astype(np.float32)
    v = workloads.random_inputs(1, h, n, dv, "fp32", seed=4322)["v"] if kind == "dv" else x["v"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").contiguous()
    if kind == "strided":  # [B][N][H][d] storage seen as [B][H][N][d] views
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).to("cuda").transpose(1, 2)
    q, k, vt = dev(x["q"]), dev(x["k"]), dev(v)
    causal = kind in ("causal", "window", "dv", "strided")
    kw, okw = {}, {}
    if kind == "window":
        kw["window"] = okw["window"] = 100
    if kind == "sparse":
        rng = np.random.default_rng(77)
        nb = -(-n // 64)
        bm = (rng.random((1, h, nb, nb)) < 0.5).astype(np.uint8)
        kw["block_mask"] = torch.from_numpy(bm).to("cuda")
        okw["block_mask"] = bm
    o, lse = fa.attn_fwd(q, k, vt, causal=causal, **kw)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for hh in range(h):
        sl = (slice(0, 1), slice(hh, hh + 1))
        hk = {} if "block_mask" not in okw else {"block_mask": okw["block_mask"][:, hh:hh + 1]}
        if "window" in okw:
            hk["window"] = okw["window"]
        ro, rl = oracle.dense_fwd(x["q"][sl], x["k"][sl], v[sl], causal=causal, **hk)
        compare(f"O[h={hh}]", o[sl], ro, "fp32")
        compare(f"LSE[h={hh}]", lse[sl], rl, LSE_TOL["fp32"])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [128, 256])
def test_rising_row_maxima(dtype, d, fa):
    """Sharp rows (q, k ~ N(0, 9)) plus a ramp added to every key, so that a
    row's maximum keeps rising (or falling) along the keys by up to about 40 in
    log2 units.  The kernels move a row's reference maximum only when a
    probability would pass 2^15 (fp16) or 2^24 (bf16); these rows pass it at
    many different blocks, and also stay below it for long runs."""
    n = 1500
    log(f"case rising row maxima dtype={dtype} d={d} N={n}")
    x = workloads.random_inputs(1, 2, n, d, dtype, seed=80 + d, qk_std=3.0, v_dist="uniform")
    ramp = np.linspace(0, 0.6, n, dtype=np.float32)[None, None, :, None]
    x["k"] = workloads.round_to_dtype(x["k"] + ramp, dtype)
    for causal in (False, True):
        o, lse = run_fwd(fa, x, dtype, causal)
        ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal)
        compare("O", o, ro, dtype)
        compare("LSE", lse, rl, LSE_TOL[dtype])


# ------------------------------------------------------------------ properties

def test_deterministic(fa):
    w = workloads.WORKLOADS["gpt2s_causal_bf16"]
    log("case determinism")
    x = workloads.make_inputs(w, B=2)
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    o0, l0 = fa.attn_fwd(q, k, v, causal=True)
    for _ in range(9):
        o1, l1 = fa.attn_fwd(q, k, v, causal=True)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_lse_optional_and_side_stream(fa):
    log("case lse=None on a side stream")
    x = workloads.random_inputs(2, 2, 333, 128, "bf16", seed=9)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    ref, _ = fa.attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa.attn_fwd(q, k, v, causal=True, return_lse=False)
    s.synchronize()
    assert lse is None
    assert torch.equal(o, ref)


def test_nonfinite_inputs_propagate(fa):
    """A NaN in V reaches every output that weighs it; scores and LSE stay finite."""
    log("case NaN input")
    x = workloads.random_inputs(1, 1, 130, 64, "bf16", seed=10)
    x["v"][0, 0, 5, 3] = np.nan
    o, lse = run_fwd(fa, x, "bf16", causal=True)
    assert np.isnan(o[0, 0, 5:, 3]).all()          # rows that attend to key 5
    keep = np.ones(64, bool)
    keep[3] = False
    assert np.isfinite(o[0, 0][:, keep]).all()     # other value columns are untouched
    assert np.isfinite(lse).all()
