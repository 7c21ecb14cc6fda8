"""GPU parity of the block-sparse forward (attn_fwd_block_sparse).

Key j is visible to query i iff the mask block (i // 64, j // 64) is nonzero
(and j <= i when causal); a row that sees no key has O = 0 and LSE = -inf.
The HIP result is compared element by element with the float64 oracle
(``oracle.dense_fwd(..., block_mask=...)``) on the same dtype-rounded inputs:
O within 2e-2 + 1e-2 |ref| (fp16/bf16) or 1e-5 (fp32), the fp32 LSE within
1e-4 + 1e-5 |ref|, and the empty rows exactly.
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


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    atol, rtol = TOL[tol]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{name}: infinite entries differ"
    err = np.abs(got[fin] - ref[fin])
    bad = ~(err <= atol + rtol * np.abs(ref[fin]))
    log(f"    {name}: max_abs={err.max() if err.size else 0:.3e} fails={int(bad.sum())}/{bad.size} "
        f"(+{int((~fin).sum())} -inf)")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance"


def run_case(fa, x, dtype, causal, mask, rows=None):
    q, k, v = (torch.from_numpy(x[n]).to("cuda").to(TORCH_DT[dtype]).contiguous() for n in "qkv")
    bm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    o, lse = fa.attn_fwd(q, k, v, causal=causal, block_mask=bm)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=causal, block_mask=mask, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    compare("O", o, ro, dtype)
    compare("LSE", lse, rl, "fp32" if dtype == "fp32" else "lse")


def random_mask(b, h, n, density, seed, empty_row=False):
    nb = -(-n // 64)
    m = (np.random.default_rng(seed).random((b, h, nb, nb)) < density).astype(np.uint8)
    if empty_row and nb > 1:
        m[..., nb // 2, :] = 0  # one query block sees nothing
    return m


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_sweep(fa, dtype, d, causal):
    cases = [(1, (1, 1), 0.5), (64, (1, 2), 0.5), (65, (2, 1), 0.6), (300, (1, 3), 0.4),
             (777, (2, 2), 0.3), (1000, (1, 2), 0.15)]
    for i, (n, (b, h), dens) in enumerate(cases):
        seed = 9600 + n + d + int(causal)
        mb, mh = (1 if i % 2 else b), (h if i % 3 else 1)
        log(f"case block-sparse dtype={dtype} d={d} causal={causal} B,H={b, h} N={n} "
            f"mask {mb}x{mh} density={dens} seed={seed}")
        x = workloads.random_inputs(b, h, n, d, dtype, seed)
        run_case(fa, x, dtype, causal, random_mask(mb, mh, n, dens, seed + 1, empty_row=(i == 3)))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_sweep_d256(fa, dtype, causal):
    """Head dim 256 (its own kernel, 32-key blocks, two 64-row query blocks per
    workgroup): random masks, broadcast or full mask axes, one query block
    that sees nothing (O = 0, LSE = -inf)."""
    cases = [(1, (1, 1), 0.5), (64, (1, 2), 0.5), (65, (2, 1), 0.6), (300, (1, 3), 0.4),
             (777, (2, 2), 0.3)]
    for i, (n, (b, h), dens) in enumerate(cases):
        seed = 9650 + n + int(causal)
        mb, mh = (1 if i % 2 else b), (h if i % 3 else 1)
        log(f"case block-sparse dtype={dtype} d=256 causal={causal} B,H={b, h} N={n} "
            f"mask {mb}x{mh} density={dens} seed={seed}")
        x = workloads.random_inputs(b, h, n, 256, dtype, seed)
        run_case(fa, x, dtype, causal, random_mask(mb, mh, n, dens, seed + 1, empty_row=(i == 3)))


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_alternating_runs_sharp_rows(fa, causal):
    """Each query block sees runs of two key tiles separated by two hidden ones,
    shifted from block to block, so the four query blocks of a workgroup walk
    different runs of one tile list and every run after the first restarts
    from a reference set earlier.  Sharp fp16 rows (scores of std 9, rising
    along the keys) move the reference at many of those restarts."""
    n, d = 1500, 128
    x = workloads.random_inputs(1, 2, n, d, "fp16", seed=9800 + int(causal), qk_std=3.0,
                                v_dist="uniform")
    ramp = np.linspace(0, 2, n, dtype=np.float32)[None, None, :, None]
    x["k"] = workloads.round_to_dtype(x["k"] + ramp, "fp16")
    nb = -(-n // 64)
    qb, kb = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask = (((kb // 2 + qb) % 2 == 0) | (kb == qb)).astype(np.uint8)[None, None]
    log(f"case block-sparse alternating runs fp16 sharp causal={causal} N={n} "
        f"density={float(mask.mean()):.2f}")
    run_case(fa, x, "fp16", causal, mask)


def test_block_sparse_all_ones_equals_plain_kernel(fa):
    """With every block visible the sparse path computes what attn_fwd does."""
    for causal in (False, True):
        x = workloads.random_inputs(1, 2, 513, 128, "bf16", 9700 + int(causal))
        q, k, v = (torch.from_numpy(x[n]).to("cuda").to(torch.bfloat16).contiguous() for n in "qkv")
        nb = -(-513 // 64)
        bm = torch.ones((1, 1, nb, nb), dtype=torch.uint8, device="cuda")
        o1, l1 = fa.attn_fwd(q, k, v, causal=causal)
        o2, l2 = fa.attn_fwd(q, k, v, causal=causal, block_mask=bm)
        torch.cuda.synchronize()
        d_o = (o1.float() - o2.float()).abs().max().item()
        d_l = (l1 - l2).abs().max().item()
        log(f"    causal={causal}: max |dO|={d_o:.3e} max |dLSE|={d_l:.3e}")
        assert d_o <= 1e-2 and d_l <= 1e-5


def test_block_sparse_all_hidden(fa):
    """A mask with no visible block: every row O = 0, LSE = -inf."""
    x = workloads.random_inputs(1, 2, 200, 64, "bf16", 9750)
    run_case(fa, x, "bf16", False, np.zeros((1, 1, 4, 4), np.uint8))


def test_block_sparse_bench_workload_all_rows(fa):
    """The measured block-sparse workload (B=1, H=16, N=8192, d=128, bf16; band,
    global and random blocks) at full size, every row of every head."""
    w = workloads.WORKLOADS["long_sparse_bf16"]
    x = workloads.make_inputs(w)
    mask = workloads.block_sparse_mask(w.N, w.H, *w.sparse)
    log(f"case block-sparse bench workload {w.name}")
    q, k, v = (torch.from_numpy(x[n]).to("cuda").to(torch.bfloat16).contiguous() for n in "qkv")
    o, lse = fa.attn_fwd(q, k, v, causal=w.causal, block_mask=torch.from_numpy(mask).to("cuda"))
    torch.cuda.synchronize()
    whole_output.compare_fwd_all_rows(o.float().cpu().numpy(), lse.cpu().numpy(), x, w.causal,
                                      w.scale, TOL["bf16"], TOL["lse"], block_mask=mask,
                                      label=f"{w.name} ")


def bwd_case(fa, x, dtype, causal, mask):
    q, k, v, do = (torch.from_numpy(x[n]).to("cuda").to(TORCH_DT[dtype]).contiguous()
                   for n in ("q", "k", "v", "do"))
    bm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    o, lse = fa.attn_fwd(q, k, v, causal=causal, block_mask=bm)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=causal, block_mask=bm)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], causal=causal, block_mask=mask)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, g.float().cpu().numpy(), r, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_sweep(fa, dtype, d, causal):
    cases = [(1, (1, 1), 0.5), (65, (2, 1), 0.6), (300, (1, 3), 0.4), (777, (1, 2), 0.3)]
    for i, (n, (b, h), dens) in enumerate(cases):
        seed = 9900 + n + d + int(causal)
        mb, mh = (1 if i % 2 else b), (h if i % 3 else 1)
        log(f"case block-sparse bwd dtype={dtype} d={d} causal={causal} B,H={b, h} N={n} "
            f"mask {mb}x{mh} density={dens} seed={seed}")
        x = workloads.random_inputs(b, h, n, d, dtype, seed, with_do=True)
        bwd_case(fa, x, dtype, causal, random_mask(mb, mh, n, dens, seed + 1, empty_row=(i == 2)))


def test_block_sparse_backward_split_key_blocks(fa):
    """Key blocks whose query-tile lists are long enough to be split over
    several dK/dV workgroups (global blocks of the mask recipe; an all-ones
    mask, where every key block splits), against the oracle, and the split
    result bitwise equal on a second call (the partials are added in chunk
    order)."""
    cases = [(4096, 2, False, workloads.block_sparse_mask(4096, 2, 1, 2, 3, seed=9950)),  # 2 chunks
             (6144, 1, True, workloads.block_sparse_mask(6144, 1, 1, 2, 3, seed=9951)),   # 3 chunks
             (4096, 1, False, np.ones((1, 1, 64, 64), np.uint8))]                       # all split
    for n, h, causal, mask in cases:
        log(f"case block-sparse bwd split N={n} H={h} causal={causal} density={mask.mean():.3f}")
        x = workloads.random_inputs(1, h, n, 128, "bf16", 9960 + n + h, with_do=True)
        bwd_case(fa, x, "bf16", causal, mask)
    n, h, causal, mask = cases[0]
    x = workloads.random_inputs(1, h, n, 128, "bf16", 9960 + n + h, with_do=True)
    q, k, v, do = (torch.from_numpy(x[m]).to("cuda").to(torch.bfloat16).contiguous() for m in ("q", "k", "v", "do"))
    bm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    o, lse = fa.attn_fwd(q, k, v, block_mask=bm)
    g1 = fa.attn_bwd(q, k, v, o, lse, do, block_mask=bm)
    g2 = fa.attn_bwd(q, k, v, o, lse, do, block_mask=bm)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
