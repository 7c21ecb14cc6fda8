"""GPU parity on seeded random combinations of the call's options.

The other parity files sweep one option at a time.  Here each case draws its
own entry point (plain, sliding window, block-sparse mask, strided views,
values of another width), dtype, head dim, batch and head counts, ragged N,
mask, scale (default, negated, zero, larger, smaller) and score spread from a
fixed seed, so that pairs of options meet that no single sweep puts together
(a negative scale under a block mask at d = 256, a packed fp32 layout with a
ragged tail, a window over batched heads, ...).  Every case is compared with
the float64 oracle on the same dtype-rounded inputs, at the bars the other
files use: O within 1e-5 (fp32) or 2e-2 + 1e-2 |ref| (fp16/bf16), the fp32
LSE within 1e-4 + 1e-5 |ref| (1e-5 for fp32), dQ, dK, dV within
2e-2 + 1e-2 |ref|, and rows that see no key (O = 0, LSE = -inf) exactly.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
TOL = {"fp32": (1e-5, 0.0), "fp16": (2e-2, 1e-2), "bf16": (2e-2, 1e-2), "lse": (1e-4, 1e-5)}
KINDS = ("plain", "window", "sparse", "strided", "dv")
N_FWD, N_BWD = 64, 28


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
    log(f"    {name}: max_abs={err.max() if err.size else 0:.3e} fails={int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance"


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DT[dtype])


def bshd(x, dtype):
    """A [B, H, N, d] view of a contiguous [B, N, H, d] device tensor holding x."""
    return dev(x.transpose(0, 2, 1, 3), dtype).transpose(1, 2)


def draw_case(rng, backward):
    """One combination: every choice comes from ``rng``."""
    dtypes = ("bf16", "fp16") if backward else ("bf16", "fp16", "fp32")
    c = {"kind": KINDS[rng.integers(len(KINDS))], "dtype": dtypes[rng.integers(len(dtypes))]}
    if c["kind"] == "dv":
        c["d"], c["dv"] = ((128, 64), (64, 128), (128, 96), (96, 128), (96, 64), (64, 96))[rng.integers(6)]
    else:
        ds = (64, 96, 128) if c["dtype"] == "fp32" else (64, 96, 128, 256)
        c["d"] = c["dv"] = int(ds[rng.integers(len(ds))])
    c["B"], c["H"] = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    # ragged lengths around the 32-key block, the 64-key tile and the 256-row query block
    c["N"] = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 900)),
                             64 * int(rng.integers(1, 14)) + int(rng.integers(-1, 2))]))
    c["N"] = max(c["N"], 1)
    c["causal"] = c["kind"] == "window" or bool(rng.integers(2))
    mult = (1.0, -1.0, 0.0, 2.0, 0.3)[rng.integers(5)]
    c["scale"] = mult / math.sqrt(c["d"])
    c["qk_std"] = 3.0 if (not backward and abs(mult) <= 1.0 and rng.integers(3) == 0) else 1.0
    if c["kind"] == "window":
        c["window"] = int(rng.integers(1, c["N"] + 40))
    if c["kind"] == "sparse":
        nb = -(-c["N"] // 64)
        mb, mh = (1 if rng.integers(2) else c["B"]), (1 if rng.integers(2) else c["H"])
        c["mask"] = (rng.random((mb, mh, nb, nb)) < rng.uniform(0.15, 0.8)).astype(np.uint8)
    if c["kind"] == "strided":
        c["layout"] = ("bshd", "packed", "mqa")[rng.integers(1 if backward else 3)]
    c["seed"] = int(rng.integers(1 << 30))
    return c


def describe(c):
    extra = {k: c[k] for k in ("window", "layout") if k in c}
    if "mask" in c:
        extra["mask"] = f"{c['mask'].shape} density {c['mask'].mean():.2f}"
    return (f"{c['kind']} {c['dtype']} B={c['B']} H={c['H']} N={c['N']} d={c['d']} dv={c['dv']} "
            f"causal={c['causal']} scale={c['scale']:.4f} qk_std={c['qk_std']} seed={c['seed']} {extra}")


def inputs(c, with_do):
    x = workloads.random_inputs(c["B"], c["H"], c["N"], c["d"], c["dtype"], c["seed"], c["qk_std"],
                                with_do=with_do)
    if c["dv"] != c["d"]:
        y = workloads.random_inputs(c["B"], c["H"], c["N"], c["dv"], c["dtype"], c["seed"] + 1,
                                    with_do=with_do)
        x["v"] = y["v"]
        if with_do:
            x["do"] = y["do"]
    if c.get("layout") == "mqa":  # one key/value head shared by every query head
        for n in "kv":
            x[n] = np.broadcast_to(x[n][:, :1], x[n].shape).copy()
    return x


def device_qkv(c, x):
    dt = c["dtype"]
    lay = c.get("layout")
    if lay == "bshd":
        return [bshd(x[n], dt) for n in "qkv"]
    if lay == "packed":  # one [B, N, 3, H, d] buffer
        t = dev(np.stack([x[n].transpose(0, 2, 1, 3) for n in "qkv"], axis=2), dt)
        return [t[:, :, i].transpose(1, 2) for i in range(3)]
    if lay == "mqa":
        q = dev(x["q"], dt)
        return [q] + [dev(x[n][:, :1], dt).expand(q.shape) for n in "kv"]
    return [dev(x[n], dt) for n in "qkv"]


def call_kwargs(c):
    kw = {"causal": c["causal"], "scale": c["scale"]}
    if "window" in c:
        kw["window"] = c["window"]
    if "mask" in c:
        kw["block_mask"] = torch.from_numpy(c["mask"]).to("cuda")
    return kw


def oracle_kwargs(c):
    kw = {"causal": c["causal"], "scale": c["scale"]}
    if "window" in c:
        kw["window"] = c["window"]
    if "mask" in c:
        kw["block_mask"] = c["mask"]
    return kw


def test_combo_layouts_are_what_they_claim():
    """The seeded draw reaches every entry point, dtype, head dim and strided
    layout, and negative and zero scales (a CPU check of the case list)."""
    rng = np.random.default_rng(2024)
    cases = [draw_case(rng, False) for _ in range(N_FWD)]
    assert {c["kind"] for c in cases} == set(KINDS)
    assert {c["dtype"] for c in cases} == {"bf16", "fp16", "fp32"}
    assert {c["d"] for c in cases} == {64, 96, 128, 256}
    assert {c.get("layout") for c in cases} >= {"bshd", "packed", "mqa"}
    assert any(c["scale"] < 0 for c in cases) and any(c["scale"] == 0 for c in cases)
    rng = np.random.default_rng(2025)
    bcases = [draw_case(rng, True) for _ in range(N_BWD)]
    assert {c["kind"] for c in bcases} == set(KINDS)
    assert {c["d"] for c in bcases} >= {64, 128, 256}


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_FWD))
def test_combo_forward(fa, i):
    rng = np.random.default_rng(2024)
    cases = [draw_case(rng, False) for _ in range(N_FWD)]
    c = cases[i]
    log(f"case combo fwd {i}: {describe(c)}")
    x = inputs(c, False)
    q, k, v = device_qkv(c, x)
    o, lse = fa.attn_fwd(q, k, v, **call_kwargs(c))
    torch.cuda.synchronize()
    ro, rl = oracle.dense_fwd(x["q"], x["k"], x["v"], **oracle_kwargs(c))
    compare("O", o.float().cpu().numpy(), ro, c["dtype"])
    compare("LSE", lse.cpu().numpy(), rl, "fp32" if c["dtype"] == "fp32" else "lse")


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_BWD))
def test_combo_backward(fa, i):
    rng = np.random.default_rng(2025)
    cases = [draw_case(rng, True) for _ in range(N_BWD)]
    c = cases[i]
    log(f"case combo bwd {i}: {describe(c)}")
    x = inputs(c, True)
    q, k, v = device_qkv(c, x)
    do = bshd(x["do"], c["dtype"]) if c.get("layout") == "bshd" else dev(x["do"], c["dtype"])
    kw = call_kwargs(c)
    o, lse = fa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.dense_bwd(x["q"], x["k"], x["v"], x["do"], **oracle_kwargs(c))
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, g.float().cpu().numpy(), r, c["dtype"])
