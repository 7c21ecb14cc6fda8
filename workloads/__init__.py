"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype the
GPU receives.  It holds none of the attention arithmetic: both the CPU oracle
and the HIP path are fed from here, and neither imports the other.

Every tensor is a C-ordered float32 array of shape [B, H, N, d] whose values are
exactly representable in the named storage dtype, so that a torch tensor made
from it in that dtype carries the very same numbers the oracle sees (upcast to
float64 there).

Shapes and value distributions follow the five workloads the method is checked
and measured on: a tiny fp32 unmasked head, a GPT-2-small-shaped causal layer, the long
context causal head, a ragged-length fp16 case with sharp softmax rows, and the
causal forward+backward case.  A sixth, the long context head under a causal
sliding window of 1024 keys, measures the window path; a seventh, the same
head under a block-sparse mask (``block_sparse_mask``: a band of neighbouring
64-key blocks, global blocks and random blocks per query block, as sparse
long-context patterns use), measures the block-sparse path.  No public dataset is involved; the GPT-2-small
shape stands in for the GPT-2 training workload named on the pages (Road to
Intelligence "FlashAttention", section "What it bought").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # storage / compute dtype of Q, K, V, O
    causal: bool
    B: int
    H: int
    N: int
    d: int
    seed: int
    qk_std: float = 1.0      # Q and K ~ N(0, qk_std^2)
    v_dist: str = "normal"   # "normal" -> N(0,1), "uniform" -> U(-1, 1)
    backward: bool = False   # also draw dO ~ N(0, 1)
    window: int | None = None  # causal sliding window: key j visible to query i iff i - W < j <= i
    sparse: tuple | None = None  # block-sparse pattern: (band, n_global, n_random, mask seed)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def pairs(self) -> int:
        """Visible (query, key) pairs of one head."""
        n, w = self.N, self.window
        if self.sparse is not None:
            raise ValueError("block-sparse pairs depend on the mask: use sparse_pairs(mask)")
        if not self.causal:
            return n * n
        if w is None or w >= n:
            return n * (n + 1) // 2
        return w * (w + 1) // 2 + (n - w) * w  # rows 0..w-1 see i+1 keys, the rest w

    def fwd_flops(self) -> int:
        """Algorithmic forward FLOPs: QK^T and PV over visible pairs only."""
        return 4 * self.d * self.pairs() * self.B * self.H

    def bwd_flops(self) -> int:
        """Algorithmic backward FLOPs: recomputed S, dP, dV, dQ, dK."""
        return 10 * self.d * self.pairs() * self.B * self.H

    def fwd_bytes(self) -> int:
        """Algorithmic forward HBM bytes: read Q, K, V once, write O and fp32 LSE."""
        elt = {"fp32": 4, "fp16": 2, "bf16": 2}[self.dtype]
        n = self.B * self.H * self.N
        return 4 * n * self.d * elt + 4 * n


# The five workloads (shapes, dtypes, masks and value distributions).
WORKLOADS = {
    "tiny_fp32_full": Workload("tiny_fp32_full", "fp32", False, 1, 1, 256, 64, seed=1),
    "gpt2s_causal_bf16": Workload("gpt2s_causal_bf16", "bf16", True, 8, 12, 1024, 64, seed=2),
    "long_causal_bf16": Workload("long_causal_bf16", "bf16", True, 1, 16, 8192, 128, seed=3),
    "ragged_sharp_fp16": Workload("ragged_sharp_fp16", "fp16", False, 2, 8, 4097, 128, seed=4,
                                  qk_std=3.0, v_dist="uniform"),
    "fwd_bwd_causal_bf16": Workload("fwd_bwd_causal_bf16", "bf16", True, 4, 16, 4096, 128, seed=5,
                                    backward=True),
    "long_window_bf16": Workload("long_window_bf16", "bf16", True, 1, 16, 8192, 128, seed=6,
                                 window=1024),
    "long_sparse_bf16": Workload("long_sparse_bf16", "bf16", False, 1, 16, 8192, 128, seed=7,
                                 sparse=(1, 2, 3, 70)),
}


def block_sparse_mask(n, heads, band, n_global, n_random, seed):
    """A uint8 [1, heads, nb, nb] block mask (nb = ceil(n / 64)): query block i
    sees key blocks i - band .. i + band, the first ``n_global`` blocks, and
    ``n_random`` further blocks drawn per (head, query block)."""
    nb = -(-n // 64)
    rng = np.random.default_rng(seed)
    m = np.zeros((1, heads, nb, nb), np.uint8)
    for h in range(heads):
        for i in range(nb):
            m[0, h, i, max(0, i - band):min(nb, i + band + 1)] = 1
            m[0, h, i, :min(nb, n_global)] = 1
            if n_random:
                m[0, h, i, rng.choice(nb, size=min(nb, n_random), replace=False)] = 1
    return m


def sparse_pairs(mask, n, causal=False):
    """Visible (query, key) pairs summed over the heads of a [1, H, nb, nb]
    block mask for sequence length n (the FLOP count of a block-sparse launch
    is 4 d times this, times the batch)."""
    nb = mask.shape[-1]
    size = np.full(nb, 64)
    size[-1] = n - 64 * (nb - 1)
    total = 0
    for h in range(mask.shape[1]):
        for i in range(nb):
            for j in np.nonzero(mask[0, h, i])[0]:
                if causal and j > i:
                    continue
                if causal and j == i:
                    total += size[i] * (size[i] + 1) // 2
                else:
                    total += int(size[i]) * int(size[j])
    return total


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.nan
    return out


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(shape, rng: np.random.Generator, std: float = 1.0, dist: str = "normal") -> np.ndarray:
    if dist == "normal":
        out = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            out *= np.float32(std)
        return out
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    raise ValueError(dist)


def make_inputs(w: Workload, *, B=None, H=None, N=None, seed=None):
    """Q, K, V (and dO for backward workloads) for workload ``w``.

    The draw order is Q, K, V, then dO, from ``numpy.random.default_rng(seed)``.
    B, H, N and seed may be overridden to get a smaller case with the same
    distributions.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (B, H, N, w.d)
    q = round_to_dtype(draw(shape, rng, w.qk_std), w.dtype)
    k = round_to_dtype(draw(shape, rng, w.qk_std), w.dtype)
    v = round_to_dtype(draw(shape, rng, 1.0, w.v_dist), w.dtype)
    out = {"q": q, "k": k, "v": v}
    if w.backward:
        out["do"] = round_to_dtype(draw(shape, rng), w.dtype)
    return out


def random_inputs(B, H, N, d, dtype, seed, qk_std=1.0, v_dist="normal", with_do=False):
    """Ad-hoc seeded inputs for parity sweeps."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    out = {
        "q": round_to_dtype(draw(shape, rng, qk_std), dtype),
        "k": round_to_dtype(draw(shape, rng, qk_std), dtype),
        "v": round_to_dtype(draw(shape, rng, 1.0, v_dist), dtype),
    }
    if with_do:
        out["do"] = round_to_dtype(draw(shape, rng), dtype)
    return out


def needle_inputs(B, H, N, d, dtype, seed, causal, amplitude=16.0, noise=0.05):
    """Structured inputs whose softmax rows are nearly one-hot.

    Query rows are cut into contiguous runs; run r owns basis direction
    ``slot = r % d``.  Every query of the run is ``amplitude * e_slot`` and one
    *target* key at or before the run's first row is ``amplitude * e_slot``, so
    each query of the run attends almost only to that key (score lead of about
    amplitude^2 * scale).  When ``causal`` is set, a *forbidden* key just after
    the run gets ``1.25 * amplitude * e_slot``: it would win if the causal mask
    let it through.  Runs are separated by one plain-noise row, which is where
    the forbidden key of the run before it sits.  Other keys and all values are small noise plus a distinct
    value row per target, so dropping, duplicating or mis-masking a tile moves
    the output by about one value norm.  Runs are placed so that targets fall
    in first, diagonal, tail and last tiles.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = draw(shape, rng) * np.float32(noise)
    k = draw(shape, rng) * np.float32(noise)
    v = draw(shape, rng, 1.0, "uniform")
    amp = np.float32(amplitude)
    # runs of varying length so boundaries land at many tile offsets
    run_lengths = [1, 7, 31, 33, 64, 65, 127, 3]
    starts = []
    pos, i = 0, 0
    while pos < N:
        L = run_lengths[i % len(run_lengths)]
        starts.append((pos, min(N, pos + L)))
        pos += L + 1  # one noise row between runs hosts the forbidden key
        i += 1
    for r, (s, e) in enumerate(starts):
        if r >= d:
            break  # every run needs its own direction; remaining rows stay noise
        slot = r
        # target key: at the run start for causal (visible to the whole run)
        t = s if causal else (s + e) // 2
        q[:, :, s:e, :] = 0.0
        q[:, :, s:e, slot] = amp
        k[:, :, t, :] = 0.0
        k[:, :, t, slot] = amp
        if causal and e < N:
            k[:, :, e, :] = 0.0
            k[:, :, e, slot] = np.float32(1.25) * amp
    return {
        "q": round_to_dtype(q, dtype),
        "k": round_to_dtype(k, dtype),
        "v": round_to_dtype(v, dtype),
    }
