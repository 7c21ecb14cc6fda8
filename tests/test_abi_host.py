"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/fa_attn.h declares, and
reject bad arguments with the documented status codes before it enqueues any
work -- so these calls never reach the GPU.
"""
import ctypes
import math
import os

import pytest

import io_aware_exact_12_amd as fa

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_DTYPE, FA_ERR_MASK, FA_ERR_SCALE, \
    FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_ALIGN, FA_ERR_WINDOW, \
    FA_ERR_STRIDE, FA_ERR_SCRATCH = range(13)

# fake, never-dereferenced addresses: validation fails before any use
P = [0x10000 * (i + 1) for i in range(8)]


def fwd(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, mask=0, scale=0.125,
        dtype=fa.BF16):
    return fa.attn_fwd_raw(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, None)


def test_library_exports_every_declared_symbol():
    declared = fa.declared_symbols()
    assert {"attn_fwd", "attn_bwd", "attn_fwd_window", "attn_bwd_window", "attn_bwd_workspace_bytes",
            "attn_fwd_kv_outer", "attn_fwd_kv_outer_workspace_bytes", "attn_fwd_strided",
            "attn_bwd_strided", "attn_fwd_block_sparse", "attn_bwd_block_sparse", "attn_fwd_dv",
            "attn_bwd_dv", "attn_bwd_block_sparse_workspace_bytes", "attn_bwd_noalloc",
            "attn_bwd_noalloc_max_rows",
            "fa_status_str",
            "fa_abi_version"} <= set(declared)
    lib = ctypes.CDLL(fa._binding.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert fa.lib().fa_abi_version() == 11


def test_status_strings():
    for st in range(13):
        assert fa.status_str(st) and fa.status_str(st) != "unknown status"
    assert fa.status_str(123) == "unknown status"


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_null_pointers(which):
    assert fwd(**{which: None}) == FA_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=-5), dict(B=-1),
                                dict(N=2**40), dict(B=2**31, H=2**31)])
def test_bad_shapes(kw):
    assert fwd(**kw) == FA_ERR_SHAPE


@pytest.mark.parametrize("d", [1, 32, 80, 127, 192, 257, 512])
def test_unsupported_head_dim(d):
    assert fwd(d=d) == FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [-1, 3, 99])
def test_bad_dtype(dtype):
    assert fwd(dtype=dtype) == FA_ERR_DTYPE


@pytest.mark.parametrize("mask", [-1, 2, 7])
def test_bad_mask(mask):
    assert fwd(mask=mask) == FA_ERR_MASK


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_bad_scale(scale):
    assert fwd(scale=scale) == FA_ERR_SCALE


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_misaligned(which):
    assert fwd(**{which: P[5] + 2}) == FA_ERR_ALIGN


def test_misaligned_lse():
    assert fwd(lse=P[6] + 2) == FA_ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attn_fwd(x, x, x)


def test_header_documents_each_status():
    text = open(fa._binding.HEADER).read()
    for name in ["FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_DTYPE", "FA_ERR_MASK",
                 "FA_ERR_SCALE", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_ALIGN",
                 "FA_ERR_WORKSPACE", "FA_ERR_WINDOW", "FA_ERR_STRIDE"]:
        assert name in text


def test_no_oracle_in_product_path():
    """The package and its C sources never reference the oracle."""
    pkg = os.path.dirname(fa.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


# ---------------------------------------------------------------- backward validation

def bwd(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[0] + 0x100000,
        B=1, H=1, N=16, d=64, mask=0, scale=0.125, dtype=fa.BF16, ws=P[1] + 0x100000, ws_bytes=1 << 20):
    return fa.attn_bwd_raw(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, mask, scale, dtype, ws, ws_bytes,
                           None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"])
def test_bwd_null_pointers(which):
    assert bwd(**{which: None}) == FA_ERR_NULL


@pytest.mark.parametrize("kw,status", [(dict(B=0), FA_ERR_SHAPE), (dict(N=-1), FA_ERR_SHAPE),
                                       (dict(d=80), FA_ERR_UNSUPPORTED), (dict(dtype=7), FA_ERR_DTYPE),
                                       (dict(mask=3), FA_ERR_MASK), (dict(scale=math.nan), FA_ERR_SCALE),
                                       (dict(dtype=fa.F32), FA_ERR_UNSUPPORTED),
                                       (dict(ws=None), FA_ERR_WORKSPACE),
                                       (dict(ws_bytes=4 * 16 - 1), FA_ERR_WORKSPACE),
                                       (dict(dq=P[6] + 4), FA_ERR_ALIGN), (dict(lse=P[5] + 2), FA_ERR_ALIGN)])
def test_bwd_validation(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_query():
    assert fa.bwd_workspace_bytes(4, 16, 4096, 128, fa.BF16) == 8 * 4 * 16 * 4096
    assert fa.bwd_workspace_bytes(0, 16, 4096, 128, fa.BF16) == 0
    assert fa.bwd_workspace_bytes(1, 1, 16, 80, fa.BF16) == 0
    assert fa.bwd_workspace_bytes(1, 1, 16, 96, fa.BF16) == 8 * 16


# ---------------------------------------------------------------- sliding window

def fwd_w(window, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, scale=0.125,
          dtype=fa.BF16):
    return fa.attn_fwd_window_raw(q, k, v, o, lse, B, H, N, d, window, scale, dtype, None)


def bwd_w(window, ws_bytes=1 << 20, **kw):
    a = dict(B=1, H=1, N=16, d=64, scale=0.125, dtype=fa.BF16, q=P[0])
    a.update(kw)
    return fa.attn_bwd_window_raw(a["q"], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0], a["B"],
                                  a["H"], a["N"], a["d"], window, a["scale"], a["dtype"], P[1],
                                  ws_bytes, None)


@pytest.mark.parametrize("window", [0, -1, -(2**40)])
def test_window_below_one_rejected(window):
    assert fwd_w(window) == FA_ERR_WINDOW
    assert bwd_w(window) == FA_ERR_WINDOW


def test_window_checks_like_the_plain_calls():
    assert fwd_w(4, q=None) == FA_ERR_NULL
    assert fwd_w(4, N=0) == FA_ERR_SHAPE
    assert fwd_w(4, d=80) == FA_ERR_UNSUPPORTED
    assert fwd_w(4, dtype=7) == FA_ERR_DTYPE
    assert fwd_w(4, scale=math.inf) == FA_ERR_SCALE
    assert fwd_w(4, q=P[0] + 8) == FA_ERR_ALIGN
    assert bwd_w(4, dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert bwd_w(4, ws_bytes=8) == FA_ERR_WORKSPACE


# ---------------------------------------------------------------- key/value-outer order

def kvo(ws=P[5], ws_bytes=1 << 30, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, mask=0, scale=0.125,
             dtype=fa.BF16)
    a.update(kw)
    return fa.attn_fwd_kv_outer_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                    a["d"], a["mask"], a["scale"], a["dtype"], ws, ws_bytes, None)


def test_kv_outer_workspace_query():
    # fp32 (4 d bytes) output state plus fp32 maximum and denominator per row
    assert fa.kv_outer_workspace_bytes(1, 16, 8192, 128, fa.BF16) == (4 * 128 + 8) * 16 * 8192
    assert fa.kv_outer_workspace_bytes(2, 3, 5, 64, fa.F16) == (4 * 64 + 8) * 30
    assert fa.kv_outer_workspace_bytes(1, 1, 16, 64, fa.F32) == 0
    assert fa.kv_outer_workspace_bytes(1, 1, 16, 80, fa.BF16) == 0
    assert fa.kv_outer_workspace_bytes(0, 1, 16, 64, fa.BF16) == 0


def test_kv_outer_validation():
    assert kvo(q=None) == FA_ERR_NULL
    assert kvo(o=None) == FA_ERR_NULL
    assert kvo(N=0) == FA_ERR_SHAPE
    assert kvo(d=80) == FA_ERR_UNSUPPORTED
    assert kvo(dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert kvo(dtype=9) == FA_ERR_DTYPE
    assert kvo(mask=3) == FA_ERR_MASK
    assert kvo(scale=math.nan) == FA_ERR_SCALE
    assert kvo(ws=None) == FA_ERR_WORKSPACE
    assert kvo(ws_bytes=(4 * 64 + 8) * 16 - 1) == FA_ERR_WORKSPACE
    assert kvo(ws=P[5] + 4) == FA_ERR_ALIGN
    assert kvo(v=P[2] + 2) == FA_ERR_ALIGN


# ---------------------------------------------------------------- strided views

DENSE = (1 * 16 * 64, 16 * 64, 64)   # B=1, H=1, N=16, d=64 as [B][H][N][d]


def fwd_s(q_st=DENSE, kv_st=DENSE, o_st=DENSE, **kw):
    a = dict(B=1, H=1, N=16, d=64, mask=0, scale=0.125, dtype=fa.BF16)
    a.update(kw)
    return fa.attn_fwd_strided_raw(P[0], P[1], P[2], P[3], P[4], a["B"], a["H"], a["N"], a["d"],
                                   q_st, kv_st, o_st, a["mask"], a["scale"], a["dtype"], None)


def bwd_s(in_st=DENSE, g_st=DENSE, **kw):
    a = dict(B=1, H=1, N=16, d=64, mask=0, scale=0.125, dtype=fa.BF16)
    a.update(kw)
    return fa.attn_bwd_strided_raw(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0], a["B"],
                                   a["H"], a["N"], a["d"], in_st, g_st, a["mask"], a["scale"],
                                   a["dtype"], P[1], 1 << 20, None)


def test_strided_null_arrays():
    assert fwd_s(q_st=None) == FA_ERR_NULL
    assert fwd_s(kv_st=None) == FA_ERR_NULL
    assert fwd_s(o_st=None) == FA_ERR_NULL
    assert bwd_s(in_st=None) == FA_ERR_NULL
    assert bwd_s(g_st=None) == FA_ERR_NULL


@pytest.mark.parametrize("st", [(-64, 1024, 64), (1024, 1024, 60), (1024, 1028, 64), (1024, 1024, 32),
                                (8, 1024, 64 + 4)])
def test_strided_rejects_unusable_input_strides(st):
    """Negative, not a multiple of 16 bytes (8 bf16 elements), or rows closer than d."""
    assert fwd_s(q_st=st) == FA_ERR_STRIDE
    assert fwd_s(kv_st=st) == FA_ERR_STRIDE
    assert bwd_s(in_st=st) == FA_ERR_STRIDE


def test_strided_fp32_alignment_is_four_elements():
    st = fa.attn_fwd_strided_raw(P[0] + 4, P[1], P[2], P[3], P[4], 1, 1, 16, 64, (0, 0, 68), DENSE,
                                 DENSE, 0, 0.125, fa.F32, None)
    assert st == FA_ERR_ALIGN                       # 68 floats = 272 bytes: the strides pass
    assert fwd_s(q_st=(0, 0, 66), dtype=fa.F32) == FA_ERR_STRIDE   # 264 bytes: not 16-aligned


def test_strided_broadcast_inputs_are_allowed_outputs_are_not():
    """k and v may share one head across all query heads (head stride 0); an
    output may not: its heads would overlap."""
    H, N, d = 4, 16, 64
    dense = (H * N * d, N * d, d)
    mqa = (N * d, 0, d)
    # a launch is not wanted here: check that the stride check passes by
    # making the next check (pointer alignment) fail instead
    st = fa.attn_fwd_strided_raw(P[0] + 2, P[1], P[2], P[3], P[4], 1, H, N, d, dense, mqa, dense, 0,
                                 0.125, fa.BF16, None)
    assert st == FA_ERR_ALIGN
    assert fa.attn_fwd_strided_raw(P[0], P[1], P[2], P[3], P[4], 1, H, N, d, dense, dense, mqa, 0,
                                   0.125, fa.BF16, None) == FA_ERR_STRIDE
    assert bwd_s(g_st=(N * d, 0, d), H=H) == FA_ERR_STRIDE


@pytest.mark.parametrize("o_st,ok", [((16 * 4 * 64, 64, 4 * 64), True),     # [B][N][H][d]
                                     ((16 * 4 * 64, 16 * 64, 64), True),    # dense
                                     ((16 * 4 * 64, 32, 4 * 64), False),    # heads overlap within a row
                                     ((16 * 4 * 64, 64, 2 * 64), False),    # rows overlap heads
                                     ((0, 16 * 64, 64), False)])            # batches overlap (B = 2)
def test_strided_output_overlap_check(o_st, ok):
    st = fa.attn_fwd_strided_raw(P[0] + 2, P[1], P[2], P[3], P[4], 2, 4, 16, 64,
                                 (16 * 4 * 64, 16 * 64, 64), (16 * 4 * 64, 16 * 64, 64), o_st, 0,
                                 0.125, fa.BF16, None)
    assert st == (FA_ERR_ALIGN if ok else FA_ERR_STRIDE)


def test_head_extent_limit():
    """One head's rows must span less than 2 GiB (one buffer resource)."""
    assert fwd(N=(1 << 24), d=64) == FA_ERR_SHAPE          # 2 GiB of bf16 rows
    assert fwd_s(q_st=(0, 0, 1 << 20), N=2048) == FA_ERR_SHAPE  # rows 2 MiB apart


# ---------------------------------------------------------------- block-sparse

def fwd_bs(mask_ptr=P[7], mb=1, mh=1, **kw):
    a = dict(q=P[0], B=2, H=3, N=200, d=64, mask=0, scale=0.125, dtype=fa.BF16)
    a.update(kw)
    return fa.attn_fwd_block_sparse_raw(a["q"], P[1], P[2], P[3], P[4], a["B"], a["H"], a["N"], a["d"],
                                        mask_ptr, mb, mh, a["mask"], a["scale"], a["dtype"], None)


def test_block_sparse_validation():
    assert fwd_bs(mask_ptr=None) == FA_ERR_NULL
    assert fwd_bs(mb=0) == FA_ERR_SHAPE
    assert fwd_bs(mb=3) == FA_ERR_SHAPE      # neither 1 nor B
    assert fwd_bs(mh=2) == FA_ERR_SHAPE      # neither 1 nor H
    assert fwd_bs(N=2048 * 64 + 1) == FA_ERR_UNSUPPORTED   # more key tiles than the list holds
    assert fwd_bs(d=80) == FA_ERR_UNSUPPORTED
    assert fwd_bs(dtype=5) == FA_ERR_DTYPE
    assert fwd_bs(mask=2) == FA_ERR_MASK
    # accepted shapes reach the pointer checks (no launch here)
    for mb, mh in ((1, 1), (2, 1), (1, 3), (2, 3)):
        assert fwd_bs(q=P[0] + 2, mb=mb, mh=mh) == FA_ERR_ALIGN
    assert fwd_bs(q=P[0] + 2, N=2048 * 64) == FA_ERR_ALIGN


def test_block_sparse_backward_validation():
    def bb(mask_ptr=P[7], mb=1, mh=1, **kw):
        a = dict(q=P[0], B=2, H=3, N=200, d=64, mask=0, scale=0.125, dtype=fa.BF16, ws=1 << 24)
        a.update(kw)
        return fa.attn_bwd_block_sparse_raw(a["q"], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0],
                                            a["B"], a["H"], a["N"], a["d"], mask_ptr, mb, mh, a["mask"],
                                            a["scale"], a["dtype"], P[1], a["ws"], None)
    assert bb(mask_ptr=None) == FA_ERR_NULL
    assert bb(mb=3) == FA_ERR_SHAPE
    assert bb(mh=2) == FA_ERR_SHAPE
    assert bb(N=2048 * 64 + 1, ws=1 << 40) == FA_ERR_UNSUPPORTED
    assert bb(dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert bb(ws=8) == FA_ERR_WORKSPACE
    assert bb(q=P[0] + 2, mb=2, mh=3) == FA_ERR_ALIGN   # accepted shapes reach the pointer checks


def test_dv_validation():
    def fdv(d, dv, q=P[0], **kw):
        a = dict(B=1, H=1, N=16, mask=0, scale=0.125, dtype=fa.BF16)
        a.update(kw)
        return fa.attn_fwd_dv_raw(q, P[1], P[2], P[3], P[4], a["B"], a["H"], a["N"], d, dv, a["mask"],
                                  a["scale"], a["dtype"], None)
    assert fdv(128, 0) == FA_ERR_SHAPE
    for d, dv in ((128, 32), (256, 32), (80, 64), (64, 80), (256, 512)):
        assert fdv(d, dv) == FA_ERR_UNSUPPORTED, (d, dv)
    for d, dv in ((256, 64), (128, 256)):                      # the d = 256 kernels: no fp32
        assert fdv(d, dv, dtype=fa.F32) == FA_ERR_UNSUPPORTED, (d, dv)
    for d, dv in ((128, 64), (64, 128), (128, 96), (96, 128), (96, 64), (64, 96), (128, 128), (96, 96),
                  (256, 64), (256, 96), (256, 128), (64, 256), (96, 256), (128, 256)):
        assert fdv(d, dv, q=P[0] + 2) == FA_ERR_ALIGN, (d, dv)  # accepted: reaches the pointer checks
    assert fdv(128, 64, q=None) == FA_ERR_NULL
    assert fdv(64, 128, N=(1 << 23)) == FA_ERR_SHAPE           # v rows of a head span 2 GiB


def test_bwd_dv_validation():
    def bdv(d, dv, q=P[0], **kw):
        a = dict(B=1, H=1, N=16, mask=0, scale=0.125, dtype=fa.BF16, ws=1 << 20)
        a.update(kw)
        return fa.attn_bwd_dv_raw(q, P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0], a["B"], a["H"],
                                  a["N"], d, dv, a["mask"], a["scale"], a["dtype"], P[1], a["ws"], None)
    assert bdv(128, 0) == FA_ERR_SHAPE
    for d, dv in ((128, 32), (256, 32), (80, 64), (64, 80), (256, 512)):
        assert bdv(d, dv) == FA_ERR_UNSUPPORTED, (d, dv)
    assert bdv(256, 128, dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert bdv(128, 64, dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert bdv(128, 64, ws=8) == FA_ERR_WORKSPACE
    for d, dv in ((128, 64), (64, 128), (128, 96), (96, 128), (96, 64), (64, 96), (128, 128), (96, 96),
                  (256, 64), (256, 96), (256, 128), (64, 256), (96, 256), (128, 256)):
        assert bdv(d, dv, q=P[0] + 2) == FA_ERR_ALIGN, (d, dv)  # accepted: reaches the pointer checks
    assert bdv(128, 64, q=None) == FA_ERR_NULL
    assert bdv(64, 128, N=(1 << 23), ws=1 << 40) == FA_ERR_SHAPE  # v rows of a head span 2 GiB


def test_wide_head_validation():
    """d = 256: the plain, sliding-window, block-sparse and d_v != d forward and
    backward (bf16 / fp16) reach the pointer checks; fp32 and every variant
    they do not take return FA_ERR_UNSUPPORTED."""
    assert fwd(d=256, q=P[0] + 2) == FA_ERR_ALIGN
    assert fwd(d=256, dtype=fa.F16, mask=1, q=P[0] + 2) == FA_ERR_ALIGN
    assert fwd(d=256, dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert fwd(d=256, N=(1 << 22)) == FA_ERR_SHAPE      # one head spans 2 GiB
    assert fwd_w(4, d=256, N=64, q=P[0] + 2) == FA_ERR_ALIGN
    assert fwd_w(64, d=256, N=64, q=P[0] + 2) == FA_ERR_ALIGN   # a window >= N is plain causal
    assert fwd_bs(d=256, q=P[0] + 2) == FA_ERR_ALIGN
    assert fa.attn_fwd_dv_raw(P[0] + 2, P[1], P[2], P[3], P[4], 1, 1, 16, 256, 128, 0, 0.1, fa.BF16,
                              None) == FA_ERR_ALIGN         # d_v != d with a 256 side: accepted
    assert fa.attn_fwd_dv_raw(P[0], P[1], P[2], P[3], P[4], 1, 1, 16, 256, 128, 0, 0.1, fa.F32,
                              None) == FA_ERR_UNSUPPORTED
    assert fa.attn_fwd_dv_raw(P[0] + 2, P[1], P[2], P[3], P[4], 1, 1, 16, 256, 256, 0, 0.1, fa.BF16,
                              None) == FA_ERR_ALIGN
    assert bwd(d=256, q=P[0] + 2) == FA_ERR_ALIGN
    assert bwd(d=256, dtype=fa.F32) == FA_ERR_UNSUPPORTED
    assert bwd_w(4, d=256, N=64, q=P[0] + 2) == FA_ERR_ALIGN
    assert fa.attn_bwd_block_sparse_raw(P[0] + 2, P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0], 1, 1,
                                        64, 256, P[7], 1, 1, 0, 0.1, fa.BF16, P[1], 1 << 20,
                                        None) == FA_ERR_ALIGN
    assert fa.bwd_workspace_bytes(1, 1, 16, 256, fa.BF16) == 8 * 16
    assert kvo(d=256) == FA_ERR_UNSUPPORTED
    assert fa.kv_outer_workspace_bytes(1, 1, 16, 256, fa.BF16) == 0


def test_block_sparse_backward_workspace():
    """The block-sparse backward needs, past attn_bwd's 8 bytes per query, a
    counter per 128 keys and fp32 partial dK and dV of four chunks per key,
    each array on a 256-byte boundary."""
    up = lambda x: (x + 255) // 256 * 256
    for B, H, N, d in ((1, 16, 8192, 128), (2, 3, 200, 64), (1, 1, 1, 96), (1, 1, 16, 256)):
        bh = B * H
        cnt = up(8 * bh * N)
        part = up(cnt + 4 * bh * (-(-N // 128)))
        want = part + 4 * 4 * bh * N * 2 * d
        assert fa.bwd_block_sparse_workspace_bytes(B, H, N, d, fa.BF16) == want
    assert fa.bwd_block_sparse_workspace_bytes(1, 1, 16, 80, fa.BF16) == 0
    need = fa.bwd_block_sparse_workspace_bytes(2, 3, 200, 64, fa.BF16)
    def bb(ws):
        return fa.attn_bwd_block_sparse_raw(P[0] + 2, P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0], 2, 3,
                                            200, 64, P[7], 1, 1, 0, 0.125, fa.BF16, P[1], ws, None)
    assert bb(need - 1) == FA_ERR_WORKSPACE
    assert bb(need) == FA_ERR_ALIGN        # big enough: reaches the pointer checks


# ------------------------------------------------------------------ caller buffers

def test_binding_rejects_mismatched_buffers():
    """The binding passes raw pointers, so every caller-supplied output or
    scratch tensor is checked against what the kernels write through it:
    shape, dtype, device and contiguity (host tensors stand in for device
    ones; the device compared is q's)."""
    torch = pytest.importorskip("torch")
    from io_aware_exact_12_amd._binding import check_buffer, check_workspace
    cpu = torch.device("cpu")
    good = torch.empty((2, 3, 5, 64), dtype=torch.bfloat16)
    check_buffer(good, "out", (2, 3, 5, 64), torch.bfloat16, cpu)          # accepted
    with pytest.raises(ValueError, match="shape"):                          # too small an out
        check_buffer(torch.empty((2, 3, 4, 64), dtype=torch.bfloat16), "out", (2, 3, 5, 64),
                     torch.bfloat16, cpu)
    with pytest.raises(TypeError, match="float16"):                         # another 16-bit type
        check_buffer(good, "out", (2, 3, 5, 64), torch.float16, cpu)
    with pytest.raises(TypeError, match="float32"):                         # bf16 lse
        check_buffer(torch.empty((2, 3, 5), dtype=torch.bfloat16), "lse", (2, 3, 5), torch.float32, cpu)
    with pytest.raises(ValueError, match="shape"):                          # lse of another shape
        check_buffer(torch.empty((2, 3, 6), dtype=torch.float32), "lse", (2, 3, 5), torch.float32, cpu)
    with pytest.raises(ValueError, match="on"):                             # another device
        check_buffer(good.to("meta"), "dq", (2, 3, 5, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="contiguous"):                     # strided lse
        check_buffer(torch.empty((2, 3, 10), dtype=torch.float32)[..., ::2], "lse", (2, 3, 5),
                     torch.float32, cpu)
    t = torch.empty((2, 5, 3, 64), dtype=torch.bfloat16).transpose(1, 2)    # [B][N][H][d] view
    check_buffer(t, "dq", (2, 3, 5, 64), torch.bfloat16, cpu, contiguous=False)
    with pytest.raises(ValueError, match="last axis"):
        check_buffer(torch.empty((2, 3, 5, 128), dtype=torch.bfloat16)[..., ::2], "dq",
                     (2, 3, 5, 64), torch.bfloat16, cpu, contiguous=False)
    ws = torch.empty(100, dtype=torch.uint8)
    check_workspace(ws, 100, cpu)
    with pytest.raises(ValueError, match="needed"):
        check_workspace(ws, 101, cpu)
    with pytest.raises(TypeError, match="uint8"):
        check_workspace(torch.empty(100, dtype=torch.int8), 100, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        check_workspace(torch.empty(200, dtype=torch.uint8)[::2], 100, cpu)
    with pytest.raises(ValueError, match="on"):
        check_workspace(ws.to("meta"), 100, cpu)


def test_dv_calls_reject_huge_n_before_multiplying():
    """attn_fwd_dv / attn_bwd_dv bound N before forming N * d_v * 4, so a huge
    N is a shape error, not an overflowed product."""
    L = fa.lib()
    huge = 1 << 61
    assert fa.attn_fwd_dv_raw(16, 16, 16, 16, None, 1, 1, huge, 128, 64, 0, 0.1, fa.BF16, None) == FA_ERR_SHAPE
    assert fa.attn_bwd_dv_raw(16, 16, 16, 16, 16, 16, 16, 16, 16, 1, 1, huge, 128, 64, 0, 0.1,
                              fa.BF16, 16, 1 << 20, None) == FA_ERR_SHAPE
    assert L is not None


def test_block_sparse_backward_grid_bound():
    """The split block-sparse backward runs up to four dK/dV workgroups per
    128-key block and head; a problem whose grid would pass 2^31 - 1 is a
    shape error before any launch."""
    st = fa.attn_bwd_block_sparse_raw(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0] + 0x100000,
                                      1, 1 << 30, 16, 64, P[1] + 0x100000, 1, 1, 0, 0.1, fa.BF16,
                                      P[2] + 0x100000, (1 << 63) - 1, None)
    assert st == FA_ERR_SHAPE
