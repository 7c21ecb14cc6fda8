"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd.

attn_bwd_noalloc runs attn_bwd's kernels with the library's fixed per-GPU
scratch in place of a caller workspace, so its gradients must be bitwise those
of attn_bwd.  Two calls in a row, the second on a smaller input, check that
the scratch left by the first call does not leak into the second; the raw
C entry point is called directly.  Shape errors are checked on the host.
"""
import sys

import numpy as np
import pytest

import io_aware_exact_12_amd as fa
import oracle
import whole_output
import workloads

torch = pytest.importorskip("torch")
FA_ERR_SCRATCH = 12


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_rejects_too_large_problems():
    """Beyond the fixed scratch (B * H * N rows) the call fails with
    FA_ERR_SCRATCH before it touches any pointer or the GPU."""
    rows = fa.noalloc_max_rows()
    assert rows == (8 << 20) // 8
    P = [0x10000 * (i + 1) for i in range(9)]
    st = fa.attn_bwd_noalloc_raw(*P, 1, 1, rows + 1, 128, 1, 0.1, fa.BF16, None)
    assert st == FA_ERR_SCRATCH, st
    st = fa.attn_bwd_noalloc_raw(*P, 2, 8, rows // 16 + 1, 128, 1, 0.1, fa.BF16, None)
    assert st == FA_ERR_SCRATCH, st
    assert "scratch" in fa.status_str(FA_ERR_SCRATCH)


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()
    cases = [(2, 8, 1537, 128, "bf16", True, 31), (1, 3, 300, 64, "fp16", False, 32)]
    for B, H, N, d, dtype, causal, seed in cases:
        log(f"case noalloc B={B} H={H} N={N} d={d} {dtype} causal={causal} seed={seed}")
        x = workloads.random_inputs(B, H, N, d, dtype, seed, with_do=True)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        q, k, v, do = (torch.from_numpy(x[n]).to("cuda").to(tdt).contiguous()
                       for n in ("q", "k", "v", "do"))
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        ref = fa.attn_bwd(q, k, v, o, lse, do, causal=causal)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        st = fa.attn_bwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     do.data_ptr(), lse.data_ptr(), got[0].data_ptr(),
                                     got[1].data_ptr(), got[2].data_ptr(), B, H, N, d,
                                     1 if causal else 0, 1.0 / np.sqrt(d),
                                     fa.BF16 if dtype == "bf16" else fa.F16,
                                     torch.cuda.current_stream().cuda_stream)
        assert st == 0, fa.status_str(st)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), f"{name} differs from attn_bwd"
        # and both within the oracle's tolerance on two heads
        grads = [t.float().cpu().numpy() for t in got]
        whole_output.compare_bwd_all_heads(grads, x, causal, 1.0 / np.sqrt(d), (2e-2, 1e-2), 2e-2,
                                           heads=[(0, 0), (B - 1, H - 1)], label="noalloc ")
    assert oracle is not None
