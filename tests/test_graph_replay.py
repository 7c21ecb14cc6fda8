"""Library calls captured in a HIP graph and replayed, as bench.py times them.

Each case runs the call eagerly once, captures the same call (same output
tensors) in a torch CUDA graph, then replays the graph several times.  Before
every replay the outputs are overwritten eagerly with NaN and the device is
synchronized; after it, every output must equal the eager result bit for bit
(forward and backward are deterministic).  The block-sparse backward case uses
a mask whose long key-block lists are split over several dK/dV workgroups, so
it also checks that the per-key-block counters the dQ kernel clears start
from zero on every replay.
"""
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


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


def to_dev(x, names, dtype=torch.bfloat16):
    return [torch.from_numpy(x[n]).to("cuda").to(dtype).contiguous() for n in names]


def replay_and_check(call, outs):
    """call() writes outs; compare graph replays of it with its eager result."""
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, ref)):
            same = torch.equal(t, e)
            log(f"    replay {r} output {i}: bitwise equal {same}")
            assert same, f"replay {r}: output {i} differs from the eager call"


def test_forward_graph_replay(fa):
    x = workloads.random_inputs(1, 2, 777, 128, "bf16", seed=12001)
    q, k, v = to_dev(x, "qkv")
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], device="cuda")
    nb = -(-777 // 64)
    bm = torch.from_numpy((np.random.default_rng(12002).random((1, 2, nb, nb)) < 0.4)
                          .astype(np.uint8)).to("cuda")
    for name, kw in (("causal", dict(causal=True)), ("none", dict(causal=False)),
                     ("window 100", dict(causal=True, window=100)),
                     ("block-sparse", dict(causal=False, block_mask=bm))):
        log(f"case forward graph replay bf16 B=1 H=2 N=777 d=128 {name}")
        replay_and_check(lambda: fa.attn_fwd(q, k, v, out=o, lse=lse,
                                             stream=torch.cuda.current_stream(), **kw), [o, lse])


def test_backward_graph_replay(fa):
    x = workloads.random_inputs(1, 2, 500, 128, "bf16", seed=12003, with_do=True)
    q, k, v, do = to_dev(x, ("q", "k", "v", "do"))
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(1, 2, 500, 128, fa.BF16), dtype=torch.uint8, device="cuda")
    log("case backward graph replay bf16 B=1 H=2 N=500 d=128 causal")
    replay_and_check(lambda: fa.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv,
                                         workspace=ws, stream=torch.cuda.current_stream()),
                     [dq, dk, dv])


def test_block_sparse_backward_graph_replay_split_lists(fa):
    n, h = 4096, 2
    mask = workloads.block_sparse_mask(n, h, 1, 2, 3, seed=12004)  # global blocks: split lists
    x = workloads.random_inputs(1, h, n, 64, "bf16", seed=12005, with_do=True)
    q, k, v, do = to_dev(x, ("q", "k", "v", "do"))
    bm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    o, lse = fa.attn_fwd(q, k, v, causal=False, block_mask=bm)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_block_sparse_workspace_bytes(1, h, n, 64, fa.BF16), dtype=torch.uint8,
                     device="cuda")
    log(f"case block-sparse backward graph replay bf16 B=1 H={h} N={n} d=64")
    replay_and_check(lambda: fa.attn_bwd(q, k, v, o, lse, do, causal=False, dq=dq, dk=dk, dv=dv,
                                         workspace=ws, block_mask=bm,
                                         stream=torch.cuda.current_stream()),
                     [dq, dk, dv])
