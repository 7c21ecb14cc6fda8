"""Pins for the float64 CPU oracle (no GPU).

The oracle is checked against facts fixed by the pages (worked examples, the
explorer's self-check, the transfer ledger), closed forms, invariants and
library routines that compute the same textbook quantity.  A final group plants
plausible mistakes in a copy of the online recurrence and shows that these
pins catch each one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

RNG = np.random.default_rng(1234)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rand(*shape, seed=0, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------- page facts

def test_two_block_row_matches_worked_example(golden_dir):
    """Road to Intelligence 'FlashAttention', 'The trick that makes tiling possible'."""
    g = _load(golden_dir, "two_block_row.json")
    tol = g["printed_tolerance"]
    scores = [x for blk in g["blocks"] for x in blk]
    # one query, d = 1, q = 1, keys = the scores, scale 1: raw scores are the page's scores
    q = np.array([[1.0]])
    k = np.array(scores, dtype=np.float64)[:, None]
    v = np.eye(len(scores))  # a one-hot value per key exposes the weights
    trace = []
    o, lse = oracle.online_fwd(q, k, v, scale=1.0, query_block=1, key_block=2, trace=trace)
    assert len(trace) == 2
    t1, t2 = trace
    assert t1["m"][0] == g["after_block_1"]["m"]
    assert abs(t1["l"][0] - g["after_block_1"]["l"]) <= tol
    assert t2["m"][0] == g["after_block_2"]["m"]
    assert abs(t2["l"][0] - g["after_block_2"]["l"]) <= tol
    # the rescale factor applied to the old sum is exp(3 - 5)
    old_sum_scaled = t2["l"][0] - (math.exp(2 - 5) + math.exp(5 - 5))
    assert abs(old_sum_scaled / t1["l"][0] - g["after_block_2"]["rescale"]) <= tol
    for printed, exact in zip(g["after_block_2"]["terms"],
                              [t1["l"][0] * math.exp(3 - 5), math.exp(2 - 5), 1.0]):
        assert abs(printed - exact) <= tol
    # direct one-pass sum
    direct = sum(math.exp(s - 5) for s in scores)
    assert abs(direct - g["direct"]["l"]) <= tol
    for printed, s in zip(g["direct"]["terms"], [1, 3, 2, 5]):
        assert abs(printed - math.exp(s - 5)) <= tol
    # and the exact values: l1 = 1 + e^-2, l2 = e^-4 + e^-2 + e^-3 + 1
    assert t1["l"][0] == pytest.approx(1 + math.exp(-2), rel=1e-15)
    assert t2["l"][0] == pytest.approx(direct, rel=1e-15)
    assert lse[0] == pytest.approx(scipy.special.logsumexp(scores), rel=1e-15)
    np.testing.assert_allclose(o[0], scipy.special.softmax(scores), rtol=1e-14)


def test_explorer_tiled_equals_dense(golden_dir):
    """'Flash Attention: IO-Aware Exact Attention', 'Check the recurrence on CPU'."""
    g = _load(golden_dir, "explorer_vectors.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in "qkv")
    dense, dense_lse = oracle.dense_fwd(q, k, v)
    for kb in g["key_blocks"]:
        tiled, lse = oracle.online_fwd(q, k, v, query_block=g["query_block"], key_block=kb)
        np.testing.assert_allclose(tiled, dense, rtol=g["rtol"], atol=g["atol"])
        np.testing.assert_allclose(lse, dense_lse, rtol=g["rtol"], atol=g["atol"])
    # the same check over every query block size and with the causal mask
    for causal in (False, True):
        ref, ref_lse = oracle.dense_fwd(q, k, v, causal=causal)
        for qb in range(1, 8):
            for kb in range(1, 8):
                o, lse = oracle.online_fwd(q, k, v, causal=causal, query_block=qb, key_block=kb)
                np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_explorer_q0_max_rises_in_every_tile(golden_dir):
    g = _load(golden_dir, "explorer_vectors.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in "qkv")
    trace = []
    oracle.online_fwd(q, k, v, query_block=2, key_block=g["q0_max_rises_with_key_block"], trace=trace)
    m0 = [t["m"][0] for t in trace if t["row0"] == 0]
    assert len(m0) == 3
    assert all(b > a for a, b in zip(m0, m0[1:]))
    # raw dots of Q0 with the six keys are -1, 0, 2, 1, 3, -1: tile maxima 0, 2, 3
    np.testing.assert_allclose(np.array(m0) * math.sqrt(2), [0, 2, 3], rtol=1e-15)
    # the values differ across keys, so the rescale of the numerator matters
    assert len({tuple(r) for r in v}) == len(v)


def test_explorer_causal_rows_closed_form(golden_dir):
    g = _load(golden_dir, "explorer_vectors.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in "qkv")
    o, lse = oracle.online_fwd(q, k, v, causal=True, query_block=2, key_block=2)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert lse[0] == pytest.approx(-1 / math.sqrt(2), rel=1e-15)
    full, full_lse = oracle.dense_fwd(q, k, v)
    np.testing.assert_allclose(o[-1], full[-1], rtol=1e-14)
    assert lse[-1] == pytest.approx(full_lse[-1], rel=1e-14)


def test_transfer_ledger(golden_dir):
    """'Loop order changes which data is reloaded': 240 versus 96 transfers."""
    g = _load(golden_dir, "transfer_ledger.json")
    for kb in range(1, 8):
        led = oracle.transfer_ledger(g["N"], g["d"], g["d_v"], g["query_block"], kb)
        for key in ("Q_read", "K_read", "V_read", "O_write"):
            assert led["tiled"][key] == g[key]
        for key in ("S_write", "S_read", "P_write", "P_read"):
            assert led["dense"][key] == g[key]
        assert led["dense_total"] == g["dense_total"]
        assert led["tiled_total"] == g["tiled_total"]
    # the S and P round trips alone move 4 N^2 elements
    # ('Why intermediate matrices cost memory traffic')
    for n in (6, 17, 64):
        led = oracle.transfer_ledger(n, 2, 2, 4, 3)
        assert led["dense_total"] - led["tiled_total"] == 4 * n * n


# ---------------------------------------------------------------- values of another width

@pytest.mark.parametrize("d,dv", [(8, 4), (4, 12)])
def test_dv_differs_from_d(d, dv):
    """V of width d_v != d ("Flash Attention: IO-Aware Exact Attention" defines V
    as N x d_v): the dense oracle against torch's attention, and the online
    recurrence of both loop orders against the dense oracle."""
    q, k = _rand(2, 70, d, seed=171, std=2), _rand(2, 70, d, seed=172, std=2)
    v = _rand(2, 70, dv, seed=173)
    for causal in (False, True):
        o, lse = oracle.dense_fwd(q, k, v, causal=causal)
        assert o.shape == (2, 70, dv)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=causal)
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
        for f in (oracle.online_fwd, oracle.online_fwd_kv_outer):
            o2, l2 = f(q, k, v, causal=causal, query_block=9, key_block=16)
            np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l2, lse, rtol=1e-13)


# ---------------------------------------------------------------- block-sparse masks

def _bm(n_qb, n_kb, seed, density=0.4, lead=()):
    return (np.random.default_rng(seed).random(lead + (n_qb, n_kb)) < density).astype(np.uint8)


def test_block_mask_all_ones_is_the_plain_mask():
    q, k, v = _rand(2, 150, 16, seed=101), _rand(2, 150, 16, seed=102), _rand(2, 150, 16, seed=103)
    ones = np.ones((3, 3), np.uint8)
    for causal in (False, True):
        ref = oracle.dense_fwd(q, k, v, causal=causal)
        got = oracle.dense_fwd(q, k, v, causal=causal, block_mask=ones)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])


def test_block_mask_one_block_is_attention_on_that_block():
    """Query block I seeing only key block J is plain attention of q_I on
    (k_J, v_J); the mask is deliberately not symmetric."""
    n = 200
    q, k, v = _rand(n, 8, seed=111, std=2), _rand(n, 8, seed=112, std=2), _rand(n, 8, seed=113)
    bm = np.zeros((4, 4), np.uint8)
    pairs = [(0, 3), (1, 0), (2, 2), (3, 1)]
    for i, j in pairs:
        bm[i, j] = 1
    o, lse = oracle.dense_fwd(q, k, v, block_mask=bm)
    for i, j in pairs:
        r = slice(64 * i, min(n, 64 * i + 64))
        c = slice(64 * j, min(n, 64 * j + 64))
        s = (q[r] @ k[c].T) / math.sqrt(8)
        np.testing.assert_allclose(o[r], scipy.special.softmax(s, axis=1) @ v[c], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[r], scipy.special.logsumexp(s, axis=1), rtol=1e-14)


def test_block_mask_block_diagonal_splits_the_sequence():
    """A block-diagonal mask is attention on each 64-row chunk separately
    (causal inside each chunk as well)."""
    n = 230
    q, k, v = _rand(2, n, 16, seed=121), _rand(2, n, 16, seed=122), _rand(2, n, 16, seed=123)
    bm = np.eye(4, dtype=np.uint8)
    for causal in (False, True):
        o, lse = oracle.dense_fwd(q, k, v, causal=causal, block_mask=bm)
        for c0 in range(0, n, 64):
            c = slice(c0, min(n, c0 + 64))
            ro, rl = oracle.dense_fwd(q[:, c], k[:, c], v[:, c], causal=causal)
            np.testing.assert_allclose(o[:, c], ro, rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(lse[:, c], rl, rtol=1e-14)


def test_block_mask_against_torch_sdpa_and_autograd():
    """Element mask built from the blocks, handed to torch's attention and
    autograd in float64 (rows that see a key)."""
    b, h, n, d = 1, 2, 170, 16
    q, k, v = (_rand(b, h, n, d, seed=130 + i) for i in range(3))
    do = _rand(b, h, n, d, seed=134)
    bm = _bm(3, 3, seed=135, density=0.6, lead=(1, h))
    bm[..., :, 0] = 1   # every row sees block 0, so no row is empty
    for causal in (False, True):
        o, lse = oracle.dense_fwd(q, k, v, causal=causal, block_mask=bm)
        vis = np.take(np.take(bm != 0, np.arange(n) // 64, axis=-2), np.arange(n) // 64, axis=-1)
        if causal:
            vis = vis & np.tril(np.ones((n, n), bool))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(vis))
        np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
        ref.backward(torch.tensor(do))
        dq, dk, dv, _, _ = oracle.dense_bwd(q, k, v, do, causal=causal, block_mask=bm)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_block_mask_empty_rows_give_zero_and_minus_inf():
    n = 130
    q, k, v = _rand(n, 8, seed=141), _rand(n, 8, seed=142), _rand(n, 8, seed=143)
    do = _rand(n, 8, seed=144)
    bm = np.ones((3, 3), np.uint8)
    bm[1, :] = 0              # rows 64..127 see nothing
    o, lse = oracle.dense_fwd(q, k, v, block_mask=bm)
    assert np.all(o[64:128] == 0) and np.all(lse[64:128] == -np.inf)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[:64]))
    dq, dk, dv, _, _ = oracle.dense_bwd(q, k, v, do, block_mask=bm)
    assert np.all(np.isfinite(dq)) and np.all(dq[64:128] == 0)
    # the other rows are untouched by the empty ones
    keep = np.r_[0:64, 128:n]
    ref = oracle.dense_fwd(q[keep], k, v, block_mask=None)
    np.testing.assert_allclose(o[keep], ref[0], rtol=1e-14, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.dense_fwd(q, k, v, block_mask=np.ones((2, 3)))


def test_block_mask_catches_a_transposed_mask():
    """Reading the mask as [key block, query block] fails the single-block pin."""
    n = 128
    q, k, v = _rand(n, 8, seed=151), _rand(n, 8, seed=152), _rand(n, 8, seed=153)
    bm = np.array([[1, 0], [1, 1]], np.uint8)
    good = oracle.dense_fwd(q, k, v, block_mask=bm)[0]
    bad = oracle.dense_fwd(q, k, v, block_mask=bm.T)[0]
    assert not np.allclose(good, bad)
    s = (q[:64] @ k[:64].T) / math.sqrt(8)
    np.testing.assert_allclose(good[:64], scipy.special.softmax(s, axis=1) @ v[:64], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- key/value-outer order

def test_kv_outer_two_block_worked_example(golden_dir):
    """The two-block row of Road to Intelligence 'FlashAttention', 'The trick that
    makes tiling possible', taken through the normalised update of
    'FlashAttention -- the same attention, made memory-aware', section 03."""
    g = _load(golden_dir, "two_block_row.json")
    scores = [x for blk in g["blocks"] for x in blk]
    q = np.array([[1.0]])
    k = np.array(scores, dtype=np.float64)[:, None]
    v = np.eye(len(scores))
    o, lse = oracle.online_fwd_kv_outer(q, k, v, scale=1.0, query_block=1, key_block=2)
    # final denominator and maximum as printed: LSE = m + ln l with m = 5
    assert abs(math.exp(lse[0] - g["after_block_2"]["m"]) - g["after_block_2"]["l"]) <= g["printed_tolerance"]
    np.testing.assert_allclose(o[0], scipy.special.softmax(scores), rtol=1e-14)
    # after the first tile alone the state is the first block's softmax
    o1, lse1 = oracle.online_fwd_kv_outer(q, k[:2], v[:2, :2], scale=1.0, query_block=1, key_block=2)
    assert abs(math.exp(lse1[0] - g["after_block_1"]["m"]) - g["after_block_1"]["l"]) <= g["printed_tolerance"]


def test_kv_outer_equals_dense(golden_dir):
    """Both loop orders reach the dense result ('Loop order changes which data is
    reloaded'): the explorer vectors and random heads, every block size."""
    g = _load(golden_dir, "explorer_vectors.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in "qkv")
    for causal in (False, True):
        ref, ref_lse = oracle.dense_fwd(q, k, v, causal=causal)
        for qb in range(1, 8):
            for kb in range(1, 8):
                o, lse = oracle.online_fwd_kv_outer(q, k, v, causal=causal, query_block=qb, key_block=kb)
                np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    q, k, v = _rand(2, 3, 45, 16, seed=81, std=2), _rand(2, 3, 45, 16, seed=82, std=2), _rand(2, 3, 45, 8, seed=83)
    for causal in (False, True):
        ref, ref_lse = oracle.dense_fwd(q, k, v, causal=causal, scale=0.3)
        for qb, kb in [(1, 45), (45, 1), (7, 16), (64, 64), (16, 7)]:
            o, lse = oracle.online_fwd_kv_outer(q, k, v, causal=causal, scale=0.3, query_block=qb,
                                                key_block=kb)
            np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_kv_outer_negative_scale_and_large_scores():
    """The scale multiplies before the maximum; scores near 700 do not overflow."""
    q, k, v = _rand(20, 8, seed=91, std=9), _rand(20, 8, seed=92, std=9), _rand(20, 8, seed=93)
    for scale in (-0.7, 2.5):
        ref, ref_lse = oracle.dense_fwd(q, k, v, causal=True, scale=scale)
        o, lse = oracle.online_fwd_kv_outer(q, k, v, causal=True, scale=scale, query_block=3, key_block=4)
        np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_loop_order_ledger_explorer(golden_dir):
    """'Loop order changes which data is reloaded': the query-outer order reads
    12 Q, 36 K, 36 V and writes 12 output elements for the explorer; the
    original order reads K and V once but reloads Q and the row state for every
    K/V block."""
    g = _load(golden_dir, "transfer_ledger.json")
    n, d, dv, qb = g["N"], g["d"], g["d_v"], g["query_block"]
    for kb in (1, 2, 3, 6):
        led = oracle.loop_order_ledger(n, d, dv, qb, kb, "q_outer")
        for key in ("Q_read", "K_read", "V_read", "O_write"):
            assert led[key] == g[key]
        assert led["O_read"] == led["stat_read"] == 0 and led["stat_write"] == n
        kv = oracle.loop_order_ledger(n, d, dv, qb, kb, "kv_outer")
        n_tiles = -(-n // kb)
        assert kv["K_read"] == n * d and kv["V_read"] == n * dv        # once
        assert kv["Q_read"] == n_tiles * n * d                         # once per K/V tile
        assert kv["O_write"] == n_tiles * n * dv
        assert kv["O_read"] == (n_tiles - 1) * n * dv                  # not before the first
        assert kv["stat_write"] == 2 * n_tiles * n
    # one query block and one K/V tile: both orders move the same data (up to
    # the statistics)
    a = oracle.loop_order_ledger(n, d, dv, n, n, "q_outer")
    b = oracle.loop_order_ledger(n, d, dv, n, n, "kv_outer")
    for key in ("Q_read", "K_read", "V_read", "O_write", "O_read"):
        assert a[key] == b[key]


def test_loop_order_ledger_causal_by_hand():
    """N = 6, two-row query blocks, two-key tiles, causal: query block 0 sees
    tile 0, block 1 tiles 0 and 1, block 2 tiles 0 to 2 (six visits, counted by
    hand); d = d_v = 2."""
    q = oracle.loop_order_ledger(6, 2, 2, 2, 2, "q_outer", causal=True)
    assert (q["Q_read"], q["K_read"], q["V_read"], q["O_write"]) == (12, 24, 24, 12)
    kv = oracle.loop_order_ledger(6, 2, 2, 2, 2, "kv_outer", causal=True)
    assert (kv["Q_read"], kv["K_read"], kv["V_read"]) == (24, 12, 12)
    assert (kv["O_read"], kv["O_write"], kv["stat_read"], kv["stat_write"]) == (12, 24, 12, 24)
    with pytest.raises(ValueError):
        oracle.loop_order_ledger(6, 2, 2, 2, 2, "diagonal")


def test_tile_merge_is_order_free():
    """The online state is a fold of per-tile summaries with a merge that is
    associative and commutative: any grouping or order of the key tiles gives
    the dense row statistics (m, l, a) of all keys, to rounding."""
    from oracle.attention import _merge, _tile_summary
    rng = np.random.default_rng(5)
    t = rng.normal(0, 3, (4, 13))
    t[1, :5] = -np.inf          # masked keys
    t[2, :] = -np.inf           # a row with no visible key
    vv = rng.normal(0, 1, (13, 3))
    cuts = [(0, 3), (3, 4), (4, 9), (9, 13)]
    parts = [_tile_summary(t[:, a:b], vv[a:b]) for a, b in cuts]
    none = (np.full(4, -np.inf), np.zeros(4), np.zeros((4, 3)))
    left = none
    for p_ in parts:
        left = _merge(left, p_)
    right = _merge(_merge(parts[3], parts[1]), _merge(parts[2], _merge(parts[0], none)))
    whole = _tile_summary(t, vv)
    for got in (left, right):
        np.testing.assert_array_equal(got[0], whole[0])
        np.testing.assert_allclose(got[1], whole[1], rtol=1e-13, atol=0)
        np.testing.assert_allclose(got[2], whole[2], rtol=1e-13, atol=1e-15)
    assert np.isneginf(left[0][2]) and left[1][2] == 0 and not left[2][2].any()
    # and the summary of all keys is the definition: l e^m = sum_j e^{t_j}
    row = 0
    np.testing.assert_allclose(whole[1][row] * np.exp(whole[0][row]), np.exp(t[row]).sum(), rtol=1e-13)


def test_loop_order_ledger_ragged_by_hand():
    """N = 5, d = 3, d_v = 2, two-row query blocks [0,2) [2,4) [4,5) and
    three-key tiles [0,3) [3,5): none of the sizes divides another.  Counted by
    hand from the loop nests of "Loop order changes which data is reloaded".

    Unmasked, key/value outer: K and V read once (15, 10); each of the two
    tiles reads all 5 query rows (2 x 15 = 30); the second tile reloads the
    output rows and both statistics (10, 10); every visit writes them back
    (2 x 10, 2 x 10).  Query outer: Q once (15), every block reads all keys
    (3 x 15 = 45 K, 3 x 10 = 30 V), O and the LSE written once (10, 5).

    Causal: block [0,2) sees tile [0,3) only; the others see both.  Key/value
    outer: tile 0 visits all three blocks (Q 15, O write 10, statistics 10),
    tile 1 the last two (Q 9, O read 6, statistics read 6, O write 6,
    statistics write 6).  Query outer: K 9 + 15 + 15 = 39, V 6 + 10 + 10 = 26."""
    kv = oracle.loop_order_ledger(5, 3, 2, 2, 3, "kv_outer")
    assert kv == {"Q_read": 30, "K_read": 15, "V_read": 10, "O_read": 10, "O_write": 20,
                  "stat_read": 10, "stat_write": 20, "total": 115}
    qo = oracle.loop_order_ledger(5, 3, 2, 2, 3, "q_outer")
    assert qo == {"Q_read": 15, "K_read": 45, "V_read": 30, "O_read": 0, "O_write": 10,
                  "stat_read": 0, "stat_write": 5, "total": 105}
    kvc = oracle.loop_order_ledger(5, 3, 2, 2, 3, "kv_outer", causal=True)
    assert kvc == {"Q_read": 24, "K_read": 15, "V_read": 10, "O_read": 6, "O_write": 16,
                   "stat_read": 6, "stat_write": 16, "total": 93}
    qoc = oracle.loop_order_ledger(5, 3, 2, 2, 3, "q_outer", causal=True)
    assert qoc == {"Q_read": 15, "K_read": 39, "V_read": 26, "O_read": 0, "O_write": 10,
                   "stat_read": 0, "stat_write": 5, "total": 95}


def _mutant_kv_outer(q, k, v, qb, kb, bug):
    """A copy of the key/value-outer merge with one deliberate mistake."""
    n, dv = q.shape[0], v.shape[1]
    out, m, ell = np.zeros((n, dv)), np.full(n, -np.inf), np.zeros(n)
    for c0 in range(0, n, kb):
        cols = np.arange(c0, min(n, c0 + kb))
        for r0 in range(0, n, qb):
            r = np.arange(r0, min(n, r0 + qb))
            t = q[r] @ k[cols].T
            m_t = t.max(1)
            p = np.exp(t - m_t[:, None])
            l_t = p.sum(1)
            m_new = np.maximum(m[r], m_t)
            keep = np.where(np.isfinite(m[r]), np.exp(m[r] - m_new), 0.0)
            take = np.exp(m_t - m_new)
            l_new = keep * ell[r] + take * l_t if bug != "no_keep_on_l" else ell[r] + take * l_t
            w_old = keep * ell[r] if bug != "no_l_old" else keep
            w_new = take if bug != "no_take_on_pv" else np.ones_like(take)
            out[r] = (w_old[:, None] * out[r] + w_new[:, None] * (p @ v[cols])) / l_new[:, None]
            m[r], ell[r] = m_new, l_new
    return out, m + np.log(ell)


@pytest.mark.parametrize("bug", ["no_l_old", "no_keep_on_l", "no_take_on_pv"])
def test_kv_outer_pins_catch_planted_mistakes(bug):
    """The dense-equality pin above rejects each mistake of the merge."""
    q, k, v = _rand(13, 4, seed=74, std=2), _rand(13, 4, seed=75, std=2), _rand(13, 4, seed=76)
    ref, ref_lse = oracle.dense_fwd(q, k, v, scale=1.0)
    good, good_lse = _mutant_kv_outer(q, k, v, 3, 4, bug=None)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(good_lse, ref_lse, rtol=1e-12, atol=1e-12)
    bad, bad_lse = _mutant_kv_outer(q, k, v, 3, 4, bug=bug)
    assert not (np.allclose(bad, ref, rtol=1e-12, atol=1e-12)
                and np.allclose(bad_lse, ref_lse, rtol=1e-12, atol=1e-12))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k = _rand(3, 37, 8, seed=1, std=2), _rand(3, 37, 8, seed=2, std=2)
    p = oracle.dense_probs(q, k, causal=causal)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-15 * 37)
    if causal:
        assert np.all(np.triu(p[0], 1) == 0)


def test_single_key_gives_value():
    q, k, v = _rand(2, 1, 5, seed=3), _rand(2, 1, 5, seed=4), _rand(2, 1, 5, seed=5)
    for fn in (lambda: oracle.dense_fwd(q, k, v, scale=0.7),
               lambda: oracle.online_fwd(q, k, v, scale=0.7, query_block=3, key_block=2)):
        o, lse = fn()
        np.testing.assert_allclose(o, v, rtol=1e-15)
        np.testing.assert_allclose(lse, 0.7 * (q * k).sum(-1), rtol=1e-14)


@pytest.mark.parametrize("n", [1, 5, 33])
def test_zero_queries_average_the_values(n):
    q = np.zeros((1, n, 4))
    k, v = _rand(1, n, 4, seed=6), _rand(1, n, 3, seed=7)
    o, lse = oracle.dense_fwd(q, k, v)
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0].mean(0), (n, 3)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-15)
    oc, lsec = oracle.online_fwd(q, k, v, causal=True, query_block=4, key_block=3)
    cm = np.cumsum(v[0], axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(oc[0], cm, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lsec[0], np.log(np.arange(1, n + 1)), rtol=1e-15, atol=1e-15)


def test_equal_values_give_that_value():
    q, k = _rand(2, 19, 6, seed=8, std=3), _rand(2, 19, 6, seed=9, std=3)
    row = _rand(6, seed=10)
    v = np.broadcast_to(row, (2, 19, 6)).copy()
    for causal in (False, True):
        o, _ = oracle.online_fwd(q, k, v, causal=causal, query_block=5, key_block=4)
        np.testing.assert_allclose(o, v, rtol=1e-13)


def test_causal_first_and_last_rows():
    q, k, v = _rand(2, 23, 8, seed=11), _rand(2, 23, 8, seed=12), _rand(2, 23, 8, seed=13)
    o, lse = oracle.dense_fwd(q, k, v, causal=True, scale=0.3)
    full, full_lse = oracle.dense_fwd(q, k, v, causal=False, scale=0.3)
    np.testing.assert_allclose(o[:, 0], v[:, 0], rtol=1e-15)
    np.testing.assert_allclose(lse[:, 0], 0.3 * (q[:, 0] * k[:, 0]).sum(-1), rtol=1e-14)
    np.testing.assert_allclose(o[:, -1], full[:, -1], rtol=1e-15)
    np.testing.assert_allclose(lse[:, -1], full_lse[:, -1], rtol=1e-15)


# ---------------------------------------------------------------- invariants

def test_key_shift_invariance():
    q, k, v = _rand(1, 2, 17, 8, seed=14), _rand(1, 2, 17, 8, seed=15), _rand(1, 2, 17, 8, seed=16)
    c = _rand(8, seed=17)
    for causal in (False, True):
        o, lse = oracle.online_fwd(q, k, v, causal=causal, scale=0.5, query_block=4, key_block=5)
        o2, lse2 = oracle.online_fwd(q, k + c, v, causal=causal, scale=0.5, query_block=4, key_block=5)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse2, lse + 0.5 * (q @ c), rtol=1e-12, atol=1e-13)


def test_permutation_invariances():
    q, k, v = _rand(3, 21, 8, seed=18), _rand(3, 21, 8, seed=19), _rand(3, 21, 8, seed=20)
    perm = np.random.default_rng(21).permutation(21)
    o, lse = oracle.online_fwd(q, k, v, query_block=4, key_block=6)
    o_kv, lse_kv = oracle.online_fwd(q, k[:, perm], v[:, perm], query_block=4, key_block=6)
    np.testing.assert_allclose(o_kv, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse_kv, lse, rtol=1e-13)
    o_q, lse_q = oracle.online_fwd(q[:, perm], k, v, query_block=4, key_block=6)
    np.testing.assert_allclose(o_q, o[:, perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse_q, lse[:, perm], rtol=1e-13)


def test_prefix_property():
    """After t tiles, a/l is attention over exactly the keys seen so far.

    'Online softmax makes tiling exact': the partial ratio a/l attends only to
    the processed keys, and alpha is zero before any key is seen.
    """
    q, k, v = _rand(1, 9, 4, seed=22), _rand(1, 9, 4, seed=23), _rand(1, 9, 3, seed=24)
    kb, scale = 2, 0.8
    for causal in (False, True):
        trace = []
        oracle.online_fwd(q, k, v, causal=causal, scale=scale, query_block=9, key_block=kb, trace=trace)
        assert len(trace) == 5
        for t in trace:
            keys = min(9, t["col0"] + kb)
            for i in range(9):
                visible = min(keys, i + 1) if causal else keys
                if visible == 0:
                    # no key seen yet: the initial state is untouched
                    assert t["m"][i] == -np.inf and t["l"][i] == 0 and np.all(t["a"][i] == 0)
                    continue
                r, rl = oracle.dense_fwd(q[0, i:i + 1], k[0, :visible], v[0, :visible], scale=scale)
                np.testing.assert_allclose(t["a"][i] / t["l"][i], r[0], rtol=1e-12, atol=1e-14)
                assert t["m"][i] + math.log(t["l"][i]) == pytest.approx(rl[0], rel=1e-12)


# ---------------------------------------------------------------- library cross-checks

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (64, 16), (130, 32)])
def test_against_torch_sdpa_and_logsumexp(causal, n, d):
    q, k, v = _rand(2, 3, n, d, seed=25), _rand(2, 3, n, d, seed=26), _rand(2, 3, n, d, seed=27)
    scale = 1.0 / math.sqrt(d)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal).numpy()
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    ref_lse = scipy.special.logsumexp(s, axis=-1)
    for o, lse in (oracle.dense_fwd(q, k, v, causal=causal),
                   oracle.online_fwd(q, k, v, causal=causal, query_block=16, key_block=24)):
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_dense_rows_subset_matches_full():
    q, k, v = _rand(2, 50, 8, seed=28), _rand(2, 50, 8, seed=29), _rand(2, 50, 8, seed=30)
    rows = np.array([0, 3, 17, 49])
    for causal in (False, True):
        o, lse = oracle.dense_fwd(q, k, v, causal=causal)
        os_, lses = oracle.dense_fwd(q, k, v, causal=causal, rows=rows)
        np.testing.assert_allclose(os_, o[:, rows], rtol=1e-14)
        np.testing.assert_allclose(lses, lse[:, rows], rtol=1e-14)


def test_negative_and_zero_scale():
    q, k, v = _rand(1, 13, 4, seed=31), _rand(1, 13, 4, seed=32), _rand(1, 13, 4, seed=33)
    for scale in (-0.9, 0.0):
        for causal in (False, True):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=causal, scale=scale).numpy()
            o, _ = oracle.online_fwd(q, k, v, causal=causal, scale=scale, query_block=3, key_block=4)
            np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.dense_fwd(q, k, v, causal=causal, scale=scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    n, d = 5, 3
    q, k, v, do = (_rand(n, d, seed=s) for s in (40, 41, 42, 43))
    scale = 0.7
    dq, dk, dv, _, _ = oracle.dense_bwd(q, k, v, do, causal=causal, scale=scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (_loss(*args_p, do, causal, scale) - _loss(*args_m, do, causal, scale)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_against_torch_autograd(causal):
    q, k, v, do = (_rand(2, 33, 8, seed=s) for s in (44, 45, 46, 47))
    dq, dk, dv, o, lse = oracle.dense_bwd(q, k, v, do, causal=causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("d,dv", [(8, 4), (4, 12)])
def test_backward_dv_differs_from_d_against_torch_autograd(d, dv):
    """Gradients with V (and dO) of width d_v != d against float64 autograd."""
    q, k = _rand(2, 29, d, seed=181), _rand(2, 29, d, seed=182)
    v, do = _rand(2, 29, dv, seed=183), _rand(2, 29, dv, seed=184)
    for causal in (False, True):
        dq, dk, dvg, o, _ = oracle.dense_bwd(q, k, v, do, causal=causal)
        assert dq.shape == q.shape and dk.shape == k.shape and dvg.shape == v.shape
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        to.backward(torch.from_numpy(do))
        np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
        for a, b in ((dq, tq.grad), (dk, tk.grad), (dvg, tv.grad)):
            np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_against_torch_autograd(causal):
    """sampled_bwd (row chunks of 7, so rows and columns cross chunk edges, and
    d_v != d) against float64 autograd on the listed rows and key columns."""
    n = 40
    q, k = _rand(1, n, 8, seed=301)[0], _rand(1, n, 8, seed=302)[0]
    v, do = _rand(1, n, 5, seed=303)[0], _rand(1, n, 5, seed=304)[0]
    rows, cols = [0, 6, 7, 20, 39], [0, 1, 13, 38, 39]
    dq, dk, dv = oracle.sampled_bwd(q, k, v, do, causal=causal, rows=rows, cols=cols, chunk=7)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=causal)
    to.backward(torch.from_numpy(do)[None])
    np.testing.assert_allclose(dq, tq.grad.numpy()[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy()[cols], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy()[cols], rtol=1e-10, atol=1e-12)


def test_backward_invariants():
    q, k, v, do = (_rand(2, 17, 6, seed=s) for s in (48, 49, 50, 51))
    for causal in (False, True):
        dq, dk, dv, _, _ = oracle.dense_bwd(q, k, v, do, causal=causal)
        # shifting every key by the same vector leaves O unchanged -> sum_j dK_j = 0
        np.testing.assert_allclose(dk.sum(-2), 0, atol=1e-12)
        # rows of P sum to one -> sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(-2), do.sum(-2), rtol=1e-12, atol=1e-12)
    veq = np.broadcast_to(_rand(6, seed=52), v.shape).copy()
    dq, dk, _, _, _ = oracle.dense_bwd(q, k, veq, do, causal=True)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)


# ---------------------------------------------------------------- sliding window
# Key j is visible to query i iff i - W < j <= i (causal only).

def _window_mask(n, w):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & (j > i - w)


def test_window_one_attends_to_self():
    """W = 1: every query sees only its own key, so O = V and LSE = scale q_i . k_i."""
    q, k, v = (_rand(2, 19, 5, seed=s) for s in (80, 81, 82))
    o, lse = oracle.dense_fwd(q, k, v, causal=True, scale=0.3, window=1)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.3 * (q * k).sum(-1), rtol=1e-14, atol=1e-14)


def _brute_window_row(q, k, v, scale, w, i):
    """Softmax over the explicit key list of row i, in plain Python."""
    keys = list(range(max(0, i - w + 1), i + 1))
    t = [scale * sum(q[i, c] * k[j, c] for c in range(q.shape[1])) for j in keys]
    mx = max(t)
    e = [math.exp(x - mx) for x in t]
    z = sum(e)
    o = [sum(e[a] * v[keys[a], c] for a in range(len(keys))) / z for c in range(v.shape[1])]
    return o, mx + math.log(z)


@pytest.mark.parametrize("w", [1, 2, 3, 5, 12, 13, 40])
def test_window_brute_force_rows(w):
    n, d = 13, 4
    q, k, v = (_rand(n, d, seed=s, std=2) for s in (83, 84, 85))
    o, lse = oracle.dense_fwd(q, k, v, causal=True, scale=0.6, window=w)
    for i in range(n):
        bo, bl = _brute_window_row(q, k, v, 0.6, w, i)
        np.testing.assert_allclose(o[i], bo, rtol=1e-12, atol=1e-12)
        assert abs(lse[i] - bl) < 1e-12
    if w < n:  # an off-by-one window is caught by the same comparison
        o_bad, _ = oracle.dense_fwd(q, k, v, causal=True, scale=0.6, window=w + 1)
        assert any(not np.allclose(o_bad[i], _brute_window_row(q, k, v, 0.6, w, i)[0], atol=1e-9)
                   for i in range(n))


def test_window_at_least_n_is_causal():
    q, k, v = (_rand(2, 21, 6, seed=s) for s in (86, 87, 88))
    ref = oracle.dense_fwd(q, k, v, causal=True)
    for w in (21, 28):
        got = oracle.dense_fwd(q, k, v, causal=True, window=w)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])


@pytest.mark.parametrize("w", [1, 4, 9, 33])
def test_window_against_torch_mask_and_autograd(w):
    n = 33
    q, k, v, do = (_rand(2, n, 8, seed=s) for s in (89, 90, 91, 92))
    dq, dk, dv, o, lse = oracle.dense_bwd(q, k, v, do, causal=True, scale=0.4, window=w)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    mask = torch.from_numpy(_window_mask(n, w))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.4)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-13)
    s = 0.4 * (q @ np.swapaxes(k, -1, -2))
    np.testing.assert_allclose(lse, scipy.special.logsumexp(np.where(_window_mask(n, w), s, -np.inf), axis=-1),
                               rtol=1e-12, atol=1e-12)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("qb,kb", [(1, 1), (3, 5), (8, 2), (64, 64)])
def test_window_online_matches_dense(qb, kb):
    q, k, v = (_rand(2, 29, 5, seed=s, std=2) for s in (93, 94, 95))
    for w in (1, 3, 7, 29):
        ro, rl = oracle.dense_fwd(q, k, v, causal=True, window=w)
        oo, ol = oracle.online_fwd(q, k, v, causal=True, window=w, query_block=qb, key_block=kb)
        np.testing.assert_allclose(oo, ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ol, rl, rtol=1e-12, atol=1e-13)


def test_window_backward_finite_differences():
    n, d, w, scale = 6, 3, 2, 0.7
    q, k, v, do = (_rand(n, d, seed=s) for s in (96, 97, 98, 99))
    dq, dk, dv, _, _ = oracle.dense_bwd(q, k, v, do, causal=True, scale=scale, window=w)

    def loss(a, b, c):
        o, _ = oracle.dense_fwd(a, b, c, causal=True, scale=scale, window=w)
        return float((o * do).sum())

    h = 1e-6
    for pos, g in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        num = np.zeros_like(base[pos])
        for idx in np.ndindex(num.shape):
            xp = [x.copy() for x in base]
            xm = [x.copy() for x in base]
            xp[pos][idx] += h
            xm[pos][idx] -= h
            num[idx] = (loss(*xp) - loss(*xm)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_window_argument_checks():
    q = _rand(4, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.dense_fwd(q, q, q, causal=False, window=2)
    with pytest.raises(ValueError):
        oracle.dense_fwd(q, q, q, causal=True, window=0)


# ---------------------------------------------------------------- inputs

def test_bf16_rounding_matches_torch_cast():
    x = np.random.default_rng(60).standard_normal(100000).astype(np.float32) * 10
    # exact ties: values halfway between two bf16 numbers
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-40, 3.4e38])])
    ours = workloads.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_needle_inputs_are_near_one_hot():
    """Needle rows attend (almost) only to their target, never the forbidden key."""
    d, n = 16, 160
    x = workloads.needle_inputs(1, 1, n, d, "bf16", seed=3, causal=True)
    o, _ = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=True)
    o_nomask, _ = oracle.dense_fwd(x["q"], x["k"], x["v"], causal=False)
    # run 0 is row 0 alone, target key 0; run 1 covers rows 2..8, target key 2, forbidden key 9
    np.testing.assert_allclose(o[0, 0, 0], x["v"][0, 0, 0], atol=1e-6)
    for i in range(2, 9):
        np.testing.assert_allclose(o[0, 0, i], x["v"][0, 0, 2], atol=1e-6)
        # without the mask the forbidden key would win by a wide margin
        assert np.abs(o_nomask[0, 0, i] - x["v"][0, 0, 9]).max() < 1e-6


def test_workload_flops_and_bytes():
    w = workloads.WORKLOADS["long_causal_bf16"]
    assert w.fwd_flops() == 4 * 128 * (8192 * 8193 // 2) * 16 == 274911461376
    assert w.fwd_bytes() == 134742016


@pytest.mark.parametrize("n,causal", [(1, False), (64, True), (300, False), (300, True), (257, True)])
def test_workload_sparse_pairs_count_the_mask(n, causal):
    """The pair count of a block-sparse launch is the number of visible entries
    of the oracle's own mask, counted by brute force."""
    m = workloads.block_sparse_mask(n, 2, 1, 1, 1, seed=5)
    q = np.ones((1, 2, n, 4))
    probs = oracle.dense_probs(q, q, causal=causal, block_mask=m)
    assert workloads.sparse_pairs(m, n, causal) == int((probs > 0).sum())


@pytest.mark.parametrize("n,win", [(1, 1), (7, 1), (7, 3), (7, 7), (7, 50), (64, 17)])
def test_workload_window_pairs_count_the_mask(n, win):
    """The pair count of a windowed workload is the number of visible entries
    of the oracle's own mask, counted by brute force."""
    w = workloads.Workload("t", "bf16", True, 1, 1, n, 16, seed=0, window=win)
    probs = oracle.dense_probs(np.eye(n, 16), np.eye(n, 16), causal=True, window=win)
    assert w.pairs() == int((probs > 0).sum())
    full = workloads.WORKLOADS["long_window_bf16"]
    assert full.pairs() == 1024 * 1025 // 2 + (8192 - 1024) * 1024


# ---------------------------------------------------------------- planted mistakes

def _mutant_online(q, k, v, causal, scale, qb, kb, bug):
    """A copy of the online recurrence with one deliberate mistake."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    n, dv = q.shape[0], v.shape[1]
    out, lse = np.empty((n, dv)), np.empty(n)
    for r0 in range(0, n, qb):
        rows = np.arange(r0, min(n, r0 + qb))
        m, ell, a = np.full(len(rows), -np.inf), np.zeros(len(rows)), np.zeros((len(rows), dv))
        for c0 in range(0, n, kb):
            cols = np.arange(c0, min(n, c0 + kb))
            t = q[rows] @ k[cols].T
            if bug != "scale_after_max":
                t = t * scale
            if causal:
                vis = cols[None, :] < rows[:, None] if bug == "strict_causal" else cols[None, :] <= rows[:, None]
                t = np.where(vis, t, -np.inf)
            m_new = np.maximum(m, t.max(1))
            ms = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - ms), 0.0)
            p = np.exp(t - ms[:, None])
            if bug == "scale_after_max":
                p = np.exp(scale * (t - ms[:, None]))
                alpha = np.where(np.isfinite(m), np.exp(scale * (m - ms)), 0.0)
            if bug == "no_alpha_on_l":
                ell = ell + p.sum(1)
            else:
                ell = alpha * ell + p.sum(1)
            if bug == "no_alpha_on_a":
                a = a + p @ v[cols]
            elif bug == "transposed_pv":
                a = alpha[:, None] * a + (p @ k[cols] if k.shape == v.shape else p @ v[cols])
            elif bug == "drop_last_tile" and c0 + kb >= n:
                pass
            else:
                a = alpha[:, None] * a + p @ v[cols]
            m = np.where(np.isfinite(m_new), m_new, m)
        out[rows] = a / ell[:, None]
        lse[rows] = m + (np.log2(ell) if bug == "lse_base2" else np.log(ell))
    return out, lse


BUGS = ["no_alpha_on_a", "no_alpha_on_l", "strict_causal", "scale_after_max",
        "transposed_pv", "drop_last_tile", "lse_base2"]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("bug", BUGS)
def test_pins_catch_planted_mistakes(bug):
    """Each mistake fails at least one of the checks used above as pins."""
    q, k, v = _rand(13, 4, seed=70, std=2), _rand(13, 4, seed=71, std=2), _rand(13, 4, seed=72)
    failures = 0
    for causal in (False, True):
        for scale in (0.5, -0.5):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=causal, scale=scale).numpy()
            s = scale * (q @ k.T)
            if causal:
                s = np.where(np.tril(np.ones((13, 13), bool)), s, -np.inf)
            ref_lse = scipy.special.logsumexp(s, axis=-1)
            o, lse = _mutant_online(q, k, v, causal, scale, 4, 3, bug)
            if not (np.allclose(o, ref, rtol=1e-10, atol=1e-12)
                    and np.allclose(lse, ref_lse, rtol=1e-10, atol=1e-12)):
                failures += 1
    assert failures > 0
    # and the unmutated recurrence passes the same checks
    o, lse = _mutant_online(q, k, v, True, 0.5, 4, 3, bug="none")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.5).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
