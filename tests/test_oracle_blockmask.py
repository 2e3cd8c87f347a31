"""Pins for the oracle's block-sparse forward (CPU only).

The block mask of the "FlashAttention" paper story (block-sparse paragraph)
marks which (query block, key block) tiles of the score matrix exist.  The
oracle's block-sparse forward is checked against the dense oracle and scipy,
through identities that fix every part of the visibility rule: a full mask is
the dense forward, an empty mask leaves every row empty, a single block is
the attention of that block's queries over that block's keys, a
block-diagonal mask is independent attention per block, per-head masks act
head by head, and the results of two disjoint masks merge into the result
of their union by the online-softmax merge.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import attn_inputs


def rand_mask(mh, nbq, nbk, density, seed):
    r = np.random.default_rng(seed)
    return (r.random((mh, nbq, nbk)) < density).astype(np.uint8)


def grid(N, bm, bn):
    return -(-N // bm), -(-N // bn)


def expand(mask_h, N, bm, bn, causal):
    """Element visibility of one head's block mask (N x N booleans)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = mask_h[i // bm, j // bn].astype(bool)
    if causal:
        vis &= j <= i
    return vis


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,bm,bn", [(1, 4, 2), (13, 4, 3), (40, 8, 8), (33, 16, 5)])
def test_full_mask_is_the_dense_forward(oracle_mod, causal, N, bm, bn):
    q, k, v = attn_inputs.make(2, 4, 2, N, 8, "fp32", seed=N + bm)
    nbq, nbk = grid(N, bm, bn)
    o, lse = oracle_mod.fwd_blockmask(q, k, v, np.ones((1, nbq, nbk), np.uint8), bm, bn,
                                      causal=causal)
    ro, rl = oracle_mod.fwd(q, k, v, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)


def test_empty_mask_leaves_every_row_empty(oracle_mod):
    q, k, v = attn_inputs.make(1, 2, 2, 20, 8, "fp32", seed=3)
    o, lse = oracle_mod.fwd_blockmask(q, k, v, np.zeros((2, 5, 4), np.uint8), 4, 5)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(4))
def test_matches_scipy_on_the_expanded_mask(oracle_mod, causal, seed):
    """Library reference: scipy softmax over the full score matrix with the
    invisible entries at -inf (rows with nothing visible are empty)."""
    N, bm, bn, d = 23, 4, 3, 5
    q, k, v = attn_inputs.make(1, 3, 3, N, d, "fp32", seed=50 + seed)
    nbq, nbk = grid(N, bm, bn)
    mask = rand_mask(3, nbq, nbk, 0.4, seed)
    scale = 0.37
    o, lse = oracle_mod.fwd_blockmask(q, k, v, mask, bm, bn, causal=causal, scale=scale)
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    for h in range(3):
        vis = expand(mask[h], N, bm, bn, causal)
        s = np.where(vis, scale * qd[0, h] @ kd[0, h].T, -np.inf)
        live = vis.any(axis=1)
        assert np.all(o[0, h][~live] == 0.0) and np.all(np.isneginf(lse[0, h][~live]))
        ref_o = softmax(s[live], axis=1) @ vd[0, h]
        np.testing.assert_allclose(o[0, h][live], ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h][live], logsumexp(s[live], axis=1), rtol=0,
                                   atol=1e-12)


def test_single_block_is_attention_of_that_block(oracle_mod):
    N, bm, bn = 30, 8, 4
    q, k, v = attn_inputs.make(1, 2, 1, N, 6, "fp32", seed=9)
    nbq, nbk = grid(N, bm, bn)
    mask = np.zeros((1, nbq, nbk), np.uint8)
    bi, bj = 2, 5
    mask[0, bi, bj] = 1
    o, lse = oracle_mod.fwd_blockmask(q, k, v, mask, bm, bn)
    rows = slice(bi * bm, min(N, (bi + 1) * bm))
    keys = slice(bj * bn, min(N, (bj + 1) * bn))
    ro, rl = oracle_mod.fwd(q[:, :, rows].contiguous(), k[:, :, keys].contiguous(),
                            v[:, :, keys].contiguous())
    np.testing.assert_allclose(o[:, :, rows], ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, rows], rl, rtol=0, atol=1e-13)
    others = np.ones(N, bool)
    others[rows] = False
    assert np.all(o[:, :, others] == 0.0) and np.all(np.isneginf(lse[:, :, others]))


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_independent_blocks(oracle_mod, causal):
    N, b = 26, 8
    q, k, v = attn_inputs.make(2, 2, 2, N, 4, "fp32", seed=21)
    nb = -(-N // b)
    mask = np.eye(nb, dtype=np.uint8)[None]
    o, lse = oracle_mod.fwd_blockmask(q, k, v, mask, b, b, causal=causal)
    for t in range(nb):
        sl = slice(t * b, min(N, (t + 1) * b))
        ro, rl = oracle_mod.fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                v[:, :, sl].contiguous(), causal=causal)
        np.testing.assert_allclose(o[:, :, sl], ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, sl], rl, rtol=0, atol=1e-13)


def test_per_head_masks_act_head_by_head(oracle_mod):
    N, bm, bn, Hq = 19, 4, 4, 4
    q, k, v = attn_inputs.make(1, Hq, 2, N, 4, "fp32", seed=31)
    nbq, nbk = grid(N, bm, bn)
    mask = rand_mask(Hq, nbq, nbk, 0.5, 7)
    o, lse = oracle_mod.fwd_blockmask(q, k, v, mask, bm, bn, causal=True)
    for h in range(Hq):
        g = h // (Hq // 2)
        ro, rl = oracle_mod.fwd_blockmask(q[:, h:h + 1].contiguous(), k[:, g:g + 1].contiguous(),
                                          v[:, g:g + 1].contiguous(), mask[h:h + 1], bm, bn,
                                          causal=True)
        np.testing.assert_array_equal(o[:, h:h + 1], ro)
        np.testing.assert_array_equal(lse[:, h:h + 1], rl)
    assert not np.array_equal(mask[0], mask[1])


def test_disjoint_masks_merge_into_their_union(oracle_mod):
    """Online-softmax merge: LSE = logaddexp(LSE1, LSE2) and
    O = e^(LSE1-LSE) O1 + e^(LSE2-LSE) O2 for a mask split into two parts."""
    N, bm, bn = 37, 8, 4
    q, k, v = attn_inputs.make(1, 2, 2, N, 6, "fp32", seed=41)
    nbq, nbk = grid(N, bm, bn)
    union = rand_mask(1, nbq, nbk, 0.7, 3)
    part = rand_mask(1, nbq, nbk, 0.5, 4) & union
    rest = union - part
    o, lse = oracle_mod.fwd_blockmask(q, k, v, union, bm, bn, causal=True)
    o1, l1 = oracle_mod.fwd_blockmask(q, k, v, part, bm, bn, causal=True)
    o2, l2 = oracle_mod.fwd_blockmask(q, k, v, rest, bm, bn, causal=True)
    merged = np.logaddexp(l1, l2)
    live = np.isfinite(merged)
    np.testing.assert_array_equal(np.isneginf(lse), ~live)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - np.where(live, merged, 0.0)))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - np.where(live, merged, 0.0)))
    ref = w1[..., None] * o1 + w2[..., None] * o2
    np.testing.assert_allclose(lse[live], merged[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[live], ref[live], rtol=0, atol=1e-12)


def test_gqa_equals_repeated_kv(oracle_mod):
    N, bm, bn = 21, 4, 8
    q, k, v = attn_inputs.make(1, 4, 2, N, 4, "fp32", seed=51)
    nbq, nbk = grid(N, bm, bn)
    mask = rand_mask(1, nbq, nbk, 0.6, 5)
    o, lse = oracle_mod.fwd_blockmask(q, k, v, mask, bm, bn, causal=True)
    kr, vr = k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1)
    ro, rl = oracle_mod.fwd_blockmask(q, kr, vr, mask, bm, bn, causal=True)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(lse, rl)


def test_rejects_bad_mask_shapes(oracle_mod):
    q, k, v = attn_inputs.make(1, 2, 2, 10, 4, "fp32", seed=1)
    with pytest.raises(ValueError):
        oracle_mod.fwd_blockmask(q, k, v, np.ones((3, 3, 5), np.uint8), 4, 2)
    with pytest.raises(ValueError):
        oracle_mod.fwd_blockmask(q, k, v, np.ones((1, 2, 5), np.uint8), 4, 2)
