"""Pins for the fp64 oracle's forward pass (CPU only).

The oracle is checked against things other than itself: the worked example
and check printed on the FlashAttention page (wineandchord.com, "CPU
reference"), library softmax/logsumexp routines, closed forms and invariants
of softmax attention.  Each pin is chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a
mis-masked key) fails at least one test.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def rng(seed):
    return np.random.default_rng(seed)


def rand(shape, seed, scale=1.0):
    return rng(seed).standard_normal(shape) * scale


def scipy_attention(q, k, v, scale, causal=False):
    """Library reference for one head: softmax rows from scipy, then a matmul."""
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    return softmax(s, axis=1) @ v, logsumexp(s, axis=1)


# ---------------------------------------------------------------- worked example
def test_worked_example_page_check(oracle_mod):
    """The page's own check: K/V-blockwise pass equals dense to 1e-12, all finite."""
    g = json.load(open(GOLDEN))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    assert q.shape[-1] == 3 and v.shape[-1] == 2  # d_v differs from d_k
    dense, lse_d = oracle_mod.fwd(q, k, v)  # default scale 1/sqrt(d_k)
    nq = q.shape[2]
    blk, lse_b = oracle_mod.fwd_blockwise(q, k, v, br=nq, bc=g["block_size"])
    assert np.all(np.isfinite(blk)) and np.all(np.isfinite(dense))
    assert np.max(np.abs(blk - dense)) < g["max_abs_error"]
    assert np.max(np.abs(lse_b - lse_d)) < g["max_abs_error"]


def test_worked_example_vs_library_softmax(oracle_mod):
    g = json.load(open(GOLDEN))
    q, k, v = (np.array(g[x]) for x in "qkv")
    o, lse = oracle_mod.fwd(q[None, None], k[None, None], v[None, None])
    ref_o, ref_lse = scipy_attention(q, k, v, 1 / np.sqrt(3))
    np.testing.assert_allclose(o[0, 0], ref_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_its_value(oracle_mod):
    q = rand((2, 3, 4, 8), 1)
    k = rand((2, 3, 1, 8), 2)
    v = rand((2, 3, 1, 5), 3)
    o, lse = oracle_mod.fwd(q, k, v, scale=0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]),
                               rtol=1e-14, atol=1e-14)


def test_two_keys_is_a_sigmoid_mix(oracle_mod):
    """With two keys softmax is the logistic function of the score gap."""
    q = rand((1, 1, 6, 4), 4)
    k = rand((1, 1, 2, 4), 5)
    v = rand((1, 1, 2, 3), 6)
    scale = 0.9
    o, lse = oracle_mod.fwd(q, k, v, scale=scale)
    s0 = scale * q[0, 0] @ k[0, 0, 0]
    s1 = scale * q[0, 0] @ k[0, 0, 1]
    w0 = expit(s0 - s1)
    ref = w0[:, None] * v[0, 0, 0] + (1 - w0)[:, None] * v[0, 0, 1]
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(s0, s1), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_weights_closed_form(oracle_mod, causal, how):
    n = 9
    q = rand((1, 2, n, 4), 7)
    if how == "zero_q":
        q[:] = 0.0
        scale = None
    else:
        scale = 0.0
    k = rand((1, 2, n, 4), 8)
    v = rand((1, 2, n, 3), 9)
    o, lse = oracle_mod.fwd(q, k, v, causal=causal, scale=scale)
    if causal:
        counts = np.arange(1, n + 1)
        ref = np.cumsum(v, axis=2) / counts[None, None, :, None]
        ref_lse = np.broadcast_to(np.log(counts), lse.shape)
    else:
        ref = np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape)
        ref_lse = np.full(lse.shape, np.log(n))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values(oracle_mod):
    n = 11
    q = rand((1, 1, 5, 6), 10, scale=3.0)
    k = np.broadcast_to(rand((1, 1, 1, 6), 11), (1, 1, n, 6)).copy()
    v = rand((1, 1, n, 4), 12)
    o, _ = oracle_mod.fwd(q, k, v)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (5, 4)),
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_expose_probabilities(oracle_mod, causal):
    """V = I makes O equal to the probability matrix P itself."""
    n = 7
    q = rand((1, 1, n, 5), 13, scale=2.0)
    k = rand((1, 1, n, 5), 14)
    v = np.eye(n)[None, None]
    p, lse = oracle_mod.fwd(q, k, v, causal=causal, scale=0.6)
    p = p[0, 0]
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)
    ref_p, ref_lse = scipy_attention(q[0, 0], k[0, 0], np.eye(n), 0.6, causal)
    np.testing.assert_allclose(p, ref_p, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- invariants
def test_joint_permutation_of_keys_and_values(oracle_mod):
    q = rand((2, 2, 6, 8), 15)
    k = rand((2, 2, 10, 8), 16)
    v = rand((2, 2, 10, 8), 17)
    perm = rng(18).permutation(10)
    o1, l1 = oracle_mod.fwd(q, k, v)
    o2, l2 = oracle_mod.fwd(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_only_lse(oracle_mod, causal):
    q = rand((1, 2, 8, 4), 19)
    k = rand((1, 2, 8, 4), 20)
    v = rand((1, 2, 8, 3), 21)
    c = rand((4,), 22)
    scale = 0.8
    o1, l1 = oracle_mod.fwd(q, k, v, causal=causal, scale=scale)
    o2, l2 = oracle_mod.fwd(q, k + c, v, causal=causal, scale=scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, scale * (q @ c), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_value_affine_map(oracle_mod, causal):
    q = rand((1, 1, 8, 4), 23)
    k = rand((1, 1, 8, 4), 24)
    v = rand((1, 1, 8, 3), 25)
    a, b = -1.7, rand((3,), 26)
    o1, _ = oracle_mod.fwd(q, k, v, causal=causal)
    o2, _ = oracle_mod.fwd(q, k, a * v + b, causal=causal)
    np.testing.assert_allclose(o2, a * o1 + b, rtol=0, atol=1e-13)


def test_causal_row_ignores_later_keys(oracle_mod):
    n = 10
    q = rand((1, 1, n, 4), 27)
    k = rand((1, 1, n, 4), 28)
    v = rand((1, 1, n, 4), 29)
    o1, l1 = oracle_mod.fwd(q, k, v, causal=True)
    for i in range(n - 1):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] = rand((1, 1, n - i - 1, 4), 100 + i, scale=5.0)
        v2[:, :, i + 1:] = rand((1, 1, n - i - 1, 4), 200 + i, scale=5.0)
        o2, l2 = oracle_mod.fwd(q, k2, v2, causal=True)
        np.testing.assert_array_equal(o1[0, 0, : i + 1], o2[0, 0, : i + 1])
        np.testing.assert_array_equal(l1[0, 0, : i + 1], l2[0, 0, : i + 1])
        assert not np.allclose(o1[0, 0, i + 1:], o2[0, 0, i + 1:])


def test_causal_first_row_and_full_last_row(oracle_mod):
    n = 6
    q = rand((1, 1, n, 4), 30)
    k = rand((1, 1, n, 4), 31)
    v = rand((1, 1, n, 4), 32)
    oc, lc = oracle_mod.fwd(q, k, v, causal=True)
    on, ln = oracle_mod.fwd(q, k, v, causal=False)
    np.testing.assert_allclose(oc[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oc[0, 0, -1], on[0, 0, -1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lc[0, 0, -1], ln[0, 0, -1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_with_repeated_kv(oracle_mod, causal):
    B, Hq, Hkv, n, d = 2, 8, 2, 9, 4
    q = rand((B, Hq, n, d), 33)
    k = rand((B, Hkv, n, d), 34)
    v = rand((B, Hkv, n, d), 35)
    o1, l1 = oracle_mod.fwd(q, k, v, causal=causal)
    rep = Hq // Hkv
    o2, l2 = oracle_mod.fwd(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1),
                            causal=causal)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # and head h really reads kv head h // rep: compare with one head by hand
    h = 5
    ref_o, ref_l = scipy_attention(q[1, h], k[1, h // rep], v[1, h // rep], 0.5, causal)
    o3, l3 = oracle_mod.fwd(q, k, v, causal=causal, scale=0.5)
    np.testing.assert_allclose(o3[1, h], ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3[1, h], ref_l, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_batches_and_heads_are_independent(oracle_mod, causal):
    q = rand((3, 2, 5, 4), 36)
    k = rand((3, 2, 5, 4), 37)
    v = rand((3, 2, 5, 2), 38)
    o, lse = oracle_mod.fwd(q, k, v, causal=causal, scale=1.3)
    for b in range(3):
        for h in range(2):
            ref_o, ref_l = scipy_attention(q[b, h], k[b, h], v[b, h], 1.3, causal)
            np.testing.assert_allclose(o[b, h], ref_o, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], ref_l, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mult", [8.0, 100.0])
def test_extreme_logits_stay_finite(oracle_mod, mult):
    q = rand((1, 2, 16, 32), 39, scale=mult)
    k = rand((1, 2, 16, 32), 40)
    v = rand((1, 2, 16, 32), 41)
    for causal in (False, True):
        o, lse = oracle_mod.fwd(q, k, v, causal=causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        for h in range(2):
            ref_o, ref_l = scipy_attention(q[0, h], k[0, h], v[0, h], 1 / np.sqrt(32), causal)
            np.testing.assert_allclose(o[0, h], ref_o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, h], ref_l, rtol=1e-14, atol=1e-12)


# ---------------------------------------------------------------- blockwise form
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(13, 13), (7, 13), (13, 7), (1, 5), (16, 16)])
@pytest.mark.parametrize("br,bc", [(1, 1), (2, 3), (3, 2), (4, 4), (5, 64), (64, 5), (99, 99)])
def test_blockwise_equals_dense(oracle_mod, causal, nq, nk, br, bc):
    q = rand((2, 4, nq, 6), 42, scale=2.0)
    k = rand((2, 2, nk, 6), 43)
    v = rand((2, 2, nk, 5), 44)
    o1, l1 = oracle_mod.fwd(q, k, v, causal=causal)
    o2, l2 = oracle_mod.fwd_blockwise(q, k, v, causal=causal, br=br, bc=bc)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- edges
def test_no_keys_gives_zero_output_and_minus_inf_lse(oracle_mod):
    q = rand((1, 1, 3, 4), 45)
    k = np.zeros((1, 1, 0, 4))
    v = np.zeros((1, 1, 0, 2))
    for fn in (oracle_mod.fwd, lambda *a: oracle_mod.fwd_blockwise(*a, br=2, bc=2)):
        o, lse = fn(q, k, v)
        assert o.shape == (1, 1, 3, 2)
        assert np.all(o == 0) and np.all(lse == -np.inf)


def test_empty_batch_and_rows(oracle_mod):
    o, lse = oracle_mod.fwd(np.zeros((0, 2, 4, 8)), np.zeros((0, 1, 4, 8)),
                            np.zeros((0, 1, 4, 8)))
    assert o.shape == (0, 2, 4, 8) and lse.shape == (0, 2, 4)
    o, lse = oracle_mod.fwd(np.zeros((1, 2, 0, 8)), np.zeros((1, 1, 4, 8)),
                            np.zeros((1, 1, 4, 8)))
    assert o.shape == (1, 2, 0, 8)


def test_bad_head_ratio_is_rejected(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.fwd(np.zeros((1, 3, 4, 8)), np.zeros((1, 2, 4, 8)), np.zeros((1, 2, 4, 8)))


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rows_equals_fwd(oracle_mod, causal):
    q = rand((2, 4, 9, 8), 46)
    k = rand((2, 2, 9, 8), 47)
    v = rand((2, 2, 9, 8), 48)
    o, lse = oracle_mod.fwd(q, k, v, causal=causal)
    rows = np.array([0, 5, 17, 35, 36, 71])
    o_r, l_r = oracle_mod.fwd_rows(q, k, v, rows, causal=causal)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(l_r, lse.reshape(-1)[rows])
    with pytest.raises(ValueError):
        oracle_mod.fwd_rows(q, k, v, np.array([72]), causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_survives_extreme_logits(oracle_mod, causal):
    """The merge must shift by the larger max: score gaps of thousands overflow
    exp() in fp64 otherwise."""
    q = rand((1, 2, 12, 16), 49, scale=1000.0)
    k = rand((1, 2, 12, 16), 50)
    v = rand((1, 2, 12, 16), 51)
    o1, l1 = oracle_mod.fwd(q, k, v, causal=causal)
    o2, l2 = oracle_mod.fwd_blockwise(q, k, v, causal=causal, br=4, bc=3)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-15, atol=1e-9)


# ---------------------------------------------------------------- bottom-right causal
@pytest.mark.parametrize("nq,nk", [(1, 9), (3, 9), (9, 9), (12, 5)])
def test_bottom_right_is_top_left_on_the_suffix(oracle_mod, nq, nk):
    """Query i of Nq sees keys j <= i + Nk - Nq: the same rows as the last Nq
    rows of the (pinned) top-left causal problem with Nk queries."""
    q = rand((2, 4, nq, 6), 60)
    k = rand((2, 2, nk, 6), 61)
    v = rand((2, 2, nk, 5), 62)
    o, lse = oracle_mod.fwd_bottom_right(q, k, v, causal=True)
    if nq <= nk:
        qfull = np.concatenate([rand((2, 4, nk - nq, 6), 63), q], axis=2)
        of, lf = oracle_mod.fwd(qfull, k, v, causal=True)
        np.testing.assert_array_equal(o, of[:, :, nk - nq:])
        np.testing.assert_array_equal(lse, lf[:, :, nk - nq:])
    else:  # the first Nq - Nk queries see nothing; the rest see keys 0..i-(Nq-Nk)
        assert np.all(o[:, :, : nq - nk] == 0) and np.all(lse[:, :, : nq - nk] == -np.inf)
        of, lf = oracle_mod.fwd(q[:, :, nq - nk:], k, v, causal=True)
        np.testing.assert_array_equal(o[:, :, nq - nk:], of)
        np.testing.assert_array_equal(lse[:, :, nq - nk:], lf)


def test_bottom_right_single_query_sees_every_key(oracle_mod):
    q = rand((1, 2, 1, 8), 64)
    k = rand((1, 2, 33, 8), 65)
    v = rand((1, 2, 33, 8), 66)
    o1, l1 = oracle_mod.fwd_bottom_right(q, k, v, causal=True)
    o2, l2 = oracle_mod.fwd(q, k, v, causal=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    for h in range(2):
        ref_o, ref_l = scipy_attention(q[0, h], k[0, h], v[0, h], 1 / np.sqrt(8))
        np.testing.assert_allclose(o1[0, h], ref_o, rtol=0, atol=1e-13)


def test_bottom_right_non_causal_equals_dense(oracle_mod):
    q = rand((1, 2, 4, 8), 67)
    k = rand((1, 1, 20, 8), 68)
    v = rand((1, 1, 20, 8), 69)
    o1, l1 = oracle_mod.fwd_bottom_right(q, k, v, causal=False)
    o2, l2 = oracle_mod.fwd(q, k, v, causal=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
