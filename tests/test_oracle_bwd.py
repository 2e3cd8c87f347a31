"""Pins for the fp64 oracle's backward pass (CPU only).

The pages keep only the softmax statistics and recompute P for the gradients
but drop the gradient formulas, so the oracle writes the textbook gradient.
It is pinned here by central finite differences of the oracle's own forward
(itself pinned in test_oracle_fwd.py), by torch's fp64 autograd through a
library softmax, and by identities every correct gradient satisfies.
"""
import numpy as np
import pytest
import torch


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(oracle_mod, q, k, v, dout, causal, scale):
    o, _ = oracle_mod.fwd(q, k, v, causal=causal, scale=scale)
    return float(np.sum(o * dout))


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, dk, dv
    (1, 1, 1, 4, 4, 3, 2),
    (1, 2, 1, 5, 5, 3, 3),
    (2, 2, 2, 3, 6, 2, 4),
    (1, 4, 2, 6, 4, 3, 2),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_gradients_match_central_differences(oracle_mod, causal, shape):
    B, Hq, Hkv, Nq, Nk, dk, dv = shape
    q = rand((B, Hq, Nq, dk), 1)
    k = rand((B, Hkv, Nk, dk), 2)
    v = rand((B, Hkv, Nk, dv), 3)
    dout = rand((B, Hq, Nq, dv), 4)
    scale = 0.7
    dq, dk_, dv_ = oracle_mod.bwd(q, k, v, dout, causal=causal, scale=scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk_), (v, dv_)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(oracle_mod, q, k, v, dout, causal, scale)
            x[idx] = old - h
            lm = loss(oracle_mod, q, k, v, dout, causal, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def torch_reference(q, k, v, dout, causal, scale, Hq, Hkv):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    rep = Hq // Hkv
    kk = tk.repeat_interleave(rep, dim=1)
    vv = tv.repeat_interleave(rep, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if causal:
        nq, nk = s.shape[-2:]
        mask = torch.ones(nq, nk, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    lse = torch.logsumexp(s, dim=-1)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 17, 17, 8, 8), (1, 3, 1, 9, 12, 5, 7),
                                   (1, 2, 2, 33, 33, 16, 16)])
def test_gradients_match_torch_autograd(oracle_mod, causal, shape):
    B, Hq, Hkv, Nq, Nk, dk, dv = shape
    q = rand((B, Hq, Nq, dk), 5, scale=1.5)
    k = rand((B, Hkv, Nk, dk), 6)
    v = rand((B, Hkv, Nk, dv), 7)
    dout = rand((B, Hq, Nq, dv), 8)
    scale = 1 / np.sqrt(dk)
    dq, dk_, dv_, lse, o, dsum = oracle_mod.bwd(q, k, v, dout, causal=causal, scale=scale,
                                                 with_stats=True)
    ro, rl, rdq, rdk, rdv = torch_reference(q, k, v, dout, causal, scale, Hq, Hkv)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dsum, np.sum(dout * ro, axis=-1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, rdq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_, rdk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_, rdv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(oracle_mod, causal):
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 per kv group."""
    B, Hq, Hkv, N, d = 2, 4, 2, 11, 6
    q = rand((B, Hq, N, d), 9)
    k = rand((B, Hkv, N, d), 10)
    v = rand((B, Hkv, N, d), 11)
    dout = rand((B, Hq, N, d), 12)
    _, dk_, dv_ = oracle_mod.bwd(q, k, v, dout, causal=causal)
    rep = Hq // Hkv
    dsum_groups = dout.reshape(B, Hkv, rep, N, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv_.sum(axis=2), dsum_groups, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_.sum(axis=2), 0.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_kill_query_and_key_gradients(oracle_mod, causal):
    B, H, N, d = 1, 2, 8, 4
    q = rand((B, H, N, d), 13)
    k = rand((B, H, N, d), 14)
    v = np.broadcast_to(rand((B, H, 1, d), 15), (B, H, N, d)).copy()
    dout = rand((B, H, N, d), 16)
    dq, dk_, dv_ = oracle_mod.bwd(q, k, v, dout, causal=causal)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk_, 0.0, rtol=0, atol=1e-13)
    assert np.abs(dv_).max() > 0.1


@pytest.mark.parametrize("causal", [False, True])
def test_first_key_only_row_has_zero_query_gradient(oracle_mod, causal):
    """Causal row 0 sees one key: its softmax is constant, so dQ_0 = 0."""
    B, H, N, d = 1, 1, 6, 4
    q = rand((B, H, N, d), 17)
    k = rand((B, H, N, d), 18)
    v = rand((B, H, N, d), 19)
    dout = rand((B, H, N, d), 20)
    dq, _, _ = oracle_mod.bwd(q, k, v, dout, causal=causal)
    if causal:
        np.testing.assert_allclose(dq[0, 0, 0], 0.0, rtol=0, atol=1e-14)
    else:
        assert np.abs(dq[0, 0, 0]).max() > 1e-3


def test_slices_equal_full_backward(oracle_mod):
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 5
    q = rand((B, Hq, N, d), 21)
    k = rand((B, Hkv, N, d), 22)
    v = rand((B, Hkv, N, d), 23)
    dout = rand((B, Hq, N, d), 24)
    for causal in (False, True):
        dq, dk_, dv_ = oracle_mod.bwd(q, k, v, dout, causal=causal)
        sl = np.array([3, 0])
        sdq, sdk, sdv = oracle_mod.bwd_slices(q, k, v, dout, sl, causal=causal)
        for t, s in enumerate(sl):
            b, g = divmod(int(s), Hkv)
            np.testing.assert_array_equal(sdq[t], dq[b, g * 2:(g + 1) * 2])
            np.testing.assert_array_equal(sdk[t], dk_[b, g])
            np.testing.assert_array_equal(sdv[t], dv_[b, g])
