"""Pins for the oracle's packed variable-length forward (CPU only).

Sequences of different lengths are packed end to end along the token axis
and addressed by offsets cu_seqlens; every token attends only within its own
sequence (a document mask), causally if asked.  The oracle is checked against
scipy on the full packed score matrix with that mask, against the dense
oracle for a single sequence, and through invariants: reordering the
sequences reorders the outputs, empty sequences change nothing, and grouped
heads equal repeated K/V.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax


def draw(Hq, Hkv, T, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(Hq, T, d, generator=g, dtype=torch.float64)
    k = torch.randn(Hkv, T, d, generator=g, dtype=torch.float64)
    v = torch.randn(Hkv, T, d, generator=g, dtype=torch.float64)
    return q, k, v


def offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("causal", [False, True])
def test_single_sequence_is_the_dense_forward(oracle_mod, causal):
    q, k, v = draw(4, 2, 37, 8, 1)
    o, lse = oracle_mod.fwd_varlen(q, k, v, [0, 37], causal=causal)
    ro, rl = oracle_mod.fwd(q[None], k[None], v[None], causal=causal)
    np.testing.assert_array_equal(o, ro[0])
    np.testing.assert_array_equal(lse, rl[0])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", [[5, 1, 9], [1, 1, 1, 1], [12, 0, 7, 3], [20]])
def test_matches_scipy_with_a_document_mask(oracle_mod, causal, lengths):
    cu = offsets(lengths)
    T = int(cu[-1])
    q, k, v = draw(2, 2, T, 5, sum(lengths))
    scale = 0.41
    o, lse = oracle_mod.fwd_varlen(q, k, v, cu, causal=causal, scale=scale)
    doc = np.repeat(np.arange(len(lengths)), lengths)
    vis = doc[:, None] == doc[None, :]
    if causal:
        vis &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    for h in range(2):
        s = np.where(vis, scale * q[h].numpy() @ k[h].numpy().T, -np.inf)
        np.testing.assert_allclose(o[h], softmax(s, axis=1) @ v[h].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_reordering_sequences_reorders_outputs(oracle_mod):
    lengths = [4, 9, 2, 6]
    cu = offsets(lengths)
    q, k, v = draw(2, 1, int(cu[-1]), 6, 7)
    o, lse = oracle_mod.fwd_varlen(q, k, v, cu, causal=True)
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    cu2 = offsets([lengths[s] for s in order])
    o2, lse2 = oracle_mod.fwd_varlen(q[:, idx], k[:, idx], v[:, idx], cu2, causal=True)
    np.testing.assert_array_equal(o2, o[:, idx])
    np.testing.assert_array_equal(lse2, lse[:, idx])


def test_empty_sequences_change_nothing(oracle_mod):
    q, k, v = draw(2, 2, 15, 4, 9)
    o, lse = oracle_mod.fwd_varlen(q, k, v, [0, 6, 15], causal=True)
    o2, lse2 = oracle_mod.fwd_varlen(q, k, v, [0, 0, 6, 6, 6, 15, 15], causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_gqa_equals_repeated_kv(oracle_mod):
    q, k, v = draw(4, 2, 18, 4, 11)
    cu = [0, 7, 18]
    o, lse = oracle_mod.fwd_varlen(q, k, v, cu, causal=True)
    o2, lse2 = oracle_mod.fwd_varlen(q, k.repeat_interleave(2, 0), v.repeat_interleave(2, 0), cu,
                                     causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_rejects_inconsistent_offsets(oracle_mod):
    q, k, v = draw(1, 1, 10, 4, 1)
    for cu in ([0, 5, 9], [1, 10], [0, 6, 4, 10], [0]):
        with pytest.raises(ValueError):
            oracle_mod.fwd_varlen(q, k, v, cu)
