"""Head dimension 256 (forward entry points only), against the fp64 oracle.

Tolerances are the 16-bit forward's: |O - O_ref| <= 2e-2 + 1e-2 |O_ref|,
|LSE - LSE_ref| <= 1e-3.  Covers the dense forward (tails, causal, GQA,
extreme logits, bf16 and fp16), split-K/V, block-sparse and packed
variable-length at d = 256; the backward rejects d = 256.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 256


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device(DEV)


def check(o, lse, ro, rl, what=""):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with no key differ"
    assert np.all(o[empty] == 0.0)
    o, ro, lse, rl = o[~empty], ro[~empty], lse[~empty], rl[~empty]
    err = np.abs(o - ro)
    bad = err > 2e-2 + 1e-2 * np.abs(ro)
    assert not bad.any(), f"{what} O: {bad.sum()} out of tolerance, max err {err.max()}"
    assert np.abs(lse - rl).max() <= 1e-3, f"{what} LSE max err {np.abs(lse - rl).max()}"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("N", [1, 63, 130, 257, 600])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_forward(oracle_mod, N, causal, dtype):
    dev = gpu()
    q, k, v = attn_inputs.make(2, 4, 2, N, D, dtype, seed=500 + N)
    o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd(q, k, v, causal=causal)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"N={N} {dtype}")


@pytest.mark.parametrize("mult", [8.0, 64.0])
def test_forward_extreme_logits_and_scales(oracle_mod, mult):
    dev = gpu()
    q, k, v = attn_inputs.make(1, 8, 2, 400, D, "bf16", seed=7, q_mult=mult)
    for scale in (None, -0.03):
        o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=scale)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.fwd(q, k, v, causal=True, scale=scale)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"x{mult} scale={scale}")


def test_splitkv(oracle_mod):
    dev = gpu()
    q, k, v = attn_inputs.make_cache(2, 8, 2, 3, 2000, D, seed=5)
    for causal in (False, True):
        o, lse = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=causal, num_splits=4)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"split causal={causal}")


def test_blocksparse(oracle_mod):
    dev = gpu()
    N = 500
    q, k, v = attn_inputs.make(1, 4, 2, N, D, "bf16", seed=9)
    r = np.random.default_rng(6)
    mask = (r.random((1, -(-N // 128), -(-N // 64))) < 0.5).astype(np.uint8)
    for causal in (False, True):
        o, lse = ea.fwd_blocksparse(q.to(dev), k.to(dev), v.to(dev),
                                    torch.from_numpy(mask).to(dev), causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, 128, 64, causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"sparse causal={causal}")


def test_varlen(oracle_mod):
    dev = gpu()
    q, k, v, cu = attn_inputs.make_varlen(4, 2, [200, 1, 129, 64], D, seed=3)
    for causal in (False, True):
        o, lse = ea.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), 200, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"varlen causal={causal}")


def test_backward_rejects_d256():
    dev = gpu()
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(1, 2, 2, 64, D, "bf16", with_dout=True))
    o, lse = ea.fwd(q, k, v)
    with pytest.raises((ea.AttnError, ValueError)):
        ea.bwd(q, k, v, o, lse, do)
