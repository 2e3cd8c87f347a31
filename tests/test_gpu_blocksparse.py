"""Block-sparse forward parity: attn_fwd_blocksparse (through the C ABI)
against the oracle's block-mask forward with 128-query x 64-key blocks.

Tolerances are the bf16 forward's: |O - O_ref| <= 2e-2 + 1e-2 |O_ref|
element-wise and |LSE - LSE_ref| <= 1e-3; a row that sees no key must be
exactly O = 0, LSE = -inf.  A full mask must reproduce attn_fwd bit for bit
(same tiles, same order, same arithmetic), an empty mask must leave every row
empty.  The full-size case is checked on whole heads that the oracle
computes from the same inputs.  Strided tensors: token-major q, k, v and
output, and the dense strides bit for bit against the dense entry point.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BQ, BK = ea.SPARSE_BLOCK_Q, ea.SPARSE_BLOCK_K


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device(DEV)


def rand_mask(mh, N, density, seed):
    r = np.random.default_rng(seed)
    nbq, nbk = -(-N // BQ), -(-N // BK)
    return (r.random((mh, nbq, nbk)) < density).astype(np.uint8)


def run(q, k, v, mask, causal, scale=None):
    dev = gpu()
    o, lse = ea.fwd_blocksparse(q.to(dev), k.to(dev), v.to(dev),
                                torch.from_numpy(mask).to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, ro, rl, what=""):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with no key differ"
    assert np.all(o[empty] == 0.0), f"{what}: a row with no key has O != 0"
    live = ~empty
    o, ro, lse, rl = o[live], ro[live], lse[live], rl[live]
    if o.size == 0:
        return
    err = np.abs(o - ro)
    bad = err > 2e-2 + 1e-2 * np.abs(ro)
    assert not bad.any(), f"{what} O: {bad.sum()} elements out of tolerance, max err {err.max()}"
    lerr = np.abs(lse - rl)
    assert lerr.max() <= 1e-3, f"{what} LSE max err {lerr.max()}"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("N", [1, 63, 128, 200, 513, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.15, 0.5])
def test_random_masks(oracle_mod, N, d, causal, density):
    q, k, v = attn_inputs.make(2, 4, 2, N, d, "bf16", seed=N + d)
    mask = rand_mask(1, N, density, seed=N * 3 + d + int(causal))
    o, lse = run(q, k, v, mask, causal)
    ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, BQ, BK, causal=causal)
    check(o, lse, ro, rl, f"N={N} d={d} causal={causal} density={density}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_per_head_masks_and_gqa(oracle_mod, d, causal):
    q, k, v = attn_inputs.make(2, 8, 2, 700, d, "bf16", seed=17)
    mask = rand_mask(8, 700, 0.4, seed=5)
    o, lse = run(q, k, v, mask, causal)
    ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, BQ, BK, causal=causal)
    check(o, lse, ro, rl, f"per-head d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_full_mask_is_the_dense_forward_bitwise(d, causal):
    dev = gpu()
    q, k, v = (t.to(dev) for t in attn_inputs.make(2, 4, 2, 777, d, "bf16", seed=23))
    mask = torch.ones((1, -(-777 // BQ), -(-777 // BK)), dtype=torch.uint8, device=dev)
    o, lse = ea.fwd_blocksparse(q, k, v, mask, causal=causal)
    fo, fl = ea.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, fo) and torch.equal(lse, fl)


@pytest.mark.parametrize("d", [64, 128])
def test_empty_mask_leaves_rows_empty(d):
    dev = gpu()
    q, k, v = (t.to(dev) for t in attn_inputs.make(1, 2, 2, 300, d, "bf16", seed=29))
    mask = torch.zeros((2, 3, 5), dtype=torch.uint8, device=dev)
    o = torch.full_like(q, 3.0)
    lse = torch.zeros(1, 2, 300, device=dev)
    ea.fwd_blocksparse(q, k, v, mask, causal=False, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_causal_mask_above_the_diagonal_only(oracle_mod):
    # blocks that lie wholly above the diagonal are dropped; rows of a query
    # block whose only block is partly above the diagonal see a prefix
    N = 512
    q, k, v = attn_inputs.make(1, 2, 2, N, 128, "bf16", seed=31)
    nbq, nbk = N // BQ, N // BK
    mask = np.zeros((1, nbq, nbk), np.uint8)
    for qb in range(nbq):
        mask[0, qb, 2 * qb + 1] = 1  # second key tile of the diagonal block
        if qb + 1 < nbq:
            mask[0, qb, 2 * qb + 2] = 1  # wholly above the diagonal: no key visible
    o, lse = run(q, k, v, mask, True)
    ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, BQ, BK, causal=True)
    assert np.isneginf(rl).any() and np.isfinite(rl).any()
    check(o, lse, ro, rl, "diagonal")


@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_scales_and_extreme_logits(oracle_mod, scale):
    q, k, v = attn_inputs.make(1, 4, 4, 600, 64, "bf16", seed=37, q_mult=8.0)
    mask = rand_mask(4, 600, 0.5, seed=9)
    for causal in (False, True):
        o, lse = run(q, k, v, mask, causal, scale=scale)
        ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, BQ, BK, causal=causal, scale=scale)
        check(o, lse, ro, rl, f"scale={scale} causal={causal}")


def test_deterministic_bitwise():
    dev = gpu()
    q, k, v = (t.to(dev) for t in attn_inputs.make(2, 8, 2, 2000, 128, "bf16", seed=41))
    mask = torch.from_numpy(rand_mask(8, 2000, 0.3, seed=2)).to(dev)
    o1, l1 = ea.fwd_blocksparse(q, k, v, mask, causal=True)
    for _ in range(3):
        o2, l2 = ea.fwd_blocksparse(q, k, v, mask, causal=True)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- full size
def test_full_size_sampled_heads(oracle_mod):
    """The benchmark's block-sparse workload (local window + strided global
    blocks + random blocks, per head), checked on two whole heads."""
    w = attn_inputs.SPARSE_WORKLOADS["local_global"]
    dev = gpu()
    q, k, v = attn_inputs.make(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed)
    mask = attn_inputs.sparse_mask(w)
    o, lse = ea.fwd_blocksparse(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(mask).to(dev),
                                causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    group = w.Hq // w.Hkv
    for h in (0, w.Hq - 1):
        g = h // group
        ro, rl = oracle_mod.fwd_blockmask(q[:, h:h + 1].contiguous(), k[:, g:g + 1].contiguous(),
                                          v[:, g:g + 1].contiguous(), mask[h:h + 1], BQ, BK,
                                          causal=w.causal)
        check(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"{w.name} head {h}")


# ---------------------------------------------------------------- strided
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_token_major_layout(oracle_mod, d, causal):
    dev = gpu()
    q, k, v = attn_inputs.make(2, 8, 2, 700, d, "bf16", seed=d + 60)
    mask = rand_mask(8, 700, 0.4, seed=d)
    qt, kt, vt = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
    o, lse = ea.fwd_blocksparse(qt, kt, vt, torch.from_numpy(mask).to(dev), causal=causal)
    torch.cuda.synchronize()
    assert o.transpose(1, 2).is_contiguous()
    ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, BQ, BK, causal=causal)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"token-major d={d}")


def test_dense_strides_are_the_dense_entry_point_bitwise():
    dev = gpu()
    B, Hq, Hkv, N, d = 2, 4, 2, 500, 128
    q, k, v = (t.to(dev) for t in attn_inputs.make(B, Hq, Hkv, N, d, "bf16", seed=61))
    mask = torch.from_numpy(rand_mask(1, N, 0.5, seed=4)).to(dev)
    o1, l1 = ea.fwd_blocksparse(q, k, v, mask, causal=True)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    ws = torch.empty(ea.attn_fwd_blocksparse_workspace_bytes(Hq, N, 1), device=dev,
                     dtype=torch.uint8)
    dense = [Hq * N * d, N * d, d, Hkv * N * d, N * d, d, Hq * N * d, N * d, d]
    st = ea.attn_fwd_blocksparse_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                                         l2.data_ptr(), mask.data_ptr(), 1, ws.data_ptr(), dense,
                                         B, Hq, Hkv, N, d, 1, d ** -0.5, ea.ATTN_BF16,
                                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == ea.ATTN_OK
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
