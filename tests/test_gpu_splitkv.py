"""Split-K/V forward parity: attn_fwd_splitkv (through the C ABI) against the
fp64 oracle's bottom-right aligned forward.

Tolerances are the bf16 forward's: |O - O_ref| <= 2e-2 + 1e-2 |O_ref|
element-wise, |LSE - LSE_ref| <= 1e-3.  A row that sees no key must come
back exactly O = 0, LSE = -inf.  Small shapes are compared in full (every
split count, tails inside a split and at Nk, rows of several heads inside one
wave); the full-size decode and append workloads are compared on whole
batches that the oracle computes from the same inputs, in the launch
configuration the benchmark times.  Strided tensors: token-major q, cache
and output at d = 64, 128, 256, a cache that is a prefix of a longer
preallocated buffer, and the dense strides bit for bit against the dense
entry point.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device(DEV)


def run(q, k, v, causal, scale=None, num_splits=0):
    dev = gpu()
    o, lse = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                            num_splits=num_splits)
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


SPLITS = [0, 1, 2, 7]


@pytest.mark.parametrize("Nq", [1, 3, 64, 130])
@pytest.mark.parametrize("Nk", [1, 63, 1000, 4097])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_full_compare(oracle_mod, Nq, Nk, d, causal):
    ns = SPLITS[(Nq + Nk + d) % 4]
    q, k, v = attn_inputs.make_cache(2, 4, 2, Nq, Nk, d, seed=Nq * 7 + Nk)
    o, lse = run(q, k, v, causal, num_splits=ns)
    ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
    check(o, lse, ro, rl, f"Nq={Nq} Nk={Nk} d={d} causal={causal} splits={ns}")


@pytest.mark.parametrize("ns", [1, 2, 3, 5, 16, 63, 64, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_split_counts(oracle_mod, ns, d):
    q, k, v = attn_inputs.make_cache(1, 8, 2, 5, 4000, d, seed=ns)
    used = ea.attn_fwd_splitkv_num_splits(1, 8, 2, 5, 4000, d, ns)
    assert 1 <= used <= min(ns, 63)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, num_splits=ns)
        ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
        check(o, lse, ro, rl, f"splits={ns} (used {used}) causal={causal}")


@pytest.mark.parametrize("heads", [(1, 1), (8, 1), (8, 2), (6, 3), (32, 8), (32, 1)])
@pytest.mark.parametrize("Nq", [1, 5, 20])
def test_head_maps(oracle_mod, heads, Nq):
    # group * Nq packed rows: waves hold rows of several query heads
    Hq, Hkv = heads
    q, k, v = attn_inputs.make_cache(2, Hq, Hkv, Nq, 777, 128, seed=Hq * 100 + Hkv + Nq)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, num_splits=3)
        ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
        check(o, lse, ro, rl, f"heads={heads} Nq={Nq} causal={causal}")


@pytest.mark.parametrize("shape", [(100, 40), (70, 1), (300, 257)])
def test_causal_rows_without_keys(oracle_mod, shape):
    # Nq > Nk with the bottom-right mask: the first Nq - Nk rows see nothing
    Nq, Nk = shape
    q, k, v = attn_inputs.make_cache(1, 4, 2, Nq, Nk, 64, seed=Nq + Nk)
    o, lse = run(q, k, v, True, num_splits=2)
    ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=True)
    assert np.isneginf(rl[..., : Nq - Nk]).all()
    check(o, lse, ro, rl, f"Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("causal", [False, True])
def test_no_keys(causal):
    dev = gpu()
    q = torch.randn(2, 4, 3, 64, device=dev).to(torch.bfloat16)
    kv = torch.zeros(8192, device=dev, dtype=torch.uint8)  # K and V of zero keys: never read
    o = torch.full_like(q, 7.0)
    lse = torch.zeros(2, 4, 3, device=dev)
    ws = torch.empty(1 << 16, device=dev, dtype=torch.uint8)
    st = ea.attn_fwd_splitkv(q.data_ptr(), kv.data_ptr(), kv.data_ptr() + 4096, o.data_ptr(),
                             lse.data_ptr(), ws.data_ptr(), 2, 4, 2, 3, 0, 64, causal, 0.125, 0,
                             ea.ATTN_BF16, None)
    torch.cuda.synchronize()
    assert st == ea.ATTN_OK
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("mult", [8.0, 64.0])
def test_extreme_logits(oracle_mod, mult):
    q, k, v = attn_inputs.make_cache(1, 8, 2, 7, 3000, 128, seed=9, q_mult=mult)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, num_splits=4)
        ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
        check(o, lse, ro, rl, f"q x{mult} causal={causal}")


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 1e-3])
def test_scales(oracle_mod, scale):
    q, k, v = attn_inputs.make_cache(1, 4, 1, 9, 1500, 64, seed=21)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, scale=scale, num_splits=3)
        ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal, scale=scale)
        check(o, lse, ro, rl, f"scale={scale} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_square_matches_the_forward(oracle_mod, d):
    # Nq == Nk: the bottom-right mask is the forward's causal mask
    dev = gpu()
    q, k, v = attn_inputs.make(2, 4, 2, 300, d, "bf16", seed=31)
    o, lse = run(q, k, v, True, num_splits=3)
    fo, fl = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    ro, rl = oracle_mod.fwd(q, k, v, causal=True)
    check(o, lse, ro, rl, "split")
    check(fo.float().cpu().numpy(), fl.cpu().numpy(), ro, rl, "forward")


def test_deterministic_bitwise():
    dev = gpu()
    q, k, v = (t.to(dev) for t in attn_inputs.make_cache(2, 16, 4, 3, 5000, 128, seed=3))
    o1, l1 = ea.fwd_splitkv(q, k, v, causal=True, num_splits=5)
    for _ in range(3):
        o2, l2 = ea.fwd_splitkv(q, k, v, causal=True, num_splits=5)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_arguments_are_rejected_before_launch():
    dev = gpu()
    q = torch.zeros(1, 4, 2, 64, device=dev, dtype=torch.bfloat16)
    kv = torch.zeros(1, 2, 100, 64, device=dev, dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 2, device=dev)
    ws = torch.empty(1 << 20, device=dev, dtype=torch.uint8)
    a = [q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr()]
    dims = [1, 4, 2, 2, 100, 64, 1, 0.125, 0, ea.ATTN_BF16, None]
    assert ea.attn_fwd_splitkv(*a, *dims) == ea.ATTN_OK
    torch.cuda.synchronize()
    bad_out = list(a)
    bad_out[3] = q.data_ptr()  # output overlaps the queries
    assert ea.attn_fwd_splitkv(*bad_out, *dims) == ea.ATTN_ERR_INVALID_ARG
    bad_ws = list(a)
    bad_ws[5] = o.data_ptr()  # workspace overlaps the output
    assert ea.attn_fwd_splitkv(*bad_ws, *dims) == ea.ATTN_ERR_INVALID_ARG
    f32 = list(dims)
    f32[9] = ea.ATTN_F32
    assert ea.attn_fwd_splitkv(*a, *f32) == ea.ATTN_ERR_UNSUPPORTED


# ---------------------------------------------------------------- full size
@pytest.mark.parametrize("name", ["decode", "append"])
def test_full_size_sampled_batches(oracle_mod, name):
    # The benchmark's launch (whole workload, default split count); the oracle
    # recomputes two whole batches from the same inputs.
    w = attn_inputs.CACHE_WORKLOADS[name]
    dev = gpu()
    q, k, v = attn_inputs.make_cache_workload(w)
    o, lse = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in (0, w.B - 1):
        ro, rl = oracle_mod.fwd_bottom_right(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=w.causal)
        check(o[b:b + 1], lse[b:b + 1], ro, rl, f"{w.name} batch {b}")


# ---------------------------------------------------------------- strided
def token_major(t, dev):
    """[B, H, N, d] -> the same values in a [B, N, H, d] buffer, viewed as [B, H, N, d]."""
    return t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)


@pytest.mark.parametrize("Nq", [1, 5, 70])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_token_major_cache(oracle_mod, Nq, d, causal):
    # q and the key/value cache token-major ([B, N, H, d]); the output too
    dev = gpu()
    q, k, v = attn_inputs.make_cache(2, 8, 2, Nq, 1500, d, seed=Nq + d)
    qt, kt, vt = (token_major(t, dev) for t in (q, k, v))
    o, lse = ea.fwd_splitkv(qt, kt, vt, causal=causal, num_splits=3)
    torch.cuda.synchronize()
    assert o.transpose(1, 2).is_contiguous()
    ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=causal)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"token-major Nq={Nq} d={d}")


def test_cache_slices_of_a_larger_buffer(oracle_mod):
    # k, v: the first Nk tokens of a longer preallocated [B, Nmax, Hkv, d] cache
    dev = gpu()
    B, Hq, Hkv, Nq, Nk, Nmax, d = 2, 8, 2, 4, 1000, 2048, 128
    q, k, v = attn_inputs.make_cache(B, Hq, Hkv, Nq, Nk, d, seed=44)
    kc = torch.zeros(B, Nmax, Hkv, d, dtype=k.dtype)
    vc = torch.zeros(B, Nmax, Hkv, d, dtype=v.dtype)
    kc[:, :Nk] = k.transpose(1, 2)
    vc[:, :Nk] = v.transpose(1, 2)
    kg = kc.to(dev)[:, :Nk].transpose(1, 2)
    vg = vc.to(dev)[:, :Nk].transpose(1, 2)
    o, lse = ea.fwd_splitkv(q.to(dev), kg, vg, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=True)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "cache slice")


@pytest.mark.parametrize("d", [64, 128])
def test_dense_strides_are_the_dense_entry_point_bitwise(d):
    dev = gpu()
    B, Hq, Hkv, Nq, Nk = 2, 8, 2, 3, 3000
    q, k, v = (t.to(dev) for t in attn_inputs.make_cache(B, Hq, Hkv, Nq, Nk, d, seed=8))
    o1, l1 = ea.fwd_splitkv(q, k, v, causal=True, num_splits=4)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    ws = torch.empty(ea.attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, 4), device=dev,
                     dtype=torch.uint8)
    dense = [Hq * Nq * d, Nq * d, d, Hkv * Nk * d, Nk * d, d, Hq * Nq * d, Nq * d, d]
    st = ea.attn_fwd_splitkv_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                                     l2.data_ptr(), ws.data_ptr(), dense, B, Hq, Hkv, Nq, Nk, d,
                                     1, d ** -0.5, 4, ea.ATTN_BF16,
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == ea.ATTN_OK
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
