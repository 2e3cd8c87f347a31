"""Packed variable-length forward parity: attn_fwd_varlen (through the C ABI)
against the oracle's packed forward (each token attends within its own
sequence).

Tolerances are the bf16 forward's: |O - O_ref| <= 2e-2 + 1e-2 |O_ref|
element-wise and |LSE - LSE_ref| <= 1e-3.  Cases cover sequences of length
0, 1, tile multiples and tails, many short sequences, head maps, both head
dims and causal modes; one sequence must reproduce attn_fwd bit for bit; the
full-size document workload is checked on whole heads.  The backward is
checked against the oracle's backward on each sequence's slices (gradient
tolerances: max |g - g_ref| <= 5e-2 max |g_ref|, relative Frobenius <= 2e-2).
Strided tensors: token-major [T, H, d] and slices of a packed QKV projection,
forward and backward, and the dense strides bit for bit against the dense
entry points.
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


def run(q, k, v, cu, causal, max_seqlen=None, scale=None):
    dev = gpu()
    lengths = (cu[1:] - cu[:-1]).tolist()
    mx = max(lengths) if max_seqlen is None else max_seqlen
    o, lse = ea.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), mx, causal=causal,
                           scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, ro, rl, what=""):
    err = np.abs(o - ro)
    bad = err > 2e-2 + 1e-2 * np.abs(ro)
    assert not bad.any(), f"{what} O: {bad.sum()} elements out of tolerance, max err {err.max()}"
    lerr = np.abs(lse - rl)
    assert lerr.max() <= 1e-3, f"{what} LSE max err {lerr.max()}"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


LENGTHS = [[1], [127, 1, 300], [0, 64, 0, 129], [1000], [128, 128, 128], [5, 700, 2, 0, 255]]


@pytest.mark.parametrize("lengths", LENGTHS, ids=[str(x) for x in LENGTHS])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_sequences(oracle_mod, lengths, d, causal):
    q, k, v, cu = attn_inputs.make_varlen(4, 2, lengths, d, seed=sum(lengths) + d)
    o, lse = run(q, k, v, cu, causal)
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=causal)
    check(o, lse, ro, rl, f"{lengths} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_many_short_sequences(oracle_mod, causal):
    r = np.random.default_rng(3)
    lengths = r.integers(0, 200, size=40).tolist()
    q, k, v, cu = attn_inputs.make_varlen(8, 2, lengths, 128, seed=5)
    o, lse = run(q, k, v, cu, causal)
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=causal)
    check(o, lse, ro, rl, f"40 sequences causal={causal}")


@pytest.mark.parametrize("heads", [(1, 1), (8, 1), (6, 3)])
def test_head_maps_and_scales(oracle_mod, heads):
    Hq, Hkv = heads
    q, k, v, cu = attn_inputs.make_varlen(Hq, Hkv, [300, 77, 513], 64, seed=Hq)
    for scale in (0.0, -0.2):
        o, lse = run(q, k, v, cu, True, scale=scale)
        ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=True, scale=scale)
        check(o, lse, ro, rl, f"heads={heads} scale={scale}")


@pytest.mark.parametrize("heads", [(16, 4), (24, 3), (32, 8), (16, 16)])
def test_head_order_over_xcds(oracle_mod, heads):
    # With Hq a multiple of 8 each sequence's heads are dealt to the XCDs in a
    # permuted order (whole kv groups per XCD); every head must still land on
    # its own rows, forward and backward, against the oracle in full.
    dev = gpu()
    Hq, Hkv = heads
    lengths = [150, 70, 300]
    q, k, v, cu = attn_inputs.make_varlen(Hq, Hkv, lengths, 64, seed=Hq + Hkv)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(Hq)).to(q.dtype)
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, max(lengths), causal=True)
    dq, dk, dv = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, max(lengths), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=True)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"heads={heads}")
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, True)
    for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grad_ok(f"{name} heads={heads}", gg, r)


def test_max_seqlen_larger_than_needed(oracle_mod):
    q, k, v, cu = attn_inputs.make_varlen(2, 2, [100, 30], 64, seed=7)
    o, lse = run(q, k, v, cu, True, max_seqlen=130)
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=True)
    check(o, lse, ro, rl)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 2), (16, 4)])
def test_one_sequence_is_the_batched_forward_bitwise(d, causal, heads):
    dev = gpu()
    q, k, v, cu = attn_inputs.make_varlen(heads[0], heads[1], [999], d, seed=11)
    q, k, v, cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    o, lse = ea.fwd_varlen(q, k, v, cu, 999, causal=causal)
    fo, fl = ea.fwd(q[None], k[None], v[None], causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, fo[0]) and torch.equal(lse, fl[0])


def test_deterministic_bitwise():
    dev = gpu()
    q, k, v, cu = (t.to(dev) for t in attn_inputs.make_varlen(8, 2, [400, 1, 2000, 33], 128,
                                                               seed=13))
    o1, l1 = ea.fwd_varlen(q, k, v, cu, 2000, causal=True)
    for _ in range(3):
        o2, l2 = ea.fwd_varlen(q, k, v, cu, 2000, causal=True)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_full_size_documents_sampled_heads(oracle_mod):
    w = attn_inputs.VARLEN_WORKLOADS["docs"]
    lengths = attn_inputs.varlen_lengths(w)
    q, k, v, cu = attn_inputs.make_varlen(w.Hq, w.Hkv, lengths, w.d, seed=w.seed)
    o, lse = run(q, k, v, cu, w.causal)
    group = w.Hq // w.Hkv
    for h in (0, w.Hq - 1):
        g = h // group
        ro, rl = oracle_mod.fwd_varlen(q[h:h + 1], k[g:g + 1], v[g:g + 1], cu.numpy(),
                                       causal=w.causal)
        check(o[h:h + 1], lse[h:h + 1], ro, rl, f"{w.name} head {h}")


# ---------------------------------------------------------------- backward
def varlen_bwd_reference(oracle_mod, q, k, v, do, cu, causal):
    """The oracle's dense backward on each sequence's slices, put back in place."""
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()):
        if b == a:
            continue
        sl = slice(a, b)
        g = oracle_mod.bwd(q[None, :, sl].contiguous(), k[None, :, sl].contiguous(),
                           v[None, :, sl].contiguous(), do[None, :, sl].contiguous(), causal=causal)
        dq[:, sl], dk[:, sl], dv[:, sl] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def grad_ok(name, g, r):
    g = g.float().cpu().numpy()
    e, m = np.abs(g - r).max(), np.abs(r).max()
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    assert e <= 5e-2 * m, f"{name}: max err {e} vs max ref {m}"
    assert np.linalg.norm(g - r) / np.linalg.norm(r) <= 2e-2, f"{name}: Frobenius"


BWD_LENGTHS = [[5, 7, 130, 1, 64], [0, 300, 0, 3], [129, 257]]


@pytest.mark.parametrize("lengths", BWD_LENGTHS, ids=[str(x) for x in BWD_LENGTHS])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_packed_sequences(oracle_mod, lengths, d, causal):
    # starts that are not multiples of 4 or 64 exercise the statistics reads
    dev = gpu()
    q, k, v, cu = attn_inputs.make_varlen(4, 2, lengths, d, seed=sum(lengths) + 7)
    g = torch.Generator().manual_seed(5)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    mx = max(lengths)
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, mx, causal=causal)
    dq, dk, dv = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, mx, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, causal)
    for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grad_ok(f"{name} {lengths} d={d}", gg, r)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_one_sequence_is_attn_bwd_bitwise(d):
    dev = gpu()
    q, k, v, cu = (t.to(dev) for t in attn_inputs.make_varlen(4, 2, [777], d, seed=9))
    do = torch.randn_like(q)
    o, lse = ea.fwd_varlen(q, k, v, cu, 777, causal=True)
    g1 = ea.bwd_varlen(q, k, v, o, lse, do, cu, 777, causal=True)
    g2 = ea.bwd(q[None], k[None], v[None], o[None], lse[None], do[None], causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b[0])


def test_backward_deterministic_and_fp16(oracle_mod):
    dev = gpu()
    lengths = [300, 1, 45, 512]
    q, k, v, cu = attn_inputs.make_varlen(8, 2, lengths, 64, seed=17, dtype="fp16")
    g = torch.Generator().manual_seed(6)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, 512, causal=True)
    ref = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, 512, causal=True)
    for _ in range(3):
        again = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, 512, causal=True)
        for a, b in zip(ref, again):
            assert torch.equal(a, b)
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, True)
    for name, gg, r in (("dQ", ref[0], rdq), ("dK", ref[1], rdk), ("dV", ref[2], rdv)):
        grad_ok(name, gg, r)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_fp16_next_sequence_with_very_negative_lse(oracle_mod, d):
    # The dK/dV stage reads statistics per 64-row query tile; the last tile of
    # a sequence reaches past its end.  Here the second document's first token
    # sees only itself with score s_00 = -20, so its LSE is -20: read as the
    # statistic of a padding row of the first document, P = e^20 would
    # overflow fp16 and 0 * inf would turn that kv head's dK/dV into NaN.
    dev = gpu()
    lengths = [100, 40]
    q, k, v, cu = attn_inputs.make_varlen(4, 2, lengths, d, seed=23, dtype="fp16")
    scale = 1.0 / d ** 0.5
    t0 = lengths[0]
    for h in range(4):
        kk = k[h // 2, t0].float()
        q[h, t0] = (kk * (-20.0 / (scale * float(kk @ kk)))).to(q.dtype)
    g = torch.Generator().manual_seed(8)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, max(lengths), causal=True)
    dq, dk, dv = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, max(lengths), causal=True)
    torch.cuda.synchronize()
    assert float(lse[0, t0]) < -19.0  # the planted statistic is there
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, True)
    for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grad_ok(f"{name} d={d}", gg, r)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_non_finite_sequence_stays_in_its_sequence(oracle_mod, d, causal):
    # A NaN and an Inf in the upstream gradient of the middle sequence make
    # that sequence's gradients non-finite; the sequences before and after it
    # must still match the oracle.  The first sequence's last query tile
    # reaches past its end into the middle sequence's rows, whose statistics
    # the dK/dV stage reads there (and must not let through).
    dev = gpu()
    lengths = [100, 40, 70]
    q, k, v, cu = attn_inputs.make_varlen(4, 2, lengths, d, seed=31 + d)
    g = torch.Generator().manual_seed(9)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    t1 = lengths[0]
    do[:, t1, 0] = float("nan")
    do[:, t1 + 1, 3] = float("inf")
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, max(lengths), causal=causal)
    dq, dk, dv = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, max(lengths), causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, causal)
    assert not np.all(np.isfinite(dk[:, t1:t1 + 40].float().cpu().numpy()))  # the planted values act
    for a, b in ((0, t1), (t1 + 40, sum(lengths))):
        sl = slice(a, b)
        for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            grad_ok(f"{name}[{a}:{b}] d={d}", gg[:, sl], r[:, sl])


def test_backward_full_size_documents_sampled_heads(oracle_mod):
    w = attn_inputs.VARLEN_WORKLOADS["docs"]
    lengths = attn_inputs.varlen_lengths(w)
    q, k, v, cu = attn_inputs.make_varlen(w.Hq, w.Hkv, lengths, w.d, seed=w.seed)
    g = torch.Generator().manual_seed(w.seed + 100)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    dev = gpu()
    mx = max(lengths)
    qg, kg, vg, dog, cug = (t.to(dev) for t in (q, k, v, do, cu))
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, mx, causal=w.causal)
    dq, dk, dv = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, mx, causal=w.causal)
    torch.cuda.synchronize()
    group = w.Hq // w.Hkv
    # kv head 0 and its query heads: dK/dV sum over the group's query heads
    hs = slice(0, group)
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q[hs], k[0:1], v[0:1], do[hs], cu, w.causal)
    grad_ok("dQ", dq[hs], rdq)
    grad_ok("dK", dk[0:1], rdk)
    grad_ok("dV", dv[0:1], rdv)


# ---------------------------------------------------------------- strided
def token_major(t, dev):
    """[H, T, d] -> the same values in a token-major [T, H, d] buffer, viewed as [H, T, d]."""
    return t.transpose(0, 1).contiguous().to(dev).transpose(0, 1)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_token_major_forward_and_backward(oracle_mod, d, causal):
    dev = gpu()
    lengths = [5, 130, 0, 64, 201]
    q, k, v, cu = attn_inputs.make_varlen(4, 2, lengths, d, seed=d + 40)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(8)).to(q.dtype)
    qt, kt, vt, dot = (token_major(t, dev) for t in (q, k, v, do))
    cug = cu.to(dev)
    o, lse = ea.fwd_varlen(qt, kt, vt, cug, 201, causal=causal)
    assert o.transpose(0, 1).is_contiguous()  # token-major output by default
    dq, dk, dv = ea.bwd_varlen(qt, kt, vt, o, lse, dot, cug, 201, causal=causal)
    torch.cuda.synchronize()
    assert dq.stride() == qt.stride() and dk.stride() == kt.stride()
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=causal)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"token-major d={d}")
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, causal)
    for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grad_ok(f"{name} token-major d={d}", gg, r)


@pytest.mark.parametrize("d", [64, 128])
def test_dense_strides_are_the_dense_entry_points_bitwise(d):
    dev = gpu()
    lengths = [100, 1, 300]
    q, k, v, cu = (t.to(dev) for t in attn_inputs.make_varlen(4, 2, lengths, d, seed=3))
    do = torch.randn_like(q)
    T = q.shape[1]
    o1, l1 = ea.fwd_varlen(q, k, v, cu, 300, causal=True)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    dense = [T * d, d] * 3
    s = torch.cuda.current_stream().cuda_stream
    assert ea.attn_fwd_varlen_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                                      l2.data_ptr(), cu.data_ptr(), dense, 3, 300, 4, 2, T, d, 1,
                                      d ** -0.5, ea.ATTN_BF16, s) == ea.ATTN_OK
    g1 = ea.bwd_varlen(q, k, v, o1, l1, do, cu, 300, causal=True)
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    ws = torch.empty(ea.attn_bwd_workspace_bytes(1, 4, 2, T, d, ea.ATTN_BF16), device=dev,
                     dtype=torch.uint8)
    assert ea.attn_bwd_varlen_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                                      l1.data_ptr(), do.data_ptr(), g2[0].data_ptr(),
                                      g2[1].data_ptr(), g2[2].data_ptr(), ws.data_ptr(),
                                      cu.data_ptr(), dense, 3, 300, 4, 2, T, d, 1, d ** -0.5,
                                      ea.ATTN_BF16, s) == ea.ATTN_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_packed_qkv_projection(oracle_mod):
    # q, k, v slices of one [T, Hq + 2 Hkv, d] projection; gradients into
    # slices of one packed gradient buffer; fp16
    dev = gpu()
    Hq, Hkv, d = 8, 2, 128
    lengths = [70, 257, 3]
    q, k, v, cu = attn_inputs.make_varlen(Hq, Hkv, lengths, d, seed=12, dtype="fp16")
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(2)).to(q.dtype)
    packed = torch.cat([q, k, v], dim=0).transpose(0, 1).contiguous().to(dev)  # [T, H, d]
    qv = packed[:, :Hq].transpose(0, 1)
    kv = packed[:, Hq:Hq + Hkv].transpose(0, 1)
    vv = packed[:, Hq + Hkv:].transpose(0, 1)
    cug = cu.to(dev)
    o, lse = ea.fwd_varlen(qv, kv, vv, cug, 257, causal=True)
    gpack = torch.full_like(packed, 7.0)
    dq = gpack[:, :Hq].transpose(0, 1)
    dk = gpack[:, Hq:Hq + Hkv].transpose(0, 1)
    dv = gpack[:, Hq + Hkv:].transpose(0, 1)
    ea.bwd_varlen(qv, kv, vv, o, lse, token_major(do, dev), cug, 257, causal=True,
                  dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=True)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "packed qkv")
    rdq, rdk, rdv = varlen_bwd_reference(oracle_mod, q, k, v, do, cu, True)
    for name, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grad_ok(f"{name} packed qkv", gg, r)
