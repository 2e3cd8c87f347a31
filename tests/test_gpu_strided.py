"""Strided-tensor forward parity: attn_fwd_strided (through the C ABI) on
[B, N, H, d] tensors and on slices of a packed QKV projection, against the
fp64 oracle on dense copies of the same values.

Tolerances are the 16-bit forward's: |O - O_ref| <= 2e-2 + 1e-2 |O_ref|,
|LSE - LSE_ref| <= 1e-3.  With the dense strides the result must be
attn_fwd's bit for bit.
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


def check(o, lse, ro, rl, what=""):
    err = np.abs(o - ro)
    bad = err > 2e-2 + 1e-2 * np.abs(ro)
    assert not bad.any(), f"{what} O: {bad.sum()} out of tolerance, max err {err.max()}"
    assert np.abs(lse - rl).max() <= 1e-3, f"{what} LSE max err {np.abs(lse - rl).max()}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_strides_are_the_forward_bitwise(d, causal):
    dev = gpu()
    q, k, v = (t.to(dev) for t in attn_inputs.make(2, 4, 2, 333, d, "bf16", seed=3))
    o, lse = ea.fwd_strided(q, k, v, causal=causal, out=torch.empty_like(q))
    fo, fl = ea.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, fo) and torch.equal(lse, fl)


@pytest.mark.parametrize("N", [1, 100, 257, 700])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_token_major_layout(oracle_mod, N, d, causal):
    # [B, N, H, d] tensors, seen as [B, H, N, d] views; O written [B, N, Hq, d]
    dev = gpu()
    q, k, v = attn_inputs.make(2, 8, 2, N, d, "bf16", seed=N + d)
    qt, kt, vt = (t.transpose(1, 2).contiguous().to(dev) for t in (q, k, v))  # [B, N, H, d]
    o, lse = ea.fwd_strided(qt.transpose(1, 2), kt.transpose(1, 2), vt.transpose(1, 2),
                            causal=causal)
    torch.cuda.synchronize()
    assert o.transpose(1, 2).is_contiguous()
    ro, rl = oracle_mod.fwd(q, k, v, causal=causal)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"N={N} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)])
def test_packed_qkv_projection(oracle_mod, dtype, heads):
    # one [B, N, Hq + 2*Hkv, d] buffer holding Q, K and V heads side by side
    dev = gpu()
    Hq, Hkv = heads
    B, N, d = 2, 450, 128
    q, k, v = attn_inputs.make(B, Hq, Hkv, N, d, dtype, seed=11)
    packed = torch.cat([q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2)], dim=2)
    packed = packed.contiguous().to(dev)  # [B, N, Hq + 2 Hkv, d]
    qv = packed[:, :, :Hq].transpose(1, 2)
    kv = packed[:, :, Hq:Hq + Hkv].transpose(1, 2)
    vv = packed[:, :, Hq + Hkv:].transpose(1, 2)
    for causal in (False, True):
        o, lse = ea.fwd_strided(qv, kv, vv, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.fwd(q, k, v, causal=causal)
        check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"packed {heads} {dtype}")


def test_output_into_a_strided_view(oracle_mod):
    # O written straight into the head slots of a wider [B, N, 2*Hq, d] buffer
    dev = gpu()
    q, k, v = attn_inputs.make(1, 4, 4, 300, 64, "bf16", seed=13)
    big = torch.full((1, 300, 8, 64), 7.0, device=dev, dtype=torch.bfloat16)
    out = big[:, :, 4:].transpose(1, 2)
    ea.fwd_strided(q.to(dev), k.to(dev), v.to(dev), causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.all(big[:, :, :4] == 7.0)  # untouched neighbours
    ro, rl = oracle_mod.fwd(q, k, v, causal=True)
    o = big[:, :, 4:].transpose(1, 2).float().cpu().numpy()
    err = np.abs(o - ro)
    assert not (err > 2e-2 + 1e-2 * np.abs(ro)).any(), err.max()


# ---------------------------------------------------------------- backward
def grads_ok(name, g, r):
    g = g.float().cpu().numpy()
    e, m = np.abs(g - r).max(), np.abs(r).max()
    assert np.all(np.isfinite(g)) and e <= 5e-2 * m, f"{name}: {e} vs {m}"
    assert np.linalg.norm(g - r) / np.linalg.norm(r) <= 2e-2, f"{name} Frobenius"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_dense_strides_are_bwd_bitwise(d, causal):
    dev = gpu()
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(2, 4, 2, 300, d, "bf16", seed=21,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=causal)
    g1 = ea.bwd_strided(q, k, v, o, lse, do, causal=causal)
    g2 = ea.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_token_major(oracle_mod, d, causal):
    dev = gpu()
    q, k, v, do = attn_inputs.make(2, 8, 2, 333, d, "bf16", seed=d + 3, with_dout=True)
    qt, kt, vt, dot = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
                       for t in (q, k, v, do))
    o, lse = ea.fwd_strided(qt, kt, vt, causal=causal)  # o is token-major too
    dq, dk, dv = ea.bwd_strided(qt, kt, vt, o, lse, dot, causal=causal)
    torch.cuda.synchronize()
    assert dq.transpose(1, 2).is_contiguous() and dk.transpose(1, 2).is_contiguous()
    rdq, rdk, rdv = oracle_mod.bwd(q, k, v, do, causal=causal)
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grads_ok(name, g, r)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_token_major_single_head_is_the_dense_backward_bitwise(d):
    """One query and one kv head, token-major: torch gives the size-1 head
    dimension of the forward's output and of dO different strides, which do
    not change the layout (once rejected as a stride mismatch).  In memory the
    layout is the dense one, so the gradients equal attn_bwd's bit for bit."""
    dev = gpu()
    q, k, v, do = attn_inputs.make(2, 1, 1, 211, d, "bf16", seed=50 + d, with_dout=True)
    qt, kt, vt, dot = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
                       for t in (q, k, v, do))
    o, lse = ea.fwd_strided(qt, kt, vt, causal=True)
    g1 = ea.bwd_strided(qt, kt, vt, o, lse, dot, causal=True)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    od, lsed = ea.fwd(qd, kd, vd, causal=True)
    g2 = ea.bwd(qd, kd, vd, od, lsed, dod, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), od) and torch.equal(lse, lsed)
    for a, b in zip(g1, g2):
        assert torch.equal(a.contiguous(), b)


def test_backward_packed_qkv(oracle_mod):
    # Q, K, V slices of one [B, N, Hq + 2 Hkv, d] buffer; dQ, dK, dV into
    # slices of one packed gradient buffer; O and dO token-major
    dev = gpu()
    B, Hq, Hkv, N, d = 2, 8, 2, 260, 128
    q, k, v, do = attn_inputs.make(B, Hq, Hkv, N, d, "fp16", seed=31, with_dout=True)
    packed = torch.cat([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().to(dev)
    qv = packed[:, :, :Hq].transpose(1, 2)
    kv = packed[:, :, Hq:Hq + Hkv].transpose(1, 2)
    vv = packed[:, :, Hq + Hkv:].transpose(1, 2)
    o, lse = ea.fwd_strided(qv, kv, vv, causal=True)
    dob = do.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    gpack = torch.full_like(packed, 9.0)
    dq = gpack[:, :, :Hq].transpose(1, 2)
    dk = gpack[:, :, Hq:Hq + Hkv].transpose(1, 2)
    dv = gpack[:, :, Hq + Hkv:].transpose(1, 2)
    ea.bwd_strided(qv, kv, vv, o, lse, dob, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle_mod.bwd(q, k, v, do, causal=True)
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        grads_ok(name, g, r)
