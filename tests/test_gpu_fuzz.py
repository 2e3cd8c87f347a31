"""Seeded random configurations across the entry points, against the fp64
oracle.

Each case draws a shape (batch, query and key/value heads, length, head
dimension), a mask, a 16-bit type, a scale (sign and magnitude) and a memory
layout (dense [B, H, N, d] or token-major [B, N, H, d]) from a fixed seed, so
the set is the same on every run.  Beside the dense and strided forward and
backward: packed variable-length sequences (forward and backward, random
lengths including empty ones), split-K/V against a cache (random query and
key counts, split requests) and block-sparse masks (random density, one mask
or one per head).  Tolerances are the forward's
(|O - O_ref| <= 2e-2 + 1e-2 |O_ref|, |LSE - LSE_ref| <= 1e-3) and the
backward's (max |g - g_ref| <= 5e-2 max |g_ref|, relative Frobenius <= 2e-2).
"""
import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def draw(seed, max_n):
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    return dict(B=int(r.integers(1, 3)), Hq=Hq, Hkv=Hkv, N=int(r.integers(1, max_n + 1)),
                d=int(r.choice([64, 128, 256])), causal=bool(r.integers(0, 2)),
                dtype=str(r.choice(["bf16", "fp16"])),
                scale=float(r.choice([-1.0, 1.0]) * r.uniform(0.02, 0.3)),
                token_major=bool(r.integers(0, 2)), seed=seed)


def tensors(c, with_dout):
    g = torch.Generator().manual_seed(c["seed"])
    td = torch.bfloat16 if c["dtype"] == "bf16" else torch.float16
    shp_q = (c["B"], c["Hq"], c["N"], c["d"])
    shp_k = (c["B"], c["Hkv"], c["N"], c["d"])
    out = [torch.randn(shp_q, generator=g), torch.randn(shp_k, generator=g),
           torch.randn(shp_k, generator=g)]
    if with_dout:
        out.append(torch.randn(shp_q, generator=g))
    return [t.to(td) for t in out]


def to_dev(t, c, dev):
    if c["token_major"]:
        return t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    return t.to(dev)


def fwd_dev(q, k, v, c):
    if c["token_major"]:
        return ea.fwd_strided(q, k, v, causal=c["causal"], scale=c["scale"])
    return ea.fwd(q, k, v, causal=c["causal"], scale=c["scale"])


@pytest.mark.parametrize("seed", range(40))
def test_forward(oracle_mod, seed):
    dev = gpu()
    c = draw(1000 + seed, 700)
    q, k, v = tensors(c, False)
    o, lse = fwd_dev(*(to_dev(t, c, dev) for t in (q, k, v)), c)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd(q, k, v, causal=c["causal"], scale=c["scale"])
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    err = np.abs(o - ro)
    assert not (err > 2e-2 + 1e-2 * np.abs(ro)).any(), f"{c}: O max err {err.max()}"
    assert np.abs(lse - rl).max() <= 1e-3, f"{c}: LSE max err {np.abs(lse - rl).max()}"


@pytest.mark.parametrize("seed", range(20))
def test_backward(oracle_mod, seed):
    dev = gpu()
    c = draw(2000 + seed, 300)
    q, k, v, do = tensors(c, True)
    qg, kg, vg, dog = (to_dev(t, c, dev) for t in (q, k, v, do))
    o, lse = fwd_dev(qg, kg, vg, c)
    if c["token_major"]:
        grads = ea.bwd_strided(qg, kg, vg, o, lse, dog, causal=c["causal"], scale=c["scale"])
    else:
        grads = ea.bwd(qg, kg, vg, o, lse, dog, causal=c["causal"], scale=c["scale"])
    torch.cuda.synchronize()
    refs = oracle_mod.bwd(q, k, v, do, causal=c["causal"], scale=c["scale"])
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        g = g.float().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{c} {name}: non-finite"
        e, m = np.abs(g - r).max(), np.abs(r).max()
        if m == 0 or (name != "dV" and m < 1e-3 * np.abs(refs[2]).max()):
            # one visible key per row: dQ and dK are zero up to rounding
            assert e <= 1e-3 * max(np.abs(refs[2]).max(), 1.0), f"{c} {name}: {e}"
            continue
        assert e <= 5e-2 * m, f"{c} {name}: max err {e} vs max ref {m}"
        fro = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert fro <= 2e-2, f"{c} {name}: Frobenius {fro}"


def check_rows(o, lse, ro, rl, what):
    """Forward tolerances; rows that see no key must be exactly O = 0, LSE = -inf."""
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with no key differ"
    assert np.all(o[empty] == 0.0), f"{what}: a row with no key has O != 0"
    o, ro, lse, rl = o[~empty], ro[~empty], lse[~empty], rl[~empty]
    if o.size == 0:
        return
    err = np.abs(o - ro)
    assert not (err > 2e-2 + 1e-2 * np.abs(ro)).any(), f"{what}: O max err {err.max()}"
    assert np.abs(lse - rl).max() <= 1e-3, f"{what}: LSE max err {np.abs(lse - rl).max()}"


def grads_ok(what, grads, refs):
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        e, m = np.abs(g - r).max(initial=0.0), np.abs(r).max(initial=0.0)
        if m == 0 or (name != "dV" and m < 1e-3 * np.abs(refs[2]).max(initial=0.0)):
            assert e <= 1e-3 * max(np.abs(refs[2]).max(initial=0.0), 1.0), f"{what} {name}: {e}"
            continue
        assert e <= 5e-2 * m, f"{what} {name}: max err {e} vs max ref {m}"
        fro = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert fro <= 2e-2, f"{what} {name}: Frobenius {fro}"


def draw_common(r):
    return dict(d=int(r.choice([64, 128, 256])), causal=bool(r.integers(0, 2)),
                dtype=str(r.choice(["bf16", "fp16"])),
                scale=float(r.choice([-1.0, 1.0]) * r.uniform(0.02, 0.3)),
                token_major=bool(r.integers(0, 2)))


@pytest.mark.parametrize("seed", range(20))
def test_varlen(oracle_mod, seed):
    dev = gpu()
    r = np.random.default_rng(3000 + seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    lengths = [int(x) for x in r.integers(0, 400, size=int(r.integers(1, 6)))]
    lengths[-1] = max(lengths[-1], 1)
    c = dict(Hq=Hq, Hkv=Hkv, lengths=lengths, **draw_common(r))
    q, k, v, cu = attn_inputs.make_varlen(Hq, Hkv, lengths, c["d"], seed=3000 + seed,
                                          dtype=c["dtype"])
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(seed)).to(q.dtype)

    def put(t):  # [H, T, d], dense or a view of a token-major [T, H, d] tensor
        if c["token_major"]:
            return t.transpose(0, 1).contiguous().to(dev).transpose(0, 1)
        return t.to(dev)

    qg, kg, vg, dog = (put(t) for t in (q, k, v, do))
    cug, mx = cu.to(dev), max(lengths)
    o, lse = ea.fwd_varlen(qg, kg, vg, cug, mx, causal=c["causal"], scale=c["scale"])
    grads = ea.bwd_varlen(qg, kg, vg, o, lse, dog, cug, mx, causal=c["causal"], scale=c["scale"])
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_varlen(q, k, v, cu.numpy(), causal=c["causal"], scale=c["scale"])
    check_rows(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, str(c))
    refs = [np.zeros(t.shape) for t in (q, k, v)]
    for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()):
        if b > a:
            sl = slice(a, b)
            g = oracle_mod.bwd(q[None, :, sl], k[None, :, sl], v[None, :, sl], do[None, :, sl],
                               causal=c["causal"], scale=c["scale"])
            for ref, part in zip(refs, g):
                ref[:, sl] = part[0]
    grads_ok(str(c), [t.float().cpu().numpy() for t in grads], refs)


@pytest.mark.parametrize("seed", range(20))
def test_splitkv(oracle_mod, seed):
    dev = gpu()
    r = np.random.default_rng(4000 + seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    Hq = Hkv * int(r.choice([1, 2, 4, 8]))
    c = dict(B=int(r.integers(1, 3)), Hq=Hq, Hkv=Hkv, Nq=int(r.integers(1, 71)),
             Nk=int(r.integers(0, 3001)), splits=int(r.integers(0, 17)), **draw_common(r))
    q, k, v = attn_inputs.make_cache(c["B"], Hq, Hkv, c["Nq"], c["Nk"], c["d"], seed=4000 + seed,
                                     dtype=c["dtype"])

    def put(t):  # [B, H, N, d], dense or a view of a token-major [B, N, H, d] tensor
        if c["token_major"]:
            return t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
        return t.to(dev)

    o, lse = ea.fwd_splitkv(put(q), put(k), put(v), causal=c["causal"], scale=c["scale"],
                            num_splits=c["splits"])
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_bottom_right(q, k, v, causal=c["causal"], scale=c["scale"])
    check_rows(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, str(c))


@pytest.mark.parametrize("seed", range(20))
def test_blocksparse(oracle_mod, seed):
    dev = gpu()
    r = np.random.default_rng(5000 + seed)
    Hkv = int(r.choice([1, 2, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    c = dict(B=int(r.integers(1, 3)), Hq=Hq, Hkv=Hkv, N=int(r.integers(1, 701)),
             density=float(r.uniform(0.0, 1.0)), per_head=bool(r.integers(0, 2)),
             **draw_common(r))
    c.pop("token_major")
    q, k, v = attn_inputs.make_cache(c["B"], Hq, Hkv, c["N"], c["N"], c["d"], seed=5000 + seed,
                                     dtype=c["dtype"])
    heads = Hq if c["per_head"] else 1
    mask = (r.random((heads, -(-c["N"] // 128), -(-c["N"] // 64))) < c["density"]).astype(np.uint8)
    o, lse = ea.fwd_blocksparse(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(mask).to(dev),
                                causal=c["causal"], scale=c["scale"])
    torch.cuda.synchronize()
    ro, rl = oracle_mod.fwd_blockmask(q, k, v, mask, 128, 64, causal=c["causal"], scale=c["scale"])
    check_rows(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, str(c))
