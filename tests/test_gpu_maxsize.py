"""Parity at the longest sequence the library accepts, N <= 2^22 (GPU).

The fp64 oracle cannot run an N x N problem of that length, so the inputs
(attn_inputs.make_long_filler) make exact references cheap: the first M keys
are zero, so every query scores exactly 0 against each of them, and query,
value and upstream-gradient rows repeat with a period of P rows.
  - Rows i < M see only zero keys: equal weights, so O_i is the mean of
    v_0..v_i and LSE_i = ln(i + 1), and dQ_i = scale * sum_j dS_ij k_j = 0.
  - Rows and keys from L = M - W on: such a row sees the L zero keys before
    L (score 0 each: total weight L, mean value vbar) and the keys from L to
    itself.  That is a causal problem of W + T + 1 rows in which key 0 stands
    for the L zero keys, its log-weight ln L carried by one extra coordinate
    (1 in every real query, ln L / scale in key 0) and its value vbar; row 0
    is a dummy query with zero upstream gradient.  The oracle gives its O,
    LSE and dQ exactly for rows L..N-1, and dK, dV for keys L..N-1, which no
    row before L sees.
  - The keys before L: since the probabilities of a row sum to 1, the dK of
    all keys sum to 0 and the dV of all keys to the sum of dO; with the
    oracle's dK, dV of keys L..N-1 that fixes the sums over the keys before L.
At d = 256 the last tiles of a slice this long lie within 32 KiB of 2^31
bytes, the end of the kernels' 32-bit offsets.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu

N = (1 << 22) - 37  # the longest accepted is 2^22; a ragged last tile
T = 1000  # drawn keys at the end
W = 256  # zero keys (and their rows) checked through the oracle as well
M = N - T
L = M - W
P = 4096


def build(d, seed, with_dout=False):
    dev = torch.device("cuda:0")
    pieces = attn_inputs.make_long_filler(M, T, d, pool=P, seed=seed, with_dout=with_dout)
    qpool, vpool, ktail, dopool = pieces
    idx = torch.arange(N, device=dev) % P
    q = qpool.to(dev)[idx]
    v = vpool.to(dev)[idx]
    k = torch.zeros((N, d), device=dev, dtype=qpool.dtype)
    k[M:] = ktail.to(dev)
    do = dopool.to(dev)[idx][None, None] if with_dout else None
    host = [None if t is None else t.double().numpy() for t in pieces]
    return host, q[None, None], k[None, None], v[None, None], do


def pool_sum(pool, n):
    """Sum of rows 0..n-1 of a sequence repeating `pool` (fp64)."""
    full, rem = divmod(n, P)
    return full * pool.sum(0) + pool[:rem].sum(0)


def augmented(host, d, scale):
    """The causal problem of rows and keys L..N-1 with key 0 standing for the
    L zero keys before them (see the module docstring)."""
    qpool, vpool, ktail, dopool = host
    rows = np.arange(L, N)
    S = N - L + 1
    qa = np.zeros((S, d + 1))
    qa[1:, :d] = qpool[rows % P]
    qa[1:, d] = 1.0
    ka = np.zeros((S, d + 1))
    ka[0, d] = math.log(L) / scale
    ka[1 + (M - L):, :d] = ktail
    va = np.zeros((S, d))
    va[0] = pool_sum(vpool, L) / L
    va[1:] = vpool[rows % P]
    doa = None
    if dopool is not None:
        doa = np.zeros((S, d))
        doa[1:] = dopool[rows % P]
    return qa[None, None], ka[None, None], va[None, None], (None if doa is None else doa[None, None])


def check(o, lse, ro, rl, what):
    err = np.abs(o - ro)
    bad = err > 2e-2 + 1e-2 * np.abs(ro)
    assert not bad.any(), f"{what} O: {bad.sum()} elements out of tolerance, max err {err.max()}"
    lerr = np.abs(lse - rl)
    assert lerr.max() <= 1e-3, f"{what} LSE max err {lerr.max()}"


def grad_ok(name, g, r):
    e, m = np.abs(g - r).max(), np.abs(r).max()
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    assert e <= 5e-2 * m, f"{name}: max err {e} vs max ref {m}"
    assert np.linalg.norm(g - r) / np.linalg.norm(r) <= 2e-2, f"{name}: Frobenius"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_forward_at_the_maximum_length(oracle_mod, d):
    host, q, k, v, _ = build(d, seed=60 + d)
    o, lse = ea.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    vpool = host[1]
    # rows before L: equal weights over the zero keys
    rows = [0, 1, 2, 63, 64, 127, 128, P - 1, P, 123457, 1 << 20, (1 << 21) + 5, L - 1]
    ro = np.stack([pool_sum(vpool, i + 1) / (i + 1) for i in rows])
    rl = np.log(np.asarray(rows, dtype=np.float64) + 1.0)
    check(o[0, 0, rows].float().cpu().numpy(), lse[0, 0, rows].cpu().numpy(), ro, rl,
          f"zero-key rows d={d}")
    # rows L..N-1 through the oracle
    qa, ka, va, _ = augmented(host, d, scale)
    ao, al = oracle_mod.fwd(qa, ka, va, causal=True, scale=scale)
    check(o[0, 0, L:].float().cpu().numpy(), lse[0, 0, L:].cpu().numpy(), ao[0, 0, 1:],
          al[0, 0, 1:], f"last rows d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_backward_at_the_maximum_length(oracle_mod, d):
    # d = 128: the dK/dV stage with V in LDS and 32-query tiles
    host, q, k, v, do = build(d, seed=70 + d, with_dout=True)
    o, lse = ea.fwd(q, k, v, causal=True)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    # rows before L see only zero keys: dQ = scale * dS K = 0 exactly
    assert not bool(dq[0, 0, :L].any()), "dQ of the zero-key rows is not 0"
    # rows and keys L..N-1 through the oracle
    qa, ka, va, doa = augmented(host, d, scale)
    rdq, rdk, rdv = oracle_mod.bwd(qa, ka, va, doa, causal=True, scale=scale)
    grad_ok("dQ last rows", dq[0, 0, L:].float().cpu().numpy(), rdq[0, 0, 1:, :d])
    grad_ok("dK last keys", dk[0, 0, L:].float().cpu().numpy(), rdk[0, 0, 1:, :d])
    grad_ok("dV last keys", dv[0, 0, L:].float().cpu().numpy(), rdv[0, 0, 1:])
    # keys before L: their sums follow from the whole sequence's
    dk_head = dk[0, 0, :L].double()
    dv_head = dv[0, 0, :L].double()
    ref_k = -rdk[0, 0, 1:, :d].sum(0)  # all dK sum to 0
    ref_v = pool_sum(host[3], N) - rdv[0, 0, 1:].sum(0)  # all dV sum to sum_i dO_i
    # each stored gradient is rounded to bf16 (relative 2^-8 at most), plus
    # the fp32 arithmetic's own error
    for name, g, ref in (("dK", dk_head, ref_k), ("dV", dv_head, ref_v)):
        s = g.sum(0).cpu().numpy()
        bound = 2.0 ** -8 * g.abs().sum(0).cpu().numpy() + 1e-2 * np.abs(ref) + 1e-3
        assert np.all(np.abs(s - ref) <= bound), (
            f"sum of {name} over the keys before L: max |diff| {np.abs(s - ref).max()}")


@pytest.mark.parametrize("d", [128, 256])
def test_splitkv_at_the_maximum_length(oracle_mod, d):
    # Nq = 3 queries of 2 heads against a cache of N keys (bottom-right
    # causal): query i sees keys 0 .. N - 3 + i, that is the M zero keys and
    # the tail up to its own position; the oracle's bottom-right forward on
    # [one key for the zero keys, the tail keys] is the exact reference.
    dev = torch.device("cuda:0")
    Nq, Hq = 3, 2
    qpool, vpool, ktail, _ = attn_inputs.make_long_filler(M, T, d, pool=P, seed=80 + d)
    idx = torch.arange(N, device=dev) % P
    v = vpool.to(dev)[idx]
    k = torch.zeros((N, d), device=dev, dtype=qpool.dtype)
    k[M:] = ktail.to(dev)
    q = qpool[:Hq * Nq].reshape(1, Hq, Nq, d).to(dev)
    o, lse = ea.fwd_splitkv(q, k[None, None], v[None, None], causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    q64, v64, k64 = qpool.double().numpy(), vpool.double().numpy(), ktail.double().numpy()
    qa = np.zeros((1, Hq, Nq, d + 1))
    qa[0, :, :, :d] = q64[:Hq * Nq].reshape(Hq, Nq, d)
    qa[0, :, :, d] = 1.0
    ka = np.zeros((1, 1, T + 1, d + 1))
    ka[0, 0, 0, d] = math.log(M) / scale
    ka[0, 0, 1:, :d] = k64
    va = np.zeros((1, 1, T + 1, d))
    va[0, 0, 0] = pool_sum(v64, M) / M
    va[0, 0, 1:] = v64[np.arange(M, N) % P]
    ro, rl = oracle_mod.fwd_bottom_right(qa, ka, va, causal=True, scale=scale)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"split-K/V d={d}")


def test_varlen_at_the_maximum_length(oracle_mod):
    # T = N packed tokens in two sequences: the first, of S1 tokens, holds
    # only zero keys (closed forms as above, and within it the dK sum to 0
    # and the dV to the sum of its dO); the second starts S1 tokens in, past
    # 4M, and is short enough for the oracle to run whole.
    d = 64
    dev = torch.device("cuda:0")
    S1 = M - 300
    host, q, k, v, do = build(d, seed=90, with_dout=True)
    qpool, vpool, ktail, dopool = host
    cu = torch.tensor([0, S1, N], dtype=torch.int32, device=dev)
    o, lse = ea.fwd_varlen(q[0], k[0], v[0], cu, S1, causal=True)
    dq, dk, dv = ea.bwd_varlen(q[0], k[0], v[0], o, lse, do[0], cu, S1, causal=True)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, P - 1, P, 1 << 20, S1 - 1]
    ro = np.stack([pool_sum(vpool, i + 1) / (i + 1) for i in rows])
    rl = np.log(np.asarray(rows, dtype=np.float64) + 1.0)
    check(o[0, rows].float().cpu().numpy(), lse[0, rows].cpu().numpy(), ro, rl,
          "first sequence")
    assert not bool(dq[0, :S1].any()), "dQ of the first sequence is not 0"
    for name, g, ref in (("dK", dk[0, :S1].double(), np.zeros(d)),
                         ("dV", dv[0, :S1].double(), pool_sum(dopool, S1))):
        s = g.sum(0).cpu().numpy()
        bound = 2.0 ** -8 * g.abs().sum(0).cpu().numpy() + 1e-2 * np.abs(ref) + 1e-3
        assert np.all(np.abs(s - ref) <= bound), (
            f"sum of {name} over the first sequence: max |diff| {np.abs(s - ref).max()}")
    # the second sequence alone
    tok = np.arange(S1, N)
    q2 = qpool[tok % P][None, None]
    k2 = np.zeros((N - S1, d))
    k2[M - S1:] = ktail
    v2 = vpool[tok % P][None, None]
    do2 = dopool[tok % P][None, None]
    r2o, r2l = oracle_mod.fwd(q2, k2[None, None], v2, causal=True)
    check(o[0, S1:].float().cpu().numpy(), lse[0, S1:].cpu().numpy(), r2o[0, 0], r2l[0, 0],
          "second sequence")
    rdq, rdk, rdv = oracle_mod.bwd(q2, k2[None, None], v2, do2, causal=True)
    grad_ok("dQ second sequence", dq[0, S1:].float().cpu().numpy(), rdq[0, 0])
    grad_ok("dK second sequence", dk[0, S1:].float().cpu().numpy(), rdk[0, 0])
    grad_ok("dV second sequence", dv[0, S1:].float().cpu().numpy(), rdv[0, 0])
