"""Backward parity: dQ, dK, dV from the HIP kernels against the fp64 oracle.

Tolerance (bf16 I/O): per gradient tensor, max |g - g_ref| <= 5e-2 * max |g_ref|.
The relative Frobenius error is also checked (<= 2e-2).  The GPU backward
consumes the GPU forward's O and LSE (as a caller would); the oracle
recomputes everything itself in fp64.  Small problems are compared in full;
the full-size workload on every (batch, kv-group) slice, which the oracle
computes separately.  Every comparison also applies an element-wise check,
|g - g_ref| <= 1e-2 max |g_ref| + 5e-2 |g_ref|.
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


def run(q, k, v, do, causal, scale=None):
    dev = gpu()
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = ea.fwd(qg, kg, vg, causal=causal, scale=scale)
    dq, dk, dv = ea.bwd(qg, kg, vg, o, lse, dog, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy() for t in (dq, dk, dv))


def check_grad(name, g, r):
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    ref_max = np.abs(r).max()
    err = np.abs(g - r).max()
    if ref_max == 0:
        assert err <= 1e-6, f"{name}: max err {err} with zero reference"
        return
    assert err <= 5e-2 * ref_max, f"{name}: max err {err} vs max ref {ref_max}"
    fro = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert fro <= 2e-2, f"{name}: relative Frobenius error {fro}"
    check_grad_elementwise(name, g, r)


def check_grad_elementwise(name, g, r, rtol=5e-2, atol_frac=1e-2):
    """Element by element, in the forward's allclose form: |g - g_ref| <=
    atol + rtol |g_ref| with rtol the 5e-2 relative bound and atol a fifth of
    the per-tensor bound (1e-2 max |g_ref|), so an entry far below the
    tensor's largest must still be right to within a few per cent of itself
    or of 1% of that largest value."""
    atol = atol_frac * np.abs(r).max()
    excess = np.abs(g - r) - (atol + rtol * np.abs(r))
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, (f"{name}: element {worst} = {g[worst]} vs {r[worst]} "
                                f"(atol {atol:.3g}); {int((excess > 0).sum())} elements out")


@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 128, 129, 200, 257, 383])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_full_compare(oracle_mod, N, d, causal):
    q, k, v, do = attn_inputs.make(2, 4, 2, N, d, "bf16", seed=2000 + N, with_dout=True)
    dq, dk, dv = run(q, k, v, do, causal)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=causal)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_grad(f"{name} N={N} d={d} causal={causal}", g, r)


@pytest.mark.parametrize("heads", [(1, 1), (8, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_head_maps(oracle_mod, heads, causal):
    Hq, Hkv = heads
    q, k, v, do = attn_inputs.make(2, Hq, Hkv, 150, 64, "bf16", seed=3 * Hq + Hkv, with_dout=True)
    dq, dk, dv = run(q, k, v, do, causal)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=causal)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_grad(name, g, r)


@pytest.mark.parametrize("heads,d", [((64, 1), 128), ((128, 8), 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_wide_head_groups(oracle_mod, heads, d, causal):
    """64 query heads on one kv head, and 128 on 8: the dK/dV stage walks (or
    splits) groups far wider than the workloads' 4."""
    Hq, Hkv = heads
    q, k, v, do = attn_inputs.make(1, Hq, Hkv, 200, d, "bf16", seed=Hq + d, with_dout=True)
    dq, dk, dv = run(q, k, v, do, causal)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=causal)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_grad(f"{name} Hq={Hq} Hkv={Hkv} d={d}", g, r)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_scales(oracle_mod, scale, causal):
    q, k, v, do = attn_inputs.make(1, 2, 1, 170, 128, "bf16", seed=9, with_dout=True)
    dq, dk, dv = run(q, k, v, do, causal, scale=scale)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=causal, scale=scale)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_grad(f"{name} scale={scale}", g, r)


def test_bwd_extreme_logits(oracle_mod):
    q, k, v, do = attn_inputs.make(1, 4, 1, 300, 128, "bf16", seed=10, q_mult=8.0, with_dout=True)
    dq, dk, dv = run(q, k, v, do, True)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=True)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_grad(name, g, r)


def test_bwd_deterministic_bitwise():
    dev = gpu()
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(2, 8, 2, 700, 128, "bf16", seed=12,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=True)
    ref = ea.bwd(q, k, v, o, lse, do, causal=True)
    for _ in range(3):
        again = ea.bwd(q, k, v, o, lse, do, causal=True)
        for a, b in zip(ref, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d64_three_stage_pipeline_deterministic(causal):
    """d=64 runs the dK/dV kernel with three LDS stages and partial load waits,
    where wave 0 issues one load more per stage than the other waves; every
    wave must wait with its own count.  Repeated launches on a full-size
    problem must agree bit for bit."""
    dev = gpu()
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(8, 16, 16, 2048, 64, "bf16", seed=13,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=causal)
    ref = ea.bwd(q, k, v, o, lse, do, causal=causal)
    for _ in range(10):
        again = ea.bwd(q, k, v, o, lse, do, causal=causal)
        for a, b in zip(ref, again):
            assert torch.equal(a, b)


def test_bwd_gqa_equals_summed_mha():
    """dK/dV of a shared kv head equal the sum over its query heads' MHA gradients."""
    dev = gpu()
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(1, 8, 2, 260, 64, "bf16", seed=13,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=True)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, do, causal=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, lse2 = ea.fwd(q, kr, vr, causal=True)
    dq2, dk2, dv2 = ea.bwd(q, kr, vr, o2, lse2, do, causal=True)
    assert torch.equal(dq, dq2)
    dk_sum = dk2.float().reshape(1, 2, 4, 260, 64).sum(2)
    dv_sum = dv2.float().reshape(1, 2, 4, 260, 64).sum(2)
    assert (dk.float() - dk_sum).abs().max() <= 2e-2 * dk_sum.abs().max()
    assert (dv.float() - dv_sum).abs().max() <= 2e-2 * dv_sum.abs().max()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_gqa_split_query_heads(oracle_mod, d, causal):
    """Few kv heads and a short sequence: the dK/dV stage splits each group's
    query heads over several workgroups (fp32 partial sums in the workspace,
    merged in a fixed order).  Parity with the oracle, and bitwise repeatable."""
    B, Hq, Hkv, N = 1, 12, 2, 300
    stats = B * Hq * 2 * 320 * 4
    assert ea.attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, ea.ATTN_BF16) > stats  # split taken
    q, k, v, do = attn_inputs.make(B, Hq, Hkv, N, d, "bf16", seed=70 + d, with_dout=True)
    dev = gpu()
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = ea.fwd(qg, kg, vg, causal=causal)
    g1 = ea.bwd(qg, kg, vg, o, lse, dog, causal=causal)
    g2 = ea.bwd(qg, kg, vg, o, lse, dog, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    rq, rk, rv = oracle_mod.bwd(q, k, v, do, causal=causal)
    for name, g, r in zip(("dQ", "dK", "dV"), g1, (rq, rk, rv)):
        check_grad(f"{name} d={d} causal={causal} (split heads)", g.float().cpu().numpy(), r)


def test_bwd_constant_values_give_zero_dq_dk():
    dev = gpu()
    q, k, v, do = attn_inputs.make(1, 2, 2, 200, 64, "bf16", seed=14, with_dout=True)
    v[:] = v[:, :, :1, :]
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = ea.fwd(qg, kg, vg, causal=True)
    dq, dk, dv = ea.bwd(qg, kg, vg, o, lse, dog, causal=True)
    # D_i = dO_i . O_i uses the bf16-rounded O, so dP - D is only ~1e-3 relative
    assert dq.float().abs().max() <= 1e-2 * dv.float().abs().max()
    assert dk.float().abs().max() <= 1e-2 * dv.float().abs().max()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_dq_statistics_equal_the_preprocess(d, causal):
    """attn_bwd_dq_stats writes the preprocess kernel's statistics bit for bit
    (padding rows included, over a buffer that starts as NaN), and its dQ is
    attn_bwd_dq's."""
    dev = gpu()
    B, Hq, Hkv, N = 2, 4, 2, 200  # Np = 256: 56 padding rows; the last block holds 72 rows
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(B, Hq, Hkv, N, d, "bf16", seed=16,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=causal)
    Np = (N + 63) // 64 * 64
    s = torch.cuda.current_stream().cuda_stream
    sc = d ** -0.5
    st_pre = torch.full((B * Hq, 2, Np), float("nan"), device=dev, dtype=torch.float32)
    st_fused = torch.full_like(st_pre, float("nan"))
    dq_pre, dq_fused = torch.empty_like(q), torch.empty_like(q)
    assert ea.attn_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), st_pre.data_ptr(),
                                  B, Hq, N, d, ea.ATTN_BF16, s) == ea.ATTN_OK
    assert ea.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                          st_pre.data_ptr(), dq_pre.data_ptr(), B, Hq, Hkv, N, d, causal, sc,
                          ea.ATTN_BF16, s) == ea.ATTN_OK
    assert ea.attn_bwd_dq_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), st_fused.data_ptr(),
                                dq_fused.data_ptr(), B, Hq, Hkv, N, d, causal, sc, ea.ATTN_BF16,
                                s) == ea.ATTN_OK
    torch.cuda.synchronize()
    assert torch.equal(st_pre.view(torch.int32), st_fused.view(torch.int32))
    assert torch.equal(dq_pre, dq_fused)


def test_staged_backward_equals_attn_bwd():
    dev = gpu()
    B, Hq, Hkv, N, d = 2, 8, 2, 333, 128
    q, k, v, do = (t.to(dev) for t in attn_inputs.make(B, Hq, Hkv, N, d, "bf16", seed=15,
                                                       with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=True)
    ref = ea.bwd(q, k, v, o, lse, do, causal=True)
    nbytes = ea.attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, ea.ATTN_BF16)
    Np = (N + 63) // 64 * 64
    # this grouped-query shape splits its query heads in the dK/dV stage, which
    # keeps partial sums in the workspace after the statistics
    assert nbytes > B * Hq * 2 * Np * 4
    ws = torch.full((nbytes // 4,), float("nan"), device=dev, dtype=torch.float32)
    stats = ws[:B * Hq * 2 * Np].view(B * Hq, 2, Np)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    s = torch.cuda.current_stream().cuda_stream
    sc = d ** -0.5
    assert ea.attn_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), stats.data_ptr(),
                                  B, Hq, N, d, ea.ATTN_BF16, s) == ea.ATTN_OK
    assert ea.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                            stats.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            B, Hq, Hkv, N, d, 1, sc, ea.ATTN_BF16, s) == ea.ATTN_OK
    assert ea.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                          stats.data_ptr(), dq.data_ptr(), B, Hq, Hkv, N, d, 1,
                          sc, ea.ATTN_BF16, s) == ea.ATTN_OK
    torch.cuda.synchronize()
    for a, b in zip(ref, (dq, dk, dv)):
        assert torch.equal(a, b)
    # row statistics: -D_i = -(dO_i . O_i), LSE_i * log2(e), zero padding
    ref_d = -(do.float() * o.float()).sum(-1).reshape(B * Hq, N)
    assert (stats[:, 0, :N] - ref_d).abs().max() <= 1e-3 * ref_d.abs().max()
    ref_l = lse.reshape(B * Hq, N) * 1.4426950408889634
    assert (stats[:, 1, :N] - ref_l).abs().max() <= 1e-5 * ref_l.abs().max()
    assert bool((stats[:, :, N:] == 0).all())
    # the two-launch order attn_bwd uses: dQ with the statistics, then dK/dV
    stats.fill_(float("nan"))
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    assert ea.attn_bwd_dq_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), stats.data_ptr(), dq2.data_ptr(),
                                B, Hq, Hkv, N, d, 1, sc, ea.ATTN_BF16, s) == ea.ATTN_OK
    assert ea.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                            stats.data_ptr(), dk2.data_ptr(), dv2.data_ptr(),
                            B, Hq, Hkv, N, d, 1, sc, ea.ATTN_BF16, s) == ea.ATTN_OK
    torch.cuda.synchronize()
    for a, b in zip(ref, (dq2, dk2, dv2)):
        assert torch.equal(a, b)


def test_bwd_empty():
    dev = gpu()
    q = torch.empty(1, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    lse = torch.empty(1, 2, 0, device=dev, dtype=torch.float32)
    dq, dk, dv = ea.bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
    assert dq.numel() == 0


# ---------------------------------------------------------------- full-size
def full_size_slices(oracle_mod, w, slices):
    q, k, v, do = attn_inputs.make_workload(w, with_dout=True)
    dev = gpu()
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = ea.fwd(qg, kg, vg, causal=w.causal)
    dq, dk, dv = ea.bwd(qg, kg, vg, o, lse, dog, causal=w.causal)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    rq, rk, rv = oracle_mod.bwd_slices(q, k, v, do, slices, causal=w.causal)
    grp = w.Hq // w.Hkv
    for t, s in enumerate(slices):
        b, g = divmod(int(s), w.Hkv)
        gq = dq[b, g * grp:(g + 1) * grp].float().cpu().numpy()
        check_grad(f"{w.name} dQ slice {s}", gq, rq[t])
        check_grad(f"{w.name} dK slice {s}", dk[b, g].float().cpu().numpy(), rk[t])
        check_grad(f"{w.name} dV slice {s}", dv[b, g].float().cpu().numpy(), rv[t])


def test_workload5_fwd_bwd_full_size_every_slice(oracle_mod):
    """Workload 5's backward compared on all 128 (batch, head) slices."""
    w = attn_inputs.WORKLOADS[5]
    full_size_slices(oracle_mod, w, list(range(w.B * w.Hkv)))


def test_gqa_backward_full_size_one_slice(oracle_mod):
    """Workload 4's backward at its full size (B=1, Hq=32, Hkv=8, N=16384,
    d=128, Q x 8, causal) in the launch the benchmark times: 128 key blocks x
    8 kv heads fill the device, so the dK/dV stage runs unsplit, at two
    waves per SIMD.  One (batch, kv head) slice, 4 query heads x 16384 rows
    and 16384 keys, is compared whole (about 12 s of fp64 oracle)."""
    w = attn_inputs.WORKLOADS[4].scaled(backward=True)
    assert ea.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, ea.ATTN_BF16) == \
        w.B * w.Hq * 2 * w.N * 4  # statistics only: no query-head split
    full_size_slices(oracle_mod, w, [5])


# The benchmark's other backward sweep shapes, with its seeds, at full size:
# one (batch, head) slice each.
SWEEP_SLICES = [
    (attn_inputs.Workload("noncausal_bf16_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, False, "bf16",
                          seed=6), 37),
    (attn_inputs.Workload("causal_bf16_B4_H32_N4000_d128", 4, 32, 32, 4000, 128, True, "bf16",
                          seed=3), 100),
    (attn_inputs.Workload("noncausal_bf16_B1_H16_N8192_d256", 1, 16, 16, 8192, 256, False, "bf16",
                          seed=9), 11),
]


@pytest.mark.parametrize("w,slice_", SWEEP_SLICES, ids=[w.name for w, _ in SWEEP_SLICES])
def test_backward_sweep_shapes_full_size_one_slice(oracle_mod, w, slice_):
    full_size_slices(oracle_mod, w, [slice_])


def test_gqa_backward_reduced_length(oracle_mod):
    """Workload 4's heads (Hq=32, Hkv=8, d=128, Q x 8, causal) at N=2048."""
    w = attn_inputs.WORKLOADS[4].scaled(N=2048, backward=True, seed=41)
    full_size_slices(oracle_mod, w, [0, 5, 7])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_xcd_slice_groups_sampled(oracle_mod, causal):
    """Shapes whose dQ (and, non-causal, dK/dV) workgroups run in XCD slice
    groups smaller than an XCD's share of slices: B=4, H=16 is 64 slices, 8 per
    XCD; non-causal N=1024 has 512 KiB of K/V per slice (groups of 4 under a
    2 MiB budget), causal N=4096 has 2 MiB (groups of 4 under 8 MiB)."""
    N = 4096 if causal else 1024
    w = attn_inputs.Workload(f"xcd_groups_B4_H16_N{N}_d128", 4, 16, 16, N, 128, causal, "bf16",
                             backward=True, seed=43)
    full_size_slices(oracle_mod, w, [0, 21, 63])


def test_gqa_backward_unsplit_sampled(oracle_mod):
    """A grouped-query backward whose 128-key blocks x kv heads already fill the
    device (B=4, Hkv=4, N=4096: 512 workgroups at d = 128), so the dK/dV stage
    keeps each group's query heads in one workgroup: no partial sums in the
    workspace."""
    w = attn_inputs.Workload("gqa_unsplit_B4_Hq8_Hkv4_N4096_d128", 4, 8, 4, 4096, 128, True,
                             "bf16", backward=True, seed=44)
    assert ea.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, ea.ATTN_BF16) == \
        w.B * w.Hq * 2 * w.N * 4
    full_size_slices(oracle_mod, w, [0, 15])
