"""The C ABI library on the host: it loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU.

The arguments are fake device addresses.  Calls that are meant to fail
validation never reach the device on any host.  Calls that are meant to pass
validation stop at the device check only where no GPU is visible; on a host
with a GPU they would launch kernels on unmapped addresses.  Every test that
makes such a call is marked ``reaches_device`` and is skipped when a device
node or a torch device is visible, so this module is safe to collect on a GPU
host as well."""
import os
import re
import subprocess

import pytest

import exact_attention_87_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _gpu_visible() -> bool:
    # /dev/kfd is the ROCm compute device node; counting torch devices does
    # not initialise the HIP runtime
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


GPU_VISIBLE = _gpu_visible()
# A test that makes at least one call expected to pass validation (and, with
# no GPU, to stop at the device check with ATTN_ERR_HIP).
reaches_device = pytest.mark.skipif(
    GPU_VISIBLE, reason="passes fake addresses through validation; with a GPU visible the call "
                        "would launch kernels on them")

@pytest.fixture(autouse=True)
def _device_reach_is_marked(request, monkeypatch):
    """Keeps the marker honest: on a host without a GPU, a test not marked
    ``reaches_device`` fails if any of its calls got past validation."""
    if GPU_VISIBLE or request.node.get_closest_marker("skipif") is not None:
        yield
        return
    reached = []
    for name in [n for n in dir(ea) if n.startswith("attn_") and callable(getattr(ea, n))]:
        fn = getattr(ea, name)

        def wrap(*a, _fn=fn, _name=name):
            r = _fn(*a)
            if isinstance(r, int) and r in (ea.ATTN_ERR_HIP, ea.ATTN_ERR_UNSUPPORTED_DEVICE):
                reached.append(_name)
            return r

        monkeypatch.setattr(ea, name, wrap)
    yield
    assert not reached, f"unmarked test reached the device check via {sorted(set(reached))}"


# Fake, 16-byte aligned, non-overlapping addresses: validation must fail
# before anything dereferences them.
Q, K, V, O, L, DO, DQ, DK, DV, WS = (0x10000000 * (i + 1) for i in range(10))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert header_functions() == ["attn_abi_version", "attn_bwd", "attn_bwd_dkdv", "attn_bwd_dq",
                                  "attn_bwd_dq_stats", "attn_bwd_noalloc", "attn_bwd_preprocess",
                                  "attn_bwd_strided", "attn_bwd_varlen",
                                  "attn_bwd_varlen_strided",
                                  "attn_bwd_workspace_bytes", "attn_fwd",
                                  "attn_fwd_blocksparse", "attn_fwd_blocksparse_strided",
                                  "attn_fwd_blocksparse_workspace_bytes",
                                  "attn_fwd_splitkv", "attn_fwd_splitkv_num_splits",
                                  "attn_fwd_splitkv_strided",
                                  "attn_fwd_splitkv_workspace_bytes", "attn_fwd_strided",
                                  "attn_fwd_varlen", "attn_fwd_varlen_strided",
                                  "attn_probe_clock", "attn_status_str"]


def test_library_loads_and_exports_every_declared_symbol():
    lib = ea.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", ea.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert ea.attn_abi_version() == 2


def test_status_strings():
    assert ea.attn_status_str(ea.ATTN_OK) == "ATTN_OK"
    assert ea.attn_status_str(ea.ATTN_ERR_INVALID_ARG) == "ATTN_ERR_INVALID_ARG"
    assert ea.attn_status_str(ea.ATTN_ERR_UNSUPPORTED_DEVICE) == "ATTN_ERR_UNSUPPORTED_DEVICE"
    assert ea.attn_status_str(99) == "unknown attn_status"


def fwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=4, Hkv=2, N=100, d=64, causal=0, scale=0.125,
             dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                       a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


def bwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, B=2, Hq=4, Hkv=2,
             N=100, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                       a["dv"], a["ws"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                       a["scale"], a["dtype"], a["stream"])


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(B=-1), dict(N=-3), dict(Hq=0), dict(Hkv=0), dict(Hq=6, Hkv=4),
    dict(causal=2), dict(causal=-1), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(dtype=7), dict(q=Q + 8), dict(o=O + 4), dict(lse=L + 2),
    dict(o=Q), dict(o=K + 64), dict(lse=Q + 1024), dict(lse=O + 16),
]


@pytest.mark.parametrize("kw", INVALID, ids=[str(k) for k in INVALID])
def test_fwd_rejects_bad_arguments(kw):
    assert fwd(**kw) == ea.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [0, 32, 96, 512])
def test_fwd_unsupported_head_dim(d):
    assert fwd(d=d) == ea.ATTN_ERR_UNSUPPORTED


@reaches_device
def test_d256_is_16_bit_only():
    # accepted by the 16-bit paths (validation passes; no GPU here)
    for dt in (ea.ATTN_BF16, ea.ATTN_F16):
        assert fwd(d=256, dtype=dt) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
        assert split(d=256, dtype=dt) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
        assert sparse(d=256, dtype=dt) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
        assert varlen(d=256, dtype=dt) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert fwd(d=256, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    for dt in (ea.ATTN_BF16, ea.ATTN_F16):
        assert bwd(d=256, dtype=dt) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert bwd(d=256, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert ea.attn_bwd_workspace_bytes(1, 1, 1, 64, 256, ea.ATTN_BF16) == 512
    assert sparse(d=256, N=(1 << 20) + 1) == ea.ATTN_ERR_UNSUPPORTED


def test_fwd_too_large_is_unsupported():
    assert fwd(N=(1 << 22) + 1) == ea.ATTN_ERR_UNSUPPORTED
    assert fwd(B=1 << 13, Hq=1 << 12, Hkv=1 << 12) == ea.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0)])
def test_empty_problem_is_ok_without_pointers(kw):
    assert fwd(q=None, k=None, v=None, o=None, lse=None, **kw) == ea.ATTN_OK
    assert bwd(q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None, dv=None,
               ws=None, **kw) == ea.ATTN_OK


BWD_INVALID = [
    dict(dout=None), dict(dq=None), dict(ws=None), dict(dk=DK + 8), dict(dq=DO),
    dict(dk=DV), dict(ws=Q + 256), dict(dv=DK + 1024), dict(Hq=3, Hkv=2), dict(causal=5),
]


@pytest.mark.parametrize("kw", BWD_INVALID, ids=[str(k) for k in BWD_INVALID])
def test_bwd_rejects_bad_arguments(kw):
    assert bwd(**kw) == ea.ATTN_ERR_INVALID_ARG


def test_bwd_fp32_is_unsupported():
    assert bwd(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert ea.attn_bwd_workspace_bytes(1, 1, 1, 16, 64, ea.ATTN_F32) == -1


def test_workspace_bytes():
    # statistics: [B*Hq][2][N rounded up to 64] fp32, rounded up to 256 bytes
    assert ea.attn_bwd_workspace_bytes(1, 1, 1, 1, 64, ea.ATTN_BF16) == 512
    assert ea.attn_bwd_workspace_bytes(8, 16, 16, 2048, 64, ea.ATTN_BF16) == 8 * 16 * 2 * 2048 * 4
    # grouped-query problem whose 128-key blocks x kv heads fill the device
    # (1024 workgroups at d = 128, one per CU): statistics only
    assert ea.attn_bwd_workspace_bytes(1, 32, 8, 16384, 128, ea.ATTN_BF16) == 32 * 2 * 16384 * 4
    # small grids: the dK/dV stage splits each group's query heads over S
    # workgroups and keeps 2 * S * B * Hkv * N * d fp32 partial sums after the
    # statistics.  S is the smallest divisor of the group reaching two rounds
    # of resident workgroups (512 at d = 128, 1536 at d = 64), else the group.
    #   B=1 Hq=32 Hkv=8 N=2048 d=128: 128 workgroups, S = 4 (the group)
    assert ea.attn_bwd_workspace_bytes(1, 32, 8, 2048, 128, ea.ATTN_BF16) == \
        32 * 2 * 2048 * 4 + 2 * 4 * 8 * 2048 * 128 * 4
    #   B=8 Hq=16 Hkv=2 N=2048 d=64: 256 workgroups, need 6, divisors of 8 -> S = 8
    assert ea.attn_bwd_workspace_bytes(8, 16, 2, 2048, 64, ea.ATTN_BF16) == \
        8 * 16 * 2 * 2048 * 4 + 2 * 8 * 8 * 2 * 2048 * 64 * 4
    #   B=2 Hq=4 Hkv=2 N=100 d=64: 4 workgroups, S = 2 (the group)
    assert ea.attn_bwd_workspace_bytes(2, 4, 2, 100, 64, ea.ATTN_BF16) == \
        2 * 4 * 2 * 128 * 4 + 2 * 2 * 2 * 2 * 100 * 64 * 4
    #   B=4 Hq=24 Hkv=2 N=1024 d=64: 64 workgroups, need 24, group 12 -> S = 12
    assert ea.attn_bwd_workspace_bytes(4, 24, 2, 1024, 64, ea.ATTN_BF16) == \
        4 * 24 * 2 * 1024 * 4 + 2 * 12 * 4 * 2 * 1024 * 64 * 4
    #   B=16 Hq=32 Hkv=4 N=1024 d=64: 512 workgroups, need 3, group 8 -> S = 4
    assert ea.attn_bwd_workspace_bytes(16, 32, 4, 1024, 64, ea.ATTN_BF16) == \
        16 * 32 * 2 * 1024 * 4 + 2 * 4 * 16 * 4 * 1024 * 64 * 4
    assert ea.attn_bwd_workspace_bytes(0, 4, 2, 100, 64, ea.ATTN_BF16) == 0
    assert ea.attn_bwd_workspace_bytes(1, 3, 2, 100, 64, ea.ATTN_BF16) == -1
    assert ea.attn_bwd_workspace_bytes(1, 4, 2, 100, 80, ea.ATTN_BF16) == -1


def test_torch_wrapper_rejects_host_tensors():
    import torch

    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.fwd(x, x, x)


def test_staged_backward_validation():
    ok = dict(B=2, Hq=4, Hkv=2, N=100, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16, stream=None)
    # empty problems are fine without pointers
    assert ea.attn_bwd_preprocess(None, None, None, None, 0, 4, 100, 64, ea.ATTN_BF16,
                                  None) == ea.ATTN_OK
    assert ea.attn_bwd_dkdv(*([None] * 7), 2, 4, 2, 0, 64, 1, 0.1, ea.ATTN_BF16, None) == ea.ATTN_OK
    assert ea.attn_bwd_dq(*([None] * 6), 2, 4, 2, 0, 64, 1, 0.1, ea.ATTN_BF16, None) == ea.ATTN_OK
    # missing / misaligned / overlapping buffers
    bad_pre = [(O, None, L, WS), (O, DO, None, WS), (O, DO, L, O + 64), (O, DO, L, WS + 4),
               (O, DO, L, L + 512)]
    for o, do, lse, st in bad_pre:
        assert ea.attn_bwd_preprocess(o, do, lse, st, 2, 4, 100, 64, ea.ATTN_BF16, None) == \
            ea.ATTN_ERR_INVALID_ARG
    args = [ok[x] for x in ("B", "Hq", "Hkv", "N", "d", "causal", "scale", "dtype", "stream")]
    assert ea.attn_bwd_dkdv(Q, K, V, DO, WS, DK, K, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dkdv(Q, K, V, DO, WS, DK, DK, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dkdv(Q, K, V, DO, WS, WS + 256, DV, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq(Q, K, V, DO, WS, WS, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq(Q, K, V, DO, None, DQ, *args) == ea.ATTN_ERR_INVALID_ARG
    bad = list(args)
    bad[2] = 3  # Hq % Hkv != 0
    assert ea.attn_bwd_dq(Q, K, V, DO, WS, DQ, *bad) == ea.ATTN_ERR_INVALID_ARG
    f32 = list(args)
    f32[7] = ea.ATTN_F32
    assert ea.attn_bwd_dkdv(Q, K, V, DO, WS, DK, DV, *f32) == ea.ATTN_ERR_UNSUPPORTED
    # the fused dQ + statistics stage: stats is an output here
    assert ea.attn_bwd_dq_stats(*([None] * 8), 2, 4, 2, 0, 64, 1, 0.1, ea.ATTN_BF16,
                                None) == ea.ATTN_OK
    assert ea.attn_bwd_dq_stats(Q, K, V, O, L, DO, WS, DQ, *bad) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq_stats(Q, K, V, O, L, DO, None, DQ, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq_stats(Q, K, V, O, L, DO, WS, WS + 256, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq_stats(Q, K, V, O, L, DO, O + 64, DQ, *args) == ea.ATTN_ERR_INVALID_ARG
    assert ea.attn_bwd_dq_stats(Q, K, V, O, L, DO, WS, DQ, *f32) == ea.ATTN_ERR_UNSUPPORTED


# ---------------------------------------------------------------- split K/V
def split(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, ws=WS, B=2, Hq=4, Hkv=2, Nq=3, Nk=1000, d=128, causal=1,
             scale=0.125, ns=0, dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["B"], a["Hq"],
                               a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                               a["ns"], a["dtype"], a["stream"])


SPLIT_INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(ws=None),
    dict(B=-1), dict(Nq=-1), dict(Nk=-5), dict(Hq=0), dict(Hkv=0), dict(Hq=6, Hkv=4),
    dict(causal=2), dict(scale=float("nan")), dict(ns=-1), dict(dtype=5), dict(q=Q + 8),
    dict(ws=WS + 4), dict(o=Q), dict(lse=O + 16), dict(ws=O), dict(ws=K + 256),
]


@pytest.mark.parametrize("kw", SPLIT_INVALID, ids=[str(k) for k in SPLIT_INVALID])
def test_splitkv_rejects_bad_arguments(kw):
    assert split(**kw) == ea.ATTN_ERR_INVALID_ARG


def test_splitkv_unsupported():
    assert split(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert split(d=96) == ea.ATTN_ERR_UNSUPPORTED
    assert split(Nk=(1 << 22) + 1) == ea.ATTN_ERR_UNSUPPORTED
    assert split(Nq=(1 << 22) + 1) == ea.ATTN_ERR_UNSUPPORTED
    assert split(Hq=64, Hkv=1, Nq=(1 << 16) + 1) == ea.ATTN_ERR_UNSUPPORTED  # > 2^22 rows per group


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0)])
def test_splitkv_empty_problem(kw):
    assert split(q=None, k=None, v=None, o=None, lse=None, ws=None, **kw) == ea.ATTN_OK
    assert ea.attn_fwd_splitkv_workspace_bytes(kw.get("B", 2), 4, 2, kw.get("Nq", 3), 100, 64,
                                               0) == 0


def test_splitkv_split_counts():
    n = ea.attn_fwd_splitkv_num_splits
    # 1000 keys = 16 tiles of 64: 7 asked -> ranges of 3 tiles -> 6 non-empty ranges
    assert n(1, 4, 2, 3, 1000, 64, 7) == 6
    assert n(1, 4, 2, 3, 1000, 64, 1) == 1
    assert n(1, 4, 2, 3, 1000, 64, 16) == 16
    assert n(1, 4, 2, 3, 1000, 64, 100) == 16  # at most one range per tile
    assert n(1, 4, 2, 3, 1, 64, 5) == 1
    assert n(1, 4, 2, 3, 0, 64, 5) == 1  # no keys: one (empty) range writes the result
    assert n(0, 4, 2, 3, 100, 64, 5) == 0
    assert n(1, 4, 2, 3, 100, 64, -1) == -1
    # chosen from the shape: one round of resident workgroups (512 at d=128),
    # at least 4 tiles per range
    assert n(8, 32, 8, 1, 32768, 128, 0) == 8
    assert n(1, 1, 1, 1, 256, 64, 0) == 1
    for args in [(2, 8, 2, 5, 4000, 128), (1, 32, 8, 64, 16384, 128), (3, 4, 4, 1, 77, 64)]:
        assert 1 <= n(*args, 0) <= (args[4] + 63) // 64


def test_splitkv_workspace_bytes():
    w = ea.attn_fwd_splitkv_workspace_bytes
    # fp32 partial O [splits][rows][d] and LSE [splits][rows], each rounded up to 256 bytes
    assert w(1, 2, 1, 3, 100, 64, 1) == 1536 + 256
    assert w(2, 4, 2, 3, 1000, 128, 7) == 6 * 24 * 128 * 4 + 768
    assert w(1, 3, 2, 1, 100, 64, 1) == -1
    assert w(1, 4, 2, 1, 100, 80, 1) == -1


# ---------------------------------------------------------------- block-sparse
MASK = 0x10000000 * 11 + 3  # any alignment is fine for the byte mask


def sparse(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, mask=MASK, mh=1, ws=WS, B=2, Hq=4, Hkv=2, N=1000, d=64,
             causal=1, scale=0.125, dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["mh"],
                                   a["ws"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                                   a["scale"], a["dtype"], a["stream"])


SPARSE_INVALID = [
    dict(q=None), dict(o=None), dict(lse=None), dict(ws=None), dict(mask=None), dict(mh=0),
    dict(mh=2), dict(mh=3, Hq=4), dict(B=-1), dict(N=-1), dict(Hq=6, Hkv=4), dict(causal=3),
    dict(scale=float("inf")), dict(o=Q), dict(ws=O + 256), dict(mask=O + 5), dict(mask=WS),
    dict(mask=L + 100), dict(q=Q + 4),
]


@pytest.mark.parametrize("kw", SPARSE_INVALID, ids=[str(k) for k in SPARSE_INVALID])
def test_blocksparse_rejects_bad_arguments(kw):
    assert sparse(**kw) == ea.ATTN_ERR_INVALID_ARG


@reaches_device
def test_blocksparse_unsupported_and_empty():
    assert sparse(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert sparse(d=96) == ea.ATTN_ERR_UNSUPPORTED
    assert sparse(N=(1 << 21) + 1) == ea.ATTN_ERR_UNSUPPORTED
    assert sparse(q=None, k=None, v=None, o=None, lse=None, mask=None, ws=None, N=0) == ea.ATTN_OK
    assert sparse(q=None, k=None, v=None, o=None, lse=None, mask=None, ws=None, B=0) == ea.ATTN_OK
    assert sparse(mh=4) != ea.ATTN_ERR_INVALID_ARG  # one mask per query head is accepted


def test_blocksparse_workspace_bytes():
    w = ea.attn_fwd_blocksparse_workspace_bytes
    # counts [mask rows] int32 and lists [mask rows][ceil(N/64)] int32, each rounded to 256
    assert w(4, 1000, 1) == 256 + 8 * 16 * 4
    assert w(4, 1000, 4) == 256 + ((32 * 16 * 4 + 255) // 256) * 256
    assert w(8, 16384, 8) == ((8 * 128 * 4 + 255) // 256) * 256 + 8 * 128 * 256 * 4
    assert w(4, 0, 1) == 0
    assert w(4, 100, 2) == -1
    assert w(4, (1 << 21) + 1, 1) == -1


# ---------------------------------------------------------------- packed variable length
CU = 0x10000000 * 12 + 4


def varlen(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, cu=CU, nseq=3, maxlen=500, Hq=4, Hkv=2, T=1000, d=64,
             causal=1, scale=0.125, dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["nseq"],
                              a["maxlen"], a["Hq"], a["Hkv"], a["T"], a["d"], a["causal"],
                              a["scale"], a["dtype"], a["stream"])


VARLEN_INVALID = [
    dict(q=None), dict(o=None), dict(lse=None), dict(cu=None), dict(cu=CU + 2), dict(nseq=-1),
    dict(maxlen=-1), dict(maxlen=1001), dict(T=-1), dict(Hq=6, Hkv=4), dict(causal=2),
    dict(scale=float("nan")), dict(o=Q + 64), dict(lse=O), dict(cu=O + 8), dict(cu=L + 4),
    dict(k=K + 8),
]


@pytest.mark.parametrize("kw", VARLEN_INVALID, ids=[str(k) for k in VARLEN_INVALID])
def test_varlen_rejects_bad_arguments(kw):
    assert varlen(**kw) == ea.ATTN_ERR_INVALID_ARG


def test_varlen_unsupported_and_empty():
    assert varlen(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert varlen(d=80) == ea.ATTN_ERR_UNSUPPORTED
    assert varlen(T=(1 << 22) + 1, maxlen=10) == ea.ATTN_ERR_UNSUPPORTED
    assert varlen(nseq=(1 << 23), Hq=4) == ea.ATTN_ERR_UNSUPPORTED
    none = dict(q=None, k=None, v=None, o=None, lse=None, cu=None)
    assert varlen(nseq=0, **none) == ea.ATTN_OK
    assert varlen(T=0, maxlen=0, **none) == ea.ATTN_OK
    assert varlen(maxlen=0, **none) == ea.ATTN_OK


@reaches_device
def test_fp16_is_accepted_where_bf16_is():
    assert ea.attn_bwd_workspace_bytes(2, 4, 2, 100, 64, ea.ATTN_F16) == \
        ea.attn_bwd_workspace_bytes(2, 4, 2, 100, 64, ea.ATTN_BF16)
    # validation passes for fp16 and stops only at the device check (no GPU here)
    assert fwd(dtype=ea.ATTN_F16) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert bwd(dtype=ea.ATTN_F16) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert split(dtype=ea.ATTN_F16) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert sparse(dtype=ea.ATTN_F16) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert varlen(dtype=ea.ATTN_F16) not in (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert fwd(dtype=3) == ea.ATTN_ERR_INVALID_ARG


# ---------------------------------------------------------------- strided tensors
def strided(strides, **kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=4, Hkv=2, N=100, d=64, causal=1, scale=0.125,
             dtype=ea.ATTN_BF16, stream=None)
    a.update(kw)
    return ea.attn_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], strides, a["B"], a["Hq"],
                               a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"],
                               a["stream"])


BNHD = [100 * 4 * 64, 64, 4 * 64, 100 * 2 * 64, 64, 2 * 64, 100 * 4 * 64, 64, 4 * 64]


@reaches_device
def test_strided_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    assert strided(BNHD) not in ok  # passes validation, stops at the device check
    for i, bad in [(2, 60), (2, 65), (1, 4), (0, -8), (5, 32), (8, 0)]:
        s = list(BNHD)
        s[i] = bad
        assert strided(s) == ea.ATTN_ERR_INVALID_ARG, (i, bad)
    huge = list(BNHD)
    huge[2] = 1 << 23  # (N + 127) * row * 2 >= 2^31
    assert strided(huge) == ea.ATTN_ERR_INVALID_ARG
    assert strided(BNHD, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert strided(BNHD, o=Q + 64) == ea.ATTN_ERR_INVALID_ARG  # output overlaps an input
    assert strided(BNHD, q=Q, k=Q + 128, v=Q + 256) not in ok  # inputs may share memory
    assert strided(BNHD, B=0, q=None, k=None, v=None, o=None, lse=None) == ea.ATTN_OK
    assert ea.lib().attn_fwd_strided(Q, K, V, O, L, None, 2, 4, 2, 100, 64, 1, 0.125, 1,
                                     None) == ea.ATTN_ERR_INVALID_ARG  # no strides


@reaches_device
def test_strided_backward_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)

    def sb(strides, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, B=2, Hq=4, Hkv=2,
                 N=100, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_bwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                                   a["dk"], a["dv"], a["ws"], strides, a["B"], a["Hq"], a["Hkv"],
                                   a["N"], a["d"], a["causal"], a["scale"], a["dtype"], None)

    assert sb(BNHD) not in ok
    bad = list(BNHD)
    bad[5] = 63
    assert sb(bad) == ea.ATTN_ERR_INVALID_ARG
    assert sb(BNHD, dq=Q) == ea.ATTN_ERR_INVALID_ARG  # a gradient over an input
    assert sb(BNHD, dk=DQ + 128) not in ok  # interleaved gradient slices are allowed
    assert sb(BNHD, dk=WS + 64) == ea.ATTN_ERR_INVALID_ARG  # a gradient over the workspace
    assert sb(BNHD, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    # token-major strides at d = 256: [B, N, H, 256]
    b256 = [100 * 4 * 256, 256, 4 * 256, 100 * 2 * 256, 256, 2 * 256, 100 * 4 * 256, 256, 4 * 256]
    assert sb(b256, d=256) not in ok


@reaches_device
def test_varlen_backward_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)

    def vb(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, cu=CU, nseq=3,
                 maxlen=500, Hq=4, Hkv=2, T=1000, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                                  a["dk"], a["dv"], a["ws"], a["cu"], a["nseq"], a["maxlen"],
                                  a["Hq"], a["Hkv"], a["T"], a["d"], a["causal"], a["scale"],
                                  a["dtype"], None)

    assert vb() not in ok
    for kw in (dict(cu=None), dict(cu=CU + 2), dict(maxlen=1001), dict(nseq=-1), dict(dq=Q),
               dict(ws=None), dict(cu=DQ + 16), dict(Hq=6, Hkv=4)):
        assert vb(**kw) == ea.ATTN_ERR_INVALID_ARG, kw
    assert vb(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert vb(d=256) not in ok
    none = dict(q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None, dv=None,
                ws=None, cu=None)
    assert vb(nseq=0, **none) == ea.ATTN_OK


@reaches_device
def test_varlen_strided_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    T, H, Hkv, d = 1000, 4, 2, 64
    tm = [d, H * d, d, Hkv * d, d, H * d]  # token-major [T, H, d] for every tensor

    def fs(strides, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, cu=CU, nseq=3, maxlen=500, Hq=H, Hkv=Hkv, T=T, d=d,
                 causal=1, scale=0.125, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_fwd_varlen_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"],
                                          strides, a["nseq"], a["maxlen"], a["Hq"], a["Hkv"],
                                          a["T"], a["d"], a["causal"], a["scale"], a["dtype"],
                                          None)

    def bs(strides, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, cu=CU, nseq=3,
                 maxlen=500, Hq=H, Hkv=Hkv, T=T, d=d, causal=1, scale=0.125, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_bwd_varlen_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"],
                                          a["dq"], a["dk"], a["dv"], a["ws"], a["cu"], strides,
                                          a["nseq"], a["maxlen"], a["Hq"], a["Hkv"], a["T"],
                                          a["d"], a["causal"], a["scale"], a["dtype"], None)

    assert fs(tm) not in ok and bs(tm) not in ok
    for bad in ([d, 32, d, Hkv * d, d, H * d],      # token stride below d
                [d, H * d + 4, d, Hkv * d, d, H * d],  # not a multiple of 8
                [-8, H * d, d, Hkv * d, d, H * d],   # negative
                [d, 1 << 22, d, Hkv * d, d, H * d]):  # rows past 2^31 bytes
        assert fs(bad) == ea.ATTN_ERR_INVALID_ARG, bad
        assert bs(bad) == ea.ATTN_ERR_INVALID_ARG, bad
    assert ea.lib().attn_fwd_varlen_strided(Q, K, V, O, L, CU, None, 3, 500, H, Hkv, T, d, 1,
                                            0.125, 1, None) == ea.ATTN_ERR_INVALID_ARG
    assert fs(tm, o=Q + 128) == ea.ATTN_ERR_INVALID_ARG  # output over an input
    assert fs(tm, q=Q, k=Q + 128, v=Q + 256) not in ok  # inputs may share memory
    assert bs(tm, dk=DQ + 128) not in ok  # interleaved gradient slices are allowed
    assert bs(tm, dk=WS + 64) == ea.ATTN_ERR_INVALID_ARG  # a gradient over the workspace
    assert bs(tm, dq=Q) == ea.ATTN_ERR_INVALID_ARG  # a gradient over an input
    assert bs(tm, cu=DQ + 16) == ea.ATTN_ERR_INVALID_ARG  # offsets inside a gradient
    assert fs(tm, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert fs(tm, nseq=0, q=None, k=None, v=None, o=None, lse=None, cu=None) == ea.ATTN_OK


@reaches_device
def test_splitkv_strided_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 3, 1000, 128
    # q, o token-major [B, Nq, Hq, d]; cache token-major [B, Nk, Hkv, d]
    tm = [Nq * Hq * d, d, Hq * d, Nk * Hkv * d, d, Hkv * d, Nq * Hq * d, d, Hq * d]

    def ss(strides, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, ws=WS, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                 causal=1, scale=0.125, ns=0, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_fwd_splitkv_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"],
                                           strides, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                                           a["d"], a["causal"], a["scale"], a["ns"], a["dtype"],
                                           None)

    assert ss(tm) not in ok
    for i, val in ((2, 64), (5, 100), (4, -8), (1, 1 << 30)):  # row < d, not x8, negative, group
        bad = list(tm)
        bad[i] = val
        assert ss(bad) == ea.ATTN_ERR_INVALID_ARG, (i, val)
    assert ea.lib().attn_fwd_splitkv_strided(Q, K, V, O, L, WS, None, B, Hq, Hkv, Nq, Nk, d, 1,
                                             0.125, 0, 1, None) == ea.ATTN_ERR_INVALID_ARG
    assert ss(tm, o=Q + 64) == ea.ATTN_ERR_INVALID_ARG  # output over an input
    assert ss(tm, ws=O + 64) == ea.ATTN_ERR_INVALID_ARG  # workspace over the output
    assert ss(tm, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    assert ss(tm, Nk=0) not in ok  # no keys: K and V are not read
    assert ss(tm, B=0, q=None, k=None, v=None, o=None, lse=None, ws=None) == ea.ATTN_OK


@reaches_device
def test_blocksparse_strided_validation():
    ok = (ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED)
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 64
    tm = [N * Hq * d, d, Hq * d, N * Hkv * d, d, Hkv * d, N * Hq * d, d, Hq * d]
    M = 0x10000000 * 13  # the mask

    def bs(strides, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, m=M, mh=1, ws=WS, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d,
                 causal=1, scale=0.125, dtype=ea.ATTN_BF16)
        a.update(kw)
        return ea.attn_fwd_blocksparse_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["m"],
                                               a["mh"], a["ws"], strides, a["B"], a["Hq"],
                                               a["Hkv"], a["N"], a["d"], a["causal"], a["scale"],
                                               a["dtype"], None)

    assert bs(tm) not in ok
    bad = list(tm)
    bad[2] = 32  # row stride below d
    assert bs(bad) == ea.ATTN_ERR_INVALID_ARG
    assert ea.lib().attn_fwd_blocksparse_strided(Q, K, V, O, L, M, 1, WS, None, B, Hq, Hkv, N, d,
                                                 1, 0.125, 1, None) == ea.ATTN_ERR_INVALID_ARG
    assert bs(tm, o=Q + 64) == ea.ATTN_ERR_INVALID_ARG
    assert bs(tm, m=O + 16) == ea.ATTN_ERR_INVALID_ARG  # mask inside the output
    assert bs(tm, mh=3) == ea.ATTN_ERR_INVALID_ARG
    assert bs(tm, dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED


def test_grid_limit_is_rejected():
    # A dispatch counts its work-items (workgroups x threads) in 32 bits.  The
    # batched checks allow up to max(8, d/8) threads per query row padded to
    # 128 rows: at d = 64, B*Hq*round_up(N, 128) < 2^29.
    assert fwd(B=1 << 20, Hq=16, Hkv=16, N=1 << 12) == ea.ATTN_ERR_UNSUPPORTED
    assert fwd(B=1 << 12, Hq=16, Hkv=16, N=8192) == ea.ATTN_ERR_UNSUPPORTED
    assert fwd(B=1 << 12, Hq=16, Hkv=16, N=8192 - 127) == ea.ATTN_ERR_UNSUPPORTED  # pads to 8192
    # one row block fewer fits: the shape passes, and the fake buffers (each
    # tens of GB) then overlap, which validation rejects
    assert fwd(B=1 << 12, Hq=16, Hkv=16, N=8192 - 128) == ea.ATTN_ERR_INVALID_ARG
    # d = 256: 32 threads per row (the statistics kernel of the backward)
    assert bwd(B=1 << 10, Hq=16, Hkv=16, N=8192, d=256) == ea.ATTN_ERR_UNSUPPORTED
    assert bwd(B=1 << 10, Hq=16, Hkv=16, N=8192 - 128, d=256) == ea.ATTN_ERR_INVALID_ARG


def vbwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, cu=CU, nseq=3,
             maxlen=500, Hq=4, Hkv=2, T=1000, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16)
    a.update(kw)
    return ea.attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                              a["dk"], a["dv"], a["ws"], a["cu"], a["nseq"], a["maxlen"], a["Hq"],
                              a["Hkv"], a["T"], a["d"], a["causal"], a["scale"], a["dtype"], None)


def test_varlen_grid_limit_is_rejected():
    # The packed grids are (sequence, head, 128-row block of the longest
    # sequence) with two threads per padded row; the header allows any
    # max_seqlen up to T, so the product can pass 2^32 work-items (and 2^32
    # workgroups) with every size individually valid.
    for call in (varlen, vbwd):
        # 1024 documents, 32 heads, longest 2^18 tokens: 2^26 workgroups, 2^34 work-items
        assert call(nseq=1024, Hq=32, Hkv=8, maxlen=1 << 18, T=1 << 18) == ea.ATTN_ERR_UNSUPPORTED
        # 2^14 + 1 documents, 64 heads, longest 2^20: more than 2^32 workgroups
        assert call(nseq=(1 << 14) + 1, Hq=64, Hkv=8, maxlen=1 << 20,
                    T=1 << 20) == ea.ATTN_ERR_UNSUPPORTED
        # 2^23 padded rows x 2 threads fit; the fake buffers then overlap
        assert call(nseq=512, Hq=16, Hkv=8, maxlen=1024, T=1 << 18) == ea.ATTN_ERR_INVALID_ARG


def test_splitkv_grid_limit_is_rejected():
    # the merge runs up to 64 threads per output row: B*Hq*Nq*64 < 2^32
    assert split(B=1 << 12, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 10, Nk=64) == ea.ATTN_ERR_UNSUPPORTED


# ---------------------------------------------------------------- clock probe
def probe(**kw):
    a = dict(out=Q, nwg=8, ticks=1000)
    a.update(kw)
    return ea.attn_probe_clock(a["out"], a["nwg"], a["ticks"], None)


PROBE_INVALID = [dict(out=None), dict(out=Q + 4), dict(nwg=0), dict(nwg=65), dict(ticks=0),
                 dict(ticks=200000001)]


@pytest.mark.parametrize("kw", PROBE_INVALID, ids=[str(k) for k in PROBE_INVALID])
def test_probe_clock_rejects_bad_arguments(kw):
    assert probe(**kw) == ea.ATTN_ERR_INVALID_ARG


@reaches_device
def test_probe_clock_passes_validation():
    assert probe() == ea.ATTN_ERR_HIP  # no GPU here: stops at the device check
    assert probe(nwg=64, ticks=200000000) == ea.ATTN_ERR_HIP


# ---------------------------------------------------------------- no-allocation backward
def noalloc(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=2, Hq=4, Hkv=2, N=100,
             d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16)
    a.update(kw)
    return ea.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                               a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                               a["causal"], a["scale"], a["dtype"], None)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == ea.ATTN_NOALLOC_SCRATCH_BYTES


NOALLOC_INVALID = [dict(q=None), dict(dout=None), dict(dq=None), dict(dk=DK + 8), dict(dq=DO),
                   dict(dk=DV), dict(dv=DK + 1024), dict(Hq=3, Hkv=2), dict(causal=5),
                   dict(scale=float("nan"))]


@pytest.mark.parametrize("kw", NOALLOC_INVALID, ids=[str(k) for k in NOALLOC_INVALID])
def test_noalloc_rejects_bad_arguments(kw):
    assert noalloc(**kw) == ea.ATTN_ERR_INVALID_ARG


def test_noalloc_sizes():
    # empty problems need no pointers
    none = dict(q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None, dv=None)
    assert noalloc(B=0, **none) == ea.ATTN_OK
    assert noalloc(dtype=ea.ATTN_F32) == ea.ATTN_ERR_UNSUPPORTED
    # the workspace attn_bwd would need must fit the static scratch (32 MiB):
    # statistics of B*Hq*Np rows at 8 bytes each, so 4M rows fit exactly ...
    cap = ea.ATTN_NOALLOC_SCRATCH_BYTES
    assert ea.attn_bwd_workspace_bytes(64, 16, 16, 4096, 64, ea.ATTN_BF16) == cap
    assert noalloc(B=64, Hq=16, Hkv=16, N=4096 + 1) == ea.ATTN_ERR_UNSUPPORTED
    # ... and a grouped-query split whose partial sums do not fit is refused
    # (B=1 Hq=32 Hkv=8 N=2048 d=128 splits 4 ways: 64.5 MiB of workspace)
    assert ea.attn_bwd_workspace_bytes(1, 32, 8, 2048, 128, ea.ATTN_BF16) > cap
    assert noalloc(B=1, Hq=32, Hkv=8, N=2048, d=128) == ea.ATTN_ERR_UNSUPPORTED


@reaches_device
def test_noalloc_passes_validation():
    assert noalloc() == ea.ATTN_ERR_HIP  # no GPU here: stops at the device check
    assert noalloc(B=64, Hq=16, Hkv=16, N=4096) == ea.ATTN_ERR_INVALID_ARG  # fake buffers overlap


def test_stride_comparison_ignores_size_one_dimensions():
    """The binding compares the strides of tensors that must share a layout
    only over dimensions of more than one element: a size-1 dimension's stride
    is never used."""
    import torch

    a = torch.empty(2, 5, 1, 8).transpose(1, 2)   # [2, 1, 5, 8], token-major
    b = torch.empty(2, 1, 5, 8)                   # dense: other size-1 stride
    assert a.stride() != b.stride()
    assert ea._same_strides(a, b)
    c = torch.empty(2, 3, 5, 8).transpose(1, 2).contiguous().transpose(1, 2)  # [2, 5, 3, 8] -> view
    assert not ea._same_strides(c, torch.empty(2, 3, 5, 8))  # real layout difference
    assert not ea._same_strides(b, torch.empty(2, 1, 6, 8))  # shapes differ
