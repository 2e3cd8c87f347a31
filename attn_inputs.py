"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and names the workload shapes; it holds
none of the attention arithmetic.  Tests, the smoke check and the benchmark
use it to feed the same values to the HIP library and to the fp64 oracle.

Recipe: one torch CPU ``Generator`` seeded per workload; draw order Q, K, V,
dO; every tensor iid N(0, 1) in fp32; for bf16 (fp16) workloads each value is
rounded to bf16 (fp16) round-to-nearest-even, and both sides consume the
rounded values.
A query multiplier (a power of two, so exact) scales Q to produce extreme
logits.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str  # "fp32" or "bf16"
    q_mult: float = 1.0
    backward: bool = False
    seed: int = 0

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the task description, in order.
WORKLOADS = {
    1: Workload("single_head_fp32_B1_H1_N128_d64", 1, 1, 1, 128, 64, False, "fp32", seed=1),
    2: Workload("noncausal_bf16_B8_H16_N1024_d64", 8, 16, 16, 1024, 64, False, "bf16", seed=2),
    3: Workload("causal_bf16_B4_H32_N4000_d128", 4, 32, 32, 4000, 128, True, "bf16", seed=3),
    4: Workload("causal_gqa_bf16_B1_Hq32_Hkv8_N16384_d128_q8", 1, 32, 8, 16384, 128, True,
                "bf16", q_mult=8.0, seed=4),
    5: Workload("causal_fwd_bwd_bf16_B8_H16_N2048_d64", 8, 16, 16, 2048, 64, True, "bf16",
                backward=True, seed=5),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[name]


def make(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
         q_mult: float = 1.0, with_dout: bool = False):
    """Draw (q, k, v[, dout]) as CPU tensors of the workload dtype, [B, H, N, d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    dout = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32) if with_dout else None
    td = torch_dtype(dtype)
    q, k, v = q.to(td), k.to(td), v.to(td)
    if q_mult != 1.0:
        q = q * q_mult  # power of two: exact in bf16 and fp32
    if dout is not None:
        dout = dout.to(td)
    return (q, k, v, dout) if with_dout else (q, k, v)


def make_workload(w: Workload, with_dout: bool | None = None):
    wd = w.backward if with_dout is None else with_dout
    return make(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, w.seed, w.q_mult, wd)


# Few queries against a long key/value cache (decode and chunked append), for
# the split-K/V forward.  Same recipe; Q is [B, Hq, Nq, d], K/V [B, Hkv, Nk, d].
@dataclass(frozen=True)
class CacheWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int = 0


CACHE_WORKLOADS = {
    "decode": CacheWorkload("decode_bf16_B8_Hq32_Hkv8_Nq1_Nk32768_d128", 8, 32, 8, 1, 32768, 128,
                            True, seed=11),
    "append": CacheWorkload("append_causal_bf16_B4_Hq32_Hkv8_Nq64_Nk16384_d128", 4, 32, 8, 64,
                            16384, 128, True, seed=12),
}


def make_cache(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int = 0,
               q_mult: float = 1.0, dtype: str = "bf16"):
    """Draw (q [B,Hq,Nq,d], k [B,Hkv,Nk,d], v [B,Hkv,Nk,d]) as CPU tensors (bf16 or fp16)."""
    td = torch_dtype(dtype)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32).to(td)
    k = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32).to(td)
    v = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32).to(td)
    if q_mult != 1.0:
        q = q * q_mult  # power of two: exact
    return q, k, v


def make_cache_workload(w: CacheWorkload):
    return make_cache(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed)


# Block-sparse forward: a block mask over tiles of 128 queries x 64 keys.  The
# mask is input data (which tiles exist), drawn here like the tensors.
@dataclass(frozen=True)
class SparseWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    window: int      # keys before each query block that it always sees
    globals_: int    # leading key tiles every query block sees
    stride: int      # every stride-th key tile is also present
    density: float   # extra random tiles, per head
    seed: int = 0


SPARSE_WORKLOADS = {
    "local_global": SparseWorkload("blocksparse_local_global_bf16_B1_Hq32_Hkv8_N16384_d128", 1, 32,
                                   8, 16384, 128, True, window=1024, globals_=2, stride=16,
                                   density=0.05, seed=13),
}


def sparse_mask(w: SparseWorkload, block_q: int = 128, block_k: int = 64):
    """uint8 numpy mask [Hq, ceil(N/block_q), ceil(N/block_k)]: a local band of
    `window` keys ending at each query block, `globals_` leading key tiles,
    every `stride`-th key tile, and random tiles of the given density (seeded,
    different per head)."""
    import numpy as np

    nbq, nbk = -(-w.N // block_q), -(-w.N // block_k)
    qb = np.arange(nbq)[:, None]
    t = np.arange(nbk)[None, :]
    q_end = np.minimum((qb + 1) * block_q, w.N)  # one past the block's last query
    local = (t * block_k < q_end) & ((t + 1) * block_k > q_end - w.window)
    base = local | (t < w.globals_) | (t % w.stride == 0)
    r = np.random.default_rng(w.seed)
    rand = r.random((w.Hq, nbq, nbk)) < w.density
    return (base[None] | rand).astype(np.uint8)


# Packed variable-length batches: documents of different lengths laid end to
# end, Q [Hq, T, d] and K/V [Hkv, T, d], with token offsets cu_seqlens.
@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    Hq: int
    Hkv: int
    T: int
    d: int
    causal: bool
    min_len: int
    max_len: int
    seed: int = 0


VARLEN_WORKLOADS = {
    "docs": VarlenWorkload("varlen_docs_bf16_Hq32_Hkv8_T16384_d128", 32, 8, 16384, 128, True,
                           min_len=32, max_len=4096, seed=14),
}


def varlen_lengths(w: VarlenWorkload):
    """Document lengths summing to w.T: log-uniform in [min_len, max_len]
    (seeded), the last one cut to fit."""
    import numpy as np

    r = np.random.default_rng(w.seed)
    lengths, total = [], 0
    while total < w.T:
        n = int(round(np.exp(r.uniform(np.log(w.min_len), np.log(w.max_len)))))
        n = min(n, w.T - total)
        lengths.append(n)
        total += n
    return lengths


def make_varlen(Hq: int, Hkv: int, lengths, d: int, seed: int = 0, dtype: str = "bf16"):
    """(q [Hq,T,d], k [Hkv,T,d], v [Hkv,T,d]) in bf16 or fp16 and int32 offsets
    cu_seqlens for sequences of the given lengths, T = sum(lengths)."""
    import numpy as np

    td = torch_dtype(dtype)
    T = int(sum(lengths))
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((Hq, T, d), generator=g, dtype=torch.float32).to(td)
    k = torch.randn((Hkv, T, d), generator=g, dtype=torch.float32).to(td)
    v = torch.randn((Hkv, T, d), generator=g, dtype=torch.float32).to(td)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return q, k, v, cu


def make_long_filler(M: int, T: int, d: int, pool: int = 4096, seed: int = 0,
                     dtype: str = "bf16", with_dout: bool = False):
    """Pieces of the maximum-length inputs: N = M + T rows of one head, whose
    first M keys are zero and whose last T keys are drawn; query, value and
    upstream-gradient rows repeat with a period of `pool` rows.

    Returns (qpool [pool, d], vpool [pool, d], ktail [T, d], dopool [pool, d]
    or None) rounded to the 16-bit type, on the CPU.  Row i of Q is
    qpool[i % pool], of V vpool[i % pool], of dO dopool[i % pool]; key i is 0
    for i < M and ktail[i - M] after.  Draw order: Q pool, key tail, V pool,
    dO pool.
    """
    g = torch.Generator().manual_seed(seed)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    qpool = torch.randn((pool, d), generator=g).to(tdt)
    ktail = torch.randn((T, d), generator=g).to(tdt)
    vpool = torch.randn((pool, d), generator=g).to(tdt)
    dopool = torch.randn((pool, d), generator=g).to(tdt) if with_dout else None
    return qpool, vpool, ktail, dopool
