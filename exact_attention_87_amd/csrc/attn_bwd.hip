// Backward pass of exact attention for gfx950, with recomputation.
//
// Method: the forward keeps only the per-row logsumexp; the backward
// recomputes the probabilities tile by tile from Q, K and that statistic
// instead of reading an N x N matrix ("FlashAttention" paper story,
// backward/recomputation paragraph; the pages do not print the gradient
// formulas, so the kernels evaluate the textbook gradient):
//   P = exp(scale Q K^T - LSE)      dV = P^T dO       dP = dO V^T
//   D_i = dO_i . O_i                dS = P o (dP - D)
//   dQ = scale dS K                 dK = scale dS^T Q
//
// Three kernels, all deterministic (no atomics):
//   pre:  D_i = dO_i . O_i into the caller's workspace.
//   dkdv: one workgroup per (batch, kv head, block of 128 keys); each wave
//         keeps its 32 keys' K and V as matrix-core operands in registers and
//         accumulates dK^T, dV^T over every query tile of every query head of
//         the group (so grouped-query heads are summed on chip).
//   dq:   one workgroup per (batch, query head, block of 128 queries); the
//         forward's tiling, with dQ^T accumulated over the key tiles.
// Probabilities use base 2: P = 2^(s*c - LSE*log2 e), c = |scale| log2 e.
// A negative scale is folded into Q's sign bit when Q is loaded.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

constexpr float kTiny = 1.17549435e-38f;  // smallest normal fp32

// ---------------------------------------------------------------- D = rowsum(dO o O)
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                      const __bf16* __restrict__ dO,
                                                      float* __restrict__ Dsum, int64_t rows) {
  constexpr int TPR = D / 8;  // lanes per row, 16 bytes each
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + row * D + part * 8);
    const u32x4 b = *(const u32x4*)(dO + row * D + part * 8);
    const bf16x8 av = bitcast<bf16x8>(a), bv = bitcast<bf16x8>(b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)av[e], (float)bv[e], acc);
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && part == 0) Dsum[row] = acc;
}

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int Hq, int Hkv, int N, int nkb, float c,
    float kscale, uint32_t qsign) {
  constexpr int NW = 4;
  constexpr int BKV = 32 * NW;  // keys per workgroup
  constexpr int BQ = 64;        // queries per tile
  constexpr int NCH = D / 8;
  constexpr int TILEB = BQ * D * 2;
  constexpr int RPP = 256 / NCH;
  constexpr int PASSES = BQ / RPP;
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;
  constexpr int BUFB = 2 * TILEB + 2 * BQ * 4;  // Q tile | dO tile | lse2 | dsum

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int BG = gridDim.x / nkb;
  const int kblk = blockIdx.x / BG;  // causal: low key blocks carry the most work
  const int bg = blockIdx.x % BG;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int group = Hq / Hkv;
  const int64_t kvoff = (int64_t)bg * N * D;
  const int key0 = kblk * BKV + w * 32;  // first key of this wave
  const int krow = key0 + l32;           // key owned by this lane

  // K^T and V^T operands of this wave's 32 keys, resident.
  bf16x8 kreg[NQC], vreg[NQC];
  {
    const bool ok = krow < N;
    const int64_t off = kvoff + (int64_t)(ok ? krow : 0) * D + hf * 8;
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      u32x4 kv = *(const u32x4*)(K + off + cc * 16);
      u32x4 vv = *(const u32x4*)(V + off + cc * 16);
      if (!ok) {
        kv = u32x4{0, 0, 0, 0};
        vv = u32x4{0, 0, 0, 0};
      }
      kreg[cc] = bitcast<bf16x8>(kv);
      vreg[cc] = bitcast<bf16x8>(vv);
    }
  }
  f32x16 dkacc[NMB], dvacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (kblk * BKV) / BQ : 0;
  const int per_head = nqt - qt0;
  const int iters = per_head > 0 ? group * per_head : 0;

  const int lrow = tid / NCH;
  const int lch = tid % NCH;
  u32x4 qst[PASSES], dost[PASSES];
  float stat = 0.f;  // threads 0..63: lse2 of row tid; 64..127: dsum of row tid-64
  auto gload = [&](int it) {
    const int hq = g * group + it / per_head;
    const int qt = qt0 + it % per_head;
    const int64_t qoff = (int64_t)(b * Hq + hq) * N;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = qt * BQ + p * RPP + lrow;
      const bool ok = row < N;
      const int64_t off = (qoff + (ok ? row : 0)) * D + lch * 8;
      u32x4 qv = *(const u32x4*)(Q + off);
      u32x4 dv = *(const u32x4*)(dO + off);
      if (!ok) {
        qv = u32x4{0, 0, 0, 0};
        dv = u32x4{0, 0, 0, 0};
      }
      qst[p] = qv ^ qsign;
      dost[p] = dv;
    }
    if (tid < 2 * BQ) {
      const int row = qt * BQ + (tid & (BQ - 1));
      const bool ok = row < N;
      if (tid < BQ)
        stat = ok ? LSE[qoff + row] * kLog2e : __builtin_inff();
      else
        stat = ok ? Dsum[qoff + row] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
    char* base = smem + buf * BUFB;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int off = tile_off<D>(p * RPP + lrow, lch);
      lds_write16(base + off, qst[p]);
      lds_write16(base + TILEB + off, dost[p]);
    }
    if (tid < 2 * BQ) ((float*)(base + 2 * TILEB))[tid] = stat;
  };

  if (iters > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    const int buf = it & 1;
    if (it + 1 < iters) gload(it + 1);
    const int qt = qt0 + it % per_head;
    const char* qtile = smem + buf * BUFB;
    const char* dotile = qtile + TILEB;
    const float* lse2 = (const float*)(qtile + 2 * TILEB);
    const float* dsum = lse2 + BQ;
#pragma unroll
    for (int qs = 0; qs < BQ / 32; ++qs) {
      const int qbase = qs * 32;
      const int qfirst = qt * BQ + qbase;
      if (CAUSAL && qfirst + 31 < key0) continue;  // every query precedes every key
      if (qfirst >= N) continue;
      // S = Q K^T and dP = dO V^T (rows: queries, columns: this wave's keys)
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NQC; ++cc) {
        const int off = tile_off<D>(qbase + l32, 2 * cc + hf);
        sacc = mfma32(bitcast<bf16x8>(lds_read16(qtile + off)), kreg[cc], sacc);
        pacc = mfma32(bitcast<bf16x8>(lds_read16(dotile + off)), vreg[cc], pacc);
      }
      const bool need_mask = CAUSAL && (key0 + 31 > qfirst);
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int q4 = qbase + 8 * rg + 4 * hf;
        const f32x4 l4 = *(const f32x4*)(lse2 + q4);
        const f32x4 d4 = *(const f32x4*)(dsum + q4);
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float p = fast_exp2(__builtin_fmaf(sacc[r], c, -l4[e]));
          if (need_mask && krow > qt * BQ + q4 + e) p = 0.f;
          pv[e] = p;
          dsv[e] = p * (pacc[r] - d4[e]);
        }
        pk[2 * rg] = pack_bf16(pv[0], pv[1]);
        pk[2 * rg + 1] = pack_bf16(pv[2], pv[3]);
        dsk[2 * rg] = pack_bf16(dsv[0], dsv[1]);
        dsk[2 * rg + 1] = pack_bf16(dsv[2], dsv[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 queries)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp) {
        const bf16x8 pb = bitcast<bf16x8>(u32x4{pk[4 * cp], pk[4 * cp + 1], pk[4 * cp + 2], pk[4 * cp + 3]});
        const bf16x8 sb =
            bitcast<bf16x8>(u32x4{dsk[4 * cp], dsk[4 * cp + 1], dsk[4 * cp + 2], dsk[4 * cp + 3]});
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const int o0 = tr_off<D>(lane, qbase + 16 * cp, 32 * mb, 0);
          const int o1 = tr_off<D>(lane, qbase + 16 * cp, 32 * mb, 1);
          const u32x2 a0 = lds_read_tr(dotile + o0), a1 = lds_read_tr(dotile + o1);
          dvacc[mb] = mfma32(bitcast<bf16x8>(u32x4{a0[0], a0[1], a1[0], a1[1]}), pb, dvacc[mb]);
          const u32x2 b0 = lds_read_tr(qtile + o0), b1 = lds_read_tr(qtile + o1);
          dkacc[mb] = mfma32(bitcast<bf16x8>(u32x4{b0[0], b0[1], b1[0], b1[1]}), sb, dkacc[mb]);
        }
      }
    }
    if (it + 1 < iters) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- store dK = kscale * dK^T^T, dV (lane: key krow; element r: feature)
  if (krow < N) {
    __bf16* dkp = dK + kvoff + (int64_t)krow * D;
    __bf16* dvp = dV + kvoff + (int64_t)krow * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        u32x2 kv, vv;
        kv[0] = pack_bf16(dkacc[mb][4 * rg] * kscale, dkacc[mb][4 * rg + 1] * kscale);
        kv[1] = pack_bf16(dkacc[mb][4 * rg + 2] * kscale, dkacc[mb][4 * rg + 3] * kscale);
        vv[0] = pack_bf16(dvacc[mb][4 * rg], dvacc[mb][4 * rg + 1]);
        vv[1] = pack_bf16(dvacc[mb][4 * rg + 2], dvacc[mb][4 * rg + 3]);
        *(u32x2*)(dkp + d0) = kv;
        *(u32x2*)(dvp + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    __bf16* __restrict__ dQ, int Hq, int Hkv, int N, int nqb, float c, float qscale,
    uint32_t qsign) {
  constexpr int NW = 4;
  constexpr int BR = 32 * NW;
  constexpr int BC = 64;
  constexpr int NCH = D / 8;
  constexpr int TILEB = BC * D * 2;
  constexpr int RPP = 256 / NCH;
  constexpr int PASSES = BC / RPP;
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem[];  // [2][K tile | V tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int BH = gridDim.x / nqb;
  const int id = blockIdx.x;
  const int qb = CAUSAL ? (nqb - 1 - id / BH) : (id / BH);
  const int bh = id % BH;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const int64_t qoff = (int64_t)bh * N * D;
  const int64_t kvoff = (int64_t)(b * Hkv + g) * N * D;
  const int q0 = qb * BR + w * 32;
  const int qrow = q0 + l32;
  const bool qok = qrow < N;

  bf16x8 qreg[NQC], doreg[NQC];
  {
    const int64_t off = qoff + (int64_t)(qok ? qrow : 0) * D + hf * 8;
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      u32x4 qv = *(const u32x4*)(Q + off + cc * 16);
      u32x4 dv = *(const u32x4*)(dO + off + cc * 16);
      if (!qok) {
        qv = u32x4{0, 0, 0, 0};
        dv = u32x4{0, 0, 0, 0};
      }
      qreg[cc] = bitcast<bf16x8>(qv ^ qsign);
      doreg[cc] = bitcast<bf16x8>(dv);
    }
  }
  const float lse2 = qok ? LSE[(int64_t)bh * N + qrow] * kLog2e : __builtin_inff();
  const float dsum = qok ? Dsum[(int64_t)bh * N + qrow] : 0.f;

  const int ntiles_all = (N + BC - 1) / BC;
  int ntiles = ntiles_all, wtiles = ntiles_all;
  if (CAUSAL) {
    ntiles = min(ntiles_all, (qb * BR + BR - 1) / BC + 1);
    wtiles = min(ntiles, (q0 + 31) / BC + 1);
  }

  const int lrow = tid / NCH;
  const int lch = tid % NCH;
  u32x4 kst[PASSES], vst[PASSES];
  auto gload = [&](int j) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = j * BC + p * RPP + lrow;
      const bool ok = row < N;
      const int64_t off = kvoff + (int64_t)(ok ? row : 0) * D + lch * 8;
      u32x4 kv = *(const u32x4*)(K + off);
      u32x4 vv = *(const u32x4*)(V + off);
      if (!ok) {
        kv = u32x4{0, 0, 0, 0};
        vv = u32x4{0, 0, 0, 0};
      }
      kst[p] = kv;
      vst[p] = vv;
    }
  };
  auto swrite = [&](int buf) {
    char* kb = smem + buf * 2 * TILEB;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int off = tile_off<D>(p * RPP + lrow, lch);
      lds_write16(kb + off, kst[p]);
      lds_write16(kb + TILEB + off, vst[p]);
    }
  };

  f32x16 dqacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dqacc[mb] = f32x16{};

  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    if (j < wtiles && q0 < N) {
      const char* kt = smem + buf * 2 * TILEB;
      const char* vt = kt + TILEB;
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        sacc[kbk] = f32x16{};
        pacc[kbk] = f32x16{};
        const int key = kbk * 32 + l32;
#pragma unroll
        for (int cc = 0; cc < NQC; ++cc) {
          const int off = tile_off<D>(key, 2 * cc + hf);
          sacc[kbk] = mfma32(bitcast<bf16x8>(lds_read16(kt + off)), qreg[cc], sacc[kbk]);
          pacc[kbk] = mfma32(bitcast<bf16x8>(lds_read16(vt + off)), doreg[cc], pacc[kbk]);
        }
      }
      const int k0 = j * BC;
      const bool need_mask = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > q0));
      uint32_t dsk[2][8];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float ds[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float p = fast_exp2(__builtin_fmaf(sacc[kbk][r + e], c, -lse2));
            if (need_mask) {
              const int key = k0 + kbk * 32 + acc_row(r + e, hf);
              if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
            }
            ds[e] = p * (pacc[kbk][r + e] - dsum);
          }
          dsk[kbk][r >> 1] = pack_bf16(ds[0], ds[1]);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int cp = 0; cp < 2; ++cp) {
            const int kbase = kbk * 32 + cp * 16;
            const u32x2 lo = lds_read_tr(kt + tr_off<D>(lane, kbase, mb * 32, 0));
            const u32x2 hi = lds_read_tr(kt + tr_off<D>(lane, kbase, mb * 32, 1));
            const bf16x8 a = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
            const bf16x8 sb = bitcast<bf16x8>(u32x4{dsk[kbk][4 * cp], dsk[kbk][4 * cp + 1],
                                                    dsk[kbk][4 * cp + 2], dsk[kbk][4 * cp + 3]});
            dqacc[mb] = mfma32(a, sb, dqacc[mb]);
          }
    }
    if (j + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  if (qok) {
    __bf16* dst = dQ + qoff + (int64_t)qrow * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        u32x2 v;
        v[0] = pack_bf16(dqacc[mb][4 * rg] * qscale, dqacc[mb][4 * rg + 1] * qscale);
        v[1] = pack_bf16(dqacc[mb][4 * rg + 2] * qscale, dqacc[mb][4 * rg + 3] * qscale);
        *(u32x2*)(dst + d0) = v;
      }
  }
}

// ---------------------------------------------------------------- launchers
struct BwdConsts {
  float c;         // |scale| log2(e), at least the smallest normal
  uint32_t qsign;  // sign bits XORed into Q when scale < 0
};

static BwdConsts bwd_consts(float scale) {
  float c = fabsf(scale) * kLog2e;
  if (!(c >= kTiny)) c = kTiny;  // scale 0: uniform probabilities, zero dQ/dK
  return BwdConsts{c, (scale < 0.f) ? 0x80008000u : 0u};
}

template <int D>
static hipError_t pre_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = (int64_t)a.B * a.Hq * a.N;
  const int64_t grid = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const __bf16*)a.o, (const __bf16*)a.dout, a.dsum, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t dkdv_t(const BwdArgs& a) {
  constexpr int BKV = 128, BQ = 64;
  const BwdConsts k = bwd_consts(a.scale);
  const int nkb = (a.N + BKV - 1) / BKV;
  const int64_t grid = (int64_t)nkb * a.B * a.Hkv;
  const size_t lds = 2 * (2 * BQ * D * 2 + 2 * BQ * 4);
  const hipError_t e = allow_lds(bwd_dkdv_kernel<D, CAUSAL>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), lds, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, a.lse, a.dsum, (__bf16*)a.dk, (__bf16*)a.dv, a.Hq,
                     a.Hkv, a.N, nkb, k.c, fabsf(a.scale), k.qsign);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t dq_t(const BwdArgs& a) {
  constexpr int BR = 128, BC = 64;
  const BwdConsts k = bwd_consts(a.scale);
  const int nqb = (a.N + BR - 1) / BR;
  const int64_t grid = (int64_t)nqb * a.B * a.Hq;
  const size_t lds = 2 * 2 * BC * D * 2;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), lds, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, a.lse, a.dsum, (__bf16*)a.dq, a.Hq, a.Hkv, a.N, nqb,
                     k.c, a.scale, k.qsign);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a) {
  if (!a.bf16) return hipErrorNotSupported;
  return a.d == 64 ? pre_t<64>(a) : pre_t<128>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  if (!a.bf16) return hipErrorNotSupported;
  if (a.d == 64) return a.causal ? dkdv_t<64, true>(a) : dkdv_t<64, false>(a);
  return a.causal ? dkdv_t<128, true>(a) : dkdv_t<128, false>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  if (!a.bf16) return hipErrorNotSupported;
  if (a.d == 64) return a.causal ? dq_t<64, true>(a) : dq_t<64, false>(a);
  return a.causal ? dq_t<128, true>(a) : dq_t<128, false>(a);
}

}  // namespace attn
