// Split-K/V forward for few queries against many keys (decode, append).
// The shape table of "FlashAttention：让精确注意力服从内存层次", section
// "训练与推理的形状不同", puts decoding at few queries against a long key
// history, bound first by key/value bandwidth; the "FlashAttention" paper
// story names FlashDecoding among the method's descendants.  Splitting the
// keys gives such shapes enough workgroups to stream K/V at HBM speed.
//
// The keys of every (batch, key/value head) are cut into splits; one
// workgroup computes, for one split, the attention of all the query rows of
// the head group (the group's query heads x Nq rows, contiguous in memory,
// so K and V are read once per group).  Each split leaves a normalised
// partial output O_s and its logsumexp LSE_s; a second kernel merges the
// splits with the pairwise (m, l, u) merge of the online softmax
// ("FlashAttention：让精确注意力服从内存层次", section "Online softmax"):
//   LSE = log sum_s e^{LSE_s},  O = sum_s e^{LSE_s - LSE} O_s.
// The causal mask is aligned to the bottom-right corner: query i of Nq sees
// keys j <= i + (Nk - Nq), the last query sees every key.
//
// The tile loop is the forward kernel's (direct global->LDS K/V tiles,
// S^T = K Q^T and O^T += V^T P^T on the 32x32x16 bf16 matrix cores, base-2
// online softmax); here the loop covers one split and the running maximum
// starts at -FLT_MAX, because a row may see no key at all inside a split.
#include "attn_device.h"
#include "attn_launch.h"

#include <float.h>

#include <algorithm>
#include <type_traits>

namespace attn {

// Two LDS stages at the highest occupancy the registers allow (3 waves per
// SIMD at d = 64, 2 at d = 128, 1 at d = 256): on decode, 2 stages at 2
// workgroups per CU (d = 128) beat 3 or 4 stages at 1 workgroup per CU by
// 5-10%; more resident workgroups, not deeper prefetch, keep more K/V bytes
// in flight.
template <int D>
struct SplitCfg {
  static constexpr int NW = 4;
  static constexpr int BR = 128;  // packed query rows per workgroup (32 per wave)
  static constexpr int BC = 64;   // keys per tile
  static constexpr int NBUF = 2;                           // LDS stages
  static constexpr int WPE = D == 64 ? 3 : D == 128 ? 2 : 1;  // waves per SIMD
  static_assert(NBUF >= 2 && NBUF <= 4, "stages");
  static constexpr int TILEB = BC * D * 2;
  static constexpr size_t LDS = (size_t)NBUF * 2 * TILEB;
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(SplitCfg<D>::WPE, SplitCfg<D>::WPE))) void fwd_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ Lpart, int Hq, int Hkv, int Nq, int Nk,
    int nrb, int nsplit, int split_len, int64_t rows_total, float c, uint32_t qsign, Layout lay) {
  using Cfg = SplitCfg<D>;
  using V8 = typename Elem<T>::v8;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, TILEB = Cfg::TILEB, NW = Cfg::NW, NBUF = Cfg::NBUF;
  constexpr int ROWB = D * 2;
  constexpr int PW = TILEB / 1024 / NW;
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem[];  // [NBUF][K tile | V tile]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Work map: row blocks of one split adjacent (they share the split's K/V).
  const int id = blockIdx.x;
  const int rb = id % nrb;
  const int t = id / nrb;
  const int split = t % nsplit;
  const int bg = t / nsplit;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int group = Hq / Hkv;
  const int R = group * Nq;                         // packed rows of the group
  const int64_t row0 = ((int64_t)b * Hq + (int64_t)g * group) * Nq;  // [B,Hq,Nq] index of row 0
  const int krs = lay.kv.r;  // key/value row stride (elements)
  const int64_t kvoff = b * lay.kv.b + g * lay.kv.h;
  const int r0 = rb * BR + w * 32;  // first packed row of this wave
  const int r = r0 + l32;           // packed row of this lane
  const int qi = r % Nq;            // its query index
  const int off = Nk - Nq;          // bottom-right diagonal offset

  // The group's query rows: head g*group + r/Nq, query r%Nq.  A padding row
  // (r >= R) reads row R-1 and is never stored.
  const int64_t qbase = b * lay.q.b + (int64_t)g * group * lay.q.h;
  const uint32_t qbytes =
      (uint32_t)(((int64_t)(group - 1) * lay.q.h + (int64_t)(Nq - 1) * lay.q.r + D) * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qbase, qbytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kvoff, slice_bytes(Nk, krs, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kvoff, slice_bytes(Nk, krs, D));

  V8 qreg[NQC];
  {
    const int rr = min(r, R - 1), hg = rr / Nq;
    const uint32_t qrow = (uint32_t)(hg * lay.q.h + (int64_t)(rr - hg * Nq) * lay.q.r);
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc)
      qreg[cc] = bitcast<V8>(buf_load16(rq, (qrow + cc * 16 + hf * 8) * 2) ^ qsign);
  }

  // Key range of the split.  With the causal mask the workgroup stops after
  // the last key any of its rows sees, and each wave after its own last key;
  // a wave holding no rows computes nothing (it still loads its share).
  const int kbeg = split * split_len;
  const int kend = min(Nk, kbeg + split_len);
  auto tiles_upto = [&](int ra, int rb_) {  // tiles of this split rows [ra, rb_] can see
    if (!CAUSAL) return (kend - kbeg + BC - 1) / BC;
    const int maxi = (ra / Nq != rb_ / Nq) ? Nq - 1 : rb_ % Nq;
    const int klim = min(maxi + off, kend - 1);  // last visible key of the range
    return klim < kbeg ? 0 : (klim - kbeg) / BC + 1;
  };
  const int wg0 = rb * BR;
  const int ntiles = tiles_upto(wg0, min(wg0 + BR - 1, R - 1));
  const int wtiles = r0 < R ? tiles_upto(r0, min(r0 + 31, R - 1)) : 0;

  uint32_t goff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int o = (w * PW + i) * 1024 + lane * 16;
    const int row = o / ROWB;
    const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
    goff[i] = (uint32_t)(row * krs + ch * 8) * 2;
  }
  auto issue = [&](int j) {
    char* kt = smem + (j % NBUF) * 2 * TILEB;
    const uint32_t tbase = (uint32_t)(kbeg + j * BC) * krs * 2;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      buf_load16_lds(rk, kt + (w * PW + i) * 1024, goff[i] + tbase);
      buf_load16_lds(rv, kt + TILEB + (w * PW + i) * 1024, goff[i] + tbase);
    }
  };

  // Wait until tile t has landed (tiles issued after it may stay in flight,
  // 2*PW loads each), then synchronise the workgroup.
  auto wait_next = [&](int t) {
    const int later = min(NBUF - 2, ntiles - 1 - t);
    if (NBUF >= 4 && later >= 2)
      wait_vm_barrier<(NBUF >= 4 ? 4 * PW : 0)>();
    else if (NBUF >= 3 && later >= 1)
      wait_vm_barrier<(NBUF >= 3 ? 2 * PW : 0)>();
    else
      wait_vm_barrier<0>();
  };

  int koff[NQC], voff[2][NMB];
#pragma unroll
  for (int cc = 0; cc < NQC; ++cc) koff[cc] = tile_off<D>(l32, 2 * cc + hf);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) voff[tt][mb] = tr_off<D>(lane, 0, mb * 32, tt);

  float ms = -FLT_MAX;  // finite: rows may see no key in this split
  float lsum = 0.f;
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};

  // One key tile of a wave, as in the dense forward: K and V^T fragments are
  // read a few products ahead of their use (K 4 ahead at d = 256, 2 below;
  // V^T pairs 2 ahead), the scores are copied once out of the product
  // accumulators for the mask and the softmax, the split's first tile sets
  // the running max up front, and a later rescale multiplies O in place.  At
  // d = 256 (one wave per SIMD, every accumulator in the accumulation
  // registers) an empty asm pins O to those registers for the rescale (written
  // plainly, the compiler moved all of O out and back on every tile).  Same
  // arithmetic and order as the previous body (all K fragments of a tile read
  // before its products, the V^T reads left to the compiler).  Measured
  // against it (same-box rotated A/B; Hq=32 Hkv=8 unless stated): d = 256
  // decode Nq=1 Nk=32768 B=8 +1%, causal append Nq=64 Nk=16384 B=4 621 -> 696
  // TFLOP/s (+12%), causal chunk Nq=512 Nk=16384 B=1 Hq=16 Hkv=2 748 -> 896
  // (+20%); d = 128 causal chunk +1.4%, decode and append +0.2 to +0.4%; d = 64
  // append +0.1%.
  auto tile_body = [&](const char* kt, const char* vt, int j) __attribute__((always_inline)) {
    constexpr int NF = 2 * NQC, KLA = D == 256 ? 4 : 2;  // score products; K fragments read ahead
    f32x16 sacc2[2];
    {
      u32x4 kf[NF];
      auto kread = [&](int i) __attribute__((always_inline)) {
        kf[i] = lds_read16(kt + (i / NQC) * 32 * ROWB + koff[i % NQC]);
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < KLA; ++i) kread(i);
      sacc2[0] = f32x16{};
      sacc2[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        if (i + KLA < NF) kread(i + KLA);
        sacc2[i / NQC] = mfma32(bitcast<V8>(kf[i]), qreg[i % NQC], sacc2[i / NQC]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KLA, 0);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + KLA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float sv[2][16];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sv[kbk][rr] = sacc2[kbk][rr];
    // mask: keys past the split / past Nk, and (causal) keys after the row's diagonal
    const int k0 = kbeg + j * BC;
    if ((k0 + BC > kend) || (CAUSAL && (k0 + BC - 1 > off))) {
      __asm__ volatile("");
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = k0 + kbk * 32 + acc_row(rr, hf);
          if ((key >= kend) || (CAUSAL && key > qi + off)) sv[kbk][rr] = -__builtin_inff();
        }
    }
    if (j == 0) {  // the split's first tile: the running maximum is set from it up front
      float mloc = sv[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mloc = __builtin_fmaxf(mloc, sv[kbk][rr]);
      mloc = __builtin_fmaxf(mloc, xor32(mloc));
      ms = __builtin_fmaxf(ms, mloc * c);
    }
    uint32_t pk[2][8];
    auto expo = [&]() __attribute__((always_inline)) {
      float ts = 0.f;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sv[kbk][rr], c, -ms));
          const float p1 = fast_exp2(__builtin_fmaf(sv[kbk][rr + 1], c, -ms));
          pk[kbk][rr >> 1] = pack2<T>(p0, p1);
          ts += p0 + p1;
        }
      return ts;
    };
    float tsum = expo();
    bool rescale = false;
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(!(tsum <= kSumMax<T>)) != 0) {
      __asm__ volatile("");
      float mloc = sv[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mloc = __builtin_fmaxf(mloc, sv[kbk][rr]);
      mloc = __builtin_fmaxf(mloc, xor32(mloc));
      const float tmax = mloc * c;
      if (__builtin_amdgcn_ballot_w64(tmax > ms + kTau<T>) != 0) {
        const float mnew = __builtin_fmaxf(ms, tmax);
        alpha = fast_exp2(ms - mnew);
        ms = mnew;
        lsum *= alpha;
        rescale = true;
        tsum = expo();
      }
    }
    lsum += tsum;
    // O^T += V^T P^T; product i: O block mb = i/4, key block (i/2)%2, half i%2
    auto pv = [&]() __attribute__((always_inline)) {
      constexpr int NP = NMB * 4, VLA = 2;  // V^T fragment pairs read ahead
      u32x2 vlo[NP], vhi[NP];
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int rows = (((i / 2) % 2) * 32 + (i % 2) * 16) * ROWB;
        vlo[i] = lds_read_tr(vt + rows + voff[0][i / 4]);
        vhi[i] = lds_read_tr(vt + rows + voff[1][i / 4]);
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < VLA; ++i) vread(i);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + VLA < NP) vread(i + VLA);
        const int kbk = (i / 2) % 2, cp = i % 2;
        const V8 a = bitcast<V8>(u32x4{vlo[i][0], vlo[i][1], vhi[i][0], vhi[i][1]});
        const V8 bp = bitcast<V8>(
            u32x4{pk[kbk][4 * cp], pk[kbk][4 * cp + 1], pk[kbk][4 * cp + 2], pk[kbk][4 * cp + 3]});
        oacc[i / 4] = mfma32(a, bp, oacc[i / 4]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * VLA, 0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + VLA < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // (after pv's definition on purpose: placed before it, the same code
    // left the allocator spilling 10-80 registers)
    if (rescale) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        f32x16 o = oacc[mb];
        if constexpr (D == 256) __asm__ volatile("" : "+a"(o));
        oacc[mb] = o * alpha;
      }
    }
    pv();
  };

  auto tile = [&](auto bufc, int j) {
    constexpr int BUF = decltype(bufc)::value;
    const char* kt = smem + BUF * 2 * TILEB;
    const char* vt = kt + TILEB;
    if (j + NBUF - 1 < ntiles) issue(j + NBUF - 1);
    if (j < wtiles) {
      tile_body(kt, vt, j);
    }
    if (j + 1 < ntiles) wait_next(j + 1);
  };

  // Prologue: tiles 0 .. NBUF-2 in flight, then wait for tile 0.
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < ntiles) issue(j);
  wait_next(0);
  for (int j = 0; j < ntiles; j += NBUF) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1);
    if constexpr (NBUF >= 3)
      if (j + 2 < ntiles) tile(std::integral_constant<int, 2 % NBUF>{}, j + 2);
    if constexpr (NBUF >= 4)
      if (j + 3 < ntiles) tile(std::integral_constant<int, 3 % NBUF>{}, j + 3);
  }

  // Partial result of this split: O_s = acc / l (fp32), LSE_s (ln); a row
  // that saw no key here gets O_s = 0, LSE_s = -inf.
  const float lfull = lsum + xor32(lsum);
  if (r < R) {
    const int64_t prow = (int64_t)split * rows_total + row0 + r;
    float* dst = Opart + prow * D;
    const bool any = lfull > 0.f;
    const float inv = any ? 1.0f / lfull : 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[mb][4 * rg + e] * inv;
        *(f32x4*)(dst + d0) = v;
      }
    if (hf == 0) Lpart[prow] = any ? (ms + __builtin_log2f(lfull)) * kLn2 : -__builtin_inff();
  }
}

// Merge of the split partials, 64 / (D/4) rows per one-wave workgroup.  Each
// lane owns 4 features of one row and folds the splits in with the
// online-softmax merge
//   m' = max(m, LSE_s),  w <- w e^{m - m'} + e^{LSE_s - m'},
//   acc <- acc e^{m - m'} + e^{LSE_s - m'} O_s,
// then O = acc / w and LSE = m + ln w.  Splits are read in groups of
// SG whose loads are all issued before any is used, so a row costs a few
// memory round trips whatever the split count.  A row no split saw gets
// O = 0, LSE = -inf.
template <typename T, int D>
__global__ __launch_bounds__(64) void split_combine_kernel(const float* __restrict__ Opart,
                                                           const float* __restrict__ Lpart,
                                                           T* __restrict__ O,
                                                           float* __restrict__ LSE, int nsplit,
                                                           int64_t rows, int Hq, int Nq,
                                                           Strides3 os) {
  constexpr int TPR = D / 4;   // lanes per row
  constexpr int RPW = 64 / TPR;  // rows per wave
  constexpr int SG = 8;        // splits whose loads are in flight together
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;
  const float ninf = -__builtin_inff();
  float m = ninf, wsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += SG) {
    float ls[SG];
    f32x4 os[SG];
#pragma unroll
    for (int t = 0; t < SG; ++t) {
      const int s = s0 + t;
      ls[t] = s < nsplit ? Lpart[(int64_t)s * rows + row] : ninf;
      os[t] = s < nsplit ? *(const f32x4*)(Opart + ((int64_t)s * rows + row) * D + part * 4)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < SG; ++t) {
      if (ls[t] == ninf) continue;  // split saw no key of this row
      if (ls[t] > m) {
        const float r = expf(m - ls[t]);  // 0 while m is still -inf
        acc *= r;
        wsum *= r;
        m = ls[t];
      }
      const float wgt = expf(ls[t] - m);
      acc += wgt * os[t];
      wsum += wgt;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  u32x2 outv;
  outv[0] = pack2<T>(acc[0] * inv, acc[1] * inv);
  outv[1] = pack2<T>(acc[2] * inv, acc[3] * inv);
  // row = (b*Hq + h)*Nq + i of the [B, Hq, Nq] rows; O at the caller's
  // strides (os.r == 0 marks the dense layout, where the row is the offset)
  T* dst = O + row * D;
  if (os.r != 0) {
    const int64_t bh = row / Nq;
    const int64_t b = bh / Hq;
    dst = O + b * os.b + (bh - b * Hq) * os.h + (row - bh * Nq) * os.r;
  }
  *(u32x2*)(dst + part * 4) = outv;
  if (part == 0) LSE[row] = wsum > 0.f ? m + logf(wsum) : ninf;
}

// ---------------------------------------------------------------- launchers
SplitPlan split_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  constexpr int BC = 64, BR = 128;
  SplitPlan p{};
  const int R = (Hq / Hkv) * Nq;
  p.nrb = (R + BR - 1) / BR;
  if (Nk == 0) {  // nothing to see: one split that writes the empty result
    p.nsplit = 1;
    p.split_len = BC;
    return p;
  }
  const int max_splits = (Nk + BC - 1) / BC;
  int ns = num_splits;
  if (ns <= 0) {
    // One round of resident workgroups (256 CUs x workgroups per CU, which
    // the waves-per-SIMD setting fixes); each split keeps at least 4 tiles.
    // More splits only add partial-output traffic and merge work.
    const int64_t resident =
        256 * (d == 64 ? SplitCfg<64>::WPE : d == 128 ? SplitCfg<128>::WPE : SplitCfg<256>::WPE);
    const int64_t wgs = (int64_t)B * Hkv * p.nrb;
    const int64_t want = (resident + wgs - 1) / wgs;
    ns = (int)std::min<int64_t>(want, std::max(1, (Nk + 4 * BC - 1) / (4 * BC)));
  }
  ns = std::max(1, std::min(ns, max_splits));
  const int tiles = (Nk + BC - 1) / BC;
  p.split_len = ((tiles + ns - 1) / ns) * BC;
  p.nsplit = (Nk + p.split_len - 1) / p.split_len;  // no empty splits
  return p;
}

size_t split_workspace_bytes(int B, int Hq, int Nq, int d, int nsplit) {
  const size_t rows = (size_t)B * Hq * Nq;
  const size_t obytes = ((size_t)nsplit * rows * d * 4 + 255) & ~(size_t)255;
  const size_t lbytes = ((size_t)nsplit * rows * 4 + 255) & ~(size_t)255;
  return obytes + lbytes;
}

template <typename T, int D, bool CAUSAL>
static hipError_t split_t(const SplitArgs& a) {
  const SplitPlan p = split_plan(a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d, a.num_splits);
  const int64_t rows = (int64_t)a.B * a.Hq * a.Nq;
  float* opart = (float*)a.workspace;
  float* lpart = (float*)((char*)a.workspace +
                          (((size_t)p.nsplit * rows * D * 4 + 255) & ~(size_t)255));
  float c = fabsf(a.scale) * kLog2e;
  if (!(c >= 1.17549435e-38f)) c = 1.17549435e-38f;  // scale 0: uniform weights
  const int64_t grid = (int64_t)p.nrb * p.nsplit * a.B * a.Hkv;
  hipError_t e = allow_lds(fwd_split_kernel<T, D, CAUSAL>, SplitCfg<D>::LDS);
  if (e != hipSuccess) return e;
  // the caller's strides, or dense [B, H, N, d] ones (Nq rows for Q and O,
  // Nk for K and V)
  Layout lay = a.lay;
  if (!lay.q.r) {
    const Strides3 q{(int64_t)a.Hq * a.Nq * D, (int64_t)a.Nq * D, D};
    const Strides3 kv{(int64_t)a.Hkv * a.Nk * D, (int64_t)a.Nk * D, D};
    lay = Layout{q, kv, q};
  }
  hipLaunchKernelGGL((fwd_split_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(256),
                     SplitCfg<D>::LDS, a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     opart, lpart, a.Hq, a.Hkv, a.Nq, a.Nk, p.nrb, p.nsplit,
                     p.split_len, rows, c, (a.scale < 0.f) ? 0x80008000u : 0u, lay);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPW = 64 / (D / 4);
  hipLaunchKernelGGL((split_combine_kernel<T, D>), dim3((unsigned)((rows + RPW - 1) / RPW)),
                     dim3(64), 0, a.stream, opart, lpart, (T*)a.o, a.lse, p.nsplit, rows, a.Hq,
                     a.Nq, a.lay.q.r ? lay.o : Strides3{0, 0, 0});
  return hipGetLastError();
}

template <typename T>
static hipError_t split_for(const SplitArgs& a) {
  if (a.d == 64) return a.causal ? split_t<T, 64, true>(a) : split_t<T, 64, false>(a);
  if (a.d == 128) return a.causal ? split_t<T, 128, true>(a) : split_t<T, 128, false>(a);
  return a.causal ? split_t<T, 256, true>(a) : split_t<T, 256, false>(a);
}

hipError_t launch_fwd_split(const SplitArgs& a) {
  if (a.dtype == kBF16) return split_for<__bf16>(a);
  if (a.dtype == kF16) return split_for<_Float16>(a);
  return hipErrorNotSupported;
}

}  // namespace attn
