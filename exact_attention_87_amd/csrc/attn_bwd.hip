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
//   pre:  per (batch, head) row statistics into the caller's workspace,
//         laid out [B*Hq][2][Np] fp32 with Np = N rounded up to 64:
//         [0] = -D_i = -(dO_i . O_i), [1] = LSE_i * log2(e); padding rows
//         are 0.  -D seeds the accumulator of dP = dO V^T, so the matrix
//         cores return dP - D directly.
//   dkdv: one workgroup per (batch, kv head, block of 128 keys); each wave
//         keeps its 32 keys' K and V as matrix-core operands in registers
//         (at d = 128 and 256 V stays in LDS, read per product, which lets
//         two workgroups share a CU at d = 128 and frees registers at 256)
//         and
//         accumulates dK^T, dV^T over every query tile of every query head of
//         the group (so grouped-query heads are summed on chip).  Query tiles
//         (Q, dO and the statistics) stream through LDS.  When that grid is
//         too small to fill the device, a group's query heads are split over
//         several workgroups per key block, each writing fp32 partial sums to
//         the workspace, and a merge kernel adds them in split order.
//   dq:   one workgroup per (batch, query head, block of 128 queries); the
//         forward's tiling, with dQ^T accumulated over key tiles that stream
//         through LDS.  The full backward of a dense problem runs dq first,
//         in a variant that computes its rows' statistics itself (it already
//         holds dO) and stores them for dkdv, so pre is not launched there.
// Probabilities use base 2: P = 2^(s*c - LSE*log2 e), c = |scale| log2 e.  A
// negative scale is folded into the sign bit of the register-resident operand
// (Q in the dq kernel, K in the dkdv kernel) as it is loaded.  Query rows
// past N read as zero (Q, dO) with zero statistics, so they add nothing to
// dK and dV without a mask.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {

constexpr float kTiny = 1.17549435e-38f;  // smallest normal fp32

// Measured choices (same-box A/B each; the alternatives are not kept):
//  - Waves per SIMD: the dK/dV kernel runs 3 at d = 64 (168 registers, with
//    operand reads in pairs and fenced phases), 2 at d = 128 and 1 at d = 256
//    (with resident K and V, the dK, dV accumulators and K, V took 336-354
//    registers at d = 128); the
//    dQ kernel runs 3 at d = 64 and 2 at d = 128.  Against 2/2/1: +5% on the
//    causal B=8 H=16 N=2048 d=64 backward.  d = 128 dK/dV at 2 waves (V in
//    LDS, 32-query tiles) against 1 wave (V in registers, 64-query tiles):
//    +4 to +12% on the d = 128 backward, except on causal query-head splits
//    (-9 to -11%), which keep the 1-wave layout.
//  - Raised wave priority (s_setprio 1) in any matrix-core phase of the dQ
//    kernel or of the dK/dV kernel at 1 or 3 waves per SIMD, or a priority
//    falling with the remaining tiles: 0 to -3%, so they do not raise it;
//    raised in their exp / dS (vector ALU) phase at d = 64 instead: -2 to
//    +2% (dK/dV), -3% with the dQ kernel's too.
//    At d = 128 (2 waves per SIMD) the dK/dV kernel raises it for the S and
//    dP products: +1 to +3.6%; around the dV/dK products instead: +0 to
//    +2.6%; fences between the dV/dK feature blocks: -1 to +1%.
//  - d = 64 dK/dV at three waves: fences between the operand groups of the
//    S and dP products (without them 3 registers spill, -2% causal), none
//    between the dV/dK products (+3% causal against one per feature block).

__host__ __device__ constexpr int stat_rows(int N) { return (N + 63) / 64 * 64; }

// ---------------------------------------------------------------- row statistics
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ stats, int N, int Np,
                                                      int64_t nslices, int Hq, Strides3 os) {
  constexpr int TPR = D / 8;  // lanes per row, 16 bytes each
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int64_t prow = (int64_t)blockIdx.x * RPB + tid / TPR;  // padded row index
  const int part = tid % TPR;
  const int64_t slice = prow / Np;
  const int i = (int)(prow - slice * Np);
  const bool live = slice < nslices && i < N;
  float acc = 0.f;
  if (live) {
    // O and dO share one stride set
    const int64_t off = (slice / Hq) * os.b + (slice % Hq) * os.h + (int64_t)i * os.r + part * 8;
    const u32x4 a = *(const u32x4*)(O + off);
    const u32x4 b = *(const u32x4*)(dO + off);
    using V8 = typename Elem<T>::v8;
    const V8 av = bitcast<V8>(a), bv = bitcast<V8>(b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)av[e], (float)bv[e], acc);
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (slice < nslices && part == 0) {
    float* st = stats + slice * 2 * Np;
    st[i] = -acc;
    st[Np + i] = live ? LSE[slice * N + i] * kLog2e : 0.f;
  }
}

// ---------------------------------------------------------------- dK, dV
// The kernel takes WIDE = CAUSAL && SPLIT: with it, d = 128 keeps V in
// registers with 64-query tiles at one workgroup per CU.
template <int D, bool WIDE = false>
struct DkdvCfg {
  static constexpr int BKV = 128;  // keys per workgroup (4 waves x 32)
  // VLDS: V of the workgroup's keys sits in LDS (read as the dP product's
  // operand) instead of registers, and query tiles hold one 32-query
  // sub-block.  d = 128: registers (256) and LDS (64.5 KiB) then allow two
  // workgroups per CU; not for causal query-head splits, whose grids are one
  // or two rounds with the heaviest key blocks setting the launch's length,
  // where a key block sharing its CU with another workgroup runs longer (-9
  // to -11% on causal split shapes, +7% on a non-causal one).  d = 256 (one
  // workgroup per CU, 128.5 KiB of LDS): the 64 registers of V relieve the
  // allocator (0-2 spilled values instead of 6-10), +4 to +9% on every d = 256
  // shape measured, split or not.
  static constexpr bool VLDS = (D == 128 && !WIDE) || D == 256;
  static constexpr int BQ = VLDS ? 32 : 64;  // queries per tile (32-query sub-blocks)
  static constexpr int NBUF = D == 64 ? 3 : 2;
  static constexpr int WPE = D == 64 ? 3 : (VLDS && D == 128) ? 2 : 1;  // waves per SIMD
  static constexpr int TILEB = BQ * D * 2;
  static constexpr int STAGEB = 2 * TILEB + 2 * BQ * 4;  // Q | dO | D | LSE*log2e
  static constexpr int VB = VLDS ? BKV * D * 2 : 0;       // V of the key block
  static constexpr size_t LDS = (size_t)NBUF * STAGEB + VB;
};

template <typename T, int D, bool CAUSAL, bool VARLEN, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DkdvCfg<D, CAUSAL && SPLIT>::WPE, DkdvCfg<D, CAUSAL && SPLIT>::WPE)))
void bwd_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                     const T* __restrict__ V, const T* __restrict__ dO,
                     const float* __restrict__ stats, T* __restrict__ dK,
                     T* __restrict__ dV, int Hq, int Hkv, int Nmax, int nkb, int xg, int desc, Layout lay, float c,
                     float dk_scale, uint32_t qsign, const int* __restrict__ cu_seqlens,
                     int ntok, int nsplit_arg, float* __restrict__ part) {
  using Cfg = DkdvCfg<D, CAUSAL && SPLIT>;
  const int nsplit = SPLIT ? nsplit_arg : 1;
  using V8 = typename Elem<T>::v8;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, NBUF = Cfg::NBUF, TILEB = Cfg::TILEB;
  constexpr int STAGEB = Cfg::STAGEB;
  constexpr int ROWB = D * 2;
  constexpr int PW = TILEB / 1024 / 4;  // 1 KiB direct loads per wave per tensor per tile
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // blockIdx = (key block, split, slice): key block major, so that under the
  // causal mask the low key blocks, which carry the most work, start first
  // (xg > 0, one split only: the XCD-aware order of xcd_item, key blocks
  // ascending within each slice group)
  const int BGS = gridDim.x / nkb;
  const int BG = BGS / nsplit;
  int kblk, split, bg;
  if (xg > 0) {
    xcd_item(nkb, BG, xg, kblk, bg);
    split = 0;
  } else {
    kblk = blockIdx.x / BGS;
    split = (blockIdx.x % BGS) / BG;
    bg = blockIdx.x % BG;
  }
  const int group = Hq / Hkv;
  // query heads g*group + hs0 .. g*group + hs1 - 1 of the kv group
  const int hs0 = split * group / nsplit, hs1 = (split + 1) * group / nsplit;
  // This workgroup's problem: one (batch, kv head) slice of Nmax rows, or for
  // packed variable-length sequences one (sequence, kv head).  Query head hq
  // reads Q at qb0 + hq*qhs, dO at ob0 + hq*ohs and its statistics at
  // sb0 + hq*2*Np; K, V, dK, dV share one stride set, O and dO another.
  int N = Nmax, g, Np, krs, qrs, ors, start = 0;
  int64_t kvoff, qb0, qhs, ob0, ohs, sb0;
  if constexpr (VARLEN) {
    const int seq = bg / Hkv;
    g = bg - seq * Hkv;
    start = min(max(cu_seqlens[seq], 0), ntok);
    const int end = min(max(cu_seqlens[seq + 1], start), ntok);
    N = end - start;
    if (kblk * BKV >= N) return;  // the whole workgroup: past this sequence's end
    Np = stat_rows(ntok);  // statistics of the packed tokens, [Hq][2][Np]
    // (head, token) strides; the batch strides are unused
    krs = lay.kv.r, qrs = lay.q.r, ors = lay.o.r;
    kvoff = g * lay.kv.h + (int64_t)start * lay.kv.r;
    qb0 = (int64_t)start * lay.q.r, qhs = lay.q.h;
    ob0 = (int64_t)start * lay.o.r, ohs = lay.o.h;
    sb0 = start;
  } else {
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    Np = stat_rows(N);
    krs = lay.kv.r, qrs = lay.q.r, ors = lay.o.r;
    kvoff = b * lay.kv.b + g * lay.kv.h;
    qb0 = b * lay.q.b, qhs = lay.q.h;
    ob0 = b * lay.o.b, ohs = lay.o.h;
    sb0 = (int64_t)b * Hq * 2 * Np;
  }
  const int key0 = kblk * BKV + w * 32;  // first key of this wave
  const int krow = key0 + l32;           // key owned by this lane

  // K^T and V^T operands of this wave's 32 keys, resident (zero past N);
  // with VLDS, V of the workgroup's 128 keys goes to LDS instead (a
  // swizzled [BKV][D] tile after the query stages, waited for with them).
  constexpr bool VLDS = Cfg::VLDS;
  V8 kreg[NQC], vreg[VLDS ? 1 : NQC];
  char* const vtile = smem + NBUF * STAGEB;
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kvoff, slice_bytes(N, krs, D));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kvoff, slice_bytes(N, krs, D));
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      const uint32_t off = (uint32_t)((krow * krs + cc * 16 + hf * 8) * 2);
      kreg[cc] = bitcast<V8>(buf_load16(rk, off) ^ qsign);  // scale's sign rides on K here
      if constexpr (!VLDS) vreg[cc] = bitcast<V8>(buf_load16(rv, off));
    }
    if constexpr (VLDS) {
      constexpr int VPW = Cfg::VB / 1024 / 4;  // 1 KiB pieces per wave
#pragma unroll
      for (int i = 0; i < VPW; ++i) {
        const int o = (w * VPW + i) * 1024 + lane * 16;
        const int row = o / ROWB;
        const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
        buf_load16_lds(rv, vtile + (w * VPW + i) * 1024,
                       (uint32_t)(((kblk * BKV + row) * krs + ch * 8) * 2));
      }
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
  const int nh = hs1 - hs0;
  const int iters = nh * per_head;
  // Step `it` takes query tile rank it / nh of head hs0 + it % nh: tile-major,
  // the group's query heads innermost.  Under the causal mask each key block
  // starts at its own diagonal tile, so with an ascending walk the
  // workgroups of one kv group would read a given Q/dO tile at different
  // times, and when the group's stream is larger than an XCD's L2 every key
  // block would fetch it from HBM again.  With `desc` the tiles are walked
  // from the last one down, so the workgroups of a group, whatever their key
  // block, read the same tiles at about the same time; taking all heads of a
  // tile before the next tile keeps them in step across heads too (walked
  // head by head, a short walk moves on to the next head while the long
  // ones are still low in the first).  The host sets desc for every causal
  // problem.  It is a runtime argument on purpose: with the direction fixed
  // at compile time the d = 256 instances spill 20-21 registers instead of
  // 7-11, and run 14% slower on the causal B=1 H=16 N=8192 backward.
  auto qtile_of = [&](int it) {
    const int r = it / nh;
    return (CAUSAL && desc) ? nqt - 1 - r : qt0 + r;
  };

  // Direct loads of a query tile: Q and dO pieces as in the forward, plus
  // the 512 bytes of statistics (wave 0, lanes 0..31).
  // (kept in registers up to d = 128; recomputed per load at d = 256)
  auto gpiece = [&](int i, int rs) {
    const int o = (w * PW + i) * 1024 + lane * 16;
    const int row = o / ROWB;
    const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
    return (uint32_t)((row * rs + ch * 8) * 2);
  };
  constexpr int PWK = D > 128 ? 1 : PW;
  uint32_t goffq[PWK], goffo[PWK];
#pragma unroll
  for (int i = 0; i < PWK; ++i) {
    goffq[i] = gpiece(i, qrs);
    goffo[i] = gpiece(i, ors);
  }
  constexpr int SLN = BQ / 4;  // lanes per statistics row of a tile (16 bytes each)
  const uint32_t soff = (uint32_t)((lane / SLN) * Np * 4 + (lane % SLN) * 16);
  auto issue = [&](int it) {
    const int hq = g * group + hs0 + it % nh;
    const int qt = qtile_of(it);
    char* base = smem + (it % NBUF) * STAGEB;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qb0 + hq * qhs, slice_bytes(N, qrs, D));
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + ob0 + hq * ohs, slice_bytes(N, ors, D));
    const uint32_t tq = (uint32_t)(qt * BQ * qrs * 2), to = (uint32_t)(qt * BQ * ors * 2);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const uint32_t gq = PWK == PW ? goffq[i % PWK] : gpiece(i, qrs);
      const uint32_t go = PWK == PW ? goffo[i % PWK] : gpiece(i, ors);
      buf_load16_lds(rq, base + (w * PW + i) * 1024, gq + tq);
      buf_load16_lds(rdo, base + TILEB + (w * PW + i) * 1024, go + to);
    }
    if (w == 0 && lane < 2 * SLN) {
      // this head's two statistics rows (lanes 0..SLN-1: -D, then LSE log2 e)
      // from the slice's (or packed sequence's) first row on.  The buffer
      // ends right after the LSE row's last row of the slice, so rows past
      // it read LSE = 0: batched slices have zero padding there anyway, and a
      // packed sequence must not read the next sequence's LSE, which could
      // make P = 2^(-LSE log2 e) overflow (fp16 once LSE < -11) and 0 * inf
      // poison dK and dV.  Their -D (the padding, or the next sequence's) is
      // replaced by 0 where the dP accumulator is seeded (phaseA).
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(stats + sb0 + (int64_t)hq * 2 * Np, (uint32_t)((Np + N) * 4));
      buf_load16_lds(rs, base + 2 * TILEB, soff + (uint32_t)qt * BQ * 4);
    }
  };
  // Loads per wave per stage, for the partial waits of a 3-stage pipeline:
  // 2*PW for Q and dO, plus one for the statistics on wave 0.  Each wave
  // must wait with its own count: allowing wave 0's count on the others
  // would let one load of the stage about to be read still be in flight.
  constexpr int LOADS = 2 * PW;
  constexpr int SLOADS = 1;
  // Wait until only the newest stage's loads may be outstanding, then
  // synchronise the workgroup (w is wave-uniform).
  auto wait_stage = [&]() {
    if (w == 0)
      wait_vm_barrier<LOADS + SLOADS>();
    else
      wait_vm_barrier<LOADS>();
  };

  // Per-lane LDS offsets inside a stage (fixed for the whole loop).  The
  // swizzle only permutes chunks within aligned groups of 16, so at d = 256
  // the second half of a row's offsets are the first half's plus 256 bytes
  // (an immediate of the LDS read) and are not kept in registers.
  constexpr int NQO = D > 128 ? NQC / 2 : NQC, NMO = D > 128 ? NMB / 2 : NMB;
  int qoff_[NQO], troff[2][NMO];
#pragma unroll
  for (int cc = 0; cc < NQO; ++cc) qoff_[cc] = tile_off<D>(l32, 2 * cc + hf);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < NMO; ++mb) troff[t][mb] = tr_off<D>(lane, 0, mb * 32, t);
  auto qo = [&](int cc) { return qoff_[cc % NQO] + (cc / NQO) * 256; };
  auto tro = [&](int t, int mb) { return troff[t][mb % NMO] + (mb / NMO) * 256; };

  // The three phases of one 32-query sub-block (rows qbase.. of the tile):
  //   A: S = Q K^T and dP - D = dO V^T - D on the matrix cores;
  //   V: P = 2^(S c - LSE), dS = P (dP - D), both packed to bf16 (vector ALU);
  //   C: dV^T += dO^T P and dK^T += Q^T dS on the matrix cores.
  // Operand reads stream two products ahead of their use in phases A and C,
  // pinned with scheduling groups.  Read in groups (all chunks at once, or
  // two at a time behind scheduling fences where registers are tight), each
  // group's LDS latency was exposed, fully so where one wave runs per SIMD.
  // Measured (same-box rotated A/B of attn_bwd, bitwise-equal gradients):
  //   - one wave per SIMD (d = 256, with the same streaming in the dQ
  //     kernel): non-causal B=1 H=16 N=8192 661 -> 779 TFLOP/s (+18%), causal
  //     655 -> 736 (+12%), causal B=2 N=4096 +10%, causal grouped-query
  //     Hq=32 Hkv=8 N=8192 +15%, a query-head split (B=2 Hq=16 Hkv=2
  //     N=4096) +13%; one chunk ahead gave about half of that, three or four
  //     no more; the split causal d = 128 stage +0.4 to +1.2%;
  //   - several waves per SIMD: causal B=8 H=16 N=2048 d=64 683 -> 697
  //     (+2.0%), non-causal B=8 H=16 N=1024 d=64 +6.7%, causal grouped-query
  //     d=64 +1.9%, causal B=4 H=32 N=4000 d=128 +3.4%, causal grouped-query
  //     N=16384 d=128 +1.4%, non-causal B=2 H=32 N=4096 d=128 +0.3%; one
  //     ahead in either phase gained less.
  auto phaseA = [&](const char* qtile, const char* dotile, const float* dsum, int qbase,
                    int qfirst, f32x16& sacc, f32x16& pacc) {
    // the dP accumulator starts at -D of each row (element 4*rg+e is row
    // qbase + 8*rg + 4*hf + e).  Packed sequences: on a sequence's last
    // query tile the rows past its end (zero Q and dO) would start at the
    // next sequence's -D; they start at 0 instead, so that their dS is 0 and
    // a non-finite value in the next sequence cannot reach this one's dK
    // through 0 * inf.
    const int lim = N - qfirst - 4 * hf;  // element 4*rg+e is a row of the sequence iff 8*rg+e < lim
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      f32x4 nd = *(const f32x4*)(dsum + qbase + 8 * rg + 4 * hf);
      if (VARLEN && qfirst + 32 > N) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (8 * rg + e >= lim) nd[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pacc[4 * rg + e] = nd[e];
    }
    sacc = f32x16{};
    {
      constexpr int LA = 2;  // chunks read ahead
      u32x4 qa[NQC], da[NQC], va[VLDS ? NQC : 1];
      auto rd = [&](int cc) __attribute__((always_inline)) {
        qa[cc] = lds_read16(qtile + qbase * ROWB + qo(cc));
        da[cc] = lds_read16(dotile + qbase * ROWB + qo(cc));
        if constexpr (VLDS) va[cc] = lds_read16(vtile + w * 32 * ROWB + qo(cc));
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cc = 0; cc < LA; ++cc) rd(cc);
#pragma unroll
      for (int cc = 0; cc < NQC; ++cc) {
        if (cc + LA < NQC) rd(cc + LA);
        sacc = mfma32(bitcast<V8>(qa[cc]), kreg[cc], sacc);
        if constexpr (VLDS)
          pacc = mfma32(bitcast<V8>(da[cc]), bitcast<V8>(va[cc]), pacc);
        else
          pacc = mfma32(bitcast<V8>(da[cc]), vreg[cc], pacc);
      }
      constexpr int RPC = VLDS ? 3 : 2;  // LDS reads per chunk
      __builtin_amdgcn_sched_group_barrier(0x100, RPC * LA, 0);
#pragma unroll
      for (int cc = 0; cc < NQC; ++cc) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (cc + LA < NQC) __builtin_amdgcn_sched_group_barrier(0x100, RPC, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phaseV = [&](const float* lse2, int qbase, int qfirst, bool diag, const f32x16& sacc,
                    const f32x16& pacc, uint32_t (&pk)[8], uint32_t (&dsk)[8]) {
    float pv[16];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 l4 = *(const f32x4*)(lse2 + qbase + 8 * rg + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[4 * rg + e] = fast_exp2(__builtin_fmaf(sacc[4 * rg + e], c, -l4[e]));
    }
    if (diag) {  // diagonal block: keys after the query get 0
      __asm__ volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (krow > qfirst + acc_row(r, hf)) pv[r] = 0.f;
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dsv[e] = pv[4 * rg + e] * pacc[4 * rg + e];
      pk[2 * rg] = pack2<T>(pv[4 * rg], pv[4 * rg + 1]);
      pk[2 * rg + 1] = pack2<T>(pv[4 * rg + 2], pv[4 * rg + 3]);
      dsk[2 * rg] = pack2<T>(dsv[0], dsv[1]);
      dsk[2 * rg + 1] = pack2<T>(dsv[2], dsv[3]);
    }
  };
  auto phaseC = [&](const char* qtile, const char* dotile, int qbase, const uint32_t (&pk)[8],
                    const uint32_t (&dsk)[8]) {
    {
      constexpr int LA = 2, NI = 2 * NMB;  // pairs read ahead; pair i: half cp = i / NMB, block mb = i % NMB
      u32x2 a0[NI], a1[NI], b0[NI], b1[NI];
      auto rd = [&](int i) __attribute__((always_inline)) {
        const int rows = (qbase + 16 * (i / NMB)) * ROWB, mb = i % NMB;
        a0[i] = lds_read_tr(dotile + rows + tro(0, mb));
        a1[i] = lds_read_tr(dotile + rows + tro(1, mb));
        b0[i] = lds_read_tr(qtile + rows + tro(0, mb));
        b1[i] = lds_read_tr(qtile + rows + tro(1, mb));
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LA; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i + LA < NI) rd(i + LA);
        const int cp = i / NMB, mb = i % NMB;
        const V8 pb = bitcast<V8>(u32x4{pk[4 * cp], pk[4 * cp + 1], pk[4 * cp + 2], pk[4 * cp + 3]});
        const V8 sb =
            bitcast<V8>(u32x4{dsk[4 * cp], dsk[4 * cp + 1], dsk[4 * cp + 2], dsk[4 * cp + 3]});
        dvacc[mb] = mfma32(bitcast<V8>(u32x4{a0[i][0], a0[i][1], a1[i][0], a1[i][1]}), pb, dvacc[mb]);
        dkacc[mb] = mfma32(bitcast<V8>(u32x4{b0[i][0], b0[i][1], b1[i][0], b1[i][1]}), sb, dkacc[mb]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * LA, 0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (i + LA < NI) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](auto bufc, int it) {
    constexpr int BUF = decltype(bufc)::value;
    const char* qtile = smem + BUF * STAGEB;
    const char* dotile = qtile + TILEB;
    const float* dsum = (const float*)(qtile + 2 * TILEB);  // -D of the tile's rows
    const float* lse2 = dsum + BQ;
    if (it + NBUF - 1 < iters) issue(it + NBUF - 1);
    const int qt = qtile_of(it);
    const int qf0 = qt * BQ, qf1 = qf0 + 32;
    // wave-uniform: which of the two 32-query sub-blocks have visible
    // (query, key) pairs, and which touch the diagonal
    const bool act0 = !((CAUSAL && qf0 + 31 < key0) || qf0 >= N);
    const bool act1 = !((CAUSAL && qf1 + 31 < key0) || qf1 >= N);
    const bool diag0 = CAUSAL && key0 + 31 > qf0;
    const bool diag1 = CAUSAL && key0 + 31 > qf1;
#pragma unroll
    for (int qs = 0; qs < BQ / 32; ++qs) {
      if (!(qs == 0 ? act0 : act1)) continue;  // wave-uniform
      f32x16 sacc, pacc;
      uint32_t pk[8], dsk[8];
      // d = 128 (two workgroups per CU): the S and dP products run at raised
      // wave priority, so one wave's products overlap the other's exp work
      if constexpr (VLDS && D == 128) __builtin_amdgcn_s_setprio(1);
      phaseA(qtile, dotile, dsum, qs * 32, qs == 0 ? qf0 : qf1, sacc, pacc);
      if constexpr (VLDS && D == 128) __builtin_amdgcn_s_setprio(0);
      phaseV(lse2, qs * 32, qs == 0 ? qf0 : qf1, qs == 0 ? diag0 : diag1, sacc, pacc, pk, dsk);
      phaseC(qtile, dotile, qs * 32, pk, dsk);
    }
    if (it + 1 < iters) {
      if (NBUF == 3 && it + 2 < iters)
        wait_stage();
      else
        wait_vm_barrier<0>();
    }
  };

#pragma unroll
  for (int it = 0; it < NBUF - 1; ++it)
    if (it < iters) issue(it);
  // A full wait here, not one that lets the second stage stay in flight: the
  // compiler's wait analysis does not see the direct-to-LDS loads (inline
  // assembly), so after a partial count it takes the last loads of K and V
  // above for still pending and waits for them inside the loop, which at run
  // time drained each step's own prefetch (vmcnt(1), then vmcnt(0), before
  // the last S and dP products).  After vmcnt(0) nothing is pending for it.
  wait_vm_barrier<0>();
  for (int it = 0; it < iters; it += NBUF) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < iters) step(std::integral_constant<int, 1>{}, it + 1);
    if constexpr (NBUF == 3)
      if (it + 2 < iters) step(std::integral_constant<int, 2 % NBUF>{}, it + 2);
  }

  // ---- split query heads: fp32 partial sums (dK unscaled, then dV), added
  // by the merge kernel in split order.  Rows are (slice, key) [BG][N] for a
  // batched problem and (kv head, token) [Hkv][T] for packed sequences, so a
  // plane holds `prows` rows per split: [2][nsplit][prows][D].
  if constexpr (SPLIT) {
    if (krow < N) {
      const int64_t prows = VARLEN ? (int64_t)Hkv * ntok : (int64_t)BG * N;
      const int64_t prow = VARLEN ? (int64_t)g * ntok + start + krow : (int64_t)bg * N + krow;
      const int64_t plane = (int64_t)nsplit * prows * D;
      float* pk = part + ((int64_t)split * prows + prow) * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = mb * 32 + rg * 8 + hf * 4;
          *(f32x4*)(pk + d0) = f32x4{dkacc[mb][4 * rg], dkacc[mb][4 * rg + 1],
                                     dkacc[mb][4 * rg + 2], dkacc[mb][4 * rg + 3]};
          *(f32x4*)(pk + plane + d0) = f32x4{dvacc[mb][4 * rg], dvacc[mb][4 * rg + 1],
                                             dvacc[mb][4 * rg + 2], dvacc[mb][4 * rg + 3]};
        }
    }
    return;
  }
  // ---- store dK = scale * (dK^T)^T (Q was not sign-flipped), dV
  // (lane: key krow; element r: feature)
  if (krow < N) {
    T* dkp = dK + kvoff + (int64_t)krow * krs;
    T* dvp = dV + kvoff + (int64_t)krow * krs;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        u32x2 kv, vv;
        kv[0] = pack2<T>(dkacc[mb][4 * rg] * dk_scale, dkacc[mb][4 * rg + 1] * dk_scale);
        kv[1] = pack2<T>(dkacc[mb][4 * rg + 2] * dk_scale, dkacc[mb][4 * rg + 3] * dk_scale);
        vv[0] = pack2<T>(dvacc[mb][4 * rg], dvacc[mb][4 * rg + 1]);
        vv[1] = pack2<T>(dvacc[mb][4 * rg + 2], dvacc[mb][4 * rg + 3]);
        *(u32x2*)(dkp + d0) = kv;
        *(u32x2*)(dvp + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------- split merge
// dK = scale * sum_s dK_s and dV = sum_s dV_s over the query-head splits, in
// split order (deterministic); one thread per 8 features of one key row.
// Rows are (slice bg = b * Hkv + g, key) of a batched problem; packed
// sequences pass BG = Hkv, N = T (rows (kv head, token)) and their offsets,
// and tokens outside [cu_seqlens[0], cu_seqlens[nseq]) are left untouched,
// as the unsplit stage leaves them.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_merge_kernel(const float* __restrict__ part,
                                                             T* __restrict__ dK, T* __restrict__ dV,
                                                             int nsplit, int BG, int Hkv, int N,
                                                             float dk_scale, Strides3 ks,
                                                             const int* __restrict__ cu_seqlens,
                                                             int nseq) {
  constexpr int TPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)BG * N;
  if (t >= rows * TPR) return;
  const int64_t row = t / TPR;  // bg * N + key
  const int f = (int)(t - row * TPR) * 8;
  if (cu_seqlens) {  // packed sequences: the tokens the sequences cover
    const int key = (int)(row % N);
    const int lo = min(max(cu_seqlens[0], 0), N);
    const int hi = min(max(cu_seqlens[nseq], lo), N);
    if (key < lo || key >= hi) return;
  }
  const int64_t plane = (int64_t)nsplit * rows * D;
  const float* pk = part + row * D + f;
  f32x4 k0 = *(const f32x4*)pk, k1 = *(const f32x4*)(pk + 4);
  f32x4 v0 = *(const f32x4*)(pk + plane), v1 = *(const f32x4*)(pk + plane + 4);
  for (int sp = 1; sp < nsplit; ++sp) {
    const float* q = pk + (int64_t)sp * rows * D;
    k0 += *(const f32x4*)q;
    k1 += *(const f32x4*)(q + 4);
    v0 += *(const f32x4*)(q + plane);
    v1 += *(const f32x4*)(q + plane + 4);
  }
  const int bg = (int)(row / N), key = (int)(row - (int64_t)bg * N);
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int64_t off = b * ks.b + g * ks.h + (int64_t)key * ks.r + f;
  u32x4 ko, vo;
  ko[0] = pack2<T>(k0[0] * dk_scale, k0[1] * dk_scale);
  ko[1] = pack2<T>(k0[2] * dk_scale, k0[3] * dk_scale);
  ko[2] = pack2<T>(k1[0] * dk_scale, k1[1] * dk_scale);
  ko[3] = pack2<T>(k1[2] * dk_scale, k1[3] * dk_scale);
  vo[0] = pack2<T>(v0[0], v0[1]);
  vo[1] = pack2<T>(v0[2], v0[3]);
  vo[2] = pack2<T>(v1[0], v1[1]);
  vo[3] = pack2<T>(v1[2], v1[3]);
  *(u32x4*)(dK + off) = ko;
  *(u32x4*)(dV + off) = vo;
}

// ---------------------------------------------------------------- dQ
template <int D>
struct DqCfg {
  static constexpr int BR = 128;  // queries per workgroup (4 waves x 32)
  static constexpr int BC = 64;   // keys per tile
  static constexpr int NBUF = D == 64 ? 3 : 2;
  static constexpr int WPE = D == 64 ? 3 : D == 128 ? 2 : 1;  // waves per SIMD
  static constexpr int TILEB = BC * D * 2;
  static constexpr size_t LDS = (size_t)NBUF * 2 * TILEB;
};

// With STATS the kernel also computes the row statistics the preprocess kernel
// would (the same sums in the same order, so bit-identical) from O, dO and LSE,
// and stores them for the dK/dV kernel launched after it.  Batched: padding
// rows included, since the workgroups of one head cover every padded row of
// its statistics.  Packed sequences: each sequence's own rows only; the dK/dV
// kernel reads no statistic past a sequence's end (its LSE row ends there,
// and -D past it is replaced by 0).
template <typename T, int D, bool CAUSAL, bool VARLEN, bool STATS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DqCfg<D>::WPE, DqCfg<D>::WPE)))
void bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                   const T* __restrict__ V, const T* __restrict__ dO,
                   const T* __restrict__ O, const float* __restrict__ LSE,
                   float* __restrict__ stats, T* __restrict__ dQ, int Hq, int Hkv,
                   int Nmax, int nqb, int xg, Layout lay, float c, float qscale, uint32_t qsign,
                   const int* __restrict__ cu_seqlens, int ntok) {
  using Cfg = DqCfg<D>;
  using V8 = typename Elem<T>::v8;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, NBUF = Cfg::NBUF, TILEB = Cfg::TILEB;
  constexpr int ROWB = D * 2;
  constexpr int PW = TILEB / 1024 / 4;
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem[];  // [NBUF][K tile | V tile]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // XCD-aware order of (query block, slice), heaviest query blocks first
  // under the causal mask (xcd_item; xg from the host)
  const int BH = gridDim.x / nqb;
  int qi, bh;
  xcd_item(nqb, BH, xg, qi, bh);
  const int qb = CAUSAL ? nqb - 1 - qi : qi;
  // One (batch, head) slice of Nmax rows, or one (sequence, head) of packed
  // variable-length sequences.  Q and dQ share one stride set, K and V
  // another, dO has O's.
  int N = Nmax, h, Np, qrs, krs, ors;
  int64_t qoff, kvoff, ooff, lrow0;  // lrow0: LSE entry of the slice's first row
  float* st;  // this head's statistics rows, from the slice's first row on
  if constexpr (VARLEN) {
    const int seq = bh / Hq;
    h = xcd_head(bh - seq * Hq, Hq);  // xg is 0 here: the plain order
    const int start = min(max(cu_seqlens[seq], 0), ntok);
    const int end = min(max(cu_seqlens[seq + 1], start), ntok);
    N = end - start;
    if (qb * BR >= N) return;  // the whole workgroup: past this sequence's end
    const int g = h / (Hq / Hkv);
    Np = stat_rows(ntok);
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    qoff = h * lay.q.h + (int64_t)start * lay.q.r;
    kvoff = g * lay.kv.h + (int64_t)start * lay.kv.r;
    ooff = h * lay.o.h + (int64_t)start * lay.o.r;
    st = stats + (int64_t)h * 2 * Np + start;
    lrow0 = (int64_t)h * ntok + start;  // LSE is [Hq, T]
  } else {
    const int b = bh / Hq;
    h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    Np = stat_rows(N);
    lrow0 = (int64_t)bh * N;
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    qoff = b * lay.q.b + h * lay.q.h;
    kvoff = b * lay.kv.b + g * lay.kv.h;
    ooff = b * lay.o.b + h * lay.o.h;
    st = stats + (int64_t)bh * 2 * Np;
  }
  const int q0 = qb * BR + w * 32;
  const int qrow = q0 + l32;

  const int ntiles_all = (N + BC - 1) / BC;
  int ntiles = ntiles_all, wtiles = ntiles_all;
  if (CAUSAL) {
    ntiles = min(ntiles_all, (qb * BR + BR - 1) / BC + 1);
    wtiles = min(ntiles, (q0 + 31) / BC + 1);
  }

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kvoff, slice_bytes(N, krs, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kvoff, slice_bytes(N, krs, D));
  uint32_t goff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int o = (w * PW + i) * 1024 + lane * 16;
    const int row = o / ROWB;
    const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
    goff[i] = (uint32_t)((row * krs + ch * 8) * 2);
  }
  auto issue = [&](int j) {
    char* kt = smem + (j % NBUF) * 2 * TILEB;
    const uint32_t tbase = (uint32_t)(j * BC * krs * 2);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      buf_load16_lds(rk, kt + (w * PW + i) * 1024, goff[i] + tbase);
      buf_load16_lds(rv, kt + TILEB + (w * PW + i) * 1024, goff[i] + tbase);
    }
  };

#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < ntiles) issue(j);

  // Q^T and dO^T operands resident; loaded after the first K/V tiles are
  // requested, so the two latencies overlap.
  V8 qreg[NQC], doreg[NQC];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qoff, slice_bytes(N, qrs, D));
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + ooff, slice_bytes(N, ors, D));
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      qreg[cc] = bitcast<V8>(buf_load16(rq, (uint32_t)((qrow * qrs + cc * 16 + hf * 8) * 2)) ^ qsign);
      doreg[cc] = bitcast<V8>(buf_load16(rdo, (uint32_t)((qrow * ors + cc * 16 + hf * 8) * 2)));
    }
  }
  V8 oreg[STATS ? NQC : 1];  // O, for D = dO . O
  float lse_row = 0.f;
  if constexpr (STATS) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + ooff, slice_bytes(N, ors, D));
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc)
      oreg[cc] = bitcast<V8>(buf_load16(ro, (uint32_t)((qrow * ors + cc * 16 + hf * 8) * 2)));
    if (qrow < N) lse_row = LSE[lrow0 + qrow];
  }
  const bool qok = qrow < N;
  float ndsum, lse2;  // -D and LSE log2(e) of this lane's row
  if constexpr (STATS) {
    // D = dO . O: per 8-column chunk an fma chain, then a pairwise tree over
    // the chunks in column order (lane l and l^32 hold alternate chunks)
    float part[NQC];
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaf((float)oreg[cc][e], (float)doreg[cc][e], a);
      part[cc] = a;
    }
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) part[cc] += __shfl_xor(part[cc], 32);
#pragma unroll
    for (int m = 1; m < NQC; m <<= 1)
#pragma unroll
      for (int i = 0; i < NQC; i += 2 * m) part[i] += part[i + m];
    ndsum = -part[0];  // rows past N read zeros: -0
    lse2 = qok ? lse_row * kLog2e : 0.f;
    if (hf == 0 && qrow < (VARLEN ? N : Np)) {
      st[qrow] = ndsum;
      st[Np + qrow] = lse2;
    }
  } else {
    ndsum = qok ? st[qrow] : 0.f;
    lse2 = qok ? st[Np + qrow] : 0.f;
  }
  f32x16 pinit;  // seeds dP^T - D
#pragma unroll
  for (int r = 0; r < 16; ++r) pinit[r] = ndsum;


  int koff[NQC], troff[2][NMB];
#pragma unroll
  for (int cc = 0; cc < NQC; ++cc) koff[cc] = tile_off<D>(l32, 2 * cc + hf);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) troff[t][mb] = tr_off<D>(lane, 0, mb * 32, t);

  f32x16 dqacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dqacc[mb] = f32x16{};

  // The operand reads of both products stream two products ahead of their
  // use, as in the dK/dV kernel (which gives the measurements of the one-wave
  // layouts; here with several waves per SIMD, against reads two chunks at a
  // time behind scheduling fences: causal B=4 H=32 N=4000 d=128 +1.3%,
  // non-causal B=2 H=32 N=4096 d=128 +1.1%, d=64 +0.1 to +0.6%; one ahead
  // lost 1%).  A fence that kept a tile's two key blocks apart (for tight
  // register budgets) is gone: with the streamed reads it cost 0.5-2.6% at
  // d = 64 and nothing at d = 128, at the same register counts.

  auto tile = [&](auto bufc, int j) {
    constexpr int BUF = decltype(bufc)::value;
    const char* kt = smem + BUF * 2 * TILEB;
    const char* vt = kt + TILEB;
    if (j + NBUF - 1 < ntiles) issue(j + NBUF - 1);
    if (j < wtiles && q0 < N) {
      const int k0 = j * BC;
      const bool edge = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > q0));  // diagonal, tail
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        // S^T = K Q^T and dP^T - D = V dO^T - D for the tile's 32-key block kbk
        f32x16 sacc = f32x16{}, pacc = pinit;
        {
          constexpr int LA = 2;  // chunks read ahead
          u32x4 ka[NQC], va[NQC];
          auto rd = [&](int cc) __attribute__((always_inline)) {
            ka[cc] = lds_read16(kt + kbk * 32 * ROWB + koff[cc]);
            va[cc] = lds_read16(vt + kbk * 32 * ROWB + koff[cc]);
          };
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cc = 0; cc < LA; ++cc) rd(cc);
#pragma unroll
          for (int cc = 0; cc < NQC; ++cc) {
            if (cc + LA < NQC) rd(cc + LA);
            sacc = mfma32(bitcast<V8>(ka[cc]), qreg[cc], sacc);
            pacc = mfma32(bitcast<V8>(va[cc]), doreg[cc], pacc);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
          for (int cc = 0; cc < NQC; ++cc) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (cc + LA < NQC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(__builtin_fmaf(sacc[r], c, -lse2));
        if (edge) {
          __asm__ volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kbk * 32 + acc_row(r, hf);
            if (key >= N || (CAUSAL && key > qrow)) pv[r] = 0.f;
          }
        }
        uint32_t dsk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          dsk[r >> 1] = pack2<T>(pv[r] * pacc[r], pv[r + 1] * pacc[r + 1]);
        // dQ^T += K^T dS^T (per mb the same accumulation order as key block
        // by key block)
        {
          constexpr int LA = 2, NI = 2 * NMB;  // products read ahead; product i: block mb = i / 2, half cp = i % 2
          u32x2 lo[NI], hi[NI];
          auto rd = [&](int i) __attribute__((always_inline)) {
            const int rows = (kbk * 32 + (i % 2) * 16) * ROWB;
            lo[i] = lds_read_tr(kt + rows + troff[0][i / 2]);
            hi[i] = lds_read_tr(kt + rows + troff[1][i / 2]);
          };
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < LA; ++i) rd(i);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if (i + LA < NI) rd(i + LA);
            const int cp = i % 2;
            const V8 a = bitcast<V8>(u32x4{lo[i][0], lo[i][1], hi[i][0], hi[i][1]});
            const V8 sb = bitcast<V8>(
                u32x4{dsk[4 * cp], dsk[4 * cp + 1], dsk[4 * cp + 2], dsk[4 * cp + 3]});
            dqacc[i / 2] = mfma32(a, sb, dqacc[i / 2]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + LA < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (j + 1 < ntiles) {
      if (NBUF == 3 && j + 2 < ntiles)
        wait_vm_barrier<2 * PW>();
      else
        wait_vm_barrier<0>();
    }
  };

  if (NBUF == 3 && ntiles > 1)
    wait_vm_barrier<2 * PW>();
  else
    wait_vm_barrier<0>();
  for (int j = 0; j < ntiles; j += NBUF) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1);
    if constexpr (NBUF == 3)
      if (j + 2 < ntiles) tile(std::integral_constant<int, 2 % NBUF>{}, j + 2);
  }

  if (qok) {
    T* dst = dQ + qoff + (int64_t)qrow * qrs;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        u32x2 v;
        v[0] = pack2<T>(dqacc[mb][4 * rg] * qscale, dqacc[mb][4 * rg + 1] * qscale);
        v[1] = pack2<T>(dqacc[mb][4 * rg + 2] * qscale, dqacc[mb][4 * rg + 3] * qscale);
        *(u32x2*)(dst + d0) = v;
      }
  }
}

// ---------------------------------------------------------------- launchers
// The strides a launch uses: the caller's, or the dense ones ([B, H, N, d],
// or [H, T, d] for packed sequences).
static Layout layout_of(const BwdArgs& a) {
  if (a.lay.q.r) return a.lay;
  return a.cu_seqlens ? dense_layout(a.Hq, a.Hkv, a.T, a.d) : dense_layout(a.Hq, a.Hkv, a.N, a.d);
}

size_t bwd_stats_bytes(int B, int Hq, int N) {
  return (size_t)B * Hq * 2 * stat_rows(N) * sizeof(float);
}

struct BwdConsts {
  float c;         // |scale| log2(e), at least the smallest normal
  uint32_t qsign;  // sign bits XORed into Q when scale < 0
};

static BwdConsts bwd_consts(float scale) {
  float c = fabsf(scale) * kLog2e;
  if (!(c >= kTiny)) c = kTiny;  // scale 0: uniform probabilities, zero dQ/dK
  return BwdConsts{c, (scale < 0.f) ? 0x80008000u : 0u};
}

template <typename T, int D>
static hipError_t pre_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int Np = stat_rows(a.N);
  const int64_t nslices = (int64_t)a.B * a.Hq;
  const int64_t grid = (nslices * Np + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const T*)a.o, (const T*)a.dout, a.lse, a.stats, a.N, Np, nslices, a.Hq,
                     layout_of(a).o);
  return hipGetLastError();
}

// Slice groups of the XCD-aware orders (xcd_group).  dQ: K/V of a slice,
// shared by the query heads of a kv group, as in the forward.  dK/dV: the Q
// and dO tiles of a kv group's query heads, per (batch, kv head) slice,
// non-causal only: under the causal mask its slice groups cost the
// heaviest-first order more than they saved (same-box A/B of attn_bwd: dQ
// groups +3% at causal B=4 H=32 N=4000 d=128 and +4% non-causal N=1024;
// dK/dV groups +2% non-causal, but -3% causal N=2048 and -2% causal
// grouped-query N=4096).  Packed variable-length slices differ in work and
// keep the plain order, with each sequence's heads permuted (xcd_head) so
// that an XCD takes whole kv groups.
static int dq_xcd_group(const BwdArgs& a, int D, bool varlen) {
  if (varlen) return 0;
  const int64_t nsl = (int64_t)a.B * a.Hq;
  const int group = a.Hq / a.Hkv;
  const int64_t bytes = (int64_t)a.N * D * 4;
  return a.causal ? xcd_group_causal(nsl, group, bytes) : xcd_group(nsl, group, bytes, kXgBudget);
}
static int dkdv_xcd_group(const BwdArgs& a, int D, bool varlen) {
  if (varlen || a.causal) return 0;
  return xcd_group((int64_t)a.B * a.Hkv, 1, (int64_t)(a.Hq / a.Hkv) * a.N * D * 4, kXgBudget);
}

// For packed variable-length sequences B is the number of sequences and N the
// longest one (they size the grid); the statistics cover the T packed tokens.
template <typename T, int D, bool CAUSAL, bool VARLEN>
static hipError_t dkdv_t(const BwdArgs& a) {
  using Cfg = DkdvCfg<D>;
  const BwdConsts k = bwd_consts(a.scale);
  const int nkb = (a.N + Cfg::BKV - 1) / Cfg::BKV;
  const int nsplit = a.nsplit;
  if (nsplit > 1 && a.part == nullptr) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)nkb * a.B * a.Hkv * nsplit;
  const Layout lay = layout_of(a);
  const int desc = a.causal ? 1 : 0;  // descending query-tile walk (qtile_of)
  if (nsplit > 1) {
    constexpr size_t lds = DkdvCfg<D, CAUSAL>::LDS;
    const hipError_t e = allow_lds(bwd_dkdv_kernel<T, D, CAUSAL, VARLEN, true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, VARLEN, true>), dim3((unsigned)grid),
                       dim3(256), lds, a.stream, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, a.stats, (T*)a.dk, (T*)a.dv, a.Hq,
                       a.Hkv, a.N, nkb, 0, desc, lay, k.c, a.scale, k.qsign, a.cu_seqlens, a.T, nsplit,
                       a.part);
  } else {
    const hipError_t e = allow_lds(bwd_dkdv_kernel<T, D, CAUSAL, VARLEN, false>, Cfg::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, VARLEN, false>), dim3((unsigned)grid),
                       dim3(256), Cfg::LDS, a.stream, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, a.stats, (T*)a.dk, (T*)a.dv, a.Hq, a.Hkv,
                       a.N, nkb, dkdv_xcd_group(a, D, VARLEN), desc, lay, k.c, a.scale, k.qsign,
                       a.cu_seqlens, a.T, 1, a.part);
  }
  if (nsplit > 1) {
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    // packed sequences: rows (kv head, token) over all T tokens
    const int BG = VARLEN ? a.Hkv : a.B * a.Hkv, Nr = VARLEN ? a.T : a.N;
    const int64_t threads = (int64_t)BG * Nr * (D / 8);
    hipLaunchKernelGGL((bwd_dkdv_merge_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, a.stream, (const float*)a.part, (T*)a.dk, (T*)a.dv, nsplit,
                       BG, a.Hkv, Nr, a.scale, lay.kv, VARLEN ? a.cu_seqlens : nullptr, a.B);
  }
  return hipGetLastError();
}

// Query-head splits of the dK/dV stage.  Its grid is key blocks x (batch, kv
// head); for grouped-query problems with few kv heads or short sequences it
// can leave most of the device idle, since every workgroup walks all query
// heads of its group.  Then the heads are split over more workgroups: the
// smallest divisor of the group that gives at least two rounds of resident
// workgroups (256 CUs x workgroups per CU), or one split per head.
int bwd_dkdv_splits(int B, int Hq, int Hkv, int N, int d) {
  const int group = Hq / Hkv;
  if (group <= 1) return 1;
  const int per_cu = d == 64 ? DkdvCfg<64>::WPE : 1;
  const int64_t target = 2LL * 256 * per_cu;
  const int64_t grid = (int64_t)((N + DkdvCfg<64>::BKV - 1) / DkdvCfg<64>::BKV) * B * Hkv;
  if (grid >= target) return 1;
  const int64_t need = (target + grid - 1) / grid;
  for (int s = 2; s < group; ++s)
    if (group % s == 0 && s >= need) return s;
  return group;
}

size_t bwd_partial_bytes(int B, int Hkv, int N, int d, int nsplit) {
  return nsplit > 1 ? (size_t)2 * nsplit * B * Hkv * N * d * sizeof(float) : 0;
}

template <typename T, int D, bool CAUSAL, bool VARLEN, bool STATS = false>
static hipError_t dq_t(const BwdArgs& a) {
  using Cfg = DqCfg<D>;
  const BwdConsts k = bwd_consts(a.scale);
  const int nqb = (a.N + Cfg::BR - 1) / Cfg::BR;
  const int64_t grid = (int64_t)nqb * a.B * a.Hq;
  const hipError_t e = allow_lds(bwd_dq_kernel<T, D, CAUSAL, VARLEN, STATS>, Cfg::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, VARLEN, STATS>), dim3((unsigned)grid),
                     dim3(256), Cfg::LDS, a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.dout, (const T*)a.o, a.lse, a.stats, (T*)a.dq, a.Hq, a.Hkv, a.N,
                     nqb, dq_xcd_group(a, D, VARLEN), layout_of(a), k.c, a.scale, k.qsign,
                     a.cu_seqlens, a.T);
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_pre_for(const BwdArgs& a) {
  if (a.d == 64) return pre_t<T, 64>(a);
  return a.d == 128 ? pre_t<T, 128>(a) : pre_t<T, 256>(a);
}
template <typename T, int D>
static hipError_t dkdv_d(const BwdArgs& a) {
  if (a.cu_seqlens)
    return a.causal ? dkdv_t<T, D, true, true>(a) : dkdv_t<T, D, false, true>(a);
  return a.causal ? dkdv_t<T, D, true, false>(a) : dkdv_t<T, D, false, false>(a);
}
template <typename T>
static hipError_t bwd_dkdv_for(const BwdArgs& a) {
  if (a.d == 64) return dkdv_d<T, 64>(a);
  return a.d == 128 ? dkdv_d<T, 128>(a) : dkdv_d<T, 256>(a);
}
template <typename T, int D>
static hipError_t dq_d(const BwdArgs& a) {
  if (a.cu_seqlens) return a.causal ? dq_t<T, D, true, true>(a) : dq_t<T, D, false, true>(a);
  return a.causal ? dq_t<T, D, true, false>(a) : dq_t<T, D, false, false>(a);
}
template <typename T>
static hipError_t bwd_dq_for(const BwdArgs& a) {
  if (a.d == 64) return dq_d<T, 64>(a);
  return a.d == 128 ? dq_d<T, 128>(a) : dq_d<T, 256>(a);
}
template <typename T, int D>
static hipError_t dq_stats_d(const BwdArgs& a) {
  if (a.cu_seqlens)
    return a.causal ? dq_t<T, D, true, true, true>(a) : dq_t<T, D, false, true, true>(a);
  return a.causal ? dq_t<T, D, true, false, true>(a) : dq_t<T, D, false, false, true>(a);
}
template <typename T>
static hipError_t bwd_dq_stats_for(const BwdArgs& a) {
  if (a.d == 64) return dq_stats_d<T, 64>(a);
  return a.d == 128 ? dq_stats_d<T, 128>(a) : dq_stats_d<T, 256>(a);
}

hipError_t launch_bwd_pre(const BwdArgs& a) {
  if (a.dtype == kBF16) return bwd_pre_for<__bf16>(a);
  if (a.dtype == kF16) return bwd_pre_for<_Float16>(a);
  return hipErrorNotSupported;
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  if (a.dtype == kBF16) return bwd_dkdv_for<__bf16>(a);
  if (a.dtype == kF16) return bwd_dkdv_for<_Float16>(a);
  return hipErrorNotSupported;
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  if (a.dtype == kBF16) return bwd_dq_for<__bf16>(a);
  if (a.dtype == kF16) return bwd_dq_for<_Float16>(a);
  return hipErrorNotSupported;
}

hipError_t launch_bwd_dq_stats(const BwdArgs& a) {
  if (a.dtype == kBF16) return bwd_dq_stats_for<__bf16>(a);
  if (a.dtype == kF16) return bwd_dq_stats_for<_Float16>(a);
  return hipErrorNotSupported;
}

}  // namespace attn
