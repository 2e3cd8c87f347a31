// Forward pass of exact attention for gfx950.
//
// Method (FlashAttention pages: "FlashAttention" paper story, tiling and
// online-softmax passages and the conceptual forward pass; wineandchord.com
// page, section "Online softmax"): a workgroup keeps a block of query rows on
// chip and streams key/value tiles through LDS.  For every tile it forms the
// scores, updates each row's running maximum m and normaliser l, rescales the
// output accumulator by 2^(m_old - m_new) when m grows, and accumulates P V.
// The N x N score matrix never leaves the chip; only O and the per-row
// logsumexp are written.
//
// bf16 kernel layout (one wave = 32 query rows, 4 waves per workgroup):
//   S^T = K Q^T on the 32x32x16 bf16 matrix cores: K tile rows come from LDS,
//     Q^T stays in registers for the whole key loop.  Each lane then owns one
//     query column and 32 of the tile's 64 keys, so the row max and sum are
//     in-lane reductions plus one exchange with lane l^32.
//   O^T += V^T P^T: P^T is reused straight from the score registers (the key
//     order of the accumulator is carried into V's transposing LDS read), so
//     the per-row rescale is a per-lane multiply.
//   Softmax runs in base 2: p = 2^(s*c - m) with c = |scale|*log2(e), one FMA
//   and one v_exp_f32 per score.  The running maximum is only moved when a
//   row's tile maximum exceeds it by more than kTau (then p <= 2^kTau); the
//   final O = acc / l and LSE use the same m, so the result is unchanged.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {


// Fair wave priority of the plain kernel where it runs without the
// matrix-core phase priority (d = 64), non-causal grids only: each wave's
// priority falls by one level per kFairTiles of its remaining key tiles.  Four
// waves of four workgroups share a SIMD; with equal priority the oldest wins,
// so they finish staggered and the SIMD ends the grid with fewer and fewer
// waves to hide latency.  Measured (same-box A/B): non-causal B=8 H=16 N=1024
// d=64 +4.7%, B=4 H=32 N=2048 +2.5%; causal grids lost 1-4% (heaviest-first
// already orders them), so they keep equal priority.
constexpr int kFairTiles = 4;

// Work map of the forward grids (nqb query blocks x BH (batch, head) slices):
// the heaviest query blocks first under the causal mask; the heads of one
// kv group are adjacent.
// Work map: (query block, slice) from the XCD-aware order (xcd_item); the
// heaviest query blocks first under the causal mask.
template <bool CAUSAL>
__device__ __forceinline__ void work_item(int nqb, int BH, int xg, int& qb, int& bh) {
  int qi;
  xcd_item(nqb, BH, xg, qi, bh);
  qb = CAUSAL ? nqb - 1 - qi : qi;
}

// Per head dim: a value for d = 64, 128 and 256.
template <int D>
constexpr int by_dim(int v64, int v128, int v256) {
  return D == 64 ? v64 : D == 128 ? v128 : v256;
}

// Plain (not software-pipelined) kernel, used at d = 64 and d = 256.
//   d = 64: four waves per SIMD (121 registers) with two LDS stages (32 KiB
//     per workgroup, four workgroups per CU); three waves with three stages
//     was 3-8% slower, and two 32-row blocks per wave (two waves per
//     workgroup) 25-30% slower.
//   d = 256: one wave per SIMD (256 VGPRs + 256 AGPRs), two stages (128 KiB).
//     The software-pipelined kernel spills thousands of registers at this
//     head dimension.
template <int D>
struct FwdCfg {
  static constexpr int NW = 4;             // waves per workgroup
  static constexpr int NB = 1;             // 32-row blocks per wave
  static constexpr int BR = 32 * NB * NW;  // query rows per workgroup
  static constexpr int BC = 64;            // keys per tile
  static constexpr int NBUF = 2;           // LDS stages
  static constexpr int WPE = by_dim<D>(4, 2, 1);  // waves per SIMD
  static constexpr int TILEB = BC * D * 2;
  static constexpr size_t LDS = (size_t)NBUF * 2 * TILEB;
};

template <typename T, int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(64 * FwdCfg<D>::NW)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WPE, FwdCfg<D>::WPE))) void fwd_mfma_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nmax, int nqb, int xg, float c,
    uint32_t qsign, const int* __restrict__ tlist, const int* __restrict__ tcount,
    int mask_heads, const int* __restrict__ cu_seqlens, int ntok, Layout lay) {
  constexpr bool SPARSE = MODE == kFwdSparse;
  using V8 = typename Elem<T>::v8;
  using Cfg = FwdCfg<D>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, NBUF = Cfg::NBUF, TILEB = Cfg::TILEB;
  constexpr int NB = Cfg::NB;  // 32-row query blocks per wave (each K/V fragment feeds NB products)
  constexpr int ROWB = D * 2;
  constexpr int NW = Cfg::NW;
  constexpr int PW = TILEB / 1024 / NW;  // 1 KiB direct loads per wave per tensor per tile
  static_assert(PW * NW * 1024 == TILEB, "tile pieces");
  constexpr int NQC = D / 16;  // k-chunks of the S contraction
  constexpr int NMB = D / 32;  // 32-row blocks of O^T
  // Raised wave priority around the matrix-core products (s_setprio 1) at
  // d = 256; not at d = 64, where four waves share a SIMD and it cost 1-3%.
  constexpr bool PRIO = D != 64;

  extern __shared__ __attribute__((aligned(16))) char smem[];  // [NBUF][K tile | V tile]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Work map: heaviest query blocks first for the causal case; the heads of
  // one key/value group are adjacent so they share K/V in cache.
  const int BH = gridDim.x / nqb;
  int qb, bh;
  work_item<CAUSAL>(nqb, BH, xg, qb, bh);
  // This workgroup's problem: one (batch, head) slice of Nmax rows, or, for a
  // packed variable-length batch, one (sequence, head) of the packed tokens;
  // offsets are in elements of Q/O, of K/V and in entries of LSE.
  int N = Nmax, h;
  int64_t qoff, kvoff, ooff, lbase;
  int qrs = D, krs = D, ors = D;  // row strides (elements) of Q, K/V and O
  if constexpr (MODE == kFwdVarlen) {
    const int seq = bh / Hq;
    h = xcd_head(bh - seq * Hq, Hq);  // xg is 0 here: the plain order
    const int start = min(max(cu_seqlens[seq], 0), ntok);
    const int end = min(max(cu_seqlens[seq + 1], start), ntok);
    N = end - start;
    if (qb * BR >= N) return;  // the whole workgroup: past this sequence's end
    const int g = h / (Hq / Hkv);
    // (head, token) strides; the batch strides are unused
    qoff = h * lay.q.h + (int64_t)start * lay.q.r;
    kvoff = g * lay.kv.h + (int64_t)start * lay.kv.r;
    ooff = h * lay.o.h + (int64_t)start * lay.o.r;
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    lbase = (int64_t)h * ntok + start;
  } else {
    const int b = bh / Hq;
    h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    qoff = b * lay.q.b + h * lay.q.h;
    kvoff = b * lay.kv.b + g * lay.kv.h;
    ooff = b * lay.o.b + h * lay.o.h;
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    lbase = (int64_t)bh * N;
  }
  const int q0 = qb * BR + w * 32 * NB;  // first query row of this wave

  // Each (batch, head) slice is one raw buffer ending after row N-1; rows
  // past N read as zero.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qoff, slice_bytes(N, qrs, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kvoff, slice_bytes(N, krs, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kvoff, slice_bytes(N, krs, D));

  // Q^T operands (one per 32-row block), resident for the whole key loop.
  V8 qreg[NB][NQC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc)
      qreg[nb][cc] = bitcast<V8>(
          buf_load16(rq, (uint32_t)(((q0 + nb * 32 + l32) * qrs + cc * 16 + hf * 8) * 2)) ^ qsign);

  const int ntiles_all = (N + BC - 1) / BC;
  int ntiles = ntiles_all;
  int wtiles = ntiles_all;
  if (CAUSAL) {
    ntiles = min(ntiles_all, (qb * BR + BR - 1) / BC + 1);
    wtiles = min(ntiles, (q0 + 32 * NB - 1) / BC + 1);
  }
  // Causal: a wave whose rows all lie past the slice's end (the last, partial
  // query block) computes nothing; it still shares the workgroup's loads and
  // barriers.  (Not under a non-causal mask: there every wave is active on
  // every tile, and the compiler drops the activity test altogether.)
  if (CAUSAL && q0 >= N) wtiles = 0;
  // Block-sparse: the key tiles of this query block's mask row (ascending,
  // already cut at the causal diagonal), copied to LDS after the stages as
  // 16-bit indices; loop position j then loads tile tiles[j].
  unsigned short* tl = (unsigned short*)(smem + NBUF * 2 * TILEB);
  if constexpr (SPARSE) {
    const int64_t mrow = (int64_t)(mask_heads == 1 ? 0 : h) * nqb + qb;
    ntiles = wtiles = tcount[mrow];
    const int* src = tlist + mrow * ntiles_all;
    for (int t = threadIdx.x; t < ntiles; t += 64 * NW) tl[t] = (unsigned short)src[t];
    __syncthreads();
  }
  auto tile_of = [&](int j) -> int {
    if constexpr (SPARSE)
      return __builtin_amdgcn_readfirstlane((int)tl[j]);
    else
      return j;
  };
  // does this wave have visible keys in loop position j (< ntiles)?
  auto wave_active = [&](int j) -> bool {
    if constexpr (SPARSE)
      return !CAUSAL || (q0 < N && tile_of(j) * BC <= q0 + 32 * NB - 1);
    else
      return j < wtiles;
  };

  // Direct global->LDS tile loads.  Wave w fills the 1 KiB pieces
  // w*PW .. w*PW+PW-1 of each tile; lane l of piece i lands at byte
  // 1024*i' + 16*l, i.e. at (row, physical chunk), and fetches the logical
  // chunk the swizzle stores there.
  uint32_t goff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int o = (w * PW + i) * 1024 + lane * 16;
    const int row = o / ROWB;
    const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
    goff[i] = (uint32_t)((row * krs + ch * 8) * 2);
  }
  auto issue = [&](int j) {
    char* kt = smem + (j % NBUF) * 2 * TILEB;  // j % NBUF is the stage tile j uses
    char* vt = kt + TILEB;
    const uint32_t tbase = (uint32_t)(tile_of(j) * BC * krs * 2);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      buf_load16_lds(rk, kt + (w * PW + i) * 1024, goff[i] + tbase);
      buf_load16_lds(rv, vt + (w * PW + i) * 1024, goff[i] + tbase);
    }
  };

  // Per-lane LDS byte offsets inside one tile, fixed for the whole loop: the
  // K operand rows (l32, +32) at chunk 2cc+hf, and the transposing-read
  // addresses of the V^T operand for key block 0 (other key blocks are
  // multiples of 16 rows further, which the swizzle leaves unchanged).
  // At d = 256 only half of them are kept: the swizzle permutes chunks
  // within aligned groups of 16, so chunk c + 16 lies 256 bytes after chunk
  // c, an immediate of the LDS read.
  constexpr int NKO = D > 128 ? NQC / 2 : NQC, NVO = D > 128 ? NMB / 2 : NMB;
  int koff_[NKO], voff_[2][NVO];
#pragma unroll
  for (int cc = 0; cc < NKO; ++cc) koff_[cc] = tile_off<D>(l32, 2 * cc + hf);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < NVO; ++mb) voff_[t][mb] = tr_off<D>(lane, 0, mb * 32, t);
  auto koff = [&](int cc) __attribute__((always_inline)) {
    return koff_[cc % NKO] + (cc / NKO) * 256;
  };
  auto voff = [&](int t, int mb) __attribute__((always_inline)) {
    return voff_[t][mb % NVO] + (mb / NVO) * 256;
  };

  float ms[NB], lsum[NB];  // running max (scaled base-2 units), this lane's share of l
  f32x16 oacc[NB][NMB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ms[nb] = -3.402823466e38f;  // finite: a row may see no key (block-sparse)
    lsum[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) oacc[nb][mb] = f32x16{};
  }

  // One key tile of a wave (d = 64 and 256; d = 128 runs the
  // software-pipelined kernel below):
  //   - K and V^T fragments are read a few products ahead of their use (K 4
  //     ahead at d = 256, 2 at d = 64; V^T pairs 2 ahead), pinned with
  //     scheduling groups;
  //   - the scores are copied once out of the product accumulators into
  //     plain values for the mask and the softmax;
  //   - on a wave's first tile (loop position 0: its first tile with visible
  //     keys, also under a block-sparse list, which is ascending) the running
  //     max, not set yet, is taken from the masked scores up front; forming p
  //     against the unset max always overflowed and was thrown away;
  //   - otherwise p is formed against the running max, and only a lane whose
  //     tile sum exceeds 2^kTau takes the row max; if that grew by more than
  //     kTau, O is rescaled.
  // d = 256 runs one wave per SIMD, so nothing else hides a wave's own
  // stalls, and at 512 registers every product accumulator lives in the
  // accumulation registers, which the vector ALU reaches only through
  // copies.  The O rescale therefore multiplies O in place behind an empty
  // asm that pins O to those registers, so O is copied out and back on that
  // rare path only; written plainly, the compiler kept a vector copy of all
  // of O at hand and moved it on every tile (about 270 extra copies per
  // tile).  Measured against the previous body (all K fragments of a key
  // block read before its products, the V^T reads left to the compiler, the
  // rescale written plainly; same arithmetic, bitwise-equal results,
  // same-box rotated A/B): d = 256 non-causal B=1 H=16 N=8192 887 -> 1058
  // TFLOP/s (+19%), causal 843 -> 997 (+18%), causal grouped-query B=2
  // Hq=16 Hkv=2 N=4096 804 -> 930 (+16%), fp16 non-causal B=4 H=16 N=2048
  // 786 -> 914 (+16%); d = 64 (four waves per SIMD) +0.2 to +1.4% (causal
  // B=8 H=16 N=2048 812 -> 824).  (Scaling each O block inside a second copy
  // of the P V loop instead measured 1% slower non-causal and 9% slower
  // causal at d = 256.)
  auto tile_body = [&](const char* kt, const char* vt, int j) __attribute__((always_inline)) {
    static_assert(NB == 1, "the tile body serves one 32-row query block per wave");
    constexpr int NF = 2 * NQC, KLA = D == 256 ? 4 : 2;  // score products; K fragments read ahead
    f32x16 sacc2[2];
    {
      u32x4 kf[NF];
      auto kread = [&](int i) __attribute__((always_inline)) {
        kf[i] = lds_read16(kt + (i / NQC) * 32 * ROWB + koff(i % NQC));
      };
      __builtin_amdgcn_sched_barrier(0);
      if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < KLA; ++i) kread(i);
      sacc2[0] = f32x16{};
      sacc2[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        if (i + KLA < NF) kread(i + KLA);
        sacc2[i / NQC] = mfma32(bitcast<V8>(kf[i]), qreg[0][i % NQC], sacc2[i / NQC]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KLA, 0);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + KLA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (PRIO) __builtin_amdgcn_s_setprio(0);
    }
    float sv[2][16];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[kbk][r] = sacc2[kbk][r];
    const int k0 = tile_of(j) * BC;
    if ((k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > q0))) {
      __asm__ volatile("");
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kbk * 32 + acc_row(r, hf);
          if ((key >= N) || (CAUSAL && key > q0 + l32)) sv[kbk][r] = -__builtin_inff();
        }
    }
    if (j == 0) {  // first tile: the running maximum is set from it up front
      float mloc = sv[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = __builtin_fmaxf(mloc, sv[kbk][r]);
      mloc = __builtin_fmaxf(mloc, xor32(mloc));
      ms[0] = __builtin_fmaxf(ms[0], mloc * c);
    }
    uint32_t pk[2][8];
    auto expo = [&](float m) __attribute__((always_inline)) {
      float ts = 0.f;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sv[kbk][r], c, -m));
          const float p1 = fast_exp2(__builtin_fmaf(sv[kbk][r + 1], c, -m));
          pk[kbk][r >> 1] = pack2<T>(p0, p1);
          ts += p0 + p1;
        }
      return ts;
    };
    float tsum = expo(ms[0]);
    bool rescale = false;
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(!(tsum <= kSumMax<T>)) != 0) {
      __asm__ volatile("");
      float mloc = sv[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = __builtin_fmaxf(mloc, sv[kbk][r]);
      mloc = __builtin_fmaxf(mloc, xor32(mloc));
      const float tmax = mloc * c;
      if (__builtin_amdgcn_ballot_w64(tmax > ms[0] + kTau<T>) != 0) {
        const float mnew = __builtin_fmaxf(ms[0], tmax);
        alpha = fast_exp2(ms[0] - mnew);
        ms[0] = mnew;
        lsum[0] *= alpha;
        rescale = true;
        tsum = expo(ms[0]);
      }
    }
    lsum[0] += tsum;
    // O^T += V^T P^T; product i: O block mb = i/4, key block (i/2)%2, half i%2
    auto pv = [&]() __attribute__((always_inline)) {
      constexpr int NP = NMB * 4, VLA = 2;  // V^T fragment pairs read ahead
      u32x2 vlo[NP], vhi[NP];
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int rows = (((i / 2) % 2) * 32 + (i % 2) * 16) * ROWB;
        vlo[i] = lds_read_tr(vt + rows + voff(0, i / 4));
        vhi[i] = lds_read_tr(vt + rows + voff(1, i / 4));
      };
      __builtin_amdgcn_sched_barrier(0);
      if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < VLA; ++i) vread(i);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + VLA < NP) vread(i + VLA);
        const int kbk = (i / 2) % 2, cp = i % 2;
        const V8 a = bitcast<V8>(u32x4{vlo[i][0], vlo[i][1], vhi[i][0], vhi[i][1]});
        const V8 bp = bitcast<V8>(
            u32x4{pk[kbk][4 * cp], pk[kbk][4 * cp + 1], pk[kbk][4 * cp + 2], pk[kbk][4 * cp + 3]});
        oacc[0][i / 4] = mfma32(a, bp, oacc[0][i / 4]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * VLA, 0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + VLA < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (PRIO) __builtin_amdgcn_s_setprio(0);
    };
    // (after pv's definition on purpose: placed before it, the same code
    // left the allocator spilling 10-80 registers)
    if (rescale) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        f32x16 o = oacc[0][mb];
        if constexpr (D == 256) __asm__ volatile("" : "+a"(o));
        oacc[0][mb] = o * alpha;
      }
    }
    pv();
  };

  // One key tile; BUF (the LDS stage) is a compile-time constant so every LDS
  // address is a fixed per-lane register plus an immediate.
  auto tile = [&](auto bufc, int j) {
    constexpr int BUF = decltype(bufc)::value;
    const char* kt = smem + BUF * 2 * TILEB;
    const char* vt = kt + TILEB;
    if constexpr (!PRIO && !CAUSAL) {
      const int rem = ntiles - j;  // wave-uniform
      if (rem > 3 * kFairTiles)
        __builtin_amdgcn_s_setprio(3);
      else if (rem > 2 * kFairTiles)
        __builtin_amdgcn_s_setprio(2);
      else if (rem > kFairTiles)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    if (j + NBUF - 1 < ntiles) issue(j + NBUF - 1);
    if (wave_active(j)) {
      tile_body(kt, vt, j);
    }
    if (j + 1 < ntiles) {
      // tile j+1 must have landed; tile j+2 (three stages) may stay in flight
      if (NBUF == 3 && j + 2 < ntiles)
        wait_vm_barrier<2 * PW>();
      else
        wait_vm_barrier<0>();
    }
  };

  // Prologue: tiles 0 .. NBUF-2 in flight, then wait for tile 0.
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < ntiles) issue(j);
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

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qrow = q0 + nb * 32 + l32;
    const float lfull = lsum[nb] + xor32(lsum[nb]);
    if (qrow < N) {
      const bool any = lfull > 0.f;  // else the row saw no key: O = 0, LSE = -inf
      const float inv = any ? 1.0f / lfull : 0.f;
      T* dst = O + ooff + (int64_t)qrow * ors;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = mb * 32 + rg * 8 + hf * 4;
          u32x2 v;
          v[0] = pack2<T>(oacc[nb][mb][4 * rg] * inv, oacc[nb][mb][4 * rg + 1] * inv);
          v[1] = pack2<T>(oacc[nb][mb][4 * rg + 2] * inv, oacc[nb][mb][4 * rg + 3] * inv);
          *(u32x2*)(dst + d0) = v;
        }
      if (hf == 0)
        LSE[lbase + qrow] =
            any ? (ms[nb] + __builtin_log2f(lfull)) * kLn2 : -__builtin_inff();
    }
  }
}

// Software-pipelined variant of the bf16 forward: while a wave turns the
// scores of key tile j into probabilities (vector ALU work), the matrix cores
// already compute the scores of tile j+1, so the two units overlap inside one
// wave instead of only across waves.  K and V have separate double-buffered
// LDS stages: K(j+2) and V(j+1) are loaded during tile j (K(j) was consumed
// one tile earlier, by the look-ahead score product), so one barrier per tile
// still suffices.  Same arithmetic and results as fwd_mfma_kernel.
// The pipelined kernel runs at d = 128 only.  At d = 64 the plain kernel at
// four waves per SIMD stays ahead (the pipelined one needs more than the 168
// registers of three waves), and at d = 256 the pipelined one spills more.
// Scheduling (same-box A/B each): 12 VALU instructions placed after each
// look-ahead MFMA (10 and 16 measured the same), K-fragment LDS reads 4 MFMAs
// ahead (2: the same; 6 spills and loses 1-10%), raised priority (1) during
// the P V products (+4-6%; 2 or 3 the same) and none during the look-ahead
// scores (raising it there changed nothing); 8 waves per workgroup lost 4%.
template <int D>
struct PipeCfg {
  static_assert(D == 128, "the pipelined forward is tuned for d = 128");
  static constexpr int NW = 4;   // waves per workgroup (32 query rows each)
  static constexpr int BR = 32 * NW;
  static constexpr int BC = 64;
  static constexpr int WPE = 2;  // waves per SIMD (244 registers)
  static constexpr int VPM = 12; // VALU instructions after each look-ahead MFMA
  static constexpr int LA = 4;   // K-fragment LDS reads issued ahead of their MFMA
  static constexpr int TILEB = BC * D * 2;
  static constexpr size_t LDS = (size_t)4 * TILEB;  // K[2] | V[2]
};

template <typename T, int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(64 * PipeCfg<D>::NW)
__attribute__((amdgpu_waves_per_eu(PipeCfg<D>::WPE, PipeCfg<D>::WPE))) void fwd_mfma_pipe_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nmax, int nqb, int xg, float c,
    uint32_t qsign, const int* __restrict__ tlist, const int* __restrict__ tcount,
    int mask_heads, const int* __restrict__ cu_seqlens, int ntok, Layout lay) {
  constexpr bool SPARSE = MODE == kFwdSparse;
  using V8 = typename Elem<T>::v8;
  using Cfg = PipeCfg<D>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, TILEB = Cfg::TILEB, NW = Cfg::NW;
  constexpr int ROWB = D * 2;
  constexpr int PW = TILEB / 1024 / NW;
  static_assert(PW * NW * 1024 == TILEB, "tile pieces");
  constexpr int NQC = D / 16;
  constexpr int NMB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem[];  // K[2] | V[2]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int BH = gridDim.x / nqb;
  int qb, bh;
  work_item<CAUSAL>(nqb, BH, xg, qb, bh);
  // This workgroup's problem: one (batch, head) slice of Nmax rows, or, for a
  // packed variable-length batch, one (sequence, head) of the packed tokens;
  // offsets are in elements of Q/O, of K/V and in entries of LSE.
  int N = Nmax, h;
  int64_t qoff, kvoff, ooff, lbase;
  int qrs = D, krs = D, ors = D;  // row strides (elements) of Q, K/V and O
  if constexpr (MODE == kFwdVarlen) {
    const int seq = bh / Hq;
    h = xcd_head(bh - seq * Hq, Hq);  // xg is 0 here: the plain order
    const int start = min(max(cu_seqlens[seq], 0), ntok);
    const int end = min(max(cu_seqlens[seq + 1], start), ntok);
    N = end - start;
    if (qb * BR >= N) return;  // the whole workgroup: past this sequence's end
    const int g = h / (Hq / Hkv);
    // (head, token) strides; the batch strides are unused
    qoff = h * lay.q.h + (int64_t)start * lay.q.r;
    kvoff = g * lay.kv.h + (int64_t)start * lay.kv.r;
    ooff = h * lay.o.h + (int64_t)start * lay.o.r;
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    lbase = (int64_t)h * ntok + start;
  } else {
    const int b = bh / Hq;
    h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    qoff = b * lay.q.b + h * lay.q.h;
    kvoff = b * lay.kv.b + g * lay.kv.h;
    ooff = b * lay.o.b + h * lay.o.h;
    qrs = lay.q.r, krs = lay.kv.r, ors = lay.o.r;
    lbase = (int64_t)bh * N;
  }
  const int q0 = qb * BR + w * 32;

  // Each (batch, head) slice is one raw buffer ending after row N-1; rows
  // past N read as zero.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qoff, slice_bytes(N, qrs, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kvoff, slice_bytes(N, krs, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kvoff, slice_bytes(N, krs, D));

  V8 qreg[NQC];
#pragma unroll
  for (int cc = 0; cc < NQC; ++cc)
    qreg[cc] = bitcast<V8>(buf_load16(rq, (uint32_t)(((q0 + l32) * qrs + cc * 16 + hf * 8) * 2)) ^ qsign);

  const int ntiles_all = (N + BC - 1) / BC;
  int ntiles = ntiles_all;
  int wtiles = ntiles_all;
  if (CAUSAL) {
    ntiles = min(ntiles_all, (qb * BR + BR - 1) / BC + 1);
    wtiles = min(ntiles, (q0 + 31) / BC + 1);
  }
  // causal: every row of this wave may lie past the slice's end.  Not under a
  // non-causal mask, where the activity test compiles away: there a runtime
  // test made the scheduled tile body spill 303 registers.
  if (CAUSAL && q0 >= N) wtiles = 0;
  // Block-sparse tile list, as in fwd_mfma_kernel (LDS after the stages).
  unsigned short* tl = (unsigned short*)(smem + 4 * TILEB);
  if constexpr (SPARSE) {
    const int64_t mrow = (int64_t)(mask_heads == 1 ? 0 : h) * nqb + qb;
    ntiles = wtiles = tcount[mrow];
    const int* src = tlist + mrow * ntiles_all;
    for (int t = threadIdx.x; t < ntiles; t += 64 * NW) tl[t] = (unsigned short)src[t];
    __syncthreads();
  }
  auto tile_of = [&](int j) -> int {
    if constexpr (SPARSE)
      return __builtin_amdgcn_readfirstlane((int)tl[j]);
    else
      return j;
  };
  auto wave_active = [&](int j) -> bool {  // j < ntiles
    if constexpr (SPARSE)
      return !CAUSAL || (q0 < N && tile_of(j) * BC <= q0 + 31);
    else
      return j < wtiles;
  };

  uint32_t goff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int o = (w * PW + i) * 1024 + lane * 16;
    const int row = o / ROWB;
    const int ch = ((o % ROWB) >> 4) ^ swz<D>(row);
    goff[i] = (uint32_t)((row * krs + ch * 8) * 2);
  }
  auto issue = [&](__amdgpu_buffer_rsrc_t r, char* dst, int j) {
    const uint32_t tbase = (uint32_t)(tile_of(j) * BC * krs * 2);
#pragma unroll
    for (int i = 0; i < PW; ++i) buf_load16_lds(r, dst + (w * PW + i) * 1024, goff[i] + tbase);
  };
  auto kstage = [&](int s) { return smem + s * TILEB; };
  auto vstage = [&](int s) { return smem + (2 + s) * TILEB; };

  int koff[NQC], voff[2][NMB];
#pragma unroll
  for (int cc = 0; cc < NQC; ++cc) koff[cc] = tile_off<D>(l32, 2 * cc + hf);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) voff[t][mb] = tr_off<D>(lane, 0, mb * 32, t);

  float ms = -3.402823466e38f, lsum = 0.f;  // finite: a row may see no key (block-sparse)
  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};

  // S^T of one tile from a K stage.
  auto scores = [&](const char* kt, f32x16 (&sacc)[2]) {
    u32x4 kfrag[2][NQC];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int cc = 0; cc < NQC; ++cc) kfrag[kbk][cc] = lds_read16(kt + kbk * 32 * ROWB + koff[cc]);
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      sacc[kbk] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NQC; ++cc)
        sacc[kbk] = mfma32(bitcast<V8>(kfrag[kbk][cc]), qreg[cc], sacc[kbk]);
    }
  };
  auto softmax_exp = [&](const f32x16 (&sacc)[2], float m, uint32_t (&pk)[2][8]) {
    float tsum = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(sacc[kbk][r], c, -m));
        const float p1 = fast_exp2(__builtin_fmaf(sacc[kbk][r + 1], c, -m));
        pk[kbk][r >> 1] = pack2<T>(p0, p1);
        tsum += p0 + p1;
      }
    return tsum;
  };

  // Tile j: scores sc (already computed) -> P -> O += P V; meanwhile the
  // scores of tile j+1 go to sn.  BUF = j % 2.
  auto tile = [&](auto bufc, int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int BUF = decltype(bufc)::value;
    if (j + 1 < ntiles) issue(rv, vstage(BUF ^ 1), j + 1);
    if (j + 2 < ntiles) issue(rk, kstage(BUF), j + 2);
    if (wave_active(j)) {
      const int k0 = tile_of(j) * BC;
      if ((k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > q0))) {
        __asm__ volatile("");
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kbk * 32 + acc_row(r, hf);
            const bool dead = (key >= N) || (CAUSAL && key > q0 + l32);
            if (dead) sc[kbk][r] = -__builtin_inff();
          }
      }
      if (j == 0) {  // a wave's first tile: the running max is taken up front
        float mloc = sc[0][0];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mloc = __builtin_fmaxf(mloc, sc[kbk][r]);
        mloc = __builtin_fmaxf(mloc, xor32(mloc));
        ms = __builtin_fmaxf(ms, mloc * c);
      }
      uint32_t pk[2][8];
      const char* vt = vstage(BUF);
      const bool ahead = j + 1 < ntiles && wave_active(j + 1);
      float tsum;
      if (ahead) {
        __builtin_amdgcn_sched_barrier(0);
        scores(kstage(BUF ^ 1), sn);
        tsum = softmax_exp(sc, ms, pk);
        {
          // K fragments stream a few MFMAs ahead of their use; the softmax
          // of tile j fills the matrix-core issue gaps.  (Without these
          // scheduling groups the same code is slower than the plain kernel.)
          constexpr int LA = Cfg::LA;
          __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
          for (int i = 0; i < 2 * NQC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (i + LA < 2 * NQC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, Cfg::VPM, 0);  // VALU
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        tsum = softmax_exp(sc, ms, pk);
      }
      if (__builtin_amdgcn_ballot_w64(!(tsum <= kSumMax<T>)) != 0) {
        __asm__ volatile("");
        float mloc = sc[0][0];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mloc = __builtin_fmaxf(mloc, sc[kbk][r]);
        mloc = __builtin_fmaxf(mloc, xor32(mloc));
        const float tmax = mloc * c;
        if (__builtin_amdgcn_ballot_w64(tmax > ms + kTau<T>) != 0) {
          const float mnew = __builtin_fmaxf(ms, tmax);
          const float alpha = fast_exp2(ms - mnew);
          ms = mnew;
          lsum *= alpha;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) oacc[mb] *= alpha;
          tsum = softmax_exp(sc, ms, pk);
        }
      }
      lsum += tsum;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int cp = 0; cp < 2; ++cp) {
            const int rows = (kbk * 32 + cp * 16) * ROWB;
            const u32x2 lo = lds_read_tr(vt + rows + voff[0][mb]);
            const u32x2 hi = lds_read_tr(vt + rows + voff[1][mb]);
            const V8 a = bitcast<V8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
            const V8 bp = bitcast<V8>(
                u32x4{pk[kbk][4 * cp], pk[kbk][4 * cp + 1], pk[kbk][4 * cp + 2], pk[kbk][4 * cp + 3]});
            oacc[mb] = mfma32(a, bp, oacc[mb]);
          }
      __builtin_amdgcn_s_setprio(0);
    }
    // V(j+1) and K(j+2) must have landed, and every wave be done with
    // K(j+1) and V(j), before their stages are refilled.
    if (j + 1 < ntiles) wait_vm_barrier<0>();
  };

  // Prologue: K(0), V(0), K(1) in flight; wait; scores of tile 0.
  if (ntiles > 0) {
    issue(rk, kstage(0), 0);
    issue(rv, vstage(0), 0);
  }
  if (ntiles > 1) issue(rk, kstage(1), 1);
  wait_vm_barrier<0>();
  f32x16 s0[2], s1[2];
  if (0 < ntiles && wave_active(0)) scores(kstage(0), s0);
  // tile 0's first step refills K stage 0 with K(2): every wave must be done
  // reading K(0) first
  wait_vm_barrier<0>();

  for (int j = 0; j < ntiles; j += 2) {
    tile(std::integral_constant<int, 0>{}, j, s0, s1);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1, s1, s0);
  }

  const int qrow = q0 + l32;
  const float lfull = lsum + xor32(lsum);
  if (qrow < N) {
    const bool any = lfull > 0.f;  // else the row saw no key: O = 0, LSE = -inf
    const float inv = any ? 1.0f / lfull : 0.f;
    T* dst = O + ooff + (int64_t)qrow * ors;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = mb * 32 + rg * 8 + hf * 4;
        u32x2 v;
        v[0] = pack2<T>(oacc[mb][4 * rg] * inv, oacc[mb][4 * rg + 1] * inv);
        v[1] = pack2<T>(oacc[mb][4 * rg + 2] * inv, oacc[mb][4 * rg + 3] * inv);
        *(u32x2*)(dst + d0) = v;
      }
    if (hf == 0)
      LSE[lbase + qrow] = any ? (ms + __builtin_log2f(lfull)) * kLn2 : -__builtin_inff();
  }
}

// fp32 forward on the vector ALUs: 32 query rows per workgroup, 8 lanes per
// row, each lane owning D/8 consecutive features; key/value tiles of 32 rows
// in LDS.  Exact online softmax (the maximum moves on every increase).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N, int nqb,
    float cl2) {
  constexpr int BR = 32, BC = 32, DS = D / 8;
  __shared__ float ks[BC][D + 4];
  __shared__ float vs[BC][D + 4];
  const int tid = threadIdx.x;
  const int BH = gridDim.x / nqb;
  const int qb = blockIdx.x / BH;
  const int bh = blockIdx.x % BH;
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int64_t qoff = (int64_t)bh * N * D;
  const int64_t kvoff = (int64_t)(b * Hkv + g) * N * D;
  const int qi = qb * BR + tid / 8;
  const int part = tid % 8;
  const bool qok = qi < N;
  float qv[DS], acc[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    qv[e] = qok ? Q[qoff + (int64_t)qi * D + part * DS + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  int ntiles = (N + BC - 1) / BC;
  if (CAUSAL) ntiles = min(ntiles, (qb * BR + BR - 1) / BC + 1);
  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();
    for (int idx = tid; idx < BC * D; idx += 256) {
      const int r = idx / D, cidx = idx % D;
      const int key = j * BC + r;
      const bool ok = key < N;
      ks[r][cidx] = ok ? K[kvoff + (int64_t)key * D + cidx] : 0.f;
      vs[r][cidx] = ok ? V[kvoff + (int64_t)key * D + cidx] : 0.f;
    }
    __syncthreads();
    float s[BC];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      float part_dot = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) part_dot = __builtin_fmaf(qv[e], ks[jj][part * DS + e], part_dot);
      part_dot += __shfl_xor(part_dot, 1);
      part_dot += __shfl_xor(part_dot, 2);
      part_dot += __shfl_xor(part_dot, 4);
      const int key = j * BC + jj;
      const bool dead = (key >= N) || (CAUSAL && key > qi);
      s[jj] = dead ? -__builtin_inff() : part_dot * cl2;
      tmax = fmaxf(tmax, s[jj]);
    }
    const float mnew = fmaxf(m, tmax);
    const float alpha = exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DS; ++e) acc[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      const float p = exp2f(s[jj] - mnew);
      l += p;
#pragma unroll
      for (int e = 0; e < DS; ++e) acc[e] = __builtin_fmaf(p, vs[jj][part * DS + e], acc[e]);
    }
    m = mnew;
  }
  if (qok) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DS; ++e) O[qoff + (int64_t)qi * D + part * DS + e] = acc[e] * inv;
    if (part == 0) LSE[(int64_t)bh * N + qi] = (m + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------- launchers
// The strides a launch uses: the caller's, or the dense [B, H, N, d] ones.
static Layout layout_of(const FwdArgs& a) {
  if (a.lay.q.r) return a.lay;
  // dense [B, H, N, d], or [H, T, d] for packed sequences
  return a.cu_seqlens ? dense_layout(a.Hq, a.Hkv, a.T, a.d) : dense_layout(a.Hq, a.Hkv, a.N, a.d);
}

// Dynamic LDS of a forward launch: the kernel's stages, plus the 16-bit tile
// list of a block-sparse launch (one entry per key tile, rounded to 16 B).
static size_t sparse_list_bytes(const FwdArgs& a, int BC) {
  return a.tlist ? ((size_t)((a.N + BC - 1) / BC) * 2 + 15) & ~(size_t)15 : 0;
}

// Slice group of the XCD-aware work order: K/V of a slice, shared by the
// query heads of a kv group.  Measured (same-box A/B against the plain
// order): non-causal with 2 MiB groups, +18% at B=8 H=32 N=1024 d=128 and
// +2-5% at d=64; causal grids lost 9% with 2 MiB groups (B=8 H=16 N=2048
// d=64) but gain 1-3% with 8 MiB ones.  Packed variable-length slices differ
// in work and keep the plain order, with each sequence's heads permuted
// (xcd_head) so that an XCD takes whole kv groups.
static int fwd_xcd_group(const FwdArgs& a, int D) {
  if (a.cu_seqlens) return 0;
  const int64_t nsl = (int64_t)a.B * a.Hq, bytes = (int64_t)a.N * D * 4;
  return a.causal ? xcd_group_causal(nsl, a.Hq / a.Hkv, bytes)
                  : xcd_group(nsl, a.Hq / a.Hkv, bytes, kXgBudget);
}

template <typename T, int D, bool CAUSAL, int MODE>
static hipError_t launch_pipe(const FwdArgs& a) {
  constexpr bool SPARSE = MODE == kFwdSparse;
  static_assert(!SPARSE || (PipeCfg<D>::BR == kSparseBlockQ && PipeCfg<D>::BC == kSparseBlockK),
                "block-sparse tiles are the forward's tiles");
  const int nqb = (a.N + PipeCfg<D>::BR - 1) / PipeCfg<D>::BR;
  const int64_t grid = (int64_t)nqb * a.B * a.Hq;
  const size_t lds = PipeCfg<D>::LDS + sparse_list_bytes(a, PipeCfg<D>::BC);
  const hipError_t e = allow_lds(fwd_mfma_pipe_kernel<T, D, CAUSAL, MODE>, lds);
  if (e != hipSuccess) return e;
  float c = fabsf(a.scale) * kLog2e;
  if (!(c >= 1.17549435e-38f)) c = 1.17549435e-38f;  // scale 0: uniform weights
  const uint32_t qsign = (a.scale < 0.f) ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_mfma_pipe_kernel<T, D, CAUSAL, MODE>), dim3((unsigned)grid),
                     dim3(64 * PipeCfg<D>::NW), lds, a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.o, a.lse, a.Hq, a.Hkv, a.N, nqb, fwd_xcd_group(a, D), c, qsign, a.tlist,
                     a.tcount, a.mask_heads, a.cu_seqlens, a.T, layout_of(a));
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, int MODE>
static hipError_t launch_mfma(const FwdArgs& a) {
  constexpr bool SPARSE = MODE == kFwdSparse;
  if constexpr (D == 128) {
    return launch_pipe<T, D, CAUSAL, MODE>(a);
  } else {
    static_assert(!SPARSE || (FwdCfg<D>::BR == kSparseBlockQ && FwdCfg<D>::BC == kSparseBlockK),
                  "block-sparse tiles are the forward's tiles");
    const int nqb = (a.N + FwdCfg<D>::BR - 1) / FwdCfg<D>::BR;
    const int64_t grid = (int64_t)nqb * a.B * a.Hq;
    const size_t lds = FwdCfg<D>::LDS + sparse_list_bytes(a, FwdCfg<D>::BC);
    const hipError_t e = allow_lds(fwd_mfma_kernel<T, D, CAUSAL, MODE>, lds);
    if (e != hipSuccess) return e;
    float c = fabsf(a.scale) * kLog2e;
    if (!(c >= 1.17549435e-38f)) c = 1.17549435e-38f;  // scale 0: uniform weights
    const uint32_t qsign = (a.scale < 0.f) ? 0x80008000u : 0u;
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL, MODE>), dim3((unsigned)grid),
                       dim3(64 * FwdCfg<D>::NW), lds, a.stream, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (T*)a.o, a.lse, a.Hq, a.Hkv, a.N, nqb, fwd_xcd_group(a, D), c, qsign, a.tlist,
                       a.tcount, a.mask_heads, a.cu_seqlens, a.T, layout_of(a));
    return hipGetLastError();
  }
}

// Runtime (head dim, causal, mode) -> kernel instantiation for element type T.
template <typename T>
static hipError_t dispatch_mfma(const FwdArgs& a) {
  // B is the number of sequences and N the longest one for a varlen launch
  const int mode = a.tlist ? kFwdSparse : a.cu_seqlens ? kFwdVarlen : kFwdDense;
  auto pick = [&](auto dc, auto cc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    constexpr bool C = decltype(cc)::value;
    if (mode == kFwdSparse) return launch_mfma<T, D, C, kFwdSparse>(a);
    if (mode == kFwdVarlen) return launch_mfma<T, D, C, kFwdVarlen>(a);
    return launch_mfma<T, D, C, kFwdDense>(a);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I256 = std::integral_constant<int, 256>;
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  if (a.d == 64) return a.causal ? pick(I64{}, Yes{}) : pick(I64{}, No{});
  if (a.d == 128) return a.causal ? pick(I128{}, Yes{}) : pick(I128{}, No{});
  return a.causal ? pick(I256{}, Yes{}) : pick(I256{}, No{});
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const FwdArgs& a) {
  constexpr int BR = 32;
  const int nqb = (a.N + BR - 1) / BR;
  const int64_t grid = (int64_t)nqb * a.B * a.Hq;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.Hq, a.Hkv, a.N, nqb, a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == kBF16) return dispatch_mfma<__bf16>(a);
  if (a.dtype == kF16) return dispatch_mfma<_Float16>(a);
  if (a.d == 64) return a.causal ? launch_f32<64, true>(a) : launch_f32<64, false>(a);
  return a.causal ? launch_f32<128, true>(a) : launch_f32<128, false>(a);
}

}  // namespace attn
