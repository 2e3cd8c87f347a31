// Host-side launch interface between the C ABI (attn_api.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Element types, numbered as the ABI's attn_dtype.
enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Element strides of one [batch, head, row, d] tensor family (d contiguous).
struct Strides3 {
  int64_t b, h;
  int r;
};
// Q (and dQ); K, V (and dK, dV); O (and dO).  r == 0 in q means "dense
// [B, H, N, d]", which the launchers fill in.
struct Layout {
  Strides3 q, kv, o;
};
inline Layout dense_layout(int Hq, int Hkv, int N, int d) {
  const Strides3 q{(int64_t)Hq * N * d, (int64_t)N * d, d};
  const Strides3 kv{(int64_t)Hkv * N * d, (int64_t)N * d, d};
  return Layout{q, kv, q};
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  Dtype dtype;
  hipStream_t stream;
  // Block-sparse (16-bit types only): per mask row (mask head, query block of 128
  // rows) the number of active key tiles of 64 keys and their ascending
  // indices, rows of ceil(N/64) entries.  Null for the dense forward.
  const int* tlist = nullptr;
  const int* tcount = nullptr;
  int mask_heads = 0;
  // Packed variable-length (16-bit types only): sequence s is tokens
  // [cu_seqlens[s], cu_seqlens[s+1]) of T; B is then the number of sequences
  // and N the longest sequence.  Null for a batched problem.
  const int* cu_seqlens = nullptr;
  int T = 0;
  // Strided tensors (dense and block-sparse modes); zero = dense layout.
  Layout lay{};
};

// Forward kernel variants: every tile, a block-sparse tile list, or packed
// variable-length sequences.
enum FwdMode { kFwdDense = 0, kFwdSparse = 1, kFwdVarlen = 2 };

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* stats;  // workspace: [B*Hq][2][N rounded up to 64] fp32 row statistics
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  Dtype dtype;
  hipStream_t stream;
  // Q and dQ; K, V, dK and dV; O and dO.  Zero = dense [B, H, N, d].
  Layout lay{};
  // Packed variable-length sequences (dK/dV and dQ stages): as in FwdArgs,
  // B sequences of at most N tokens out of T; the statistics then cover the
  // T packed tokens ([Hq][2][T rounded up to 64]).
  const int* cu_seqlens = nullptr;
  int T = 0;
  // dK/dV stage: a kv group's query heads split over this many workgroups
  // per key block, each writing fp32 partial sums to `part` (workspace after
  // the statistics) that a merge kernel adds in split order.  1 = no split.
  int nsplit = 1;
  float* part = nullptr;
};

// Split-K/V forward (16-bit types): queries [B,Hq,Nq,d], keys/values [B,Hkv,Nk,d],
// bottom-right aligned causal mask; workspace holds the per-split partials.
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* workspace;
  int B, Hq, Hkv, Nq, Nk, d;
  bool causal;
  float scale;
  int num_splits;  // requested; <= 0 picks one from the shape
  Dtype dtype;     // kBF16 or kF16
  hipStream_t stream;
  Layout lay{};    // element strides; all zero: dense [B, H, Nq|Nk, d]
};

struct SplitPlan {
  int nrb;        // 128-row blocks of one head group's packed query rows
  int nsplit;     // splits actually used (every split holds at least one key)
  int split_len;  // keys per split, a multiple of 64
};

SplitPlan split_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);
size_t split_workspace_bytes(int B, int Hq, int Nq, int d, int nsplit);
hipError_t launch_fwd_split(const SplitArgs& a);

hipError_t launch_fwd(const FwdArgs& a);
// Block-sparse forward: compacts the byte mask [mask_heads][ceil(N/128)]
// [ceil(N/64)] into tile lists in the workspace, then runs the forward.
constexpr int kSparseBlockQ = 128, kSparseBlockK = 64;
size_t sparse_workspace_bytes(int Hq, int N, int mask_heads);
hipError_t launch_fwd_sparse(const FwdArgs& a, const unsigned char* mask, void* workspace);
// Slice group xg of the XCD-aware work order (xcd_item) for nsl slices that
// each stream `bytes` of data through L2, shared by `share` adjacent slices:
// the largest divisor of nsl/8 whose data fit `budget`.  When one group
// would cover all of an XCD's slices, or not even one slice fits: the plain
// order (0), or for shared data its restriction to whole sharing groups per
// XCD (nsl/8).  0 when nsl % 8 != 0.
inline int xcd_group(int64_t nsl, int share, int64_t bytes, int64_t budget) {
  if (nsl <= 0 || (nsl & 7) || nsl > (1LL << 30) || bytes <= 0) return 0;
  const int64_t S8 = nsl >> 3;
  const int whole = share > 1 ? (int)S8 : 0;
  if (bytes > budget) return whole;
  // ceil(G / share) * bytes <= budget  <=>  G <= floor(budget / bytes) * share
  const int64_t gmax = (budget / bytes) * share;
  int64_t best = 1;
  for (int64_t f = 1; f * f <= S8; ++f) {  // divisors of S8 in pairs (f, S8 / f)
    if (S8 % f) continue;
    if (f <= gmax && f > best) best = f;
    if (S8 / f <= gmax && S8 / f > best) best = S8 / f;
  }
  return best == S8 ? whole : (int)best;
}
// L2 budgets of the slice groups: causal grids also need their heaviest
// blocks of many slices in flight at once, so they take larger groups.
constexpr int64_t kXgBudget = 2 << 20, kXgBudgetCausal = 8 << 20;
// The slice group of a causal grid.  A group of one unshared slice per XCD
// leaves too few of the heaviest query blocks in flight at a time: there the
// plain order is the faster one (by 2.5-3% on the forward and dQ stage of
// the causal B=1 H=16 N=8192 d=256 and B=4 H=32 N=4000 d=128 problems), and
// smaller budgets than this one, which would group the causal d=64 problems,
// made them 5-20% slower than the plain order.
inline int xcd_group_causal(int64_t nsl, int share, int64_t bytes) {
  const int g = xcd_group(nsl, share, bytes, kXgBudgetCausal);
  return g == 1 && share == 1 ? 0 : g;
}

// Bytes of the backward row-statistics workspace.
size_t bwd_stats_bytes(int B, int Hq, int N);
// Scratch of the entry point that allocates nothing: a static device array of
// this many bytes per device (attn_noalloc.hip), and its device address on the
// current device (looked up on first use, then cached).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);
// Measurement helper (attn_clock.hip): nwg one-wave workgroups, each storing
// the shader-clock cycles and 100 MHz real-time ticks elapsed over a spin of
// at most `ticks` ticks to out[2i], out[2i+1].
hipError_t launch_clock_probe(unsigned long long* out, int nwg, unsigned ticks, hipStream_t stream);
// Query-head splits of the dK/dV stage for a dense problem (1 when the grid
// of key blocks x kv heads already fills the device), and the bytes of fp32
// partial sums they need (0 for one split).
int bwd_dkdv_splits(int B, int Hq, int Hkv, int N, int d);
size_t bwd_partial_bytes(int B, int Hkv, int N, int d, int nsplit);
// Backward stages; each launches one kernel on a.stream.
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
// dQ that also computes and stores the row statistics (batched: padding rows
// included; packed sequences: the rows of each sequence),
// so the dK/dV stage can follow it with no preprocess launch.
hipError_t launch_bwd_dq_stats(const BwdArgs& a);

}  // namespace attn
