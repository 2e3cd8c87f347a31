// C ABI of the exact-attention library (declared in include/attn.h):
// argument validation, the per-device architecture check and dispatch to the
// gfx950 kernels.  Nothing here allocates device memory or synchronises
// (unless ATTN_DEBUG is set, below).
#include <algorithm>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

// The ABI's enum arguments may carry any int a C caller passed; they are read
// as int before any comparison (loading an out-of-range value through the C++
// enum type would be undefined behaviour).
template <typename E>
int as_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_arch_state[kMaxDevices];

attn_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_HIP;
  if (dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? ATTN_OK : ATTN_ERR_UNSUPPORTED_DEVICE;
}

// ATTN_DEBUG set to anything but "" or "0" in the environment (read at each
// call): every entry point waits for the kernels it launched, so a kernel
// that fails reports ATTN_ERR_HIP from the call that launched it instead of
// from a later HIP call.  For debugging only: it serialises the caller's
// stream, and a stream under graph capture cannot be synchronised.
bool debug_sync() {
  const char* v = std::getenv("ATTN_DEBUG");
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

// Status of an entry point whose launches returned e on `stream`.
attn_status launched(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return ATTN_ERR_HIP;
  if (debug_sync() && hipStreamSynchronize(stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// A dispatch's grid size is a 32-bit count of work-items: `units` work units
// of `per_unit` threads each must stay below 2^32 (a larger grid would be
// truncated, leaving most of the problem uncomputed).
bool dispatch_fits(int64_t units, int64_t per_unit) {
  return units >= 0 && per_unit > 0 && units < ((int64_t)1 << 32) / per_unit;
}

// Shape checks common to both passes.  Returns ATTN_OK and sets *empty when
// the problem has no rows.
attn_status check_shape(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                        int dtype, bool* empty) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  // d = 256: 16-bit paths only (the callers below say which)
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  // Limits of the kernels' 32-bit grid, row and byte offsets: one (batch,
  // head) slice stays below 1 GiB.
  if ((int64_t)B * Hq > (1 << 24) || N > (1 << 22)) return ATTN_ERR_UNSUPPORTED;
  // Every launch over the query rows fits one dispatch: its work-items
  // (workgroups x threads) stay below 2^32.  The most per row are the
  // statistics kernel's d/8 lanes (at least 8: the fp32 forward), over rows
  // padded to the 128-row blocks of the matrix-core grids.
  if (!dispatch_fits((int64_t)B * Hq * round_up(N, 128), std::max(8, d / 8)))
    return ATTN_ERR_UNSUPPORTED;
  *empty = (B == 0 || N == 0);
  return ATTN_OK;
}

struct Buf {
  const void* p;
  size_t bytes;
};

// Every buffer non-null and 16-byte aligned; no output overlaps an input or
// another output.
attn_status check_buffers(std::initializer_list<Buf> ins, std::initializer_list<Buf> outs) {
  for (const Buf& b : ins)
    if (!b.p || !aligned16(b.p)) return ATTN_ERR_INVALID_ARG;
  for (const Buf& b : outs)
    if (!b.p || !aligned16(b.p)) return ATTN_ERR_INVALID_ARG;
  auto R = [](const Buf& b) { return Range{(uintptr_t)b.p, (uintptr_t)b.p + b.bytes}; };
  for (const Buf& o : outs) {
    for (const Buf& i : ins)
      if (overlaps(R(o), R(i))) return ATTN_ERR_INVALID_ARG;
    for (const Buf& o2 : outs)
      if (&o != &o2 && overlaps(R(o), R(o2))) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

struct Sizes {
  size_t q, kv, l, st;  // bytes of [B,Hq,N,d] and [B,Hkv,N,d] 16-bit, [B,Hq,N] fp32, statistics
};

Sizes sizes(int B, int Hq, int Hkv, int N, int d) {
  return Sizes{(size_t)B * Hq * N * d * 2, (size_t)B * Hkv * N * d * 2,
               (size_t)B * Hq * N * sizeof(float), attn::bwd_stats_bytes(B, Hq, N)};
}

// Checks shared by the backward entry points.  On success fills *a's shape
// fields; a->N == 0 marks an empty problem (nothing to launch).
attn_status bwd_common(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       int dtype, void* stream, attn::BwdArgs* a) {
  *a = attn::BwdArgs{};
  bool empty = false;
  attn_status st = check_shape(B, Hq, Hkv, N, d, causal, scale, dtype, &empty);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (empty) return ATTN_OK;  // a->N stays 0
  a->B = B, a->Hq = Hq, a->Hkv = Hkv, a->N = N, a->d = d;
  a->causal = causal == 1, a->scale = scale, a->dtype = (attn::Dtype)dtype;
  a->stream = (hipStream_t)stream;
  return ATTN_OK;
}

// attn_bwd_workspace_bytes on an int dtype.
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int dtype) {
  bool empty = false;
  if (check_shape(B, Hq, Hkv, N, d, 0, 1.0f, dtype, &empty) != ATTN_OK) return (size_t)-1;
  if (dtype == ATTN_F32) return (size_t)-1;
  if (empty) return 0;
  const size_t stats = (attn::bwd_stats_bytes(B, Hq, N) + 255) & ~(size_t)255;
  const size_t part = attn::bwd_partial_bytes(B, Hkv, N, d, attn::bwd_dkdv_splits(B, Hq, Hkv, N, d));
  return stats + ((part + 255) & ~(size_t)255);
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return 2; }

const char* attn_status_str(attn_status s) {
  switch (as_int(s)) {  // any int a C caller passed
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_UNSUPPORTED_DEVICE: return "ATTN_ERR_UNSUPPORTED_DEVICE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "unknown attn_status";
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int N, int d, int causal, float scale, attn_dtype dtype,
                     void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  bool empty = false;
  attn_status st = check_shape(B, Hq, Hkv, N, d, causal, scale, dt, &empty);
  if (st != ATTN_OK) return st;
  if (dt == ATTN_F32 && d == 256) return ATTN_ERR_UNSUPPORTED;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_INVALID_ARG;
  const size_t es = dt == ATTN_F32 ? 4 : 2;
  const size_t qbytes = (size_t)B * Hq * N * d * es;
  const size_t kvbytes = (size_t)B * Hkv * N * d * es;
  const size_t lbytes = (size_t)B * Hq * N * sizeof(float);
  const Range rq{(uintptr_t)q, (uintptr_t)q + qbytes}, rk{(uintptr_t)k, (uintptr_t)k + kvbytes},
      rv{(uintptr_t)v, (uintptr_t)v + kvbytes}, ro{(uintptr_t)o, (uintptr_t)o + qbytes},
      rl{(uintptr_t)lse, (uintptr_t)lse + lbytes};
  for (Range in : {rq, rk, rv})
    if (overlaps(ro, in) || overlaps(rl, in)) return ATTN_ERR_INVALID_ARG;
  if (overlaps(ro, rl)) return ATTN_ERR_INVALID_ARG;

  st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal == 1, scale, (attn::Dtype)dt,
                  (hipStream_t)stream};
  return launched(attn::launch_fwd(a), a.stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, attn_dtype dtype) {
  return bwd_workspace_bytes(B, Hq, Hkv, N, d, as_int(dtype));
}

namespace {
// The dK/dV stage's query-head split for a dense problem and its fp32
// partial sums, which live in the workspace after the statistics.
void set_split(attn::BwdArgs* a, void* workspace) {
  a->nsplit = attn::bwd_dkdv_splits(a->B, a->Hq, a->Hkv, a->N, a->d);
  const size_t stats = (attn::bwd_stats_bytes(a->B, a->Hq, a->N) + 255) & ~(size_t)255;
  a->part = a->nsplit > 1 ? (float*)((char*)workspace + stats) : nullptr;
}

// attn_bwd's launches on validated arguments: the dQ stage, which also writes
// the row statistics, then the dK/dV stage (and its merge when it splits).
// Every workspace byte either kernel reads is written earlier in the same
// call, so the workspace needs no initialisation.
attn_status bwd_launch(attn::BwdArgs* a, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout, void* dq, void* dk,
                       void* dv, void* workspace) {
  a->q = q, a->k = k, a->v = v, a->o = o, a->lse = lse, a->dout = dout;
  a->dq = dq, a->dk = dk, a->dv = dv, a->stats = (float*)workspace;
  set_split(a, workspace);
  if (attn::launch_bwd_dq_stats(*a) != hipSuccess) return ATTN_ERR_HIP;
  return launched(attn::launch_bwd_dkdv(*a), a->stream);
}
}  // namespace

static_assert(ATTN_NOALLOC_SCRATCH_BYTES == attn::kNoallocScratchBytes,
              "header scratch size is the library's");

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
                     float scale, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  const size_t wbytes = bwd_workspace_bytes(B, Hq, Hkv, N, d, dt);
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {o, z.q}, {lse, z.l}, {dout, z.q}},
                     {{dq, z.q}, {dk, z.kv}, {dv, z.kv}, {workspace, wbytes}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  return bwd_launch(&a, q, k, v, o, lse, dout, dq, dk, dv, workspace);
}

attn_status attn_probe_clock(unsigned long long* out, int nwg, unsigned ticks, void* stream) {
  if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 7u) != 0) return ATTN_ERR_INVALID_ARG;
  if (nwg < 1 || nwg > 64 || ticks < 1 || ticks > 200000000u) return ATTN_ERR_INVALID_ARG;
  const attn_status st = check_device();
  if (st != ATTN_OK) return st;
  return launched(attn::launch_clock_probe(out, nwg, ticks, (hipStream_t)stream), (hipStream_t)stream);
}

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                             attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const size_t wbytes = bwd_workspace_bytes(B, Hq, Hkv, N, d, dt);
  if (wbytes > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_UNSUPPORTED;
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {o, z.q}, {lse, z.l}, {dout, z.q}},
                     {{dq, z.q}, {dk, z.kv}, {dv, z.kv}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  void* scratch = nullptr;
  if (attn::noalloc_scratch(&scratch) != hipSuccess) return ATTN_ERR_HIP;
  // The static scratch is a different allocation from every caller buffer.
  return bwd_launch(&a, q, k, v, o, lse, dout, dq, dk, dv, scratch);
}

attn_status attn_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, float* stats, void* dq, int B,
                              int Hq, int Hkv, int N, int d, int causal, float scale,
                              attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {o, z.q}, {lse, z.l}, {dout, z.q}},
                     {{stats, z.st}, {dq, z.q}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse, a.dout = dout;
  a.stats = stats, a.dq = dq;
  return launched(attn::launch_bwd_dq_stats(a), a.stream);
}

attn_status attn_bwd_preprocess(const void* o, const void* dout, const float* lse, float* stats,
                                int B, int Hq, int N, int d, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  attn_status st = bwd_common(B, Hq, Hq, N, d, 0, 1.0f, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const Sizes z = sizes(B, Hq, Hq, N, d);
  st = check_buffers({{o, z.q}, {dout, z.q}, {lse, z.l}}, {{stats, z.st}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.o = o, a.dout = dout, a.lse = lse, a.stats = stats;
  return launched(attn::launch_bwd_pre(a), a.stream);
}

attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                          float* stats, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                          int causal, float scale, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  const size_t wbytes = bwd_workspace_bytes(B, Hq, Hkv, N, d, dt);
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  set_split(&a, stats);
  if (a.nsplit > 1)  // the partial sums are written after the statistics
    st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {dout, z.q}},
                       {{stats, wbytes}, {dk, z.kv}, {dv, z.kv}});
  else
    st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {dout, z.q}, {stats, z.st}},
                       {{dk, z.kv}, {dv, z.kv}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.q = q, a.k = k, a.v = v, a.dout = dout, a.stats = stats;
  a.dk = dk, a.dv = dv;
  return launched(attn::launch_bwd_dkdv(a), a.stream);
}

attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                        const float* stats, void* dq, int B, int Hq, int Hkv, int N, int d,
                        int causal, float scale, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {dout, z.q}, {stats, z.st}}, {{dq, z.q}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.q = q, a.k = k, a.v = v, a.dout = dout, a.stats = (float*)stats, a.dq = dq;
  return launched(attn::launch_bwd_dq(a), a.stream);
}

}  // extern "C"

// ------------------------------------------------------------ split K/V
namespace {

// Shape checks of the split-K/V forward.  Sets *empty when there are no
// query rows (Nk == 0 with query rows is a real problem: every row sees no
// key).
attn_status split_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                        int num_splits, int dtype, bool* empty) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 0) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  // 32-bit offsets: one key/value slice and one head group's query rows
  // stay below 1 GiB; the grid stays below 2^31 workgroups.
  if ((int64_t)B * Hq > (1 << 24) || Nq > (1 << 22) || Nk > (1 << 22)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)(Hq / Hkv) * Nq > (1 << 22)) return ATTN_ERR_UNSUPPORTED;
  *empty = (B == 0 || Nq == 0);
  if (*empty) return ATTN_OK;
  const attn::SplitPlan p = attn::split_plan(B, Hq, Hkv, Nq, Nk, d, num_splits);
  // one dispatch each: 256-thread workgroups per (range, slice, row block),
  // and the merge's (at most) 64 threads per output row
  if (!dispatch_fits((int64_t)p.nrb * p.nsplit * B * Hkv, 256) ||
      !dispatch_fits((int64_t)B * Hq * Nq, 64))
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  bool empty = false;
  if (split_shape(B, Hq, Hkv, Nq, Nk, d, 0, 1.0f, num_splits, ATTN_BF16, &empty) != ATTN_OK)
    return -1;
  if (empty) return 0;
  return attn::split_plan(B, Hq, Hkv, Nq, Nk, d, num_splits).nsplit;
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                        int num_splits) {
  const int ns = attn_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (ns < 0) return (size_t)-1;
  if (ns == 0) return 0;
  return attn::split_workspace_bytes(B, Hq, Nq, d, ns);
}

attn_status attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                             void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                             int causal, float scale, int num_splits, attn_dtype dtype,
                             void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  bool empty = false;
  attn_status st = split_shape(B, Hq, Hkv, Nq, Nk, d, causal, scale, num_splits, dt, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  const size_t qb = (size_t)B * Hq * Nq * d * 2, kvb = (size_t)B * Hkv * Nk * d * 2;
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  const size_t wb = attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits);
  st = check_buffers({{q, qb}, {k, kvb}, {v, kvb}}, {{o, qb}, {lse, lb}, {workspace, wb}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  attn::SplitArgs a{q,  k,  v, o,           lse,   workspace,  B,
                    Hq, Hkv, Nq, Nk, d, causal == 1, scale, num_splits, (attn::Dtype)dt,
                    (hipStream_t)stream};
  return launched(attn::launch_fwd_split(a), a.stream);
}

}  // extern "C"

// ------------------------------------------------------------ stride checks
namespace {

// One tensor family's strides from the caller's array (batch, head, row).
attn::Strides3 strides_at(const long long* s, int i) {
  return attn::Strides3{(int64_t)s[3 * i], (int64_t)s[3 * i + 1], (int)s[3 * i + 2]};
}

// Strides the kernels can address: non-negative, 16-byte multiples, rows at
// least d apart, and every row index up to N + 127 (the padded tail of a tile)
// at a 32-bit byte offset.
bool strides_ok(const long long* s, int i, int N, int d) {
  const long long b = s[3 * i], h = s[3 * i + 1], r = s[3 * i + 2];
  if (b < 0 || h < 0 || r < d || (b % 8) || (h % 8) || (r % 8)) return false;
  return ((long long)(N + 127) * r + d) * 2 < (1ll << 31);
}

// Bytes from a tensor's base to the end of its last element.
size_t extent(const long long* s, int i, int B, int H, int N, int d) {
  return (size_t)(((long long)(B - 1) * s[3 * i] + (long long)(H - 1) * s[3 * i + 1] +
                   (long long)(N - 1) * s[3 * i + 2] + d) * 2);
}

}  // namespace

namespace {

// The block-sparse forward on dense tensors (strides == nullptr) or with
// the caller's 9 strides.
attn_status fwd_blocksparse_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const unsigned char* block_mask, int mask_heads, void* workspace,
                                 const long long* strides, int B, int Hq, int Hkv, int N, int d,
                                 int causal, float scale, int dtype, void* stream) {
  bool empty = false;
  attn_status st = check_shape(B, Hq, Hkv, N, d, causal, scale, dtype, &empty);
  if (st != ATTN_OK) return st;
  if (!(mask_heads == 1 || mask_heads == Hq)) return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  // the tile list lives in LDS beside the stages (128 KiB of them at d = 256)
  if (N > (d == 256 ? (1 << 20) : (1 << 21))) return ATTN_ERR_UNSUPPORTED;
  if (empty) return ATTN_OK;
  const size_t nqb = ((size_t)N + ATTN_SPARSE_BLOCK_Q - 1) / ATTN_SPARSE_BLOCK_Q;
  const size_t nkt = ((size_t)N + ATTN_SPARSE_BLOCK_K - 1) / ATTN_SPARSE_BLOCK_K;
  const Sizes z = sizes(B, Hq, Hkv, N, d);
  size_t eq = z.q, ek = z.kv, eo = z.q;
  if (strides) {
    for (int i = 0; i < 3; ++i)
      if (!strides_ok(strides, i, N, d)) return ATTN_ERR_INVALID_ARG;
    eq = extent(strides, 0, B, Hq, N, d);
    ek = extent(strides, 1, B, Hkv, N, d);
    eo = extent(strides, 2, B, Hq, N, d);
  }
  const size_t mb = (size_t)mask_heads * nqb * nkt;
  const size_t wb = attn_fwd_blocksparse_workspace_bytes(Hq, N, mask_heads);
  st = check_buffers({{q, eq}, {k, ek}, {v, ek}}, {{o, eo}, {lse, z.l}, {workspace, wb}});
  if (st != ATTN_OK) return st;
  // the mask is an input too (any alignment: it is read byte by byte)
  if (!block_mask) return ATTN_ERR_INVALID_ARG;
  const Range rm{(uintptr_t)block_mask, (uintptr_t)block_mask + mb};
  const Range outs[] = {{(uintptr_t)o, (uintptr_t)o + eo},
                        {(uintptr_t)lse, (uintptr_t)lse + z.l},
                        {(uintptr_t)workspace, (uintptr_t)workspace + wb}};
  for (const Range& r : outs)
    if (overlaps(rm, r)) return ATTN_ERR_INVALID_ARG;
  st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal == 1, scale, (attn::Dtype)dtype,
                  (hipStream_t)stream};
  a.mask_heads = mask_heads;
  if (strides)
    a.lay = attn::Layout{strides_at(strides, 0), strides_at(strides, 1), strides_at(strides, 2)};
  return launched(attn::launch_fwd_sparse(a, block_mask, workspace), a.stream);
}

}  // namespace

// ------------------------------------------------------------ block-sparse
static_assert(ATTN_SPARSE_BLOCK_Q == attn::kSparseBlockQ && ATTN_SPARSE_BLOCK_K == attn::kSparseBlockK,
              "header block sizes are the kernels' tiles");

extern "C" {

size_t attn_fwd_blocksparse_workspace_bytes(int Hq, int N, int mask_heads) {
  if (Hq < 1 || N < 0 || N > (1 << 21) || !(mask_heads == 1 || mask_heads == Hq))
    return (size_t)-1;
  if (N == 0) return 0;
  return attn::sparse_workspace_bytes(Hq, N, mask_heads);
}

attn_status attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const unsigned char* block_mask, int mask_heads, void* workspace,
                                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                 attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  return fwd_blocksparse_impl(q, k, v, o, lse, block_mask, mask_heads, workspace, nullptr, B, Hq,
                              Hkv, N, d, causal, scale, dt, stream);
}

attn_status attn_fwd_blocksparse_strided(const void* q, const void* k, const void* v, void* o,
                                         float* lse, const unsigned char* block_mask,
                                         int mask_heads, void* workspace,
                                         const long long* strides, int B, int Hq, int Hkv, int N,
                                         int d, int causal, float scale, attn_dtype dtype,
                                         void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  if (!strides) return ATTN_ERR_INVALID_ARG;
  return fwd_blocksparse_impl(q, k, v, o, lse, block_mask, mask_heads, workspace, strides, B, Hq,
                              Hkv, N, d, causal, scale, dt, stream);
}

}  // extern "C"

// ------------------------------------------------------------ packed variable length

namespace {

// Strides of packed-sequence tensors: (head, token) pairs for q, for k and v,
// and for o, in elements; the checks of strides_ok on one [1, H, T, d] slice.
bool varlen_strides_ok(const long long* s, int T, int d) {
  for (int i = 0; i < 3; ++i) {
    const long long full[3] = {0, s[2 * i], s[2 * i + 1]};
    if (!strides_ok(full, 0, T, d)) return false;
  }
  return true;
}
size_t varlen_extent(const long long* s, int i, int H, int T, int d) {
  return (size_t)(((long long)(H - 1) * s[2 * i] + (long long)(T - 1) * s[2 * i + 1] + d) * 2);
}
attn::Layout varlen_layout(const long long* s) {
  auto st = [&](int i) { return attn::Strides3{0, (int64_t)s[2 * i], (int)s[2 * i + 1]}; };
  return attn::Layout{st(0), st(1), st(2)};
}

// The packed variable-length forward, dense [H, T, d] (strides == nullptr)
// or with the caller's (head, token) strides.
attn_status fwd_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens, const long long* strides, int nseq,
                            int max_seqlen, int Hq, int Hkv, int T, int d, int causal, float scale,
                            int dtype, void* stream) {
  if (nseq < 0 || max_seqlen < 0 || T < 0 || max_seqlen > T) return ATTN_ERR_INVALID_ARG;
  bool empty = false;
  attn_status st = check_shape(1, Hq, Hkv, T, d, causal, scale, dtype, &empty);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)nseq * Hq > (1 << 24)) return ATTN_ERR_UNSUPPORTED;
  // the grid is (sequence, head, 128-row block of the longest sequence)
  if (!dispatch_fits((int64_t)nseq * Hq * round_up(max_seqlen, 128), 2)) return ATTN_ERR_UNSUPPORTED;
  if (nseq == 0 || T == 0 || max_seqlen == 0) return ATTN_OK;  // no rows to compute
  const Sizes z = sizes(1, Hq, Hkv, T, d);
  size_t eq = z.q, ek = z.kv, eo = z.q;
  if (strides) {
    if (!varlen_strides_ok(strides, T, d)) return ATTN_ERR_INVALID_ARG;
    eq = varlen_extent(strides, 0, Hq, T, d);
    ek = varlen_extent(strides, 1, Hkv, T, d);
    eo = varlen_extent(strides, 2, Hq, T, d);
  }
  st = check_buffers({{q, eq}, {k, ek}, {v, ek}}, {{o, eo}, {lse, z.l}});
  if (st != ATTN_OK) return st;
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u)) return ATTN_ERR_INVALID_ARG;
  const Range rc{(uintptr_t)cu_seqlens, (uintptr_t)cu_seqlens + ((size_t)nseq + 1) * 4};
  if (overlaps(rc, Range{(uintptr_t)o, (uintptr_t)o + eo}) ||
      overlaps(rc, Range{(uintptr_t)lse, (uintptr_t)lse + z.l}))
    return ATTN_ERR_INVALID_ARG;
  st = check_device();
  if (st != ATTN_OK) return st;
  // B = sequences and N = the longest sequence size the grid
  attn::FwdArgs a{q, k, v, o, lse, nseq, Hq, Hkv, max_seqlen, d, causal == 1, scale,
                  (attn::Dtype)dtype, (hipStream_t)stream};
  a.cu_seqlens = cu_seqlens;
  a.T = T;
  if (strides) a.lay = varlen_layout(strides);
  return launched(attn::launch_fwd(a), a.stream);
}


// The packed variable-length backward, dense [H, T, d] (strides == nullptr)
// or with the caller's (head, token) strides.  Strided gradients may be
// interleaved slices of one packed buffer, so they are checked only against
// the inputs, the workspace and the offsets.
attn_status bwd_varlen_impl(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* workspace, const int* cu_seqlens, const long long* strides,
                            int nseq, int max_seqlen, int Hq, int Hkv, int T, int d, int causal,
                            float scale, int dtype, void* stream) {
  if (nseq < 0 || max_seqlen < 0 || T < 0 || max_seqlen > T) return ATTN_ERR_INVALID_ARG;
  attn::BwdArgs a;
  // the packed tokens as one [1, H, T, d] problem: shapes, statistics, workspace
  attn_status st = bwd_common(1, Hq, Hkv, T, d, causal, scale, dtype, stream, &a);
  if (st != ATTN_OK) return st;
  if ((int64_t)nseq * Hq > (1 << 24)) return ATTN_ERR_UNSUPPORTED;
  // the dK/dV and dQ grids are (sequence, head, 128-row block of the longest
  // sequence), at most two threads per padded row
  if (!dispatch_fits((int64_t)nseq * Hq * round_up(max_seqlen, 128), 2)) return ATTN_ERR_UNSUPPORTED;
  if (a.N == 0 || nseq == 0 || max_seqlen == 0) return ATTN_OK;  // no rows
  const size_t wbytes = bwd_workspace_bytes(1, Hq, Hkv, T, d, dtype);
  const Sizes z = sizes(1, Hq, Hkv, T, d);
  size_t eq = z.q, ek = z.kv, eo = z.q;
  if (strides) {
    if (!varlen_strides_ok(strides, T, d)) return ATTN_ERR_INVALID_ARG;
    eq = varlen_extent(strides, 0, Hq, T, d);
    ek = varlen_extent(strides, 1, Hkv, T, d);
    eo = varlen_extent(strides, 2, Hq, T, d);
  }
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u)) return ATTN_ERR_INVALID_ARG;
  const Range rc{(uintptr_t)cu_seqlens, (uintptr_t)cu_seqlens + ((size_t)nseq + 1) * 4};
  if (!strides) {
    st = check_buffers({{q, z.q}, {k, z.kv}, {v, z.kv}, {o, z.q}, {lse, z.l}, {dout, z.q}},
                       {{dq, z.q}, {dk, z.kv}, {dv, z.kv}, {workspace, wbytes}});
    if (st != ATTN_OK) return st;
  } else {
    const Buf ins[] = {{q, eq}, {k, ek}, {v, ek}, {o, eo}, {lse, z.l}, {dout, eo}};
    for (const Buf& b : ins)
      if (!b.p || !aligned16(b.p)) return ATTN_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
    const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + wbytes};
    const Buf grads[] = {{dq, eq}, {dk, ek}, {dv, ek}};
    for (const Buf& g : grads) {
      if (!g.p || !aligned16(g.p)) return ATTN_ERR_INVALID_ARG;
      const Range rg{(uintptr_t)g.p, (uintptr_t)g.p + g.bytes};
      if (overlaps(rg, rw)) return ATTN_ERR_INVALID_ARG;
      for (const Buf& b : ins)
        if (overlaps(rg, Range{(uintptr_t)b.p, (uintptr_t)b.p + b.bytes})) return ATTN_ERR_INVALID_ARG;
    }
    for (const Buf& b : ins)
      if (overlaps(rw, Range{(uintptr_t)b.p, (uintptr_t)b.p + b.bytes})) return ATTN_ERR_INVALID_ARG;
  }
  const Range outs[] = {{(uintptr_t)dq, (uintptr_t)dq + eq},
                        {(uintptr_t)dk, (uintptr_t)dk + ek},
                        {(uintptr_t)dv, (uintptr_t)dv + ek},
                        {(uintptr_t)workspace, (uintptr_t)workspace + wbytes}};
  for (const Range& r : outs)
    if (overlaps(rc, r)) return ATTN_ERR_INVALID_ARG;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse, a.dout = dout;
  a.dq = dq, a.dk = dk, a.dv = dv, a.stats = (float*)workspace;
  if (strides) a.lay = varlen_layout(strides);
  // the two gradient stages per (sequence, head) with B = sequences and N =
  // the longest sequence: dQ, which also stores the row statistics of every
  // sequence's tokens, then dK/dV
  a.B = nseq, a.N = max_seqlen, a.cu_seqlens = cu_seqlens, a.T = T;
  // Query-head split of the dK/dV stage, chosen on the grid it launches
  // (sequences x longest sequence) like a batched problem, and capped by the
  // split the workspace was sized for ([1, H, T, d]): the partial sums are
  // kept per (kv head, token), which that size covers for any count up to it.
  {
    const int s = std::min(attn::bwd_dkdv_splits(nseq, Hq, Hkv, max_seqlen, d),
                           attn::bwd_dkdv_splits(1, Hq, Hkv, T, d));
    const size_t stats = (attn::bwd_stats_bytes(1, Hq, T) + 255) & ~(size_t)255;
    a.nsplit = s;
    a.part = s > 1 ? (float*)((char*)workspace + stats) : nullptr;
  }
  if (attn::launch_bwd_dq_stats(a) != hipSuccess) return ATTN_ERR_HIP;
  return launched(attn::launch_bwd_dkdv(a), a.stream);
}

}  // namespace

extern "C" {

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens, int nseq, int max_seqlen, int Hq, int Hkv,
                            int T, int d, int causal, float scale, attn_dtype dtype,
                            void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens, nullptr, nseq, max_seqlen, Hq, Hkv, T, d,
                         causal, scale, dt, stream);
}

attn_status attn_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int* cu_seqlens, const long long* strides,
                                    int nseq, int max_seqlen, int Hq, int Hkv, int T, int d,
                                    int causal, float scale, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  if (!strides) return ATTN_ERR_INVALID_ARG;
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens, strides, nseq, max_seqlen, Hq, Hkv, T, d,
                         causal, scale, dt, stream);
}

}  // extern "C"


// ------------------------------------------------------------ strided tensors
extern "C" {

attn_status attn_fwd_splitkv_strided(const void* q, const void* k, const void* v, void* o,
                                     float* lse, void* workspace, const long long* strides, int B,
                                     int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                     float scale, int num_splits, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  bool empty = false;
  attn_status st = split_shape(B, Hq, Hkv, Nq, Nk, d, causal, scale, num_splits, dt, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!strides) return ATTN_ERR_INVALID_ARG;
  if (!strides_ok(strides, 0, Nq, d) || !strides_ok(strides, 1, Nk, d) ||
      !strides_ok(strides, 2, Nq, d))
    return ATTN_ERR_INVALID_ARG;
  // a head group's query rows are addressed from the group's first head
  const long long group_rows = ((long long)(Hq / Hkv - 1) * strides[1] +
                                (long long)(Nq - 1) * strides[2] + d) * 2;
  if (group_rows >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const size_t eq = extent(strides, 0, B, Hq, Nq, d), ek = extent(strides, 1, B, Hkv, Nk, d),
               eo = extent(strides, 2, B, Hq, Nq, d);
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  const size_t wb = attn_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits);
  const size_t ekv = Nk == 0 ? 0 : ek;  // no keys: K and V are never read
  st = check_buffers({{q, eq}, {k, ekv}, {v, ekv}}, {{o, eo}, {lse, lb}, {workspace, wb}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  attn::SplitArgs a{q,  k,  v, o,           lse,   workspace,  B,
                    Hq, Hkv, Nq, Nk, d, causal == 1, scale, num_splits, (attn::Dtype)dt,
                    (hipStream_t)stream};
  a.lay = attn::Layout{strides_at(strides, 0), strides_at(strides, 1), strides_at(strides, 2)};
  return launched(attn::launch_fwd_split(a), a.stream);
}

attn_status attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                             const long long* strides, int B, int Hq, int Hkv, int N, int d,
                             int causal, float scale, attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  bool empty = false;
  attn_status st = check_shape(B, Hq, Hkv, N, d, causal, scale, dt, &empty);
  if (st != ATTN_OK) return st;
  if (dt == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (empty) return ATTN_OK;
  if (!strides) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (!strides_ok(strides, i, N, d)) return ATTN_ERR_INVALID_ARG;
  const size_t eq = extent(strides, 0, B, Hq, N, d), ek = extent(strides, 1, B, Hkv, N, d),
               eo = extent(strides, 2, B, Hq, N, d), el = (size_t)B * Hq * N * sizeof(float);
  st = check_buffers({{q, eq}, {k, ek}, {v, ek}}, {{o, eo}, {lse, el}});
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal == 1, scale, (attn::Dtype)dt,
                  (hipStream_t)stream};
  a.lay = attn::Layout{strides_at(strides, 0), strides_at(strides, 1), strides_at(strides, 2)};
  return launched(attn::launch_fwd(a), a.stream);
}

attn_status attn_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, const long long* strides, int B, int Hq, int Hkv,
                             int N, int d, int causal, float scale, attn_dtype dtype,
                             void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  attn::BwdArgs a;
  const size_t wbytes = bwd_workspace_bytes(B, Hq, Hkv, N, d, dt);
  attn_status st = bwd_common(B, Hq, Hkv, N, d, causal, scale, dt, stream, &a);
  if (st != ATTN_OK) return st;
  if (a.N == 0) return ATTN_OK;  // empty problem
  if (!strides) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (!strides_ok(strides, i, N, d)) return ATTN_ERR_INVALID_ARG;
  const size_t eq = extent(strides, 0, B, Hq, N, d), ek = extent(strides, 1, B, Hkv, N, d),
               eo = extent(strides, 2, B, Hq, N, d), el = (size_t)B * Hq * N * sizeof(float);
  // The gradients may be interleaved slices of one buffer (a packed dQKV), so
  // their extents may overlap each other; each must still stay clear of every
  // input and of the workspace.
  const Buf ins[] = {{q, eq}, {k, ek}, {v, ek}, {o, eo}, {lse, el}, {dout, eo}};
  const Buf grads[] = {{dq, eq}, {dk, ek}, {dv, ek}};
  for (const Buf& b : ins)
    if (!b.p || !aligned16(b.p)) return ATTN_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + wbytes};
  for (const Buf& g : grads) {
    if (!g.p || !aligned16(g.p)) return ATTN_ERR_INVALID_ARG;
    const Range rg{(uintptr_t)g.p, (uintptr_t)g.p + g.bytes};
    if (overlaps(rg, rw)) return ATTN_ERR_INVALID_ARG;
    for (const Buf& b : ins)
      if (overlaps(rg, Range{(uintptr_t)b.p, (uintptr_t)b.p + b.bytes})) return ATTN_ERR_INVALID_ARG;
  }
  for (const Buf& b : ins)
    if (overlaps(rw, Range{(uintptr_t)b.p, (uintptr_t)b.p + b.bytes})) return ATTN_ERR_INVALID_ARG;
  st = check_device();
  if (st != ATTN_OK) return st;
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse, a.dout = dout;
  a.dq = dq, a.dk = dk, a.dv = dv, a.stats = (float*)workspace;
  a.lay = attn::Layout{strides_at(strides, 0), strides_at(strides, 1), strides_at(strides, 2)};
  set_split(&a, workspace);
  // dQ first: it also writes the row statistics the dK/dV stage reads
  if (attn::launch_bwd_dq_stats(a) != hipSuccess) return ATTN_ERR_HIP;
  return launched(attn::launch_bwd_dkdv(a), a.stream);
}

attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* workspace, const int* cu_seqlens, int nseq, int max_seqlen,
                            int Hq, int Hkv, int T, int d, int causal, float scale,
                            attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, nullptr, nseq,
                         max_seqlen, Hq, Hkv, T, d, causal, scale, dt, stream);
}

attn_status attn_bwd_varlen_strided(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, void* workspace, const int* cu_seqlens,
                                    const long long* strides, int nseq, int max_seqlen, int Hq,
                                    int Hkv, int T, int d, int causal, float scale,
                                    attn_dtype dtype, void* stream) {
  const int dt = as_int(dtype);  // any int a C caller passed
  if (!strides) return ATTN_ERR_INVALID_ARG;
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, strides, nseq,
                         max_seqlen, Hq, Hkv, T, d, causal, scale, dt, stream);
}

}  // extern "C"
