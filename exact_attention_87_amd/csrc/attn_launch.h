// Host-side launch interface between the C ABI (attn_api.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  bool bf16;
  hipStream_t stream;
};

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
  bool bf16;
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
// Bytes of the backward row-statistics workspace.
size_t bwd_stats_bytes(int B, int Hq, int N);
// Backward stages; each launches one kernel on a.stream.
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace attn
