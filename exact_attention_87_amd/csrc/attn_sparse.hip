// Block-sparse forward: only the (query block, key block) score tiles that a
// 0/1 block mask marks are computed ("FlashAttention" paper story,
// block-sparse paragraph: the zero blocks of the mask are skipped, which
// generalises the causal tile skip).  The mask is given per tile of the
// forward kernels (128 query rows x 64 keys).  A small kernel first compacts
// each mask row into the ascending list of its set tiles, cut at the causal
// diagonal; the forward kernels then walk that list instead of every tile.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// One wave per mask row (mask head, query block): ballot over 64 tiles at a
// time, prefix counts place each set tile.
__global__ __launch_bounds__(64) void sparse_compact_kernel(const unsigned char* __restrict__ mask,
                                                            int* __restrict__ tcount,
                                                            int* __restrict__ tlist, int nqb,
                                                            int nkt, int causal) {
  const int64_t row = blockIdx.x;
  const int qb = (int)(row % nqb);
  const unsigned char* m = mask + row * nkt;
  int* out = tlist + row * nkt;
  const int lane = threadIdx.x;
  // last key tile any query of this block can see
  const int last = causal ? min(nkt - 1, (qb * kSparseBlockQ + kSparseBlockQ - 1) / kSparseBlockK)
                          : nkt - 1;
  int count = 0;
  for (int base = 0; base <= last; base += 64) {
    const int t = base + lane;
    const bool on = t <= last && m[t] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    const int pre = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (on) out[count + pre] = t;
    count += __builtin_popcountll(bal);
  }
  if (lane == 0) tcount[row] = count;
}

static size_t count_bytes(int rows) { return ((size_t)rows * 4 + 255) & ~(size_t)255; }

size_t sparse_workspace_bytes(int Hq, int N, int mask_heads) {
  (void)Hq;
  const int nqb = (N + kSparseBlockQ - 1) / kSparseBlockQ;
  const int nkt = (N + kSparseBlockK - 1) / kSparseBlockK;
  const int rows = mask_heads * nqb;
  return count_bytes(rows) + (((size_t)rows * nkt * 4 + 255) & ~(size_t)255);
}

hipError_t launch_fwd_sparse(const FwdArgs& a0, const unsigned char* mask, void* workspace) {
  const int nqb = (a0.N + kSparseBlockQ - 1) / kSparseBlockQ;
  const int nkt = (a0.N + kSparseBlockK - 1) / kSparseBlockK;
  const int rows = a0.mask_heads * nqb;
  int* tcount = (int*)workspace;
  int* tlist = (int*)((char*)workspace + count_bytes(rows));
  hipLaunchKernelGGL(sparse_compact_kernel, dim3((unsigned)rows), dim3(64), 0, a0.stream, mask,
                     tcount, tlist, nqb, nkt, a0.causal ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FwdArgs a = a0;
  a.tlist = tlist;
  a.tcount = tcount;
  return launch_fwd(a);
}

}  // namespace attn
