// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 matrix-core and LDS-transpose builtins, the LDS
// tile swizzle and small lane helpers.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax: the running maximum only moves when a tile's maximum
// exceeds it by more than tau (base-2 units), so probabilities stay below
// 2^tau; a lane whose tile sum passes 2^tau takes the max path.  Any tau
// keeps the result: O and LSE use the same maximum, and P keeps the 16-bit
// type's relative precision at any magnitude.  A large tau makes the max
// path rare for extreme logits.  The bound is the P type's range: fp16 P
// must stay below 65504 (tau = 15); bf16 has fp32's exponent range.  The
// price is headroom: the fp32 output accumulators hold up to 2^tau x N x
// max|v|, so with bf16 inputs they overflow once N x max|v| reaches 2^98
// (about 3e29) rather than fp32's 3.4e38; fp16 inputs (|v| <= 65504) cannot
// reach it for N <= 2^22.
// (Measured on the extreme-logit grouped-query forward: tau 8 -> 16 took it
// from 1010 to 1056 TFLOP/s, and 15 -> 30 for bf16 from 1080 to 1120; the
// other workloads did not change.)
template <typename T>
struct Tau;
template <>
struct Tau<__bf16> {
  static constexpr int v = 30;
};
template <>
struct Tau<_Float16> {
  static constexpr int v = 15;  // fp16 P < 2^15 < 65504
};
static_assert(Tau<__bf16>::v >= 1 && Tau<__bf16>::v <= 30, "rescale threshold");
template <typename T>
constexpr float kTau = (float)Tau<T>::v;
template <typename T>
constexpr float kSumMax = (float)(1u << Tau<T>::v);

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "bitcast size");
  return __builtin_bit_cast(To, x);
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Lane l holds A[l%32][8*(l/32) + 0..7], B[8*(l/32) + 0..7][l%32] and
// D[8*(r/4) + 4*(l/32) + r%4][l%32] in element r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with fp16 operands (same operand and result layout).
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16-bit element types of the matrix-core kernels: T is __bf16 or _Float16.
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  using v8 = bf16x8;
};
template <>
struct Elem<_Float16> {
  using v8 = f16x8;
};

// Accumulator row held in element r of lane l of a 32x32 MFMA result.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane i element r is the (i%4)-th 16-bit value of the 8 bytes
// addressed by lane 4*r + i/4 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return bitcast<u32x2>(v);
}

__device__ __forceinline__ u32x4 lds_read16(const char* p) { return *(const lds_u32x4*)(p); }
__device__ __forceinline__ void lds_write16(char* p, u32x4 v) { *(lds_u32x4*)(p) = v; }

// Value of x held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t other = (threadIdx.x & 32) ? r[0] : r[1];
  return __uint_as_float(other);
}

// Two fp32 -> packed bf16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return bitcast<uint32_t>(v);
}

// Two fp32 -> packed fp16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return bitcast<uint32_t>(v);
}

// Two fp32 -> two packed 16-bit values of type T.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (__is_same(T, _Float16))
    return pack_f16(lo, hi);
  else
    return pack_bf16(lo, hi);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tile swizzle.  A tile row (one key or query) of D bf16 is D/8 chunks of
// 16 bytes; logical chunk ch of row `row` is stored at chunk ch ^ swz(row).
// The map makes both access patterns of the kernels conflict-free on the 64
// banks: 16 consecutive rows reading one logical chunk (matrix-core operand
// loads), and 4 consecutive rows x 4 aligned chunks (transposing reads).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128 || D == 256) {
    // rows of 256 or 512 bytes start on the same bank, so a 16-byte chunk's
    // bank group is its index mod 16 and the same XOR serves both
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    static_assert(D == 64, "head dim");
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int ch) {
  return row * (D * 2) + ((ch ^ swz<D>(row)) << 4);
}

// Byte offset, inside a swizzled [rows][D] tile, of the 8 bytes this lane
// feeds to a transposing read that yields the 32x16 operand
//   A[m][k] = T[kbase + key(k)][dbase + m],   m = lane%32,
// with k ordered like the accumulator rows of a 32x32 MFMA result:
// element j of lane l is row kbase + 8*(j/4) + 4*(l/32) + j%4.  Call with
// t = 0 for elements 0..3 and t = 1 for elements 4..7.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int kbase, int dbase, int t) {
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int row = kbase + 8 * t + 4 * (G >> 1) + r;
  const int d = dbase + 16 * (G & 1) + 4 * q;
  return tile_off<D>(row, d >> 3) + ((d & 7) << 1);
}

// XCD-aware work order over a grid of nmaj x nsl workgroups (nmaj major
// blocks, e.g. query blocks, of nsl slices).  Workgroup ids are dealt round
// robin to the 8 XCDs, each with its own L2.  With xg > 0, XCD x (ids = x
// mod 8) takes the contiguous slices x*nsl/8 .. (x+1)*nsl/8 - 1 in groups of
// xg slices, each group major-block-major: the workgroups reading one slice's
// tiles run together on one L2, and adjacent slices that share their data
// (the query heads of a kv group) do too.  xg = 0: the plain order, major
// index id / nsl.  A bijection when nsl % 8 == 0 and xg divides nsl / 8.
__device__ __forceinline__ void xcd_item(int nmaj, int nsl, int xg, int& maj, int& sl) {
  const int id = blockIdx.x;
  if (xg > 0) {
    const int x = id & 7, l = id >> 3;
    const int per = xg * nmaj;
    const int p = l / per, r = l - p * per;
    maj = r / xg;
    sl = x * (nsl >> 3) + p * xg + (r - maj * xg);
  } else {
    maj = id / nsl;
    sl = id % nsl;
  }
}

// Head of slice index i (0 <= i < H) of a packed sequence in the plain
// order.  There slice seq*H + i goes to XCD i % 8 when H % 8 == 0, which
// would spread the query heads of one kv head over several XCDs, each then
// fetching that head's K/V.  This bijection gives XCD x the contiguous heads
// x*H/8 .. (x+1)*H/8 - 1 instead: whole kv groups, or as few XCDs per kv
// head as the group size allows, while every XCD still gets H/8 heads of
// every sequence.  Other H: the identity.
__device__ __forceinline__ int xcd_head(int i, int H) {
  return (H & 7) ? i : (i & 7) * (H >> 3) + (i >> 3);
}

// Raw buffer resource over [base, base + bytes): loads beyond the range
// return zeros, which is how tail rows and keys are padded.  Word 3 is the
// gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Bytes of a buffer over rows 0..n-1 of stride rs elements, d 16-bit
// elements each (the last row ends the buffer).
__device__ __forceinline__ uint32_t slice_bytes(int n, int rs, int d) {
  return n > 0 ? (uint32_t)(((int64_t)(n - 1) * rs + d) * 2) : 0u;
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes per lane from the buffer straight into LDS: lane l's data lands at
// lds + 16*l (lds must be the same for the whole wave; it goes through M0,
// with the one wait state a following LDS load needs after an M0 write).
// Written as inline assembly on purpose: the compiler's own waitcnt
// insertion treats every later LDS read as possibly aliasing a pending
// buffer-to-LDS load and waits for all of them, which would serialise the
// prefetch of the next tiles into every tile.  The kernels instead wait with
// explicit vmcnt counts before each workgroup barrier (wait_vm_barrier).
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(m0), "v"(off), "s"(r)
                   : "memory", "m0");
}

// Wait until at most n vector-memory loads of this wave are outstanding, then
// synchronise the workgroup.  Compiler fences keep LDS accesses on their side.
template <int n>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  constexpr int imm = (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Allow a kernel to use more than the default 64 KiB of dynamic LDS (gfx950
// has 160 KiB per workgroup).  Idempotent; cheap after the first call.
template <typename Kernel>
inline hipError_t allow_lds(Kernel* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace attn
