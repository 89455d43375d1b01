// Shared device and host helpers for the gfx950 kernels of the block-sparse attention library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "bsa.h"

namespace bsa {

// ------------------------------------------------------------------------------- types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {  // tag type: bfloat16 storage (uint16 bit patterns in memory)
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float -> bfloat16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ------------------------------------------------------------------ MFMA fragments
// A k-step covers 16 values of the contraction index.  In both operands lane l holds the
// 8 consecutive contraction indices 8*(l/32) .. 8*(l/32)+7 of row/column (l % 32).
// bf16: one v_mfma_f32_32x32x16_bf16.  fp32: eight v_mfma_f32_32x32x2f32, the i-th taking
// element i of each lane (its contraction index 8*(l/32)+i), which together cover the same
// 16 indices.  Accumulator layout (32x32): lane l, element j holds row
// 8*(j/4) + 4*(l/32) + (j%4), column l % 32.
template <typename T>
struct Frag;
template <>
struct Frag<bf16_t> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  f32x8 v;
};

__device__ __forceinline__ f32x16 mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const Frag<float>& a, const Frag<float>& b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

// Load 8 consecutive elements (16 B for bf16, 32 B for fp32) as a fragment.
__device__ __forceinline__ void load_frag(Frag<bf16_t>& f, const bf16_t* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  f.v = *reinterpret_cast<const f32x8*>(p);
}
// Load elements p[0..3] and p[8..11] as one fragment (the permuted contraction order in
// which lane halves hold runs of 4: see the P V product).
__device__ __forceinline__ void load_frag_split(Frag<bf16_t>& f, const bf16_t* p) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  f.v = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ void load_frag_split(Frag<float>& f, const float* p) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 8);
  f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// float16 operands for the P V product of bfloat16 inputs: P in [0, 256] and V tiles whose
// values fit float16 keep 11 significand bits instead of 8.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
struct Frag16 {
  f16x8 v;
};
__device__ __forceinline__ f32x16 mma(const Frag16& a, const Frag16& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void load_frag_split(Frag16& f, const bf16_t* p) {  // float16 bits stored in a bf16_t slot
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  f.v = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ void frag16_from_f32(Frag16& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = static_cast<_Float16>(x[i]);
}
// Two floats -> packed float16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v;
  v[0] = static_cast<_Float16>(lo);
  v[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void zero_frag(Frag<bf16_t>& f) {
  f.v = bf16x8{};
}
__device__ __forceinline__ void zero_frag(Frag<float>& f) { f.v = f32x8{}; }

// Element conversions.
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return bf16_t{f32_to_bf16(x)};
}
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

// Fragment from 8 floats (rounding to the operand type).
__device__ __forceinline__ void frag_from_f32(Frag<bf16_t>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = static_cast<__bf16>(x[i]);
}
__device__ __forceinline__ void frag_from_f32(Frag<float>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = x[i];
}

// Value from the lane 32 positions away (lanes l and l^32 swap).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, workgroups dispatched round-robin

// ------------------------------------------------------------------ swizzled LDS rows
// Unpadded LDS rows of ROWB bytes with an XOR swizzle of 16-byte chunks: chunk c of row r
// sits at chunk position c ^ ((r / RP) & MASK), where RP rows share one 256-byte bank line;
// the 16 lanes of a fragment read then hit 16 distinct chunks.  Tiles land in such rows by
// direct global-to-LDS copies, each lane fetching the chunk that the swizzle puts in its slot.
template <int ROWB>
struct Swz {
  static constexpr int CPR = ROWB / 16;
  static constexpr int RP = ROWB >= 256 ? 1 : 256 / ROWB;
  static constexpr int MASK = (CPR < 16 ? CPR : 16) - 1;
  static __device__ __forceinline__ int pos(int r, int c) { return c ^ ((r / RP) & MASK); }
  static __device__ __forceinline__ const uint4* chunk(const void* base, int r, int c) {
    return reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(base) + r * ROWB + pos(r, c) * 16);
  }
};

// Fragment of 8 consecutive elements starting at element e0 of swizzled row `row`.
template <typename S>
__device__ __forceinline__ void swz_frag(Frag<bf16_t>& f, const void* base, int row, int e0) {
  f.v = __builtin_bit_cast(bf16x8, *S::chunk(base, row, e0 / 8));
}
template <typename S>
__device__ __forceinline__ void swz_frag(Frag<float>& f, const void* base, int row, int e0) {
  const f32x4 lo = __builtin_bit_cast(f32x4, *S::chunk(base, row, e0 / 4));
  const f32x4 hi = __builtin_bit_cast(f32x4, *S::chunk(base, row, e0 / 4 + 1));
  f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Wait for this wave's outstanding global memory operations, tile copies included.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// s_waitcnt vmcnt(N): at most N vector memory operations of this wave still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Workgroup barrier for copy pipelines: waits for this wave's LDS operations and then for
// every wave, but not for outstanding global loads, including copies into LDS, which are
// awaited explicitly with wait_vmem_n (the compiler's own barrier lowering would wait for all
// of them).  The memory clobber keeps memory accesses on their side of it.
__device__ __forceinline__ void pipe_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ host helpers
inline bsa_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? BSA_OK : BSA_E_HIP;
}

inline bool valid_dtype(int dtype) { return dtype == BSA_F32 || dtype == BSA_BF16; }
inline size_t dtype_size(int dtype) { return dtype == BSA_BF16 ? 2 : 4; }

}  // namespace bsa
