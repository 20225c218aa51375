// Device helpers shared by the gfx950 matrix-core kernels (forward and backward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace longattn {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi of a packed bf16 pair, in fp32 (one dot product with (1, 1)).  Softmax rows sum
// the weights after their rounding to bf16, the values the matrix cores multiply with the value
// rows, so that the normalised weights of a row add up to one.
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  constexpr uint32_t kOnes = 0x3f803f80u;  // (1.0, 1.0) in bf16
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, kOnes), acc, false);
}

// sigmoid(x) = 1 / (1 + e^-x), from the hardware exp2 and reciprocal (saturates to 0 and 1).
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + exp2_fast(-1.44269504088896340736f * x));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// s if bit `bit` of w is set, else ninf (which holds -inf): a sign-extended one-bit field
// extract and a bitfield select (the and/or form below compiles to v_bfi_b32).  Plain code, not
// inline assembly: s is often a matrix-core result, and only instructions the compiler sees get
// the wait states a vector read of such a result needs.
__device__ __forceinline__ float keep_if_bit(float s, uint32_t w, int bit, float ninf) {
  const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)w, bit, 1);
  return __uint_as_float((sel & __float_as_uint(s)) | (~sel & __float_as_uint(ninf)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const void, p)));
}

// Logical workgroup id such that consecutive ids run on the same XCD.  Workgroups are handed to
// the 8 XCDs round robin, so neighbouring query tiles (which re-read the same K/V rows) would
// otherwise land in 8 different L2 caches.  This is a bijection on [0, G).
// Balancing priority of a wave whose workgroup has `rem` key tiles left: 3 with six or more, 2
// with four or five, 1 with two or three, 0 for the last one.  The hardware issues the waves of
// the oldest workgroup on a SIMD first, so of the workgroups that share a CU the first finishes in
// about half the time of the last, and in the final round of a grid the CU then runs with fewer
// and fewer workgroups; with the priority the workgroups of a CU progress and finish together.
__device__ __forceinline__ void balancing_priority(int rem) {
  if (rem >= 6) __builtin_amdgcn_s_setprio(3);
  else if (rem >= 4) __builtin_amdgcn_s_setprio(2);
  else if (rem >= 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ int xcd_remap(int x, int G) {
  const int q = G >> 3, r = G & 7;
  const int xcd = x & 7, idx = x >> 3;
  return xcd * q + min(xcd, r) + idx;
}

// 16-byte chunk swizzles.  K: 16 consecutive rows reading the same logical chunk land in 16
// distinct bank groups (64 banks of 4 bytes).  V: the transposing read of 4 consecutive rows x
// 64 bytes by 32 lanes lands in distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 64) return (row >> 1) & 7;
  else return row & 15;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 64) return ((row >> 1) & 1) << 2;
  else return (row & 3) << 2;
}

// Wait until at most n of this wave's vector-memory loads are outstanding (gfx9 s_waitcnt
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0, dword data format).  Loads at
// offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// One 16-byte buffer load per lane straight into LDS: lane l's 16 bytes (from byte offset voff
// of the resource) land at LDS byte address lds_base + 16*l.  Inline assembly so that the
// compiler does not treat it as an LDS store it must order against LDS reads of other stages
// (it would wait for every load in flight); the wave waits for these loads itself (vmcnt) before
// the tile barrier.  No output registers; the operands are consumed when the load issues.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// One 4-byte buffer load per lane straight into LDS: lane l's word lands at lds_base + 4*l.
__device__ __forceinline__ void lds_dma4(const u32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

}  // namespace mfma
}  // namespace longattn
