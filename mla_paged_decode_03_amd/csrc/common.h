// Shared device helpers for the gfx950 kernels (wave64, MFMA, bf16/fp8).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// D += A * B on a 32x32x16 bf16 tile.  Lane l holds A[l%32][8*(l/32)+e] and
// B[8*(l/32)+e][l%32] (e = 0..7); D[i][j] lives in lane j + 32*((i/4)%2),
// element 4*(i/8) + i%4.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Tiles of a per-head batched GEMM in a 1-D launch.  The dispatcher deals workgroups to
// the 8 XCDs round-robin, so launch index L runs on XCD L % 8; XCD x takes the tiles
// x * per_xcd .. (x + 1) * per_xcd - 1 in (head, m block, n block) order, so the tiles
// that read one head's operands run on one XCD and share its L2.  The launch has
// 8 * per_xcd workgroups, per_xcd = ceil(tiles / 8); false past the last tile.
struct HeadTile {
  int h, mb, nb;
};
__device__ __forceinline__ bool head_tile(int nbk, int mbk, int H, HeadTile* t) {
  const int64_t tiles = (int64_t)nbk * mbk * H;
  const int64_t per_xcd = (tiles + 7) / 8;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= tiles) return false;
  t->nb = (int)(item % nbk);
  t->mb = (int)((item / nbk) % mbk);
  t->h = (int)(item / ((int64_t)nbk * mbk));
  return true;
}

// Round-to-nearest-even float -> bf16 pattern (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2_t));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 pair (round to nearest even), one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, f16x2_t));
}
// Packed fp16 pair -> two floats (exact).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[1];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Four OCP e4m3fn bytes -> four bf16 values (two dwords), one instruction per pair.
// Every e4m3fn value is exact in bf16, so a scale of 1 makes the conversion exact.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
  u32x2_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// Load through the constant address space: with a wave-uniform address this
// becomes a scalar (SMEM) load instead of a vector load.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Combines a value with the one held by lane l ^ 32 (the other half of the MFMA
// layout).  v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with both operands holding x, each lane ends up with its
// own value in one result and its partner's in the other.  The second operand passes
// through an empty asm so that the compiler cannot see the two operands are equal
// (it folds the second result into the first when it can).
__device__ __forceinline__ uint2 half_pair(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("" : "+v"(b));
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const uint2 r = half_pair(x);
  return fmaxf(__builtin_bit_cast(float, r.x), __builtin_bit_cast(float, r.y));
}
__device__ __forceinline__ float half_sum(float x) {
  const uint2 r = half_pair(x);
  return __builtin_bit_cast(float, r.x) + __builtin_bit_cast(float, r.y);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace mla
