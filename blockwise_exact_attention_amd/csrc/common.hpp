// Device-side helpers shared by the gfx950 attention kernels: vector types,
// bf16 rounding, the bf16 MFMA wrapper and the mask bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bea {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Two floats -> two bf16 (round to nearest even) packed low/high in a dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16), one wave.
// Lane l supplies A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32]; it
// receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in element r.
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b,
                                                 f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

// Key j may be seen by query row i iff dlo <= j - i <= dhi and j < l_k.  The
// host folds causal, the window and both offsets into (dlo, dhi), saturated
// to int32: with qpos = q_offset + i, kpos = k_offset + j and
// delta = q_offset - k_offset, causal gives j - i <= delta, the window gives
// delta - win_l <= j - i <= delta + win_r.
struct MaskBounds {
  int dlo;
  int dhi;
};

}  // namespace bea
