// Device-side building blocks shared by the MoE kernels (gfx950 / CDNA4).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bfloat16 <-> float32 (bf16 kept as raw 16-bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// Matrix-core tile: v_mfma_f32_32x32x16_bf16.
//   A fragment: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]
//   B fragment: lane l holds B[8*(l/32) .. +7][l % 32]  (k-contiguous per column)
//   C: lane l holds column l % 32, value v at row 8*(v/4) + 4*(l/32) + v%4
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ int mfma_c_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes:
// out[j] holds column j of the input, rows 0..7 in order.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // low half <- row 2d, high half <- row 2d+1, both taken from column j
      out[j][d] = __builtin_amdgcn_perm(in[2 * d + 1][j >> 1], in[2 * d][j >> 1], sel);
    }
  }
}

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

template <typename T>
__device__ __forceinline__ T shfl(T v, int src) { return __shfl(v, src, kWave); }
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
// Maximum over the wave, returned uniformly: DPP steps within each row of 16
// lanes (swap neighbours, swap pairs, mirror halves of 8, mirror the 16),
// then the four row results read as scalars. No LDS traffic.
__device__ __forceinline__ float wave_max_dpp(float v) {
  auto step = [](float x, auto ctrl) {
    constexpr int c = decltype(ctrl)::value;
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), c, 0xF, 0xF, false)));
  };
  v = step(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  v = step(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  v = step(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v = step(v, std::integral_constant<int, 0x140>{});  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

}  // namespace moe
