// Workgroup-level bf16 matrix-core tile pieces for gfx950.
//
// A workgroup is 256 threads = 4 waves laid out 2 x 2 over a BM x BN output
// tile; wave (wm, wn) owns rows [wm*BM/2, (wm+1)*BM/2) and columns
// [wn*BN/2, (wn+1)*BN/2) as FM x FN blocks of 32 x 32 (v_mfma_f32_32x32x16_bf16).
// Both operands sit in LDS k-contiguous: As[row][k], Bs[col][k], with a row
// pitch of BK + 8 elements so that the 16-byte fragment reads of 32 lanes on
// consecutive rows fall in distinct banks.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kBK = 64;            // k extent of one LDS stage
constexpr int kLdk = kBK + 8;      // LDS row pitch in bf16 elements
constexpr int kThreads = 256;

// One k-stage of MFMA work for this wave: acc += A_tile(wave rows) * B_tile(wave cols),
// summed over NP planes of B (NP > 1 splits a float32 operand into bf16 parts).
template <int FM, int FN, int NP, int BN>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                          int wrow0, int wcol0, f32x16 (&acc)[FM][FN]) {
  const int lane = lane_id();
  const int r = lane & 31;
  const int kq = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    u32x4 a[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      a[fm] = *reinterpret_cast<const u32x4*>(As + (wrow0 + fm * 32 + r) * kLdk + ks * 16 + kq);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      u32x4 b[FN];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        b[fn] = *reinterpret_cast<const u32x4*>(Bs + (p * BN + wcol0 + fn * 32 + r) * kLdk + ks * 16 + kq);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32x32x16(a[fm], b[fn], acc[fm][fn]);
    }
  }
}

// Rows of a k-contiguous matrix (row pointer per tile row) -> registers.
// Thread t moves 16-byte chunk (t & 7) of tile rows (t >> 3) + 32*i.
// Chunks at or past K are zero.
template <int ROWS>
struct KRowsLoader {
  static constexpr int kPer = ROWS / 32;
  u32x4 v[kPer];

  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr row_ptr, int k0, int K) {
    const int t = threadIdx.x;
    const int c = t & 7;
    const int kk = k0 + c * 8;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = (t >> 3) + 32 * i;
      if (kk < K) {
        v[i] = *reinterpret_cast<const u32x4*>(row_ptr(row) + kk);
      } else {
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* __restrict__ S) const {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = (t >> 3) + 32 * i;
      *reinterpret_cast<u32x4*>(S + row * kLdk + c * 8) = v[i];
    }
  }
};

// A 64 (k) x 256 (n) block of an n-contiguous matrix -> registers -> LDS as
// Bs[n][k]. Thread t holds the 8 x 8 block of k rows 8*(t & 7) .. +7 and tile
// columns 8*(t >> 3) .. +7; `col_of(slot0)` maps a tile column to the matrix
// column (or -1 if the 8 columns are out of range).
struct NColsTransposeLoader {
  u32x4 v[8];
  template <typename ColOf>
  __device__ __forceinline__ void load(const uint16_t* __restrict__ W, int64_t ldw, ColOf col_of, int k0, int K) {
    const int t = threadIdx.x;
    const int kb = t & 7;
    const int col = col_of((t >> 3) * 8);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = k0 + kb * 8 + r;
      if (col >= 0 && k < K) {
        v[r] = *reinterpret_cast<const u32x4*>(W + int64_t(k) * ldw + col);
      } else {
        v[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* __restrict__ S) const {
    const int t = threadIdx.x;
    const int kb = t & 7;
    const int n0 = (t >> 3) * 8;
    u32x4 o[8];
    transpose8x8_b16(v, o);
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(S + (n0 + j) * kLdk + kb * 8) = o[j];
  }
};

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
}

// Exclusive scan over a block of NT threads; returns the prefix, writes the total.
template <int NT = 256>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp /* >= NT/64 ints */, int& total) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) s_tmp[w] = inc;
  __syncthreads();
  int base = 0;
  int tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int s = s_tmp[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

}  // namespace moe
