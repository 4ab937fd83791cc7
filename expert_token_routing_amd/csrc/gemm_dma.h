// Matrix-core tile pieces fed by direct global->LDS loads (gfx950).
//
// A workgroup of 256 threads (4 waves, 2 x 2) computes a BM x 256 output tile
// in k stages of 64. Each stage is brought into LDS by 16-byte
// buffer_load_dwordx4 ... lds: lane l of a wave writes LDS bytes
// [base + 16 l, base + 16 l + 16), so the per-lane global offset picks the
// LDS layout. Two stages are double buffered and the next stage's loads are in
// flight while the current one is multiplied.
//
// LDS layouts (both conflict-free on the 64 banks of 4 bytes of gfx950):
//  * A (k-contiguous rows): row r occupies bytes [128 r, 128 r + 128); its
//    16-byte chunk c (k = 8c .. 8c+7) sits at chunk position c ^ ((r >> 1) & 7),
//    so 16 lanes reading one chunk of 16 consecutive rows (ds_read_b128) hit 16
//    different 16-byte slots of a 256-byte bank window.
//  * B (n-contiguous, [k][n] as in memory): 4 x 16 blocks of 128 bytes, block
//    (kq, nq) = rows 4kq .. 4kq+3, columns 16nq .. 16nq+15, at byte
//    128 (kq * BN/16 + nq), row r of the block at +32 r. ds_read_b64_tr_b16
//    reads one block per group of 16 lanes and hands lane i the 4 k-values of
//    column i; two such reads give the 8 k-values of an MFMA B fragment.
#pragma once

#include "moe_device.h"

namespace moe {
namespace dma {

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kBN = 256;
constexpr int kNQ = kBN / 16;                 // 16-column blocks per B stage
constexpr int kBStageBytes = kBK * kBN * 2;   // 32 KiB

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define MOE_LDS __attribute__((address_space(3)))

// Wait until at most N vector-memory operations of this wave are outstanding
// (expcnt / lgkmcnt left alone), then barrier the workgroup.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}
// All LDS reads of this wave done, then barrier (before a buffer is refilled).
__device__ __forceinline__ void wait_lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, no stride, `bytes` addressable
// (accesses beyond read as zero), default data format.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = int(bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return i32x4{int32_t(uint32_t(a)), int32_t(uint32_t(a >> 32) & 0xFFFFu), n, 0x00020000};
}

// 16 bytes per lane from buffer `rsrc` at byte voff + soff into LDS at
// lds_base + 16 * lane. Written as inline assembly so the compiler does not
// treat the in-flight transfer as a pending LDS write (it would otherwise wait
// for all of them before any LDS read); completion is awaited explicitly with
// s_waitcnt vmcnt. No register is written by the instruction; M0 (the LDS
// base) is an input the compiler sets.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, const MOE_LDS char* lds_base) {
  const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds_base));
  // one wait state between the M0 write and the LDS-direct load
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}

// A stage: BM rows x 64 k from a k-contiguous matrix. Wave w issues BM/32
// loads; load i fills tile rows 8 (i*4 + w) .. +7. The buffer starts at the
// tile's first row; per-lane byte offsets are fixed for the tile and the k
// stage goes in the scalar offset.
template <int BM>
struct ALoader {
  i32x4 rsrc;
  uint32_t voff[BM / 32];
  __device__ __forceinline__ void init(const uint16_t* tile_base, int lda, int rows) {
    rsrc = buffer_rsrc(tile_base, int64_t(rows) * lda * 2);
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int r = 8 * (i * 4 + w) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[i] = uint32_t(min(r, rows - 1)) * uint32_t(lda) * 2u + 16u * uint32_t(c);
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* As, int k0) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i)
      dma16(rsrc, voff[i], 2u * uint32_t(k0), As + 8 * (i * 4 + w) * 128);
  }
};

// B stage: 64 k x 256 n of an n-contiguous matrix (leading dimension ldw).
// Wave w issues 8 loads; load j fills blocks 8 (j*4 + w) .. +7 (kq = block / 16).
// col_of(s) maps tile column s (a multiple of 8) to a valid matrix column.
struct BLoader {
  i32x4 rsrc;
  uint32_t voff[8];
  uint32_t stage_bytes;
  template <typename ColOf>
  __device__ __forceinline__ void init(const uint16_t* W, int ldw, int K, ColOf col_of) {
    rsrc = buffer_rsrc(W, int64_t(K) * ldw * 2);
    stage_bytes = uint32_t(ldw) * 2u;
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 8 * (j * 4 + w) + (lane >> 3);
      const int kq = blk / kNQ;
      const int nq = blk % kNQ;
      const int r = (lane & 7) >> 1;
      const int c = lane & 1;
      voff[j] = uint32_t(4 * kq + r) * uint32_t(ldw) * 2u + 2u * uint32_t(col_of(16 * nq + 8 * c));
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* Bs, int k0) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      dma16(rsrc, voff[j], uint32_t(k0) * stage_bytes, Bs + 8 * (j * 4 + w) * 128);
  }
};

// Per-lane LDS byte offsets of this wave's MFMA fragments inside one stage.
// A: row m = wrow0 + fm*32 + (lane & 31) at 128 m (+ 4096 fm as an
//    immediate), chunk (2 ks + lane/32) ^ ((m >> 1) & 7): one base per ks.
// B: block (kq, nq) with kq = 4 ks + 2 (lane/32) (+1 for the upper four k),
//    nq = wcol0/16 + 2 fn + ((lane >> 4) & 1): one base, the rest immediates.
struct FragAddr {
  uint32_t a[4];
  uint32_t b;
  __device__ __forceinline__ void init(int wrow0, int wcol0) {
    const int lane = lane_id();
    const int m = wrow0 + (lane & 31);
    const int sw = (m >> 1) & 7;
    const int khalf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = uint32_t(m * 128 + 16 * ((2 * ks + khalf) ^ sw));
    b = uint32_t((2 * khalf * kNQ + wcol0 / 16 + ((lane >> 4) & 1)) * 128 + 8 * (lane & 15));
  }
};

template <int FM, int FN>
__device__ __forceinline__ void load_frags(const MOE_LDS char* As, const MOE_LDS char* Bs, const FragAddr& fa, int ks,
                                           u32x4 (&a)[FM], u32x4 (&b)[FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) a[fm] = *reinterpret_cast<const MOE_LDS u32x4*>(As + fa.a[ks] + fm * 4096);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const MOE_LDS char* p0 = Bs + fa.b + ks * (4 * kNQ * 128) + fn * 256;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0 + kNQ * 128));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    b[fn] = u32x4{l2.x, l2.y, h2.x, h2.y};
  }
}

// One 64-deep stage of MFMA work for this wave's FM x FN blocks of 32 x 32;
// the fragments of the next 16-deep step load while the current one multiplies.
template <int FM, int FN>
__device__ __forceinline__ void mma_stage(const MOE_LDS char* As, const MOE_LDS char* Bs, const FragAddr& fa,
                                          f32x16 (&acc)[FM][FN]) {
  u32x4 a[2][FM], b[2][FN];
  load_frags<FM, FN>(As, Bs, fa, 0, a[0], b[0]);
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    if (ks + 1 < kBK / 16) load_frags<FM, FN>(As, Bs, fa, ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32x32x16(a[ks & 1][fm], b[ks & 1][fn], acc[fm][fn]);
  }
}

}  // namespace dma
}  // namespace moe
