// Matrix-core tile pieces fed by direct global->LDS loads (gfx950).
//
// A workgroup of 512 threads (8 waves, 2 x 4) computes a BM x 256 output tile
// in k stages of 32. Each stage is brought into LDS by 16-byte
// buffer_load_dwordx4 ... lds: lane l of a wave writes LDS bytes
// [base + 16 l, base + 16 l + 16), so the per-lane global offset picks the
// LDS layout. A ring of kStages stages keeps kStages - 1 of them in flight
// while one is multiplied, enough bytes to cover the HBM latency.
//
// LDS layouts (both conflict-free on the 64 banks of 4 bytes of gfx950):
//  * A (k-contiguous rows): row r occupies bytes [64 r, 64 r + 64); its
//    16-byte chunk c (k = 8c .. 8c+7) sits at chunk position c ^ ((r >> 2) & 3),
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

constexpr int kBK = 32;
constexpr int kStages = 4;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 256;
constexpr int kNQ = kBN / 16;                 // 16-column blocks per B stage
constexpr int kBStageBytes = kBK * kBN * 2;   // 16 KiB
constexpr int kARowBytes = kBK * 2;           // 64

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
// All LDS reads of this wave returned (vmcnt / expcnt left alone).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}
// All LDS reads of this wave done, then barrier (before a buffer is refilled).
__device__ __forceinline__ void wait_lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, no stride, `bytes` addressable
// (accesses beyond read as zero), default data format.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = int(bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  // the values are the same on every lane; say so, so they live in SGPRs
  return i32x4{__builtin_amdgcn_readfirstlane(int32_t(uint32_t(a))),
               __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane(n), 0x00020000};
}

// 16 bytes per lane from buffer `rsrc` at byte voff + soff into LDS at
// lds_base + 16 * lane. Written as inline assembly so the compiler does not
// treat the in-flight transfer as a pending LDS write (it would otherwise wait
// for all of them before any LDS read); completion is awaited explicitly with
// s_waitcnt vmcnt. No register is written by the instruction; M0 (the LDS
// base) is an input the compiler sets.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, const MOE_LDS char* lds_base) {
  const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds_base));
  // keep the scalar offset in an SGPR (soffset takes no literal constants)
  asm volatile("" : "+s"(soff));
  // one wait state between the M0 write and the LDS-direct load
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}

// A stage: BM rows x 32 k from a k-contiguous matrix. Wave w issues BM/128
// loads; load i fills tile rows 16 (i*8 + w) .. +15. The buffer starts at the
// tile's first row; per-lane byte offsets are fixed for the tile and the k
// stage goes in the scalar offset.
template <int BM>
struct ALoader {
  static constexpr int kPer = BM / 16 / kWaves;
  i32x4 rsrc;
  uint32_t voff[kPer];
  __device__ __forceinline__ void init(const uint16_t* tile_base, int lda, int rows) {
    rsrc = buffer_rsrc(tile_base, int64_t(rows) * lda * 2);
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = 16 * (i * kWaves + w) + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      voff[i] = uint32_t(min(r, rows - 1)) * uint32_t(lda) * 2u + 16u * uint32_t(c);
    }
  }
  // Same tile, but tile row r is row src_row(r) of the whole matrix `base`
  // (rows.. rows_total) -- a gather, used to read token vectors in place.
  template <typename SrcRow>
  __device__ __forceinline__ void init_gather(const uint16_t* base, int lda, int rows_total, int rows,
                                              SrcRow src_row) {
    rsrc = buffer_rsrc(base, int64_t(rows_total) * lda * 2);
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = 16 * (i * kWaves + w) + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      voff[i] = uint32_t(src_row(min(r, rows - 1))) * uint32_t(lda) * 2u + 16u * uint32_t(c);
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* As, int k0) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rsrc, voff[i], 2u * uint32_t(k0), As + 16 * (i * kWaves + w) * kARowBytes);
  }
};

// B stage: 32 k x 256 n of an n-contiguous matrix (leading dimension ldw).
// Wave w issues 2 loads; load j fills blocks 8 (j*8 + w) .. +7 (kq = block / 16).
// col_of(s) maps tile column s (a multiple of 8) to a valid matrix column.
struct BLoader {
  static constexpr int kPer = kBK / 4 * kNQ / 8 / kWaves;  // 2
  i32x4 rsrc;
  uint32_t voff[kPer];
  uint32_t stage_bytes;
  template <typename ColOf>
  __device__ __forceinline__ void init(const uint16_t* W, int ldw, int K, ColOf col_of) {
    rsrc = buffer_rsrc(W, int64_t(K) * ldw * 2);
    stage_bytes = uint32_t(ldw) * 2u;
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int blk = 8 * (j * kWaves + w) + (lane >> 3);
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
    for (int j = 0; j < kPer; ++j) dma16(rsrc, voff[j], uint32_t(k0) * stage_bytes, Bs + 8 * (j * kWaves + w) * 128);
  }
};

// Per-lane LDS byte offsets of this wave's MFMA fragments inside one stage.
// A: row m = wrow0 + fm*32 + (lane & 31) at 64 m (+ 2048 fm as an
//    immediate), chunk (2 ks + lane/32) ^ ((m >> 2) & 3): one base per ks.
// B: block (kq, nq) with kq = 4 ks + 2 (lane/32) (+1 for the upper four k),
//    nq = wcol0/16 + 2 fn + ((lane >> 4) & 1): one base, the rest immediates.
struct FragAddr {
  uint32_t a[kBK / 16];
  uint32_t b;
  __device__ __forceinline__ void init(int wrow0, int wcol0) {
    const int lane = lane_id();
    const int m = wrow0 + (lane & 31);
    const int sw = (m >> 2) & 3;
    const int khalf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) a[ks] = uint32_t(m * kARowBytes + 16 * ((2 * ks + khalf) ^ sw));
    b = uint32_t((2 * khalf * kNQ + wcol0 / 16 + ((lane >> 4) & 1)) * 128 + 8 * (lane & 15));
  }
};

template <int FM, int FN>
struct Frags {
  u32x4 a[FM];
  u32x4 b[FN];
};

// Issue the LDS reads of one 16-deep step's fragments (FM b128 + 2 FN tr reads).
template <int FM, int FN>
__device__ __forceinline__ void load_frags(const MOE_LDS char* As, const MOE_LDS char* Bs, const FragAddr& fa, int ks,
                                           Frags<FM, FN>& f) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
    f.a[fm] = *reinterpret_cast<const MOE_LDS u32x4*>(As + fa.a[ks] + fm * 32 * kARowBytes);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const MOE_LDS char* p0 = Bs + fa.b + ks * (4 * kNQ * 128) + fn * 256;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0 + kNQ * 128));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    f.b[fn] = u32x4{l2.x, l2.y, h2.x, h2.y};
  }
}

template <int FM, int FN>
__device__ __forceinline__ void mma_frags(const Frags<FM, FN>& f, f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32x32x16(f.a[fm], f.b[fn], acc[fm][fn]);
}

// Ask the scheduler to alternate the region's MFMAs with its LDS reads, so
// the reads of the next step stream in under the current step's MFMAs.
template <int FM, int FN>
__device__ __forceinline__ void interleave_mfma_with_reads() {
  constexpr int kMfma = FM * FN;
  constexpr int kReads = FM + 2 * FN;
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
#pragma unroll
  for (int i = kMfma; i < kReads; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}

}  // namespace dma
}  // namespace moe
