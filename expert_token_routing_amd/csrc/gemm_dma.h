// Matrix-core tile pieces fed by direct global->LDS loads (gfx950).
//
// Operands are brought into LDS by 16-byte buffer_load_dwordx4 ... lds: lane l
// of a wave writes LDS bytes [base + 16 l, base + 16 l + 16), so the per-lane
// global offset picks the LDS layout. Completion is tracked with s_waitcnt
// vmcnt per wave plus a workgroup barrier.
//
// LDS layouts (conflict-free on the 64 banks of 4 bytes of gfx950):
//  * k-contiguous rows (token rows, router weight planes): row r holds the
//    stage's k range contiguously; its 16-byte chunks are XOR-swizzled with
//    row bits so that 16 lanes reading one chunk of 16 consecutive rows
//    (ds_read_b128) hit 16 different 16-byte slots of a 256-byte bank window.
//  * n-contiguous weights ([k][n] as in memory): 4 x 16 blocks of 128 bytes,
//    block (kq, nq) = rows 4kq .. 4kq+3, columns 16nq .. 16nq+15, row r of
//    the block at +32 r. ds_read_b64_tr_b16 reads one block per group of 16
//    lanes and hands lane i the 4 k-values of column i; two such reads give
//    the 8 k-values of an MFMA B fragment.
#pragma once

#include "moe_device.h"

namespace moe {
namespace dma {

constexpr int kBK = 32;                       // k per stage of the router pipeline
constexpr int kStages = 4;                    // router pipeline depth
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
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
// wait_vm_barrier<n> for a wave-uniform n known only at run time; n above
// MAX waits for MAX (stricter, never looser).
template <int MAX>
__device__ __forceinline__ void wait_vm_barrier_dyn(int n) {
  if constexpr (MAX == 0) {
    wait_vm_barrier<0>();
  } else {
    if (n >= MAX)
      wait_vm_barrier<MAX>();
    else
      wait_vm_barrier_dyn<MAX - 1>(n);
  }
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
// s_waitcnt vmcnt. M0 (the LDS base) is an input the compiler sets.
// The compiler does not look inside the assembly for hazards: a memory
// instruction that reads an SGPR written by a vector instruction (the
// compiler may produce the scalar offset with v_readlane when it keeps
// scalars in vector-register lanes) needs 5 wait states, else it may use the
// old value. So the offset is first copied by a scalar move, whose result
// needs none; the move also gives the wait state after the M0 write. (The
// build scans the generated code for such a write to the descriptor.)
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, const MOE_LDS char* lds_base) {
  const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds_base));
  // keep the scalar offset in an SGPR (soffset takes no literal constants)
  asm volatile("" : "+s"(soff));
  uint32_t s;
  asm volatile("s_mov_b32 %0, %3\n\tbuffer_load_dwordx4 %1, %2, %0 offen lds"
               : "=&s"(s)
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

// ROWS k-contiguous rows x 64 k (128 bytes per row, one whole line per
// request). Row r occupies LDS bytes [128 r, 128 r + 128); its chunk c
// (k = 8c .. 8c+7) sits at position c ^ ((r >> 1) & 7). Load i of wave w
// fills rows 8 (i * kWaves + w) .. +7, 8 lanes per row.
template <int ROWS>
struct RowLoader64 {
  static constexpr int kPer = ROWS / 8 / kWaves;
  i32x4 rsrc;
  uint32_t voff[kPer];
  __device__ __forceinline__ void init(const uint16_t* tile_base, int ld, int rows) {
    rsrc = buffer_rsrc(tile_base, int64_t(rows) * ld * 2);
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = 8 * (i * kWaves + w) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[i] = uint32_t(min(r, rows - 1)) * uint32_t(ld) * 2u + 16u * uint32_t(c);
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* dst, int k0) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rsrc, voff[i], 2u * uint32_t(k0), dst + 1024 * (i * kWaves + w));
  }
};

// ---------------------------------------------------------------------------
// Expert-panel tiles: a block of up to kRowsMax rows of one expert (its rows
// split evenly over ceil(rows / kRowsMax) blocks) x kBN weight columns.
// v_mfma_f32_16x16x32_bf16:
//   A fragment: lane l holds A[l % 16][8*(l/16) .. +7]
//   B fragment: lane l holds B[8*(l/16) .. +7][l % 16]
//   C: lane l holds column l % 16, rows 4*(l/16) .. +3
// 8 waves: kWR wave rows x kWC wave columns of 64. 16-row fragment f of the
// tile belongs to wave row f % kWR (as its fragment f / kWR), so any row count
// splits over the wave rows to within one fragment.
// ---------------------------------------------------------------------------
namespace panel {

constexpr int kWR = 2;                       // wave rows (kWaves / kWR wave columns of 64)
constexpr int kWC = kWaves / kWR;
constexpr int kBN = 64 * kWC;                // weight columns per tile
constexpr int kFMMax = 9;                    // 16-row fragments per wave row
constexpr int kRowsMax = 16 * kFMMax * kWR;  // rows per tile
constexpr int kFN = 4;                       // 16-column fragments per wave
constexpr int kNQ = kBN / 16;                // 16-column blocks of a B stage
constexpr int kSK = 64;                      // k per LDS stage (32 or 64)
constexpr int kSub = kSK / 32;               // MFMA k steps per stage
constexpr int kRowBytes = kSK * 2;           // bytes of one A row in a stage (64 or 128)
constexpr int kLanesPerRow = kRowBytes / 16; // 4 or 8
constexpr int kRowsPerLoad = 64 / kLanesPerRow;
constexpr int kBStage = kSK * kBN * 2;
// Pipeline depth by tile height: a tile of FMT fragments per wave row has an
// A stage of 16 kWR FMT rows, and gets 4 stages when 4 fit in the LDS left
// beside the tile schedule's tables (about 8 KiB), else 2. Only FMT = 1 tiles
// (up to 32 rows: few rows per expert, where the weight stream is the whole
// cost) get 4, keeping twice the weight bytes in flight. A depth of 3 would
// fit up to FMT = 4, but the buffer rotation modulo 3 made the kernel spill
// registers.
constexpr int kLdsBudget = 160 * 1024 - 8 * 1024 - 512;
constexpr int a_stage_bytes(int fmt) { return 16 * kWR * fmt * kRowBytes; }
constexpr int stages_for(int fmt) {
  return kLdsBudget / (a_stage_bytes(fmt) + kBStage) >= 4 ? 4 : 2;
}
constexpr int lds_bytes_max() {
  int m = 0;
  for (int f = 1; f <= kFMMax; ++f) {
    const int b = stages_for(f) * (a_stage_bytes(f) + kBStage);
    m = b > m ? b : m;
  }
  return m;
}
constexpr int kLdsBytes = lds_bytes_max();
static_assert(2 * (a_stage_bytes(kFMMax) + kBStage) <= kLdsBudget, "two stages of the tallest tile must fit in LDS");

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Position of 16-byte chunk c of row r inside the row: rows are kRowBytes
// long, so a 256-byte bank window holds 256 / kRowBytes rows; the swizzle
// makes the 16 rows read by a 16-lane ds_read_b128 phase (same chunk) land on
// 16 different 16-byte slots.
__device__ __forceinline__ int a_chunk_pos(int r, int c) {
  return kSK == 32 ? (c ^ ((r >> 2) & 3)) : (c ^ ((r >> 1) & 7));
}

// A stage: R16 rows (a multiple of 16) x kSK k. Load j (kRowsPerLoad rows,
// kLanesPerRow lanes per row) is issued by wave j % 8; wave w issues
// count(w) of them, at most kPerMax.
struct ALoaderP {
  static constexpr int kPerMax = (kRowsMax / kRowsPerLoad + kWaves - 1) / kWaves;
  i32x4 rsrc;
  uint32_t voff[kPerMax];
  int count;
  template <typename SrcRow>
  __device__ __forceinline__ void init(const uint16_t* base, int64_t bytes, int lda, int rows, int r16,
                                       SrcRow src_row) {
    rsrc = buffer_rsrc(base, bytes);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nloads = r16 / kRowsPerLoad;
    count = __builtin_amdgcn_readfirstlane(max(0, (nloads - w + kWaves - 1) / kWaves));
#pragma unroll
    for (int i = 0; i < kPerMax; ++i) {
      const int r = kRowsPerLoad * (i * kWaves + w) + lane / kLanesPerRow;
      const int c = a_chunk_pos(r, lane % kLanesPerRow);
      voff[i] = uint32_t(src_row(min(r, rows - 1))) * uint32_t(lda) * 2u + 16u * uint32_t(c);
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* As, int k0) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPerMax; ++i)
      if (i < count) dma16(rsrc, voff[i], 2u * uint32_t(k0), As + 1024 * (i * kWaves + w));
  }
  // A stage whose k range holds only its first 32 values (the end of K): the
  // lanes of the second half read the first half again instead, so no
  // request reaches past a row's end (the extra k values are multiplied as
  // zeros). A lane's logical chunk is (lane % 8) ^ ((4 w + lane / 16) % 8)
  // for every load i: the row of load i is 64 i + 8 w + lane / 8, and 64 i
  // does not change the swizzle bits.
  __device__ __forceinline__ void issue_half(MOE_LDS char* As, int k0) const {
    static_assert(kSK == 64 && kRowsPerLoad == 8 && kWaves == 8, "chunk of a lane independent of the load");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = lane_id();
    uint32_t back = ((lane & 7) ^ ((4 * w + (lane >> 4)) & 7)) >= 4 ? 64u : 0u;
    // opaque here, so the adjusted offsets are formed only when this runs
    // (once per tile) instead of being kept in registers across the k loop
    asm volatile("" : "+v"(back));
#pragma unroll
    for (int i = 0; i < kPerMax; ++i)
      if (i < count) dma16(rsrc, voff[i] - back, 2u * uint32_t(k0), As + 1024 * (i * kWaves + w));
  }
};

// Block (kq, nq) of a B stage sits at 128 (kq * kNQ + (nq ^ b_swz(kq))): the
// four 16-lane groups of a transposing read take blocks kq = 2 g (+1) of one
// nq, and the LDS serves groups 0, 1 (and 2, 3) in one pass; unswizzled their
// blocks are 4 KiB apart on the same 32 banks, swizzled they sit on the two
// halves of the 64 banks.
__device__ __forceinline__ int b_swz(int kq) { return (kq >> 1) & 1; }

// B stage: kSK k x kBN columns of an n-contiguous matrix, 4 x 16 blocks of
// 128 bytes (swizzled as above); load j of wave w fills block positions
// 8 (j * 8 + w) .. +7.
struct BLoaderP {
  static constexpr int kPer = kSK / 4 * kNQ / 8 / kWaves;
  i32x4 rsrc;
  uint32_t voff[kPer];
  uint32_t stage_bytes;
  template <typename ColOf>
  __device__ __forceinline__ void init(const uint16_t* W, int ldw, int K, ColOf col_of) {
    rsrc = buffer_rsrc(W, int64_t(K) * ldw * 2);
    stage_bytes = uint32_t(ldw) * 2u * kSK;
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int blk = 8 * (j * kWaves + w) + (lane >> 3);
      const int kq = blk / kNQ, nq = (blk % kNQ) ^ b_swz(kq);
      const int r = (lane & 7) >> 1, c = lane & 1;
      voff[j] = uint32_t(4 * kq + r) * uint32_t(ldw) * 2u + 2u * uint32_t(col_of(16 * nq + 8 * c));
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* Bs, int stage) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < kPer; ++j) dma16(rsrc, voff[j], uint32_t(stage) * stage_bytes, Bs + 1024 * (j * kWaves + w));
  }
  // A stage holding only k rows 0..31 (the end of K): loads j >= kPer / 2
  // (k rows 32..63, see init) read rows 0..31 again, so none reaches past the
  // matrix; those k values are multiplied as zeros.
  __device__ __forceinline__ void issue_half(MOE_LDS char* Bs, int stage) const {
    static_assert(kSK == 64 && kNQ == 16 && kPer == 4, "loads 0, 1 hold k rows 0..31");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      dma16(rsrc, voff[j % (kPer / 2)], uint32_t(stage) * stage_bytes, Bs + 1024 * (j * kWaves + w));
  }
};

// Per-lane LDS offsets of one wave's fragments in a stage.
// A: fragment i of wave row wm covers tile rows 16 (kWR i + wm) .. +15; lane l
//    reads row 16 (kWR i + wm) + (l & 15), chunk 4 q + (l >> 4) of k step q
//    (swizzled; the swizzle depends on row bits that fragment i does not
//    change), so one base per k step plus 16 kWR kRowBytes i.
// B: fragment j = columns 64 wn + 16 j; lane group g = l >> 4 takes k
//    32 q + 8g .. +7 from blocks (8 q + 2g, nq) and (8 q + 2g + 1, nq).
// B fragment j of group g is block column 4 wn + (j ^ b_swz(2 g)) (b_swz of
// 2 g and 2 g + 1 agree, and so do those of the k steps' 8 q + 2 g): even
// fragments at b_e + 128 j, odd ones at b_o + 128 j.
struct FragAddrP {
  uint32_t a[kSub];
  uint32_t b_e, b_o;
  __device__ __forceinline__ void init(int wm, int wn) {
    const int lane = lane_id();
    const int r = 16 * wm + (lane & 15);
#pragma unroll
    for (int q = 0; q < kSub; ++q) a[q] = uint32_t(r * kRowBytes + 16 * a_chunk_pos(r, 4 * q + (lane >> 4)));
    const uint32_t b = uint32_t((2 * (lane >> 4) * kNQ + 4 * wn) * 128 + 8 * (lane & 15));
    const uint32_t sw = uint32_t(128 * b_swz(2 * (lane >> 4)));
    b_e = b + sw;
    b_o = b - sw;
  }
};

template <int Q>
__device__ __forceinline__ u32x4 read_a(const MOE_LDS char* As, const FragAddrP& fa, int i) {
  return *reinterpret_cast<const MOE_LDS u32x4*>(As + fa.a[Q] + 16 * kWR * kRowBytes * i);
}
template <int Q>
__device__ __forceinline__ u32x4 read_b(const MOE_LDS char* Bs, const FragAddrP& fa, int j) {
  const MOE_LDS char* p0 = Bs + ((j & 1) ? fa.b_o : fa.b_e) + Q * 8 * kNQ * 128 + 128 * j;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4*)(p0 + kNQ * 128));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2.x, l2.y, h2.x, h2.y};
}

}  // namespace panel

}  // namespace dma
}  // namespace moe
