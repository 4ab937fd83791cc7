// Calibration kernels (include/moe_calib.h): a buffer of known size read once
// with the 16-byte direct-to-LDS loads the GEMM operand stages use, and a
// register-only matrix-core loop for the attainable bf16 rate.
#include "moe_calib.h"

#include "../csrc/gemm_dma.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kSlots = 4;        // LDS slots of 1 KiB per wave, reused round robin
constexpr int kInFlight = 16;    // loads a wave keeps outstanding at most

// Wait until at most N loads of this wave are outstanding (no barrier).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

// Chunk c (1 KiB) is read by wave c % (grid waves): lane l fetches bytes
// 16 l .. 16 l + 15 of it. What lands in LDS is never read.
__global__ void __launch_bounds__(kThreads) dma_read_kernel(const char* src, int chunks) {
  __shared__ __attribute__((aligned(1024))) char buf[kWaves * kSlots * 1024];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));  // wave-uniform
  const moe::dma::i32x4 rsrc = moe::dma::buffer_rsrc(src, int64_t(chunks) * 1024);
  const uint32_t voff = 16u * uint32_t(moe::lane_id());
  const int stride = int(gridDim.x) * kWaves;
  int n = 0;
  for (int c = int(blockIdx.x) * kWaves + w; c < chunks; c += stride, ++n) {
    if (n >= kInFlight) wait_vm<kInFlight - 1>();
    moe::dma::dma16(rsrc, voff, uint32_t(c) * 1024u,
                    (MOE_LDS char*)buf + (w * kSlots + (n % kSlots)) * 1024);
  }
  // no load may still be writing LDS when the workgroup ends
  wait_vm<0>();
}

// 8 independent accumulator chains per wave; the operands depend on the
// lane so they are not constants.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* sink) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const uint32_t l = moe::lane_id();
  const moe::u32x4 a = {0x3F803F80u ^ l, 0x3F003F00u, 0x3F803F80u, 0x3E803E80u ^ l};
  const moe::u32x4 b = {0x3F003F00u, 0x3F803F80u ^ l, 0x3E803E80u, 0x3F803F80u};
  f32x4v acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, float(c)};
  // Written as assembly with the accumulators in VGPRs, so the compiler
  // does not shuttle them between register files inside the loop. A chain's
  // next MFMA comes 7 MFMAs (112 cycles) after its last, well past the
  // result latency; the nops cover the VALU writes before the loop and the
  // VALU reads after it.
  moe::u32x4 ra = a, rb = b;
  // the operands are all in place before the nops (they are asm operands)
  asm volatile("s_nop 7"
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
                 "+v"(acc[7]), "+v"(ra), "+v"(rb));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(ra), "v"(rb));
  }
  // and read only after these
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
                 "+v"(acc[7]));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1.25e-37f) sink[0] = s;  // never true for these operands
}

}  // namespace

extern "C" int moe_calib_mfma_loop(int iters, int waves_per_simd, float* sink, double* flop, hipStream_t stream) {
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8 || !sink || !flop) return -1;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -4;
  // 4-wave workgroups: one wave per SIMD each
  const int grid = cus * waves_per_simd;
  *flop = double(grid) * 4.0 * double(iters) * 8.0 * 16384.0;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int moe_calib_dma_read(const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return 0;
  if (!src || (reinterpret_cast<uintptr_t>(src) & 15) || bytes % 1024 || bytes > (size_t(1) << 30)) return -1;
  const int chunks = int(bytes / 1024);
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -4;
  const int grid = int(std::min<int64_t>(int64_t(cus) * 4, (chunks + kWaves - 1) / kWaves));
  hipLaunchKernelGGL(dma_read_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<const char*>(src), chunks);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
