// The matrix-core issue bound of the Newton-Schulz product kernels, for measurement only
// (built as libmuon_mfma_loop.so, called by bench.py; not part of the library's ABI).
//
// mfma_loop runs a product kernel's grid and its per-wave MFMA count with nothing else: each
// of the 4 waves of a block issues `iters` K steps of 2 * NACC v_mfma_f32_32x32x16_bf16
// (two 16-deep slices into NACC accumulator blocks of 32x32: 16 for the 128x128 register
// tile of the apply and four-block kernels, 4 for the 64x64 one of the 128x128-tile kernel)
// on operands held in registers (random bf16 values, distinct for every fragment), with no
// memory traffic in the loop. Dynamic LDS of
// `lds_bytes` per block reproduces the product kernel's blocks per compute unit. The time
// of such a launch is what the product kernel would take if its matrix cores never waited
// for data, at the clock the device holds while they run; each block's first wave records
// its shader-clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) at
// the start and end of its loop, from which that clock follows.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A bf16 with a random sign and mantissa and an exponent within 2^-4 .. 2^3, from a hash of
// (thread, register, element): operands that toggle the multipliers as data does (the
// matrix cores' power, and so the clock the device holds, depends on it).
__device__ __forceinline__ __bf16 noise_bf16(uint32_t t, uint32_t reg, uint32_t e) {
  uint32_t h = t * 0x9E3779B1u ^ (reg * 0x85EBCA77u + e * 0xC2B2AE3Du);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t bits = (h & 0x807Fu) | ((123u + ((h >> 16) & 7u)) << 7);
  return __builtin_bit_cast(__bf16, (uint16_t)bits);
}

// Each K step: two 16-deep slices, each into the NACC accumulator blocks from its own
// operand fragments (SQ x SQ blocks from SQ left and SQ right fragments, as the product
// kernels' register tiles do).
template <int NACC>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* sink, uint64_t* stamps) {
  extern __shared__ char lds[];  // sized by the launch only: sets the blocks per CU
  constexpr int SQ = NACC == 16 ? 4 : 2;
  const int t = threadIdx.x;
  bf16x8 a[2][SQ], b[2][SQ];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < SQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[s][i][e] = noise_bf16(t, 2 * (SQ * s + i), e);
        b[s][i][e] = noise_bf16(t, 2 * (SQ * s + i) + 1, e);
      }
  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int k = 0; k < iters; ++k) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[s][i % SQ], a[s][i / SQ], acc[i], 0,
                                                          0, 0);
  }
  // the accumulators are read only after the loop: the last MFMAs have retired when the
  // end stamps are read
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[i][r];
  sink[(size_t)blockIdx.x * 256 + t] = sum;
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (t == 0) {
    uint64_t* s = stamps + 4 * (size_t)blockIdx.x;
    s[0] = c0;
    s[1] = c1;
    s[2] = r0;
    s[3] = r1;
  }
  (void)lds;
}

}  // namespace

// One launch of `blocks` x 256 threads, timed like the library's per-launch profiling:
// start and end events taken from the kernel's own dispatch (hipExtLaunchKernel), so that
// the time spans the kernel only. sink: blocks * 256 floats; stamps: blocks * 4 uint64
// (device). nacc: 16 or 4. Synchronises the stream, stores the kernel time in *us and
// returns 0, or -1 for invalid arguments, or the hipError_t of a failed HIP call.
extern "C" int muon_mfma_loop(int blocks, int nacc, int iters, int lds_bytes, float* sink,
                              uint64_t* stamps, hipStream_t stream, float* us) {
  if (blocks < 1 || iters < 1 || lds_bytes < 0 || lds_bytes > 160 * 1024 || !sink || !stamps ||
      !us || (nacc != 16 && nacc != 4))
    return -1;
  const void* fn = nacc == 16 ? reinterpret_cast<const void*>(&mfma_loop<16>)
                              : reinterpret_cast<const void*>(&mfma_loop<4>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return (int)e;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  if ((e = hipEventCreate(&t0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&t1)) != hipSuccess) {
    (void)hipEventDestroy(t0);
    return (int)e;
  }
  if (nacc == 16)
    hipExtLaunchKernelGGL(mfma_loop<16>, dim3(blocks), dim3(256), lds_bytes, stream, t0, t1, 0u,
                          iters, sink, stamps);
  else
    hipExtLaunchKernelGGL(mfma_loop<4>, dim3(blocks), dim3(256), lds_bytes, stream, t0, t1, 0u,
                          iters, sink, stamps);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipEventSynchronize(t1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
  *us = 1e3f * ms;
  (void)hipEventDestroy(t0);
  (void)hipEventDestroy(t1);
  return (int)e;
}
