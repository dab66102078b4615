// MFMA rate probe: a measurement aid, not part of the optimizer step.
//
// Each wave runs `iters` steps of bf16 MFMAs on 12 operand fragments (16 bytes
// per lane each): either 16 v_mfma_f32_32x32x16_bf16 on 4 x 2 accumulator
// blocks (the layout of a 128 x 64 wave sub-tile, two k16 halves per step) or
// 32 v_mfma_f32_16x16x32_bf16 on 8 x 4 slabs (the same sub-tile, one K step of
// 32) -- the same 524288 flops per wave and step either way.  The fragments
// either stay in registers (loaded once from `src`) or are read fresh from LDS
// one step ahead of their MFMAs, as the GEMM engine reads them (contiguous
// 16-byte lanes, rotating over five 32 KB stages).  Eight waves per workgroup
// and 160 KB of LDS keep one workgroup per compute unit, two waves per SIMD.
// There is no DMA and no epilogue, so the rate this reaches bounds what an
// MFMA schedule with these operand reads can reach on the same data.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeLds = 160 * 1024;
constexpr int kProbeFrags = 12;

// Fragments of step `it` from LDS: fragment f of this lane at stage it % 5.
__device__ __forceinline__ void probe_read(const uint8_t* lds, int it, int wave, int lane,
                                           bf16x8 (&f)[kProbeFrags]) {
  const int st = (it % 5) * 32768 + wave * 4096 + lane * 16;
#pragma unroll
  for (int i = 0; i < kProbeFrags; ++i)
    f[i] = *(const bf16x8*)(lds + (st + i * 1024 + (i >= 8 ? 8192 : 0)) % kProbeLds);
}

template <bool F16>
struct ProbeAcc;

template <>
struct ProbeAcc<false> {
  f32x16 acc[4][2];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
  // two k16 halves: P fragments 4h .. 4h+3, Q fragments 8 + 2h, 9 + 2h
  __device__ __forceinline__ void step(const bf16x8 (&f)[kProbeFrags]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[8 + 2 * h + j], f[4 * h + i],
                                                              acc[i][j], 0, 0, 0);
  }
  __device__ float sum() const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    return s;
  }
};

template <>
struct ProbeAcc<true> {
  f32x4 acc[8][4];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // P slabs: fragments 0 .. 7, Q slabs: 8 .. 11
  __device__ __forceinline__ void step(const bf16x8 (&f)[kProbeFrags]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[8 + j], f[i], acc[i][j], 0, 0, 0);
  }
  __device__ float sum() const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    return s;
  }
};

// src: 512 threads x 12 fragments x 8 bf16 (98304 bytes); out: one float per
// thread; clk[0], clk[1]: shader-clock and 100 MHz real-time ticks, summed
// over workgroups.  iters is even.
template <bool F16, bool LDS>
__global__ __launch_bounds__(512) void mfma_probe_kernel(const uint16_t* __restrict__ src,
                                                         float* __restrict__ out, int iters,
                                                         unsigned long long* clk) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kProbeLds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bf16x8* s = (const bf16x8*)src;
  bf16x8 fa[kProbeFrags], fb[kProbeFrags];
  if (LDS) {
    for (int o = threadIdx.x * 16; o < kProbeLds; o += 512 * 16)
      *(bf16x8*)(lds + o) = s[(o / 16) % (512 * kProbeFrags)];
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < kProbeFrags; ++i) {
      fa[i] = s[threadIdx.x * kProbeFrags + i];
      fb[i] = s[((threadIdx.x + 256) & 511) * kProbeFrags + i];
    }
  }
  ProbeAcc<F16> a;
  a.zero();
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  if (LDS) probe_read(lds, 0, wave, lane, fa);
  for (int it = 0; it < iters; it += 2) {
    if (LDS) probe_read(lds, it + 1, wave, lane, fb);
    __builtin_amdgcn_sched_barrier(0);
    a.step(fa);
    __builtin_amdgcn_sched_barrier(0);
    if (LDS) probe_read(lds, it + 2, wave, lane, fa);
    __builtin_amdgcn_sched_barrier(0);
    a.step(fb);
    __builtin_amdgcn_sched_barrier(0);
  }
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = a.sum();
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    atomicAdd(&clk[0], (unsigned long long)(t1 - t0));
    atomicAdd(&clk[1], (unsigned long long)(r1 - r0));
  }
}

}  // namespace

hipError_t launch_mfma_probe(bool f16, bool from_lds, const void* src, float* out, int iters,
                             int workgroups, unsigned long long* clk, hipStream_t s) {
  const dim3 grid(workgroups), block(512);
  const uint16_t* in = (const uint16_t*)src;
  if (f16 && from_lds)
    hipLaunchKernelGGL((mfma_probe_kernel<true, true>), grid, block, 0, s, in, out, iters, clk);
  else if (f16)
    hipLaunchKernelGGL((mfma_probe_kernel<true, false>), grid, block, 0, s, in, out, iters, clk);
  else if (from_lds)
    hipLaunchKernelGGL((mfma_probe_kernel<false, true>), grid, block, 0, s, in, out, iters, clk);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<false, false>), grid, block, 0, s, in, out, iters, clk);
  return hipGetLastError();
}

}  // namespace matopt
