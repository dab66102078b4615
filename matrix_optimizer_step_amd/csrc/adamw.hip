// Fused AdamW step over a ragged batch of flat tensors: the non-2D tail of an
// owner's parameters (LayerNorm weights and biases), which MatrixFSDP section
// 5.1 puts on AdamW (lr 1e-3, weight decay 1e-2, betas (0.9, 0.999), eps 1e-8,
// no schedule).  The pages name the optimizer without writing its update; this
// is the standard decoupled form:
//
//   m <- beta1 m + (1 - beta1) g                 float64, stored as float32
//   v <- beta2 v + (1 - beta2) g^2               float64, stored as float32
//   p <- p - lr wd p - step_size m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
//                                                float64, one rounding to p's dtype
//
// with step_size = lr / (1 - beta1^t) and the stored m, v in the last line.
// One pass over every tensor: a block of 256 threads takes 2048 consecutive
// elements of one tensor, thread t the runs start + 4t + (0..3) and start +
// 1024 + 4t + (0..3), so that every load and store instruction of a wave
// covers one contiguous span (512 bytes of bf16, 1 KB of float32) and the
// streaming (non-temporal) accesses move whole lines; element accesses at a
// tail.  Roofline: HBM bandwidth; algorithmic bytes per element 22 for bf16
// parameters (read p, g: 2 + 2, m, v: 4 + 4; write p, m, v) and 28 for
// float32 parameters.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int kThreads = 256;
constexpr int kRun = 4;                  // consecutive elements per run
constexpr int kRuns = 2;                 // runs per thread, kThreads * kRun apart
static_assert(kThreads * kRun * kRuns == kAdamwTask, "task size");

// kRun consecutive elements of a parameter or gradient as float
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&f)[kRun]) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 v = gload_nt<u32x2>(p);
    f[0] = lo_bf(v.x); f[1] = hi_bf(v.x); f[2] = lo_bf(v.y); f[3] = hi_bf(v.y);
  } else {
    const f32x4 v = gload_nt<f32x4>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&f)[kRun]) {
  if constexpr (sizeof(T) == 2)
    gstore_nt<u32x2>(p, u32x2{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3])});
  else
    gstore_nt<f32x4>(p, f32x4{f[0], f[1], f[2], f[3]});
}

template <typename T>
__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamwParams P) {
  using Tr = Elem<T>;
  const VecTask task = P.tasks[blockIdx.x];
  const VecDesc& d = P.vecs[task.t];
  T* p = (T*)d.p;
  const T* g = (const T*)d.g;
  float pe[kRuns][kRun], ge[kRuns][kRun], me[kRuns][kRun], ve[kRuns][kRun];
  int64_t e0[kRuns];
  int cnt[kRuns];
#pragma unroll
  for (int h = 0; h < kRuns; ++h) {
    e0[h] = task.start + (int64_t)kThreads * kRun * h + (int64_t)threadIdx.x * kRun;
    const int64_t left = d.n - e0[h];
    cnt[h] = left <= 0 ? 0 : left < kRun ? (int)left : kRun;
  }
  // all loads first (p, g, m and v are distinct buffers; the compiler cannot
  // know it, and a load written after a store would wait for it)
#pragma unroll
  for (int h = 0; h < kRuns; ++h) {
    if (cnt[h] == kRun) {   // e0 is a multiple of 4: aligned vector accesses
      load4<T>(p + e0[h], pe[h]);
      load4<T>(g + e0[h], ge[h]);
      const f32x4 m = gload_nt<f32x4>(d.m + e0[h]), v = gload_nt<f32x4>(d.v + e0[h]);
      me[h][0] = m.x; me[h][1] = m.y; me[h][2] = m.z; me[h][3] = m.w;
      ve[h][0] = v.x; ve[h][1] = v.y; ve[h][2] = v.z; ve[h][3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < kRun; ++i) {
        pe[h][i] = ge[h][i] = me[h][i] = ve[h][i] = 0.f;
        if (i < cnt[h]) {
          pe[h][i] = Tr::load1(p, e0[h] + i);
          ge[h][i] = Tr::load1(g, e0[h] + i);
          me[h][i] = gload<float>(d.m + e0[h] + i);
          ve[h][i] = gload<float>(d.v + e0[h] + i);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kRuns; ++h)
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const double gd = ge[h][i], pd = pe[h][i];
      const float ms = (float)fma(P.b1, (double)me[h][i], P.omb1 * gd);
      const float vs = (float)fma(P.b2, (double)ve[h][i], P.omb2 * gd * gd);
      const double denom = fma(sqrt((double)vs), P.inv_sqrt_bc2, P.eps);
      const double pn = fma(-P.wdl, pd, pd) - P.step_size * (double)ms / denom;
      me[h][i] = ms;
      ve[h][i] = vs;
      pe[h][i] = Tr::round_store(pn);
    }
#pragma unroll
  for (int h = 0; h < kRuns; ++h) {
    if (cnt[h] == kRun) {
      store4<T>(p + e0[h], pe[h]);
      gstore_nt<f32x4>(d.m + e0[h], f32x4{me[h][0], me[h][1], me[h][2], me[h][3]});
      gstore_nt<f32x4>(d.v + e0[h], f32x4{ve[h][0], ve[h][1], ve[h][2], ve[h][3]});
    } else {
      for (int i = 0; i < cnt[h]; ++i) {
        Tr::store1(p, e0[h] + i, pe[h][i]);
        gstore<float>(d.m + e0[h] + i, me[h][i]);
        gstore<float>(d.v + e0[h] + i, ve[h][i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_adamw(int dt, const AdamwParams& p, int n_tasks, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(adamw_kernel<uint16_t>, dim3(n_tasks), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, dim3(n_tasks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
