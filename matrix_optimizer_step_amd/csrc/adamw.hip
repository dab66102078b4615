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
// One pass over every tensor: each thread takes 8 consecutive elements of one
// tensor (vector accesses when all 8 are in range, element accesses at the
// tail).  Roofline: HBM bandwidth; algorithmic bytes per element 22 for bf16
// parameters (read p, g: 2 + 2, m, v: 4 + 4; write p, m, v) and 28 for
// float32 parameters.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;   // elements per thread

template <typename T>
__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamwParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;            // elements per 16-byte chunk of p and g
  constexpr int NC = kPer / E;        // chunks of p (and g) per thread
  const VecTask task = P.tasks[blockIdx.x];
  const VecDesc& d = P.vecs[task.t];
  const int64_t e0 = task.start + (int64_t)threadIdx.x * kPer;
  if (e0 >= d.n) return;
  T* p = (T*)d.p;
  const T* g = (const T*)d.g;
  float pe[kPer], ge[kPer], me[kPer], ve[kPer];
  const int cnt = (int)(d.n - e0 < kPer ? d.n - e0 : kPer);
  if (cnt == kPer) {
    // base pointers are 16-byte aligned and e0 is a multiple of 8
    u32x4 pr[NC], gr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      pr[c] = gload<u32x4>(p + e0 + c * E);
      gr[c] = gload<u32x4>(g + e0 + c * E);
    }
    const f32x4 m0 = gload<f32x4>(d.m + e0), m1 = gload<f32x4>(d.m + e0 + 4);
    const f32x4 v0 = gload<f32x4>(d.v + e0), v1 = gload<f32x4>(d.v + e0 + 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      Tr::unpack(pr[c], pe + c * E);
      Tr::unpack(gr[c], ge + c * E);
    }
    me[0] = m0.x; me[1] = m0.y; me[2] = m0.z; me[3] = m0.w;
    me[4] = m1.x; me[5] = m1.y; me[6] = m1.z; me[7] = m1.w;
    ve[0] = v0.x; ve[1] = v0.y; ve[2] = v0.z; ve[3] = v0.w;
    ve[4] = v1.x; ve[5] = v1.y; ve[6] = v1.z; ve[7] = v1.w;
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      pe[i] = ge[i] = me[i] = ve[i] = 0.f;
      if (i < cnt) {
        pe[i] = Tr::load1(p, e0 + i);
        ge[i] = Tr::load1(g, e0 + i);
        me[i] = gload<float>(d.m + e0 + i);
        ve[i] = gload<float>(d.v + e0 + i);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const double gd = ge[i], pd = pe[i];
    const float ms = (float)fma(P.b1, (double)me[i], P.omb1 * gd);
    const float vs = (float)fma(P.b2, (double)ve[i], P.omb2 * gd * gd);
    const double denom = fma(sqrt((double)vs), P.inv_sqrt_bc2, P.eps);
    const double pn = fma(-P.wdl, pd, pd) - P.step_size * (double)ms / denom;
    me[i] = ms;
    ve[i] = vs;
    pe[i] = Tr::round_store(pn);
  }
  if (cnt == kPer) {
#pragma unroll
    for (int c = 0; c < NC; ++c) gstore<u32x4>(p + e0 + c * E, Tr::pack(pe + c * E));
    gstore<f32x4>(d.m + e0, f32x4{me[0], me[1], me[2], me[3]});
    gstore<f32x4>(d.m + e0 + 4, f32x4{me[4], me[5], me[6], me[7]});
    gstore<f32x4>(d.v + e0, f32x4{ve[0], ve[1], ve[2], ve[3]});
    gstore<f32x4>(d.v + e0 + 4, f32x4{ve[4], ve[5], ve[6], ve[7]});
  } else {
    for (int i = 0; i < cnt; ++i) {
      Tr::store1(p, e0 + i, pe[i]);
      gstore<float>(d.m + e0 + i, me[i]);
      gstore<float>(d.v + e0 + i, ve[i]);
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
