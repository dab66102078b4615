// RMNP comparator step, one fused memory-bound pass per row (blog post,
// section 1: each row of the momentum divided by its L2 norm; appendix
// rmnp_local: momentum in place, float32 row sums, update scaled by
// sqrt(max(1, rows/cols))):
//
//   V_i <- mu*V_i + G_i            (one rounding to storage, stored once)
//   n_i  = ||V_i||_2               (float32 sum of squares of the stored V_i)
//   W_i <- W_i - lr*s * V_i / max(n_i, eps)   (one rounding)
//
// Register-resident variants keep the updated row in VGPRs between the norm
// and the update, so each element moves 10 bytes (bf16: read G, V, W; write V,
// W) -- the algorithmic minimum.  A row belongs to one wave (WPR = 1, four rows
// per workgroup) or to a whole workgroup (WPR = 4); each lane holds NCH
// 16-byte chunks.  The streaming variant (any width, scalar accesses) makes two
// passes and recomputes the momentum in the second one; it serves rows wider
// than the register capacity or widths that are not a multiple of the vector.
//
// Roofline: HBM bandwidth; algorithmic bytes per element 10 (bf16) / 20 (fp32).
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int kThreads = 256;

template <typename T, int WPR, int NCH>
__global__ __launch_bounds__(kThreads) void rmnp_kernel(RmnpParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;
  constexpr int LPR = 64 * WPR;   // lanes per row
  __shared__ float red[4];

  const RmnpTask task = P.tasks[blockIdx.x];
  const MatDesc& d = P.mats[task.mat];
  const int wave = threadIdx.x >> 6;
  const int64_t row = task.row0 + (WPR == 1 ? wave : 0);
  const int lr_idx = (WPR == 1 ? (threadIdx.x & 63) : threadIdx.x);
  const bool active = row < d.rows;
  const int64_t cols = d.cols;
  const int64_t nchunks = cols / E;

  T* vrow = (T*)d.v + row * cols;
  const T* grow = (const T*)d.g + row * cols;
  T* wrow = (T*)d.w + row * cols;

  // All loads of the row first (V, G and W are distinct buffers, but the
  // compiler cannot know that, so a load written after the V store would wait
  // for it), then the momentum, its sum of squares and the V stores.
  //
  // float32 rows load without a branch: a lane whose chunk lies past the
  // row's end loads the row's first chunk (a valid address) and never uses
  // it.  Behind a branch per chunk the compiler copies the float32 register
  // arrays around (eight chunks per lane took ~500 registers); the bfloat16
  // variants keep the branch, which costs them fewer registers than the
  // unconditional float64 momentum of the unused chunks would.
  constexpr bool CLAMP = sizeof(T) == 4;
  u32x4 vreg[NCH], greg[NCH], wreg[NCH];
  float ss = 0.f;
  if (active) {
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int64_t ch = lr_idx + (int64_t)LPR * p;
      if (CLAMP) {
        const int64_t cl = ch < nchunks ? ch : 0;
        vreg[p] = gload_nt<u32x4>(vrow + cl * E);
        greg[p] = gload_nt<u32x4>(grow + cl * E);
        wreg[p] = gload_nt<u32x4>(wrow + cl * E);
      } else if (ch < nchunks) {
        vreg[p] = gload_nt<u32x4>(vrow + ch * E);
        greg[p] = gload_nt<u32x4>(grow + ch * E);
        wreg[p] = gload_nt<u32x4>(wrow + ch * E);
      }
    }
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int64_t ch = lr_idx + (int64_t)LPR * p;
      if (ch < nchunks) {
        float fv[E], fg[E], vn[E];
        Tr::unpack(vreg[p], fv);
        Tr::unpack(greg[p], fg);
        Tr::template fma_store_n<E>(P.mu, fv, fg, vn);
#pragma unroll
        for (int e = 0; e < E; ++e) ss = fmaf(vn[e], vn[e], ss);
        vreg[p] = Tr::pack(vn);
        gstore_nt<u32x4>(vrow + ch * E, vreg[p]);
      }
    }
  }
  float tot = wave_sum(ss);
  if (WPR > 1) {
    if ((threadIdx.x & 63) == 0) red[wave] = tot;
    __syncthreads();
    tot = (red[0] + red[1]) + (red[2] + red[3]);
  }
  if (!active) return;
  const float inv = 1.f / fmaxf(sqrtf(tot), P.eps);
  const float step = -P.lr * d.upd_scale * inv;
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int64_t ch = lr_idx + (int64_t)LPR * p;
    if (ch < nchunks) {
      float fv[E], fw[E], wn[E];
      Tr::unpack(vreg[p], fv);
      Tr::unpack(wreg[p], fw);
      Tr::template fma_store_n<E>(step, fv, fw, wn);
      gstore_nt<u32x4>(wrow + ch * E, Tr::pack(wn));
    }
  }
}

// Streaming two-pass variant: one row per workgroup, scalar accesses.
template <typename T>
__global__ __launch_bounds__(kThreads) void rmnp_stream_kernel(RmnpParams P) {
  using Tr = Elem<T>;
  __shared__ float red[4];
  const RmnpTask task = P.tasks[blockIdx.x];
  const MatDesc& d = P.mats[task.mat];
  const int64_t row = task.row0;
  const int64_t cols = d.cols;
  T* vrow = (T*)d.v + row * cols;
  const T* grow = (const T*)d.g + row * cols;
  T* wrow = (T*)d.w + row * cols;
  float ss = 0.f;
  for (int64_t c = threadIdx.x; c < cols; c += kThreads) {
    const float v = Tr::fma_store(P.mu, Tr::load1(vrow, c), Tr::load1(grow, c));
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / fmaxf(sqrtf(tot), P.eps);
  const float step = -P.lr * d.upd_scale * inv;
  for (int64_t c = threadIdx.x; c < cols; c += kThreads) {
    const float v = Tr::fma_store(P.mu, Tr::load1(vrow, c), Tr::load1(grow, c));
    Tr::store1(vrow, c, v);
    Tr::store1(wrow, c, Tr::fma_store(step, v, Tr::load1(wrow, c)));
  }
}

// Column-cut RMNP, the two local halves on a column slice of each matrix (blog
// post, section 3, the column-cut layout; appendix rmnp_colcut).  One wave per
// row, four rows per workgroup, any width.  d.partials points at the matrix's
// first entry of the [sum of rows] row-sum vector; d.upd_scale uses the whole
// matrix's shape.
//   partial: V <- mu*V + G (one rounding, stored); rowsq[r] = sum of the stored
//            V[r, :]^2 over this slice in float32 -- per lane over its chunks in
//            order, then a fixed wave tree (deterministic, batch independent).
//   apply:   W <- W - lr*s * V / max(sqrt(rowsq[r]), eps)   (one rounding),
//            after the row sums were summed over all slices.
// Each lane handles chunks lane, lane + 64, ...; eight chunks' loads are issued
// before their stores.  Algorithmic bytes per element (bf16): partial 6 (read
// G, V; write V), apply 6 (read V, W; write W).
constexpr int kColcutUnroll = 8;

template <typename T>
__global__ __launch_bounds__(kThreads) void colcut_partial_kernel(ColcutParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;
  const RmnpTask task = P.tasks[blockIdx.x];
  const MatDesc& d = P.mats[task.mat];
  const int64_t row = task.row0 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= d.rows) return;
  const int64_t cols = d.cols;
  T* vrow = (T*)d.v + row * cols;
  const T* grow = (const T*)d.g + row * cols;
  float ss = 0.f;
  if (d.vec_ok) {
    const int64_t nch = cols / E;
    for (int64_t base = lane; base < nch; base += 64 * kColcutUnroll) {
      u32x4 vv[kColcutUnroll], gg[kColcutUnroll];
#pragma unroll
      for (int u = 0; u < kColcutUnroll; ++u) {
        const int64_t ch = base + 64 * u;
        if (ch < nch) {
          vv[u] = gload_nt<u32x4>(vrow + ch * E);
          gg[u] = gload_nt<u32x4>(grow + ch * E);
        }
      }
#pragma unroll
      for (int u = 0; u < kColcutUnroll; ++u) {
        const int64_t ch = base + 64 * u;
        if (ch < nch) {
          float fv[E], fg[E], vn[E];
          Tr::unpack(vv[u], fv);
          Tr::unpack(gg[u], fg);
          Tr::template fma_store_n<E>(P.mu, fv, fg, vn);
#pragma unroll
          for (int e = 0; e < E; ++e) ss = fmaf(vn[e], vn[e], ss);
          gstore_nt<u32x4>(vrow + ch * E, Tr::pack(vn));
        }
      }
    }
  } else {
    for (int64_t c = lane; c < cols; c += 64) {
      const float v = Tr::fma_store(P.mu, Tr::load1(vrow, c), Tr::load1(grow, c));
      Tr::store1(vrow, c, v);
      ss = fmaf(v, v, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) gstore<float>(d.partials + row, ss);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void colcut_apply_kernel(ColcutParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;
  const RmnpTask task = P.tasks[blockIdx.x];
  const MatDesc& d = P.mats[task.mat];
  const int64_t row = task.row0 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= d.rows) return;
  const int64_t cols = d.cols;
  const T* vrow = (const T*)d.v + row * cols;
  T* wrow = (T*)d.w + row * cols;
  const float inv = 1.f / fmaxf(sqrtf(gload<float>(d.partials + row)), P.eps);
  const float step = -P.lr * d.upd_scale * inv;
  if (d.vec_ok) {
    const int64_t nch = cols / E;
    for (int64_t base = lane; base < nch; base += 64 * kColcutUnroll) {
      u32x4 vv[kColcutUnroll], ww[kColcutUnroll];
#pragma unroll
      for (int u = 0; u < kColcutUnroll; ++u) {
        const int64_t ch = base + 64 * u;
        if (ch < nch) {
          vv[u] = gload_nt<u32x4>(vrow + ch * E);
          ww[u] = gload_nt<u32x4>(wrow + ch * E);
        }
      }
#pragma unroll
      for (int u = 0; u < kColcutUnroll; ++u) {
        const int64_t ch = base + 64 * u;
        if (ch < nch) {
          float fv[E], fw[E], wn[E];
          Tr::unpack(vv[u], fv);
          Tr::unpack(ww[u], fw);
          Tr::template fma_store_n<E>(step, fv, fw, wn);
          gstore_nt<u32x4>(wrow + ch * E, Tr::pack(wn));
        }
      }
    }
  } else {
    for (int64_t c = lane; c < cols; c += 64)
      Tr::store1(wrow, c, Tr::fma_store(step, Tr::load1(vrow, c), Tr::load1(wrow, c)));
  }
}

template <typename T>
hipError_t launch_t(int wpr, int nch, const RmnpParams& p, int n, hipStream_t s) {
  dim3 g(n), b(kThreads);
#define MATOPT_RMNP_CASE(W, N)                                                   \
  if (wpr == W && nch == N) {                                                    \
    hipLaunchKernelGGL((rmnp_kernel<T, W, N>), g, b, 0, s, p);                   \
    return hipGetLastError();                                                    \
  }
  MATOPT_RMNP_CASE(1, 1)
  MATOPT_RMNP_CASE(1, 2)
  MATOPT_RMNP_CASE(1, 4)
  MATOPT_RMNP_CASE(1, 8)
  MATOPT_RMNP_CASE(4, 4)
  MATOPT_RMNP_CASE(4, 8)
  MATOPT_RMNP_CASE(4, 16)
#undef MATOPT_RMNP_CASE
  if (nch == 0) {
    hipLaunchKernelGGL(rmnp_stream_kernel<T>, g, b, 0, s, p);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rmnp(int dt, int wpr, int nch, const RmnpParams& p, int n_tasks,
                       hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  return dt == DT_BF16 ? launch_t<uint16_t>(wpr, nch, p, n_tasks, s)
                       : launch_t<float>(wpr, nch, p, n_tasks, s);
}

hipError_t launch_colcut(int dt, bool apply, const ColcutParams& p, int n_tasks, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  dim3 g(n_tasks), b(kThreads);
  if (dt == DT_BF16) {
    if (apply) hipLaunchKernelGGL(colcut_apply_kernel<uint16_t>, g, b, 0, s, p);
    else hipLaunchKernelGGL(colcut_partial_kernel<uint16_t>, g, b, 0, s, p);
  } else {
    if (apply) hipLaunchKernelGGL(colcut_apply_kernel<float>, g, b, 0, s, p);
    else hipLaunchKernelGGL(colcut_partial_kernel<float>, g, b, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace matopt
