// Memory-bound kernels that open and (for ns_steps == 0) close the Muon step.
//
// prep_kernel      one tile of 4096 elements: for a float32 matrix that is
//                  transposed, a 64x64 tile of the padded original-orientation
//                  matrix; otherwise (X0 has V's layout) a contiguous run of the
//                  padded X0, so that every access streams whole rows.
// prep_t_kernel    the same for a bf16 matrix that is transposed, on 64 x 128
//                  tiles (its own launch, after prep_kernel's).
//                  Momentum V <- mu*V + G (blog post, section 1: heavy ball; one
//                  rounding to storage: see Elem::fma_store), partial sum of squares of the stored V
//                  (the Frobenius norm that opens the appendix's Newton-Schulz
//                  routine), and the first iterate X0 written into the workspace
//                  in X orientation (transposed through LDS when rows > cols,
//                  the routine's transpose), zero in the padding.  X0 is the
//                  stored V itself: the scale 1/(||V||+eps) is applied in float32
//                  inside the first iteration's products, not rounded into X0.
//                  When V already has X0's layout (bf16, not transposed, sides
//                  multiples of the GEMM tile) X0 is not written at all: the
//                  first iteration reads V (the descriptor's x0in).
//                  Algorithmic HBM bytes per element: bf16 read G,V + write V,X0
//                  = 8 (fp32: 16).
// finalize_kernel  xs = 1/(sqrt(sum partials) + eps), one block per matrix, fixed
//                  summation order (deterministic, batch independent).
// scale_out_kernel ns_steps == 0: O = xs*V, written as O or applied to W.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum4(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrepParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;              // elements per 16-byte chunk
  constexpr int CPR = kPrepTile / E;    // chunks per tile row
  constexpr int NCH = kPrepTile * kPrepTile / (kThreads * E);  // chunks per thread
  __shared__ float tileT[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];

  const PrepTile tile = P.tiles[blockIdx.x];
  const MatDesc& d = P.mats[tile.mat];
  const int64_t rows = d.rows, cols = d.cols;
  const int r_base = tile.tr * kPrepTile, c_base = tile.tc * kPrepTile;
  const bool vec = d.vec_ok != 0;
  const bool transposed = d.transposed != 0;
  const int64_t ldx = d.np;
  T* __restrict__ x0 = (T*)d.x[0];

  // All loads of the tile first, then the arithmetic and the stores: V, G and
  // the outputs are distinct buffers, but the compiler cannot know that, so
  // loads written after a store would wait for it.
  // Element (r, c) of each chunk.  Untransposed: the tile index counts runs of
  // kThreads * NCH chunks of the padded mp x np X0 (the same count as 64x64
  // tiles: both cover 4096 elements); np is a multiple of E, so no chunk
  // straddles a row.
  bool inb[NCH];
  int64_t offs[NCH], er[NCH], ec[NCH];
  u32x4 vraw[NCH], graw[NCH];
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int q = threadIdx.x + kThreads * p;
    int64_t r = r_base + q / CPR, c = c_base + (q % CPR) * E;
    if (!transposed) {
      const int64_t x = ((int64_t)tile.idx * (kThreads * NCH) + q) * E;
      r = x / ldx;
      c = x - r * ldx;
    }
    er[p] = r;
    ec[p] = c;
    inb[p] = r < rows && c < cols;
    offs[p] = r * cols + c;
    if (inb[p] && vec) {
      vraw[p] = gload_nt<u32x4>((const T*)d.v + offs[p]);
      if (P.momentum) graw[p] = gload_nt<u32x4>((const T*)d.g + offs[p]);
    }
  }

  float vals[NCH][E];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int64_t r = er[p], c = ec[p];
    const int64_t off = offs[p];
    float vn[E];
    if (inb[p]) {
      if (vec) {
        float vv[E];
        Tr::unpack(vraw[p], vv);
        if (P.momentum) {
          float gg[E];
          Tr::unpack(graw[p], gg);
#pragma unroll
          for (int e = 0; e < E; ++e) vn[e] = Tr::fma_store(P.mu, vv[e], gg[e]);
          gstore_nt<u32x4>((T*)d.v + off, Tr::pack(vn));
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) vn[e] = vv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          vn[e] = 0.f;
          if (c + e < cols) {
            float vv = Tr::load1(d.v, off + e);
            if (P.momentum) {
              vv = Tr::fma_store(P.mu, vv, Tr::load1(d.g, off + e));
              Tr::store1(d.v, off + e, vv);
            }
            vn[e] = vv;
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) vn[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ss = fmaf(vn[e], vn[e], ss);
      vals[p][e] = vn[e];
    }
    if (!transposed && !d.x0_is_v) {
      gstore<u32x4>(x0 + r * ldx + c, Tr::pack(vn));
    }
  }

  if (transposed) {
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int q = threadIdx.x + kThreads * p;
      const int rr = q / CPR, cc = (q % CPR) * E;
#pragma unroll
      for (int e = 0; e < E; ++e) tileT[rr][cc + e] = vals[p][e];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int q = threadIdx.x + kThreads * p;
      const int xr = q / CPR;        // original column within the tile
      const int xc = (q % CPR) * E;  // original row offset within the tile
      float t[E];
#pragma unroll
      for (int e = 0; e < E; ++e) t[e] = tileT[xc + e][xr];
      gstore<u32x4>(x0 + (int64_t)(c_base + xr) * ldx + r_base + xc, Tr::pack(t));
    }
  }

  const float tot = block_sum4(ss, red);
  if (threadIdx.x == 0) gstore<float>(d.partials + tile.idx, tot);
}

// Transposed bf16 matrices: a tile is 64 original rows x kPrepTileT (128)
// original columns, 256-byte runs of every row it reads and writes (against
// 128 with 64 x 64 tiles: 4-11% faster on the tall shapes of the Llama-3-8B
// and 32B-class sets), staged as bfloat16 in LDS (the stored V is a bfloat16
// value) and written out as 128 X0 rows of 64 elements.  Its own launch keeps
// the 17 KB of LDS off the other tiles.
constexpr int kPrepTC = kPrepTileT;
__global__ __launch_bounds__(kThreads) void prep_t_kernel(PrepParams P) {
  using Tr = Elem<uint16_t>;
  constexpr int E = 8;
  constexpr int CPR = kPrepTC / E;                             // chunks per tile row: 16
  constexpr int NCH = kPrepTile * kPrepTC / (kThreads * E);    // 4
  constexpr int PITCH = kPrepTC + 8;                           // bf16 elements per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t lt[kPrepTile * PITCH];
  __shared__ float red[4];
  const PrepTile tile = P.tiles[blockIdx.x];
  const MatDesc& d = P.mats[tile.mat];
  const int64_t rows = d.rows, cols = d.cols;
  const int64_t r_base = (int64_t)tile.tr * kPrepTile, c_base = (int64_t)tile.tc * kPrepTC;
  const int64_t ldx = d.np;
  uint16_t* __restrict__ x0 = (uint16_t*)d.x[0];
  bool inb[NCH];
  int64_t offs[NCH];
  u32x4 vraw[NCH], graw[NCH];
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int q = threadIdx.x + kThreads * p;
    const int64_t r = r_base + q / CPR, c = c_base + (q % CPR) * E;
    inb[p] = r < rows && c < cols;
    offs[p] = r * cols + c;
    if (inb[p] && d.vec_ok) {
      vraw[p] = gload_nt<u32x4>((const uint16_t*)d.v + offs[p]);
      if (P.momentum) graw[p] = gload_nt<u32x4>((const uint16_t*)d.g + offs[p]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int q = threadIdx.x + kThreads * p;
    const int64_t c = c_base + (q % CPR) * E;
    float vn[E];
    if (inb[p]) {
      if (d.vec_ok) {
        float vv[E];
        Tr::unpack(vraw[p], vv);
        if (P.momentum) {
          float gg[E];
          Tr::unpack(graw[p], gg);
#pragma unroll
          for (int e = 0; e < E; ++e) vn[e] = Tr::fma_store(P.mu, vv[e], gg[e]);
          gstore_nt<u32x4>((uint16_t*)d.v + offs[p], Tr::pack(vn));
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) vn[e] = vv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          vn[e] = 0.f;
          if (c + e < cols) {
            float vv = Tr::load1(d.v, offs[p] + e);
            if (P.momentum) {
              vv = Tr::fma_store(P.mu, vv, Tr::load1(d.g, offs[p] + e));
              Tr::store1(d.v, offs[p] + e, vv);
            }
            vn[e] = vv;
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) vn[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) ss = fmaf(vn[e], vn[e], ss);
    *(u32x4*)(lt + (q / CPR) * PITCH + (q % CPR) * E) = Tr::pack(vn);
  }
  __syncthreads();
  // X0 row c_base + j (original column j of the tile), elements r_base + 8k .. +7
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int q = threadIdx.x + kThreads * p;
    const int j = q >> 3, k = q & 7;
    uint32_t h[E];
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = lt[(8 * k + e) * PITCH + j];
    gstore<u32x4>(x0 + (c_base + j) * ldx + r_base + 8 * k,
                  u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16)});
  }
  const float tot = block_sum4(ss, red);
  if (threadIdx.x == 0) gstore<float>(d.partials + tile.idx, tot);
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeParams P) {
  __shared__ double red[4];
  const MatDesc& d = P.mats[blockIdx.x];
  double s = 0.0;
  for (int i = threadIdx.x; i < d.n_prep; i += kThreads) s += (double)gload<float>(d.partials + i);
  s = wave_sum_d(s);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    gstore<float>(d.xs, (float)(1.0 / (sqrt(tot) + (double)P.eps)));
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void scale_out_kernel(ScaleOutParams P) {
  using Tr = Elem<T>;
  constexpr int E = Tr::E;
  constexpr int CPR = kPrepTile / E;
  constexpr int NCH = kPrepTile * kPrepTile / (kThreads * E);
  const PrepTile tile = P.tiles[blockIdx.x];
  const MatDesc& d = P.mats[tile.mat];
  const int64_t rows = d.rows, cols = d.cols;
  const float xs = gload<float>(d.xs);
  const float step = -P.lr * d.upd_scale;
  // the prep tiles of a transposed bf16 matrix are kPrepTileT wide
  const int tw = sizeof(T) == 2 && d.transposed ? kPrepTileT : kPrepTile;
  for (int h = 0; h < tw / kPrepTile; ++h)
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int q = threadIdx.x + kThreads * p;
    const int64_t r = tile.tr * kPrepTile + q / CPR;
    const int64_t c0 = (int64_t)tile.tc * tw + h * kPrepTile + (q % CPR) * E;
    if (r >= rows) continue;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t c = c0 + e;
      if (c >= cols) break;
      const int64_t off = r * cols + c;
      const float o = xs * Tr::load1(d.v, off);
      if (P.out_kind == OUT_O) {
        store_any(d.o, P.out_dt, off, o);
      } else {
        const float wo = Tr::load1(d.w, off);
        Tr::store1(d.w, off, P.wdl == 0.0 ? Tr::fma_store(step, o, wo)
                                          : Tr::round_store(w_update(wo, step, o, P.wdl)));
      }
    }
  }
}

}  // namespace

hipError_t launch_prep_t(const PrepParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(prep_t_kernel, dim3(n_tiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prep(int dt, const PrepParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(prep_kernel<uint16_t>, dim3(n_tiles), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(prep_kernel<float>, dim3(n_tiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeParams& p, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(count), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scale_out(int dt, const ScaleOutParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(scale_out_kernel<uint16_t>, dim3(n_tiles), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(scale_out_kernel<float>, dim3(n_tiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
