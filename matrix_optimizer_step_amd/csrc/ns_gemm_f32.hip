// Newton-Schulz matrix products in float32 (the fp32 storage path), grouped over
// a ragged batch.  The same three stages and tile tables as the bf16 MFMA
// kernel (ns_gemm_bf16.hip), on a simpler engine: 64 x 64 output tiles, 256
// threads each owning a 4 x 4 block, K step 16, float32 FMA accumulation.  The
// polynomial is split between the stages here (B = b A + c A A, then
// X' = a X + B X): nothing is rounded to bf16 in between, so the split and the
// folded form (B = aI + bA + cAA, X' = B X) agree to float32 rounding.
// No reduced-precision products are used anywhere on this path.
//
// Roofline: a dense contraction bound by the float32 vector FMA rate; in
// practice this path serves small fp32 matrices and is latency bound.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int TM = 64;     // tile rows == cols == symmetric block
constexpr int TK = 16;
constexpr int NTHR = 256;
constexpr int PITCH = TM + 4;

enum OpMode { MODE_DIRECT = 0, MODE_TRANS = 1, MODE_SYM = 2 };

struct OpSrc {
  const float* ptr;
  int64_t ld;
  int r0;
  int mode;
};

// Fill s[k][r] (k < TK, r < TM) with operand rows r0.. and k columns k0..
__device__ __forceinline__ void load_op(const OpSrc& o, int k0, float (*s)[PITCH]) {
  const int t = threadIdx.x;
  const bool tr = o.mode == MODE_TRANS || (o.mode == MODE_SYM && (k0 / TM) < (o.r0 / TM));
  if (!tr) {
    const int row = t >> 2, kc = (t & 3) * 4;
    const f32x4 v = gload<f32x4>(o.ptr + (int64_t)(o.r0 + row) * o.ld + k0 + kc);
    s[kc + 0][row] = v.x;
    s[kc + 1][row] = v.y;
    s[kc + 2][row] = v.z;
    s[kc + 3][row] = v.w;
  } else {
    const int k = t >> 4, rc = (t & 15) * 4;
    const f32x4 v = gload<f32x4>(o.ptr + (int64_t)(k0 + k) * o.ld + o.r0 + rc);
    *(f32x4*)&s[k][rc] = v;
  }
}

__global__ __launch_bounds__(NTHR) void ns_gemm_f32_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(16))) float ps[TK][PITCH];
  __shared__ __attribute__((aligned(16))) float qs[TK][PITCH];

  const GemmTile tile = P.tiles[blockIdx.x];
  if (tile.mat < 0) return;   // idle entry padding an XCD stream
  const MatDesc d = P.mats[tile.mat];
  const int stage = P.stage;
  const int i0 = tile.ti * TM, j0 = tile.tj * TM;
  const int64_t mp = d.mp, np = d.np;
  // memory safety: an entry outside the matrix's output grid does nothing
  if (i0 < 0 || j0 < 0 || i0 + TM > mp || j0 + TM > (stage == 2 ? np : mp)) return;
  const float* xcur = (const float*)(P.first ? d.x0in : P.cur ? d.x[1] : d.x[0]);
  float* xnext = (float*)(P.cur ? d.x[0] : d.x[1]);

  OpSrc sp, sq;
  int K;
  if (stage == 0) {
    sp = {xcur, np, i0, MODE_DIRECT};
    sq = {xcur, np, j0, MODE_DIRECT};
    K = (int)np;
  } else if (stage == 1) {
    sp = {(const float*)d.a, mp, i0, MODE_SYM};
    sq = {(const float*)d.a, mp, j0, MODE_SYM};
    K = (int)mp;
  } else {
    sp = {(const float*)d.b, mp, i0, MODE_SYM};
    sq = {xcur, np, j0, MODE_TRANS};
    K = (int)mp;
  }

  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    load_op(sp, k0, ps);
    load_op(sq, k0, qs);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      const float4 a = *(const float4*)&ps[k][ty * 4];
      const float4 b = *(const float4*)&qs[k][tx * 4];
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }

  const float xs = gload<float>(d.xs);
  const float s_first = P.first ? xs : 1.f;
  const int64_t rows = d.rows, cols = d.cols;
  const float upd = -P.lr * d.upd_scale;
  const int64_t ib = i0 + ty * 4, jb = j0 + tx * 4;

  if (stage == 0) {
    const float s2 = s_first * s_first;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      gstore<f32x4>((float*)d.a + (ib + r) * mp + jb,
                    f32x4{acc[r][0] * s2, acc[r][1] * s2, acc[r][2] * s2, acc[r][3] * s2});
    return;
  }
  if (stage == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 ain = gload<f32x4>((const float*)d.a + (ib + r) * mp + jb);
      gstore<f32x4>((float*)d.b + (ib + r) * mp + jb,
                    f32x4{fmaf(P.b, ain.x, P.c * acc[r][0]), fmaf(P.b, ain.y, P.c * acc[r][1]),
                          fmaf(P.b, ain.z, P.c * acc[r][2]), fmaf(P.b, ain.w, P.c * acc[r][3])});
    }
    return;
  }
  float val[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 xin = gload<f32x4>(xcur + (ib + r) * np + jb);
    val[r][0] = s_first * fmaf(P.a, xin.x, acc[r][0]);
    val[r][1] = s_first * fmaf(P.a, xin.y, acc[r][1]);
    val[r][2] = s_first * fmaf(P.a, xin.z, acc[r][2]);
    val[r][3] = s_first * fmaf(P.a, xin.w, acc[r][3]);
  }
  if (P.out_kind == OUT_NEXT_X) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      gstore<f32x4>(xnext + (ib + r) * np + jb, f32x4{val[r][0], val[r][1], val[r][2], val[r][3]});
    return;
  }
  // Last iteration: original orientation (transposed back when rows > cols).
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t xi = ib + r, xj = jb + c;
      const int64_t orow = d.transposed ? xj : xi;
      const int64_t ocol = d.transposed ? xi : xj;
      if (orow >= rows || ocol >= cols) continue;
      const int64_t off = orow * cols + ocol;
      if (P.out_kind == OUT_O) {
        store_any(d.o, P.out_dt, off, val[r][c]);
      } else {
        float* w = (float*)d.w + off;
        const float wo = gload<float>(w);
        // one rounding: float32 fma without decay, float64 then float32 with it
        gstore<float>(w, P.wdl == 0.0 ? fmaf(upd, val[r][c], wo)
                                      : (float)w_update(wo, upd, val[r][c], P.wdl));
      }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(ns_gemm_f32_kernel, dim3(n_tiles), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
