// Newton-Schulz matrix products in float32 (the fp32 storage path), grouped over
// a ragged batch.  The same three stages as the bf16 MFMA kernel
// (ns_gemm_bf16.hip) on a simpler engine: 32 x 32 output tiles (kGridF32; the
// matrices are padded to kTileF32 = 64), four waves per tile, each wave
// running its own K loop over every fourth K step of 16 and holding a 4 x 4
// block of the tile per lane in float32 FMA accumulators; the four partial
// tiles are summed in a fixed order through LDS at the end (deterministic).
// Small tiles and the K split keep a small matrix's launch short: a 256 x 512
// Gram is 36 tiles of 512 / 4 K values per wave.  The polynomial is split
// between the stages here (B = b A + c A A, then X' = a X + B X): nothing is
// rounded to bf16 in between, so the split and the folded form
// (B = aI + bA + cAA, X' = B X) agree to float32 rounding.  A and B are
// stored as their upper 32 x 32 tiles only (the Gram and polynomial tables
// hold ti <= tj), X whole.  No reduced-precision products are used anywhere
// on this path.
//
// Roofline: a dense contraction bound by the float32 vector FMA rate; in
// practice this path serves small fp32 matrices and is latency bound.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

constexpr int TM = kGridF32;   // tile rows == cols == symmetric block
constexpr int TK = 16;         // K step of one wave
constexpr int NWAVE = 4;
constexpr int NTHR = 64 * NWAVE;
constexpr int PITCH = TM + 4;  // floats per staged k row

enum OpMode { MODE_DIRECT = 0, MODE_TRANS = 1, MODE_SYM = 2 };

struct OpSrc {
  const float* ptr;
  int64_t ld;
  int r0;
  int mode;
};

// One operand slice of a wave's K step (TM rows x TK k values, k0 a multiple
// of TK), 8 floats per lane, loaded into registers.
struct OpRegs {
  f32x4 v[2];
};

__device__ __forceinline__ bool op_trans(const OpSrc& o, int k0) {
  // symmetric A stored as upper tiles: left of the diagonal block, rows r0..
  // of A are columns r0.. of the upper tile above
  return o.mode == MODE_TRANS || (o.mode == MODE_SYM && (k0 / TM) < (o.r0 / TM));
}

__device__ __forceinline__ void op_load(const OpSrc& o, int k0, int lane, OpRegs& r) {
  if (!op_trans(o, k0)) {   // element (row, k) at ptr[(r0 + row) * ld + k0 + k]
    const float* p = o.ptr + (int64_t)(o.r0 + (lane >> 1)) * o.ld + k0 + (lane & 1) * 8;
    r.v[0] = gload<f32x4>(p);
    r.v[1] = gload<f32x4>(p + 4);
  } else {                  // element (row, k) at ptr[(k0 + k) * ld + r0 + row]
    const float* p = o.ptr + (int64_t)(k0 + (lane >> 2)) * o.ld + o.r0 + (lane & 3) * 8;
    r.v[0] = gload<f32x4>(p);
    r.v[1] = gload<f32x4>(p + 4);
  }
}

// Stage the slice as s[k][row].
__device__ __forceinline__ void op_store(const OpSrc& o, int k0, int lane, const OpRegs& r,
                                         float (*s)[PITCH]) {
  if (!op_trans(o, k0)) {
    const int row = lane >> 1, kc = (lane & 1) * 8;
    const float f[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w,
                        r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) s[kc + q][row] = f[q];
  } else {
    const int k = lane >> 2, rc = (lane & 3) * 8;
    *(f32x4*)&s[k][rc] = r.v[0];
    *(f32x4*)&s[k][rc + 4] = r.v[1];
  }
}

__global__ __launch_bounds__(NTHR) void ns_gemm_f32_kernel(GemmParams P) {
  // per wave: two buffers of P and Q slices; reused for the partial tiles
  __shared__ __attribute__((aligned(16))) float stg[NWAVE][2][2][TK][PITCH];

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

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ty = lane >> 3, tx = lane & 7;   // 4 x 4 block at rows 4 ty, columns 4 tx
  float acc[4][4] = {};
  // wave w takes K steps w, w + 4, ... (K is a multiple of 64: every wave
  // gets the same count); its loads of step s+1 are in flight while step s
  // is multiplied out of the other buffer
  const int nsteps = K / TK;
  float (*buf)[2][TK][PITCH] = stg[wave];
  int b = 0;
  if (wave < nsteps) {
    OpRegs rp, rq;
    op_load(sp, wave * TK, lane, rp);
    op_load(sq, wave * TK, lane, rq);
    op_store(sp, wave * TK, lane, rp, buf[0][0]);
    op_store(sq, wave * TK, lane, rq, buf[0][1]);
  }
  for (int st = wave; st < nsteps; st += NWAVE) {
    const bool more = st + NWAVE < nsteps;
    OpRegs rp, rq;
    if (more) {
      op_load(sp, (st + NWAVE) * TK, lane, rp);
      op_load(sq, (st + NWAVE) * TK, lane, rq);
    }
    // the staged slice was written by this wave's own lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      const float4 a = *(const float4*)&buf[b][0][k][ty * 4];
      const float4 c = *(const float4*)&buf[b][1][k][tx * 4];
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(av[r], cv[q], acc[r][q]);
    }
    if (more) {
      // the other buffer was last read one step ago, by this wave only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      op_store(sp, (st + NWAVE) * TK, lane, rp, buf[b ^ 1][0]);
      op_store(sq, (st + NWAVE) * TK, lane, rq, buf[b ^ 1][1]);
    }
    b ^= 1;
  }

  // partial tiles: wave w's 32 x 32 block at red[w] (row-major, pitch TM + 4)
  __syncthreads();
  float* red = &stg[0][0][0][0][0];
  constexpr int RP = TM + 4;
  static_assert(NWAVE * TM * RP <= NWAVE * 2 * 2 * TK * PITCH, "partials fit the staging");
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *(f32x4*)&red[wave * TM * RP + (ty * 4 + r) * RP + tx * 4] =
        f32x4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f32x4 t = *(const f32x4*)&red[(ty * 4 + r) * RP + tx * 4];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      const f32x4 u = *(const f32x4*)&red[w * TM * RP + (ty * 4 + r) * RP + tx * 4];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    acc[r][0] = t.x;
    acc[r][1] = t.y;
    acc[r][2] = t.z;
    acc[r][3] = t.w;
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
