// Newton-Schulz matrix products on bf16 MFMA (gfx950), grouped over a ragged
// batch of matrices: one launch per stage covers every matrix of the batch.
//
// The three products of one iteration (blog post, appendix Newton-Schulz
// routine, written in factored form) all reduce to C[i][j] = sum_k P[i][k]Q[j][k]
// with both operands staged in LDS as [row][k] tiles:
//
//   stage 0 (Gram)    A = s^2 * X X^T     P = Q = X rows (k contiguous in HBM)
//                     only tiles ti <= tj are computed (A is symmetric).
//   stage 1 (poly)    B = b*A + c*A A     P = Q = A rows; A A = A A^T.  Only the
//                     upper tiles of A exist: a k-block left of the diagonal
//                     block is read from the mirrored upper tile and transposed
//                     on its way into LDS.  Only tiles ti <= tj are computed.
//   stage 2 (apply)   X' = s*(a*X + B X)  P = B rows (mirrored reads as above),
//                     Q = X^T rows: X is read k-row-major and transposed into
//                     LDS.  Every tile is computed.
//
// s is the Frobenius scale 1/(||V||+eps) on the first iteration, 1 afterwards.
//
// Tile: 256 x 256 outputs per workgroup of 4 waves (each wave 128 x 128 =
// 4 x 4 blocks of v_mfma_f32_32x32x16_bf16), K step 64, two LDS stages of
// 2 x 256 x 64 bf16 (128 KB total).  LDS rows are 128 bytes; the 16-byte chunk
// index is XOR-swizzled with (row ^ row>>3) & 7 so that MFMA fragment reads,
// direct stores and transposed stores are all free of bank conflicts.
//
// The epilogue stages each wave's accumulators through LDS (float32) so that
// every global store is a contiguous row segment.  On the last iteration the
// result is written in the original orientation as O or folded straight into
// W <- W - lr*sqrt(max(1,rows/cols))*O (so O never round-trips through HBM).
//
// Roofline: a dense contraction; algorithmic flops per tile are 2*256*256*K
// (K = n for stage 0, m for stages 1 and 2).  Bound: bf16 MFMA peak.
#include "common.hpp"
#include "device_util.hpp"

namespace matopt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;            // tile rows == tile cols == symmetric block
constexpr int BK = 64;             // K step
constexpr int NTHR = 256;
constexpr int OPB = BM * BK * 2;   // bytes of one operand tile in LDS (32 KB)
constexpr int STG = 2 * OPB;       // one pipeline stage (P and Q)
constexpr int LDS_BYTES = 2 * STG; // two stages
constexpr int EP_PITCH = 132;      // float pitch of the epilogue staging rows
constexpr int EP_WAVE_BYTES = 32 * EP_PITCH * 4;
static_assert(4 * EP_WAVE_BYTES <= LDS_BYTES, "epilogue staging must fit");

__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row ^ (row >> 3)) & 7u)) << 4);
}

struct OpRegs {
  uint4 r[8];
};

// Rows r0..r0+255 of a row-major matrix, k columns k0..k0+63.  Thread t loads
// 16-byte chunk (t & 7) of rows (t >> 3) + 32q.
__device__ __forceinline__ void load_direct(const uint16_t* __restrict__ src, int64_t ld,
                                            int r0, int k0, OpRegs& R) {
  const int t = threadIdx.x;
  const uint16_t* p = src + (int64_t)(r0 + (t >> 3)) * ld + k0 + (t & 7) * 8;
#pragma unroll
  for (int q = 0; q < 8; ++q) R.r[q] = *(const uint4*)(p + (int64_t)(32 * q) * ld);
}

__device__ __forceinline__ void store_direct(uint8_t* lds, const OpRegs& R) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) *(uint4*)(lds + lds_off((t >> 3) + 32 * q, t & 7)) = R.r[q];
}

// Operand rows r0..r0+255 taken from the COLUMNS of rows k0..k0+63 of a
// row-major matrix (i.e. the transpose).  Thread t = (a = t & 31, b = t >> 5)
// loads the 8x8 block k0+8b.., r0+8a.. (eight 16-byte row segments).
__device__ __forceinline__ void load_trans(const uint16_t* __restrict__ src, int64_t ld,
                                           int r0, int k0, OpRegs& R) {
  const int t = threadIdx.x;
  const uint16_t* p = src + (int64_t)(k0 + 8 * (t >> 5)) * ld + r0 + 8 * (t & 31);
#pragma unroll
  for (int e = 0; e < 8; ++e) R.r[e] = *(const uint4*)(p + (int64_t)e * ld);
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 8x8 transpose of 16-bit elements: R.r[e] holds k = 8b+e for operand rows
// 8a..8a+7; output row 8a+c gets k = 8b..8b+7 as one 16-byte LDS chunk b.
__device__ __forceinline__ void store_trans(uint8_t* lds, const OpRegs& R) {
  const int t = threadIdx.x;
  const int a = t & 31, b = t >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int d = c >> 1;
    uint4 o;
    o.x = __builtin_amdgcn_perm(dw(R.r[1], d), dw(R.r[0], d), sel);
    o.y = __builtin_amdgcn_perm(dw(R.r[3], d), dw(R.r[2], d), sel);
    o.z = __builtin_amdgcn_perm(dw(R.r[5], d), dw(R.r[4], d), sel);
    o.w = __builtin_amdgcn_perm(dw(R.r[7], d), dw(R.r[6], d), sel);
    *(uint4*)(lds + lds_off(8 * a + c, b)) = o;
  }
}

enum OpMode { MODE_DIRECT = 0, MODE_TRANS = 1, MODE_SYM = 2 };

struct OpSrc {
  const uint16_t* ptr;
  int64_t ld;
  int r0;
  int mode;
};

__device__ __forceinline__ bool op_trans(const OpSrc& s, int k0) {
  return s.mode == MODE_TRANS || (s.mode == MODE_SYM && (k0 / BM) < (s.r0 / BM));
}

__device__ __forceinline__ void op_load(const OpSrc& s, int k0, bool tr, OpRegs& R) {
  if (tr) load_trans(s.ptr, s.ld, s.r0, k0, R);
  else load_direct(s.ptr, s.ld, s.r0, k0, R);
}

__device__ __forceinline__ void op_store(uint8_t* lds, bool tr, const OpRegs& R) {
  if (tr) store_trans(lds, R);
  else store_direct(lds, R);
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTHR, NTHR), amdgpu_waves_per_eu(1, 1)))
void ns_gemm_bf16_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  const GemmTile tile = P.tiles[blockIdx.x];
  const MatDesc d = P.mats[tile.mat];
  const int stage = P.stage;
  const int i0 = tile.ti * BM, j0 = tile.tj * BM;
  const int64_t mp = d.mp, np = d.np;
  const uint16_t* xcur = (const uint16_t*)(P.cur ? d.x[1] : d.x[0]);
  uint16_t* xnext = (uint16_t*)(P.cur ? d.x[0] : d.x[1]);

  OpSrc sp, sq;
  int K;
  if (stage == 0) {
    sp = {xcur, np, i0, MODE_DIRECT};
    sq = {xcur, np, j0, MODE_DIRECT};
    K = (int)np;
  } else if (stage == 1) {
    sp = {(const uint16_t*)d.a, mp, i0, MODE_SYM};
    sq = {(const uint16_t*)d.a, mp, j0, MODE_SYM};
    K = (int)mp;
  } else {
    sp = {(const uint16_t*)d.b, mp, i0, MODE_SYM};
    sq = {xcur, np, j0, MODE_TRANS};
    K = (int)mp;
  }
  const int nk = K / BK;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wi0 = (wave >> 1) * 128;   // wave sub-tile origin (rows)
  const int wj0 = (wave & 1) * 128;    // wave sub-tile origin (cols)
  const int frow = lane & 31;          // fragment row within a 32-block
  const int fkc = lane >> 5;           // fragment k chunk (0/1) within a k16 step

  f32x16 acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  OpRegs rp, rq;
  {
    const bool tp = op_trans(sp, 0), tq = op_trans(sq, 0);
    op_load(sp, 0, tp, rp);
    op_load(sq, 0, tq, rq);
    op_store(lds, tp, rp);
    op_store(lds + OPB, tq, rq);
  }
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    uint8_t* cur = lds + (ks & 1) * STG;
    uint8_t* nxt = lds + ((ks + 1) & 1) * STG;
    const bool more = ks + 1 < nk;
    bool tp = false, tq = false;
    if (more) {
      const int k0 = (ks + 1) * BK;
      tp = op_trans(sp, k0);
      tq = op_trans(sq, k0);
      op_load(sp, k0, tp, rp);
      op_load(sq, k0, tq, rq);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 pf[4], qf[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        pf[bi] = *(const bf16x8*)(cur + lds_off(wi0 + 32 * bi + frow, 2 * kk + fkc));
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        qf[bj] = *(const bf16x8*)(cur + OPB + lds_off(wj0 + 32 * bj + frow, 2 * kk + fkc));
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[bj], pf[bi], acc[bi][bj],
                                                               0, 0, 0);
    }
    if (more) {
      op_store(nxt, tp, rp);
      op_store(nxt + OPB, tq, rq);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[bi][bj][r] (operands swapped in the MFMA) holds
  //   C[wi0 + 32bi + (lane & 31)][wj0 + 32bj + 8(r>>2) + 4(lane>>5) + (r&3)].
  float* stg = (float*)(lds + wave * EP_WAVE_BYTES);
  const float xs = d.xs[0];
  const float s_first = P.first ? xs : 1.f;
  const bool last = stage == 2 && P.out_kind != OUT_NEXT_X;
  const bool out_trans = last && d.transposed;
  const int64_t rows = d.rows, cols = d.cols;
  const float upd = -P.lr * d.upd_scale;

#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v = make_float4(acc[bi][bj][4 * g], acc[bi][bj][4 * g + 1],
                               acc[bi][bj][4 * g + 2], acc[bi][bj][4 * g + 3]);
        *(float4*)(stg + frow * EP_PITCH + 32 * bj + 8 * g + 4 * fkc) = v;
      }
    __syncthreads();

    const int ib = i0 + wi0 + 32 * bi;   // first X-orientation row of this stripe
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
      const int q = lane + 64 * p;
      const int rr = q >> 5, c4 = (q & 31) * 4;
      const int64_t i = ib + rr;
      const int64_t j = j0 + wj0 + c4;
      float4 v = *(const float4*)(stg + rr * EP_PITCH + c4);
      if (stage == 0) {
        const float s2 = s_first * s_first;
        uint2 o = make_uint2(pack_bf2(v.x * s2, v.y * s2), pack_bf2(v.z * s2, v.w * s2));
        *(uint2*)((uint16_t*)d.a + i * mp + j) = o;
      } else if (stage == 1) {
        const uint2 ain = *(const uint2*)((const uint16_t*)d.a + i * mp + j);
        const float b = P.b, c = P.c;
        uint2 o = make_uint2(pack_bf2(fmaf(b, lo_bf(ain.x), c * v.x), fmaf(b, hi_bf(ain.x), c * v.y)),
                             pack_bf2(fmaf(b, lo_bf(ain.y), c * v.z), fmaf(b, hi_bf(ain.y), c * v.w)));
        *(uint2*)((uint16_t*)d.b + i * mp + j) = o;
      } else {
        const uint2 xin = *(const uint2*)(xcur + i * np + j);
        const float a = P.a;
        float4 val;
        val.x = s_first * fmaf(a, lo_bf(xin.x), v.x);
        val.y = s_first * fmaf(a, hi_bf(xin.x), v.y);
        val.z = s_first * fmaf(a, lo_bf(xin.y), v.z);
        val.w = s_first * fmaf(a, hi_bf(xin.y), v.w);
        if (!last) {
          uint2 o = make_uint2(pack_bf2(val.x, val.y), pack_bf2(val.z, val.w));
          *(uint2*)(xnext + i * np + j) = o;
        } else if (out_trans) {
          *(float4*)(stg + rr * EP_PITCH + c4) = val;   // transposed pass below
        } else if (i < rows) {
          // original orientation == X orientation: row i, columns j..j+3
          const float vv[4] = {val.x, val.y, val.z, val.w};
          if (P.out_kind == OUT_O) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < cols) store_any(d.o, P.out_dt, i * cols + j + e, vv[e]);
          } else {
            uint16_t* w = (uint16_t*)d.w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < cols) {
                const int64_t off = i * cols + j + e;
                w[off] = (uint16_t)f64_to_bf16(fma((double)upd, (double)vv[e], (double)bf2f(w[off])));
              }
          }
        }
      }
    }
    if (out_trans) {
      __syncthreads();
      // Output row jr (original) = X column j0+wj0+jj; original columns are the
      // X rows ib + 4ic .. +3.
#pragma unroll 4
      for (int p = 0; p < 16; ++p) {
        const int q = lane + 64 * p;
        const int ic = q & 7, jj = q >> 3;
        const int64_t jr = j0 + wj0 + jj;
        const int64_t ic0 = ib + 4 * ic;
        if (jr >= rows) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t ccol = ic0 + e;
          if (ccol >= cols) break;
          const float val = stg[(4 * ic + e) * EP_PITCH + jj];
          const int64_t off = jr * cols + ccol;
          if (P.out_kind == OUT_O) {
            store_any(d.o, P.out_dt, off, val);
          } else {
            uint16_t* w = (uint16_t*)d.w;
            w[off] = (uint16_t)f64_to_bf16(fma((double)upd, (double)val, (double)bf2f(w[off])));
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(ns_gemm_bf16_kernel, dim3(n_tiles), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
