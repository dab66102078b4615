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
// index is XOR-swizzled with (row >> 1) & 7 so that MFMA fragment reads (16
// rows, one chunk), direct and transposed stores (two rows, 8 chunks each) are
// free of bank conflicts, and the fragment address of every 32-row block is a
// constant offset from one per-lane base.
//
// Main loop: global loads of step t+1 are issued first, the 64 MFMAs of step t
// run on double-buffered fragments, and the LDS stores of step t+1 are issued
// between the second and third k16 sub-steps, while queued MFMAs execute.
//
// Epilogue: each wave stages its accumulators through its own LDS region
// (float32) so that every global store is a contiguous row segment; the
// epilogue inputs (A for the polynomial, X for apply) are prefetched during
// the last K step and one stripe ahead.  On the last iteration the result is
// written in the original orientation as O, or folded straight into
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

// LDS has 64 banks of 4 bytes and serves 16 lanes of a 16-byte access per
// cycle: even rows occupy banks 0-31, odd rows banks 32-63.  The chunk swizzle
// (row >> 1) & 7 makes 16 consecutive rows at one logical chunk (an MFMA
// fragment read) hit 16 distinct bank groups.
__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row >> 1) & 7u)) << 4);
}

struct OpRegs {
  u32x4 r[8];
};

// Rows r0..r0+255 of a row-major matrix, k columns k0..k0+63.  Thread t loads
// 16-byte chunk (t & 7) of rows (t >> 3) + 32q.
__device__ __forceinline__ void load_direct(const uint16_t* src, int64_t ld, int r0, int k0,
                                            OpRegs& R) {
  const int t = threadIdx.x;
  const uint16_t* p = src + (int64_t)(r0 + (t >> 3)) * ld + k0 + (t & 7) * 8;
#pragma unroll
  for (int q = 0; q < 8; ++q) R.r[q] = gload<u32x4>(p + (int64_t)(32 * q) * ld);
}

__device__ __forceinline__ void store_direct(uint8_t* lds, const OpRegs& R) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) *(u32x4*)(lds + lds_off((t >> 3) + 32 * q, t & 7)) = R.r[q];
}

// Operand rows r0..r0+255 taken from the COLUMNS of rows k0..k0+63 of a
// row-major matrix (i.e. the transpose).  Thread t = (b = t & 7, a = t >> 3)
// loads the 8x8 block k0+8b.., r0+8a.. (eight 16-byte row segments; one load
// instruction covers 8 rows x 128 contiguous bytes per wave).
__device__ __forceinline__ void load_trans(const uint16_t* src, int64_t ld, int r0, int k0,
                                           OpRegs& R) {
  const int t = threadIdx.x;
  const uint16_t* p = src + (int64_t)(k0 + 8 * (t & 7)) * ld + r0 + 8 * (t >> 3);
#pragma unroll
  for (int e = 0; e < 8; ++e) R.r[e] = gload<u32x4>(p + (int64_t)e * ld);
}

// 8x8 transpose of 16-bit elements: R.r[e] holds k = 8b+e for operand rows
// 8a..8a+7; output row 8a+c gets k = 8b..8b+7 as one 16-byte LDS chunk b.
// Eight consecutive lanes write the 8 chunks of one row; lanes with odd a
// write rows in the order c ^ 1, so the two 8-lane halves of a 16-lane group
// land in opposite bank halves (conflict free).
__device__ __forceinline__ void store_trans(uint8_t* lds, const OpRegs& R) {
  const int t = threadIdx.x;
  const int a = t >> 3, b = t & 7;
  const uint32_t flip = (uint32_t)(a & 1);
  const uint32_t sel_even = flip ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = flip ? 0x05040100u : 0x07060302u;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? sel_odd : sel_even;   // row 8a + (c ^ flip)
    const int d = c >> 1;
    u32x4 o;
    o.x = __builtin_amdgcn_perm(R.r[1][d], R.r[0][d], sel);
    o.y = __builtin_amdgcn_perm(R.r[3][d], R.r[2][d], sel);
    o.z = __builtin_amdgcn_perm(R.r[5][d], R.r[4][d], sel);
    o.w = __builtin_amdgcn_perm(R.r[7][d], R.r[6][d], sel);
    *(u32x4*)(lds + lds_off(8 * a + (c ^ flip), b)) = o;
  }
}

struct Operands {
  const uint16_t* p;   // P source
  const uint16_t* q;   // Q source
  int64_t ldp, ldq;
  int rp0, rq0;        // operand row origins (i0, j0)
};

struct WaveGeo {
  int wi0, wj0, frow, fkc;
};

// MFMA fragments of k16 sub-step kk: P rows wi0 + 32bi + (lane & 31) and Q rows
// wj0 + 32bj + (lane & 31), k chunk 2kk + (lane >> 5).
__device__ __forceinline__ void read_frags(const uint8_t* base, int kk, const WaveGeo& g,
                                           bf16x8 (&p)[4], bf16x8 (&q)[4]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
    p[bi] = *(const bf16x8*)(base + lds_off(g.wi0 + 32 * bi + g.frow, 2 * kk + g.fkc));
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
    q[bj] = *(const bf16x8*)(base + OPB + lds_off(g.wj0 + 32 * bj + g.frow, 2 * kk + g.fkc));
}

__device__ __forceinline__ void op_load_rt(bool tr, const uint16_t* src, int64_t ld, int r0,
                                           int k0, OpRegs& R) {
  if (tr) load_trans(src, ld, r0, k0, R);
  else load_direct(src, ld, r0, k0, R);
}

__device__ __forceinline__ void op_store_rt(bool tr, uint8_t* lds, const OpRegs& R) {
  if (tr) store_trans(lds, R);
  else store_direct(lds, R);
}

// 16 MFMAs of one k16 sub-step.
__device__ __forceinline__ void mfma16(f32x16 (&acc)[4][4], const bf16x8 (&p)[4],
                                       const bf16x8 (&q)[4]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[bj], p[bi], acc[bi][bj], 0, 0, 0);
}

// The 64 MFMAs of one K step on LDS stage `cur`.  Fragments of sub-step kk+1 are
// read while the MFMAs of sub-step kk run.  When `store`, the staged operand
// registers are written to LDS stage `nxt` between sub-steps 1 and 2 (the
// writes drain while the queued MFMAs execute).  Scheduling fences keep every
// sub-step's loads next to its MFMAs, which bounds the registers in flight.
__device__ __forceinline__ void kstep(f32x16 (&acc)[4][4], const uint8_t* cur, uint8_t* nxt,
                                      bool store, bool tp, bool tq, const OpRegs& rp,
                                      const OpRegs& rq, const WaveGeo& g) {
  bf16x8 pa[4], qa[4], pb[4], qb[4];
  read_frags(cur, 0, g, pa, qa);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(cur, 1, g, pb, qb);
  mfma16(acc, pa, qa);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(cur, 2, g, pa, qa);
  mfma16(acc, pb, qb);
  __builtin_amdgcn_sched_barrier(0);
  if (store) {
    op_store_rt(tp, nxt, rp);
    op_store_rt(tq, nxt + OPB, rq);
  }
  __builtin_amdgcn_sched_barrier(0);
  read_frags(cur, 3, g, pb, qb);
  mfma16(acc, pa, qa);
  __builtin_amdgcn_sched_barrier(0);
  mfma16(acc, pb, qb);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void prefetch_stripe(const uint16_t* src, int64_t ld, int64_t row0,
                                                int64_t col0, int lane, u32x2 (&dst)[16]) {
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int q = lane + 64 * p;
    dst[p] = gload<u32x2>(src + (row0 + (q >> 5)) * ld + col0 + (q & 31) * 4);
  }
}

// Stage acc[BI][*] (32 rows of the wave's 128 x 128 sub-tile) into the wave's
// LDS region as float32 rows.  acc[BI][bj][r] holds
//   C[32BI + (lane & 31)][32bj + 8(r>>2) + 4(lane>>5) + (r&3)]   (wave-local)
// (operands swapped in the MFMA, so 4 consecutive columns per register group).
template <int BI>
__device__ __forceinline__ void stage_stripe(const f32x16 (&acc)[4][4], float* stg, int frow,
                                             int fkc) {
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = {acc[BI][bj][4 * g], acc[BI][bj][4 * g + 1], acc[BI][bj][4 * g + 2],
                       acc[BI][bj][4 * g + 3]};
      *(f32x4*)(stg + frow * EP_PITCH + 32 * bj + 8 * g + 4 * fkc) = v;
    }
}

// Final output of 4 consecutive original-orientation columns c0..c0+3 of row r:
// O (float32 or bf16) or the fused weight update W <- W + upd * val rounded
// once.  Vector accesses when the row is a whole number of 16-byte chunks and
// the 4 columns are in range, element accesses at a ragged edge.
template <int OUT>
__device__ __forceinline__ void write_out4(const MatDesc& d, const GemmParams& P, int64_t r,
                                           int64_t c0, const float (&v)[4], float upd) {
  const int64_t cols = d.cols;
  const int64_t off = r * cols + c0;
  if (d.vec_ok && c0 + 3 < cols) {
    if (OUT == OUT_O) {
      if (P.out_dt == DT_F32) gstore<f32x4>((float*)d.o + off, f32x4{v[0], v[1], v[2], v[3]});
      else gstore<u32x2>((uint16_t*)d.o + off, u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])});
    } else {
      uint16_t* w = (uint16_t*)d.w + off;
      const u32x2 wo = gload<u32x2>(w);
      const float w4[4] = {lo_bf(wo.x), hi_bf(wo.x), lo_bf(wo.y), hi_bf(wo.y)};
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f64_to_bf16(fma((double)upd, (double)v[e], (double)w4[e]));
      gstore<u32x2>(w, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (c0 + e >= cols) break;
    if (OUT == OUT_O) {
      store_any(d.o, P.out_dt, off + e, v[e]);
    } else {
      uint16_t* w = (uint16_t*)d.w + off + e;
      const float wo = bf2f(gload<uint16_t>(w));
      gstore<uint16_t>(w, (uint16_t)f64_to_bf16(fma((double)upd, (double)v[e], (double)wo)));
    }
  }
}

// Epilogue of one wave's 128 x 128 sub-tile, one 32-row stripe at a time (a
// rolled loop: only the accumulator staging is specialised per stripe, which
// keeps the kernel small enough for the instruction cache).  Each stripe is
// staged through the wave's own LDS region (LDS executes one wave's accesses in
// order, so no workgroup barrier is needed) and written row-wise: 16 chunks of
// 4 consecutive columns per lane.  The epilogue input of the next stripe (A for
// the polynomial, X for apply) is prefetched while the current one is written.
template <int STAGE, int OUT>
__device__ __forceinline__ void epilogue(const MatDesc& d, const GemmParams& P,
                                         const f32x16 (&acc)[4][4], float* stg,
                                         const uint16_t* ep_src, int64_t ep_ld, uint16_t* out,
                                         int64_t ld_out, int i0, int j0, int lane, int frow,
                                         int fkc, float s_first, u32x2 (&ecur)[16]) {
  constexpr bool EP_IN = STAGE != 0;
  const int64_t rows = d.rows, cols = d.cols;
  const bool out_trans = OUT != OUT_NEXT_X && d.transposed;
  const float upd = -P.lr * d.upd_scale;
  u32x2 enext[16];
#pragma unroll 1
  for (int bi = 0; bi < 4; ++bi) {
    if (EP_IN && bi + 1 < 4) prefetch_stripe(ep_src, ep_ld, i0 + 32 * (bi + 1), j0, lane, enext);
    switch (bi) {
      case 0: stage_stripe<0>(acc, stg, frow, fkc); break;
      case 1: stage_stripe<1>(acc, stg, frow, fkc); break;
      case 2: stage_stripe<2>(acc, stg, frow, fkc); break;
      default: stage_stripe<3>(acc, stg, frow, fkc); break;
    }
    __builtin_amdgcn_wave_barrier();

    const int64_t ib = i0 + 32 * bi;   // first X-orientation row of this stripe
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int q = lane + 64 * p;
      const int rr = q >> 5, c4 = (q & 31) * 4;
      const int64_t i = ib + rr;
      const int64_t j = j0 + c4;
      const f32x4 v = *(const f32x4*)(stg + rr * EP_PITCH + c4);
      if (STAGE == 0) {
        const float s2 = s_first * s_first;
        const u32x2 o = {pack_bf2(v.x * s2, v.y * s2), pack_bf2(v.z * s2, v.w * s2)};
        gstore<u32x2>(out + i * ld_out + j, o);
      } else if (STAGE == 1) {
        const u32x2 ain = ecur[p];
        const float b = P.b, c = P.c;
        const u32x2 o = {pack_bf2(fmaf(b, lo_bf(ain.x), c * v.x), fmaf(b, hi_bf(ain.x), c * v.y)),
                         pack_bf2(fmaf(b, lo_bf(ain.y), c * v.z), fmaf(b, hi_bf(ain.y), c * v.w))};
        gstore<u32x2>(out + i * ld_out + j, o);
      } else {
        const u32x2 xin = ecur[p];
        const float a = P.a;
        f32x4 val;
        val.x = s_first * fmaf(a, lo_bf(xin.x), v.x);
        val.y = s_first * fmaf(a, hi_bf(xin.x), v.y);
        val.z = s_first * fmaf(a, lo_bf(xin.y), v.z);
        val.w = s_first * fmaf(a, hi_bf(xin.y), v.w);
        if (OUT == OUT_NEXT_X) {
          const u32x2 o = {pack_bf2(val.x, val.y), pack_bf2(val.z, val.w)};
          gstore<u32x2>(out + i * ld_out + j, o);
        } else if (out_trans) {
          *(f32x4*)(stg + rr * EP_PITCH + c4) = val;   // transposed pass below
        } else if (i < rows && j < cols) {
          // original orientation == X orientation: row i, columns j..j+3
          const float vv[4] = {val.x, val.y, val.z, val.w};
          write_out4<OUT>(d, P, i, j, vv, upd);
        }
      }
    }
    if (OUT != OUT_NEXT_X && out_trans) {
      __builtin_amdgcn_wave_barrier();
      // Output row jr (original) = X column j0+jj; original columns are the X
      // rows ib + 4ic .. +3.
#pragma unroll 2
      for (int p = 0; p < 16; ++p) {
        const int q = lane + 64 * p;
        const int ic = q & 7, jj = q >> 3;
        const int64_t jr = j0 + jj;
        const int64_t ic0 = ib + 4 * ic;
        if (jr >= rows || ic0 >= cols) continue;
        float vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = stg[(4 * ic + e) * EP_PITCH + jj];
        write_out4<OUT>(d, P, jr, ic0, vv, upd);
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (EP_IN) {
#pragma unroll
      for (int p = 0; p < 16; ++p) ecur[p] = enext[p];
    }
  }
}

// One kernel per stage (and, for apply, per output kind), so that each carries
// only its own operand modes and epilogue.
template <int STAGE, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHR, NTHR), amdgpu_waves_per_eu(1, 1)))
void ns_gemm_bf16_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  const GemmTile tile = P.tiles[blockIdx.x];
  if (tile.mat < 0) return;   // idle entry padding an XCD stream
  const MatDesc d = P.mats[tile.mat];
  const int i0 = tile.ti * BM, j0 = tile.tj * BM;
  const int64_t mp = d.mp, np = d.np;
  const uint16_t* xcur = (const uint16_t*)(P.cur ? d.x[1] : d.x[0]);
  uint16_t* xnext = (uint16_t*)(P.cur ? d.x[0] : d.x[1]);

  // Operands and the number of leading K steps each one is read transposed:
  // symmetric storage transposes the k-blocks left of the operand's row block.
  Operands op;
  int K, tP, tQ;
  if (STAGE == 0) {
    op = {xcur, xcur, np, np, i0, j0};
    K = (int)np;
    tP = tQ = 0;
  } else if (STAGE == 1) {
    op = {(const uint16_t*)d.a, (const uint16_t*)d.a, mp, mp, i0, j0};
    K = (int)mp;
    tP = i0 / BK;
    tQ = j0 / BK;
  } else {
    op = {(const uint16_t*)d.b, xcur, mp, np, i0, j0};
    K = (int)mp;
    tP = i0 / BK;
    tQ = K / BK;
  }
  const int nk = K / BK;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  WaveGeo g;
  g.wi0 = (wave >> 1) * 128;   // wave sub-tile origin (rows)
  g.wj0 = (wave & 1) * 128;    // wave sub-tile origin (cols)
  g.frow = lane & 31;          // fragment row within a 32-block
  g.fkc = lane >> 5;           // fragment k chunk (0/1) within a k16 step

  f32x16 acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  // prologue: step 0 into stage 0.  Operand P (Q) is read transposed for the
  // first tP (tQ) K steps.
  OpRegs rp, rq;
  op_load_rt(tP > 0, op.p, op.ldp, op.rp0, 0, rp);
  op_load_rt(tQ > 0, op.q, op.ldq, op.rq0, 0, rq);
  op_store_rt(tP > 0, lds, rp);
  op_store_rt(tQ > 0, lds + OPB, rq);
  __syncthreads();

  // steps 1..nk-1: load step t, compute step t-1
  for (int t = 1; t < nk; ++t) {
    const bool tp = t < tP, tq = t < tQ;
    op_load_rt(tp, op.p, op.ldp, op.rp0, t * BK, rp);
    op_load_rt(tq, op.q, op.ldq, op.rq0, t * BK, rq);
    __builtin_amdgcn_sched_barrier(0);
    kstep(acc, lds + ((t - 1) & 1) * STG, lds + (t & 1) * STG, true, tp, tq, rp, rq, g);
    __syncthreads();
  }

  // last K step; prefetch the first epilogue stripe meanwhile
  const int64_t ep_ld = STAGE == 1 ? mp : np;
  const uint16_t* ep_src = STAGE == 1 ? (const uint16_t*)d.a : xcur;
  u32x2 ecur[16];
  if (STAGE != 0) prefetch_stripe(ep_src, ep_ld, i0 + g.wi0, j0 + g.wj0, lane, ecur);
  kstep(acc, lds + ((nk - 1) & 1) * STG, nullptr, false, false, false, rp, rq, g);
  __syncthreads();

  uint16_t* out = STAGE == 0 ? (uint16_t*)d.a : STAGE == 1 ? (uint16_t*)d.b : xnext;
  const int64_t ld_out = STAGE == 2 ? np : mp;
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  epilogue<STAGE, OUT>(d, P, acc, (float*)(lds + wave * EP_WAVE_BYTES), ep_src, ep_ld, out,
                       ld_out, i0 + g.wi0, j0 + g.wj0, lane, g.frow, g.fkc, s_first, ecur);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  const dim3 grid(n_tiles), block(NTHR);
  if (p.stage == 0)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<0, OUT_NEXT_X>), grid, block, 0, s, p);
  else if (p.stage == 1)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<1, OUT_NEXT_X>), grid, block, 0, s, p);
  else if (p.out_kind == OUT_NEXT_X)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_NEXT_X>), grid, block, 0, s, p);
  else if (p.out_kind == OUT_O)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_O>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_W_UPDATE>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
