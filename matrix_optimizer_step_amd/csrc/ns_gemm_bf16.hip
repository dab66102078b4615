// Newton-Schulz matrix products on bf16 MFMA (gfx950), grouped over a ragged
// batch of matrices: one launch per stage covers every matrix of the batch.
//
// The three products of one iteration (blog post, appendix Newton-Schulz
// routine, written in factored form) all reduce to C[i][j] = sum_k P[i][k]Q[j][k]:
//
//   stage 0 (Gram)    A = s^2 * X X^T          P = Q = X rows (k contiguous in HBM)
//   stage 1 (poly)    B = a*I + b*A + c*A A    P = A rows, Q = A columns (A A = A A^T)
//   stage 2 (apply)   X' = s * B X             P = B rows, Q = X columns
//
// s is the Frobenius scale 1/(||V||+eps) on the first iteration, 1 afterwards.
// B is the whole polynomial p(A) = aI + bA + cA^2, stored in bf16, so that
// apply is one product with nothing read back in its epilogue (a X + (bA +
// cA^2) X = p(A) X; folding a into B's diagonal is as accurate as adding a X
// in float32, because X' is rounded to bf16 at the same relative precision).
// A and B are symmetric: only tiles ti <= tj are computed and stored (a
// diagonal tile whole).  A row block of A or B is read k-major from the upper
// tiles above it for the k-blocks left of its diagonal block (each k row of an
// operand tile is 512 contiguous bytes) and row-major (64 contiguous bytes per
// row and K step) from there on: apply reads B's rows so, the polynomial A's
// rows i0.. as P and, A being symmetric, A's rows j0.. as Q (its columns).  X
// is read row-major by the Gram and k-major (through its columns) by apply.
//
// Engine.  A 256 x 256 output tile per workgroup of 8 waves, two per SIMD
// (each wave 128 x 64, the 128 accumulators per lane in VGPRs within the 256
// a wave has at two waves per SIMD; while one wave of a SIMD waits on LDS the
// other issues MFMAs).  The Gram, polynomial and apply launches compute on
// v_mfma_f32_16x16x32_bf16 (8 x 4 slabs of 16 x 16 per wave; see "16 x 16 x
// 32 MFMA engine" below); the single diagonal tiles keep the 32 x 32 x 16
// form (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 per wave, two k16 sub-steps per K step), which the
// rest of this comment describes where the two differ.  A 4-wave variant
// (128 x 128 per wave, accumulators in AGPRs) is kept behind MATOPT_*_WAVES.
// The
// K loop runs in steps of 32 through NS = 5 LDS stages of 32 KB (one 256 x 32
// tile per operand), filled by global_load_lds_dwordx4 (HBM -> LDS without
// registers) three steps ahead of use, in the layout the tile has in HBM.
// MFMA fragments come from ds_read_b128 (row-major) or from two
// ds_read_b64_tr_b16 (k-major: the LDS transpose read hands lane i of each
// 16-lane group element i & 3 of the 64-bit chunks addressed by lanes
// 4e + (i >> 2), e = 0..3).  Both layouts are XOR-swizzled so that the 16
// lanes of a 16-byte access or the 32 lanes of an 8-byte access hit distinct
// LDS banks (64 banks of 4 B); the DMA lanes pick their source addresses to
// realise the swizzle.
//
// One barrier per K step, placed between its two k16 sub-steps (on the 16 x
// 16 x 32 engine: between the step's two halves of MFMAs): before it each
// wave waits for its own DMA of the next step (explicit vmcnt), after it the
// DMA of a step three ahead is issued into the stage everyone has finished
// with.  The fragment reads of the next sub-step are interleaved with the
// MFMAs of the current one (explicit scheduling groups).  Apply pairs the DMA
// of consecutive K steps (kloop2) so that the two 64-byte halves of each
// 128-byte line of its row-major B rows are fetched from L2 once.
//
// Diagonal tiles (ti == tj) of the Gram and the polynomial compute only the 36
// of their 64 32 x 32 blocks on and above the diagonal, from one operand
// panel, 9 MFMAs per SIMD and k16 sub-step instead of 16, and write the blocks
// above the diagonal twice (diag_tile; the Gram's diagonal pairs, diag_pair16,
// also skip the lower 16 x 16 slab of blocks on the diagonal).
//
// Epilogue: the last apply (which writes the caller's orientation) stages
// each wave's accumulators through its own LDS region (float32) so that every
// global store is a contiguous row segment.  The Gram, the polynomial and a
// non-final apply skip the staging: their accumulators go straight to whole
// 2 KB blocks of A, B or X' with lane swaps across 16-lane groups
// (v_permlane16_swap; v_permlane32_swap on the 32 x 32 x 16 form), the
// polynomial reading A at the lanes' own output positions;
// where every tile of the non-final apply has the same K extent, that launch
// runs persistent (one workgroup per CU) and issues the next tile's DMA
// before these stores.  On the last iteration the result is
// written in the original orientation as O, or folded straight into
// W <- W - lr*sqrt(max(1,rows/cols))*O (so O never round-trips through HBM).
//
// Roofline: a dense contraction; algorithmic flops per tile are 2*256*256*K
// (K = n for stage 0, m for stages 1 and 2).  Bound: bf16 MFMA peak.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "device_util.hpp"

// K loop DMA schedule per stage: 1 pairs the loads of consecutive K steps
// (kloop2), 0 spreads each step's DMA over two steps (kloop).  Pairing halves
// the L1 -> L2 line requests of an operand read row-major from a plain
// row-major matrix but shortens some prefetch distances.  On the GPT-2 Large
// set the Gram (whose first iteration reads X0 plain) is 9% slower with it;
// with A and B stored in 32 x 32 blocks every load covers whole lines anyway,
// and the polynomial runs 2.4% faster spread, apply 0.7% faster paired.
#ifndef MATOPT_PAIR_GRAM
#define MATOPT_PAIR_GRAM 0
#endif
#ifndef MATOPT_PAIR_POLY
#define MATOPT_PAIR_POLY 0
#endif
#ifndef MATOPT_PAIR_APPLY
#define MATOPT_PAIR_APPLY 1
#endif
// Stages on the 16 x 16 x 32 engine (1) or on 32 x 32 x 16 MFMAs (0): apply,
// and the off-diagonal tiles of the Gram and the polynomial.
#ifndef MATOPT_APPLY_MFMA16
#define MATOPT_APPLY_MFMA16 1
#endif
#ifndef MATOPT_GRAM_MFMA16
#define MATOPT_GRAM_MFMA16 1
#endif
#ifndef MATOPT_POLY_MFMA16
#define MATOPT_POLY_MFMA16 1
#endif
// Diagonal Gram and polynomial tiles compute only their upper 36 of 64 blocks.
#ifndef MATOPT_DIAG_TILES
#define MATOPT_DIAG_TILES 1
#endif

namespace matopt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define MATOPT_LDS __attribute__((address_space(3)))

constexpr int BM = 256;               // tile rows == tile cols == symmetric block
constexpr int BK = 32;                // K step
constexpr int NS = 5;                 // LDS stages
constexpr int OPB = BM * BK * 2;      // bytes of one operand tile (16 KB)
constexpr int STG = 2 * OPB;          // one stage: P then Q (32 KB)
constexpr int LDS_BYTES = NS * STG;   // 160 KB
// Epilogue geometry of a wave whose sub-tile is 128 rows x WN columns (WN =
// 128 with four waves, 64 with eight): staging rows of WN + 4 floats, LPR
// lanes per staged row, IPL 8-column items per lane and 32-row stripe.
template <int WN>
struct Ep {
  static constexpr int PITCH = WN + 4;
  static constexpr int LPR = WN / 8;
  static constexpr int IPL = WN / 16;
  static constexpr int RPI = 64 / LPR;   // rows between a lane's items
  // float offset of staged row r: rows 16-31 sit 16 floats (banks) further on,
  // so that the eight rows of a transposed read (rows 8i + e, i = 0..3) that
  // 32 lanes touch together spread over all 64 banks
  __device__ static constexpr int row(int r) { return r * PITCH + 16 * (r >> 4); }
  static constexpr int WAVE_BYTES = (32 * PITCH + 16) * 4;
};
static_assert(4 * Ep<128>::WAVE_BYTES <= LDS_BYTES && 8 * Ep<64>::WAVE_BYTES <= LDS_BYTES,
              "epilogue staging must fit");

// ---------------------------------------------------------------- LDS layouts
// Row-major tile: 256 rows x 32 k = 64-byte rows of four 16-byte chunks; the
// chunk index is XORed with (row >> 2) & 3.  Sixteen consecutive rows at one
// logical chunk (an MFMA fragment read) land on 16 distinct bank groups.
__device__ __forceinline__ uint32_t rm_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ ((row >> 2) & 3u)) << 4);
}

// k-major tile: 32 k rows x 256 operand rows = 512-byte k rows of eight 64-byte
// units; the unit index is XORed with (k & 3).  Four consecutive k rows at one
// logical unit land in the four distinct 64-byte bank quarters.
__device__ __forceinline__ uint32_t km_off(uint32_t k, uint32_t col) {
  return k * 512u + ((((col >> 5) ^ (k & 3u)) & 7u) << 6) + ((col & 31u) << 1);
}

// DMA of one operand tile for one K step (k0..k0+31), 4 instructions per wave.
// Each instruction writes 1 KB of LDS at dst + 16*lane; lane L therefore loads
// the 16 source bytes that belong at that (swizzled) position.
//   row-major: block b covers rows 16b..16b+15; lane L -> row 16b + L/4,
//              logical chunk (L & 3) ^ ((L >> 4) & 3).
//   k-major:   block b covers k rows 2b, 2b+1; lane L -> k row 2b + L/32, unit
//              ((L & 31) >> 2) ^ ((2b + L/32) & 3), 16-byte piece L & 3.
// Addresses are a wave-uniform 64-bit base plus a 32-bit lane offset relative
// to the tile origin (so that the load takes its base from scalar registers).
// Operand read modes over the K loop: always row-major, always k-major, or
// k-major for the steps left of the operand's diagonal block (t < t_km, read
// from the mirrored upper tile of a symmetric matrix) and row-major after.
enum OpKind { OP_RM = 0, OP_KM = 1, OP_SPLIT = 2 };

// Item q of a mirror (transposed) read of a staged block (32 rows, pitch 36
// floats: eight rows span 32 banks) whose result goes to a blocked workspace
// matrix (the diagonal tiles' blocks above the diagonal): staged
// column jj = tr_jj(q), rows 8 ic .. 8 ic + 7 with ic = tr_ic(q).  The 16
// lanes of a quarter-wave take one ic and 16 consecutive columns, so each of
// their 4-byte reads meets a distinct bank (with ic = q & 3, lanes with ic and
// ic+2 share one); a store instruction still writes whole 64-byte block rows.
__device__ __forceinline__ int tr_ic(int q) { return (q >> 4) & 3; }
__device__ __forceinline__ int tr_jj(int q) { return (q & 15) + 16 * (q >> 6); }

// The workspace matrices -- the iterates X after the first iteration, A and B
// -- are stored in 32 x 32 blocks of 2 KB, row-major inside and in the block
// grid, so that every operand load of a K step (16 rows x 64 B, or 2 k rows
// of 8 column units) and every 16-byte epilogue item stays within whole
// 128-byte lines of one block.  Address of element (r, c) of such a matrix
// with ld columns (r, c, ld multiples of 32 where blocks start).
template <class Ptr>
__device__ __forceinline__ Ptr blk_at(Ptr base, int64_t r, int64_t c, int64_t ld) {
  const int64_t off = (((r >> 5) * (ld >> 5) + (c >> 5)) << 11) + ((r & 31) << 6) + ((c & 31) << 1);
  return reinterpret_cast<Ptr>(reinterpret_cast<uintptr_t>(base) + off);
}

template <int KIND>
struct OperandDma {
  const char* org_rm;   // byte address of the row-major origin (row r0)
  const char* org_km;   // byte address of the k-major origin (column r0)
  uint32_t rs;          // bytes between consecutive rows (k rows) as addressed
  uint32_t us;          // bytes between 32-column units (k-major)
  int64_t rm_b2, rm_b1; // row-major block b: (b >> 1) * rm_b2 + (b & 1) * rm_b1
  int64_t rm_t, km_t;   // bytes per K step, row-major / k-major
  uint32_t off_rm;      // lane offset of row-major blocks
  uint32_t off_km0;     // lane offset of k-major blocks with b even
  uint32_t off_km1;     // lane offset of k-major blocks with b odd
  int t_km;             // steps t < t_km are k-major
  int t_wrap;           // step t reads K step t - t_wrap from t_wrap on (the
                        // split-precision apply reads B twice)

  // Plain: src is a row-major matrix with ld elements per row.  Blocked: src
  // is an iterate X stored in 32 x 32 blocks (2 KB each, row-major inside,
  // ld/32 blocks per block row), so that a row-major block (16 rows x 64 B)
  // is 1 KB of one block and a k-major block (2 k rows x 8 units) is eight
  // whole 128-byte lines (the two 64-byte rows of each unit are adjacent).
  __device__ void init(const uint16_t* src, int64_t ld, int r0, int tkm, int lane,
                       bool blocked = false) {
    t_km = tkm;
    t_wrap = 1 << 30;
    if (!blocked) {
      rs = (uint32_t)(ld * 2);
      us = 64u;
      rm_b2 = 32 * (int64_t)rs;
      rm_b1 = 16 * (int64_t)rs;
      rm_t = BK * 2;
      km_t = BK * (int64_t)rs;
      org_rm = (const char*)(src + (int64_t)r0 * ld);
      org_km = (const char*)(src + r0);
    } else {
      const int64_t blkrow = (ld / 32) * 2048;   // bytes per block row
      rs = 64u;
      us = 2048u;
      rm_b2 = blkrow;
      rm_b1 = 1024;
      rm_t = 2048;
      km_t = blkrow;
      org_rm = (const char*)src + (int64_t)(r0 / 32) * blkrow;
      org_km = (const char*)src + (int64_t)(r0 / 32) * 2048;
    }
    off_rm = (uint32_t)(lane >> 2) * rs + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    // (2b + L/32) & 3 is L/32 for even b and 2 + L/32 for odd b
    const uint32_t lo = (uint32_t)(lane >> 5) * rs + 16u * (lane & 3);
    off_km0 = lo + us * (((lane & 31) >> 2) ^ (lane >> 5));
    off_km1 = lo + us * (((lane & 31) >> 2) ^ (2 + (lane >> 5)));
  }

  __device__ __forceinline__ bool is_km(int t) const {
    return KIND == OP_KM || (KIND == OP_SPLIT && t < t_km);
  }

  template <int Q, int BPW>
  __device__ __forceinline__ void block(bool km, int t, uint8_t* tile, int wave) const {
    const int b = BPW * wave + Q;   // parity of b is that of Q (BPW is even)
    t = t >= t_wrap ? t - t_wrap : t;   // uniform
    const char* base = km ? org_km + t * km_t + 2 * b * (int64_t)rs
                          : org_rm + (b >> 1) * rm_b2 + (b & 1) * rm_b1 + t * rm_t;   // uniform
    const uint32_t kmoff = (Q & 1) ? off_km1 : off_km0;
    // per-lane offset chosen arithmetically (km is uniform)
    const uint32_t off = off_rm ^ ((off_rm ^ kmoff) & (km ? 0xffffffffu : 0u));
    __builtin_amdgcn_global_load_lds((const MATOPT_GAS void*)(base + off),
                                     (MATOPT_LDS void*)(tile + 1024 * b), 16, 0, 0);
  }

  // BPW blocks per wave (4 with four waves, 2 with eight): block b = BPW*wave + q
  template <int BPW = 4>
  __device__ __forceinline__ void issue(int t, uint8_t* tile, int wave) const {
    const bool km = is_km(t);
    block<0, BPW>(km, t, tile, wave);
    block<1, BPW>(km, t, tile, wave);
    if (BPW == 4) {
      block<2, BPW>(km, t, tile, wave);
      block<3, BPW>(km, t, tile, wave);
    }
  }
};

// Per-lane LDS offsets of the MFMA fragments (relative to the wave's operand
// row origin inside an operand tile).  A fragment covers 32 operand rows and a
// k16 sub-step kk: lane l holds row (l & 31), k = 16kk + 8(l >> 5) .. +7.
//   row-major: one ds_read_b128 at rm_off(row, 2kk + (l >> 5)); the 32-row
//              block bb adds 2048*bb (the swizzle depends on row & 12 only).
//   k-major:   two ds_read_b64_tr_b16.  16-lane group G covers rows
//              16(G & 1) .. +15 and k rows 16kk + 8(G >> 1) .. +7; lane c = 4e + h
//              of the group points at k row (.. + e) and rows +4h .. +4h+3 (and
//              k row + 4 for the second read), so lane c receives row +c at 4
//              consecutive k.  The unit swizzle (bb ^ e) differs per lane and
//              block, hence one offset per block; kk and the second read are
//              immediates (8192*kk, 2048).
struct FragOffsets {
  uint32_t rm[2];   // by kk
  uint32_t km[4];   // by block bb (kk = 0, first read)
  uint32_t kmq[2];  // eight-wave layout: Q blocks of the wave, origin included
  __device__ void init(int lane) {
    const int r = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) rm[kk] = rm_off(r, 2 * kk + hi);
    const int G = lane >> 4, c = lane & 15, e = c >> 2, h = c & 3;
    const int kr = 8 * (G >> 1) + e;
    const int col = 16 * (G & 1) + 4 * h;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) km[bb] = kr * 512 + ((bb ^ e) << 6) + 2 * col;
  }
  // Q columns from wq0 (a multiple of 64): block BB = wq0/32 + bb of the tile,
  // whose unit swizzle (BB ^ e) & 7 can carry into bit 2 of BB
  __device__ void init_q64(int lane, int wq0) {
    const int G = lane >> 4, c = lane & 15, e = c >> 2, h = c & 3;
    const int kr = 8 * (G >> 1) + e;
    const int col = 16 * (G & 1) + 4 * h;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
      kmq[bb] = kr * 512 + ((((wq0 >> 5) + bb) ^ e) & 7) * 64 + 2 * col;
  }
};

template <bool KM>
__device__ __forceinline__ bf16x8 frag(const uint8_t* tile, int wo, int bb, int kk,
                                       const FragOffsets& fo) {
  if (!KM) {
    return *(const bf16x8*)(tile + wo * 64 + 2048 * bb + fo.rm[kk]);
  } else {
    // wo is a multiple of 128: its unit bits (wo >> 5) never meet the swizzle
    const uint8_t* base = tile + (wo >> 5) * 64 + fo.km[bb] + 8192 * kk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base + 2048));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

struct WaveGeo {
  int wi0, wj0, frow, fkc;
};

template <bool PKM, bool QKM, int NBJ>
__device__ __forceinline__ void read_frags(const uint8_t* stage, int kk, const WaveGeo& g,
                                           const FragOffsets& fo, bf16x8 (&p)[4],
                                           bf16x8 (&q)[NBJ]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) p[bi] = frag<PKM>(stage, g.wi0, bi, kk, fo);
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
    if (NBJ == 4 || !QKM) {
      q[bj] = frag<QKM>(stage + OPB, g.wj0, bj, kk, fo);
    } else {   // eight-wave layout, k-major Q
      const uint8_t* base = stage + OPB + fo.kmq[bj] + 8192 * kk;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base + 2048));
      q[bj] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
}

// 16 MFMAs of one k16 sub-step (operands swapped: acc[bi][bj] holds C^T blocks,
// i.e. 4 consecutive output columns per register group).
template <int NBJ>
__device__ __forceinline__ void mfma16(f32x16 (&acc)[4][NBJ], const bf16x8 (&p)[4],
                                       const bf16x8 (&q)[NBJ]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[bj], p[bi], acc[bi][bj], 0, 0, 0);
}

// Wait until at most N DMA instructions of this wave are still in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence (a fence would wait for every DMA
// in flight); LDS ordering is explicit through wait_vm and the K-step
// structure.
__device__ __forceinline__ void bar_raw() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int SG_MFMA = 0x008;
constexpr int SG_VMEM_RD = 0x020;
constexpr int SG_DS_RD = 0x100;

template <int WN>
__device__ __forceinline__ void prefetch_stripe(const uint16_t* src, int64_t ld, int64_t row0,
                                                int64_t col0, int lane,
                                                u32x4 (&dst)[Ep<WN>::IPL]) {
  // lane q = lane + 64p reads row row0 + q/LPR, columns col0 + 8(q % LPR) .. +7;
  // item p starts RPI*p rows down (byte offsets)
  // (src in 32 x 32 blocks)
  using G = Ep<WN>;
#pragma unroll
  for (int p = 0; p < G::IPL; ++p)
    dst[p] = gload<u32x4>(blk_at(src, row0 + lane / G::LPR + G::RPI * p,
                                 col0 + (lane % G::LPR) * 8, ld));
}

// Stage acc[BI][*] (32 rows of the wave's 128 x 128 sub-tile) into the wave's
// LDS region as float32 rows.  acc[BI][bj][r] holds
//   C[32BI + (lane & 31)][32bj + 8(r>>2) + 4(lane>>5) + (r&3)]   (wave-local)
// (operands swapped in the MFMA, so 4 consecutive columns per register group).
template <int BI, int NBJ>
__device__ __forceinline__ void stage_stripe(const f32x16 (&acc)[4][NBJ], float* stg, int frow,
                                             int fkc) {
  using G = Ep<32 * NBJ>;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = {acc[BI][bj][4 * g], acc[BI][bj][4 * g + 1], acc[BI][bj][4 * g + 2],
                       acc[BI][bj][4 * g + 3]};
      *(f32x4*)(stg + G::row(frow) + 32 * bj + 8 * g + 4 * fkc) = v;
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
      float u[4];
      w_update_f32_n<4>(w4, upd, v, P.wdl, u);
      gstore<u32x2>(w, u32x2{pack_bf2(u[0], u[1]), pack_bf2(u[2], u[3])});
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
      gstore<uint16_t>(w, (uint16_t)w_update_bf16(wo, upd, v[e], P.wdl));
    }
  }
}

// Last-iteration output of one staged stripe (rows ib .. ib+31 of the X
// orientation, the wave's WN columns from j0), in the original orientation:
// item p of lane q = lane + 64p covers 8 consecutive original columns of one
// original row -- row ib + q/LPR, columns j0 + 8(q % LPR) when not transposed;
// row j0 + q/4, columns ib + 8(q & 3) when transposed.  The staged values are
// scaled by s (the Frobenius scale when this is also the first iteration, else
// 1) as they are read.  Stripes that lie wholly inside a matrix with 16-byte
// rows take an unrolled path with 16-byte accesses, the stripe's W chunks
// per lane all read before the first is used; others a rolled per-item path.
template <int OUT, bool TRANS, int WN>
__device__ __forceinline__ void final_pass(const MatDesc& d, const GemmParams& P, const float* stg,
                                           int64_t ib, int64_t j0, int lane, float upd,
                                           float s) {
  using G = Ep<WN>;
  const int64_t rows = d.rows, cols = d.cols;
  const bool full = d.vec_ok && (TRANS ? (j0 + WN <= rows && ib + 32 <= cols)
                                       : (ib + 32 <= rows && j0 + WN <= cols));
  auto item = [&](int p, int64_t& r, int64_t& c, float (&lo)[4], float (&hi)[4]) {
    const int q = lane + 64 * p;
    if (!TRANS) {
      // with 16 lanes per row, lanes 8-15 read the two halves in the other
      // order (LDS banks); with 8, consecutive rows already meet other banks
      const int rr = q / G::LPR, c8 = (q % G::LPR) * 8;
      r = ib + rr;
      c = j0 + c8;
      const bool hs = G::LPR == 16 && (q & 8) != 0;
      const float* src = stg + G::row(rr) + c8;
      const f32x4 r0 = *(const f32x4*)(src + (hs ? 4 : 0));
      const f32x4 r1 = *(const f32x4*)(src + (hs ? 0 : 4));
      const f32x4 v0 = hs ? r1 : r0, v1 = hs ? r0 : r1;
      lo[0] = s * v0.x; lo[1] = s * v0.y; lo[2] = s * v0.z; lo[3] = s * v0.w;
      hi[0] = s * v1.x; hi[1] = s * v1.y; hi[2] = s * v1.z; hi[3] = s * v1.w;
    } else {
      // four consecutive lanes per output row: each quarter-wave reads or
      // writes four 64-byte row segments of the caller's W / O (the row skew
      // of the staging keeps these column reads free of bank conflicts)
      const int ic = q & 3, jj = q >> 2;
      r = j0 + jj;
      c = ib + 8 * ic;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = s * stg[G::row(8 * ic + e) + jj];
        hi[e] = s * stg[G::row(8 * ic + 4 + e) + jj];
      }
    }
  };
  if (full) {
    u32x4 wpre[G::IPL];
    if (OUT == OUT_W_UPDATE) {
#pragma unroll
      for (int p = 0; p < G::IPL; ++p) {
        const int q = lane + 64 * p;
        const int64_t r = TRANS ? j0 + (q >> 2) : ib + q / G::LPR;
        const int64_t c = TRANS ? ib + 8 * (q & 3) : j0 + (q % G::LPR) * 8;
        wpre[p] = gload<u32x4>((const uint16_t*)d.w + r * cols + c);
      }
    }
#pragma unroll
    for (int p = 0; p < G::IPL; ++p) {
      int64_t r, c;
      float lo[4], hi[4];
      item(p, r, c, lo, hi);
      const int64_t off = r * cols + c;
      if (OUT == OUT_O) {
        if (P.out_dt == DT_F32) {
          gstore<f32x4>((float*)d.o + off, f32x4{lo[0], lo[1], lo[2], lo[3]});
          gstore<f32x4>((float*)d.o + off + 4, f32x4{hi[0], hi[1], hi[2], hi[3]});
        } else {
          gstore<u32x4>((uint16_t*)d.o + off, u32x4{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]),
                                                     pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])});
        }
      } else {
        const u32x4 wo = wpre[p];
        const float w8[8] = {lo_bf(wo.x), hi_bf(wo.x), lo_bf(wo.y), hi_bf(wo.y),
                             lo_bf(wo.z), hi_bf(wo.z), lo_bf(wo.w), hi_bf(wo.w)};
        const float o8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        float u[8];
        w_update_f32_n<8>(w8, upd, o8, P.wdl, u);
        gstore<u32x4>((uint16_t*)d.w + off, u32x4{pack_bf2(u[0], u[1]), pack_bf2(u[2], u[3]),
                                                  pack_bf2(u[4], u[5]), pack_bf2(u[6], u[7])});
      }
    }
  } else {
#pragma unroll 1
    for (int p = 0; p < G::IPL; ++p) {
      int64_t r, c;
      float lo[4], hi[4];
      item(p, r, c, lo, hi);
      if (r >= rows) continue;
      if (c < cols) write_out4<OUT>(d, P, r, c, lo, upd);
      if (c + 4 < cols) write_out4<OUT>(d, P, r, c + 4, hi, upd);
    }
  }
}

// Apply before the last iteration: the wave's sub-tile goes straight from the
// accumulators to the next iterate in HBM, without LDS staging; each 32 x 32
// block is one 2 KB block of the iterate's blocked layout.  Register group g of
// acc[bi][bj] holds, for row 32bi + (lane & 31), columns 32bj + 8g + 4(lane>>5)
// + 0..3.  After packing to bf16, one v_permlane32_swap per packed register
// trades group 1 of the low half-wave for group 0 of the high half (and group 3
// for group 2): lane l then holds columns 32bj + 8(lane>>5) + 16h + 0..7 for
// h = 0, 1 -- two 16-byte stores per block and lane, the pair of instructions
// writing the whole 2 KB block.
// The 16 values v of one accumulator block of a lane (v[4g + e] at row
// (lane & 31), column 8g + 4(lane >> 5) + e of the block), packed to bf16 and
// stored through the lane swaps above into the 2 KB block at blk (row-major
// inside, this lane's row and column offset already added).
__device__ __forceinline__ void store_block_direct(const float (&v)[16], uint16_t* blk) {
  uint32_t pk[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    pk[g][0] = pack_bf2(v[4 * g], v[4 * g + 1]);
    pk[g][1] = pack_bf2(v[4 * g + 2], v[4 * g + 3]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(pk[2 * h][k], pk[2 * h + 1][k], false, false);
      pk[2 * h][k] = r[0];
      pk[2 * h + 1][k] = r[1];
    }
  gstore<u32x4>(blk, u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]});
  gstore<u32x4>(blk + 16, u32x4{pk[2][0], pk[2][1], pk[3][0], pk[3][1]});
}

template <int NBJ>
__device__ __forceinline__ void store_acc_direct(const f32x16 (&acc)[4][NBJ], uint16_t* out,
                                                 int64_t ld, int64_t i0, int64_t j0, int lane,
                                                 float s) {
  // out is stored in 32 x 32 blocks (see OperandDma): block (bi, bj) of the
  // wave is the 2 KB block ((i0 >> 5) + bi, (j0 >> 5) + bj), row-major inside
  const int64_t nb = ld / 32;
  uint16_t* base = out + ((i0 >> 5) * nb + (j0 >> 5)) * 1024 + (lane & 31) * 32 + 8 * (lane >> 5);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = s * acc[bi][bj][r];
      store_block_direct(v, base + (bi * nb + bj) * 1024);
    }
}

// The split-precision iterate (GemmParams::split): the high part bf16(v) as
// store_acc_direct writes it, and the low part bf16(v - bf16(v)) -- v - bf16(v)
// is exact in float32 -- at the same position of the matrix stacked below
// (lo_off elements further on), so that hi + lo carries about 16 bits.
// v = s * a rounded to float32, and lo = v - bf16(v), exact in float32.  No
// contraction: fused as fma(s, a, -bf16(v)) the low part would carry the
// product's own rounding error on some paths and not on others.
__device__ __forceinline__ void split_parts(const f32x16& a, float s, float (&v)[16],
                                            float (&lo)[16]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    v[r] = s * a[r];
    lo[r] = v[r] - bf2f(f2bf(v[r]));
  }
}

template <int NBJ>
__device__ __forceinline__ void store_acc_direct_split(const f32x16 (&acc)[4][NBJ], uint16_t* out,
                                                       int64_t ld, int64_t i0, int64_t j0,
                                                       int lane, float s, int64_t lo_off) {
  const int64_t nb = ld / 32;
  uint16_t* base = out + ((i0 >> 5) * nb + (j0 >> 5)) * 1024 + (lane & 31) * 32 + 8 * (lane >> 5);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj) {
      float v[16], lo[16];
      split_parts(acc[bi][bj], s, v, lo);
      store_block_direct(v, base + (bi * nb + bj) * 1024);
      store_block_direct(lo, base + lo_off + (bi * nb + bj) * 1024);
    }
}

// The polynomial's epilogue, straight from the accumulators as well (B has no
// mirror): B = a I + b A + c (A A) with the A values read at the lanes' own
// accumulator positions (8 bytes per register group), one 32-row stripe of
// blocks ahead; a_first holds stripe 0, read during the last K step.
template <int NBJ>
__device__ __forceinline__ void poly_a_stripe(const uint16_t* A, int64_t ld, int64_t r0,
                                              int64_t j0, int lane, u32x2 (&dst)[NBJ][4]) {
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      dst[bj][g] = gload<u32x2>(blk_at(A, r0 + (lane & 31), j0 + 32 * bj + 8 * g + 4 * (lane >> 5), ld));
}

template <int NBJ>
__device__ __forceinline__ void poly_store_direct(const f32x16 (&acc)[4][NBJ], uint16_t* out,
                                                  const uint16_t* A, int64_t ld, int64_t i0,
                                                  int64_t j0, int lane, float a, float b, float c,
                                                  const u32x2 (&a_first)[NBJ][4]) {
  const int64_t nb = ld / 32;
  uint16_t* base = out + ((i0 >> 5) * nb + (j0 >> 5)) * 1024 + (lane & 31) * 32 + 8 * (lane >> 5);
  u32x2 ac[NBJ][4], an[NBJ][4];
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
    for (int g = 0; g < 4; ++g) ac[bj][g] = a_first[bj][g];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    if (bi + 1 < 4) poly_a_stripe<NBJ>(A, ld, i0 + 32 * (bi + 1), j0, lane, an);
    const int64_t row = i0 + 32 * bi + (lane & 31);
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj) {
      float v[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = j0 + 32 * bj + 8 * g + 4 * (lane >> 5);
        const float av[4] = {lo_bf(ac[bj][g].x), hi_bf(ac[bj][g].x), lo_bf(ac[bj][g].y),
                             hi_bf(ac[bj][g].y)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[4 * g + e] = fmaf(b, av[e], fmaf(c, acc[bi][bj][4 * g + e], row == col + e ? a : 0.f));
      }
      store_block_direct(v, base + (bi * nb + bj) * 1024);
    }
    if (bi + 1 < 4) {
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
        for (int g = 0; g < 4; ++g) ac[bj][g] = an[bj][g];
    }
  }
}

// Epilogue of one wave's 128 x WN sub-tile, one 32-row stripe at a time (a
// rolled loop: only the accumulator staging is specialised per stripe, which
// keeps the kernel small enough for the instruction cache).  Each stripe is
// staged through the wave's own LDS region (LDS executes one wave's accesses in
// order, so no workgroup barrier is needed) and written row-wise: WN/16 chunks
// of 8 consecutive columns (16-byte stores) per lane.  The polynomial's epilogue input (the A tile
// of the same position) is prefetched one stripe ahead; Gram and apply read
// nothing back.
// Staging of stripe BI of a 32 x 32 x 16 layout sub-tile (stage_stripe).
template <int NBJ>
struct Stage32 {
  const f32x16 (&acc)[4][NBJ];
  int frow, fkc;
  template <int BI>
  __device__ __forceinline__ void stage(float* stg) const {
    stage_stripe<BI, NBJ>(acc, stg, frow, fkc);
  }
};

template <int STAGE, int OUT, int NBJ, bool MIRROR, class Stager>
__device__ __forceinline__ void epilogue_staged(const MatDesc& d, const GemmParams& P,
                                                const Stager& st, float* stg,
                                                const uint16_t* ep_src, int64_t ep_ld,
                                                uint16_t* out, int64_t ld_out, int i0, int j0,
                                                int lane, float s_first,
                                                u32x4 (&ecur)[Ep<32 * NBJ>::IPL]);

template <int STAGE, int OUT, int NBJ, bool MIRROR = false>
__device__ __forceinline__ void epilogue(const MatDesc& d, const GemmParams& P,
                                         const f32x16 (&acc)[4][NBJ], float* stg,
                                         const uint16_t* ep_src, int64_t ep_ld, uint16_t* out,
                                         int64_t ld_out, int i0, int j0, int lane, int frow,
                                         int fkc, float s_first,
                                         u32x4 (&ecur)[Ep<32 * NBJ>::IPL]) {
  const Stage32<NBJ> st{acc, frow, fkc};
  epilogue_staged<STAGE, OUT, NBJ, MIRROR>(d, P, st, stg, ep_src, ep_ld, out, ld_out, i0, j0,
                                           lane, s_first, ecur);
}

// The staged epilogue for any accumulator layout: Stager::stage<BI>(stg)
// writes stripe BI (rows 32 BI .. +31 of the wave's sub-tile) as float32 rows
// of Ep<32 NBJ> into the wave's LDS region.
template <int STAGE, int OUT, int NBJ, bool MIRROR, class Stager>
__device__ __forceinline__ void epilogue_staged(const MatDesc& d, const GemmParams& P,
                                                const Stager& st, float* stg,
                                                const uint16_t* ep_src, int64_t ep_ld,
                                                uint16_t* out, int64_t ld_out, int i0, int j0,
                                                int lane, float s_first,
                                                u32x4 (&ecur)[Ep<32 * NBJ>::IPL]) {
  constexpr int WN = 32 * NBJ;
  using G = Ep<WN>;
  static_assert(STAGE != 0, "the Gram stores its tiles from the accumulators");
  constexpr bool EP_IN = STAGE == 1;
  const bool out_trans = OUT != OUT_NEXT_X && d.transposed;
  const float upd = -P.lr * d.upd_scale;
  u32x4 enext[G::IPL];
#pragma unroll 1
  for (int bi = 0; bi < 4; ++bi) {
    if (EP_IN && bi + 1 < 4)
      prefetch_stripe<WN>(ep_src, ep_ld, i0 + 32 * (bi + 1), j0, lane, enext);
    switch (bi) {
      case 0: st.template stage<0>(stg); break;
      case 1: st.template stage<1>(stg); break;
      case 2: st.template stage<2>(stg); break;
      default: st.template stage<3>(stg); break;
    }
    __builtin_amdgcn_wave_barrier();

    const int64_t ib = i0 + 32 * bi;   // first X-orientation row of this stripe
    if (STAGE != 2 || OUT == OUT_NEXT_X) {
      // Polynomial and non-final apply (four-wave builds): 8 consecutive columns (one
      // 16-byte store) per lane item.  With 16 lanes per row, lanes 8-15 read
      // their two float4 halves in the other order so that the 16 lanes of a
      // row meet distinct LDS banks.
      const float sc = s_first;
#pragma unroll
      for (int p = 0; p < G::IPL; ++p) {
        const int q = lane + 64 * p;
        const int rr = q / G::LPR, c8 = (q % G::LPR) * 8;
        const bool hs = G::LPR == 16 && (q & 8) != 0;
        float* src = stg + G::row(rr) + c8;
        const f32x4 r0 = *(const f32x4*)(src + (hs ? 4 : 0));
        const f32x4 r1 = *(const f32x4*)(src + (hs ? 0 : 4));
        const f32x4 v0 = hs ? r1 : r0, v1 = hs ? r0 : r1;
        f32x4 a0, a1;
        if (STAGE == 1) {
          // a*I + b*A + c*(A A): a on the diagonal (global row i == column j)
          const u32x4 ain = ecur[p];
          const float a = P.a, b = P.b, c = P.c;
          const int64_t dg = (ib + rr) - (j0 + c8);
          a0 = f32x4{fmaf(b, lo_bf(ain.x), fmaf(c, v0.x, dg == 0 ? a : 0.f)),
                     fmaf(b, hi_bf(ain.x), fmaf(c, v0.y, dg == 1 ? a : 0.f)),
                     fmaf(b, lo_bf(ain.y), fmaf(c, v0.z, dg == 2 ? a : 0.f)),
                     fmaf(b, hi_bf(ain.y), fmaf(c, v0.w, dg == 3 ? a : 0.f))};
          a1 = f32x4{fmaf(b, lo_bf(ain.z), fmaf(c, v1.x, dg == 4 ? a : 0.f)),
                     fmaf(b, hi_bf(ain.z), fmaf(c, v1.y, dg == 5 ? a : 0.f)),
                     fmaf(b, lo_bf(ain.w), fmaf(c, v1.z, dg == 6 ? a : 0.f)),
                     fmaf(b, hi_bf(ain.w), fmaf(c, v1.w, dg == 7 ? a : 0.f))};
        } else {
          a0 = f32x4{v0.x * sc, v0.y * sc, v0.z * sc, v0.w * sc};
          a1 = f32x4{v1.x * sc, v1.y * sc, v1.z * sc, v1.w * sc};
        }
        gstore<u32x4>(blk_at(out, ib + rr, j0 + c8, ld_out),
                      u32x4{pack_bf2(a0.x, a0.y), pack_bf2(a0.z, a0.w), pack_bf2(a1.x, a1.y),
                            pack_bf2(a1.z, a1.w)});
        if (MIRROR) {   // the mirror pass reads the final values (each lane its own items)
          *(f32x4*)src = a0;
          *(f32x4*)(src + 4) = a1;
        }
      }
      if (MIRROR) {
        // B stored whole (split precision): the stripe transposed into the
        // mirror tile -- row j0 + jj, columns ib + 8 ic .. +7 (four lanes per
        // row, as the transposed final pass reads the staging)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < G::IPL; ++p) {
          const int q = lane + 64 * p;
          const int ic = q & 3, jj = q >> 2;
          float vv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = stg[G::row(8 * ic + e) + jj];
          gstore<u32x4>(blk_at(out, j0 + jj, ib + 8 * ic, ld_out),
                        u32x4{pack_bf2(vv[0], vv[1]), pack_bf2(vv[2], vv[3]),
                              pack_bf2(vv[4], vv[5]), pack_bf2(vv[6], vv[7])});
        }
      }
    }
    if (OUT != OUT_NEXT_X) {
      __builtin_amdgcn_wave_barrier();
      if (out_trans) final_pass<OUT, true, WN>(d, P, stg, ib, j0, lane, upd, s_first);
      else final_pass<OUT, false, WN>(d, P, stg, ib, j0, lane, upd, s_first);
    }
    __builtin_amdgcn_wave_barrier();
    if (EP_IN) {
#pragma unroll
      for (int p = 0; p < G::IPL; ++p) ecur[p] = enext[p];
    }
  }
}

// One K step t (not the last).  Sub-step 0 runs on fragments read earlier
// while the sub-step-1 fragments of step t are read and (DQ) the Q half of the
// DMA of step t+NS-2 is issued into the stage of step t-2; then the wave waits
// for its DMA of step t+1, meets the other waves, and runs sub-step 1 while the
// sub-step-0 fragments of step t+1 are read and (DP) the P half of the DMA of
// step t+NS-1 is issued into the stage of step t-1.  Splitting each step's DMA
// over both halves keeps the address unit's queue short, so a DMA instruction
// never holds up the MFMAs behind it.  VMW is the vmcnt that leaves in flight
// only the DMA issued after that of step t+1.  (P0, Q0) are the operand
// layouts of step t, (P1, Q1) those of step t+1 (true: k-major).
//
// The stage pointers name distinct stages (NS >= 4); declaring them restrict
// tells the compiler that these fragment reads never alias the DMA written
// here, so it adds no wait of its own for the DMA before an LDS read.  No
// LDS-read wait is needed before the barrier either: every read of step t-1's
// stage was consumed by an MFMA of step t-1, before this point.
template <bool P0, bool Q0, bool P1, bool Q1, int VMW, bool DQ, bool DP, int NBJ, int BPW,
          class OpP, class OpQ>
__device__ __forceinline__ void kstep(f32x16 (&acc)[4][NBJ], bf16x8 (&pa)[4], bf16x8 (&qa)[NBJ],
                                      bf16x8 (&pb)[4], bf16x8 (&qb)[NBJ], int t, const OpP& dp,
                                      const OpQ& dq, const WaveGeo& g, const FragOffsets& fo,
                                      int wave, const uint8_t* __restrict__ cur,
                                      const uint8_t* __restrict__ nxt,
                                      uint8_t* __restrict__ dst_q, uint8_t* __restrict__ dst_p) {
  constexpr int NM = 4 * NBJ;                                // MFMAs of a k16 sub-step
  constexpr int RD0 = (P0 ? 8 : 4) + (Q0 ? 2 : 1) * NBJ;    // LDS reads of a k16 sub-step
  constexpr int RD1 = (P1 ? 8 : 4) + (Q1 ? 2 : 1) * NBJ;
  constexpr int VEV = 8 / BPW;   // one DMA instruction per VEV interleaved MFMAs
  read_frags<P0, Q0, NBJ>(cur, 1, g, fo, pb, qb);
  if (DQ) dq.template issue<BPW>(t + NS - 2, dst_q + OPB, wave);
  mfma16<NBJ>(acc, pa, qa);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD0 / 8, 0);
    if (DQ && i % VEV == VEV - 1) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  if (NM > 8) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM - 8, 0);
  __builtin_amdgcn_sched_barrier(0);

  wait_vm<VMW>();
  bar_raw();
  if (DP) dp.template issue<BPW>(t + NS - 1, dst_p, wave);
  read_frags<P1, Q1, NBJ>(nxt, 0, g, fo, pa, qa);
  mfma16<NBJ>(acc, pb, qb);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD1 / 8, 0);
    if (DP && i % VEV == VEV - 1) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  if (NM > 8) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM - 8, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Prologue: DMA of steps 0 .. NS-3 and the P half of step NS-2, wait for step
// 0, first fragments (layouts P0, Q0 of step 0).  The reads alias only the DMA
// of step 0 (s0); the compiler's own wait for it is the same vmcnt as the
// explicit one.  A wave issues 2*BPW DMA instructions per step.
template <bool P0, bool Q0, int NBJ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kprologue(bf16x8 (&pa)[4], bf16x8 (&qa)[NBJ], const OpP& dp,
                                          const OpQ& dq, const WaveGeo& g, const FragOffsets& fo,
                                          int wave, uint8_t* __restrict__ s0,
                                          uint8_t* __restrict__ rest) {
  constexpr int DPS = 2 * BPW;
  dp.template issue<BPW>(0, s0, wave);
  dq.template issue<BPW>(0, s0 + OPB, wave);
#pragma unroll
  for (int t = 1; t < NS - 2; ++t) {
    dp.template issue<BPW>(t, rest + (t - 1) * STG, wave);
    dq.template issue<BPW>(t, rest + (t - 1) * STG + OPB, wave);
  }
  dp.template issue<BPW>(NS - 2, rest + (NS - 3) * STG, wave);
  wait_vm<DPS * (NS - 3) + DPS / 2>();
  bar_raw();
  read_frags<P0, Q0, NBJ>(s0, 0, g, fo, pa, qa);
}

__device__ __forceinline__ uint32_t stage_wrap(uint32_t x) {
  return x >= (uint32_t)LDS_BYTES ? x - (uint32_t)LDS_BYTES : x;
}

// Register state of one tile's K loop and the stage of its current step: the
// wave's 4 x NBJ accumulator blocks (NBJ = 4: 128 x 128 with four waves; 2:
// 128 x 64 with eight).
template <int NBJ>
struct KState {
  f32x16 acc[4][NBJ];
  bf16x8 pa[4], qa[NBJ], pb[4], qb[NBJ];
  uint32_t sc;   // LDS offset of step t's stage
  int t;
};

// Steady steps t < t_end with both DMA halves and layouts (P0, Q0) -> (P1, Q1).
template <bool P0, bool Q0, bool P1, bool Q1, int NBJ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void ksteps(KState<NBJ>& k, int t_end, const OpP& dp, const OpQ& dq,
                                       const WaveGeo& g, const FragOffsets& fo, int wave,
                                       uint8_t* lds) {
  for (; k.t < t_end; ++k.t) {
    kstep<P0, Q0, P1, Q1, 4 * BPW, true, true, NBJ, BPW>(
        k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
        lds + stage_wrap(k.sc + STG), lds + stage_wrap(k.sc + (NS - 2) * STG),
        lds + stage_wrap(k.sc + (NS - 1) * STG));
    k.sc = stage_wrap(k.sc + STG);
  }
}

// Steps nk-4 .. nk-2 (no DMA after the Q half of step nk-1, issued in step
// nk-4) and the sub-step-1 fragments of the last step, layouts (PF, QF).
template <bool PF, bool QF, int NBJ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kdrain(KState<NBJ>& k, const OpP& dp, const OpQ& dq,
                                       const WaveGeo& g, const FragOffsets& fo, int wave,
                                       uint8_t* lds) {
  constexpr int DPS = 2 * BPW;   // DMA instructions per wave and step
  kstep<PF, QF, PF, QF, DPS * 2, true, false, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds + stage_wrap(k.sc + (NS - 2) * STG), lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep<PF, QF, PF, QF, DPS, false, false, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep<PF, QF, PF, QF, 0, false, false, NBJ, BPW>(k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g,
                                                   fo, wave, lds + k.sc,
                                                   lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  read_frags<PF, QF, NBJ>(lds + k.sc, 1, g, fo, k.pb, k.qb);
}

// All K steps of one tile but the last, and the last step's sub-step-1
// fragments (in k.pb, k.qb).  P is k-major for t < bP and in layout PF from
// then on (bP is 0 or the first step of P's diagonal block, at most nk - 8, so
// the switch lies in the steady range).  Q is in layout QF, or with QS
// k-major for t < bQ and in layout QF from then on (a multiple of 8, at most
// nk - 8; bQ > bP, or with QEQ bQ >= bP: a diagonal tile in this loop).  The
// step that switches both layouts at once is left out of builds that never
// need it (it costs the register allocator dearly).
template <bool PF, bool QF, bool QS, bool QEQ, int NBJ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kloop(KState<NBJ>& k, int nk, int bP, int bQ, const OpP& dp,
                                      const OpQ& dq, const WaveGeo& g, const FragOffsets& fo,
                                      int wave, uint8_t* lds) {
  constexpr bool QA = QS ? true : QF;   // Q layout before bQ
  if (bP > 0) kprologue<true, QA, NBJ, BPW>(k.pa, k.qa, dp, dq, g, fo, wave, lds, lds + STG);
  else if (QS && bQ > 0) kprologue<PF, QA, NBJ, BPW>(k.pa, k.qa, dp, dq, g, fo, wave, lds, lds + STG);
  else kprologue<PF, QF, NBJ, BPW>(k.pa, k.qa, dp, dq, g, fo, wave, lds, lds + STG);
  k.sc = 0;
  k.t = 0;
  if (bP > 0) {
    ksteps<true, QA, true, QA, NBJ, BPW>(k, bP - 1, dp, dq, g, fo, wave, lds);
    if constexpr (QS && QEQ) {
      if (bQ == bP) ksteps<true, QA, PF, QF, NBJ, BPW>(k, bP, dp, dq, g, fo, wave, lds);
      else ksteps<true, QA, PF, QA, NBJ, BPW>(k, bP, dp, dq, g, fo, wave, lds);
    } else {
      ksteps<true, QA, PF, QA, NBJ, BPW>(k, bP, dp, dq, g, fo, wave, lds);
    }
  }
  if (QS && bQ > bP) {
    ksteps<PF, QA, PF, QA, NBJ, BPW>(k, bQ - 1, dp, dq, g, fo, wave, lds);
    ksteps<PF, QA, PF, QF, NBJ, BPW>(k, bQ, dp, dq, g, fo, wave, lds);
  }
  ksteps<PF, QF, PF, QF, NBJ, BPW>(k, nk - NS + 1, dp, dq, g, fo, wave, lds);
  kdrain<PF, QF, NBJ, BPW>(k, dp, dq, g, fo, wave, lds);
}

// Paired DMA schedule.  A row-major operand uses 64 bytes of each 128-byte
// line per K step and the other 64 bytes in the next step; the vector L1
// fetches whole lines, so issuing the two steps' loads of a line far apart
// fetches it from L2 twice.  Here the DMA of steps s and s+1 (s even) is
// issued back to back (the same line BPW loads apart), so the second load of a
// line finds it in (or on its way into) the L1: P(s), P(s+1) after the barrier of step s-3
// (odd) into the stages of s-5 and s-4, Q(s), Q(s+1) before the barrier of step
// s-2 (even) into the same two stages, both free by then.  The wait before the
// barrier of step t (for step t+1) leaves in flight P(t+2), P(t+3), Q(t+2),
// Q(t+3) when t is even and Q(t+2) when t is odd.  d0, d1 are the stages of
// steps t+2, t+3 (even t) or t+3, t+4 (odd t).
template <class Op, int BPW>
__device__ __forceinline__ void issue_pair(const Op& op, int s, uint8_t* a, uint8_t* b, int wave) {
  // step s first, then s+1: a wait that leaves BPW loads in flight covers step s
  op.template issue<BPW>(s, a, wave);
  op.template issue<BPW>(s + 1, b, wave);
}

// XW > 0: when xw is set, XW more vector memory instructions (stores issued
// after this tile's prologue DMA, older than this step's DMA) may stay in
// flight at the wait.
template <bool P0, bool Q0, bool P1, bool Q1, int VMW, bool QPAIR, bool PPAIR, int NBJ, int BPW,
          class OpP, class OpQ, int XW = 0>
__device__ __forceinline__ void kstep2(f32x16 (&acc)[4][NBJ], bf16x8 (&pa)[4], bf16x8 (&qa)[NBJ],
                                       bf16x8 (&pb)[4], bf16x8 (&qb)[NBJ], int t, const OpP& dp,
                                       const OpQ& dq, const WaveGeo& g, const FragOffsets& fo,
                                       int wave, const uint8_t* __restrict__ cur,
                                       const uint8_t* __restrict__ nxt, uint8_t* __restrict__ d0,
                                       uint8_t* __restrict__ d1, bool xw = false) {
  constexpr int NM = 4 * NBJ;
  constexpr int RD0 = (P0 ? 8 : 4) + (Q0 ? 2 : 1) * NBJ;
  constexpr int RD1 = (P1 ? 8 : 4) + (Q1 ? 2 : 1) * NBJ;
  constexpr int ND0 = QPAIR ? 2 * BPW : 0, ND1 = PPAIR ? 2 * BPW : 0;
  read_frags<P0, Q0, NBJ>(cur, 1, g, fo, pb, qb);
  if (QPAIR) issue_pair<OpQ, BPW>(dq, t + 2, d0 + OPB, d1 + OPB, wave);
  mfma16<NBJ>(acc, pa, qa);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD0 / 8, 0);
    if ((i + 1) * ND0 / 8 > i * ND0 / 8) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  if (NM > 8) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM - 8, 0);
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (XW > 0) {
    if (xw) wait_vm<VMW + XW>();
    else wait_vm<VMW>();
  } else {
    wait_vm<VMW>();
  }
  bar_raw();
  if (PPAIR) issue_pair<OpP, BPW>(dp, t + 3, d0, d1, wave);
  read_frags<P1, Q1, NBJ>(nxt, 0, g, fo, pa, qa);
  mfma16<NBJ>(acc, pb, qb);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD1 / 8, 0);
    if ((i + 1) * ND1 / 8 > i * ND1 / 8) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  if (NM > 8) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM - 8, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One even and one odd step with the paired DMA: layouts (PE, Q) -> (PM, Q)
// -> (PO, Q) for steps t, t+1, t+2.
template <bool PE, bool PM, bool PO, bool QF, int NBJ, int BPW, int XW = 0, class OpP, class OpQ>
__device__ __forceinline__ void kpair(KState<NBJ>& k, const OpP& dp, const OpQ& dq,
                                      const WaveGeo& g, const FragOffsets& fo, int wave,
                                      uint8_t* lds, bool xw = false) {
  constexpr int DPS = 2 * BPW;
  kstep2<PE, QF, PM, QF, 2 * DPS, true, false, NBJ, BPW, OpP, OpQ, XW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds + stage_wrap(k.sc + 2 * STG),
      lds + stage_wrap(k.sc + 3 * STG), xw);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep2<PM, QF, PO, QF, BPW, false, true, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds + stage_wrap(k.sc + 3 * STG),
      lds + stage_wrap(k.sc + 4 * STG));
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
}

// Step 0's fragments (P k-major when bP > 0).  The stage pointer is declared
// restrict, as in kstep2, so that the compiler orders these reads after the
// DMA through the explicit waits alone.
template <bool PF, bool QF, int NBJ>
__device__ __forceinline__ void first_frags(bool pkm, const uint8_t* __restrict__ s0,
                                            const WaveGeo& g, const FragOffsets& fo,
                                            bf16x8 (&pa)[4], bf16x8 (&qa)[NBJ]) {
  if (pkm) read_frags<true, QF, NBJ>(s0, 0, g, fo, pa, qa);
  else read_frags<PF, QF, NBJ>(s0, 0, g, fo, pa, qa);
}

// Prologue DMA of the paired schedule: P(0), Q(0), P(1), Q(1), P(2), P(3)
// into stages 0..3 (all four free).
template <int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kprologue2_issue(const OpP& dp, const OpQ& dq, int wave,
                                                 uint8_t* lds) {
  dp.template issue<BPW>(0, lds, wave);
  dq.template issue<BPW>(0, lds + OPB, wave);
  dp.template issue<BPW>(1, lds + STG, wave);
  dq.template issue<BPW>(1, lds + STG + OPB, wave);
  issue_pair<OpP, BPW>(dp, 2, lds + 2 * STG, lds + 3 * STG, wave);
}

// All K steps of one tile but the last, paired DMA (same contract as kloop
// without QS; nk and bP are even), after the prologue DMA: wait for step 0
// (the 2 DPS most recent vector memory instructions may still be in flight:
// P(2), P(3), Q(1), P(1)), then the steady pairs and the drain.  pend: XW
// vector memory instructions (at most as many as were issued) followed the
// prologue DMA before this call -- the previous tile's stores -- and may stay
// in flight at the waits of steps -1 and 0, which need only DMA older than
// them; the wait of step 1 needs Q(2), issued after them, so they have landed
// by then whatever the count.
template <bool PF, bool QF, int NBJ, int BPW, int XW = 0, class OpP, class OpQ>
__device__ __forceinline__ void kloop2_rest(KState<NBJ>& k, int nk, int bP, const OpP& dp,
                                            const OpQ& dq, const WaveGeo& g,
                                            const FragOffsets& fo, int wave, uint8_t* lds,
                                            bool pend = false) {
  constexpr int DPS = 2 * BPW;
  {
    if constexpr (XW > 0) {
      if (pend) wait_vm<2 * DPS + XW>();
      else wait_vm<2 * DPS>();
    } else {
      wait_vm<2 * DPS>();
    }
    bar_raw();
    first_frags<PF, QF, NBJ>(bP > 0, lds, g, fo, k.pa, k.qa);
  }
  k.sc = 0;
  k.t = 0;
  if (bP > 0) {
    for (; k.t < bP - 2;)
      kpair<true, true, true, QF, NBJ, BPW, XW>(k, dp, dq, g, fo, wave, lds, pend && k.t == 0);
    kpair<true, true, PF, QF, NBJ, BPW, XW>(k, dp, dq, g, fo, wave, lds, pend && k.t == 0);
  }
  for (; k.t < nk - 4;)
    kpair<PF, PF, PF, QF, NBJ, BPW, XW>(k, dp, dq, g, fo, wave, lds, pend && k.t == 0);
  // step nk-4 issues Q(nk-2), Q(nk-1), the last DMA; nk-3 and nk-2 issue none
  kstep2<PF, QF, PF, QF, 2 * DPS, true, false, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds + stage_wrap(k.sc + 2 * STG),
      lds + stage_wrap(k.sc + 3 * STG));
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep2<PF, QF, PF, QF, BPW, false, false, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep2<PF, QF, PF, QF, 0, false, false, NBJ, BPW>(
      k.acc, k.pa, k.qa, k.pb, k.qb, k.t, dp, dq, g, fo, wave, lds + k.sc,
      lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  read_frags<PF, QF, NBJ>(lds + k.sc, 1, g, fo, k.pb, k.qb);
}

template <bool PF, bool QF, int NBJ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kloop2(KState<NBJ>& k, int nk, int bP, const OpP& dp,
                                       const OpQ& dq, const WaveGeo& g, const FragOffsets& fo,
                                       int wave, uint8_t* lds) {
  kprologue2_issue<BPW>(dp, dq, wave, lds);
  kloop2_rest<PF, QF, NBJ, BPW>(k, nk, bP, dp, dq, g, fo, wave, lds);
}

// ------------------------------------------- 16 x 16 x 32 MFMA engine
// The apply stage's K loop on v_mfma_f32_16x16x32_bf16 in place of the
// 32 x 32 x 16 form: each wave's 128 x 64 sub-tile is 8 x 4 slabs of 16 x 16,
// each K step of 32 one MFMA per slab (32 per wave and step: the same flops
// and the same LDS fragment bytes).  On this part the 16 x 16 form draws less
// power per flop on random data, so the clock it sustains under load is
// higher (a register-only MFMA loop: 1.93 against 1.71 GHz; with its LDS
// reads: 1.86 against 1.71 GHz).  A K step is issued as two halves (P slabs
// 0-3, then 4-7, each against the step's four Q slabs); the barrier and the
// DMA sit between the halves as in kstep2, and Q is double-buffered across
// steps (the next step's Q slabs are read while the second half still uses
// this step's).
//
// Fragments cover 16 operand rows and the whole K step: lane l holds row
// (l & 15) of the slab at the 8 k of octet o = oct16(l >> 4).
//   row-major: one ds_read_b128 at rm_off(l & 15, o) from the slab's first
//              row (the chunk swizzle depends on row & 12 only);
//   k-major:   two ds_read_b64_tr_b16; lane c = 4e + h of 16-lane group G
//              points at k row 8o + e (8o + 4 + e for the second read, 2048
//              bytes on) and slab rows 4h .. 4h+3, so that lane c receives
//              slab row c at four consecutive k.
// Accumulator slab (i, j) of a lane holds C[16i + (l & 15)][16j + 4(l >> 4)
// + 0..3] (operands swapped, as in mfma16).
// The k octet (16 bytes of a row-major row, 8 k rows of a k-major tile) that
// 16-lane group G of a fragment holds: 0, 3, 1, 2 for G = 0..3, the same in
// every fragment of both operands (any fixed assignment computes the same
// sums).  With this one the row-major reads (ds_read_b128, the row swizzle of
// rm_off) are free of bank conflicts: rocprofv3 counts bank-conflict cycles
// equal to half the LDS active cycles with octet G, none with this order.
// The transposing reads still meet a 2-way conflict (the two 16-lane groups
// one of them serves read the same unit positions of two octets); a layout
// that swapped unit halves in odd octets removed it, but the per-read offset
// arithmetic it needs cost more than the conflict (same-box A/B: apply +1.6%,
// polynomial -2%, last apply -1%).
__device__ __forceinline__ int oct16(int G) { return (0x2130 >> (4 * G)) & 15; }

struct Frag16 {
  uint32_t rm;       // row-major, from the slab's first row
  uint32_t kmp[4];   // k-major P slabs, by slab pair s >> 1 (wave origin added at the read)
  uint32_t kmq[2];   // k-major Q slabs of the wave, by slab pair, origin included
  __device__ void init(int lane, int wq0) {
    const int G = lane >> 4, c = lane & 15, e = c >> 2, h = c & 3;
    const int o = oct16(G);
    rm = rm_off(c, o);
    const int kr = 8 * o + e;
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) kmp[sp] = kr * 512 + ((sp ^ e) << 6) + 8 * h;
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
      kmq[sp] = kr * 512 + (((((wq0 >> 5) + sp) ^ e) & 7) << 6) + 8 * h;
  }
};

// P slabs S0 .. S0+3 of the wave (origin wo, a multiple of 128: its unit bits
// never meet the swizzle).
template <bool KM, int S0>
__device__ __forceinline__ void read_p16(const uint8_t* __restrict__ stage, int wo,
                                         const Frag16& f,
                                         bf16x8 (&p)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = S0 + i;
    if (!KM) {
      p[i] = *(const bf16x8*)(stage + (wo + 16 * s) * 64 + f.rm);
    } else {
      const uint8_t* base = stage + 2 * wo + 32 * (s & 1) + f.kmp[s >> 1];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base + 2048));
      p[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
}

// The wave's four Q slabs (origin wq0, a multiple of 64; k-major or row-major).
template <bool KM = true>
__device__ __forceinline__ void read_q16(const uint8_t* __restrict__ stage, int wq0,
                                         const Frag16& f, bf16x8 (&q)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!KM) {
      q[j] = *(const bf16x8*)(stage + OPB + (wq0 + 16 * j) * 64 + f.rm);
    } else {
      const uint8_t* base = stage + OPB + 32 * (j & 1) + f.kmq[j >> 1];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base + 2048));
      q[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
}

template <int I0>
__device__ __forceinline__ void mfma_half16(f32x4 (&acc)[8][4], const bf16x8 (&p)[4],
                                            const bf16x8 (&q)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[I0 + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[j], p[i], acc[I0 + i][j], 0, 0, 0);
}

struct KState16 {
  f32x4 acc[8][4];
  bf16x8 pa[4], pb[4], qa[4], qb[4];
  uint32_t sc;
  int t;
};

// 16 MFMAs with RD LDS reads and ND (<= 4) DMA instructions spread among
// them, in four groups of four MFMAs.
template <int RD, int ND>
__device__ __forceinline__ void sched16() {
  static_assert(RD % 4 == 0 && ND <= 4, "reads in whole groups, at most one DMA per group");
  constexpr int R = RD / 4, RA = (R + 1) / 2, RB = R / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if (RA > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RA, 0);
    if ((i + 1) * ND / 4 > i * ND / 4) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    if (RB > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RB, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One K step (the contract of kstep2): P in layout P0 this step and P1 the
// next; Q k-major; qc holds this step's Q slabs, qn receives the next step's.
template <bool P0, bool P1, int VMW, bool QPAIR, bool PPAIR, int BPW, class OpP, class OpQ,
          int XW = 0>
__device__ __forceinline__ void kstep16(KState16& k, bf16x8 (&qc)[4], bf16x8 (&qn)[4],
                                        const OpP& dp, const OpQ& dq, const WaveGeo& g,
                                        const Frag16& f, int wave,
                                        const uint8_t* __restrict__ cur,
                                        const uint8_t* __restrict__ nxt, uint8_t* __restrict__ d0,
                                        uint8_t* __restrict__ d1, bool xw = false) {
  constexpr int RD0 = P0 ? 8 : 4;
  constexpr int RD1 = (P1 ? 8 : 4) + 8;
  constexpr int ND0 = QPAIR ? 2 * BPW : 0, ND1 = PPAIR ? 2 * BPW : 0;
  read_p16<P0, 4>(cur, g.wi0, f, k.pb);
  if (QPAIR) issue_pair<OpQ, BPW>(dq, k.t + 2, d0 + OPB, d1 + OPB, wave);
  mfma_half16<0>(k.acc, k.pa, qc);
  sched16<RD0, ND0>();

  if constexpr (XW > 0) {
    if (xw) wait_vm<VMW + XW>();
    else wait_vm<VMW>();
  } else {
    wait_vm<VMW>();
  }
  bar_raw();
  if (PPAIR) issue_pair<OpP, BPW>(dp, k.t + 3, d0, d1, wave);
  read_p16<P1, 0>(nxt, g.wi0, f, k.pa);
  read_q16<true>(nxt, g.wj0, f, qn);
  mfma_half16<4>(k.acc, k.pb, qc);
  sched16<RD1, ND1>();
}

template <bool PE, bool PM, bool PO, int BPW, int XW = 0, class OpP, class OpQ>
__device__ __forceinline__ void kpair16(KState16& k, const OpP& dp, const OpQ& dq,
                                        const WaveGeo& g, const Frag16& f, int wave,
                                        uint8_t* lds, bool xw = false) {
  constexpr int DPS = 2 * BPW;
  kstep16<PE, PM, 2 * DPS, true, false, BPW, OpP, OpQ, XW>(
      k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc, lds + stage_wrap(k.sc + STG),
      lds + stage_wrap(k.sc + 2 * STG), lds + stage_wrap(k.sc + 3 * STG), xw);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep16<PM, PO, BPW, false, true, BPW>(k, k.qb, k.qa, dp, dq, g, f, wave, lds + k.sc,
                                         lds + stage_wrap(k.sc + STG),
                                         lds + stage_wrap(k.sc + 3 * STG),
                                         lds + stage_wrap(k.sc + 4 * STG));
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
}

// Step 0's fragments (P k-major when pkm), through a restrict stage pointer as
// in first_frags.
template <bool PF>
__device__ __forceinline__ void first_frags16(bool pkm, const uint8_t* __restrict__ s0,
                                              const WaveGeo& g, const Frag16& f, bf16x8 (&pa)[4],
                                              bf16x8 (&qa)[4]) {
  if (pkm) {
    read_p16<true, 0>(s0, g.wi0, f, pa);
    read_q16<true>(s0, g.wj0, f, qa);
  } else {
    read_p16<PF, 0>(s0, g.wi0, f, pa);
    read_q16<true>(s0, g.wj0, f, qa);
  }
}

template <bool PKM, bool QKM>
__device__ __forceinline__ void first_frags16q(const uint8_t* __restrict__ s0, const WaveGeo& g,
                                               const Frag16& f, bf16x8 (&pa)[4],
                                               bf16x8 (&qa)[4]) {
  read_p16<PKM, 0>(s0, g.wi0, f, pa);
  read_q16<QKM>(s0, g.wj0, f, qa);
}

// kloop2_rest on 16 x 16 x 32 MFMAs (the same DMA schedule and waits).  On
// return the last step (nk - 1, odd) has its fragments in pa, pb and qb.
template <bool PF, int BPW, int XW = 0, class OpP, class OpQ>
__device__ __forceinline__ void kloop16_rest(KState16& k, int nk, int bP, const OpP& dp,
                                             const OpQ& dq, const WaveGeo& g, const Frag16& f,
                                             int wave, uint8_t* lds, bool pend = false) {
  constexpr int DPS = 2 * BPW;
  {
    if constexpr (XW > 0) {
      if (pend) wait_vm<2 * DPS + XW>();
      else wait_vm<2 * DPS>();
    } else {
      wait_vm<2 * DPS>();
    }
    bar_raw();
    first_frags16<PF>(bP > 0, lds, g, f, k.pa, k.qa);
  }
  k.sc = 0;
  k.t = 0;
  if (bP > 0) {
    for (; k.t < bP - 2;) kpair16<true, true, true, BPW, XW>(k, dp, dq, g, f, wave, lds, pend && k.t == 0);
    kpair16<true, true, PF, BPW, XW>(k, dp, dq, g, f, wave, lds, pend && k.t == 0);
  }
  for (; k.t < nk - 4;) kpair16<PF, PF, PF, BPW, XW>(k, dp, dq, g, f, wave, lds, pend && k.t == 0);
  kstep16<PF, PF, 2 * DPS, true, false, BPW>(k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc,
                                             lds + stage_wrap(k.sc + STG),
                                             lds + stage_wrap(k.sc + 2 * STG),
                                             lds + stage_wrap(k.sc + 3 * STG));
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep16<PF, PF, BPW, false, false, BPW>(k, k.qb, k.qa, dp, dq, g, f, wave, lds + k.sc,
                                          lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep16<PF, PF, 0, false, false, BPW>(k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc,
                                        lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  read_p16<PF, 4>(lds + k.sc, g.wi0, f, k.pb);
}

// One K step with each step's DMA spread over its two halves (the contract of
// kstep): P in layouts P0 -> P1 and Q in Q0 -> Q1 from this step to the next.
template <bool P0, bool Q0, bool P1, bool Q1, int VMW, bool DQ, bool DP, int BPW, class OpP,
          class OpQ>
__device__ __forceinline__ void kstep16s(KState16& k, bf16x8 (&qc)[4], bf16x8 (&qn)[4],
                                         const OpP& dp, const OpQ& dq, const WaveGeo& g,
                                         const Frag16& f, int wave,
                                         const uint8_t* __restrict__ cur,
                                         const uint8_t* __restrict__ nxt,
                                         uint8_t* __restrict__ dst_q, uint8_t* __restrict__ dst_p) {
  constexpr int RD0 = P0 ? 8 : 4;
  constexpr int RD1 = (P1 ? 8 : 4) + (Q1 ? 8 : 4);
  read_p16<P0, 4>(cur, g.wi0, f, k.pb);
  if (DQ) dq.template issue<BPW>(k.t + NS - 2, dst_q + OPB, wave);
  mfma_half16<0>(k.acc, k.pa, qc);
  sched16<RD0, DQ ? BPW : 0>();

  wait_vm<VMW>();
  bar_raw();
  if (DP) dp.template issue<BPW>(k.t + NS - 1, dst_p, wave);
  read_p16<P1, 0>(nxt, g.wi0, f, k.pa);
  read_q16<Q1>(nxt, g.wj0, f, qn);
  mfma_half16<4>(k.acc, k.pb, qc);
  sched16<RD1, DP ? BPW : 0>();
}

// Steady steps in pairs (t even) up to t_end (even), layouts (PE, QE) ->
// (PM, QM) -> (PO, QO) for steps t, t+1, t+2 of each pair.
template <bool PE, bool QE, bool PM, bool QM, bool PO, bool QO, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void ksteps16(KState16& k, int t_end, const OpP& dp, const OpQ& dq,
                                         const WaveGeo& g, const Frag16& f, int wave,
                                         uint8_t* lds) {
  for (; k.t < t_end;) {
    kstep16s<PE, QE, PM, QM, 4 * BPW, true, true, BPW>(
        k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc, lds + stage_wrap(k.sc + STG),
        lds + stage_wrap(k.sc + (NS - 2) * STG), lds + stage_wrap(k.sc + (NS - 1) * STG));
    k.sc = stage_wrap(k.sc + STG);
    ++k.t;
    kstep16s<PM, QM, PO, QO, 4 * BPW, true, true, BPW>(
        k, k.qb, k.qa, dp, dq, g, f, wave, lds + k.sc, lds + stage_wrap(k.sc + STG),
        lds + stage_wrap(k.sc + (NS - 2) * STG), lds + stage_wrap(k.sc + (NS - 1) * STG));
    k.sc = stage_wrap(k.sc + STG);
    ++k.t;
  }
}

// kloop on 16 x 16 x 32 MFMAs (the same DMA schedule, waits and layout
// switches; bP and bQ are multiples of 8, so every switch falls between the
// two steps of a pair).  On return the last step (nk - 1, odd) has its
// fragments in pa, pb and qb.
template <bool PF, bool QF, bool QS, bool QEQ, int BPW, class OpP, class OpQ>
__device__ __forceinline__ void kloop16(KState16& k, int nk, int bP, int bQ, const OpP& dp,
                                        const OpQ& dq, const WaveGeo& g, const Frag16& f,
                                        int wave, uint8_t* lds) {
  constexpr bool QA = QS ? true : QF;   // Q layout before bQ
  constexpr int DPS = 2 * BPW;
  // prologue DMA: steps 0 .. NS-3 and the P half of step NS-2
  dp.template issue<BPW>(0, lds, wave);
  dq.template issue<BPW>(0, lds + OPB, wave);
#pragma unroll
  for (int t = 1; t < NS - 2; ++t) {
    dp.template issue<BPW>(t, lds + t * STG, wave);
    dq.template issue<BPW>(t, lds + t * STG + OPB, wave);
  }
  dp.template issue<BPW>(NS - 2, lds + (NS - 2) * STG, wave);
  wait_vm<DPS * (NS - 3) + DPS / 2>();
  bar_raw();
  if (bP > 0) first_frags16q<true, QA>(lds, g, f, k.pa, k.qa);
  else if (QS && bQ > 0) first_frags16q<PF, QA>(lds, g, f, k.pa, k.qa);
  else first_frags16q<PF, QF>(lds, g, f, k.pa, k.qa);
  k.sc = 0;
  k.t = 0;
  if (bP > 0) {
    ksteps16<true, QA, true, QA, true, QA, BPW>(k, bP - 2, dp, dq, g, f, wave, lds);
    if constexpr (QS && QEQ) {
      if (bQ == bP) ksteps16<true, QA, true, QA, PF, QF, BPW>(k, bP, dp, dq, g, f, wave, lds);
      else ksteps16<true, QA, true, QA, PF, QA, BPW>(k, bP, dp, dq, g, f, wave, lds);
    } else {
      ksteps16<true, QA, true, QA, PF, QA, BPW>(k, bP, dp, dq, g, f, wave, lds);
    }
  }
  if (QS && bQ > bP) {
    ksteps16<PF, QA, PF, QA, PF, QA, BPW>(k, bQ - 2, dp, dq, g, f, wave, lds);
    ksteps16<PF, QA, PF, QA, PF, QF, BPW>(k, bQ, dp, dq, g, f, wave, lds);
  }
  ksteps16<PF, QF, PF, QF, PF, QF, BPW>(k, nk - NS + 1, dp, dq, g, f, wave, lds);
  // drain: step nk-4 issues the last DMA (the Q half of step nk-1)
  kstep16s<PF, QF, PF, QF, DPS * 2, true, false, BPW>(
      k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc, lds + stage_wrap(k.sc + STG),
      lds + stage_wrap(k.sc + (NS - 2) * STG), lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep16s<PF, QF, PF, QF, DPS, false, false, BPW>(k, k.qb, k.qa, dp, dq, g, f, wave,
                                                   lds + k.sc, lds + stage_wrap(k.sc + STG),
                                                   lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  kstep16s<PF, QF, PF, QF, 0, false, false, BPW>(k, k.qa, k.qb, dp, dq, g, f, wave, lds + k.sc,
                                                 lds + stage_wrap(k.sc + STG), lds, lds);
  k.sc = stage_wrap(k.sc + STG);
  ++k.t;
  read_p16<PF, 4>(lds + k.sc, g.wi0, f, k.pb);
}

// Two horizontally adjacent slabs (16 x 32 of a 32 x 32 block) of a lane,
// values already final, packed to bf16 and stored as one 16-byte piece per
// lane.  Lane l holds columns 4q .. 4q+3 (q = l >> 4) of each slab; one
// v_permlane16_swap per packed register trades the odd 16-lane groups' left
// slab values for the even groups' right slab values, so that lane l then
// holds 8 consecutive columns: 8(q >> 1) + 16(q & 1) .. +7 of row (l & 15).
__device__ __forceinline__ void store_pair16(const float (&a)[4], const float (&b)[4],
                                             uint16_t* dst) {
  const auto r0 = __builtin_amdgcn_permlane16_swap(pack_bf2(a[0], a[1]), pack_bf2(b[0], b[1]),
                                                   false, false);
  const auto r1 = __builtin_amdgcn_permlane16_swap(pack_bf2(a[2], a[3]), pack_bf2(b[2], b[3]),
                                                   false, false);
  gstore<u32x4>(dst, u32x4{r0[0], r1[0], r0[1], r1[1]});
}

// A wave's 128 x 64 accumulator sub-tile (16 x 16 layout), times s, into the
// 32 x 32 blocks of a blocked matrix: blk0 is the wave's first block, nb the
// blocks per block row.  With split, the low parts go lo_off elements on.
__device__ __forceinline__ void store_acc16(const f32x4 (&acc)[8][4], uint16_t* blk0, int64_t nb,
                                            int lane, float s, bool split, int64_t lo_off) {
  const int q = lane >> 4;
  uint16_t* base = blk0 + (lane & 15) * 32 + 8 * (q >> 1) + 16 * (q & 1);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const f32x4& a = acc[2 * bi + i2][2 * bj];
        const f32x4& b = acc[2 * bi + i2][2 * bj + 1];
        uint16_t* dst = base + (bi * nb + bj) * 1024 + i2 * 512;
        if (split) {
#pragma clang fp contract(off)
          float va[4], vb[4], la[4], lb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            va[e] = s * a[e];
            vb[e] = s * b[e];
            la[e] = va[e] - bf2f(f2bf(va[e]));
            lb[e] = vb[e] - bf2f(f2bf(vb[e]));
          }
          store_pair16(va, vb, dst);
          store_pair16(la, lb, dst + lo_off);
        } else {
          float va[4], vb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            va[e] = s * a[e];
            vb[e] = s * b[e];
          }
          store_pair16(va, vb, dst);
        }
      }
}

// Stage stripe BI (rows 32 BI .. +31: slabs 2 BI, 2 BI + 1) of a 16 x 16
// layout sub-tile into the wave's LDS region, in the layout stage_stripe
// writes (float32 rows of Ep<64>), for final_pass.
template <int BI>
__device__ __forceinline__ void stage_stripe16(const f32x4 (&acc)[8][4], float* stg, int lane) {
  using G = Ep<64>;
#pragma unroll
  for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4*)(stg + G::row(16 * i2 + (lane & 15)) + 16 * j + 4 * (lane >> 4)) =
          acc[2 * BI + i2][j];
}

// Staging of stripe BI of a 16 x 16 x 32 layout sub-tile (stage_stripe16).
struct Stage16 {
  const f32x4 (&acc)[8][4];
  int lane;
  template <int BI>
  __device__ __forceinline__ void stage(float* stg) const {
    stage_stripe16<BI>(acc, stg, lane);
  }
};

// The last apply's epilogue (O or the fused weight update) of a 16 x 16
// layout sub-tile: as epilogue() for the last iteration, one staged 32-row
// stripe at a time.
template <int OUT>
__device__ __forceinline__ void epilogue_final16(const MatDesc& d, const GemmParams& P,
                                                 const f32x4 (&acc)[8][4], float* stg, int i0,
                                                 int j0, int lane, float s_first) {
  const bool out_trans = d.transposed;
  const float upd = -P.lr * d.upd_scale;
#pragma unroll 1
  for (int bi = 0; bi < 4; ++bi) {
    switch (bi) {
      case 0: stage_stripe16<0>(acc, stg, lane); break;
      case 1: stage_stripe16<1>(acc, stg, lane); break;
      case 2: stage_stripe16<2>(acc, stg, lane); break;
      default: stage_stripe16<3>(acc, stg, lane); break;
    }
    __builtin_amdgcn_wave_barrier();
    const int64_t ib = i0 + 32 * bi;
    if (out_trans) final_pass<OUT, true, 64>(d, P, stg, ib, j0, lane, upd, s_first);
    else final_pass<OUT, false, 64>(d, P, stg, ib, j0, lane, upd, s_first);
    __builtin_amdgcn_wave_barrier();
  }
}

// An off-diagonal Gram tile (an upper tile of A = s^2 X X^T) on the 16 x 16 x
// 32 engine: P and Q row-major, the spread DMA schedule of kloop.
template <class OpP, class OpQ>
__device__ __forceinline__ void gram_tile16(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                            const OpQ& dq, const WaveGeo& g, int nk, int i0,
                                            int j0, int wave, int lane, uint8_t* lds) {
  constexpr int BPW = 2;
  Frag16 f;
  f.init(lane, g.wj0);
  KState16 k;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) k.acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop16<false, false, false, false, BPW>(k, nk, 0, 0, dp, dq, g, f, wave, lds);
  mfma_half16<0>(k.acc, k.pa, k.qb);
  mfma_half16<4>(k.acc, k.pb, k.qb);
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const int64_t nb = d.mp / 32;
  uint16_t* blk0 = (uint16_t*)d.a + (((int64_t)(i0 + g.wi0) >> 5) * nb + ((j0 + g.wj0) >> 5)) * 1024;
  store_acc16(k.acc, blk0, nb, lane, s_first * s_first, false, 0);
}

// An off-diagonal polynomial tile (B = a I + b A + c A A, an upper tile) on the
// 16 x 16 x 32 engine.  The epilogue swaps each lane's float32 values across
// 16-lane groups (v_permlane16_swap) so that a lane holds 8 consecutive
// columns of one row, reads A's 8 values there (16 bytes, all sixteen reads
// issued before the last MFMAs) and writes B's 8 values in one store.
template <bool QEQ, class OpP, class OpQ>
__device__ __forceinline__ void poly_tile16(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                            const OpQ& dq, const WaveGeo& g, int nk, int bP,
                                            int bQ, int i0, int j0, int wave, int lane,
                                            uint8_t* lds) {
  constexpr int BPW = 2;
  Frag16 f;
  f.init(lane, g.wj0);
  KState16 k;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) k.acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop16<false, false, true, QEQ, BPW>(k, nk, bP, bQ, dp, dq, g, f, wave, lds);
  const int64_t mp = d.mp;
  const uint16_t* A = (const uint16_t*)d.a;
  const int q = lane >> 4;
  const int64_t r0 = i0 + g.wi0 + (lane & 15);
  const int64_t c0 = j0 + g.wj0 + 8 * (q >> 1) + 16 * (q & 1);
  // slab i, block column bj of the wave: (i >> 1) block rows and bj blocks on
  // from the lane's first element, plus 16 rows (512 elements) for odd i
  const uint32_t nb = (uint32_t)(mp / 32);
  const int64_t boff = blk_at((const uint16_t*)nullptr, r0, c0, mp) - (const uint16_t*)nullptr;
  const uint16_t* Ab = A + boff;
  uint16_t* Bb = (uint16_t*)d.b + boff;
  auto eoff = [&](int i, int bj) -> uint32_t {
    return ((uint32_t)(i >> 1) * nb + (uint32_t)bj) * 1024u + (uint32_t)(i & 1) * 512u;
  };
  u32x4 av[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) av[i][bj] = gload<u32x4>(Ab + eoff(i, bj));
  mfma_half16<0>(k.acc, k.pa, k.qb);
  mfma_half16<4>(k.acc, k.pb, k.qb);
  const float a = P.a, b = P.b, c = P.c;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(k.acc[i][2 * bj][e]),
                                                        __float_as_uint(k.acc[i][2 * bj + 1][e]),
                                                        false, false);
        x[e] = __uint_as_float(r[0]);
        x[4 + e] = __uint_as_float(r[1]);
      }
      const int64_t row = r0 + 16 * i, col = c0 + 32 * bj;
      const u32x4 A8 = av[i][bj];
      const float aa[8] = {lo_bf(A8.x), hi_bf(A8.x), lo_bf(A8.y), hi_bf(A8.y),
                           lo_bf(A8.z), hi_bf(A8.z), lo_bf(A8.w), hi_bf(A8.w)};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = fmaf(b, aa[e], fmaf(c, x[e], row == col + e ? a : 0.f));
      gstore<u32x4>(Bb + eoff(i, bj), u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                            pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])});
    }
}

// An off-diagonal tile of the split-precision polynomial (B stored whole: the
// staged epilogue also writes the mirror tile) on the 16 x 16 x 32 engine.
template <bool QEQ, class OpP, class OpQ>
__device__ __forceinline__ void poly_mirror_tile16(const MatDesc& d, const GemmParams& P,
                                                   const OpP& dp, const OpQ& dq, const WaveGeo& g,
                                                   int nk, int bP, int bQ, int i0, int j0,
                                                   int wave, int lane, uint8_t* lds) {
  constexpr int BPW = 2;
  Frag16 f;
  f.init(lane, g.wj0);
  KState16 k;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) k.acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop16<false, false, true, QEQ, BPW>(k, nk, bP, bQ, dp, dq, g, f, wave, lds);
  const int64_t mp = d.mp;
  u32x4 ecur[Ep<64>::IPL];
  prefetch_stripe<64>((const uint16_t*)d.a, mp, i0 + g.wi0, j0 + g.wj0, lane, ecur);
  mfma_half16<0>(k.acc, k.pa, k.qb);
  mfma_half16<4>(k.acc, k.pb, k.qb);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const Stage16 st{k.acc, lane};
  epilogue_staged<1, OUT_NEXT_X, 2, true>(d, P, st, (float*)(lds + wave * Ep<64>::WAVE_BYTES),
                                          (const uint16_t*)d.a, mp, (uint16_t*)d.b, mp,
                                          i0 + g.wi0, j0 + g.wj0, lane, s_first, ecur);
}

// One apply tile (one tile per workgroup) on the 16 x 16 x 32 engine, with
// the paired DMA schedule of kloop2.
template <int OUT, class OpP, class OpQ>
__device__ __forceinline__ void apply_tile16(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                             const OpQ& dq, const WaveGeo& g, int nk, int bP,
                                             uint16_t* xnext, int i0, int j0, int wave, int lane,
                                             uint8_t* lds) {
  constexpr int BPW = 2;
  Frag16 f;
  f.init(lane, g.wj0);
  KState16 k;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) k.acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kprologue2_issue<BPW>(dp, dq, wave, lds);
  kloop16_rest<false, BPW>(k, nk, bP, dp, dq, g, f, wave, lds);
  mfma_half16<0>(k.acc, k.pa, k.qb);
  mfma_half16<4>(k.acc, k.pb, k.qb);
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const int64_t mp = d.mp, np = d.np;
  if (OUT == OUT_NEXT_X) {
    const int64_t nb = np / 32;
    uint16_t* blk0 = xnext + (((int64_t)(i0 + g.wi0) >> 5) * nb + ((j0 + g.wj0) >> 5)) * 1024;
    store_acc16(k.acc, blk0, nb, lane, s_first, P.split, mp * np);
    return;
  }
  // all fragment reads done: the stages become epilogue staging
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();
  epilogue_final16<OUT>(d, P, k.acc, (float*)(lds + wave * Ep<64>::WAVE_BYTES), i0 + g.wi0,
                        j0 + g.wj0, lane, s_first);
}


// ------------------------------------------------------- diagonal tiles
// A Gram or polynomial tile on the diagonal (ti == tj) has P = Q (the same 256
// operand rows) and a symmetric output, so only the 36 blocks on and above
// the diagonal of its 8 x 8 grid of 32 x 32 blocks are computed, from one
// operand panel (half the DMA of an ordinary tile).  In 64 x 64 super-blocks
// (a 4 x 4 grid): waves 0-3 (type A) each take diagonal super-block (d, d),
// d = wave (blocks (2d,2d), (2d,2d+1), (2d+1,2d+1)), and one half of
// super-block (1,3) or (2,3) (blocks (2+d, 6), (2+d, 7)); waves 4-7 (type B)
// each take one off-diagonal super-block, (0,1), (0,2), (0,3) or (1,2).  A
// SIMD runs one wave of each type: 5 + 4 = 9 MFMAs per k16 sub-step instead of
// 16.  Each wave reads 5 (A) or 4 (B) fragments per sub-step ("slots", any
// of the panel's eight 32-row fragments).  Every block off the 32-block
// diagonal is also written transposed, so the stored tile is whole and
// exactly symmetric.
template <bool TA>
struct DiagGeo {
  static constexpr int NSL = TA ? 5 : 4;   // fragment slots
  static constexpr int NB = TA ? 5 : 4;    // accumulator blocks
  int f[NSL];                              // fragment (32-row block) of each slot
  int br[NB], bc[NB];                      // block row / column of each accumulator
  __device__ void init(int wave) {
    if (TA) {
      const int dd = wave;                 // 0..3
      f[0] = 2 * dd; f[1] = 2 * dd + 1; f[2] = 2 + dd; f[3] = 6; f[4] = 7;
      br[0] = 2 * dd;     bc[0] = 2 * dd;
      br[1] = 2 * dd;     bc[1] = 2 * dd + 1;
      br[2] = 2 * dd + 1; bc[2] = 2 * dd + 1;
      br[3] = 2 + dd;     bc[3] = 6;
      br[4] = 2 + dd;     bc[4] = 7;
    } else {
      const int u = wave - 4;              // super-blocks (0,1) (0,2) (0,3) (1,2)
      const int I = u == 3 ? 1 : 0, J = u == 3 ? 2 : u + 1;
      f[0] = 2 * I; f[1] = 2 * I + 1; f[2] = 2 * J; f[3] = 2 * J + 1;
      br[0] = 2 * I;     bc[0] = 2 * J;
      br[1] = 2 * I;     bc[1] = 2 * J + 1;
      br[2] = 2 * I + 1; bc[2] = 2 * J;
      br[3] = 2 * I + 1; bc[3] = 2 * J + 1;
    }
  }
};

// LDS offsets of the slots' fragments (kk = 0, first read): row-major 2048 f
// (fo.rm[kk] added at the read); k-major as FragOffsets::km for 32-row block f.
template <bool PKM, int NSL>
__device__ __forceinline__ void slot_offsets(const int (&f)[NSL], int lane, uint32_t (&so)[NSL]) {
  const int G = lane >> 4, c = lane & 15, e = c >> 2, h = c & 3;
  const int kr = 8 * (G >> 1) + e;
  const int col = 16 * (G & 1) + 4 * h;
#pragma unroll
  for (int j = 0; j < NSL; ++j)
    so[j] = PKM ? (uint32_t)(kr * 512 + ((f[j] ^ e) << 6) + 2 * col) : (uint32_t)(2048 * f[j]);
}

template <bool PKM, int NSL>
__device__ __forceinline__ void read_slots(const uint8_t* stage, int kk, const uint32_t (&so)[NSL],
                                           const FragOffsets& fo, bf16x8 (&fr)[NSL]) {
#pragma unroll
  for (int j = 0; j < NSL; ++j) {
    if (!PKM) {
      fr[j] = *(const bf16x8*)(stage + so[j] + fo.rm[kk]);
    } else {
      const uint8_t* base = stage + so[j] + 8192 * kk;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MATOPT_LDS s16x4*)(base + 2048));
      fr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
}

// Step 0's slots (k-major when pkm), through a restrict stage pointer so that
// the explicit wait alone orders them after the DMA (as first_frags).
template <int NSL>
__device__ __forceinline__ void first_slots(bool pkm, const uint8_t* __restrict__ s0,
                                            const uint32_t (&sok)[NSL],
                                            const uint32_t (&so)[NSL], const FragOffsets& fo,
                                            bf16x8 (&fr)[NSL]) {
  if (pkm) read_slots<true, NSL>(s0, 0, sok, fo, fr);
  else read_slots<false, NSL>(s0, 0, so, fo, fr);
}

// MFMAs of one k16 sub-step (first operand: the column fragment, second: the
// row fragment, so that acc holds the block transposed as in mfma16).
//   type A slots: f2d, f2d+1, f2+d, f6, f7
//   type B slots: f2I, f2I+1, f2J, f2J+1
template <bool TA>
__device__ __forceinline__ void mfma_diag(f32x16 (&acc)[DiagGeo<TA>::NB],
                                          const bf16x8 (&fr)[DiagGeo<TA>::NSL]) {
  if (TA) {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[0], fr[0], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[1], fr[0], acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[1], fr[1], acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[3], fr[2], acc[3], 0, 0, 0);
    acc[4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[DiagGeo<TA>::NSL - 1], fr[2],
                                                     acc[DiagGeo<TA>::NB - 1], 0, 0, 0);
  } else {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2], fr[0], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[3], fr[0], acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2], fr[1], acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[3], fr[1], acc[3], 0, 0, 0);
  }
}

// One K step t of a diagonal tile (as kstep, P panel only): sub-step 0 on
// fragments read earlier while those of sub-step 1 are read; wait for the DMA
// of step t+1; barrier; (DP) the DMA of step t+4 into the stage of step t-1;
// sub-step 1 while the sub-step-0 fragments of step t+1 are read.  PKM / PKM1:
// the panel layout of step t / t+1 (true: k-major), with slot offsets so / so1.
template <bool PKM, bool PKM1, bool TA, int VMW, bool DP, class OpP>
__device__ __forceinline__ void kstep_diag(f32x16 (&acc)[DiagGeo<TA>::NB],
                                           bf16x8 (&fa)[DiagGeo<TA>::NSL],
                                           bf16x8 (&fb)[DiagGeo<TA>::NSL], int t, const OpP& dp,
                                           const uint32_t (&so)[DiagGeo<TA>::NSL],
                                           const uint32_t (&so1)[DiagGeo<TA>::NSL],
                                           const FragOffsets& fo, int wave,
                                           const uint8_t* __restrict__ cur,
                                           const uint8_t* __restrict__ nxt,
                                           uint8_t* __restrict__ dst_p) {
  constexpr int NSL = DiagGeo<TA>::NSL, NB = DiagGeo<TA>::NB;
  static_assert(NSL == NB, "one fragment slot per accumulator block");
  constexpr int RDS = PKM ? 2 : 1;   // LDS instructions per fragment
  constexpr int RDS1 = PKM1 ? 2 : 1;
  read_slots<PKM, NSL>(cur, 1, so, fo, fb);
  mfma_diag<TA>(acc, fa);
#pragma unroll
  for (int i = 0; i < NB; ++i) {   // NB == NSL: one fragment per MFMA
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RDS, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<VMW>();
  bar_raw();
  if (DP) dp.template issue<2>(t + NS - 1, dst_p, wave);
  read_slots<PKM1, NSL>(nxt, 0, so1, fo, fa);
  mfma_diag<TA>(acc, fb);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RDS1, 0);
    if (DP && i < 2) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one block of a diagonal tile: staged through the wave's LDS
// region (32 rows of 36 floats), written row-wise (two 16-byte items per
// lane), then (off the 32-block diagonal) transposed into the mirror block.
// Gram: value s^2 * acc.  Polynomial: a*I + b*A + c*acc with the A block
// read first (ain: this lane's two items).
template <int STAGE>
__device__ __forceinline__ void diag_block_write(float* stg, uint16_t* out, int64_t ld, int64_t r0,
                                                 int64_t c0, bool mirror, int lane, float sc,
                                                 const GemmParams& P, const u32x4 (&ain)[2]);

template <int STAGE>
__device__ __forceinline__ void diag_block_out(const f32x16& acc, float* stg, uint16_t* out,
                                               int64_t ld, int64_t r0, int64_t c0, bool mirror,
                                               int lane, float sc, const GemmParams& P,
                                               const u32x4 (&ain)[2]) {
  constexpr int PITCH = 36;
  const int frow = lane & 31, fkc = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(f32x4*)(stg + frow * PITCH + 8 * g + 4 * fkc) =
        f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  __builtin_amdgcn_wave_barrier();
  diag_block_write<STAGE>(stg, out, ld, r0, c0, mirror, lane, sc, P, ain);
}

// The write-out of a staged diagonal-tile block (32 rows of 36 floats).
template <int STAGE>
__device__ __forceinline__ void diag_block_write(float* stg, uint16_t* out, int64_t ld, int64_t r0,
                                                 int64_t c0, bool mirror, int lane, float sc,
                                                 const GemmParams& P, const u32x4 (&ain)[2]) {
  constexpr int PITCH = 36;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = lane + 64 * p;
    const int rr = q >> 2, c8 = (q & 3) * 8;
    float* src = stg + rr * PITCH + c8;
    const f32x4 v0 = *(const f32x4*)src, v1 = *(const f32x4*)(src + 4);
    f32x4 a0, a1;
    if (STAGE == 0) {
      a0 = f32x4{v0.x * sc, v0.y * sc, v0.z * sc, v0.w * sc};
      a1 = f32x4{v1.x * sc, v1.y * sc, v1.z * sc, v1.w * sc};
    } else {
      const u32x4 ai = ain[p];
      const float a = P.a, b = P.b, c = P.c;
      const int64_t dg = (r0 + rr) - (c0 + c8);   // 0..7 on the matrix diagonal
      a0 = f32x4{fmaf(b, lo_bf(ai.x), fmaf(c, v0.x, dg == 0 ? a : 0.f)),
                 fmaf(b, hi_bf(ai.x), fmaf(c, v0.y, dg == 1 ? a : 0.f)),
                 fmaf(b, lo_bf(ai.y), fmaf(c, v0.z, dg == 2 ? a : 0.f)),
                 fmaf(b, hi_bf(ai.y), fmaf(c, v0.w, dg == 3 ? a : 0.f))};
      a1 = f32x4{fmaf(b, lo_bf(ai.z), fmaf(c, v1.x, dg == 4 ? a : 0.f)),
                 fmaf(b, hi_bf(ai.z), fmaf(c, v1.y, dg == 5 ? a : 0.f)),
                 fmaf(b, lo_bf(ai.w), fmaf(c, v1.z, dg == 6 ? a : 0.f)),
                 fmaf(b, hi_bf(ai.w), fmaf(c, v1.w, dg == 7 ? a : 0.f))};
    }
    gstore<u32x4>(blk_at(out, r0 + rr, c0 + c8, ld),
                  u32x4{pack_bf2(a0.x, a0.y), pack_bf2(a0.z, a0.w), pack_bf2(a1.x, a1.y),
                        pack_bf2(a1.z, a1.w)});
    if (mirror) {   // the transposed pass reads the final values
      *(f32x4*)src = a0;
      *(f32x4*)(src + 4) = a1;
    }
  }
  if (mirror) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int q = lane + 64 * p;
      const int ic = tr_ic(q), jj = tr_jj(q);
      float vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = stg[(8 * ic + e) * PITCH + jj];
      gstore<u32x4>(blk_at(out, c0 + jj, r0 + 8 * ic, ld),
                    u32x4{pack_bf2(vv[0], vv[1]), pack_bf2(vv[2], vv[3]), pack_bf2(vv[4], vv[5]),
                          pack_bf2(vv[6], vv[7])});
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// K loop and epilogue of a diagonal tile for one wave type.  Stage 0: P = X
// rows, out A.  Stage 1: P = A rows, out B.  Both panels are row-major.
template <int STAGE, bool TA, class OpP>
__device__ __forceinline__ void diag_tile(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                          int nk, int bP, int i0, int wave, int lane,
                                          uint8_t* lds) {
  constexpr int NSL = DiagGeo<TA>::NSL, NB = DiagGeo<TA>::NB;
  constexpr int BPW = 2;   // 16 one-KB blocks of the panel over 8 waves
  DiagGeo<TA> geo;
  geo.init(wave);
  FragOffsets fo;
  fo.init(lane);
  // the panel is row-major from step bP on; before it (polynomial: the k
  // blocks left of the diagonal, read through the upper tiles) k-major
  uint32_t so[NSL], sok[NSL];
  slot_offsets<false, NSL>(geo.f, lane, so);
  slot_offsets<true, NSL>(geo.f, lane, sok);
  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  bf16x8 fa[NSL], fb[NSL];

  // prologue: panel DMA of steps 0..3, wait for step 0
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) dp.template issue<BPW>(t, lds + t * STG, wave);
  wait_vm<BPW * (NS - 2)>();
  bar_raw();
  first_slots<NSL>(bP > 0, lds, sok, so, fo, fa);
  uint32_t sc = 0;
  int t = 0;
  // steady: DMA of step t+4; in flight after t+1's: t+2, t+3.  bP (a multiple
  // of 8, at most nk - 8) lies in the steady range.
  for (; t < bP - 1; ++t) {
    kstep_diag<true, true, TA, 2 * BPW, true>(acc, fa, fb, t, dp, sok, sok, fo, wave, lds + sc,
                                              lds + stage_wrap(sc + STG),
                                              lds + stage_wrap(sc + (NS - 1) * STG));
    sc = stage_wrap(sc + STG);
  }
  if (bP > 0) {
    kstep_diag<true, false, TA, 2 * BPW, true>(acc, fa, fb, t, dp, sok, so, fo, wave, lds + sc,
                                               lds + stage_wrap(sc + STG),
                                               lds + stage_wrap(sc + (NS - 1) * STG));
    sc = stage_wrap(sc + STG);
    ++t;
  }
  for (; t < nk - NS + 1; ++t) {
    kstep_diag<false, false, TA, 2 * BPW, true>(acc, fa, fb, t, dp, so, so, fo, wave, lds + sc,
                                                lds + stage_wrap(sc + STG),
                                                lds + stage_wrap(sc + (NS - 1) * STG));
    sc = stage_wrap(sc + STG);
  }
  kstep_diag<false, false, TA, 2 * BPW, false>(acc, fa, fb, t, dp, so, so, fo, wave, lds + sc,
                                               lds + stage_wrap(sc + STG), lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_diag<false, false, TA, BPW, false>(acc, fa, fb, t, dp, so, so, fo, wave, lds + sc,
                                           lds + stage_wrap(sc + STG), lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_diag<false, false, TA, 0, false>(acc, fa, fb, t, dp, so, so, fo, wave, lds + sc,
                                         lds + stage_wrap(sc + STG), lds);
  sc = stage_wrap(sc + STG);
  // last step (nk-1)
  read_slots<false, NSL>(lds + sc, 1, so, fo, fb);
  mfma_diag<TA>(acc, fa);
  mfma_diag<TA>(acc, fb);

  // epilogue inputs (polynomial: the A blocks at the output positions)
  const int64_t ld = d.mp;
  u32x4 ain[NB][2];
  if (STAGE == 1) {
    const uint16_t* A = (const uint16_t*)d.a;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = lane + 64 * p;
        ain[b][p] = gload<u32x4>(blk_at(A, i0 + 32 * geo.br[b] + (q >> 2),
                                        i0 + 32 * geo.bc[b] + (q & 3) * 8, ld));
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();
  float* stg = (float*)(lds + wave * (32 * 36 * 4));
  uint16_t* out = STAGE == 0 ? (uint16_t*)d.a : (uint16_t*)d.b;
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const float sc2 = s_first * s_first;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    diag_block_out<STAGE>(acc[b], stg, out, ld, i0 + 32 * geo.br[b], i0 + 32 * geo.bc[b],
                          geo.br[b] != geo.bc[b], lane, sc2, P, ain[b]);
}

// Two diagonal tiles of one matrix in one workgroup (a "diagonal pair"): the
// first tile's operand panel fills the P slot of every stage, the second's
// the Q slot, with the ordinary DMA schedule.  Each wave takes both pieces of
// index d = wave & 3 of its tile (the type-A piece, 5 blocks, and the type-B
// piece, 4 blocks, as in DiagGeo): waves 0-3 the first tile, waves 4-7 the
// second.  That is 9 MFMAs per wave and k16 sub-step, 18 per SIMD, about 1.125
// ordinary tiles, so the pair keeps pace with the other tiles of the matrix,
// which read the same operand panels through L2 at the same time (a single
// diagonal tile runs ahead of them and fetches its panel on its own).
struct PairGeo {
  static constexpr int NSL = 9, NB = 9;
  int f[NSL];              // fragment (32-row block of the wave's panel) per slot
  int br[NB], bc[NB];      // block row / column per accumulator
  __device__ void init(int d) {
    DiagGeo<true> a;
    a.init(d);
    DiagGeo<false> b;
    b.init(d + 4);
#pragma unroll
    for (int j = 0; j < 5; ++j) { f[j] = a.f[j]; br[j] = a.br[j]; bc[j] = a.bc[j]; }
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[5 + j] = b.f[j]; br[5 + j] = b.br[j]; bc[5 + j] = b.bc[j]; }
  }
};

// The type-A MFMAs on slots 0-4 (accumulators 0-4), the type-B ones on slots
// 5-8 (accumulators 5-8); operand order as in mfma_diag.
__device__ __forceinline__ void mfma_pair(f32x16 (&acc)[9], const bf16x8 (&fr)[9]) {
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[0], fr[0], acc[0], 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[1], fr[0], acc[1], 0, 0, 0);
  acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[1], fr[1], acc[2], 0, 0, 0);
  acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[3], fr[2], acc[3], 0, 0, 0);
  acc[4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[4], fr[2], acc[4], 0, 0, 0);
  acc[5] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[7], fr[5], acc[5], 0, 0, 0);
  acc[6] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[8], fr[5], acc[6], 0, 0, 0);
  acc[7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[7], fr[6], acc[7], 0, 0, 0);
  acc[8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[8], fr[6], acc[8], 0, 0, 0);
}

// One K step of a diagonal pair: the DMA of kstep (both operands), the
// fragment reads and MFMAs of the wave's 9 slots.
template <bool PKM, int VMW, bool DQ, bool DP, class OpP, class OpQ>
__device__ __forceinline__ void kstep_pair(f32x16 (&acc)[9], bf16x8 (&fa)[9], bf16x8 (&fb)[9],
                                           int t, const OpP& dp, const OpQ& dq,
                                           const uint32_t (&so)[9], const FragOffsets& fo,
                                           int wave, const uint8_t* __restrict__ cur,
                                           const uint8_t* __restrict__ nxt,
                                           uint8_t* __restrict__ dst_q,
                                           uint8_t* __restrict__ dst_p) {
  constexpr int RDS = PKM ? 2 : 1;
  read_slots<PKM, 9>(cur, 1, so, fo, fb);
  if (DQ) dq.template issue<2>(t + NS - 2, dst_q + OPB, wave);
  mfma_pair(acc, fa);
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RDS, 0);
    if (DQ && (i == 3 || i == 7)) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<VMW>();
  bar_raw();
  if (DP) dp.template issue<2>(t + NS - 1, dst_p, wave);
  read_slots<PKM, 9>(nxt, 0, so, fo, fa);
  mfma_pair(acc, fb);
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RDS, 0);
    if (DP && (i == 3 || i == 7)) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// K loop (the schedule of kloop with bP = 0) and epilogue of a diagonal pair
// with tiles at block rows i0 (P slot) and i1 (Q slot).
template <int STAGE, class OpP, class OpQ>
__device__ __forceinline__ void diag_pair(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                          const OpQ& dq, int nk, int i0, int i1, int wave,
                                          int lane, uint8_t* lds) {
  constexpr bool PKM = false;   // the panels are row-major in both stages
  constexpr int BPW = 2, DPS = 2 * BPW;
  PairGeo geo;
  geo.init(wave & 3);
  FragOffsets fo;
  fo.init(lane);
  uint32_t so[9];
  slot_offsets<PKM, 9>(geo.f, lane, so);
  const uint32_t panel = wave < 4 ? 0u : (uint32_t)OPB;
#pragma unroll
  for (int j = 0; j < 9; ++j) so[j] += panel;
  f32x16 acc[9];
#pragma unroll
  for (int b = 0; b < 9; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  bf16x8 fa[9], fb[9];

  // prologue (as kprologue): steps 0 .. NS-3 and the P half of step NS-2
  dp.template issue<BPW>(0, lds, wave);
  dq.template issue<BPW>(0, lds + OPB, wave);
#pragma unroll
  for (int t = 1; t < NS - 2; ++t) {
    dp.template issue<BPW>(t, lds + t * STG, wave);
    dq.template issue<BPW>(t, lds + t * STG + OPB, wave);
  }
  dp.template issue<BPW>(NS - 2, lds + (NS - 2) * STG, wave);
  wait_vm<DPS * (NS - 3) + BPW>();
  bar_raw();
  read_slots<PKM, 9>(lds, 0, so, fo, fa);
  uint32_t sc = 0;
  int t = 0;
  for (; t < nk - NS + 1; ++t) {
    kstep_pair<PKM, 2 * DPS, true, true>(acc, fa, fb, t, dp, dq, so, fo, wave, lds + sc,
                                         lds + stage_wrap(sc + STG),
                                         lds + stage_wrap(sc + (NS - 2) * STG),
                                         lds + stage_wrap(sc + (NS - 1) * STG));
    sc = stage_wrap(sc + STG);
  }
  kstep_pair<PKM, 2 * DPS, true, false>(acc, fa, fb, t, dp, dq, so, fo, wave, lds + sc,
                                        lds + stage_wrap(sc + STG),
                                        lds + stage_wrap(sc + (NS - 2) * STG), lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_pair<PKM, DPS, false, false>(acc, fa, fb, t, dp, dq, so, fo, wave, lds + sc,
                                     lds + stage_wrap(sc + STG), lds, lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_pair<PKM, 0, false, false>(acc, fa, fb, t, dp, dq, so, fo, wave, lds + sc,
                                   lds + stage_wrap(sc + STG), lds, lds);
  sc = stage_wrap(sc + STG);
  read_slots<PKM, 9>(lds + sc, 1, so, fo, fb);
  mfma_pair(acc, fa);
  mfma_pair(acc, fb);

  const int64_t ld = d.mp;
  const int r0 = wave < 4 ? i0 : i1;   // this wave's tile
  u32x4 ain[9][2];
  if (STAGE == 1) {
    const uint16_t* A = (const uint16_t*)d.a;
#pragma unroll
    for (int b = 0; b < 9; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = lane + 64 * p;
        ain[b][p] = gload<u32x4>(blk_at(A, r0 + 32 * geo.br[b] + (q >> 2),
                                        r0 + 32 * geo.bc[b] + (q & 3) * 8, ld));
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();
  float* stg = (float*)(lds + wave * (32 * 36 * 4));
  uint16_t* out = STAGE == 0 ? (uint16_t*)d.a : (uint16_t*)d.b;
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const float sc2 = s_first * s_first;
#pragma unroll
  for (int b = 0; b < 9; ++b)
    diag_block_out<STAGE>(acc[b], stg, out, ld, r0 + 32 * geo.br[b], r0 + 32 * geo.bc[b],
                          geo.br[b] != geo.bc[b], lane, sc2, P, ain[b]);
}

// MFMAs with RD LDS reads (at most three per MFMA) and ND DMA instructions
// (at most one per MFMA) spread evenly among NM of them.
template <int NM, int RD, int ND>
__device__ __forceinline__ void sched_spread() {
  static_assert(RD <= 3 * NM && ND <= NM, "spread");
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    const int nr = (i + 1) * RD / NM - i * RD / NM;
    if (nr >= 1) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
    if (nr >= 2) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
    if (nr >= 3) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
    if ((i + 1) * ND / NM > i * ND / NM) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// A diagonal pair on the 16 x 16 x 32 engine (the blocks and slots of
// PairGeo; row-major panels).  Each 32-row slot is two 16-row slab fragments
// over the whole K step, each 32 x 32 block 2 x 2 slabs; a block on the
// 32-block diagonal computes only its upper three slabs (its lower slab is
// written as the mirror of the upper right one), 34 MFMAs per wave and step
// instead of the 36 of the 32 x 32 form.  A step runs in two halves: the
// type-A blocks (0-4, slots 0-4) while slots 5-8 of the step are read, then
// after the barrier the type-B blocks (5-8) while slots 0-4 of the next step
// are read.
__device__ __forceinline__ void mfma_pair16a(f32x4 (&acc)[9][2][2], const bf16x8 (&fr)[9][2]) {
  // blocks 0 and 2 are on the diagonal (row slot == column slot)
  constexpr int R[5] = {0, 0, 1, 2, 2}, C[5] = {0, 1, 1, 3, 4};
#pragma unroll
  for (int b = 0; b < 5; ++b)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        if ((b == 0 || b == 2) && i2 == 1 && j2 == 0) continue;
        acc[b][i2][j2] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[C[b]][j2], fr[R[b]][i2], acc[b][i2][j2], 0, 0, 0);
      }
}

__device__ __forceinline__ void mfma_pair16b(f32x4 (&acc)[9][2][2], const bf16x8 (&fr)[9][2]) {
  constexpr int R[4] = {5, 5, 6, 6}, C[4] = {7, 8, 7, 8};
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2)
        acc[5 + b][i2][j2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            fr[C[b]][j2], fr[R[b]][i2], acc[5 + b][i2][j2], 0, 0, 0);
}

// Slots J0 .. J1-1 (both slab halves) of a row-major panel stage.
template <int J0, int J1>
__device__ __forceinline__ void read_pair16(const uint8_t* __restrict__ stage,
                                            const uint32_t (&so)[9], bf16x8 (&fr)[9][2]) {
#pragma unroll
  for (int j = J0; j < J1; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) fr[j][h] = *(const bf16x8*)(stage + so[j] + 1024 * h);
}

template <int VMW, bool DQ, bool DP, class OpP, class OpQ>
__device__ __forceinline__ void kstep_pair16(f32x4 (&acc)[9][2][2], bf16x8 (&fr)[9][2], int t,
                                             const OpP& dp, const OpQ& dq,
                                             const uint32_t (&so)[9], int wave,
                                             const uint8_t* __restrict__ cur,
                                             const uint8_t* __restrict__ nxt,
                                             uint8_t* __restrict__ dst_q,
                                             uint8_t* __restrict__ dst_p) {
  read_pair16<5, 9>(cur, so, fr);
  if (DQ) dq.template issue<2>(t + NS - 2, dst_q + OPB, wave);
  mfma_pair16a(acc, fr);
  sched_spread<18, 8, DQ ? 2 : 0>();
  wait_vm<VMW>();
  bar_raw();
  if (DP) dp.template issue<2>(t + NS - 1, dst_p, wave);
  read_pair16<0, 5>(nxt, so, fr);
  mfma_pair16b(acc, fr);
  sched_spread<16, 10, DP ? 2 : 0>();
}

template <int STAGE, class OpP, class OpQ>
__device__ __forceinline__ void diag_pair16(const MatDesc& d, const GemmParams& P, const OpP& dp,
                                            const OpQ& dq, int nk, int i0, int i1, int wave,
                                            int lane, uint8_t* lds) {
  constexpr int BPW = 2, DPS = 2 * BPW;
  PairGeo geo;
  geo.init(wave & 3);
  const uint32_t panel = wave < 4 ? 0u : (uint32_t)OPB;
  const uint32_t rm = rm_off(lane & 15, oct16(lane >> 4));
  uint32_t so[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) so[j] = 2048u * geo.f[j] + panel + rm;
  f32x4 acc[9][2][2];
#pragma unroll
  for (int b = 0; b < 9; ++b)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) acc[b][i2][j2] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 fr[9][2];

  // prologue (as kprologue): steps 0 .. NS-3 and the P half of step NS-2
  dp.template issue<BPW>(0, lds, wave);
  dq.template issue<BPW>(0, lds + OPB, wave);
#pragma unroll
  for (int t = 1; t < NS - 2; ++t) {
    dp.template issue<BPW>(t, lds + t * STG, wave);
    dq.template issue<BPW>(t, lds + t * STG + OPB, wave);
  }
  dp.template issue<BPW>(NS - 2, lds + (NS - 2) * STG, wave);
  wait_vm<DPS * (NS - 3) + BPW>();
  bar_raw();
  read_pair16<0, 5>(lds, so, fr);
  uint32_t sc = 0;
  int t = 0;
  for (; t < nk - NS + 1; ++t) {
    kstep_pair16<2 * DPS, true, true>(acc, fr, t, dp, dq, so, wave, lds + sc,
                                      lds + stage_wrap(sc + STG),
                                      lds + stage_wrap(sc + (NS - 2) * STG),
                                      lds + stage_wrap(sc + (NS - 1) * STG));
    sc = stage_wrap(sc + STG);
  }
  kstep_pair16<2 * DPS, true, false>(acc, fr, t, dp, dq, so, wave, lds + sc,
                                     lds + stage_wrap(sc + STG),
                                     lds + stage_wrap(sc + (NS - 2) * STG), lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_pair16<DPS, false, false>(acc, fr, t, dp, dq, so, wave, lds + sc,
                                  lds + stage_wrap(sc + STG), lds, lds);
  sc = stage_wrap(sc + STG);
  ++t;
  kstep_pair16<0, false, false>(acc, fr, t, dp, dq, so, wave, lds + sc,
                                lds + stage_wrap(sc + STG), lds, lds);
  sc = stage_wrap(sc + STG);
  read_pair16<5, 9>(lds + sc, so, fr);
  mfma_pair16a(acc, fr);
  mfma_pair16b(acc, fr);

  const int64_t ld = d.mp;
  const int r0 = wave < 4 ? i0 : i1;   // this wave's tile
  u32x4 ain[9][2];
  if (STAGE == 1) {
    const uint16_t* A = (const uint16_t*)d.a;
#pragma unroll
    for (int b = 0; b < 9; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = lane + 64 * p;
        ain[b][p] = gload<u32x4>(blk_at(A, r0 + 32 * geo.br[b] + (q >> 2),
                                        r0 + 32 * geo.bc[b] + (q & 3) * 8, ld));
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();
  constexpr int PITCH = 36;
  float* stg = (float*)(lds + wave * (32 * PITCH * 4));
  uint16_t* out = STAGE == 0 ? (uint16_t*)d.a : (uint16_t*)d.b;
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  const float sc2 = s_first * s_first;
  const int q = lane >> 4, rr = lane & 15;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool dblk = b == 0 || b == 2;   // on the 32-block diagonal
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        if (dblk && i2 == 1 && j2 == 0) continue;
        *(f32x4*)(stg + (16 * i2 + rr) * PITCH + 16 * j2 + 4 * q) = acc[b][i2][j2];
      }
    if (dblk) {   // lower left slab = the upper right one transposed
#pragma unroll
      for (int e = 0; e < 4; ++e) stg[(16 + 4 * q + e) * PITCH + rr] = acc[b][0][1][e];
    }
    __builtin_amdgcn_wave_barrier();
    diag_block_write<STAGE>(stg, out, ld, r0 + 32 * geo.br[b], r0 + 32 * geo.bc[b],
                            geo.br[b] != geo.bc[b], lane, sc2, P, ain[b]);
  }
}

// One kernel per stage (and, for apply, per output kind), so that each carries
// only its own operand layouts and epilogue.
// NW = 8 (every stage, by default): eight waves of 128 x 64, two per SIMD, so
// that one wave's MFMAs run while the other waits on LDS, DMA or the barrier;
// the DMA of a step is spread over all eight waves (two 1 KB blocks per
// operand each).  NW = 4 (four waves of 128 x 128, one per SIMD) remains a
// build-time alternative (MATOPT_*_WAVES).
template <int STAGE, int OUT, int NW, bool MIR>
__device__ __forceinline__ void gemm_tile(const GemmParams& P, uint8_t* lds) {
  static_assert(NW == 4 || NW == 8, "layout");
  constexpr int NBJ = NW == 4 ? 4 : 2;   // 32-column blocks per wave
  constexpr int WN = 32 * NBJ;           // columns per wave
  constexpr int BPW = NW == 4 ? 4 : 2;   // DMA blocks per wave and operand
  // Gram: P = Q = X rows.  A and B hold their upper tiles only (diagonal
  // tiles whole), so a row block of either is read k-major, through the upper
  // tiles above it, for the k blocks left of its diagonal block, and
  // row-major from there on.  Polynomial: P = rows i0.. of A, Q = rows j0.. of
  // A (A's columns j0.., A being symmetric), both read that way; every tile
  // ends its K loop with both operands row-major.  Apply: P = B rows; Q = X
  // columns (k-major).
  constexpr int PK = STAGE == 0 ? OP_RM : OP_SPLIT;
  constexpr int QK = STAGE == 0 ? OP_RM : STAGE == 1 ? OP_SPLIT : OP_KM;
  constexpr bool PF = false;        // P layout (from its diagonal block on)
  constexpr bool QF = STAGE == 2;   // Q layout (polynomial: from its diagonal block on)
  constexpr bool QS = STAGE == 1;   // Q k-major before step bQ

  const GemmTile tile = P.tiles[blockIdx.x];
  if (tile.mat < 0) return;   // idle entry padding an XCD stream
  const MatDesc d = P.mats[tile.mat];
  // tj < 0 marks a diagonal pair (Gram and polynomial tables only): block rows
  // ti and -tj-1
  const bool pair = tile.tj < 0;
  const int i0 = tile.ti * BM, j0 = pair ? i0 : tile.tj * BM;
  const int64_t mp = d.mp, np = d.np;
  // memory safety: an entry outside the matrix's output grid does nothing
  if (i0 < 0 || i0 + BM > mp || j0 + BM > (STAGE == 2 ? np : mp) || (pair && STAGE == 2)) return;
  const uint16_t* xcur = (const uint16_t*)(P.first ? d.x0in : P.cur ? d.x[1] : d.x[0]);
  uint16_t* xnext = (uint16_t*)(P.cur ? d.x[0] : d.x[1]);
  // split precision, apply after the first iteration: Q runs over the stacked
  // [hi; lo] iterate (K = 2 mp) and P over B twice (B is stored whole then)
  const bool ksplit = STAGE == 2 && P.split && !P.first;
  // K is a multiple of 256, so nk >= 8 > NS - 1
  const int nk = (int)(STAGE == 0 ? np : ksplit ? 2 * mp : mp) / BK;
  // polynomial and apply: P is k-major for steps t < bP (never for the
  // split-precision apply: B whole); polynomial: Q for steps t < bQ
  // (bP <= bQ <= nk - 8)
  const int bP = STAGE == 0 || (STAGE == 2 && P.split) ? 0 : i0 / BK;
  const int bQ = STAGE == 1 ? j0 / BK : 0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  OperandDma<PK> dp;
  OperandDma<QK> dq;
  // the first iteration reads X0 (V itself or the prep copy) in the plain
  // layout; later ones read the iterate the previous apply stored in blocks
  const bool xblk = !P.first;
  if (STAGE == 0) {
    dp.init(xcur, np, i0, 0, lane, xblk);
    dq.init(xcur, np, j0, 0, lane, xblk);
  } else if (STAGE == 1) {
    dp.init((const uint16_t*)d.a, mp, i0, bP, lane, true);
    dq.init((const uint16_t*)d.a, mp, j0, bQ, lane, true);
  } else {
    dp.init((const uint16_t*)d.b, mp, i0, bP, lane, true);
    if (ksplit) dp.t_wrap = (int)(mp / BK);
    dq.init(xcur, np, j0, nk, lane, xblk);
  }

  if constexpr ((STAGE == 0 || STAGE == 1) && NW == 8 && MATOPT_DIAG_TILES) {
    if (pair) {   // only the Gram's tables hold diagonal pairs
      if constexpr (STAGE == 0) {
        const int i1 = (-tile.tj - 1) * BM;
        if (i1 < 0 || i1 + BM > mp) return;
        OperandDma<PK> dq1;
        dq1.init(xcur, np, i1, 0, lane, xblk);
        if constexpr (MATOPT_GRAM_MFMA16) diag_pair16<STAGE>(d, P, dp, dq1, nk, i0, i1, wave, lane, lds);
        else diag_pair<STAGE>(d, P, dp, dq1, nk, i0, i1, wave, lane, lds);
      }
      return;
    }
    if (tile.ti == tile.tj) {   // wave-uniform (one tile per workgroup)
      if (wave < 4) diag_tile<STAGE, true>(d, P, dp, nk, bP, i0, wave, lane, lds);
      else diag_tile<STAGE, false>(d, P, dp, nk, bP, i0, wave, lane, lds);
      return;
    }
  }

  WaveGeo g;
  g.wi0 = NW == 4 ? (wave >> 1) * 128 : (wave >> 2) * 128;   // wave sub-tile origin (rows)
  g.wj0 = NW == 4 ? (wave & 1) * 128 : (wave & 3) * 64;      // wave sub-tile origin (cols)
  g.frow = lane & 31;
  g.fkc = lane >> 5;
  if constexpr (STAGE == 2 && NW == 8 && MATOPT_APPLY_MFMA16 && MATOPT_PAIR_APPLY) {
    apply_tile16<OUT>(d, P, dp, dq, g, nk, bP, xnext, i0, j0, wave, lane, lds);
    return;
  }
  if constexpr (STAGE == 0 && NW == 8 && MATOPT_GRAM_MFMA16 && !MATOPT_PAIR_GRAM) {
    gram_tile16(d, P, dp, dq, g, nk, i0, j0, wave, lane, lds);
    return;
  }
  if constexpr (STAGE == 1 && NW == 8 && MIR && MATOPT_POLY_MFMA16 && !MATOPT_PAIR_POLY) {
    poly_mirror_tile16<!(NW == 8 && MATOPT_DIAG_TILES)>(d, P, dp, dq, g, nk, bP, bQ, i0, j0, wave,
                                                        lane, lds);
    return;
  }
  if constexpr (STAGE == 1 && NW == 8 && !MIR && MATOPT_POLY_MFMA16 && !MATOPT_PAIR_POLY) {
    poly_tile16<!(NW == 8 && MATOPT_DIAG_TILES)>(d, P, dp, dq, g, nk, bP, bQ, i0, j0, wave, lane,
                                                 lds);
    return;
  }
  FragOffsets fo;
  fo.init(lane);
  if (NW == 8) fo.init_q64(lane, g.wj0);

  KState<NBJ> k;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) k.acc[bi][bj][r] = 0.f;
  constexpr bool PAIRED = STAGE == 0 ? MATOPT_PAIR_GRAM : STAGE == 1 ? MATOPT_PAIR_POLY
                                                                     : MATOPT_PAIR_APPLY;
  static_assert(!(PAIRED && QS), "the paired schedule keeps one Q layout");
  // diagonal polynomial tiles take this path unless diag_tile handles them
  constexpr bool QEQ = !(NW == 8 && MATOPT_DIAG_TILES);
  if constexpr (PAIRED) kloop2<PF, QF, NBJ, BPW>(k, nk, bP, dp, dq, g, fo, wave, lds);
  else kloop<PF, QF, QS, QEQ, NBJ, BPW>(k, nk, bP, bQ, dp, dq, g, fo, wave, lds);

  // last K step (its fragments are read); the first epilogue stripe is
  // fetched meanwhile
  const int64_t ep_ld = mp;
  const uint16_t* ep_src = (const uint16_t*)d.a;
  u32x4 ecur[Ep<WN>::IPL];
  u32x2 afirst[NBJ][4];
  mfma16<NBJ>(k.acc, k.pa, k.qa);
  if (STAGE == 1 && NW == 8 && !MIR)
    poly_a_stripe<NBJ>((const uint16_t*)d.a, mp, i0 + g.wi0, j0 + g.wj0, lane, afirst);
  else if (STAGE == 1)
    prefetch_stripe<WN>(ep_src, ep_ld, i0 + g.wi0, j0 + g.wj0, lane, ecur);
  mfma16<NBJ>(k.acc, k.pb, k.qb);
  if (STAGE == 1 && NW == 8 && !MIR) {
    poly_store_direct<NBJ>(k.acc, (uint16_t*)d.b, (const uint16_t*)d.a, mp, i0 + g.wi0, j0 + g.wj0,
                           lane, P.a, P.b, P.c, afirst);
    return;
  }
  if (STAGE == 2 && OUT == OUT_NEXT_X) {
    const float s_first = P.first ? gload<float>(d.xs) : 1.f;
    if (P.split)
      store_acc_direct_split<NBJ>(k.acc, xnext, np, i0 + g.wi0, j0 + g.wj0, lane, s_first,
                                  (int64_t)mp * np);
    else
      store_acc_direct<NBJ>(k.acc, xnext, np, i0 + g.wi0, j0 + g.wj0, lane, s_first);
    return;
  }
  if (STAGE == 0) {   // an upper tile of A, scaled by s^2 on the first iteration
    const float s_first = P.first ? gload<float>(d.xs) : 1.f;
    store_acc_direct<NBJ>(k.acc, (uint16_t*)d.a, mp, i0 + g.wi0, j0 + g.wj0, lane,
                          s_first * s_first);
    return;
  }
  if constexpr (STAGE != 0) {
  // all fragment reads done (consumed above): the stages become epilogue staging
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  bar_raw();

  uint16_t* out = STAGE == 1 ? (uint16_t*)d.b : xnext;
  const int64_t ld_out = STAGE == 2 ? np : mp;
  const float s_first = P.first ? gload<float>(d.xs) : 1.f;
  epilogue<STAGE, OUT, NBJ, MIR>(d, P, k.acc, (float*)(lds + wave * Ep<WN>::WAVE_BYTES), ep_src, ep_ld, out,
                       ld_out, i0 + g.wi0, j0 + g.wj0, lane, g.frow, g.fkc, s_first,
                       ecur);
  }
}

// The kernel: one tile per workgroup (MIR: the polynomial also writes B's
// mirror tiles, for the split-precision apply).  With P.clk set (profiling only), the
// first lane of each workgroup also adds the shader-clock ticks (s_memtime)
// and the 100 MHz real-time ticks (s_memrealtime) that its tile took to
// P.clk[0] and P.clk[1] -- their ratio is the clock the tiles ran at.
template <int STAGE, int OUT, int NW, bool MIR = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu(NW / 4, NW / 4)))
void ns_gemm_bf16_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  const bool clk = P.clk != nullptr;
  uint64_t t0 = 0, r0 = 0;
  if (clk) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  gemm_tile<STAGE, OUT, NW, MIR>(P, lds);
  if (clk && threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    atomicAdd(&P.clk[0], (unsigned long long)(t1 - t0));
    atomicAdd(&P.clk[1], (unsigned long long)(r1 - r0));
  }
}

// ------------------------------------------- persistent non-final apply
// X' = B X for every iteration but the last (iterate stored in blocks from
// registers, LDS idle after the K loop).  Workgroup w walks XCD stream
// x = w mod 8 (table positions 8k + x) at k = w/8, w/8 + G, w/8 + 2G, ...
// (G workgroups per stream, at most one per compute unit of the XCD), so
// that the tiles running together on an XCD stay consecutive in its stream,
// as with one tile per workgroup.  Between two tiles nothing waits on the
// epilogue: once every wave has read the last K step's fragments, the next
// tile's prologue DMA is issued, then the finished tile's accumulators are
// stored behind it, and the next K loop starts as soon as its first step has
// landed (the stores may stay in flight through its step 0).

// Tile and matrix tables are read through the constant address space
// (scalar loads: they are not written while the kernel runs).
#define MATOPT_CAS __attribute__((address_space(4)))

struct ApplyTask {
  const uint16_t* b;    // B, blocked, mp x mp
  const uint16_t* xc;   // current iterate (plain X0 on the first iteration)
  uint16_t* out;        // next iterate: this wave's 32 x 32 block origin
  int32_t mp, np, i0, j0;
  float s;              // Frobenius scale on the first iteration, else 1
};

// Table entry pos as a task; false for idle or out-of-range entries.
__device__ __forceinline__ bool apply_task(const GemmParams& P, int pos, const WaveGeo& g,
                                           ApplyTask& t) {
  const MATOPT_CAS GemmTile& tile = ((const MATOPT_CAS GemmTile*)P.tiles)[pos];
  const int mat = tile.mat, ti = tile.ti, tj = tile.tj;
  if (mat < 0 || tj < 0) return false;
  const MATOPT_CAS MatDesc& d = ((const MATOPT_CAS MatDesc*)P.mats)[mat];
  t.mp = d.mp;
  t.np = d.np;
  t.i0 = ti * BM;
  t.j0 = tj * BM;
  if (t.i0 < 0 || t.i0 + BM > t.mp || t.j0 + BM > t.np) return false;
  t.b = (const uint16_t*)d.b;
  t.xc = (const uint16_t*)(P.first ? d.x0in : P.cur ? d.x[1] : d.x[0]);
  uint16_t* xn = (uint16_t*)(P.cur ? d.x[0] : d.x[1]);
  const int64_t nb = t.np / 32;
  t.out = xn + (((int64_t)(t.i0 + g.wi0) >> 5) * nb + ((t.j0 + g.wj0) >> 5)) * 1024;
  t.s = P.first ? *(const MATOPT_CAS float*)d.xs : 1.f;
  return true;
}

__device__ __forceinline__ void apply_persist(const GemmParams& P, uint8_t* lds) {
  constexpr int NBJ = 2, BPW = 2;
  constexpr int NST = 2 * 4 * NBJ;   // store instructions per wave and tile (bf16 iterate)
  const int xcd = (int)(blockIdx.x & 7);
  const int G = (int)(gridDim.x >> 3);
  const int L = P.n_tiles >> 3;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WaveGeo g;
  g.wi0 = (wave >> 2) * 128;
  g.wj0 = (wave & 3) * 64;
  g.frow = lane & 31;
  g.fkc = lane >> 5;
  FragOffsets fo;
  fo.init(lane);
  fo.init_q64(lane, g.wj0);

  int kpos = (int)(blockIdx.x >> 3);
  ApplyTask cur;
  bool have = false;
  for (; kpos < L; kpos += G)
    if (apply_task(P, 8 * kpos + xcd, g, cur)) {
      have = true;
      break;
    }
  if (!have) return;

  const bool xblk = !P.first;
  const bool ksplit = P.split && !P.first;
  OperandDma<OP_SPLIT> dp;
  OperandDma<OP_KM> dq;
  int nk = 0, bP = 0;
  auto setup = [&](const ApplyTask& t) {
    // split precision: K runs over the stacked [hi; lo] iterate, P over B twice
    nk = (ksplit ? 2 * t.mp : t.mp) / BK;
    bP = P.split ? 0 : t.i0 / BK;
    dp.init(t.b, t.mp, t.i0, bP, lane, true);
    if (ksplit) dp.t_wrap = t.mp / BK;
    dq.init(t.xc, t.np, t.j0, nk, lane, xblk);
  };
  setup(cur);
  kprologue2_issue<BPW>(dp, dq, wave, lds);

  KState<NBJ> k;
  bool pend = false;
  for (;;) {
    ApplyTask nx;
    bool more = false;
    for (int kn = kpos + G; kn < L; kn += G)
      if (apply_task(P, 8 * kn + xcd, g, nx)) {
        more = true;
        kpos = kn;
        break;
      }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
        for (int r = 0; r < 16; ++r) k.acc[bi][bj][r] = 0.f;
    kloop2_rest<false, true, NBJ, BPW, NST>(k, nk, bP, dp, dq, g, fo, wave, lds, pend);
    mfma16<NBJ>(k.acc, k.pa, k.qa);
    mfma16<NBJ>(k.acc, k.pb, k.qb);
    if (more) {
      // every wave has read its last fragments: the stages are free
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bar_raw();
      setup(nx);
      kprologue2_issue<BPW>(dp, dq, wave, lds);
    }
    const int64_t nb = cur.np / 32;
    uint16_t* base = cur.out + (lane & 31) * 32 + 8 * (lane >> 5);
    if (P.split) {   // the stacked low part starts mp x np elements further on
      const int64_t lo_off = (int64_t)cur.mp * cur.np;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) {
          float v[16], lo[16];
          split_parts(k.acc[bi][bj], cur.s, v, lo);
          store_block_direct(v, base + (bi * nb + bj) * 1024);
          store_block_direct(lo, base + lo_off + (bi * nb + bj) * 1024);
        }
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = cur.s * k.acc[bi][bj][r];
          store_block_direct(v, base + (bi * nb + bj) * 1024);
        }
    }
    if (!more) break;
    cur = nx;
    pend = true;
  }
}

// apply_persist on the 16 x 16 x 32 engine.
__device__ __forceinline__ void apply_persist16(const GemmParams& P, uint8_t* lds) {
  constexpr int BPW = 2;
  constexpr int NST = 16;   // store instructions per wave and tile (bf16 iterate)
  const int xcd = (int)(blockIdx.x & 7);
  const int G = (int)(gridDim.x >> 3);
  const int L = P.n_tiles >> 3;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WaveGeo g;
  g.wi0 = (wave >> 2) * 128;
  g.wj0 = (wave & 3) * 64;
  g.frow = lane & 31;
  g.fkc = lane >> 5;
  Frag16 f;
  f.init(lane, g.wj0);

  int kpos = (int)(blockIdx.x >> 3);
  ApplyTask cur;
  bool have = false;
  for (; kpos < L; kpos += G)
    if (apply_task(P, 8 * kpos + xcd, g, cur)) {
      have = true;
      break;
    }
  if (!have) return;

  const bool xblk = !P.first;
  const bool ksplit = P.split && !P.first;
  OperandDma<OP_SPLIT> dp;
  OperandDma<OP_KM> dq;
  int nk = 0, bP = 0;
  auto setup = [&](const ApplyTask& t) {
    nk = (ksplit ? 2 * t.mp : t.mp) / BK;
    bP = P.split ? 0 : t.i0 / BK;
    dp.init(t.b, t.mp, t.i0, bP, lane, true);
    if (ksplit) dp.t_wrap = t.mp / BK;
    dq.init(t.xc, t.np, t.j0, nk, lane, xblk);
  };
  setup(cur);
  kprologue2_issue<BPW>(dp, dq, wave, lds);

  KState16 k;
  bool pend = false;
  for (;;) {
    ApplyTask nx;
    bool more = false;
    for (int kn = kpos + G; kn < L; kn += G)
      if (apply_task(P, 8 * kn + xcd, g, nx)) {
        more = true;
        kpos = kn;
        break;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) k.acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    kloop16_rest<false, BPW, NST>(k, nk, bP, dp, dq, g, f, wave, lds, pend);
    mfma_half16<0>(k.acc, k.pa, k.qb);
    mfma_half16<4>(k.acc, k.pb, k.qb);
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bar_raw();
      setup(nx);
      kprologue2_issue<BPW>(dp, dq, wave, lds);
    }
    store_acc16(k.acc, cur.out, cur.np / 32, lane, cur.s, P.split, (int64_t)cur.mp * cur.np);
    if (!more) break;
    cur = nx;
    pend = true;
  }
}

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu(NW / 4, NW / 4)))
void ns_apply_persist_kernel(GemmParams P) {
  static_assert(NW == 8, "eight-wave layout only");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  const bool clk = P.clk != nullptr;
  uint64_t t0 = 0, r0 = 0;
  if (clk) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  if (MATOPT_APPLY_MFMA16) apply_persist16(P, lds);
  else apply_persist(P, lds);
  if (clk && threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    atomicAdd(&P.clk[0], (unsigned long long)(t1 - t0));
    atomicAdd(&P.clk[1], (unsigned long long)(r1 - r0));
  }
}

}  // namespace

#ifndef MATOPT_APPLY_WAVES
#define MATOPT_APPLY_WAVES 8
#endif
#ifndef MATOPT_GRAM_WAVES
#define MATOPT_GRAM_WAVES 8
#endif
#ifndef MATOPT_POLY_WAVES
#define MATOPT_POLY_WAVES 8
#endif
#ifndef MATOPT_FINAL_WAVES
#define MATOPT_FINAL_WAVES 8
#endif

// How the bf16 Gram (stage 0) and polynomial (stage 1) launches treat the
// diagonal tiles of their tables: 0 computes them whole, 1 computes their
// upper 36 of 64 blocks, 2 does so with two tiles per workgroup (table entries
// with tj < 0).  The host builds the tables to match.
int gemm_bf16_diag_mode(int stage) {
  if (!MATOPT_DIAG_TILES) return 0;
  if (stage == 0) return MATOPT_GRAM_WAVES == 8 ? 2 : 0;
  if (stage == 1) return MATOPT_POLY_WAVES == 8 ? 1 : 0;
  return 0;
}

// Workgroups per XCD of the persistent apply: one per compute unit (0: one
// tile per workgroup instead).  Taken only where every tile of the launch has
// the same K extent: the fixed walk of a stream balances equal tiles as well
// as the dispatcher does, but not tiles of unequal length (measured on sets
// that mix K = 1024 .. 8192: apply 1-3% slower than one tile per workgroup,
// against 0.7% faster on equal tiles).
#ifndef MATOPT_APPLY_PERSIST
#define MATOPT_APPLY_PERSIST 1
#endif

// Compute units per XCD of the current device (0 if unknown), cached per device.
int persist_per_xcd() {
  static std::atomic<int> per[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = per[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = std::max(1, cus / 8);
    per[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t launch_gemm_bf16(const GemmParams& p_in, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  constexpr int GW = MATOPT_GRAM_WAVES, PW = MATOPT_POLY_WAVES;
  constexpr int AW = MATOPT_APPLY_WAVES, FW = MATOPT_FINAL_WAVES;
  GemmParams p = p_in;
  p.n_tiles = n_tiles;
  const dim3 grid(n_tiles);
  if (MATOPT_APPLY_PERSIST && AW == 8 && p.stage == 2 && p.out_kind == OUT_NEXT_X &&
      p.uniform_k && n_tiles % 8 == 0) {
    const int per = persist_per_xcd();
    if (per > 0) {
      const int g = std::min(per, n_tiles / 8);
      hipLaunchKernelGGL((ns_apply_persist_kernel<8>), dim3(8 * g), dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.stage == 0)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<0, OUT_NEXT_X, GW>), grid, dim3(64 * GW), 0, s, p);
  else if (p.stage == 1 && p.split)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<1, OUT_NEXT_X, PW, true>), grid, dim3(64 * PW), 0, s, p);
  else if (p.stage == 1)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<1, OUT_NEXT_X, PW>), grid, dim3(64 * PW), 0, s, p);
  else if (p.out_kind == OUT_NEXT_X)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_NEXT_X, AW>), grid, dim3(64 * AW), 0, s, p);
  else if (p.out_kind == OUT_O)
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_O, FW>), grid, dim3(64 * FW), 0, s, p);
  else
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<2, OUT_W_UPDATE, FW>), grid, dim3(64 * FW), 0, s, p);
  return hipGetLastError();
}

}  // namespace matopt
