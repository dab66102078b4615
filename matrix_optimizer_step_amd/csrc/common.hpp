// Internal declarations shared by the host side and the kernels of libmatopt.
//
// Data layout in HBM (one matrix of a batch; "X orientation" is the matrix the
// Newton-Schulz iteration works on: the stored matrix, or its transpose when it
// has more rows than columns, so that X is m x n with m <= n):
//
//   caller buffers   W, G, V: rows x cols, row-major, storage dtype.
//   workspace        X[0], X[1]: mp x np (ping-pong iterates, X orientation)
//                    A, B:       mp x mp (Gram and polynomial; only the tiles on
//                                         or above the diagonal are written)
//                    partials:   one float per prep tile (sum of squares)
//                    xs:         one float per matrix, 1/(||V||_F + eps)
//   mp, np are m, n rounded up to the GEMM tile (256 for bf16, 64 for fp32); the
//   padding is written as zeros by the prep kernel and stays zero through the
//   iteration, so the GEMM main loop needs no bounds checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace matopt {

enum Dtype : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// Output of the last Newton-Schulz apply stage.
enum OutKind : int32_t {
  OUT_NEXT_X = 0,   // not the last iteration: write X_next (workspace)
  OUT_O = 1,        // ns_orthogonalize: write O in the original orientation
  OUT_W_UPDATE = 2  // muon step: W <- W - lr*s*O in the original orientation
};

struct MatDesc {
  void* w;              // caller W (muon) or unused
  const void* g;        // caller G (muon) or unused
  void* v;              // caller V (muon) / NS input x (read only)
  void* o;              // NS output (ns_orthogonalize) or unused
  int64_t rows, cols;   // original shape
  int32_t m, n;         // X orientation, m <= n
  int32_t mp, np;       // padded to the GEMM tile
  int32_t transposed;   // rows > cols
  int32_t vec_ok;       // cols is a multiple of the 16-byte vector width
  float upd_scale;      // sqrt(max(1, rows/cols))
  int32_t prep_tiles_c; // prep tiles along the padded original columns
  void* x[2];           // iterates, mp x np, leading dimension np
  const void* x0in;     // the first iteration's input: V itself when x0_is_v,
                        // else x[0] (filled by the prep kernel)
  void* a;              // Gram,       mp x mp, leading dimension mp
  void* b;              // polynomial, mp x mp, leading dimension mp
  float* xs;            // this matrix's Frobenius scale
  float* partials;      // this matrix's first prep-tile partial
  int32_t n_prep;       // prep tiles of this matrix
  int32_t x0_is_v;      // bf16, not transposed, no padding: X0 would be a copy
                        // of the stored V in the same layout, so it is not written
};

// Prep tile: 64 x 64 block of the padded original-orientation matrix (64 x
// kPrepTileT for a transposed bf16 matrix); an untransposed matrix's prep
// kernel reads the tile index idx as a run of 4096 elements of X0 instead.
struct PrepTile {
  int32_t mat, tr, tc, idx;   // idx: tile index within the matrix
};

// GEMM output tile (ti, tj) of matrix `mat`.
struct GemmTile {
  int32_t mat, ti, tj, pad_;
};

struct PrepParams {
  const MatDesc* mats;
  const PrepTile* tiles;
  float mu;
  int32_t momentum;   // 1: V <- mu V + G and store V;  0: read x only
};

struct FinalizeParams {
  const MatDesc* mats;
  float eps;
};

struct GemmParams {
  const MatDesc* mats;
  const GemmTile* tiles;
  // 0: A = X X^T;  1: B = aI + bA + cAA (bf16) or bA + cAA (fp32);
  // 2: X' = B X (bf16) or aX + BX (fp32)
  int32_t stage;
  int32_t cur;        // index of the current iterate buffer
  int32_t first;      // first iteration: fold the Frobenius scale in
  int32_t out_kind;   // OutKind (stage 2)
  int32_t out_dt;     // dtype of O for OUT_O
  // split precision (bf16 path): the polynomial stores B whole, every apply
  // but the last stores its iterate as bf16 hi over bf16 lo (2 mp x np), and
  // the applies after the first run K over both parts
  int32_t split;
  int32_t n_tiles;    // entries of `tiles` (set by the launcher)
  int32_t uniform_k;  // every tile of the table has the same K extent
  float a, b, c, lr;
  double wdl;         // lr * weight decay (exact product), 0: no decay
  // profiling only (else NULL): [0] += shader-clock ticks, [1] += 100 MHz
  // real-time ticks, summed over the launch's workgroups (bf16 kernel)
  unsigned long long* clk;
};

// ns_steps == 0: O = xs * V directly (prep tiles over the original orientation).
struct ScaleOutParams {
  const MatDesc* mats;
  const PrepTile* tiles;
  int32_t out_kind;   // OUT_O or OUT_W_UPDATE
  int32_t out_dt;
  float lr;
  double wdl;         // lr * weight decay, 0: no decay
};

// RMNP: a block handles `rows_per_block` consecutive rows of one matrix.
struct RmnpTask {
  int32_t mat, row0;
};

struct RmnpParams {
  const MatDesc* mats;
  const RmnpTask* tasks;
  float mu, lr, eps;
};

// Column-cut RMNP halves: a block handles 4 consecutive rows (one per wave).
struct ColcutParams {
  const MatDesc* mats;   // partials: this matrix's row-sum entries
  const RmnpTask* tasks;
  float mu, lr, eps;
};

// AdamW over flat tensors: one descriptor per tensor, one task per 2048
// consecutive elements of a tensor (256 threads x 8).
struct VecDesc {
  void* p;          // parameters (storage dtype)
  const void* g;    // gradient (storage dtype)
  float* m;         // first moment, float32
  float* v;         // second moment, float32
  int64_t n;        // elements
};

struct VecTask {
  int32_t t, pad_;
  int64_t start;
};

struct AdamwParams {
  const VecDesc* vecs;
  const VecTask* tasks;
  double b1, omb1, b2, omb2;   // betas and 1 - betas
  double step_size;            // lr / (1 - beta1^t)
  double inv_sqrt_bc2;         // 1 / sqrt(1 - beta2^t)
  double eps, wdl;             // eps; lr * weight decay
};

constexpr int kAdamwTask = 2048;

// Per-call binding of the caller's pointers into the descriptors a launch
// reads.  A plan (built once per list of shapes) holds descriptor templates;
// every call launches bind_kernel, whose by-value arguments carry up to
// kBindMax pointer sets, to write the descriptors of this call:
//   BIND_NS      MatDesc; p = {w, g, v, o}; x[], a, b, xs, partials of the
//                template are byte offsets from `base` (the workspace);
//                x0in = v when x0_is_v, else x[0]
//   BIND_ROWS    MatDesc; p = {w, g, v, -}; nothing relocated (RMNP)
//   BIND_COLCUT  MatDesc; p = {w, g, v, -}; partials is a byte offset from
//                `base` (the caller's row-sum vector)
//   BIND_VEC     VecDesc; p = {p, g, m, v} (AdamW)
enum BindMode : int32_t { BIND_NS = 0, BIND_ROWS = 1, BIND_COLCUT = 2, BIND_VEC = 3 };
constexpr int kBindMax = 112;
struct BindPtrs {
  const void* p[4];
};
struct BindArgs {
  void* dst;           // descriptor array (device)
  const void* tmpl;    // template array (device, plan memory)
  const char* base;    // relocation base (see BindMode)
  int32_t first, n;    // descriptors first .. first+n-1 (n <= kBindMax)
  int32_t mode, pad_;
  BindPtrs ptr[kBindMax];
};
static_assert(sizeof(BindArgs) <= 3712, "bind arguments must stay well inside the kernarg limit");

// Table upload through kernel arguments (the allocation-free entry point
// fills its device-side tables this way: no host buffer has to outlive the
// call and nothing is copied from pageable memory).  n is a multiple of 16.
constexpr int kUploadBytes = 3584;
struct UploadArgs {
  void* dst;
  uint32_t n, pad_;
  alignas(16) uint8_t data[kUploadBytes];
};

// Tile geometry.  Prep tiles are 64 x 64 (64 x kPrepTileT for bf16 matrices
// that are transposed: 256-byte runs of every row they read and write).
constexpr int kPrepTile = 64;
constexpr int kPrepTileT = 128;
constexpr int kTileBf16 = 256;
constexpr int kTileF32 = 64;   // float32 padding granule
constexpr int kGridF32 = 32;   // float32 GEMM output tile (divides kTileF32)

// Launchers (each defined next to its kernel).
hipError_t launch_prep(int dt, const PrepParams& p, int n_tiles, hipStream_t s);
// Prep of the bf16 matrices that are transposed (64 x kPrepTileT tiles).
hipError_t launch_prep_t(const PrepParams& p, int n_tiles, hipStream_t s);
hipError_t launch_finalize(const FinalizeParams& p, int count, hipStream_t s);
hipError_t launch_scale_out(int dt, const ScaleOutParams& p, int n_tiles, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams& p, int n_tiles, hipStream_t s);
// MFMA rate probe (probe.hip), a measurement aid: 32 x 32 x 16 or 16 x 16 x 32
// MFMAs on register or LDS operands; clk accumulates shader and real-time ticks.
hipError_t launch_mfma_probe(bool f16, bool from_lds, const void* src, float* out, int iters,
                             int workgroups, unsigned long long* clk, hipStream_t s);
// Diagonal tiles of the bf16 Gram (stage 0) / polynomial (stage 1): 0 whole,
// 1 upper 36 of 64 blocks, 2 the same two per workgroup (entries with tj < 0).
int gemm_bf16_diag_mode(int stage);
hipError_t launch_gemm_f32(const GemmParams& p, int n_tiles, hipStream_t s);
// RMNP kernel variants: rows of one wave (wpr=1) or of a whole block (wpr=4),
// holding `nch` 16-byte chunks per lane in registers; nch == 0 selects the
// streaming two-pass variant (any width, scalar loads).
hipError_t launch_rmnp(int dt, int wpr, int nch, const RmnpParams& p, int n_tasks,
                       hipStream_t s);
hipError_t launch_adamw(int dt, const AdamwParams& p, int n_tasks, hipStream_t s);
// Column-cut RMNP: apply == false launches the partial half, true the update.
hipError_t launch_colcut(int dt, bool apply, const ColcutParams& p, int n_tasks, hipStream_t s);
// One bind launch (a.n <= kBindMax descriptors).
hipError_t launch_bind(const BindArgs& a, hipStream_t s);
// One upload launch (a.n <= kUploadBytes bytes).
hipError_t launch_upload(const UploadArgs& a, hipStream_t s);

}  // namespace matopt
