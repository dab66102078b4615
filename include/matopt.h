/*
 * matopt.h -- C ABI of the owner-local Muon step engine for MI355X (gfx950).
 *
 * The library runs, on one GPU, the optimizer step an owner rank applies to the
 * whole 2D matrices it owns (MatrixFSDP, arXiv 2607.05895, sections 3 and 4.4),
 * with the step itself as the blog post "Optimizers In A Sharded World: Muon's
 * O(mn) Vs RMNP's Zero" defines it (section 1; appendix "The Code That Ran"):
 *
 *   momentum        V <- mu*V + G                              (heavy ball)
 *   normalisation   X0 = V / (||V||_F + eps)
 *   transpose       work on X0^T when rows > cols (strict)
 *   ns_steps times  A = X X^T ; B = a*I + b*A + c*A*A ; X = B*X
 *   update          W <- W - lr * sqrt(max(1, rows/cols)) * O     (O = last X,
 *                                                                 transposed back)
 *
 * and the RMNP comparator (same post, section 1 and the appendix's rmnp_local):
 *
 *   V <- mu*V + G ;  u_i = V_i / max(||V_i||_2, eps) ;  W <- W - lr*s*u
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All matrix pointers are DEVICE pointers to contiguous row-major storage owned
 *   by the caller.  The library keeps no pointer after a call returns.
 * - Host-side arrays (matopt_mat lists, row/col arrays, pointer arrays) are read
 *   during the call only.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *   the call returns without synchronising.  Keep every buffer alive until the
 *   stream has completed the work.
 * - Argument errors are detected before anything is enqueued and leave every
 *   buffer untouched.  A failed launch returns MATOPT_ERR_HIP.  A device fault
 *   surfaces at the caller's next synchronisation.  matopt_last_error_detail()
 *   returns a thread-local text for the last non-OK status of the calling thread.
 * - Scalars are float32; NaN/Inf in matrix data propagate and are not checked.
 * - W, G, V (and the workspace) must not overlap each other (MATOPT_ERR_ALIAS is
 *   reported for exactly equal base pointers and for overlapping ranges).
 * - count == 0 is a no-op returning MATOPT_OK.
 * - Calls on one stream are ordered.  Calls that share a workspace must not run
 *   concurrently on different streams.
 * - Plans.  The first call of an entry point with a given list of shapes (and
 *   dtype; for the column-cut apply also full_cols) builds a plan: descriptor
 *   templates and the tile and task tables of every launch, which depend on
 *   the shapes only.  Building it allocates one device buffer (stream-ordered,
 *   on `stream`) and copies the tables into it on `stream`.  Every later call
 *   with the same shapes reuses it whatever its pointers: it allocates nothing,
 *   frees nothing, copies nothing from host memory and never synchronises the
 *   host -- this call's pointers reach the device as kernel arguments of a
 *   small bind launch that writes the descriptors (into the workspace for the
 *   Newton-Schulz entry points, into the plan for the others; there, a call
 *   whose pointers equal those already bound skips the launch).  Calls that use
 *   one plan are therefore chained: a call on another stream than the previous
 *   call of the same plan first waits (on the device) for that call's work.
 *   At most 64 plans are cached; an evicted plan is freed, stream-ordered,
 *   once the device has finished every call that used it.
 */
#ifndef MATOPT_H
#define MATOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MATOPT_F32 = 0,  /* IEEE float32 */
    MATOPT_BF16 = 1, /* bfloat16 (round to nearest even on every store) */
    /* Newton-Schulz entry points only: bfloat16 storage and bf16 MFMA products
     * as MATOPT_BF16, but each iterate is carried to the next product with X
     * as a bf16 high part plus a bf16 low part (x - hi), about 16 significant
     * bits: the products B*X run over both parts (twice the K of the plain
     * path) and B is stored whole.  On ill-conditioned inputs, whose small
     * singular values sit where the quintic's fifth iterate is steep, this
     * keeps O within 2e-2 of the exact iteration where bf16 iterates cannot.
     * Needs the workspace matopt_workspace_bytes reports for this dtype. */
    MATOPT_BF16_SPLIT = 2
} matopt_dtype;

typedef enum {
    MATOPT_OK = 0,
    MATOPT_ERR_NULL = 1,       /* a required pointer is NULL */
    MATOPT_ERR_SHAPE = 2,      /* rows or cols < 1, or a size too large */
    MATOPT_ERR_DTYPE = 3,      /* unsupported dtype or dtype combination */
    MATOPT_ERR_PARAM = 4,      /* non-finite scalar, ns_steps outside [0, 64], count < 0 */
    MATOPT_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required */
    MATOPT_ERR_ALIAS = 6,      /* two buffers overlap */
    MATOPT_ERR_ALIGN = 7,      /* a pointer is not 16-byte aligned */
    MATOPT_ERR_DEVICE = 8,     /* the current device is not gfx950 / no device */
    MATOPT_ERR_HIP = 9,        /* a HIP runtime call or a launch failed */
    MATOPT_ERR_INTERNAL = 10
} matopt_status;

/* One matrix of a batch: W (in/out), G (in), V (in/out), all rows x cols,
 * contiguous row-major, same dtype, 16-byte aligned. */
typedef struct {
    void* w;
    const void* g;
    void* v;
    int64_t rows;
    int64_t cols;
} matopt_mat;

/*
 * Bytes of device workspace muon_step_batched / ns_orthogonalize_batched need for
 * this list of shapes in dtype `dt` (the compute dtype: BF16 selects the bf16
 * MFMA path, F32 the float32 path).  Returns 0 on invalid arguments.  Pure host
 * function; the result depends on the shapes only.
 */
size_t matopt_workspace_bytes(const int64_t* rows, const int64_t* cols,
                              int32_t count, matopt_dtype dt);

/*
 * One Muon step on every matrix of `mats` (blog post, appendix muon_sc step on a
 * whole matrix; MatrixFSDP section 4.4 owner-local step).
 *   dt          storage and compute dtype of W, G, V: MATOPT_BF16 (bf16 storage,
 *               bf16 MFMA products with float32 accumulation) or MATOPT_F32
 *               (float32 storage and float32 products).
 *   mu          momentum (0.95 on the pages); lr learning rate.
 *   ns_steps    Newton-Schulz iterations, 0..64 (5 on the pages).
 *   a, b, c     Newton-Schulz coefficients ((3.4445, -4.7750, 2.0315) on the pages).
 *   eps         added to the Frobenius norm (1e-7 on the pages), >= 0.
 *   workspace   device buffer of at least matopt_workspace_bytes(...) bytes,
 *               256-byte aligned, contents on entry irrelevant, clobbered.
 * V and W are updated in place; G is read only.
 */
matopt_status muon_step_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                float mu, float lr, int32_t ns_steps,
                                float a, float b, float c, float eps,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The Muon step of muon_step_batched with no workspace argument and no device
 * allocation of any kind, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Its workspace and its tile tables live in a file-scope device array of
 * MATOPT_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU, held from the first
 * call on that GPU until the process ends; each call rewrites the tables in it
 * through kernel arguments (nothing is copied from host memory).  A list of
 * shapes whose workspace (matopt_workspace_bytes) plus tables exceed the array
 * is rejected with MATOPT_ERR_WORKSPACE before anything is enqueued -- about
 * four 1280 x 1280 bf16 matrices fit.  Results are bit-identical to
 * muon_step_batched's; arguments and errors are otherwise the same.  All calls
 * on one GPU share that GPU's array, which keeps the last call's contents
 * (nothing in it has to be zero on entry); calls that overlap on one GPU --
 * on different streams without ordering between them -- race on it, so the
 * caller must order them.  With profiling off (matopt_profile_enable), a
 * call enqueues kernel launches only (no memory operation, event or
 * synchronisation), so it can be captured into a HIP graph; a captured step
 * replays with the pointers and scalars it was captured with.
 */
#define MATOPT_NOALLOC_SCRATCH_BYTES (64u << 20)
matopt_status muon_step_batched_noalloc(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                        float mu, float lr, int32_t ns_steps,
                                        float a, float b, float c, float eps, void* stream);

/*
 * The Muon step with decoupled weight decay folded into the update, the
 * configuration the MatrixFSDP paper trains with (section 5.1: weight decay
 * 1e-2, momentum 0.5, two Newton-Schulz steps):
 *   W <- W - lr * (wd * W + sqrt(max(1, rows/cols)) * O)     (one rounding)
 * Decoupled (the decay scales W by lr*wd and does not pass through the
 * orthogonalization) is the reading taken for the paper's "weight decay".
 *   wd          weight decay, finite (MATOPT_ERR_PARAM otherwise); wd = 0 gives
 *               exactly muon_step_batched's result.
 * Every other argument, the workspace and the error behaviour are those of
 * muon_step_batched.
 */
matopt_status muon_step_batched_wd(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                   float mu, float lr, float wd, int32_t ns_steps,
                                   float a, float b, float c, float eps,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * One RMNP step on every matrix of `mats` (blog post, section 1 RMNP direction and
 * the appendix's rmnp_local step): V <- mu*V + G (one rounding to storage); row
 * sums of squares of the stored V in float32; W <- W - lr*sqrt(max(1,rows/cols)) *
 * V_i / max(||V_i||, eps) (one rounding).  eps: 1e-12 on the pages, >= 0.
 * Needs no workspace.
 */
matopt_status rmnp_step_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                float mu, float lr, float eps, void* stream);

/*
 * Column-cut RMNP, the two local halves on one rank (blog post, section 3, the
 * column-cut layout; appendix rmnp_colcut).  Each matrix of `mats` is this
 * rank's column slice (rows x cols) of a whole matrix (rows x full_cols[i]).
 * The row sums of squares of all matrices form one float32 vector `rowsq` of
 * sum(rows) entries, matrix i's rows starting after those of matrices 0..i-1.
 * Between the two calls the caller sums `rowsq` over the ranks that hold the
 * other slices (one all-reduce); on a single rank nothing happens in between.
 *
 * rmnp_colcut_partial_batched: V <- mu*V + G (one rounding to storage), then
 *   rowsq[row] = sum over this slice of the stored V[row, :]^2, in float32 in a
 *   fixed order (deterministic).  mats[i].w is not used (may be NULL).
 *   rowsq: DEVICE pointer, 4-byte aligned, overwritten.
 * rmnp_colcut_apply_batched: W <- W - lr*sqrt(max(1, rows/full_cols[i])) *
 *   V / max(sqrt(rowsq[row]), eps)   (one rounding).  mats[i].g is not used
 *   (may be NULL); V and rowsq are read only.  eps: 1e-7 in the column-cut
 *   listing, >= 0.  full_cols: HOST array of count entries, each >= the slice's
 *   cols (MATOPT_ERR_SHAPE otherwise), or NULL for full_cols[i] = cols.
 * Both need no workspace; rowsq must not overlap any matrix (MATOPT_ERR_ALIAS).
 */
matopt_status rmnp_colcut_partial_batched(const matopt_mat* mats, int32_t count,
                                          matopt_dtype dt, float mu, float* rowsq,
                                          void* stream);
matopt_status rmnp_colcut_apply_batched(const matopt_mat* mats, int32_t count,
                                        matopt_dtype dt, float lr, float eps,
                                        const float* rowsq, const int64_t* full_cols,
                                        void* stream);

/* One flat tensor of the AdamW tail: p (in/out) and g (in) in the storage
 * dtype, m and v (in/out) float32, n elements each, 16-byte aligned. */
typedef struct {
    void* p;
    const void* g;
    float* m;
    float* v;
    int64_t n;
} matopt_vec;

/*
 * One AdamW step on every tensor of `vecs`: the non-2D tail of an owner's
 * parameters (LayerNorm weights, biases), which MatrixFSDP section 5.1 updates
 * with AdamW (lr 1e-3, weight decay 1e-2, betas (0.9, 0.999), eps 1e-8).  The
 * pages do not write the update out; it is the standard decoupled form:
 *   m <- beta1*m + (1-beta1)*g ;  v <- beta2*v + (1-beta2)*g^2   (float32)
 *   p <- p - lr*wd*p - lr/(1-beta1^step) * m / (sqrt(v)/sqrt(1-beta2^step) + eps)
 * computed in float64 from the stored m, v, p rounded once to `dt`.
 *   dt      storage dtype of p and g (BF16 or F32); m, v are always float32.
 *   step    1-based count of steps including this one (>= 1).
 *   beta1, beta2 in [0, 1); lr, wd finite; eps finite and >= 0.
 * All pointers are DEVICE pointers; buffers must not overlap (MATOPT_ERR_ALIAS).
 * Needs no workspace.
 */
matopt_status adamw_step_batched(const matopt_vec* vecs, int32_t count, matopt_dtype dt,
                                 float lr, float beta1, float beta2, float eps, float wd,
                                 int32_t step, void* stream);

/*
 * Newton-Schulz only (the appendix's routine): o[i] = NS(x[i]) for each matrix,
 * in the original orientation.  x[i]: rows[i] x cols[i] in `in_dt` (selects the
 * compute path as `dt` does above); o[i]: same shape in `out_dt` (F32 or BF16).
 * x is read only.  Used to read the orthogonalized direction out directly.
 */
matopt_status ns_orthogonalize_batched(const void* const* x, void* const* o,
                                       const int64_t* rows, const int64_t* cols,
                                       int32_t count, matopt_dtype in_dt,
                                       matopt_dtype out_dt, int32_t ns_steps,
                                       float a, float b, float c, float eps,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Human-readable name of a status code (static storage). */
const char* matopt_status_string(matopt_status s);

/* Thread-local detail text of the last non-OK status returned to this thread. */
const char* matopt_last_error_detail(void);

/* Library ABI version (major*10000 + minor*100 + patch). */
int32_t matopt_version(void);

/*
 * Kernel timing for benchmarks.  While enabled, every launch of the library is
 * bracketed by hipEvents on the stream it is launched on, and per-kernel-class
 * elapsed times are accumulated when matopt_profile_read() is called (which
 * synchronises on those events).  Classes: 0 momentum+norm+X0 build,
 * 1 norm finalize, 2 Gram X X^T, 3 polynomial a*I+b*A+c*A*A, 4 apply B*X
 * (incl. fused update on the last step), 5 ns_steps==0 output, 6 RMNP,
 * 7 column-cut RMNP partial, 8 column-cut RMNP apply, 9 AdamW, 10 descriptor
 * bind.
 */
#define MATOPT_PROFILE_CLASSES 11
matopt_status matopt_profile_enable(int32_t on);
/* ms[k], launches[k] for k < MATOPT_PROFILE_CLASSES; resets the accumulators. */
matopt_status matopt_profile_read(double* ms, int64_t* launches);
/*
 * Shader clock (MHz) the bf16 GEMM launches of classes 2, 3 and 4 ran at while
 * profiling was on (current device): each workgroup adds the ticks of the
 * shader-clock and the 100 MHz real-time counters over its tile, mhz[k] is
 * 100 * (sum of shader ticks) / (sum of real-time ticks); 0 for classes
 * without data.  Synchronises the device; resets the counters.  Switching
 * profiling on allocates a 176-byte device buffer per device (once).
 * mhz: HOST array of MATOPT_PROFILE_CLASSES entries.
 */
matopt_status matopt_profile_read_clock(double* mhz);

/*
 * Diagnostics of the plan cache, cumulative since the library was loaded:
 * out[0] plans built, out[1] device allocations, out[2] device frees, out[3]
 * bind launches (one per 112 descriptors of a call).  Writes the first n <=
 * MATOPT_COUNTERS values to the HOST array out; MATOPT_ERR_PARAM otherwise.
 */
#define MATOPT_COUNTERS 4
matopt_status matopt_counters(int64_t* out, int32_t n);

/*
 * MFMA rate probe: a measurement aid, not part of the optimizer step.  It
 * bounds what a bf16 MFMA schedule can reach on this part with given operand
 * data, for comparing the two MFMA forms the GEMM engine can use.  Each of
 * `workgroups` workgroups (512 threads: 8 waves, one workgroup per compute
 * unit) runs `iters` steps per wave of 524288 flops each: 16
 * v_mfma_f32_32x32x16_bf16 (form 32) or 32 v_mfma_f32_16x16x32_bf16 (form
 * 16) on 12 operand fragments per lane, which stay in registers (from_lds 0)
 * or are read fresh from LDS one step ahead (from_lds 1, as the GEMM engine
 * reads them).  No DMA, no epilogue.
 *   src: DEVICE, 49152 bfloat16 values (98304 bytes), the operand data;
 *   out: DEVICE, workgroups * 512 floats (written: per-thread sums, so that
 *        no MFMA is dead code);
 *   clk: DEVICE, 2 uint64 accumulators, ADDED to: the shader-clock ticks and
 *        the 100 MHz real-time ticks of each workgroup's MFMA loop (their
 *        ratio times 100 is the clock in MHz).
 * Flops per call: workgroups * 8 * iters * 524288.  iters even, in
 * [2, 2^22]; workgroups in [1, 2^20]; pointers 16-byte aligned.  Enqueued on
 * `stream`; argument errors are reported before anything is enqueued.
 */
matopt_status matopt_mfma_probe(int32_t form, int32_t from_lds, const void* src, float* out,
                                int32_t iters, int32_t workgroups, uint64_t* clk,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MATOPT_H */
