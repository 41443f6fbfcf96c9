/*
 * tgrad.h - C ABI of the TensorGRaD optimizer step on AMD MI355X (gfx950).
 *
 * One handle optimises one weight tensor W of shape (I_1, ..., I_d) with the
 * TensorGRaD step. The gradient G splits into a sparse part S, held on an index set
 * Omega (the k = floor(rho * N) entries of largest |G|, taken out first), and a Tucker
 * low-rank part of what remains, R = G - scatter(S). Adam keeps its moments on the
 * small Tucker core and on the k sparse values. The full-size update comes back
 * through one factor product per mode; the sparse update is added into that same
 * buffer, and W is then updated in place. Omega and the factors are recomputed every
 * T steps: a top-k by magnitude, and an HOSVD from each mode's Gram matrix.
 *
 * Sources (no code exists on them): the nullthought.net summary of "TensorGRaD:
 * Tensor Gradient Robust Decomposition for Memory-Efficient Neural Operator
 * Training", sections 2-3 (G = L + S, sparse part extracted first, Tucker on the
 * residual, separate Adam updates, scatter-add after reconstruction, half-precision
 * weights with fp32 optimizer state, re-selection every T steps); the pith.science
 * review of arXiv 2501.02379, "What carries the argument" (factors reused for T
 * steps, projection to a core, Adam moments on the core, mode-wise reconstruction,
 * COO sparse set by top-k magnitude) and its appendix M excerpt of Theorem 2
 * (project, update optimizer states, project back).
 *
 * Conventions for every call:
 *   - Tensors are dense, contiguous, row-major (last index fastest). complex64 is
 *     interleaved (re, im) fp32 pairs. Element (linear) indices count complex
 *     elements, not floats.
 *   - Device pointers are HIP device addresses on the device that was current at
 *     tgrad_init; `stream` is a hipStream_t (NULL = the default stream). Every call
 *     that takes a stream only enqueues work on it and returns without waiting;
 *     device faults surface at the caller's next synchronisation.
 *   - Host pointers (marked host) are ordinary CPU memory; calls taking them
 *     synchronise the device before returning.
 *   - Return value: TGRAD_OK or an error code below; no call throws. After
 *     TGRAD_EHIP, tgrad_last_error() gives the HIP error string.
 *   - One handle is used by one host thread and one stream at a time. Separate
 *     handles are independent.
 */
#ifndef TGRAD_H
#define TGRAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tgrad_handle tgrad_t;

/* Storage dtype of the weight and the gradient. Optimizer state is always fp32. */
enum tgrad_dtype { TGRAD_F32 = 0, TGRAD_F16 = 1, TGRAD_BF16 = 2, TGRAD_C64 = 3 };

enum tgrad_status {
  TGRAD_OK = 0,
  TGRAD_EINVAL = 1,   /* invalid argument (null pointer, size or range) */
  TGRAD_ENOMEM = 2,   /* device allocation failed */
  TGRAD_EHIP = 3,     /* a HIP call or kernel launch failed */
  TGRAD_ESTATE = 4    /* call not valid in the handle's current state */
};

#define TGRAD_MAX_NDIM 8
#define TGRAD_MAX_FACTOR_DIM 128  /* largest I_n of a mode with r_n < I_n */

/*
 * Create a handle on the current HIP device and allocate all optimizer state.
 *   ndim            number of modes d, 1..8
 *   shape[d]        I_n >= 1; N = prod I_n must be < 2^32
 *   tucker_ranks[d] r_n in [1, I_n]. r_n == I_n keeps mode n uncompressed (identity
 *                   factor, no mode product); r_n < I_n needs I_n <= 128 and
 *                   r_n <= N / I_n (the rank of the mode-n unfolding).
 *   dtype           enum tgrad_dtype of W and G
 *   sparse_ratio    rho in [0, 1]; k = floor(rho * N) computed in IEEE double
 *   T               refresh period >= 1: a refresh runs before every step t with
 *                   (t - 1) mod T == 0, t = 1, 2, ... (pith.science: factors and
 *                   Omega reused for T steps; nullthought section 3)
 *   lr, beta1, beta2, eps   Adam: lr >= 0, beta in [0, 1), eps >= 0
 * Moments start at zero, t = 0. The handle owns every device buffer it allocates.
 * Errors: TGRAD_EINVAL, TGRAD_ENOMEM, TGRAD_EHIP. *out is NULL on error.
 */
int tgrad_init(tgrad_t **out, int ndim, const int64_t *shape, const int64_t *tucker_ranks,
               int dtype, double sparse_ratio, int64_t T, double lr, double beta1,
               double beta2, double eps);

/*
 * One optimizer step on device buffers `weight` (W, updated in place) and `grad`
 * (G, caller-owned, N elements of dtype, 16-byte aligned, only read).
 *   t <- t + 1; if a refresh is due for t and tgrad_refresh was not already called
 *   for it, refresh from `grad` first. Then: S = G[Omega] (fp32) and R = G with
 *   Omega zeroed; core C = R x_1 U1^H ... x_d Ud^H; Adam on C and on S (fp32
 *   moments); Delta = N_C x_1 U1 ... x_d Ud with lambda N_S added at Omega;
 *   W <- round(W * decay - lr * Delta), one rounding per element (lambda = 1 and
 *   decay = 1 unless tgrad_set_options says otherwise; nullthought section 3 step
 *   order; pith.science Theorem 2).
 * Both buffers must stay valid until the work on `stream` completes.
 * Errors: TGRAD_EINVAL (null handle/pointer, grad not 16-byte aligned), TGRAD_EHIP.
 * On an error t is not advanced (a refresh that completed for this t stays valid).
 */
int tgrad_step(tgrad_t *h, void *weight, const void *grad, void *stream);

/*
 * Several tensors' steps as one call (many small FNO layers per optimizer step):
 * tgrad_step(hs[i], weights[i], grads[i], .) for i < n, issued on up to four internal
 * streams (per device, created on first use, default priority) that start after the
 * work already queued on `stream`; `stream` then waits for all of them, so later work
 * on it sees every update. The tensors' kernels overlap on the device, filling the
 * tail of each launch with another tensor's work; each handle's results are bit for
 * bit those of tgrad_step. The handles must be distinct and on one device; calls are
 * serialised by an internal mutex. Errors: TGRAD_EINVAL (n < 0, a NULL array or entry,
 * a grad not 16-byte aligned, a repeated handle, handles on different devices), or the
 * first failing step's status (the steps before it are issued and joined).
 */
int tgrad_step_many(tgrad_t *const *hs, void *const *weights, const void *const *grads, int n,
                    void *stream);

/*
 * Refresh Omega and the Tucker factors from `grad` (device, N elements of dtype,
 * 16-byte aligned):
 * Omega = the k largest magnitudes (ties to the lowest linear index), stored
 * ascending; each U(n) (r_n < I_n) = the r_n leading eigenvectors of the mode-n Gram
 * matrix of the residual, descending eigenvalue order, each column scaled so its
 * largest-magnitude entry (lowest row on ties) is real positive. `grad` is only
 * read. Moments and t are untouched; the refresh serves step t + 1.
 * (nullthought section 3: re-select sparse indices and low-rank subspace every T
 * steps; pith.science: top-k magnitude, Tucker/HOSVD factors.)
 * Errors: TGRAD_EINVAL (null handle/pointer, grad not 16-byte aligned), TGRAD_EHIP.
 */
int tgrad_refresh(tgrad_t *h, const void *grad, void *stream);

/* Free every buffer of the handle. The caller synchronises first. NULL is a no-op. */
int tgrad_destroy(tgrad_t *h);

/* Static description of an error code; never NULL. */
const char *tgrad_status_string(int status);
/* Last HIP error message recorded on the handle (empty string if none). */
const char *tgrad_last_error(const tgrad_t *h);

/* ---------------------------------------------------------------- introspection.
 * Not on the hot path. Host buffers; each call synchronises the device. */

typedef struct tgrad_info {
  int64_t ndim, dtype, numel, k, core_numel, T, t;
  int64_t shape[TGRAD_MAX_NDIM];
  int64_t ranks[TGRAD_MAX_NDIM];
  int64_t state_bytes;      /* moments, core, factors, Omega (optimizer state) */
  int64_t workspace_bytes;  /* transient buffers owned by the handle */
  /* The eigensolver at the last refresh (0 before any): the most Jacobi sweeps any mode
   * took to reach its off-diagonal bound (0 for a mode that the tridiagonal route for
   * real modes up to 64 served), and the number of modes that reached the sweep cap
   * first (their factors are then less accurate than the bound promises). */
  int64_t eig_sweeps_max;
  int64_t eig_unconverged;
} tgrad_info;

/* Synchronises the device once the handle has refreshed (to read the eigensolver
 * report). Errors: TGRAD_EINVAL, TGRAD_EHIP. */
int tgrad_get_info(const tgrad_t *h, tgrad_info *out);

/* Omega, k uint32 linear indices ascending. cap = capacity of out (elements). */
int tgrad_get_omega(tgrad_t *h, uint32_t *out, int64_t cap);

/* U(n) as I_n x r_n row-major fp32 (complex: interleaved pairs, 2 I_n r_n floats).
 * TGRAD_EINVAL for an identity mode (r_n == I_n) or too small cap (floats). */
int tgrad_get_factor(tgrad_t *h, int mode, float *out, int64_t cap);

/* Gram-matrix eigenvalues of mode n from the last refresh, I_n doubles, descending. */
int tgrad_get_eigvals(tgrad_t *h, int mode, double *out, int64_t cap);

/* Adam moments (fp32; complex = pairs): core m, v (core_numel*P each) and sparse m,
 * v (k*P each). Any pointer may be NULL to skip it. */
int tgrad_get_moments(tgrad_t *h, float *m_core, float *v_core, float *m_sparse,
                      float *v_sparse);

/* Test hooks: replace Omega (k ascending unique indices < N) or U(n) (layout as
 * tgrad_get_factor) from host memory, and mark the handle refreshed for step t + 1
 * so the next step uses them. */
int tgrad_set_omega(tgrad_t *h, const uint32_t *omega, int64_t k);
int tgrad_set_factor(tgrad_t *h, int mode, const float *U, int64_t n_floats);
int tgrad_mark_refreshed(tgrad_t *h);

/* Test hook: while `delta` is set, every step also writes its fp32 update before the
 * weight rounding, Delta = Delta_L + lambda N_S at Omega (the value W * decay - lr * Delta
 * is rounded from), into `delta`: a caller-owned device buffer of N * P floats (P = 2
 * for complex64, interleaved), 16-byte aligned, valid until the stream's work is done.
 * The kernels that write it are separate instantiations of the weight-update launches,
 * with the same arithmetic; W is updated as usual. NULL turns the capture off.
 * Errors: TGRAD_EINVAL (NULL handle, misaligned buffer). */
int tgrad_debug_capture_delta(tgrad_t *h, float *delta);

/* Test / benchmark hook: when the last two modes are both compressed and a slab of
 * them fits in LDS, the projection's first two mode products and the reconstruction's
 * last two run as one launch each (the default). For bf16/fp16 tensors with small
 * enough slabs those launches use one wave per slab on bf16 MFMAs (exact bf16 splits of
 * the fp32 operands), otherwise workgroup-wide fp32 MFMA tiles; where mode d-3 is also
 * compressed (I(d-3) a multiple of 16 up to 64, rank <= 32), the projection's first
 * launch takes mode d-3 as well (one workgroup per index of the leading modes), and,
 * where I(d-3) is a multiple of 12 up to 64 (16-bit weights, 16-byte aligned), so does
 * the reconstruction's last launch, with the merge and the weight update (the mode d-2
 * tensor stays on chip). enable = 0 selects one launch per mode; 1 the fused form
 * (default choice of kernels); 2 the fused two-mode form with the workgroup-tile kernel
 * only; 3 the fused two-mode form with the slab kernels, without the three-mode
 * launches; 4 as 1 but with the two-mode reconstruction. enable = 1 to 4 returns
 * TGRAD_EINVAL where the fused form does not apply. The unfused plan projects a residual copy of grad, so enable = 0 allocates an
 * N-element workspace the first time (TGRAD_ENOMEM if that fails). Results agree to
 * fp32 rounding; takes effect at the next step. */
int tgrad_set_fusion(tgrad_t *h, int enable);

/* Test / benchmark hook: in a bf16/fp16 tensor whose last three modes are all
 * compressed, a refresh forms their three Grams in one launch that reads the residual
 * once (pith.science "What carries the argument": every factor comes from the Gram of
 * its mode's unfolding, and each Gram is a sum over slabs of the last three modes, so
 * one staged slab serves all three). It applies when the two modes before the last are
 * at most 64, the last at most 32, and one slab of the three modes is a multiple of 8
 * elements and at most 128 KiB; the input must be 16-byte aligned (otherwise one launch
 * per mode is used). Bit 0 of enable = 1 selects it (the default; TGRAD_EINVAL where it
 * does not apply), 0 one Gram launch per mode. Bit 1 (enable = 2 or 3) makes every Gram
 * launch read the gradient itself and clear Omega's entries in its staged tiles through
 * the membership bitmask, instead of reading the residual copy the top-k pass writes
 * (the default, enable 0 or 1). Results agree to fp32 rounding of the partial sums;
 * takes effect at the next refresh. */
int tgrad_set_gram_fusion(tgrad_t *h, int enable);

/* Test / benchmark hook: work that runs on a second stream the handle owns (created by
 * tgrad_init, default priority), forked from the caller's stream and joined back before
 * the call's later work, so every call stays ordered on the caller's stream.
 *  adam: when the COO gather is folded into the first projection launch and further
 *        launches follow it, the Adam update of the k sparse values (the nullthought
 *        summary, section 3: S and the low-rank core keep separate Adam states) waits
 *        for that first launch and overlaps the projection's later launches and the
 *        core's Adam update; the reconstruction waits for it. The update is element-wise:
 *        results are bit-identical either way. The fork and the join cost about 10 us a
 *        step, so adam = 1 (the default) selects it only when the sparse part holds at
 *        least 2^22 values (k, times 2 for complex data); 2 whenever it applies; 0 runs
 *        both updates in one launch on the caller's stream. Its launch is named
 *        adam_sparse (tgrad_kernel_name).
 *  eig:  at a refresh whose last three modes' Grams come from one launch (see
 *        tgrad_set_gram_fusion), the eigensolver of the compressed modes before them
 *        (pith.science "What carries the argument": each factor from its own mode's
 *        Gram) runs beside that launch, which then leaves one CU per such matrix free.
 *        1 (default) or 0. With fewer workgroups the three-mode launch sums its partial
 *        Grams in another grouping, so factors agree to fp64 rounding of the Grams.
 * Takes effect at the next step or refresh. */
int tgrad_set_stream_overlap(tgrad_t *h, int adam, int eig);

/* Test / benchmark hook: with the fused launch plan, two neighbouring compressed modes
 * ahead of the trailing ones (the projection's last two products, the reconstruction's
 * first two) run as one launch. The tensor between the two products is never written
 * (pith.science "What carries the argument": the projection and reconstruction are
 * chains of mode-wise products, so any two neighbours may be contracted together).
 * It applies to real tensors when the product of the sizes after the two modes is a
 * multiple of 16 and both modes' sizes on each side are multiples of 4 up to 64.
 * enable = 1 selects it (the default; TGRAD_EINVAL where it does not apply), 0 one
 * launch per mode. Results agree to fp32 rounding; takes effect at the next step. */
int tgrad_set_pair_fusion(tgrad_t *h, int enable);

/* Test / benchmark hook: a single mode product on fp32 data (the projection's later
 * modes, the reconstruction's leading ones) runs on a streaming kernel where it applies:
 * every wave owns all output rows of 64 consecutive trailing columns and loads the next
 * such tile while it multiplies the current one, without LDS staging or workgroup
 * barriers (pith.science "What carries the argument": projection and reconstruction are
 * chains of mode-wise products). It applies when the mode has at most 64 values on
 * either side (complex data: Re and Im of the factor in two accumulator sets) and the
 * trailing part is at least 32 values (complex: 16) and a multiple of 4 (complex: 2).
 * Products over the last mode (no trailing part: the one-mode plan's first projection
 * and its weight-updating last reconstruction) run on a kernel that streams rows of the
 * tensor with the factor in registers, where the factor fits. enable = 1 selects both
 * (the default), 0 the tiled kernel for every single mode product; enable = n >= 2
 * selects them with at most n - 1 workgroups of 4 waves for the first (so that small
 * tensors exercise a wave's walk over several tiles). Negative enable: TGRAD_EINVAL.
 * Results agree to fp32 rounding; takes effect at the next step. */
int tgrad_set_stream_products(tgrad_t *h, int enable);

/* ---------------------------------------------------------------- variants.
 * Choices the method leaves open, as options of a handle (defaults: the plain method,
 * bit for bit):
 *   weight_decay   decoupled decay as in AdamW (the nullthought summary trains L and S
 *                  with AdamW; the pith.science page's experiment settings use weight
 *                  decay 1e-4 and 2e-6): W <- round(fp32(W) * decay - lr * Delta) with
 *                  decay = fp32(1 - lr * weight_decay) formed in fp64. >= 0; default 0.
 *   sparse_scale   lambda, the sparse scale factor the pith.science page lists among the
 *                  method's hyper-parameters (its value is not reported): Delta at Omega
 *                  gets fp32(lambda) * N_S instead of N_S. Finite; default 1.
 *   selection      how a refresh picks Omega (pith.science "What carries the argument":
 *                  top-k magnitude or random sampling): TGRAD_SELECT_TOPK, or
 *                  TGRAD_SELECT_RANDK = a uniformly random k-subset: element e gets the top
 *                  31 bits of SplitMix64's output for the state
 *                  seed + 0x9E3779B97F4A7C15 * (t * 2^32 + e + 1), t the step the refresh
 *                  serves, and the k largest keys (ties to the lowest index) are taken.
 *   remap_moments  0 (default): the sparse Adam moments stay with their position in
 *                  Omega across a refresh; 1: they follow their element, and an element
 *                  new to Omega starts from zero moments. Enabling it allocates two more
 *                  k*P fp32 buffers and a second bitmask (synchronises the device).
 *   seed           rand-k base seed.
 *   order          the decomposition order (pith.science lists "sparse then low-rank" as
 *                  the tuned choice; the nullthought summary reports the reverse as
 *                  worse): TGRAD_ORDER_SPARSE_FIRST (default), or
 *                  TGRAD_ORDER_LOWRANK_FIRST: a refresh takes the Tucker factors from the
 *                  HOSVD of G itself and Omega as the top-k of the fp32 residual G - L,
 *                  L = (G x_n Un^H ...) x_n Un ... with the core in fp32; a step projects
 *                  the whole G to the core, reconstructs L and takes S = (G - L)[Omega].
 *                  Enabling it allocates an N-element fp32 workspace (complex: 2N).
 * Options take effect at the next step or refresh. Errors: TGRAD_EINVAL (NULL, a
 * negative or non-finite weight_decay, a non-finite sparse_scale, an unknown selection,
 * remap or order value), TGRAD_ENOMEM, TGRAD_EHIP. */
enum tgrad_selection { TGRAD_SELECT_TOPK = 0, TGRAD_SELECT_RANDK = 1 };
enum tgrad_order { TGRAD_ORDER_SPARSE_FIRST = 0, TGRAD_ORDER_LOWRANK_FIRST = 1 };
typedef struct tgrad_options {
  double weight_decay;
  double sparse_scale;
  int32_t selection;
  int32_t remap_moments;
  uint64_t seed;
  int32_t order;
  int32_t reserved;   /* 0 */
} tgrad_options;
void tgrad_default_options(tgrad_options *out);
int tgrad_set_options(tgrad_t *h, const tgrad_options *opt);
int tgrad_get_options(const tgrad_t *h, tgrad_options *out);

/* ---------------------------------------------------------------- checkpoint.
 * The optimizer state as one host byte string, to stop and resume training: the step
 * count and refresh mark, Omega, every U(n) with its Gram eigenvalues, and the core and
 * sparse Adam moments. tgrad_state_size gives its length (-1 for a NULL handle).
 * tgrad_save_state writes it into `buf` (cap >= that size, host memory).
 * The header also records T, lr, betas, eps and every tgrad_options field.
 * tgrad_load_state restores it into a handle created with the same shape, Tucker ranks,
 * dtype, sparse_ratio, T, betas and eps, and set to the same options; only the learning
 * rate may differ (the loading handle's lr is used, as a schedule would change it).
 * Steps then continue exactly as they would have in the saved handle.
 * Both synchronise the device. Errors: TGRAD_EINVAL (NULL, too small a buffer, a size,
 * header, shape, hyper-parameter, option or Omega that does not match), TGRAD_EHIP. */
int64_t tgrad_state_size(tgrad_t *h);
int tgrad_save_state(tgrad_t *h, void *buf, int64_t cap);
int tgrad_load_state(tgrad_t *h, const void *buf, int64_t size);

/* ---------------------------------------------------------------- without allocation.
 * For callers that cannot allocate device memory while they run: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * tgrad_refresh_noalloc is tgrad_refresh (same kernels and results: Omega bit for bit,
 * factors to fp32 rounding of the Gram partial sums) with every scratch buffer its
 * kernels use -- the top-k workspace, the Gram partial sums and the Gram matrices -- in
 * one file-scope device array of the library, TGRAD_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends, instead of the handle's workspace. Its Gram launches read
 * `grad` with Omega's entries cleared through the membership bitmask, so no residual
 * copy is written, and where the partial sums would not fit they use fewer workgroups.
 * It calls no hipMalloc or hipFree (the array's address is looked up once per GPU).
 * Every call on one GPU uses that GPU's array, which keeps the last call's contents (the
 * kernels clear what must start at zero): calls that overlap on one GPU, from several
 * threads or streams, race. Per-launch timing is not recorded during the call.
 * Errors: as tgrad_refresh; TGRAD_EINVAL also when the refresh needs more than the array
 * holds (the top-k workspace grows as 16 N / 1024 bytes, so N up to about 2.9e9 fits; a
 * Gram partial sum needs 8 (I_n P)^2 bytes per workgroup) or the handle uses the
 * low-rank-first order (which needs full-size intermediates); TGRAD_EHIP when the
 * array's address cannot be obtained. */
#define TGRAD_NOALLOC_SCRATCH_BYTES (48ull << 20)
int tgrad_refresh_noalloc(tgrad_t *h, const void *grad, void *stream);

/* ---------------------------------------------------------------- launch record.
 * The kernel launches of the last tgrad_step, tgrad_refresh or tgrad_refresh_noalloc call
 * on the handle, in issue order (a step that refreshed lists the refresh's first), with
 * the algorithmic work of each: bytes_read and bytes_written count once every gradient,
 * weight, intermediate, index, moment and sparse value the launch's part of the method
 * needs (the membership bitmask and word ranks are counted only where a top-k pass
 * produces them or a masked Gram reads them); flops are 2 K M per column of each mode
 * product and Gram (K, M the real sizes of the contracted and produced mode). modes: bit
 * n set when the launch contracts mode n. Host memory; no device work.
 * Returns the number of launches (the first min(cap, number) are written to out), or
 * -1 for a NULL handle, cap < 0 or out NULL with cap > 0. */
typedef struct tgrad_launch {
  int32_t kernel;   /* kernel id, see tgrad_kernel_name */
  int32_t modes;
  int64_t bytes_read, bytes_written, flops;
} tgrad_launch;
int tgrad_last_launches(const tgrad_t *h, tgrad_launch *out, int cap);

/* ---------------------------------------------------------------- timing.
 * When enabled, every kernel launch of step/refresh is bracketed by HIP events on
 * the launch stream (at most max_records launches are kept). tgrad_timing_read
 * synchronises, then returns per-kernel-id totals: launches[id] and ms[id] for
 * id < n_ids (n_ids <= TGRAD_MAX_KERNEL_IDS) and resets the records. */
#define TGRAD_MAX_KERNEL_IDS 48
int tgrad_timing_enable(tgrad_t *h, int enable, int max_records);
int tgrad_timing_read(tgrad_t *h, int64_t *launches, double *ms, int n_ids);
/* Restricts the timing above to the launches of kernel id (0 <= id <
 * TGRAD_MAX_KERNEL_IDS, see tgrad_kernel_name), so that a timed run carries one event
 * pair per launch of that kernel and none around the others; id = -1 times every launch
 * again (the default). Errors: TGRAD_EINVAL (NULL handle, id out of range). */
int tgrad_timing_only(tgrad_t *h, int id);
const char *tgrad_kernel_name(int id);

#ifdef __cplusplus
}
#endif
#endif /* TGRAD_H */
