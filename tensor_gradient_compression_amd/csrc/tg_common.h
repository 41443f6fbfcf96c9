// Internal declarations shared by the HIP sources of libtgrad (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_C64 = 3 };

// bf16 held as its 16-bit pattern.
struct bf16_t { uint16_t b; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x.b) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
// Round to nearest even (gfx950's v_cvt_pk_bf16_f32); a NaN stays a NaN.
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  const __bf16 h = (__bf16)x;
  bf16_t r;
  __builtin_memcpy(&r.b, &h, 2);
  return r;
}
template <typename T> __device__ __forceinline__ T zero_of();
template <> __device__ __forceinline__ float zero_of<float>() { return 0.0f; }
template <> __device__ __forceinline__ _Float16 zero_of<_Float16>() { return (_Float16)0.0f; }
template <> __device__ __forceinline__ bf16_t zero_of<bf16_t>() { bf16_t z; z.b = 0; return z; }

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt) and not for its global loads, stores or global->LDS transfers (vmcnt), which
// __syncthreads() would also wait for. Kernels that double-buffer with global_load_lds
// publish a transfer with an explicit s_waitcnt before the barrier that precedes its
// first read. The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Position of element e in Omega given the membership bitmask and per-word ranks.
__device__ __forceinline__ uint32_t omega_rank(const uint64_t* mask, const uint32_t* rank,
                                               uint64_t e, uint64_t word) {
  uint32_t bit = (uint32_t)(e & 63u);
  return rank[e >> 6] + (uint32_t)__popcll(word & ((1ull << bit) - 1ull));
}

struct AdamK {
  float b1, c1, b2, c2, eps, bc1, bc2;
  float lam;   // sparse scale: N_S = lam * (Adam update of S); 1 for the plain method
};

// Kernel ids for per-launch timing (names in tgrad_kernel_name).
enum KernelId {
  KID_TOPK_INIT = 0, KID_TOPK_HIST, KID_TOPK_SELECT, KID_TOPK_COUNT, KID_TOPK_SCAN,
  KID_TOPK_COMPACT, KID_MASK_FROM_OMEGA, KID_GATHER, KID_PROJECT, KID_ADAM,
  KID_RECONSTRUCT, KID_RECON_APPLY, KID_APPLY_DENSE, KID_GRAM, KID_GRAM_REDUCE,
  KID_EIG, KID_FILL, KID_PROJECT_FIRST, KID_PROJECT_FUSED2, KID_RECON_FUSED2_APPLY,
  KID_RECON_FUSED2, KID_REMAP, KID_PROJECT_FUSED3, KID_GRAM3, KID_PROJECT_PAIR, KID_RECON_PAIR,
  KID_RECON_FUSED3_APPLY, KID_STREAM_PROJECT, KID_STREAM_RECONSTRUCT, KID_CSPLIT_OPERAND,
  KID_CSPLIT_COMBINE, KID_ROW_PROJECT, KID_ROW_RECON_APPLY, KID_ADAM_SPARSE, KID_COUNT_
};

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `s` and returns hipGetLastError().

constexpr int TOPK_HIST_BINS = 32768;
struct TopkWs {
  uint32_t* hist;       // TOPK_HIST_BINS bins
  uint64_t* state;      // TopkState (4 x u64)
  uint32_t* ucount;     // 2 per unit
  uint32_t* uoff;       // 2 per unit
  uint32_t* ctot;       // 2 per scan chunk of 8192 units
};
uint64_t topk_units(uint64_t N);
uint64_t topk_chunks(uint64_t N);
// Omega = the k largest keys, ties to the lowest index. randk == 0: magnitude keys of G;
// randk != 0: element e's key is the top 31 bits of SplitMix64's output for the state
// rk_base + 0x9E3779B97F4A7C15 * e (G is then read only for the residual).
hipError_t launch_topk(int dt, const void* G, uint64_t N, uint32_t k, const TopkWs& ws,
                       uint32_t* omega, uint64_t* mask, uint32_t* rank, void* resid,
                       int randk, uint64_t rk_base, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx);
// Sparse moments that follow their element across a refresh: for each j < k with
// e = omega_new[j], (m, v)_new[j] = (m, v)_old[i] if e is in the old Omega (bitmask and
// word ranks of the old Omega give its position i), else 0 (P floats each).
hipError_t launch_remap_moments(const uint64_t* mask_old, const uint32_t* rank_old,
                                const uint32_t* omega_new, uint32_t k, uint32_t P,
                                const float* m_old, const float* v_old, float* m_new,
                                float* v_new, hipStream_t s);
hipError_t launch_mask_from_omega(const uint32_t* omega, uint32_t k, uint64_t* mask,
                                  uint32_t* rank, uint64_t nwords, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t v, hipStream_t s);
hipError_t launch_fill_u64(uint64_t* p, uint64_t n, uint64_t v, hipStream_t s);

hipError_t launch_gather(int dt, void* G, const uint32_t* omega, uint32_t k, float* S,
                         hipStream_t s);
// Low-rank first: S[j] = fp32(G[omega[j]]) - L[omega[j]] (L fp32, P values per element)
hipError_t launch_gather_sub(int dt, const void* G, const float* L, const uint32_t* omega,
                             uint32_t k, float* S, hipStream_t s);
// L[i] <- fp32(G[i]) - L[i] for the n fp32 values of L (complex: re, im pairs)
hipError_t launch_resid_sub(int dt, const void* G, float* L, uint64_t n, hipStream_t s);

// core input dtype: DT_F32 for an fp32 buffer (complex: pairs, P folded into n_core)
hipError_t launch_adam(int core_dt, const void* g_core, float* u_core, float* m_core,
                       float* v_core, uint64_t n_core, float* S, float* m_s, float* v_s,
                       uint64_t n_s, AdamK a, hipStream_t s);
// the k sparse values' update alone: S <- lam * Adam(S), moments m_s, v_s
hipError_t launch_adam_sparse(float* S, float* m_s, float* v_s, uint64_t n_s, AdamK a,
                              hipStream_t s);
// W <- round(fp32(W) * decay - lr * Delta) (decay = fp32(1 - lr * weight_decay); 1 exactly
// without decay)
// delta != NULL (a test capture): Delta, the fp32 update after the sparse merge, is
// also written there (N * P floats).
hipError_t launch_apply_dense(int dt, void* W, const float* u_core, const uint64_t* mask,
                              const uint32_t* rank, const float* u_s, uint64_t N, float lr,
                              float decay, int has_sparse, float* delta, hipStream_t s);

// Complex mode products too wide for one real-block product: Re M and Im M as (rows x
// cols) fp32 matrices from the (2 rows) x (2 cols) real-block operand M, and the
// combination y1 <- y1 + i y2 of the two real products' outputs (y1 = (Re M) x and
// y2 = (Im M) x on the interleaved view; npairs complex values).
hipError_t launch_split_operand(const float* M, uint32_t rows, uint32_t cols, float* re,
                                float* im, hipStream_t s);
hipError_t launch_csplit_combine(float* y1, const float* y2, uint64_t npairs, hipStream_t s);

// Mode product Y[a, jj, b] = sum_kk M[jj, kk] X[a, kk, b] over the (A, I, B, P) view.
struct ModeProd {
  const void* X;   // input, dtype in_dt (P == 2 only with fp32)
  int in_dt;
  const float* M;  // (R*P) x (I*P) row-major
  uint32_t A, I, B, R, P;
  // epilogue: apply == 0 -> store fp32 to Y;
  // apply == 1 -> W <- round(W * decay - lr*(acc + uS@Omega))
  int apply;
  float* Y;
  void* W;
  int w_dt;
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;
  const uint32_t* omega;   // Omega ascending, |Omega| = kS (apply)
  uint64_t kS;
  float lr;
  float decay;
  int has_sparse;
  int force_ncb;           // 0: choose the tile width automatically
  int max_wg;              // streaming kernel: at most this many workgroups (0: no cap)
  // complex (P == 2), streaming kernel only: Re M and Im M as R x I fp32 matrices (the
  // streaming kernel applies to a complex product only when both are given)
  const float* Mre;
  const float* Mim;
  // row kernel only, store form over the gradient: also perform the COO gather,
  // gather_S[j] = X[omega[j]] (fp32, through mask and rank), and project X with Omega
  // cleared (X itself is only read)
  float* gather_S;
  // apply only, a test capture: when not NULL the fp32 update (acc + uS@Omega) is also
  // stored here, one float per output value (a separate kernel instantiation)
  float* delta;
};
size_t modeprod_lds_bytes(const ModeProd& mp);
hipError_t launch_modeprod(const ModeProd& mp, int num_cu, hipStream_t s);
// The same product streamed by independent waves (k_streamprod.hip): fp32 input and
// output (store epilogue), I <= 64, R <= 64 (complex with Mre and Mim), B (complex:
// 2 B) >= 32 and a multiple of 4, X and Y 16-byte aligned.
bool streamprod_supported(const ModeProd& mp);
// A product over the last mode (B == 1) as a stream of rows (k_rowprod.hip): store form
// (fp32, f16 or bf16 input; complex as fp32 pairs with the real-block operand) or
// weight-updating form (fp32 input); K = I P and N = R P small enough for M to sit in
// registers, the input below 2^31 bytes.
bool rowprod_supported(const ModeProd& mp);
hipError_t launch_rowprod(const ModeProd& mp, int num_cu, hipStream_t s);
hipError_t launch_streamprod(const ModeProd& mp, int num_cu, hipStream_t s);

// Two trailing mode products in one launch over slabs (A, I1, I2, P) -> (A, R1, R2, P).
// M1 is (R1*P) x (I1*P) (mode d-1), M2 is (R2*P) x (I2*P) (mode d). recon = 0: mode d
// first (projection); recon = 1: mode d-1 first (reconstruction), optionally applying.
struct ModeProd2 {
  const void* X;
  int in_dt;
  uint32_t P, A, I1, I2, R1, R2;
  int recon;
  const float* M1;
  const float* M2;
  int apply;
  float* Y;
  void* W;
  int w_dt;
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;
  const uint32_t* omega;
  uint64_t kS;
  float lr;
  float decay;
  int has_sparse;
  uint32_t force_ta;       // 0: choose the slabs per tile automatically
  // projection only: also perform the COO gather on the staged input, S[j] = X[omega[j]]
  // (fp32), and project the staged input with Omega zeroed (X itself is only read)
  float* gather_S;
  // three-mode projection: the mode before the two (full size I0, rank R0, operand M0);
  // A then counts (unit, i0) slabs
  uint32_t I0, R0;
  const float* M0;
  // reconstruction with apply, a test capture: when not NULL the fp32 update after the
  // sparse merge is also stored here (N * P floats; a separate kernel instantiation)
  float* delta;
};
uint32_t modeprod2_tile(const ModeProd2& mp);   // 0: does not fit
hipError_t launch_modeprod2(const ModeProd2& mp, int num_cu, hipStream_t s);
// The same two products for 16-bit data, one wave per slab on bf16 MFMAs (projection
// with the gather folded in, or reconstruction with merge and apply); supported when
// P == 1, the slab sizes are small enough (full-size side I1 <= 64, I2 <= 32; core side
// R1 <= 32, R2 <= 16) and the buffers are 16-byte aligned.
bool slab2_supported(const ModeProd2& mp, int num_cu);
hipError_t launch_slab2(const ModeProd2& mp, int num_cu, hipStream_t s);
// Projection over the last three modes in one launch (16-bit data, gather folded in as
// above): one workgroup of 16 waves per index of the leading modes at a time, supported
// when I0 is a multiple of 16 up to 64, R0 <= 32 and the two trailing modes fit the slab
// kernel.
bool slab3_supported(const ModeProd2& mp);
hipError_t launch_slab3(const ModeProd2& mp, int num_cu, hipStream_t s);
// The reconstruction's last three modes with the sparse merge and the weight update in
// one launch (16-bit weights): a workgroup of 12 waves per index of the leading modes at
// a time. mp: recon = 1, apply = 1, I0..I2 the core-side and R0..R2 the full sizes of the
// three modes, A counts (unit, core-side index of mode d-2) blocks, M0..M2 the
// reconstruction operands (full x core). Supported when the full size of mode d-2 is a
// multiple of 12 up to 64, its rank is at most 32, the two trailing modes fit the slab
// kernel, and the buffers are 16-byte aligned.
bool rec3_supported(const ModeProd2& mp);
hipError_t launch_rec3(const ModeProd2& mp, int num_cu, hipStream_t s);

// Two neighbouring mode products (n, n+1) of a real fp32 tensor viewed as (A, I0, I1, C)
// in one launch: Y[a, j0, j1, c] = sum_i0 M0[j0, i0] sum_i1 M1[j1, i1] X[a, i0, i1, c]
// (M0 J0 x I0, M1 J1 x I1, row-major). Supported when C % 16 == 0, I0 is a multiple of
// 4 up to 64, I1 is one of 16, 24, 32, 48, 64, J0, J1 <= 64 and X is 16-byte aligned.
struct ModePair {
  const float* X;
  float* Y;
  const float* M0;
  const float* M1;
  uint32_t A, I0, I1, J0, J1;
  uint64_t C;
};
bool pair_supported(const ModePair& mp);
hipError_t launch_pair(const ModePair& mp, hipStream_t s);

// Gram of the (A, I, B, P) view with Omega entries treated as zero:
// out[x, y] (fp64, (I*P) x (I*P)) = sum over (a, b) of X[a, x, b] X[a, y, b].
struct GramArgs {
  const void* X;
  int dt;
  uint32_t A, I, B, P;
  const uint64_t* mask;  // NULL -> no masking
  double* partial;       // nblk * (I*P)^2
  double* out;           // (I*P)^2
  uint32_t max_blocks;   // 0: as many workgroups (partial sums) as fill the GPU; else at most this
};
uint32_t gram_blocks(const GramArgs& g, int num_cu);
// fp32 / complex64 Grams with I <= 64 and no mask (k_gram32.hip): the launch geometry
// (ok = false where that kernel does not apply) and the launch into `partial`
struct G32Geo {
  bool ok;
  uint32_t grid, P;
  size_t lds;
  alignas(8) unsigned char kbytes[96];
};
G32Geo gram32_geo(const GramArgs& g, int num_cu);
hipError_t launch_gram32(const G32Geo& geo, double* partial, hipStream_t s);
uint32_t gram_reduce_groups();   // partial buffer holds (blocks + groups) * (I*P)^2
size_t gram_lds_bytes(const GramArgs& g);
hipError_t launch_gram(const GramArgs& g, int num_cu, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx);
// Sum nblk partials of n2 fp64 values (RGROUPS stage rows follow them) into out.
hipError_t gram_reduce(double* partial, uint32_t nblk, uint32_t n2, double* out, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx);

// Grams of the last three modes (a, b, c) of a 16-bit tensor viewed as A contiguous
// slabs of Ia x Ib x Ic, from one read: out[m] (fp64, I_m x I_m) as launch_gram gives
// for each of the three modes. Supported for bf16/fp16 when Ia, Ib <= 64, Ic <= 32, a
// slab is a multiple of 8 elements and at most 128 KiB, and X is 16-byte aligned.
// `partial` holds gram3_partial_doubles() values.
struct Gram3Args {
  const void* X;
  int dt;
  uint32_t A, Ia, Ib, Ic;
  const uint64_t* mask;  // Omega's membership bitmask: entries in it read as zero; NULL: none
  double* partial;
  double* out[3];
};
bool gram3_supported(const Gram3Args& g, int num_cu);
uint64_t gram3_partial_doubles(const Gram3Args& g, int num_cu);
hipError_t launch_gram3(const Gram3Args& g, int num_cu, hipStream_t s,
                        void (*mark)(void*, int, bool), void* mctx);

// Eigen-decomposition of the Gram (stacked real (I*P)^2 fp64) and factor outputs.
struct EigArgs {
  const double* gram;
  uint32_t I, r, P;
  float* U;      // I x r (x P)
  float* Mproj;  // (r*P) x (I*P)
  float* Mrec;   // (I*P) x (r*P)
  double* eigvals;  // I
  int* status;      // written: sweeps taken, or -1 if the sweep cap came first
};
size_t eig_lds_bytes(uint32_t I, uint32_t P);
hipError_t launch_eig(const EigArgs* e, int count, hipStream_t s);   // one workgroup each

}  // namespace tg
