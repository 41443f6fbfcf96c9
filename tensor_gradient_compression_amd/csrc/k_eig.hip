// Small symmetric / Hermitian eigensolver for the HOSVD factors, on device.
//
// U(n) = the r_n leading eigenvectors of the mode-n Gram matrix of the residual
// (pith.science "What carries the argument": Tucker / higher-order SVD factors U^(n);
// its appendix M excerpt: the factors are orthonormal, P^T P = I). One workgroup
// diagonalises one I x I matrix held in LDS in fp64. Real matrices up to 64 take the
// tridiagonal route (k_eig_tri, below); the Jacobi kernels serve complex matrices, modes
// wider than 64, and the real matrices the tridiagonal route hands over. The parallel
// cyclic Jacobi method: each sweep visits every (p, q) pair once, in I - 1 rounds of disjoint
// pairs (round-robin order); within a round every rotation is computed from the same
// matrix, then all column updates (A <- A J, V <- V J) and all row updates
// (A <- J^H A) are applied. Hermitian rotations first turn a_pq real with a phase on
// column q, then apply the real rotation. Sweeps stop when the off-diagonal energy is
// below 1e-20 of the total (an off-diagonal norm of 1e-10 of the matrix norm, so an
// eigenvector errs by about 1e-10 over its relative eigengap), or after MAX_SWEEPS
// sweeps; each matrix reports the sweeps it took, or -1 when the cap came first (0
// when the tridiagonal route served it).
//
// Outputs (pages silent on eigenvector order, sign and phase): eigenvalues descending
// (equal values keep index order); each selected column scaled by a unit scalar so its
// largest-magnitude entry (lowest row on ties) is real positive; U stored fp32, and
// from those fp32 values the two MFMA operand matrices of the mode products: Mproj
// ((r*P) x (I*P), the real form of U^H) and Mrec ((I*P) x (r*P), the real form of U).
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int NTH = 256;
constexpr int MAX_SWEEPS = 40;
constexpr int EIG_HANDOFF = -2;   // status of a matrix the tridiagonal route leaves to Jacobi

struct EK1 {
  const double* gram;
  float* U;
  float* Mproj;
  float* Mrec;
  double* eigvals;
  int* status;
  uint32_t n, r;
};
// One workgroup per matrix; up to 8 matrices (one per compressed mode) per launch.
// handoff_only: act only on the matrices whose status is EIG_HANDOFF.
struct EK {
  EK1 m[8];
  int handoff_only;
};

// ---------------------------------------------------------------- real symmetric case
// Same method and arithmetic as above (parallel cyclic Jacobi in fp64, round-robin
// pairs, each rotation from the same matrix, A <- J^T A J as the column rotation then
// the row rotation), organised for one 1024-thread workgroup per matrix: per round, the
// rotations are formed, then one pass applies the two-sided update to every 2 x 2 block
// (pair a rows, pair b columns) of A and the column rotation to V. Every element sees
// the same operations in the same order as a column pass followed by a row pass.
constexpr int NTS = 1024;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 1/x (normal x) and 1/sqrt(x) (positive normal x): v_rcp_f64 / v_rsq_f64 and two Newton
// steps
__device__ __forceinline__ double rcp64(double x) {
  double y = __builtin_amdgcn_rcp(x);
  y = fma(y, fma(-x, y, 1.0), y);
  return fma(y, fma(-x, y, 1.0), y);
}
__device__ __forceinline__ double rsq64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = fma(0.5 * y, fma(-x * y, y, 1.0), y);
  return fma(0.5 * y, fma(-x * y, y, 1.0), y);
}

__global__ void __launch_bounds__(NTS) k_eig_sym(EK kk) {
  extern __shared__ double sm[];
  const EK1& k = kk.m[blockIdx.x];
  if (kk.handoff_only && *k.status != EIG_HANDOFF) return;   // the same for every thread
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t n = k.n;
  const uint32_t LD = n + 1;          // odd row stride: column walks hit distinct banks
  const uint32_t nn = n * LD;
  double* A = sm;
  double* V = A + nn;
  double2* cs = (double2*)(V + nn);   // 32 rotations: (cos, sin), the sign of a_pq folded in
  double* red = (double*)(cs + 32);   // 2 x 16 wave partials
  int* order = (int*)(red + 32);      // 64

  for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTS) {
    const uint32_t i = idx0 / n, j = idx0 - i * n;
    A[i * LD + j] = 0.5 * (k.gram[(uint64_t)i * n + j] + k.gram[(uint64_t)j * n + i]);
    V[i * LD + j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();

  const uint32_t m = n + (n & 1u);   // even number of players; player n is a bye
  const uint32_t half = m / 2;
  // this thread's share of every round (n <= 64, so half * half <= NTS and n * half <=
  // 2 NTS): the 2 x 2 block (blk_a, blk_b) of A and rows vi[h] of V's column pair vb[h]
  const int blk_a = tid < half * half ? (int)(tid / half) : -1;
  const int blk_b = tid < half * half ? (int)(tid - (tid / half) * half) : -1;
  int vb[2];
  uint32_t vi[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t t = tid + (uint32_t)h * NTS;
    vb[h] = t < n * half ? (int)(t / n) : -1;
    vi[h] = t < n * half ? t - (t / n) * n : 0u;
  }
  int sweeps = -1;
  for (int sweep = 0;; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTS) {
      const uint32_t i = idx0 / n, j = idx0 - i * n;
      const double a = A[i * LD + j];
      tot += a * a;
      if (i != j) off += a * a;
    }
    off = wave_sum(off);
    tot = wave_sum(tot);
    if (lane == 0) {
      red[wave] = off;
      red[16 + wave] = tot;
    }
    __syncthreads();
    off = 0.0;
    tot = 0.0;
    for (int w = 0; w < NTS / 64; ++w) {
      off += red[w];
      tot += red[16 + w];
    }
    if (!(off > 1e-20 * tot)) {
      sweeps = sweep;
      break;
    }
    if (sweep == MAX_SWEEPS) break;

    for (uint32_t round = 0; round + 1 < m; ++round) {
      // pair j of this round: the players at positions j and m - 1 - j of the round-robin
      // (position 0 fixed, the others rotated by `round`); q = -1 for a bye
      auto pair = [&](uint32_t j, int& p, int& q) {
        auto player = [&](uint32_t pos) -> uint32_t {
          if (pos == 0) return 0u;
          uint32_t x = pos - 1u + round;   // < 2 (m - 1)
          if (x >= m - 1u) x -= m - 1u;
          return 1u + x;
        };
        const uint32_t x = player(j), y = player(m - 1 - j);
        const uint32_t lo = x < y ? x : y, hi = x < y ? y : x;
        p = (int)lo;
        q = hi < n ? (int)hi : -1;
      };
      if (tid < half) {
        int p, q;
        pair(tid, p, q);
        double c = 1.0, ss = 0.0;
        if (q >= 0) {
          const double app = A[p * LD + p], aqq = A[q * LD + q];
          const double xr = A[p * LD + q];
          const double rr = fabs(xr);
          if (rr > 0.0) {
            // theta, t and c from the hardware reciprocal and reciprocal square root,
            // each refined by two Newton steps: the angle is as good as a divided one,
            // and c, s are orthogonal to fp64 rounding (both come from the same t)
            const double d = 2.0 * rr;
            const double theta = d >= 2.2250738585072014e-308 ? (aqq - app) * rcp64(d)
                                                             : (aqq - app) / d;
            double t;
            if (fabs(theta) > 1e100) {
              t = 0.5 * rcp64(theta);
            } else {
              const double u = theta * theta + 1.0;
              t = (theta >= 0.0 ? 1.0 : -1.0) * rcp64(fabs(theta) + u * rsq64(u));
            }
            c = rsq64(t * t + 1.0);
            ss = (t * c) * (xr >= 0.0 ? 1.0 : -1.0);
          }
        }
        cs[tid] = make_double2(c, ss);
      }
      __syncthreads();
      // A: block (pair a rows) x (pair b columns); a bye or an unrotated pair acts as
      // the identity on its index
      if (blk_a >= 0) {
        const uint32_t a = (uint32_t)blk_a, b = (uint32_t)blk_b;
        int pa, qa, pb, qb;
        pair(a, pa, qa);
        pair(b, pb, qb);
        const double2 csa = cs[a], csb = cs[b];
        const double ca = csa.x, sa = csa.y, cb = csb.x, sb = csb.y;
        const bool ra = qa >= 0 && sa != 0.0, rb = qb >= 0 && sb != 0.0;
        if (ra || rb) {
        double x00 = A[pa * LD + pb];
        double x01 = qb >= 0 ? A[pa * LD + qb] : 0.0;
        double x10 = qa >= 0 ? A[qa * LD + pb] : 0.0;
        double x11 = (qa >= 0 && qb >= 0) ? A[qa * LD + qb] : 0.0;
        if (rb) {   // columns pb, qb
          const double y00 = cb * x00 - sb * x01, y01 = sb * x00 + cb * x01;
          const double y10 = cb * x10 - sb * x11, y11 = sb * x10 + cb * x11;
          x00 = y00; x01 = y01; x10 = y10; x11 = y11;
        }
        if (ra) {   // rows pa, qa
          const double z00 = ca * x00 - sa * x10, z10 = sa * x00 + ca * x10;
          const double z01 = ca * x01 - sa * x11, z11 = sa * x01 + ca * x11;
          x00 = z00; x10 = z10; x01 = z01; x11 = z11;
        }
        A[pa * LD + pb] = x00;
        if (qb >= 0) A[pa * LD + qb] = x01;
        if (qa >= 0) A[qa * LD + pb] = x10;
        if (qa >= 0 && qb >= 0) A[qa * LD + qb] = x11;
        }
      }
      // V <- V J (columns)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (vb[h] < 0) continue;
        const uint32_t b = (uint32_t)vb[h], i = vi[h];
        int pb, qb;
        pair(b, pb, qb);
        const double2 csb = cs[b];
        const double cb = csb.x, sb = csb.y;
        if (qb < 0 || sb == 0.0) continue;
        const double vx = V[i * LD + pb], vy = V[i * LD + qb];
        V[i * LD + pb] = cb * vx - sb * vy;
        V[i * LD + qb] = sb * vx + cb * vy;
      }
      __syncthreads();
    }
  }

  if (tid == 0) *k.status = sweeps;
  // Descending order of the diagonal, equal values in index order: rank of each entry.
  if (tid < n) {
    const double d = A[tid * LD + tid];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const double e = A[j * LD + j];
      rank += (e > d || (e == d && j < tid)) ? 1u : 0u;
    }
    order[rank] = (int)tid;
  }
  __syncthreads();
  if (tid < n) k.eigvals[tid] = A[order[tid] * LD + order[tid]];

  // one wave per selected column: largest |entry| (lowest row on ties) made positive
  const uint32_t r = k.r;
  for (uint32_t c = wave; c < r; c += NTS / 64) {
    const uint32_t src = (uint32_t)order[c];
    const double x = lane < n ? V[lane * LD + src] : 0.0;
    double best = lane < n ? x * x : -1.0;
    uint32_t bi = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off, 64);
      const uint32_t oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    const double vmax = __shfl(x, bi, 64);
    const double sr = vmax != 0.0 ? (vmax > 0.0 ? 1.0 : -1.0) : 1.0;
    if (lane < n) {
      const float u = (float)(x * sr);
      k.U[(uint64_t)lane * r + c] = u;
      k.Mproj[(uint64_t)c * n + lane] = u;
      k.Mrec[(uint64_t)lane * r + c] = u;
    }
  }
}

// ---------------------------------------------------------------- real symmetric, I <= 64
// Tridiagonal route for real matrices, the default for I <= 64: Householder reduction
// A = Q T Q^T; all eigenvalues of T by multisection on Sturm counts; the r leading
// eigenvectors of T by inverse iteration; each brought back to A's basis by the
// reflectors. Jacobi needs I - 1 workgroup-synchronised rounds per sweep and 8-10
// sweeps; here only the reduction (I - 2 steps of three barriers) is synchronised, and
// every later stage runs each eigenvalue or vector on its own lanes without a barrier.
//
// Reduction step c (column c below the diagonal, length m = I - 1 - c): the reflector
// H = I - tau v v^T with v_0 = 1 that maps x = A[c+1:, c] to beta e_1, beta = -sign(x_0)
// ||x||, tau = (beta - x_0) / beta, v = x / (x_0 - beta) past v_0 (tau = 0 and no step
// when x is already a multiple of e_1); then the trailing block B <- H B H as the
// symmetric rank-2 update B - v w^T - w v^T with p = tau B v and w = p - (tau / 2)
// (p^T v) v. The update keeps B exactly symmetric (both triangles add the same two
// products).
//
// Eigenvalues: the number of eigenvalues of T below x is the number of sign changes in
// the leading principal minors of T - x I, P_0 = 1, P_1 = d_0 - x, P_k = (d_{k-1} - x)
// P_{k-1} - e_{k-2}^2 P_{k-2} (Sylvester's law of inertia on T - x I = L D L^T; a zero
// minor is taken as a tiny negative one, a zero pivot counting as negative). The pair
// (P_k, P_{k-1}) is rescaled by a power of two every four terms, which keeps every sign.
// Sixteen lanes own eigenvalue j (ascending): each step they count at the sixteen inner
// points of a 17-part split of the bracket [a, b] (count(a) <= j < count(b), from the
// Gershgorin interval) and keep the part that holds it; 14 steps shrink the bracket by
// 17^14 > 2^57 for the r leading eigenvalues, 6 steps by 17^6 for the others, which are
// only reported.
//
// Eigenvectors: for each of the r largest eigenvalues (one lane each) two rounds of
// inverse iteration, (T - lambda I) y = z then z = y / ||y||, from a fixed pseudo-random
// z: Gaussian elimination with partial pivoting between neighbouring rows (a zero pivot
// replaced by eps ||T||), the factors kept in LDS for the back substitution. An
// eigenvalue known to about eps ||T|| makes one round converge already. Inverse
// iteration leaves eigenvectors of eigenvalues closer than its error bound
// non-orthogonal: when two of the r leading eigenvalues lie within 1e-9 ||T|| of each
// other (or any eigenvalue is not a number) the matrix is handed to the Jacobi kernel,
// which runs after this one and acts only on matrices marked so.
//
// The matrix is scaled by a power of two first, so that no product overflows or
// underflows, and the eigenvalues are scaled back exactly. A zero matrix, or one with an
// infinite entry, goes to the Jacobi kernel as well.
constexpr int NTQ = 1024;
constexpr uint32_t QP = NTQ / 64;   // lanes per row, column or eigenvalue (one DPP row)
static_assert(QP == 16, "the row reductions span 16 lanes");
// multisection steps: the r leading eigenvalues, which the inverse iteration and the
// eigengap test use, to (QP + 1)^-14 < 2^-57 of the Gershgorin interval; the others, which
// are only reported, to (QP + 1)^-6 < 5e-8 of it
constexpr int MS_STEPS = 14;
constexpr int MS_STEPS_TAIL = 6;
constexpr uint32_t LDY = 65;      // row stride of the eigenvectors of T in LDS

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmin(v, __shfl_xor(v, off, 64));
  return v;
}

// Reductions over a row of 16 lanes by data-parallel-primitive moves (quad butterflies,
// then the half-row and row mirrors): every lane of the row ends with the same sum, added
// in the same order. A wave's total adds the four row sums read from lanes 0, 16, 32, 48.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  v += dpp_f64<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ double lane_value(double v, int at) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, at);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), at);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_total(double v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// eigenvalues of the tridiagonal (d, e) below x, from de[k] = (d_k, e_{k-1}^2) in LDS,
// padded past k = I - 1 up to a multiple of four terms with (above the Gershgorin
// interval, 0), which leave every sign as it is. A zero minor is replaced by -2^-1000
// (a zero pivot counts as negative), and sign changes are counted from the sign bits.
__device__ uint32_t sturm_count(const double2* de, uint32_t nt, double x) {
  double p0 = 1.0, p1 = de[0].x - x;
  p1 = p1 == 0.0 ? -9.332636185032189e-302 : p1;
  uint32_t cnt = (uint32_t)(__builtin_bit_cast(uint64_t, p1) >> 63);
  for (uint32_t k0 = 1; k0 < nt; k0 += 4) {
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const double2 t = de[k0 + u];
      double p2 = (t.x - x) * p1 - t.y * p0;
      p2 = p2 == 0.0 ? -9.332636185032189e-302 : p2;
      cnt += (uint32_t)((__builtin_bit_cast(uint64_t, p2) ^ __builtin_bit_cast(uint64_t, p1)) >> 63);
      p0 = p1;
      p1 = p2;
    }
    int ex;
    (void)frexp(fmax(fabs(p0), fabs(p1)), &ex);
    p0 = ldexp(p0, -ex);
    p1 = ldexp(p1, -ex);
  }
  return cnt;
}

// a fixed pseudo-random start vector entry in [-1, 1) for row k of solve c
__device__ __forceinline__ double start_entry(uint32_t k, uint32_t c) {
  uint32_t h = k * 0x9E3779B1u + c * 0x85EBCA77u + 0x165667B1u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return (double)h * (1.0 / 4294967296.0) * 2.0 - 1.0;
}

// solves of the inverse iteration per batch (one lane each): 32 for real matrices; 16 for
// Hermitian ones, whose two planes of A leave less LDS for the elimination rows
template <int P> constexpr uint32_t tri_batch() { return P == 1 ? 32u : 16u; }

template <int P>
size_t eig_tri_lds_p(uint32_t I) {
  const size_t LD = I | 1u;
  return (P * I * LD + 64 * LDY + 4 * 64 * tri_batch<P>() + (3 * P + 3) * 64 + 24 + 2 * 68) *
         sizeof(double);
}
size_t eig_tri_lds(uint32_t I) { return eig_tri_lds_p<1>(I); }
size_t eig_trih_lds(uint32_t I) { return eig_tri_lds_p<2>(I); }

// P = 1: real symmetric matrices. P = 2: Hermitian ones, from the stacked real Gram
// (rows and columns i P + p). The reflectors are then complex, H = I - tau v v^H with
// v_0 = 1 and a complex tau chosen so that H^H x = beta e_1 with beta real (tau =
// (beta - x_0) / beta, v = x / (x_0 - beta) past v_0, beta = -sign(Re x_0) ||x||), and the
// trailing block takes B <- H^H B H as B - v w^H - w v^H with p = tau B v and w = p -
// (tau / 2) (p^H v) v. Every column, the last included, is reduced, so T is real
// symmetric tridiagonal and the multisection and inverse iteration are the real ones.
// The eigenvectors come back as X = H_0 H_1 ... H_{I-2} Y, complex.
template <int P>
__global__ void __launch_bounds__(NTQ) k_eig_tri(EK kk) {
  extern __shared__ double sm[];
  const EK1& k = kk.m[blockIdx.x];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t n = k.n, r = k.r;
  constexpr uint32_t SB = tri_batch<P>();
  const uint32_t LD = n | 1u;          // odd row stride: column walks hit distinct banks
  double2* de = (double2*)sm;          // (d_k, e_{k-1}^2), padded to 1 + 4 ceil((I - 1) / 4)
                                       // (first: 16-byte reads need 16-byte alignment)
  double* A = sm + 2 * 68;             // n x LD (P = 2: the real plane, then the imaginary
                                       // one); the reflectors end up below its diagonal
  double* Ai = A + (P - 1) * n * LD;   // P = 2: the imaginary plane
  double* Y = A + P * n * LD;          // the eigenvectors of T (columns), rows of LDY
  double* W = Y + 64 * LDY;            // elimination rows of SB solves: W[(4 k + a) SB + s]
  double* hv = W + 4 * 64 * SB;        // the current reflector (P = 2: re, then im)
  double* pw = hv + 64 * P;            // p = tau B v
  double* dv = pw + 64 * P;            // T's diagonal
  double* ev = dv + 64;                // T's off-diagonal
  double* tv = ev + 64;                // the taus (P = 2: re, then im)
  double* lam = tv + 64 * P;           // the eigenvalues, ascending
  double* red = lam + 64;              // wave partials; [16], [17]: the Gershgorin interval

  // the power-of-two scale that brings the largest |entry| of the (stacked) Gram into
  // [0.5, 1); for a Hermitian matrix every diagonal entry is a sum of two diagonal entries
  // of the stacked Gram, so its largest eigenvalue is at least that largest entry too
  const uint32_t K = P * n;
  double mx = 0.0;
  for (uint32_t q = tid; q < K * K; q += NTQ) mx = fmax(mx, fabs(k.gram[q]));
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (uint32_t w = 1; w < NTQ / 64; ++w) mx = fmax(mx, red[w]);
  // a zero matrix (every basis is an eigenbasis) and one with an infinite entry go to
  // Jacobi: after the scaling every other matrix has a largest eigenvalue magnitude of
  // at least 1/2, which the pivot floor of the inverse iteration relies on
  if (!(mx > 0.0 && mx <= 1.7976931348623157e308)) {   // the same for every thread
    if (tid == 0) *k.status = EIG_HANDOFF;
    return;
  }
  int ex = 0;
  (void)frexp(mx, &ex);
  const double scale = ldexp(1.0, -ex);
  for (uint32_t q = tid; q < n * n; q += NTQ) {
    const uint32_t i = q / n, j = q - i * n;
    if constexpr (P == 1) {
      A[i * LD + j] = (0.5 * (k.gram[(uint64_t)i * n + j] + k.gram[(uint64_t)j * n + i])) * scale;
    } else {
      // H[i][j] = sum_c x_i conj(x_j): re from the (p, p) blocks, im from the cross ones,
      // symmetrised as the Jacobi kernel does
      auto G = [&](uint32_t a, uint32_t b) { return k.gram[(uint64_t)a * K + b]; };
      const double re1 = G(2 * i, 2 * j) + G(2 * i + 1, 2 * j + 1);
      const double im1 = G(2 * i + 1, 2 * j) - G(2 * i, 2 * j + 1);
      const double re2 = G(2 * j, 2 * i) + G(2 * j + 1, 2 * i + 1);
      const double im2 = G(2 * j + 1, 2 * i) - G(2 * j, 2 * i + 1);
      A[i * LD + j] = (0.5 * (re1 + re2)) * scale;
      Ai[i * LD + j] = (0.5 * (im1 - im2)) * scale;
    }
  }
  __syncthreads();

  // Householder reduction to tridiagonal form
  const uint32_t ri = tid / QP, part = tid % QP;   // row (or column) and its share
  const uint32_t nred = P == 1 ? (n >= 2 ? n - 2 : 0) : n - 1;   // columns reduced
  for (uint32_t c = 0; c < nred; ++c) {
    const uint32_t m = n - 1 - c, b = c + 1;
    if (wave == 0) {
      if constexpr (P == 1) {
        const double x = lane < m ? A[(b + lane) * LD + c] : 0.0;
        const double sig = wave_total(lane >= 1 ? x * x : 0.0);
        const double x0 = lane_value(x, 0);
        double tau = 0.0, beta = x0, inv = 0.0;
        if (sig > 0.0) {
          const double mu = sqrt(x0 * x0 + sig);
          beta = x0 <= 0.0 ? mu : -mu;
          tau = (beta - x0) * rcp64(beta);
          inv = rcp64(x0 - beta);
        }
        const double v = lane == 0 ? 1.0 : x * inv;
        if (lane < m) {
          hv[lane] = v;
          A[(b + lane) * LD + c] = v;
        }
        if (lane == 0) {
          tv[c] = tau;
          ev[c] = beta;
          dv[c] = A[c * LD + c];
        }
      } else {
        const double xr = lane < m ? A[(b + lane) * LD + c] : 0.0;
        const double xi = lane < m ? Ai[(b + lane) * LD + c] : 0.0;
        const double sig = wave_total(lane >= 1 ? xr * xr + xi * xi : 0.0);
        const double x0r = lane_value(xr, 0), x0i = lane_value(xi, 0);
        double tr = 0.0, ti = 0.0, beta = x0r, ir = 0.0, ii = 0.0;
        if (sig > 0.0 || x0i != 0.0) {
          const double mu = sqrt(x0r * x0r + x0i * x0i + sig);
          beta = x0r <= 0.0 ? mu : -mu;
          const double rb = rcp64(beta);
          tr = (beta - x0r) * rb;
          ti = -x0i * rb;
          // 1 / (x_0 - beta)
          const double dr = x0r - beta, di = x0i;
          const double den = rcp64(dr * dr + di * di);
          ir = dr * den;
          ii = -di * den;
        }
        const double vr = lane == 0 ? 1.0 : xr * ir - xi * ii;
        const double vi = lane == 0 ? 0.0 : xr * ii + xi * ir;
        if (lane < m) {
          hv[lane] = vr;
          hv[64 + lane] = vi;
          A[(b + lane) * LD + c] = vr;
          Ai[(b + lane) * LD + c] = vi;
        }
        if (lane == 0) {
          tv[c] = tr;
          tv[64 + c] = ti;
          ev[c] = beta;
          dv[c] = A[c * LD + c];
        }
      }
    }
    __syncthreads();
    if constexpr (P == 1) {
      const double tau = tv[c];
      if (tau == 0.0) continue;   // the same for every thread
      double sp = 0.0;
      if (ri < m)
        for (uint32_t j = part; j < m; j += QP) sp += A[(b + ri) * LD + b + j] * hv[j];
      sp = row16_sum(sp);
      if (ri < m && part == 0) pw[ri] = tau * sp;
      __syncthreads();
      const double kd = 0.5 * tau * wave_total(lane < m ? pw[lane] * hv[lane] : 0.0);
      if (ri < m) {
        const double vi = hv[ri], wi = pw[ri] - kd * vi;
        for (uint32_t j = part; j < m; j += QP) {
          const double vj = hv[j], wj = pw[j] - kd * vj;
          A[(b + ri) * LD + b + j] -= vi * wj + wi * vj;
        }
      }
    } else {
      const double tr = tv[c], ti = tv[64 + c];
      if (tr == 0.0 && ti == 0.0) continue;   // the same for every thread
      // sp = (B v)_ri, then p = tau sp
      double sr = 0.0, si = 0.0;
      if (ri < m)
        for (uint32_t j = part; j < m; j += QP) {
          const double br = A[(b + ri) * LD + b + j], bi = Ai[(b + ri) * LD + b + j];
          const double vr = hv[j], vi = hv[64 + j];
          sr += br * vr - bi * vi;
          si += br * vi + bi * vr;
        }
      sr = row16_sum(sr);
      si = row16_sum(si);
      if (ri < m && part == 0) {
        pw[ri] = tr * sr - ti * si;
        pw[64 + ri] = tr * si + ti * sr;
      }
      __syncthreads();
      // kd = (tau / 2) (p^H v)
      const double pr = lane < m ? pw[lane] : 0.0, pim = lane < m ? pw[64 + lane] : 0.0;
      const double hr = lane < m ? hv[lane] : 0.0, him = lane < m ? hv[64 + lane] : 0.0;
      const double qr = wave_total(pr * hr + pim * him);
      const double qi = wave_total(pr * him - pim * hr);
      const double kr = 0.5 * (tr * qr - ti * qi), ki = 0.5 * (tr * qi + ti * qr);
      if (ri < m) {
        const double vir = hv[ri], vii = hv[64 + ri];
        const double wir = pw[ri] - (kr * vir - ki * vii);
        const double wii = pw[64 + ri] - (kr * vii + ki * vir);
        for (uint32_t j = part; j < m; j += QP) {
          const double vjr = hv[j], vji = hv[64 + j];
          const double wjr = pw[j] - (kr * vjr - ki * vji);
          const double wji = pw[64 + j] - (kr * vji + ki * vjr);
          // v_i conj(w_j) + w_i conj(v_j)
          A[(b + ri) * LD + b + j] -= (vir * wjr + vii * wji) + (wir * vjr + wii * vji);
          Ai[(b + ri) * LD + b + j] -= (vii * wjr - vir * wji) + (wii * vjr - wir * vji);
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (P == 1 && n >= 2) {
      dv[n - 2] = A[(n - 2) * LD + n - 2];
      ev[n - 2] = A[(n - 1) * LD + n - 2];
    }
    dv[n - 1] = A[(n - 1) * LD + n - 1];
    ev[n - 1] = 0.0;
  }
  __syncthreads();

  // the Gershgorin interval, widened a little
  if (wave == 0) {
    const double dl = lane < n ? dv[lane] : 0.0;
    const double eb = lane < n ? fabs(ev[lane]) : 0.0;
    const double ea = (lane >= 1 && lane < n) ? fabs(ev[lane - 1]) : 0.0;
    const double lo = wave_min(lane < n ? dl - ea - eb : 1.7976931348623157e308);
    const double hi = wave_max(lane < n ? dl + ea + eb : -1.7976931348623157e308);
    const double pad = 8.881784197001252e-16 * fmax(fabs(lo), fabs(hi)) + 1e-300;
    if (lane == 0) {
      red[16] = lo - pad;
      red[17] = hi + pad;
    }
    const double ep = (lane >= 1 && lane < n) ? ev[lane - 1] : 0.0;
    de[lane] = make_double2(lane < n ? dl : hi + pad + 1.0, ep * ep);
    if (lane < 4) de[64 + lane] = make_double2(hi + pad + 1.0, 0.0);
  }
  __syncthreads();

  // multisection: lanes QP j .. QP j + QP - 1 bracket eigenvalue j
  {
    const uint32_t j = tid / QP, q = tid % QP, base = lane & ~(QP - 1);
    const uint32_t nt = 1 + 4 * ((n + 2) / 4);   // terms: 1, then groups of four
    const double step = 1.0 / (double)(QP + 1);
    double a = red[16], b = red[17];
    // the same for a lane group; groups past n have no eigenvalue
    const int steps = j >= n ? 0 : (j + r >= n ? MS_STEPS : MS_STEPS_TAIL);
    for (int it = 0; it < steps; ++it) {
      const double w = b - a;
      const uint32_t cq = sturm_count(de, nt, a + w * ((double)(q + 1) * step));
      // the first point of the group whose count passes j
      const uint64_t hit = (__ballot(cq > j) >> base) & ((1ull << QP) - 1);
      const uint32_t f = hit ? (uint32_t)__builtin_ctzll(hit) : QP;
      const double na = f == 0 ? a : a + w * ((double)f * step);
      const double nb = f == QP ? b : a + w * ((double)(f + 1) * step);
      a = na;
      b = nb;
    }
    if (q == 0 && j < n) lam[j] = 0.5 * (a + b);
  }
  __syncthreads();

  // hand near-degenerate leading eigenvalues (and non-numbers) to the Jacobi kernel
  const double nrm = fmax(fabs(lam[0]), fabs(lam[n - 1]));
  {
    bool bad = lane < n && !(lam[lane] == lam[lane]);
    if (lane + 1 < r) {
      const double gap = lam[n - 1 - lane] - lam[n - 2 - lane];
      bad = bad || !(gap > 1e-9 * nrm);
    }
    if (__ballot(bad) != 0) {   // the same in every wave
      if (tid == 0) *k.status = EIG_HANDOFF;
      return;
    }
  }
  if (tid < n) k.eigvals[tid] = ldexp(lam[n - 1 - tid], ex);
  if (tid == 0) *k.status = 0;

  // inverse iteration, one lane per leading eigenvalue, SB at a time
  if (wave == 0) {
    const double tiny = 2.220446049250313e-16 * fmax(nrm, 0.25);
    for (uint32_t c0 = 0; c0 < r; c0 += SB) {
      const uint32_t c = c0 + lane;
      if (lane < SB && c < r) {
        const double lm = lam[n - 1 - c];
        for (uint32_t i = 0; i < n; ++i) Y[i * LDY + c] = start_entry(i, c);
        for (int round = 0; round < 2; ++round) {
          // elimination: the current row (u0, u1, u2 | rc) against row k + 1
          double u0 = dv[0] - lm, u1 = n > 1 ? ev[0] : 0.0, u2 = 0.0, rc = Y[c];
          for (uint32_t i = 0; i + 1 < n; ++i) {
            double n0 = ev[i], n1 = dv[i + 1] - lm, n2 = i + 2 < n ? ev[i + 1] : 0.0;
            double rn = Y[(i + 1) * LDY + c];
            if (fabs(n0) > fabs(u0)) {
              double t;
              t = u0; u0 = n0; n0 = t;
              t = u1; u1 = n1; n1 = t;
              t = u2; u2 = n2; n2 = t;
              t = rc; rc = rn; rn = t;
            }
            if (u0 == 0.0) u0 = tiny;
            const double iv = rcp64(u0);
            const double l = n0 * iv;
            W[(4 * i + 0) * SB + lane] = iv;
            W[(4 * i + 1) * SB + lane] = u1;
            W[(4 * i + 2) * SB + lane] = u2;
            W[(4 * i + 3) * SB + lane] = rc;
            u0 = n1 - l * u1;
            u1 = n2 - l * u2;
            u2 = 0.0;
            rc = rn - l * rc;
          }
          if (fabs(u0) < tiny) u0 = u0 >= 0.0 ? tiny : -tiny;
          W[(4 * (n - 1) + 0) * SB + lane] = rcp64(u0);
          W[(4 * (n - 1) + 1) * SB + lane] = 0.0;
          W[(4 * (n - 1) + 2) * SB + lane] = 0.0;
          W[(4 * (n - 1) + 3) * SB + lane] = rc;
          // back substitution, then y / ||y||
          double y1 = 0.0, y2 = 0.0, ss = 0.0;
          for (uint32_t i = n; i-- > 0;) {
            const double y = (W[(4 * i + 3) * SB + lane] - W[(4 * i + 1) * SB + lane] * y1 -
                              W[(4 * i + 2) * SB + lane] * y2) * W[(4 * i + 0) * SB + lane];
            Y[i * LDY + c] = y;
            ss += y * y;
            y2 = y1;
            y1 = y;
          }
          const double is = ss > 0.0 && ss <= 1.7976931348623157e308 ? rsq64(ss) : 1.0;
          for (uint32_t i = 0; i < n; ++i) Y[i * LDY + c] *= is;
        }
      }
    }
  }
  __syncthreads();

  // back to A's basis: X = H_0 H_1 ... Y, QP lanes per column, no barrier
  constexpr int NR = 64 / QP;
  const uint32_t col = tid / QP;
  const bool act = col < r;
  if constexpr (P == 1) {
    // rows part + QP t of column tid / QP in registers; the lane groups of columns past r
    // skip the loop (whole waves when r is a multiple of 4)
    double yv[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const uint32_t row = part + QP * t;
      yv[t] = (act && row < n) ? Y[row * LDY + col] : 0.0;
    }
    for (int c = act ? (int)nred - 1 : -1; c >= 0; --c) {
      const double tau = tv[c];
      if (tau == 0.0) continue;   // the same for every active thread
      const uint32_t b = (uint32_t)c + 1;
      double vv[NR], u = 0.0;
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        const uint32_t row = part + QP * t;
        const double v = A[(row < n ? row : n - 1) * LD + c];
        vv[t] = (row >= b && row < n) ? v : 0.0;
      }
#pragma unroll
      for (int t = 0; t < NR; ++t) u += vv[t] * yv[t];
      u = row16_sum(u) * tau;
#pragma unroll
      for (int t = 0; t < NR; ++t) yv[t] -= vv[t] * u;
    }
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const uint32_t row = part + QP * t;
      if (act && row < n) Y[row * LDY + col] = yv[t];
    }
    __syncthreads();

    // one wave per selected column: largest |entry| (lowest row on ties) made positive
    for (uint32_t c = wave; c < r; c += NTQ / 64) {
      const double x = lane < n ? Y[lane * LDY + c] : 0.0;
      double best = lane < n ? x * x : -1.0;
      uint32_t bi = lane;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ob = __shfl_xor(best, off, 64);
        const uint32_t oi = __shfl_xor(bi, off, 64);
        if (ob > best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      const double vmax = __shfl(x, bi, 64);
      const double sr = vmax != 0.0 ? (vmax > 0.0 ? 1.0 : -1.0) : 1.0;
      if (lane < n) {
        const float u = (float)(x * sr);
        k.U[(uint64_t)lane * r + c] = u;
        k.Mproj[(uint64_t)c * n + lane] = u;
        k.Mrec[(uint64_t)lane * r + c] = u;
      }
    }
  } else {
    double yr[NR], yi[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const uint32_t row = part + QP * t;
      yr[t] = (act && row < n) ? Y[row * LDY + col] : 0.0;
      yi[t] = 0.0;
    }
    for (int c = act ? (int)nred - 1 : -1; c >= 0; --c) {
      const double tr = tv[c], ti = tv[64 + c];
      if (tr == 0.0 && ti == 0.0) continue;   // the same for every active thread
      const uint32_t b = (uint32_t)c + 1;
      double vr[NR], vi[NR], ur = 0.0, ui = 0.0;
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        const uint32_t row = part + QP * t;
        const uint32_t rr = row < n ? row : n - 1;
        const bool in = row >= b && row < n;
        const double a = A[rr * LD + c], ai = Ai[rr * LD + c];
        vr[t] = in ? a : 0.0;
        vi[t] = in ? ai : 0.0;
      }
      // u = tau (v^H x)
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        ur += vr[t] * yr[t] + vi[t] * yi[t];
        ui += vr[t] * yi[t] - vi[t] * yr[t];
      }
      ur = row16_sum(ur);
      ui = row16_sum(ui);
      const double qr = tr * ur - ti * ui, qi = tr * ui + ti * ur;
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        yr[t] -= vr[t] * qr - vi[t] * qi;
        yi[t] -= vr[t] * qi + vi[t] * qr;
      }
    }
    // the column's largest-|.| entry (lowest row on ties) made real positive by a unit
    // scalar, then U, Mproj (the real form of U^H) and Mrec (of U); the QP lanes of a
    // column are one DPP row
    double best = -1.0;
    uint32_t bi = 0;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const uint32_t row = part + QP * t;
      const double m2 = row < n ? yr[t] * yr[t] + yi[t] * yi[t] : -1.0;
      if (m2 > best) {   // rows ascend with t: the first of equal values is the lowest row
        best = m2;
        bi = row;
      }
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off, 64);
      const uint32_t oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    // the winning entry: from the lane of the row group that holds row bi
    const uint32_t owner = (lane & ~(QP - 1)) + (bi % QP);
    double wr = 0.0, wi = 0.0;
#pragma unroll
    for (int t = 0; t < NR; ++t)
      if (bi / QP == (uint32_t)t) {
        wr = yr[t];
        wi = yi[t];
      }
    const double vmr = __shfl(wr, owner, 64), vmi = __shfl(wi, owner, 64);
    const double mag = sqrt(vmr * vmr + vmi * vmi);
    const double sr = mag > 0.0 ? vmr / mag : 1.0;     // scale = conj(phase)
    const double si = mag > 0.0 ? -vmi / mag : 0.0;
    if (act) {
      const uint64_t KP = 2ull * n, RP = 2ull * r;
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        const uint32_t i = part + QP * t;
        if (i < n) {
          const float ur = (float)(yr[t] * sr - yi[t] * si);
          const float ui = (float)(yr[t] * si + yi[t] * sr);
          k.U[((uint64_t)i * r + col) * 2] = ur;
          k.U[((uint64_t)i * r + col) * 2 + 1] = ui;
          k.Mproj[(2 * col) * KP + 2 * i] = ur;
          k.Mproj[(2 * col) * KP + 2 * i + 1] = ui;
          k.Mproj[(2 * col + 1) * KP + 2 * i] = -ui;
          k.Mproj[(2 * col + 1) * KP + 2 * i + 1] = ur;
          k.Mrec[(2 * i) * RP + 2 * col] = ur;
          k.Mrec[(2 * i) * RP + 2 * col + 1] = -ui;
          k.Mrec[(2 * i + 1) * RP + 2 * col] = ui;
          k.Mrec[(2 * i + 1) * RP + 2 * col + 1] = ur;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- Hermitian, I <= 64
// The Hermitian form of k_eig_sym: one 1024-thread workgroup per matrix, A and V in LDS
// as real and imaginary planes (fp64), per round the rotations (c, s and the phase
// e^{i phi} = a_pq / |a_pq|) formed by one thread per pair, then one pass that applies
// the two-sided update to every 2 x 2 block (pair a rows, pair b columns) of A and the
// column update to V. Every element sees the operations of a column pass followed by a
// row pass in the same order: columns, y' = e^{-i phi} y on column q then the real
// rotation; rows, y' = e^{+i phi} y on row q then the real rotation.
__global__ void __launch_bounds__(NTS) k_eig_herm(EK kk) {
  extern __shared__ double sm[];
  const EK1& k = kk.m[blockIdx.x];
  if (kk.handoff_only && *k.status != EIG_HANDOFF) return;   // the same for every thread
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t n = k.n;
  const uint32_t LD = n + 1;
  const uint32_t nn = n * LD;
  double* Ar = sm;
  double* Ai = Ar + nn;
  double* Vr = Ai + nn;
  double* Vi = Vr + nn;
  double4* cs = (double4*)(Vi + nn);   // 32 rotations: (c, s, cos phi, sin phi)
  double* red = (double*)(cs + 32);    // 2 x 16 wave partials
  int* order = (int*)(red + 32);       // 64

  // the Hermitian matrix from the stacked real Gram (rows and columns i P + p),
  // symmetrised
  const uint32_t K = 2 * n;
  for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTS) {
    const uint32_t i = idx0 / n, j = idx0 - i * n;
    auto G = [&](uint32_t a, uint32_t b) { return k.gram[(uint64_t)a * K + b]; };
    const double re1 = G(2 * i, 2 * j) + G(2 * i + 1, 2 * j + 1);
    const double im1 = G(2 * i + 1, 2 * j) - G(2 * i, 2 * j + 1);
    const double re2 = G(2 * j, 2 * i) + G(2 * j + 1, 2 * i + 1);
    const double im2 = G(2 * j + 1, 2 * i) - G(2 * j, 2 * i + 1);
    Ar[i * LD + j] = 0.5 * (re1 + re2);
    Ai[i * LD + j] = 0.5 * (im1 - im2);
    Vr[i * LD + j] = (i == j) ? 1.0 : 0.0;
    Vi[i * LD + j] = 0.0;
  }
  __syncthreads();

  const uint32_t m = n + (n & 1u);
  const uint32_t half = m / 2;
  const int blk_a = tid < half * half ? (int)(tid / half) : -1;
  const int blk_b = tid < half * half ? (int)(tid - (tid / half) * half) : -1;
  int vb[2];
  uint32_t vi[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t t = tid + (uint32_t)h * NTS;
    vb[h] = t < n * half ? (int)(t / n) : -1;
    vi[h] = t < n * half ? t - (t / n) * n : 0u;
  }
  int sweeps = -1;
  for (int sweep = 0;; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTS) {
      const uint32_t i = idx0 / n, j = idx0 - i * n;
      const double a2 = Ar[i * LD + j] * Ar[i * LD + j] + Ai[i * LD + j] * Ai[i * LD + j];
      tot += a2;
      if (i != j) off += a2;
    }
    off = wave_sum(off);
    tot = wave_sum(tot);
    if (lane == 0) {
      red[wave] = off;
      red[16 + wave] = tot;
    }
    __syncthreads();
    off = 0.0;
    tot = 0.0;
    for (int w = 0; w < NTS / 64; ++w) {
      off += red[w];
      tot += red[16 + w];
    }
    if (!(off > 1e-20 * tot)) {
      sweeps = sweep;
      break;
    }
    if (sweep == MAX_SWEEPS) break;

    for (uint32_t round = 0; round + 1 < m; ++round) {
      auto pair = [&](uint32_t j, int& p, int& q) {
        auto player = [&](uint32_t pos) -> uint32_t {
          if (pos == 0) return 0u;
          uint32_t x = pos - 1u + round;
          if (x >= m - 1u) x -= m - 1u;
          return 1u + x;
        };
        const uint32_t x = player(j), y = player(m - 1 - j);
        const uint32_t lo = x < y ? x : y, hi = x < y ? y : x;
        p = (int)lo;
        q = hi < n ? (int)hi : -1;
      };
      if (tid < half) {
        int p, q;
        pair(tid, p, q);
        double c = 1.0, sn = 0.0, pc = 1.0, ps = 0.0;
        if (q >= 0) {
          const double app = Ar[p * LD + p], aqq = Ar[q * LD + q];
          const double xr = Ar[p * LD + q], xi = Ai[p * LD + q];
          const double rr = sqrt(xr * xr + xi * xi);
          if (rr > 0.0) {
            const double theta = (aqq - app) / (2.0 * rr);
            double t;
            if (fabs(theta) > 1e100) {
              t = 0.5 / theta;
            } else {
              t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            }
            c = 1.0 / sqrt(t * t + 1.0);
            sn = t * c;
            pc = xr / rr;
            ps = xi / rr;
          }
        }
        cs[tid] = make_double4(c, sn, pc, ps);
      }
      __syncthreads();
      if (blk_a >= 0) {
        const uint32_t a = (uint32_t)blk_a, b = (uint32_t)blk_b;
        int pa, qa, pb, qb;
        pair(a, pa, qa);
        pair(b, pb, qb);
        const double4 ra4 = cs[a], rb4 = cs[b];
        const bool ra = qa >= 0 && ra4.y != 0.0, rb = qb >= 0 && rb4.y != 0.0;
        if (ra || rb) {
          double x00r = Ar[pa * LD + pb], x00i = Ai[pa * LD + pb];
          double x01r = qb >= 0 ? Ar[pa * LD + qb] : 0.0, x01i = qb >= 0 ? Ai[pa * LD + qb] : 0.0;
          double x10r = qa >= 0 ? Ar[qa * LD + pb] : 0.0, x10i = qa >= 0 ? Ai[qa * LD + pb] : 0.0;
          double x11r = (qa >= 0 && qb >= 0) ? Ar[qa * LD + qb] : 0.0;
          double x11i = (qa >= 0 && qb >= 0) ? Ai[qa * LD + qb] : 0.0;
          if (rb) {   // columns pb, qb: y' = e^{-i phi} y, then the rotation
            const double c = rb4.x, sn = rb4.y, pc = rb4.z, ps = rb4.w;
            const double y0r = pc * x01r + ps * x01i, y0i = pc * x01i - ps * x01r;
            const double y1r = pc * x11r + ps * x11i, y1i = pc * x11i - ps * x11r;
            const double n00r = c * x00r - sn * y0r, n00i = c * x00i - sn * y0i;
            const double n01r = sn * x00r + c * y0r, n01i = sn * x00i + c * y0i;
            const double n10r = c * x10r - sn * y1r, n10i = c * x10i - sn * y1i;
            const double n11r = sn * x10r + c * y1r, n11i = sn * x10i + c * y1i;
            x00r = n00r; x00i = n00i; x01r = n01r; x01i = n01i;
            x10r = n10r; x10i = n10i; x11r = n11r; x11i = n11i;
          }
          if (ra) {   // rows pa, qa: y' = e^{+i phi} y, then the rotation
            const double c = ra4.x, sn = ra4.y, pc = ra4.z, ps = ra4.w;
            const double y0r = pc * x10r - ps * x10i, y0i = pc * x10i + ps * x10r;
            const double y1r = pc * x11r - ps * x11i, y1i = pc * x11i + ps * x11r;
            const double n00r = c * x00r - sn * y0r, n00i = c * x00i - sn * y0i;
            const double n10r = sn * x00r + c * y0r, n10i = sn * x00i + c * y0i;
            const double n01r = c * x01r - sn * y1r, n01i = c * x01i - sn * y1i;
            const double n11r = sn * x01r + c * y1r, n11i = sn * x01i + c * y1i;
            x00r = n00r; x00i = n00i; x10r = n10r; x10i = n10i;
            x01r = n01r; x01i = n01i; x11r = n11r; x11i = n11i;
          }
          Ar[pa * LD + pb] = x00r;
          Ai[pa * LD + pb] = x00i;
          if (qb >= 0) {
            Ar[pa * LD + qb] = x01r;
            Ai[pa * LD + qb] = x01i;
          }
          if (qa >= 0) {
            Ar[qa * LD + pb] = x10r;
            Ai[qa * LD + pb] = x10i;
          }
          if (qa >= 0 && qb >= 0) {
            Ar[qa * LD + qb] = x11r;
            Ai[qa * LD + qb] = x11i;
          }
        }
      }
      // V <- V J (columns)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (vb[h] < 0) continue;
        const uint32_t b = (uint32_t)vb[h], i = vi[h];
        int pb, qb;
        pair(b, pb, qb);
        const double4 rb4 = cs[b];
        if (qb < 0 || rb4.y == 0.0) continue;
        const double c = rb4.x, sn = rb4.y, pc = rb4.z, ps = rb4.w;
        const double xr = Vr[i * LD + pb], xi = Vi[i * LD + pb];
        const double y0r = Vr[i * LD + qb], y0i = Vi[i * LD + qb];
        const double yr = pc * y0r + ps * y0i, yi = pc * y0i - ps * y0r;
        Vr[i * LD + pb] = c * xr - sn * yr;
        Vi[i * LD + pb] = c * xi - sn * yi;
        Vr[i * LD + qb] = sn * xr + c * yr;
        Vi[i * LD + qb] = sn * xi + c * yi;
      }
      __syncthreads();
    }
  }

  if (tid == 0) *k.status = sweeps;
  // descending order of the diagonal, equal values in index order
  if (tid < n) {
    const double d = Ar[tid * LD + tid];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const double e = Ar[j * LD + j];
      rank += (e > d || (e == d && j < tid)) ? 1u : 0u;
    }
    order[rank] = (int)tid;
  }
  __syncthreads();
  if (tid < n) k.eigvals[tid] = Ar[order[tid] * LD + order[tid]];

  // one wave per selected column: its largest-|.| entry (lowest row on ties) made real
  // positive by a unit scalar, then U, Mproj (the real form of U^H) and Mrec (of U)
  const uint32_t r = k.r;
  for (uint32_t cc = wave; cc < r; cc += NTS / 64) {
    const uint32_t src = (uint32_t)order[cc];
    const double xr = lane < n ? Vr[lane * LD + src] : 0.0;
    const double xi = lane < n ? Vi[lane * LD + src] : 0.0;
    double best = lane < n ? xr * xr + xi * xi : -1.0;
    uint32_t bi = lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const uint32_t oi = __shfl_xor(bi, o, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    const double vr = __shfl(xr, bi, 64), vim = __shfl(xi, bi, 64);
    const double mag = sqrt(vr * vr + vim * vim);
    const double sr = mag > 0.0 ? vr / mag : 1.0;     // scale = conj(phase)
    const double si = mag > 0.0 ? -vim / mag : 0.0;
    if (lane < n) {
      const uint32_t i = lane;
      const float ur = (float)(xr * sr - xi * si);
      const float ui = (float)(xr * si + xi * sr);
      k.U[((uint64_t)i * r + cc) * 2] = ur;
      k.U[((uint64_t)i * r + cc) * 2 + 1] = ui;
      const uint64_t KP = 2ull * n, RP = 2ull * r;
      k.Mproj[(2 * cc) * KP + 2 * i] = ur;
      k.Mproj[(2 * cc) * KP + 2 * i + 1] = ui;
      k.Mproj[(2 * cc + 1) * KP + 2 * i] = -ui;
      k.Mproj[(2 * cc + 1) * KP + 2 * i + 1] = ur;
      k.Mrec[(2 * i) * RP + 2 * cc] = ur;
      k.Mrec[(2 * i) * RP + 2 * cc + 1] = -ui;
      k.Mrec[(2 * i + 1) * RP + 2 * cc] = ui;
      k.Mrec[(2 * i + 1) * RP + 2 * cc + 1] = ur;
    }
  }
}

size_t eig_herm_lds(uint32_t I) {
  const size_t nn = (size_t)I * (I + 1);
  return (4 * nn + 4 * 32 + 32) * sizeof(double) + 64 * sizeof(int);
}

// ---------------------------------------------------------------- 64 < I <= 128
// The same parallel cyclic Jacobi (round-robin pairs, rotations formed from one matrix
// per round, A <- J^H A J with the column rotation then the row rotation, the Hermitian
// phase on column q), for matrices too large to hold A and V in LDS in fp64: A is kept
// as its packed upper triangle (row i holds a_ii .. a_in; a_ji = conj(a_ij)), and V in
// registers, in round-robin position order: lane j of a wave holds, for 8 of V's rows,
// the two columns that pair j of the current round joins, so a round's column rotation
// is local to the lane; between rounds the players move one position on, which moves
// each held column to a neighbouring lane (two shuffles). 1024 threads: 16 waves of
// V rows; the A update visits the pair blocks (a <= b), the block (b, a) being its
// conjugate transpose. Eigenvector columns are gathered through LDS (the packed A's
// space, 64 columns at a time) for the canonical sign / phase and the outputs.
constexpr int NTB = 1024;
constexpr int RPW = 8;   // V rows a wave holds (I <= 16 RPW)

__device__ __forceinline__ uint32_t tri(uint32_t n, uint32_t i, uint32_t j) {   // i <= j
  return i * n - (i * (i - 1u)) / 2u + (j - i);
}

template <bool CPLX>
__global__ void __launch_bounds__(NTB) k_eig_big(EK kk) {
  extern __shared__ double sm[];
  const EK1& k = kk.m[blockIdx.x];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t n = k.n;
  const uint32_t npk = n * (n + 1) / 2;
  const uint32_t area = npk > 64u * n ? npk : 64u * n;   // A, later 64 columns of V
  double* Ar = sm;
  double* Ai = CPLX ? Ar + area : nullptr;
  double* rot = (CPLX ? Ai : Ar) + area;   // pair j: c, s, Re e^{i phi}, Im e^{i phi}
  double* red = rot + 4 * 64;              // 2 x 16 wave partials
  double* diag = red + 32;                 // 128
  int* rpq = (int*)(diag + 128);           // pair j: p, q (q = -1 for a bye)
  int* order = rpq + 128;                  // 128

  const uint32_t m = n + (n & 1u);
  const uint32_t half = m / 2;
  auto player = [&](uint32_t pos, uint32_t g) -> uint32_t {
    if (pos == 0) return 0u;
    uint32_t x = pos - 1u + g;
    if (x >= m - 1u) x -= m - 1u;
    return 1u + x;
  };
  auto pair = [&](uint32_t j, uint32_t g, int& p, int& q) {
    const uint32_t x = player(j, g), y = player(m - 1 - j, g);
    const uint32_t lo = x < y ? x : y, hi = x < y ? y : x;
    p = (int)lo;
    q = hi < n ? (int)hi : -1;
  };

  // A from the Gram (symmetrised; complex: the Hermitian matrix of the stacked real Gram)
  const uint32_t K = CPLX ? 2 * n : n;
  for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTB) {
    const uint32_t i = idx0 / n, j = idx0 - i * n;
    if (i > j) continue;
    const uint32_t t = tri(n, i, j);
    if (CPLX) {
      auto G = [&](uint32_t a, uint32_t b) { return k.gram[(uint64_t)a * K + b]; };
      const double re1 = G(2 * i, 2 * j) + G(2 * i + 1, 2 * j + 1);
      const double im1 = G(2 * i + 1, 2 * j) - G(2 * i, 2 * j + 1);
      const double re2 = G(2 * j, 2 * i) + G(2 * j + 1, 2 * i + 1);
      const double im2 = G(2 * j + 1, 2 * i) - G(2 * j, 2 * i + 1);
      Ar[t] = 0.5 * (re1 + re2);
      Ai[t] = 0.5 * (im1 - im2);
    } else {
      Ar[t] = 0.5 * (k.gram[(uint64_t)i * n + j] + k.gram[(uint64_t)j * n + i]);
    }
  }
  // V = I in the positions of round 0: slot `lane`, rows wave + 16 r
  double fr[RPW], sr[RPW], fi[RPW], si[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const uint32_t i = wave + 16u * r;
    fr[r] = (lane < half && player(lane, 0) == i) ? 1.0 : 0.0;
    sr[r] = (lane < half && player(m - 1 - lane, 0) == i) ? 1.0 : 0.0;
    fi[r] = 0.0;
    si[r] = 0.0;
  }

  auto getA = [&](int r, int c, double& xr, double& xi) {
    if (r < 0 || c < 0) { xr = 0.0; xi = 0.0; return; }
    if (r <= c) {
      const uint32_t t = tri(n, (uint32_t)r, (uint32_t)c);
      xr = Ar[t];
      xi = CPLX ? Ai[t] : 0.0;
    } else {
      const uint32_t t = tri(n, (uint32_t)c, (uint32_t)r);
      xr = Ar[t];
      xi = CPLX ? -Ai[t] : 0.0;
    }
  };
  auto putA = [&](int r, int c, double xr, double xi) {
    if (r < 0 || c < 0) return;
    if (r <= c) {
      const uint32_t t = tri(n, (uint32_t)r, (uint32_t)c);
      Ar[t] = xr;
      if (CPLX) Ai[t] = xi;
    } else {
      const uint32_t t = tri(n, (uint32_t)c, (uint32_t)r);
      Ar[t] = xr;
      if (CPLX) Ai[t] = -xi;
    }
  };

  int sweeps = -1;
  for (int sweep = 0;; ++sweep) {
    __syncthreads();   // A complete (set-up or the last round)
    double off = 0.0, tot = 0.0;
    for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTB) {
      const uint32_t i = idx0 / n, j = idx0 - i * n;
      if (i > j) continue;
      const uint32_t t = tri(n, i, j);
      const double a2 = Ar[t] * Ar[t] + (CPLX ? Ai[t] * Ai[t] : 0.0);
      if (i == j) {
        tot += a2;
      } else {
        off += 2.0 * a2;
        tot += 2.0 * a2;
      }
    }
    off = wave_sum(off);
    tot = wave_sum(tot);
    if (lane == 0) {
      red[wave] = off;
      red[16 + wave] = tot;
    }
    __syncthreads();
    off = 0.0;
    tot = 0.0;
    for (int w = 0; w < NTB / 64; ++w) {
      off += red[w];
      tot += red[16 + w];
    }
    if (!(off > 1e-20 * tot)) {
      sweeps = sweep;
      break;
    }
    if (sweep == MAX_SWEEPS) break;

    for (uint32_t round = 0; round + 1 < m; ++round) {
      // 1. the round's rotations (pair tid), from the matrix as the last round left it
      if (tid < half) {
        int p, q;
        pair(tid, round, p, q);
        double c = 1.0, s = 0.0, pr = 1.0, pi = 0.0;
        if (q >= 0) {
          const double app = Ar[tri(n, p, p)], aqq = Ar[tri(n, q, q)];
          const uint32_t t = tri(n, p, q);
          const double xr = Ar[t], xi = CPLX ? Ai[t] : 0.0;
          const double rr = CPLX ? sqrt(xr * xr + xi * xi) : fabs(xr);
          if (rr > 0.0) {
            const double d = 2.0 * rr;
            const double theta = d >= 2.2250738585072014e-308 ? (aqq - app) * rcp64(d)
                                                             : (aqq - app) / d;
            double tt;
            if (fabs(theta) > 1e100) {
              tt = 0.5 * rcp64(theta);
            } else {
              const double u = theta * theta + 1.0;
              tt = (theta >= 0.0 ? 1.0 : -1.0) * rcp64(fabs(theta) + u * rsq64(u));
            }
            c = rsq64(tt * tt + 1.0);
            s = tt * c;
            if (CPLX) {
              pr = xr / rr;
              pi = xi / rr;
            } else {
              pr = xr >= 0.0 ? 1.0 : -1.0;
            }
          }
        }
        rot[4 * tid + 0] = c;
        rot[4 * tid + 1] = s;
        rot[4 * tid + 2] = pr;
        rot[4 * tid + 3] = pi;
        rpq[2 * tid] = p;
        rpq[2 * tid + 1] = q;
      }
      __syncthreads();
      // 2. A <- J^H A J on the pair blocks (a <= b)
      for (uint32_t bi = tid; bi < half * half; bi += NTB) {
        const uint32_t a = bi / half, b = bi - a * half;
        if (a > b) continue;
        const int pa = rpq[2 * a], qa = rpq[2 * a + 1], pb = rpq[2 * b], qb = rpq[2 * b + 1];
        const double ca = rot[4 * a], sa = rot[4 * a + 1], par = rot[4 * a + 2], pai = rot[4 * a + 3];
        const double cb = rot[4 * b], sb = rot[4 * b + 1], pbr = rot[4 * b + 2], pbi = rot[4 * b + 3];
        const bool ra = qa >= 0 && sa != 0.0, rb = qb >= 0 && sb != 0.0;
        if (!ra && !rb) continue;
        double x00r, x00i, x01r, x01i, x10r, x10i, x11r, x11i;
        getA(pa, pb, x00r, x00i);
        getA(pa, qb, x01r, x01i);
        getA(qa, pb, x10r, x10i);
        getA(qa, qb, x11r, x11i);
        if (rb) {   // columns pb, qb: y' = conj(ph_b) y; x <- c x - s y', y <- s x + c y'
          auto col = [&](double& xr, double& xi, double& yr, double& yi) {
            const double ur = pbr * yr + pbi * yi, ui = pbr * yi - pbi * yr;
            const double nxr = cb * xr - sb * ur, nxi = cb * xi - sb * ui;
            const double nyr = sb * xr + cb * ur, nyi = sb * xi + cb * ui;
            xr = nxr; xi = nxi; yr = nyr; yi = nyi;
          };
          col(x00r, x00i, x01r, x01i);
          col(x10r, x10i, x11r, x11i);
        }
        if (ra) {   // rows pa, qa: y' = ph_a y; x <- c x - s y', y <- s x + c y'
          auto row = [&](double& xr, double& xi, double& yr, double& yi) {
            const double ur = par * yr - pai * yi, ui = par * yi + pai * yr;
            const double nxr = ca * xr - sa * ur, nxi = ca * xi - sa * ui;
            const double nyr = sa * xr + ca * ur, nyi = sa * xi + ca * ui;
            xr = nxr; xi = nxi; yr = nyr; yi = nyi;
          };
          row(x00r, x00i, x10r, x10i);
          row(x01r, x01i, x11r, x11i);
        }
        if (a == b) {   // pa < qa: the upper entries of the diagonal block
          putA(pa, pa, x00r, CPLX ? 0.0 : x00i);
          putA(pa, qa, x01r, x01i);
          putA(qa, qa, x11r, CPLX ? 0.0 : x11i);
        } else {
          putA(pa, pb, x00r, x00i);
          putA(pa, qb, x01r, x01i);
          putA(qa, pb, x10r, x10i);
          putA(qa, qb, x11r, x11i);
        }
      }
      // 3. V <- V J on the lane's pair, then every held column moves one position on
      if (lane < half) {
        int p, q;
        pair(lane, round, p, q);
        const double c = rot[4 * lane], s = rot[4 * lane + 1];
        const double phr = rot[4 * lane + 2], phi = rot[4 * lane + 3];
        if (q >= 0 && s != 0.0) {
          const bool fp = player(lane, round) == (uint32_t)p;   // the first slot holds p
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            const double vpr = fp ? fr[r] : sr[r], vpi = fp ? fi[r] : si[r];
            const double vqr = fp ? sr[r] : fr[r], vqi = fp ? si[r] : fi[r];
            const double yr = phr * vqr + phi * vqi, yi = phr * vqi - phi * vqr;   // conj(ph) vq
            const double npr = c * vpr - s * yr, npi = c * vpi - s * yi;
            const double nqr = s * vpr + c * yr, nqi = s * vpi + c * yi;
            if (fp) {
              fr[r] = npr; fi[r] = npi; sr[r] = nqr; si[r] = nqi;
            } else {
              sr[r] = npr; si[r] = npi; fr[r] = nqr; fi[r] = nqi;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const double fnr = __shfl(fr[r], (int)lane + 1, 64), snr = __shfl(sr[r], (int)lane - 1, 64);
        const double f1r = __shfl(fr[r], 1, 64);
        double fni = 0.0, sni = 0.0, f1i = 0.0;
        if (CPLX) {
          fni = __shfl(fi[r], (int)lane + 1, 64);
          sni = __shfl(si[r], (int)lane - 1, 64);
          f1i = __shfl(fi[r], 1, 64);
        }
        if (lane == 0) {
          sr[r] = f1r;
          si[r] = f1i;
        } else if (lane < half) {
          const double nfr = lane + 1 == half ? sr[r] : fnr;
          const double nfi = lane + 1 == half ? si[r] : fni;
          sr[r] = snr;
          si[r] = sni;
          fr[r] = nfr;
          fi[r] = nfi;
        }
        __builtin_amdgcn_sched_barrier(0);   // one row's shuffles in flight at a time
      }
      __syncthreads();   // the rotations and A are rewritten next round
    }
  }
  __syncthreads();
  if (tid == 0) *k.status = sweeps;
  if (tid < n) diag[tid] = Ar[tri(n, tid, tid)];
  __syncthreads();
  // descending order of the diagonal, equal values in index order
  if (tid < n) {
    const double d = diag[tid];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const double e = diag[j];
      rank += (e > d || (e == d && j < tid)) ? 1u : 0u;
    }
    order[rank] = (int)tid;
  }
  __syncthreads();
  if (tid < n) k.eigvals[tid] = diag[order[tid]];

  // columns of V through LDS, 64 players at a time (column-major, n rows each); one wave
  // per selected column: largest |entry| (lowest row on ties) made real positive
  const uint32_t r = k.r;
  for (uint32_t cb = 0; cb < n; cb += 64) {
    __syncthreads();
    if (lane < half) {
      const uint32_t xs[2] = {player(lane, 0), player(m - 1 - lane, 0)};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = xs[h];
        if (x >= n || x < cb || x >= cb + 64) continue;
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          const uint32_t i = wave + 16u * rr;
          if (i >= n) continue;
          Ar[(x - cb) * n + i] = h == 0 ? fr[rr] : sr[rr];
          if (CPLX) Ai[(x - cb) * n + i] = h == 0 ? fi[rr] : si[rr];
        }
      }
    }
    __syncthreads();
    for (uint32_t c = wave; c < r; c += NTB / 64) {
      const uint32_t src = (uint32_t)order[c];
      if (src < cb || src >= cb + 64) continue;
      const double* colr = Ar + (src - cb) * n;
      const double* coli = CPLX ? Ai + (src - cb) * n : nullptr;
      double best = -1.0;
      uint32_t bi = 0;
      for (uint32_t i = lane; i < n; i += 64) {
        const double vr = colr[i], vi = CPLX ? coli[i] : 0.0;
        const double a2 = vr * vr + vi * vi;
        if (a2 > best) { best = a2; bi = i; }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ob = __shfl_xor(best, off, 64);
        const uint32_t oi = __shfl_xor(bi, off, 64);
        if (ob > best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      const double mr = colr[bi], mi = CPLX ? coli[bi] : 0.0;
      const double mag = sqrt(mr * mr + mi * mi);
      const double scr = mag > 0.0 ? mr / mag : 1.0;   // scale = conj(phase)
      const double sci = mag > 0.0 ? -mi / mag : 0.0;
      for (uint32_t i = lane; i < n; i += 64) {
        const double xr = colr[i], xi = CPLX ? coli[i] : 0.0;
        const float ur = (float)(xr * scr - xi * sci);
        const float ui = (float)(xr * sci + xi * scr);
        if (CPLX) {
          k.U[((uint64_t)i * r + c) * 2] = ur;
          k.U[((uint64_t)i * r + c) * 2 + 1] = ui;
          const uint64_t KP = 2ull * n, RP = 2ull * r;
          k.Mproj[(2 * c) * KP + 2 * i] = ur;
          k.Mproj[(2 * c) * KP + 2 * i + 1] = ui;
          k.Mproj[(2 * c + 1) * KP + 2 * i] = -ui;
          k.Mproj[(2 * c + 1) * KP + 2 * i + 1] = ur;
          k.Mrec[(2 * i) * RP + 2 * c] = ur;
          k.Mrec[(2 * i) * RP + 2 * c + 1] = -ui;
          k.Mrec[(2 * i + 1) * RP + 2 * c] = ui;
          k.Mrec[(2 * i + 1) * RP + 2 * c + 1] = ur;
        } else {
          k.U[(uint64_t)i * r + c] = ur;
          k.Mproj[(uint64_t)c * n + i] = ur;
          k.Mrec[(uint64_t)i * r + c] = ur;
        }
      }
    }
  }
}

size_t eig_big_lds(uint32_t I, uint32_t P) {
  const size_t npk = (size_t)I * (I + 1) / 2;
  const size_t area = npk > 64u * (size_t)I ? npk : 64u * (size_t)I;
  return (area * P + 4 * 64 + 32 + 128) * sizeof(double) + (128 + 128) * sizeof(int);
}

}  // namespace

size_t eig_lds_bytes(uint32_t I, uint32_t P) {
  const size_t nn = (size_t)I * (I + 1);
  const size_t mats = (P == 2 ? 4 : 2) * nn;
  return (mats + 4 * 32 + NTH) * sizeof(double) + (32 + 32 + 64) * sizeof(int);
}

hipError_t launch_eig(const EigArgs* e, int count, hipStream_t s) {
  if (count < 1 || count > 8) return hipErrorInvalidValue;
  const bool cplx = e[0].P == 2;
  // matrices up to 64 on the LDS-resident kernels, larger ones (up to 128) on k_eig_big
  EK ks{}, kb{};
  int ns = 0, nb = 0;
  size_t lds_s = 0, lds_b = 0, lds_j = 0;
  for (int i = 0; i < count; ++i) {
    if (e[i].I > 128 || e[i].r > e[i].I || e[i].r < 1 || e[i].P != e[0].P) return hipErrorInvalidValue;
    const bool big = e[i].I > 64;
    EK1& m = big ? kb.m[nb++] : ks.m[ns++];
    m.gram = e[i].gram;
    m.U = e[i].U;
    m.Mproj = e[i].Mproj;
    m.Mrec = e[i].Mrec;
    m.eigvals = e[i].eigvals;
    m.status = e[i].status;
    m.n = e[i].I;
    m.r = e[i].r;
    const size_t b = big ? eig_big_lds(e[i].I, e[i].P)
                         : (cplx ? eig_trih_lds(e[i].I) : eig_tri_lds(e[i].I));
    size_t& l = big ? lds_b : lds_s;
    if (b > l) l = b;
    if (!big) lds_j = std::max(lds_j, cplx ? eig_herm_lds(e[i].I) : eig_lds_bytes(e[i].I, 1));
  }
  auto go = [&](auto fn, int nm, int nt, size_t lds, const EK& args) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t err = hipFuncSetAttribute((const void*)fn,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(fn, dim3(nm), dim3(nt), lds, s, args);
    return hipGetLastError();
  };
  if (ns) {
    // the tridiagonal route, then Jacobi on the matrices it handed over
    hipError_t err = cplx ? go(k_eig_tri<2>, ns, NTQ, lds_s, ks) : go(k_eig_tri<1>, ns, NTQ, lds_s, ks);
    if (err != hipSuccess) return err;
    EK kj = ks;
    kj.handoff_only = 1;
    err = cplx ? go(k_eig_herm, ns, NTS, lds_j, kj) : go(k_eig_sym, ns, NTS, lds_j, kj);
    if (err != hipSuccess) return err;
  }
  if (nb) {
    hipError_t err = cplx ? go(k_eig_big<true>, nb, NTB, lds_b, kb)
                          : go(k_eig_big<false>, nb, NTB, lds_b, kb);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace tg
