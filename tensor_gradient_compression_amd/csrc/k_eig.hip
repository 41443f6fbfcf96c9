// Small symmetric / Hermitian eigensolver for the HOSVD factors, on device.
//
// U(n) = the r_n leading eigenvectors of the mode-n Gram matrix of the residual
// (pith.science "What carries the argument": Tucker / higher-order SVD factors U^(n);
// its appendix M excerpt: the factors are orthonormal, P^T P = I). One workgroup
// diagonalises one I x I matrix (I <= 64) held in LDS in fp64 with the parallel cyclic
// Jacobi method: each sweep visits every (p, q) pair once, in I - 1 rounds of disjoint
// pairs (round-robin order); within a round every rotation is computed from the same
// matrix, then all column updates (A <- A J, V <- V J) and all row updates
// (A <- J^H A) are applied. Hermitian rotations first turn a_pq real with a phase on
// column q, then apply the real rotation. Sweeps stop when the off-diagonal energy is
// below 1e-20 of the total (an off-diagonal norm of 1e-10 of the matrix norm, so an
// eigenvector errs by about 1e-10 over its relative eigengap), or after MAX_SWEEPS
// sweeps; each matrix reports the sweeps it took, or -1 when the cap came first.
//
// Outputs (pages silent on eigenvector order, sign and phase): eigenvalues descending
// (equal values keep index order); each selected column scaled by a unit scalar so its
// largest-magnitude entry (lowest row on ties) is real positive; U stored fp32, and
// from those fp32 values the two MFMA operand matrices of the mode products: Mproj
// ((r*P) x (I*P), the real form of U^H) and Mrec ((I*P) x (r*P), the real form of U).
#include "tg_common.h"

namespace tg {

namespace {

constexpr int NTH = 256;
constexpr int MAX_SWEEPS = 40;

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
struct EK {
  EK1 m[8];
};

__device__ __forceinline__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = NTH / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

template <bool CPLX>
__global__ void __launch_bounds__(NTH) k_eig(EK kk) {
  extern __shared__ double sm[];
  const EK1& k = kk.m[blockIdx.x];
  const int tid = threadIdx.x;
  const uint32_t n = k.n;
  const uint32_t LD = n + 1;          // odd row stride: column walks hit distinct banks
  const uint32_t nn = n * LD;
  double* Ar = sm;
  double* Ai = CPLX ? Ar + nn : nullptr;
  double* Vr = CPLX ? Ai + nn : Ar + nn;
  double* Vi = CPLX ? Vr + nn : nullptr;
  double* tail = (CPLX ? Vi : Vr) + nn;
  double* rc = tail;          // 32 pairs max
  double* rs = rc + 32;
  double* rpc = rs + 32;      // cos(phi)
  double* rps = rpc + 32;     // sin(phi)
  double* red = rps + 32;     // NTH
  int* rp = (int*)(red + NTH);
  int* rq = rp + 32;
  int* order = rq + 32;       // 64

  // Hermitian (or symmetric) matrix from the stacked real Gram, symmetrised.
  const uint32_t K = CPLX ? 2 * n : n;
  for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTH) {
    const uint32_t i = idx0 / n, j = idx0 - i * n;
    const uint32_t idx = i * LD + j;
    if (CPLX) {
      auto G = [&](uint32_t a, uint32_t b) { return k.gram[(uint64_t)a * K + b]; };
      const double re1 = G(2 * i, 2 * j) + G(2 * i + 1, 2 * j + 1);
      const double im1 = G(2 * i + 1, 2 * j) - G(2 * i, 2 * j + 1);
      const double re2 = G(2 * j, 2 * i) + G(2 * j + 1, 2 * i + 1);
      const double im2 = G(2 * j + 1, 2 * i) - G(2 * j, 2 * i + 1);
      Ar[idx] = 0.5 * (re1 + re2);
      Ai[idx] = 0.5 * (im1 - im2);
      Vi[idx] = 0.0;
    } else {
      Ar[idx] = 0.5 * (k.gram[(uint64_t)i * K + j] + k.gram[(uint64_t)j * K + i]);
    }
    Vr[idx] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();

  const uint32_t m = n + (n & 1u);   // even number of players; player n is a bye
  const uint32_t half = m / 2;
  int sweeps = -1;
  for (int sweep = 0;; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (uint32_t idx0 = tid; idx0 < n * n; idx0 += NTH) {
      const uint32_t i = idx0 / n, j = idx0 - i * n;
      const uint32_t idx = i * LD + j;
      const double a2 = Ar[idx] * Ar[idx] + (CPLX ? Ai[idx] * Ai[idx] : 0.0);
      tot += a2;
      if (i != j) off += a2;
    }
    off = block_sum(off, red);
    tot = block_sum(tot, red);
    if (!(off > 1e-20 * tot)) {
      sweeps = sweep;
      break;
    }
    if (sweep == MAX_SWEEPS) break;

    for (uint32_t round = 0; round + 1 < m; ++round) {
      if ((uint32_t)tid < half) {
        auto player = [&](uint32_t pos) -> uint32_t {
          return pos == 0 ? 0u : 1u + (pos - 1u + round) % (m - 1u);
        };
        uint32_t p = player(tid), q = player(m - 1 - tid);
        if (p > q) { uint32_t t = p; p = q; q = t; }
        double c = 1.0, s = 0.0, pc = 1.0, ps = 0.0;
        if (q < n) {
          const double app = Ar[p * LD + p], aqq = Ar[q * LD + q];
          const double xr = Ar[p * LD + q], xi = CPLX ? Ai[p * LD + q] : 0.0;
          const double rr = CPLX ? sqrt(xr * xr + xi * xi) : fabs(xr);
          if (rr > 0.0) {
            const double theta = (aqq - app) / (2.0 * rr);
            double t;
            if (fabs(theta) > 1e100) {
              t = 0.5 / theta;
            } else {
              t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            }
            c = 1.0 / sqrt(t * t + 1.0);
            s = t * c;
            if (CPLX) {
              pc = xr / rr;
              ps = xi / rr;
            } else {
              pc = xr >= 0.0 ? 1.0 : -1.0;
            }
          }
        }
        rc[tid] = c;
        rs[tid] = s;
        rpc[tid] = pc;
        rps[tid] = ps;
        rp[tid] = (int)p;
        rq[tid] = (q < n) ? (int)q : -1;
      }
      __syncthreads();
      // Real case: the phase is the sign of a_pq; folding it into s gives the usual
      // real rotation (c, s*sign) for the symmetric 2x2 problem.
      // Column updates: A[:, p], A[:, q] and V[:, p], V[:, q].
      for (uint32_t idx = tid; idx < n * half; idx += NTH) {
        const uint32_t j = idx / n, i = idx - j * n;
        const int q = rq[j];
        if (q < 0 || rs[j] == 0.0) continue;
        const int p = rp[j];
        const double c = rc[j], s = rs[j], pc = rpc[j], ps = rps[j];
        if (CPLX) {
          // y' = e^{-i phi} * y
          {
            const double xr = Ar[i * LD + p], xi = Ai[i * LD + p];
            const double yr0 = Ar[i * LD + q], yi0 = Ai[i * LD + q];
            const double yr = pc * yr0 + ps * yi0, yi = pc * yi0 - ps * yr0;
            Ar[i * LD + p] = c * xr - s * yr;
            Ai[i * LD + p] = c * xi - s * yi;
            Ar[i * LD + q] = s * xr + c * yr;
            Ai[i * LD + q] = s * xi + c * yi;
          }
          {
            const double xr = Vr[i * LD + p], xi = Vi[i * LD + p];
            const double yr0 = Vr[i * LD + q], yi0 = Vi[i * LD + q];
            const double yr = pc * yr0 + ps * yi0, yi = pc * yi0 - ps * yr0;
            Vr[i * LD + p] = c * xr - s * yr;
            Vi[i * LD + p] = c * xi - s * yi;
            Vr[i * LD + q] = s * xr + c * yr;
            Vi[i * LD + q] = s * xi + c * yi;
          }
        } else {
          const double ss = s * pc;
          const double x = Ar[i * LD + p], y = Ar[i * LD + q];
          Ar[i * LD + p] = c * x - ss * y;
          Ar[i * LD + q] = ss * x + c * y;
          const double vx = Vr[i * LD + p], vy = Vr[i * LD + q];
          Vr[i * LD + p] = c * vx - ss * vy;
          Vr[i * LD + q] = ss * vx + c * vy;
        }
      }
      __syncthreads();
      // Row updates: A[p, :], A[q, :] <- J^H A.
      for (uint32_t idx = tid; idx < n * half; idx += NTH) {
        const uint32_t j = idx / n, col = idx - j * n;
        const int q = rq[j];
        if (q < 0 || rs[j] == 0.0) continue;
        const int p = rp[j];
        const double c = rc[j], s = rs[j], pc = rpc[j], ps = rps[j];
        if (CPLX) {
          // y' = e^{+i phi} * y
          const double xr = Ar[p * LD + col], xi = Ai[p * LD + col];
          const double yr0 = Ar[q * LD + col], yi0 = Ai[q * LD + col];
          const double yr = pc * yr0 - ps * yi0, yi = pc * yi0 + ps * yr0;
          Ar[p * LD + col] = c * xr - s * yr;
          Ai[p * LD + col] = c * xi - s * yi;
          Ar[q * LD + col] = s * xr + c * yr;
          Ai[q * LD + col] = s * xi + c * yi;
        } else {
          const double ss = s * pc;
          const double x = Ar[p * LD + col], y = Ar[q * LD + col];
          Ar[p * LD + col] = c * x - ss * y;
          Ar[q * LD + col] = ss * x + c * y;
        }
      }
      __syncthreads();
    }
  }

  if (tid == 0) *k.status = sweeps;
  // Descending order of the diagonal, equal values in index order.
  if (tid == 0) {
    uint64_t used = 0;
    for (uint32_t pos = 0; pos < n; ++pos) {
      int best = -1;
      double bv = 0.0;
      for (uint32_t i = 0; i < n; ++i) {
        if ((used >> i) & 1ull) continue;
        const double d = Ar[i * LD + i];
        if (best < 0 || d > bv) { best = (int)i; bv = d; }
      }
      used |= 1ull << best;
      order[pos] = best;
    }
  }
  __syncthreads();
  for (uint32_t i = tid; i < n; i += NTH) k.eigvals[i] = Ar[order[i] * LD + order[i]];

  const uint32_t r = k.r;
  const uint32_t P = CPLX ? 2 : 1;
  for (uint32_t c = tid; c < r; c += NTH) {
    const uint32_t src = (uint32_t)order[c];
    uint32_t imax = 0;
    double best = -1.0;
    for (uint32_t i = 0; i < n; ++i) {
      const double vr = Vr[i * LD + src], vi = CPLX ? Vi[i * LD + src] : 0.0;
      const double a2 = vr * vr + vi * vi;
      if (a2 > best) { best = a2; imax = i; }
    }
    const double vr = Vr[imax * LD + src], vi = CPLX ? Vi[imax * LD + src] : 0.0;
    const double mag = sqrt(vr * vr + vi * vi);
    const double sr = mag > 0.0 ? vr / mag : 1.0;     // scale = conj(phase)
    const double si = mag > 0.0 ? -vi / mag : 0.0;
    for (uint32_t i = 0; i < n; ++i) {
      const double xr = Vr[i * LD + src], xi = CPLX ? Vi[i * LD + src] : 0.0;
      const float ur = (float)(xr * sr - xi * si);
      const float ui = (float)(xr * si + xi * sr);
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
    (void)P;
  }
}

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

}  // namespace

size_t eig_lds_bytes(uint32_t I, uint32_t P) {
  const size_t nn = (size_t)I * (I + 1);
  const size_t mats = (P == 2 ? 4 : 2) * nn;
  return (mats + 4 * 32 + NTH) * sizeof(double) + (32 + 32 + 64) * sizeof(int);
}

hipError_t launch_eig(const EigArgs* e, int count, hipStream_t s) {
  if (count < 1 || count > 8) return hipErrorInvalidValue;
  EK k;
  size_t lds = 0;
  for (int i = 0; i < count; ++i) {
    if (e[i].I > 64 || e[i].r > e[i].I || e[i].r < 1 || e[i].P != e[0].P) return hipErrorInvalidValue;
    k.m[i].gram = e[i].gram;
    k.m[i].U = e[i].U;
    k.m[i].Mproj = e[i].Mproj;
    k.m[i].Mrec = e[i].Mrec;
    k.m[i].eigvals = e[i].eigvals;
    k.m[i].status = e[i].status;
    k.m[i].n = e[i].I;
    k.m[i].r = e[i].r;
    const size_t b = eig_lds_bytes(e[i].I, e[i].P);
    if (b > lds) lds = b;
  }
  const bool cplx = e[0].P == 2;
  auto fn = cplx ? k_eig<true> : k_eig_sym;
  if (lds > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)fn,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(fn, dim3(count), dim3(cplx ? NTH : NTS), lds, s, k);
  return hipGetLastError();
}

}  // namespace tg
