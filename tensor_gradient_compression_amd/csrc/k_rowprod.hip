// A mode product over the last mode, streamed by independent waves: the first launch of
// the one-mode-per-launch projection and the last (weight-updating) launch of its
// reconstruction, where the product's trailing part B is 1.
//
// Same product as k_modeprod.hip (pith.science "What carries the argument": projection
// to the core and reconstruction by mode-wise products; appendix M Theorem 2), with the
// sparse update added after the low-rank reconstruction (nullthought summary section 3)
// in the weight-updating form. With B = 1 the tensor is a matrix of A rows of K = I P
// contiguous values (complex data folded into its real (re, im) pairs, the operand in its
// real-block form), and the product is Y = X M^T: rows of K values in, rows of N = R P
// values out. No contraction index has a long contiguous run across rows, so the
// one-mode kernels' column tiles do not apply.
//
// Organisation. A tile is 16 consecutive rows; each wave takes tiles strided over all
// waves of the grid and holds M in registers (every lane's B operands for every k-step
// and 16-column block), so the only memory traffic is the stream of rows:
//  * Lane (li, lg) loads row 16 t + li, values VPL lg .. VPL lg + VPL - 1 of each group
//    of 4 VPL consecutive values (VPL = 4 fp32 or 8 16-bit values: one 16-byte load).
//    Value v of group q is the lane's A operand of k-step VPL q + v, whose four k
//    indices (one per lane group) are 4 VPL q + VPL lg + v: a fixed permutation of k
//    that the B operands (M) follow, so each load feeds VPL fp32 MFMAs
//    (v_mfma_f32_16x16x4_f32, fp32 accumulation; 16-bit values are exact in fp32).
//  * Values past the row's end (in the last group only) are masked to +0 with a per-lane
//    bit mask (they belong to the next row); rows past A read zero (out-of-range buffer
//    offsets) and are not written.
//  * The next tile's loads go into a second register set while this tile is
//    multiplied, as in k_streamprod.hip.
//  * Store form: lane (li, lg) holds rows 16 t + 4 lg + v, column 16 cb + li of Y.
//    Weight-updating form: W <- round(W * decay - lr * (Y + N_S at Omega)) per value,
//    Omega looked up by element through its bitmask and word ranks (a complex element's
//    two values share one bit), and the fp32 update optionally captured (a test hook);
//    the tile is re-read from LDS in runs of 8 consecutive values per lane.
#include "tg_common.h"

namespace tg {

namespace {

constexpr int RP_WPB = 4;   // waves per workgroup
constexpr int RP_NT = RP_WPB * 64;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

struct RPK {
  const void* X;        // (A, K) rows, input dtype
  float* Y;             // (A, N) fp32 (store form)
  void* W;              // (A, N) weights (weight-updating form)
  const float* M;       // N x K row-major fp32
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;      // N_S, P values per Omega entry
  float* delta;         // test capture of the fp32 update (NULL: off)
  float* gS;            // store form with the COO gather: S[j] = X[omega[j]] (fp32)
  uint64_t nwords;      // bitmask words
  uint64_t ntiles;      // ceil(A / 16)
  uint32_t A, K, N, P;
  float lr, decay;
  int has_sparse;
};

template <typename XT> struct RowIn;
template <> struct RowIn<float> {
  static constexpr int VPL = 4;
  __device__ static float val(const u32x4& w, int v) { return __uint_as_float(w[v]); }
};
template <> struct RowIn<_Float16> {
  static constexpr int VPL = 8;
  __device__ static float val(const u32x4& w, int v) {
    const uint32_t h = (w[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
};
template <> struct RowIn<bf16_t> {
  static constexpr int VPL = 8;
  __device__ static float val(const u32x4& w, int v) {
    const uint32_t h = (w[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
    return __uint_as_float(h << 16);
  }
};

// NQ: groups of 4 VPL values per row (K <= 4 VPL NQ); NCB: 16-column blocks of N
// (N <= 16 NCB); EPI 0: store Y; EPI 1: update W (type WT; complex weights as fp32
// pairs with P = 2). GATH (store form): X is the gradient itself; the COO gather
// S[j] = X[omega[j]] happens on the loaded rows, whose Omega values are then cleared
// before the product (X is only read): each lane prefetches, with its row groups, the
// bitmask and rank words of their elements.
template <typename XT, int NQ, int NCB, int EPI, typename WT, bool GATH>
__global__ void __launch_bounds__(RP_NT) k_rowprod(RPK k) {
  constexpr int VPL = RowIn<XT>::VPL;
  constexpr int NS = NQ * VPL;   // k-steps
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t K = k.K, N = k.N;

  // B operands: mb[s][cb] = M[16 cb + li][k(s, lg)], k(s, lg) = 4 VPL (s / VPL) + VPL lg +
  // s % VPL (zero past K or N)
  float mb[NS][NCB];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint32_t kk = 4 * VPL * (s / VPL) + VPL * lg + (s % VPL);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const uint32_t n = 16 * cb + li;
      const bool ok = kk < K && n < N;
      const float v = k.M[ok ? n * K + kk : 0];
      mb[s][cb] = ok ? v : 0.0f;
    }
  }
  // only the last group can hold values past the row's end (the same for every row):
  // a bit mask that keeps this lane's live values of it
  u32x4 keep;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t k0 = 4 * VPL * (NQ - 1) + VPL * lg;
    if constexpr (VPL == 4) {
      keep[j] = k0 + j < K ? 0xFFFFFFFFu : 0u;
    } else {
      keep[j] = (k0 + 2 * j < K ? 0x0000FFFFu : 0u) | (k0 + 2 * j + 1 < K ? 0xFFFF0000u : 0u);
    }
  }

  const uint64_t TW = (uint64_t)gridDim.x * RP_WPB;
  const uint64_t t0 = (uint64_t)blockIdx.x * RP_WPB + wv;
  if (t0 >= k.ntiles) return;
  const uint32_t es = (uint32_t)sizeof(XT);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)k.X, 0, (int)((uint64_t)k.A * K * es), 0x00020000);

  // Weight-updating form: the weight runs of tile t (run r of a lane: values 8 lane +
  // 512 r of the tile, NW 16-byte pieces) are loaded with the tile's rows, a tile ahead
  // of their use; runs past the tile or the tensor read zero and are not used.
  constexpr int NR = EPI ? (NCB + 1) / 2 : 1;
  constexpr int NW = EPI ? (int)(8 * sizeof(WT) / 16) : 1;
  const uint32_t esw = (uint32_t)sizeof(WT);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      EPI ? k.W : (void*)k.Y, 0, EPI ? (int)((uint64_t)k.A * N * esw) : 0, 0x00020000);
  auto tile_values = [&](uint64_t t) -> uint32_t {
    const uint64_t rows = k.A - 16 * t < 16 ? k.A - 16 * t : 16;
    return (uint32_t)rows * N;
  };
  auto wload = [&](uint64_t t, u32x4 (&w)[NR][NW]) {
    if constexpr (EPI) {
      const uint32_t nv = tile_values(t);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t f = 8 * lane + 512 * r;
        const uint32_t off = f < nv ? (uint32_t)((16 * t * N + f) * esw) : OOB;
#pragma unroll
        for (int q = 0; q < NW; ++q)
          w[r][q] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(off + 16 * q), 0, 0);
      }
    }
  };
  // row 16 t + li's groups into b (rows past A: out of range, zero)
  auto load = [&](uint64_t t, u32x4 (&b)[NQ]) {
    const uint64_t row = 16 * t + li;
    const uint32_t base = row < k.A ? (uint32_t)(row * K * es) + VPL * lg * es : OOB;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      b[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(base + 4 * VPL * q * es), 0, 0);
  };
  // GATH: the bitmask and rank words of group q's elements (its first element e0 and
  // the word after, which the group may reach into)
  constexpr int NG = GATH ? NQ : 1;
  struct GW {
    uint64_t m0[NG], m1[NG];
    uint32_t r0[NG], r1[NG];
  };
  const uint32_t P = k.P;
  auto gfirst = [&](uint64_t t, int q) -> uint64_t {
    const uint64_t row = 16 * t + li;
    const uint32_t k0 = 4 * VPL * q + VPL * lg;
    return row < k.A && k0 < K ? (row * K + k0) / P : 0;
  };
  auto gload = [&](uint64_t t, GW& g) {
    if constexpr (GATH) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint64_t w = gfirst(t, q) >> 6;
        const uint64_t w1 = w + 1 < k.nwords ? w + 1 : w;
        g.m0[q] = k.mask[w];
        g.m1[q] = k.mask[w1];
        g.r0[q] = k.rank[w];
        g.r1[q] = k.rank[w1];
      }
    }
  };
  // GATH: S[j] = X[omega[j]] for the Omega elements among b's values, which are then
  // cleared (+0 is the zero bit pattern of every input type)
  auto gather = [&](uint64_t t, u32x4 (&b)[NQ], const GW& g) {
    if constexpr (GATH) {
      constexpr uint32_t NEL = VPL;   // values of a group; elements: NEL / P
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint64_t row = 16 * t + li;
        const uint32_t k0 = 4 * VPL * q + VPL * lg;
        const uint32_t vlive = row < k.A && k0 < K ? (K - k0 < NEL ? K - k0 : NEL) : 0u;
        const uint32_t nel = vlive / P;   // live elements of the group
        const uint64_t e0 = gfirst(t, q);
        const uint32_t sh = (uint32_t)(e0 & 63);
        const uint64_t win = sh ? (g.m0[q] >> sh) | (g.m1[q] << (64 - sh)) : g.m0[q];
        const uint32_t bits = (uint32_t)win & ((1u << nel) - 1u);
        if (!bits) continue;
        u32x4 zm = {0u, 0u, 0u, 0u};
#pragma unroll
        for (uint32_t j = 0; j < NEL; ++j) {
          if (j >= nel || !((bits >> j) & 1u)) continue;
          const uint32_t lb = sh + j;
          const uint32_t r = lb < 64
                                 ? g.r0[q] + (uint32_t)__popcll(g.m0[q] & ((1ull << lb) - 1ull))
                                 : g.r1[q] +
                                       (uint32_t)__popcll(g.m1[q] & ((1ull << (lb - 64)) - 1ull));
          for (uint32_t p = 0; p < P; ++p) {
            const uint32_t v = j * P + p;
            k.gS[(uint64_t)r * P + p] = RowIn<XT>::val(b[q], (int)v);
            if constexpr (VPL == 4)
              zm[v] = 0xFFFFFFFFu;
            else
              zm[v >> 1] |= 0xFFFFu << (16 * (v & 1));
          }
        }
        b[q] = b[q] & ~zm;
      }
    }
  };
  // (values past the row's end belong to the next row: masked to +0 before use)
  auto multiply = [&](const u32x4 (&b)[NQ], f4 (&acc)[NCB]) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
    const u32x4 last = b[NQ - 1] & keep;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float a = RowIn<XT>::val(s / VPL == NQ - 1 ? last : b[s / VPL], s % VPL);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, mb[s][cb], acc[cb], 0, 0, 0);
    }
  };
  // Weight-updating form: the tile (16 rows of N values, one contiguous run of W) goes
  // through this wave's LDS region so that each lane then takes runs of 8 consecutive
  // values: one 16-byte weight load and store (16-bit weights), and one bitmask word for
  // the run's elements (a run starts at a multiple of 8 values, so its 8 / P elements
  // share a 64-element word).
  extern __shared__ float rp_smem[];
  LDS float* const tl = (LDS float*)rp_smem + wv * 16 * N;   // [16][N]
  auto finish = [&](uint64_t t, const f4 (&acc)[NCB], const u32x4 (&wr)[NR][NW]) {
    if constexpr (EPI == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint64_t row = 16 * t + 4 * lg + v;
        if (row >= k.A) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint32_t n = 16 * cb + li;
          if (n < N) k.Y[row * N + n] = acc[cb][v];
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint32_t n = 16 * cb + li;
          if (n < N) tl[(4 * lg + v) * N + n] = acc[cb][v];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t nv = tile_values(t);   // values of this tile
      const uint64_t o0 = 16 * t * N;       // the tile's first value in W
      WT* const W = (WT*)k.W;
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const uint32_t f = 8 * lane + 512 * rr;
        if (f >= nv) continue;
        float u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = f + j < nv ? tl[f + j] : 0.0f;
        const uint64_t o = o0 + f;
        const uint32_t nj = nv - f < 8 ? nv - f : 8;
        if (k.has_sparse) {
          const uint64_t e0 = o / k.P;            // the run's first element
          const uint32_t ne = (nj + k.P - 1) / k.P;
          const uint64_t word = k.mask[e0 >> 6];
          const uint32_t sh = (uint32_t)(e0 & 63);
          const uint32_t bits = (uint32_t)(word >> sh) & ((1u << ne) - 1u);
          if (bits) {
            const uint32_t base = omega_rank(k.mask, k.rank, e0, word);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t ej = (uint32_t)j / k.P;
              if ((uint32_t)j < nj && ((bits >> ej) & 1u)) {
                const uint32_t r = base + (uint32_t)__popc(bits & ((1u << ej) - 1u));
                u[j] = u[j] + k.uS[(uint64_t)r * k.P + ((uint32_t)j - ej * k.P)];
              }
            }
          }
        }
        if (nj == 8) {
          // 16 bytes (16-bit weights) or 32 bytes (fp32) at a 16-byte aligned offset
          u32x4 raw[NW];
#pragma unroll
          for (int q = 0; q < NW; ++q) raw[q] = wr[rr][q];
          WT w8[8];
          __builtin_memcpy(w8, raw, sizeof(w8));
#pragma unroll
          for (int j = 0; j < 8; ++j) w8[j] = from_f32<WT>(to_f32(w8[j]) * k.decay - k.lr * u[j]);
          __builtin_memcpy(raw, w8, sizeof(w8));
#pragma unroll
          for (int q = 0; q < NW; ++q) *((u32x4*)(W + o) + q) = raw[q];
        } else {
          for (uint32_t j = 0; j < nj; ++j)
            W[o + j] = from_f32<WT>(to_f32(W[o + j]) * k.decay - k.lr * u[j]);
        }
        if (k.delta)
          for (uint32_t j = 0; j < nj; ++j) k.delta[o + j] = u[j];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  f4 acc[NCB];
  u32x4 bA[NQ], bB[NQ];
  u32x4 wA[NR][NW], wB[NR][NW];
  GW gA, gB;
  load(t0, bA);
  wload(t0, wA);
  gload(t0, gA);
  const uint64_t t1 = t0 + TW < k.ntiles ? t0 + TW : t0;
  load(t1, bB);
  wload(t1, wB);
  gload(t1, gB);
  __builtin_amdgcn_sched_barrier(0);
  gather(t0, bA, gA);
  multiply(bA, acc);
  finish(t0, acc, wA);
  for (uint64_t t = t0 + TW; t < k.ntiles;) {
    const uint64_t tn = t + TW < k.ntiles ? t + TW : t;
    load(tn, bA);
    wload(tn, wA);
    gload(tn, gA);
    __builtin_amdgcn_sched_barrier(0);
    gather(t, bB, gB);
    multiply(bB, acc);
    finish(t, acc, wB);
    t += TW;
    if (t >= k.ntiles) break;
    const uint64_t tm = t + TW < k.ntiles ? t + TW : t;
    load(tm, bB);
    wload(tm, wB);
    gload(tm, gB);
    __builtin_amdgcn_sched_barrier(0);
    gather(t, bA, gA);
    multiply(bA, acc);
    finish(t, acc, wA);
    t += TW;
  }
}

struct PlanR {
  RPK k;
  int nq, ncb, vpl;
  bool ok;
};

PlanR plan_r(const ModeProd& mp) {
  PlanR p{};
  p.ok = false;
  if (mp.B != 1 || mp.A == 0 || mp.I == 0 || mp.R == 0) return p;
  if (mp.apply ? (mp.in_dt != DT_F32 || !mp.W) : !mp.Y) return p;
  if (mp.gather_S && (mp.apply || !mp.mask || !mp.rank)) return p;
  // weight runs of 8 values in 16-byte accesses: W 16-byte aligned, its bytes within
  // one buffer resource
  if (mp.apply && (uintptr_t)mp.W % 16 != 0) return p;
  if (mp.apply && (uint64_t)mp.A * mp.R * mp.P * (mp.w_dt == DT_F32 ? 4 : 2) >= 0x7FFFFFFFull)
    return p;
  const uint32_t P = mp.P;
  const uint64_t K = (uint64_t)mp.I * P, N = (uint64_t)mp.R * P;
  const int es = mp.in_dt == DT_F32 ? 4 : 2;
  p.vpl = es == 4 ? 4 : 8;
  // 16-byte loads at 4-byte aligned offsets: 16-bit rows of an even length
  if (es == 2 && K % 2 != 0) return p;
  if ((uintptr_t)mp.X % 4 != 0) return p;
  // buffer offsets within one resource: the whole input below 2^31 bytes
  if ((uint64_t)mp.A * K * es >= 0x7FFFFFFFull) return p;
  p.nq = (int)((K + 4 * p.vpl - 1) / (4 * p.vpl));
  p.ncb = (int)((N + 15) / 16);
  // M in registers: at most 64 values a lane
  if (p.nq > 5 || p.ncb > 5 || p.nq * p.vpl * p.ncb > 64) return p;
  RPK& k = p.k;
  k.X = mp.X;
  k.Y = mp.Y;
  k.W = mp.W;
  k.M = mp.M;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.uS = mp.uS;
  k.delta = mp.delta;
  k.gS = mp.gather_S;
  k.nwords = ((uint64_t)mp.A * mp.I + 63) / 64;
  k.A = mp.A;
  k.K = (uint32_t)K;
  k.N = (uint32_t)N;
  k.P = P;
  k.lr = mp.lr;
  k.decay = mp.decay;
  k.has_sparse = mp.has_sparse;
  k.ntiles = ((uint64_t)mp.A + 15) / 16;
  p.ok = true;
  return p;
}

template <typename XT, int NQ, int NCB, int EPI, typename WT>
hipError_t rp_launch(const PlanR& p, int num_cu, hipStream_t s) {
  if constexpr (NQ * RowIn<XT>::VPL * NCB > 64) {
    return hipErrorInvalidValue;
  } else {
    void (*fn)(RPK) = k_rowprod<XT, NQ, NCB, EPI, WT, false>;
    if constexpr (EPI == 0)
      if (p.k.gS) fn = k_rowprod<XT, NQ, NCB, EPI, WT, true>;
    const size_t lds = EPI ? (size_t)RP_WPB * 16 * p.k.N * 4 : 0;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, RP_NT, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidValue;
    uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * (uint64_t)per_cu;
    const uint64_t need = (p.k.ntiles + RP_WPB - 1) / RP_WPB;
    if (grid > need) grid = need;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(RP_NT), lds, s, p.k);
    return hipGetLastError();
  }
}
template <typename XT, int NQ, int EPI, typename WT>
hipError_t rp_ncb(const PlanR& p, int num_cu, hipStream_t s) {
  switch (p.ncb) {
    case 1: return rp_launch<XT, NQ, 1, EPI, WT>(p, num_cu, s);
    case 2: return rp_launch<XT, NQ, 2, EPI, WT>(p, num_cu, s);
    case 3: return rp_launch<XT, NQ, 3, EPI, WT>(p, num_cu, s);
    case 4: return rp_launch<XT, NQ, 4, EPI, WT>(p, num_cu, s);
    default: return rp_launch<XT, NQ, 5, EPI, WT>(p, num_cu, s);
  }
}
template <typename XT, int EPI, typename WT>
hipError_t rp_nq(const PlanR& p, int num_cu, hipStream_t s) {
  switch (p.nq) {
    case 1: return rp_ncb<XT, 1, EPI, WT>(p, num_cu, s);
    case 2: return rp_ncb<XT, 2, EPI, WT>(p, num_cu, s);
    case 3: return rp_ncb<XT, 3, EPI, WT>(p, num_cu, s);
    case 4: return rp_ncb<XT, 4, EPI, WT>(p, num_cu, s);
    default: return rp_ncb<XT, 5, EPI, WT>(p, num_cu, s);
  }
}

}  // namespace

bool rowprod_supported(const ModeProd& mp) { return plan_r(mp).ok; }

hipError_t launch_rowprod(const ModeProd& mp, int num_cu, hipStream_t s) {
  const PlanR p = plan_r(mp);
  if (!p.ok) return hipErrorInvalidValue;
  if (!mp.apply) {
    switch (mp.in_dt) {
      case DT_F32: return rp_nq<float, 0, float>(p, num_cu, s);
      case DT_F16: return rp_nq<_Float16, 0, float>(p, num_cu, s);
      case DT_BF16: return rp_nq<bf16_t, 0, float>(p, num_cu, s);
    }
    return hipErrorInvalidValue;
  }
  switch (mp.w_dt) {
    case DT_F32: return rp_nq<float, 1, float>(p, num_cu, s);
    case DT_F16: return rp_nq<float, 1, _Float16>(p, num_cu, s);
    case DT_BF16: return rp_nq<float, 1, bf16_t>(p, num_cu, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
