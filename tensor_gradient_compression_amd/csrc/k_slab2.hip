// Two trailing mode products of a 16-bit tensor, one wave per slab, on MFMAs.
//
// Same mathematics as the two-mode kernel in k_modeprod2.hip (pith.science "What
// carries the argument": projection to the core and reconstruction by mode-wise
// products; appendix M Theorem 2), with the COO gather folded into the projection and
// the sparse merge plus weight update folded into the reconstruction (nullthought
// summary section 3). The tensor is A slabs of the last two modes, (A, I1, I2).
//   projection:     Y[i1, r2] = sum_i2 X[i1, i2] M2[r2, i2]     (mode d)
//                   Z[j1, r2] = sum_i1 M1[j1, i1] Y[i1, r2]     (mode d-1)
//   reconstruction: Y[i1, j2] = sum_j1 M1[i1, j1] Z[j1, j2]     (mode d-1)
//                   O[i1, i2] = sum_j2 Y[i1, j2] M2[i2, j2]     (mode d)
//                   W <- round(W * decay - lr * (O + N_S at Omega))
//
// Organisation. Wave w of a grid of TW waves takes slabs w, w + TW, w + 2 TW, ... (the
// grid moves through the tensor as one window) and owns a private slice of LDS; no
// workgroup barrier is used. While a wave computes a slab, the DMA engine brings the
// input of its next slab (global_load_lds, 16-byte pieces; the reconstruction also
// brings the weights of the current slab), and the Omega indices (and N_S) of the next
// slab and the bitmask words that bound the slab after it arrive in registers. A slab's
// output leaves at the start of the wave's next slab, before that slab's transfers are
// issued, and is waited for only after that slab has been computed. A wave's LDS
// operations execute in issue order, so data passed between its lanes through LDS
// needs no barrier.
//
// Arithmetic. The projection's first product (mode d) runs on v_mfma_f32_16x16x32_bf16:
// the factor matrix is split into three bf16 parts, x = x0 + x1 + x2 with
// |x - x0 - x1 - x2| <= 2^-27 |x| (bf16 keeps fp32's exponent range, so each part takes
// the next 8 significand bits); bf16 data are exact as they are and fp16 data split
// exactly into two bf16 parts. Every part product is exact in fp32; those whose parts'
// orders sum above 2 (each below 2^-24 of the full product) are dropped, so the result
// agrees with an fp32 GEMM to the level of fp32 rounding. Every other product takes fp32
// operands as they are, on v_mfma_f32_16x16x4_f32. Accumulation is fp32 throughout.
#include <type_traits>

#include "tg_common.h"
#include "k_slab_common.h"

namespace tg {

namespace {

constexpr int WPB = 4;            // waves per workgroup
constexpr int NT = WPB * 64;


struct S2K {
  const void* X;        // projection: the gradient (A, I1, I2), only read
  const float* Zin;     // reconstruction: fp32 input (A, R1, R2)
  void* W;              // reconstruction: weights (A, I1, I2)
  float* Y;             // projection: fp32 output (A, R1, R2)
  const float* M1;      // projection: R1 x I1; reconstruction: I1 x R1 (row-major fp32)
  const float* M2;      // projection: R2 x I2; reconstruction: I2 x R2
  const uint64_t* mask;
  const uint32_t* rank;
  const uint32_t* omega;
  float* S;             // projection: gathered S (written); reconstruction: N_S (read)
  float* delta;         // reconstruction with CAP: the fp32 update O is stored here too
  uint64_t kS;          // |Omega|; 0: no sparse part
  uint32_t A, I1, I2, R1, R2;
  uint32_t slab_e;      // I1 * I2
  uint32_t lds_wave;       // LDS bytes per wave
  uint32_t off_b1, off_y, off_o;   // per-wave byte offsets (second input buffer, Y, output)
  uint32_t off_w0;      // reconstruction: the W buffer
  uint32_t ly;          // row stride (floats) of the fp32 intermediate in LDS
  uint32_t ydelta;      // reconstruction: float offset of Y inside the output region
  uint32_t trash;       // float offset (in the output region) of 64 per-lane slots that
                        // take the writes of padding lanes, so no write needs a branch
  float lr, decay;
};

__device__ __forceinline__ unsigned short bf_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
__device__ __forceinline__ float bf_val(unsigned short b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ void split3(float x, unsigned short& a, unsigned short& b,
                                       unsigned short& c) {
  a = bf_bits(x);
  const float r = x - bf_val(a);
  b = bf_bits(r);
  c = bf_bits(r - bf_val(b));
}
__device__ __forceinline__ void split2(float x, unsigned short& a, unsigned short& b) {
  a = bf_bits(x);
  b = bf_bits(x - bf_val(a));
}
__device__ __forceinline__ f4 mma(const u16x8& a, const u16x8& b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// (a0 + a1)(b0 + b1 + b2) for exact two-part data: the five with i + j <= 2
__device__ __forceinline__ f4 mma_2x3(const u16x8& a0, const u16x8& a1, const u16x8* b, f4 c) {
  c = mma(a0, b[2], c);
  c = mma(a1, b[1], c);
  c = mma(a0, b[1], c);
  c = mma(a1, b[0], c);
  return mma(a0, b[0], c);
}
// Eight consecutive 16-bit values at a 2-byte aligned LDS address, as four packed dwords:
// five aligned dword reads and a funnel shift by 0 or 16 bits (eight 16-bit reads
// otherwise). The last read may reach up to 18 bytes past the run; callers keep that
// inside their LDS and mask what lies outside the row.
__device__ __forceinline__ u32x4 lds_run8(const LDS unsigned char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)p;
  const LDS uint32_t* const d = (const LDS uint32_t*)(p - (a & 2u));
  const uint32_t sh = (a & 2u) * 8;
  uint32_t w[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) w[i] = d[i];
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
  return r;
}
// Per-lane mask keeping values 8 lg + 2 i (+1) < n of a run, packed as lds_run8 gives them.
__device__ __forceinline__ u32x4 run_keep(uint32_t lg, uint32_t n) {
  u32x4 m;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = 8 * lg + 2 * i;
    m[i] = (x < n ? 0x0000FFFFu : 0u) | (x + 1 < n ? 0xFFFF0000u : 0u);
  }
  return m;
}


// Wave w takes slabs w, w + TW, w + 2 TW, ... (TW = waves in the grid), so the whole
// grid streams through one moving window of the tensor.
__device__ __forceinline__ uint32_t total_waves() { return gridDim.x * (uint32_t)WPB; }


// 16-bit storage types seen as their bit patterns (LDS holds raw 16-bit words)
template <typename T> struct Bits16;
template <> struct Bits16<bf16_t> {
  // x as bf16 parts: exact in one
  static constexpr int NP = 1;
  __device__ static void parts(unsigned short raw, unsigned short* p) { p[0] = raw; }
  __device__ static float value(unsigned short raw) { return bf_val(raw); }
};
template <> struct Bits16<_Float16> {
  static constexpr int NP = 2;
  __device__ static void parts(unsigned short raw, unsigned short* p) {
    const float x = (float)__builtin_bit_cast(_Float16, raw);
    split2(x, p[0], p[1]);   // 11 significand bits: exact in two bf16 parts
  }
  __device__ static float value(unsigned short raw) {
    return (float)__builtin_bit_cast(_Float16, raw);
  }
};


// ------------------------------------------------------------------ projection
// NRB1: 16-row blocks of I1 (I1 <= 16 NRB1 <= 64); NRB2: 16-row blocks of R1 (<= 32).
// I2 <= 32 and R2 <= 16 (one k chunk and one column block in pass 1).
// Pass 1 (mode d) runs on bf16 MFMAs: X exact (bf16) or in two exact parts (fp16),
// M2 in three parts. Pass 2 (mode d-1) runs on v_mfma_f32_16x16x4_f32 directly on the
// fp32 intermediate: its k index i1 = 4 NRB1 * (lane / 16) + step, so every lane reads
// its part of a column of Y as consecutive 16-byte pieces.
template <typename XT, int NRB1, int NRB2>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 8))) k_proj2s(S2K k) {
  constexpr int KS2 = 4 * NRB1;   // fp32 MFMA k-steps of pass 2
  extern __shared__ float smem[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t gw = blockIdx.x * WPB + wv;
  if (gw >= k.A) return;
  const uint32_t TW = total_waves();
  const uint32_t cnt = (k.A - 1 - gw) / TW + 1;   // slabs of this wave
  LDS unsigned char* const base = (LDS unsigned char*)smem + wv * k.lds_wave;
  LDS unsigned char* const xb0 = base;
  LDS unsigned char* const xb1 = base + k.off_b1;
  LDS float* const Y1 = (LDS float*)(base + k.off_y);   // [r2 < 16][i1 < 16 NRB1], stride ly
  LDS float* const So = (LDS float*)(base + k.off_o);   // [R1][R2]
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I1 = k.I1, I2 = k.I2, R1 = k.R1, R2 = k.R2, LY = k.ly;
  const uint32_t slab_e = k.slab_e;
  const uint64_t N = (uint64_t)k.A * slab_e;
  const uint64_t kS = k.kS;
  const bool sparse = kS > 0;
  const u32x4 keep1 = run_keep(lg, I2);   // pass 1: i2 = 8 lg + e < I2

  // pass 1 B[k = i2][col = r2] = M2[r2][i2] in three bf16 parts
  u16x8 b1[3];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t i2 = 8 * lg + e;
    const float v = (li < R2 && i2 < I2) ? k.M2[li * I2 + i2] : 0.0f;
    unsigned short a, b, c;
    split3(v, a, b, c);
    b1[0][e] = a; b1[1][e] = b; b1[2][e] = c;
  }
  // pass 2 A[row = j1][k = i1] = M1[j1][i1], i1 = KS2 * lg + step
  float a2[NRB2][KS2];
#pragma unroll
  for (int rb = 0; rb < NRB2; ++rb)
#pragma unroll
    for (int t = 0; t < KS2; ++t) {
      const uint32_t j1 = 16 * rb + li, i1 = KS2 * lg + t;
      a2[rb][t] = (j1 < R1 && i1 < I1) ? k.M1[j1 * I1 + i1] : 0.0f;
    }

  const XT* X = (const XT*)k.X;
  const uint32_t xchunks = slab_e * 2 / 16;
  // bitmask words and ranks at the start and the end of slab s, and its Omega range
  auto bounds = [&](uint32_t s, BoundsV& b) {
    b = load_bounds(k.mask, k.rank, (uint64_t)s * slab_e, slab_e, N, lane);
  };
  auto range = [&](uint32_t s, const BoundsV& b, uint64_t& lo, uint64_t& hi) {
    lo = rank_at(lane_u64(b.m, 0), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 0),
                 (uint64_t)s * slab_e, N, kS);
    hi = rank_at(lane_u64(b.m, 1), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 1),
                 (uint64_t)(s + 1) * slab_e, N, kS);
  };
  OmegaPipe op;
  if (sparse) {
    BoundsV w;
    bounds(gw, w);
    wait_vm0();
    range(gw, w, op.lo[0], op.hi[0]);
#pragma unroll
    for (int i = 0; i < NOM; ++i) {
      const uint64_t j = op.lo[0] + lane + 64 * i;
      op.om[0][i] = k.omega[j < kS ? j : kS - 1];
    }
    if (cnt > 1) bounds(gw + TW, op.bw);
  }
  wave_dma(X + (uint64_t)gw * slab_e, xchunks, xb0, lane);

  uint32_t nq_prev = 0;
  uint64_t out_prev = 0;
  // slab i of this wave, in slot `cur` (= i % 2)
  auto slab = [&](uint32_t i, auto slot) {
    constexpr int cur = decltype(slot)::value, nxt = cur ^ 1;
    const uint32_t n = gw + i * TW;   // this slab
    wait_vm0();   // slab n, its Omega indices and the next slab's bounds have landed
    wave_fence();
    if (sparse && i + 1 < cnt) range(n + TW, op.bw, op.lo[nxt], op.hi[nxt]);
    // the previous slab's output leaves (waited for at the next slab)
    for (uint32_t q = lane; q < nq_prev; q += 64)
      *(f4*)(k.Y + out_prev + 4 * q) = *(const LDS f4*)(So + 4 * q);
    wait_lgkm0();
    wave_fence();
    // next slab's transfer, Omega indices and range bound
    if (i + 1 < cnt) {
      wave_dma(X + (uint64_t)(n + TW) * slab_e, xchunks, cur ? xb0 : xb1, lane);
      if (sparse) {
#pragma unroll
        for (int q = 0; q < NOM; ++q) {
          const uint64_t j = op.lo[nxt] + lane + 64 * q;
          op.om[nxt][q] = k.omega[j < kS ? j : kS - 1];
        }
        if (i + 2 < cnt) bounds(n + 2 * TW, op.bw);
      }
    }

    LDS unsigned short* const xs = (LDS unsigned short*)(cur ? xb1 : xb0);
    const uint64_t e_lo = (uint64_t)n * slab_e;
    if (sparse) {
      // S[j] = X[omega[j]] and X[omega[j]] <- 0 in the LDS copy (+0 is the zero bit
      // pattern of both 16-bit formats); the gradient in HBM is only read
      auto take = [&](uint64_t j, uint32_t om) {
        const uint32_t loc = (uint32_t)(om - e_lo);
        k.S[j] = Bits16<XT>::value(xs[loc]);
        xs[loc] = 0;
      };
      // the prefetched entries: every value read before any is cleared
      const uint64_t jlo = op.lo[cur], jhi = op.hi[cur];
      float sv[NOM];
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = jlo + lane + 64 * q;
        sv[q] = j < jhi ? Bits16<XT>::value(xs[(uint32_t)(op.om[cur][q] - e_lo)]) : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = jlo + lane + 64 * q;
        if (j < jhi) {
          k.S[j] = sv[q];
          xs[(uint32_t)(op.om[cur][q] - e_lo)] = 0;
        }
      }
      for (uint64_t j = jlo + 64 * NOM + lane; j < jhi; j += 64) take(j, k.omega[j]);
      wave_fence();
    }

    // pass 1 (mode d): rows i1, k = i2, columns r2
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) {
      const uint32_t i1 = 16 * rb + li;
      u16x8 xp[Bits16<XT>::NP];
      if constexpr (Bits16<XT>::NP == 1) {
        // row i1 (rows past I1 read row I1 - 1 and are masked to zero), i2 = 8 lg + e
        const u32x4 w = lds_run8((const LDS unsigned char*)xs + (min(i1, I1 - 1) * I2 + 8 * lg) * 2);
        xp[0] = __builtin_bit_cast(u16x8, w & (i1 < I1 ? keep1 : u32x4{0u, 0u, 0u, 0u}));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t i2 = 8 * lg + e;
          const unsigned short raw =
              (i1 < I1 && i2 < I2) ? xs[i1 * I2 + i2]
                                   : (unsigned short)0;
          unsigned short p[2];
          Bits16<XT>::parts(raw, p);
#pragma unroll
          for (int h = 0; h < Bits16<XT>::NP; ++h) xp[h][e] = p[h];
        }
      }
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (Bits16<XT>::NP == 1) {
        acc = mma(xp[0], b1[2], acc);
        acc = mma(xp[0], b1[1], acc);
        acc = mma(xp[0], b1[0], acc);
      } else {
        acc = mma_2x3(xp[0], xp[1], b1, acc);
      }
      *(LDS f4*)(Y1 + li * LY + 16 * rb + 4 * lg) = acc;
    }
    wave_fence();
    // pass 2 (mode d-1): rows j1, k = i1, columns r2
    f4 acc2[NRB2];
#pragma unroll
    for (int rb = 0; rb < NRB2; ++rb) acc2[rb] = f4{0.f, 0.f, 0.f, 0.f};
    const LDS float* yc = Y1 + li * LY + KS2 * lg;
#pragma unroll
    for (int q = 0; q < KS2 / 4; ++q) {
      const f4 y = *(const LDS f4*)(yc + 4 * q);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int rb = 0; rb < NRB2; ++rb)
          acc2[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2[rb][4 * q + t], y[t], acc2[rb], 0, 0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < NRB2; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t j1 = 16 * rb + 4 * lg + v;
        So[(j1 < R1 && li < R2) ? j1 * R2 + li : k.trash + lane] = acc2[rb][v];
      }
    wave_fence();
    nq_prev = R1 * R2 / 4;
    out_prev = (uint64_t)n * R1 * R2;
  };
  for (uint32_t i = 0; i < cnt; i += 2) {
    slab(i, Slot<0>{});
    if (i + 1 < cnt) slab(i + 1, Slot<1>{});
  }
  // the last slab's output
  wait_lgkm0();
  for (uint32_t q = lane; q < nq_prev; q += 64)
    *(f4*)(k.Y + out_prev + 4 * q) = *(const LDS f4*)(So + 4 * q);
}

// ------------------------------------------------------------------ reconstruction
// NRB1: 16-row blocks of I1 (<= 64); NCB2: 16-column blocks of I2 (<= 32); KS1: fp32
// MFMA k-steps of pass 1 (R1 <= 4 KS1 <= 32); R2 <= 16. Both products run on
// v_mfma_f32_16x16x4_f32 straight from fp32 data: pass 1 (mode d-1) with k index
// j1 = KS1 (lane / 16) + step, pass 2 (mode d) with j2 = 4 (lane / 16) + step; the factor
// operands stay in registers, and pass 1's row blocks are independent accumulation
// chains interleaved step by step. CAP (a test instantiation) also stores the fp32
// update O (after the sparse merge, before the weight rounding) to k.delta.
template <typename WT, int NRB1, int NCB2, int KS1, bool CAP>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) k_rec2s(S2K k) {
  extern __shared__ float smem[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t gw = blockIdx.x * WPB + wv;
  if (gw >= k.A) return;
  const uint32_t TW = total_waves();
  const uint32_t cnt = (k.A - 1 - gw) / TW + 1;   // slabs of this wave
  LDS unsigned char* const base = (LDS unsigned char*)smem + wv * k.lds_wave;
  LDS unsigned char* const zb0 = base;
  LDS unsigned char* const zb1 = base + k.off_b1;
  LDS unsigned char* const wb = base + k.off_w0;
  LDS float* const Ob = (LDS float*)(base + k.off_o);   // [I1][I2]; Y [i1][ly] at Ob + ydelta
  LDS float* const Yb = Ob + k.ydelta;
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I1 = k.I1, I2 = k.I2, R1 = k.R1, R2 = k.R2, LY = k.ly;
  const uint32_t slab_e = k.slab_e, slab_z = R1 * R2;
  const uint64_t N = (uint64_t)k.A * slab_e;
  const uint64_t kS = k.kS;
  const bool sparse = kS > 0;
  const float lr = k.lr, decay = k.decay;
  const bool decayed = decay != 1.0f;

  // pass 1 A[row = i1][k = j1] = M1[i1][j1], j1 = KS1 lg + step
  float a1[NRB1][KS1];
#pragma unroll
  for (int rb = 0; rb < NRB1; ++rb)
#pragma unroll
    for (int t = 0; t < KS1; ++t) {
      const uint32_t i1 = 16 * rb + li, j1 = KS1 * lg + t;
      a1[rb][t] = (i1 < I1 && j1 < R1) ? k.M1[i1 * R1 + j1] : 0.0f;
    }
  // pass 2 B[k = j2][col = i2] = M2[i2][j2], j2 = 4 lg + step
  float b2[NCB2][4];
#pragma unroll
  for (int cb = 0; cb < NCB2; ++cb)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t i2 = 16 * cb + li, j2 = 4 * lg + t;
      b2[cb][t] = (i2 < I2 && j2 < R2) ? k.M2[i2 * R2 + j2] : 0.0f;
    }

  const WT* Wg = (const WT*)k.W;
  const uint32_t zchunks = slab_z * 4 / 16, wchunks = slab_e * 2 / 16;
  // bitmask words and ranks at the start and the end of slab s, and its Omega range
  // (scalar loads here: this kernel has no register room for the vector form, and none
  // of its LDS waits falls between a fetch and its use a slab later)
  auto bounds = [&](uint32_t s, uint64_t* w) {
    const uint64_t elo = (uint64_t)s * slab_e, ehi = elo + slab_e;
    const uint64_t wl = elo >> 6, wh = ehi < N ? ehi >> 6 : 0;
    const __attribute__((address_space(4))) uint64_t* m =
        (const __attribute__((address_space(4))) uint64_t*)k.mask;
    const __attribute__((address_space(4))) uint32_t* r =
        (const __attribute__((address_space(4))) uint32_t*)k.rank;
    w[0] = m[wl];
    w[1] = r[wl];
    w[2] = m[wh];
    w[3] = r[wh];
  };
  auto range = [&](uint32_t s, const uint64_t* w, uint64_t& lo, uint64_t& hi) {
    lo = rank_at(w[0], (uint32_t)w[1], (uint64_t)s * slab_e, N, kS);
    hi = rank_at(w[2], (uint32_t)w[3], (uint64_t)(s + 1) * slab_e, N, kS);
  };
  uint64_t bws[4] = {0, 0, 0, 0};   // the slab after: mask, rank at its start; at its end
  OmegaPipe op;
  if (sparse) {
    uint64_t w[4];
    bounds(gw, w);
    range(gw, w, op.lo[0], op.hi[0]);
#pragma unroll
    for (int i = 0; i < NOM; ++i) {
      const uint64_t j = op.lo[0] + lane + 64 * i;
      const uint64_t jc = j < kS ? j : kS - 1;
      op.om[0][i] = k.omega[jc];
      op.us[0][i] = k.S[jc];
    }
    if (cnt > 1) bounds(gw + TW, bws);
  }
  wave_dma(k.Zin + (uint64_t)gw * slab_z, zchunks, zb0, lane);

  uint32_t nq_prev = 0;
  uint64_t out_prev = 0;
  // slab i of this wave (i < cnt) after the previous slab's weights have been written;
  // i == cnt writes the last slab's weights and returns true. Omega data of this slab in
  // slot 0, of the next in slot 1 (moved to slot 0 after the slab: unrolling this loop to
  // alternate the slots would cost the registers that keep it at four waves per SIMD).
  auto slab = [&](uint32_t i) -> bool {
    constexpr int cur = 0, nxt = 1;
    const int par = i & 1;            // LDS buffer of this slab's Z
    const uint32_t n = gw + i * TW;   // this slab (i < cnt)
    wait_vm0();   // Z of this slab, W of the previous one, Omega data; older stores
    wave_fence();
    if (sparse && i + 1 < cnt) range(n + TW, bws, op.lo[nxt], op.hi[nxt]);
    // the previous slab: W <- round(W * decay - lr * O), 16-byte pieces (the stores are
    // waited for at the next slab)
    for (uint32_t q = lane; q < nq_prev; q += 64) {
      const f4 o0 = *(const LDS f4*)(Ob + 8 * q);
      const f4 o1 = *(const LDS f4*)(Ob + 8 * q + 4);
      typedef unsigned int u4v __attribute__((ext_vector_type(4)));
      const u4v wraw = *(const LDS u4v*)(wb + 16 * q);
      const WT* ws = (const WT*)&wraw;
      WT o[8];
      if (decayed) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = from_f32<WT>(to_f32(ws[e]) * decay - lr * o0[e]);
          o[4 + e] = from_f32<WT>(to_f32(ws[4 + e]) * decay - lr * o1[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = from_f32<WT>(to_f32(ws[e]) - lr * o0[e]);
          o[4 + e] = from_f32<WT>(to_f32(ws[4 + e]) - lr * o1[e]);
        }
      }
      *(uint4*)((WT*)k.W + out_prev + 8 * q) = *(const uint4*)o;
      if constexpr (CAP) {
        *(f4*)(k.delta + out_prev + 8 * q) = o0;
        *(f4*)(k.delta + out_prev + 8 * q + 4) = o1;
      }
    }
    if (i == cnt) return true;
    wait_lgkm0();
    wave_fence();
    // this slab's W (used at the next slab), the next slab's Z and Omega data
    wave_dma(Wg + (uint64_t)n * slab_e, wchunks, wb, lane);
    if (i + 1 < cnt) {
      wave_dma(k.Zin + (uint64_t)(n + TW) * slab_z, zchunks, par ? zb0 : zb1, lane);
      if (sparse) {
#pragma unroll
        for (int q = 0; q < NOM; ++q) {
          const uint64_t j = op.lo[nxt] + lane + 64 * q;
          const uint64_t jc = j < kS ? j : kS - 1;
          op.om[nxt][q] = k.omega[jc];
          op.us[nxt][q] = k.S[jc];
        }
        if (i + 2 < cnt) bounds(n + 2 * TW, bws);
      }
    }

    const LDS float* const zs = (const LDS float*)(par ? zb1 : zb0);
    // pass 1 (mode d-1): rows i1, k = j1, columns j2
    float zv[KS1];
#pragma unroll
    for (int t = 0; t < KS1; ++t) {
      const uint32_t j1 = KS1 * lg + t;
      zv[t] = (j1 < R1 && li < R2) ? zs[j1 * R2 + li] : 0.0f;
    }
    f4 acc1[NRB1];
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) acc1[rb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KS1; ++t)
#pragma unroll
      for (int rb = 0; rb < NRB1; ++rb)
        acc1[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[rb][t], zv[t], acc1[rb], 0, 0, 0);
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) Yb[(16 * rb + 4 * lg + v) * LY + li] = acc1[rb][v];
    wave_fence();
    // pass 2 (mode d): rows i1, k = j2, columns i2; Y's block rb is read before O's
    // block rb is written over it (their placement keeps block rb + 1 intact)
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) {
      const f4 y = *(const LDS f4*)(Yb + (16 * rb + li) * LY + 4 * lg);
      f4 acc[NCB2];
#pragma unroll
      for (int cb = 0; cb < NCB2; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int cb = 0; cb < NCB2; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(y[t], b2[cb][t], acc[cb], 0, 0, 0);
      wave_fence();
#pragma unroll
      for (int cb = 0; cb < NCB2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t i1 = 16 * rb + 4 * lg + v, i2 = 16 * cb + li;
          Ob[(i1 < I1 && i2 < I2) ? i1 * I2 + i2 : k.trash + lane] = acc[cb][v];
        }
    }
    wave_fence();
    if (sparse) {
      const uint64_t e_lo = (uint64_t)n * slab_e;
      // the prefetched entries: all reads, then all writes (distinct elements; lanes
      // past the range use their trash slot)
      const uint64_t jlo = op.lo[cur], jhi = op.hi[cur];
      uint32_t loc[NOM];
      float cv[NOM];
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = jlo + lane + 64 * q;
        loc[q] = j < jhi ? (uint32_t)(op.om[cur][q] - e_lo) : k.trash + lane;
      }
#pragma unroll
      for (int q = 0; q < NOM; ++q) cv[q] = Ob[loc[q]];
#pragma unroll
      for (int q = 0; q < NOM; ++q) Ob[loc[q]] = cv[q] + op.us[cur][q];
      for (uint64_t j = jlo + 64 * NOM + lane; j < jhi; j += 64) {
        const uint32_t loc = (uint32_t)(k.omega[j] - e_lo);
        Ob[loc] = Ob[loc] + k.S[j];
      }
      wave_fence();
    }
    nq_prev = slab_e / 8;
    out_prev = (uint64_t)n * slab_e;
    return false;
  };
  for (uint32_t i = 0;; ++i) {
    if (slab(i)) break;
    op.lo[0] = op.lo[1];
    op.hi[0] = op.hi[1];
#pragma unroll
    for (int q = 0; q < NOM; ++q) {
      op.om[0][q] = op.om[1][q];
      op.us[0][q] = op.us[1][q];
    }
  }
}

// ------------------------------------------------------------------ three-mode projection
// The last three modes in one launch. A unit is one index of the leading modes: I0 slabs
// of I1 x I2 (contiguous). A workgroup of WPB3 waves takes one unit at a time (units
// strided over the grid) in rounds of WPB3 slabs: in round c wave w projects slab
// WPB3 c + w over modes d and d-1 exactly as the two-mode kernel does (Omega gathered and
// zeroed in its staged copy) and leaves the R1 x R2 result as row w of a round stack in
// LDS; after one barrier every wave adds the round's share of the mode d-2 product,
// Y[u] (R0 x R1 R2) += M0[:, round] x stack, to the output tiles it owns (fp32
// accumulators on v_mfma_f32_16x16x4_f32), and writes them after the unit's last round.
// Two round stacks alternate with the workgroup's round count (across units too), so one
// barrier per round suffices. Pass 1's accumulators
// feed pass 2 directly: the 16x16 MFMA result layout (rows 4 (lane / 16) + v, column
// lane % 16) is pass 2's B-operand layout when its k index runs over rows in the order
// (block, v, lane / 16).
constexpr int WPB3 = 16;
constexpr int NT3 = WPB3 * 64;

struct S3K {
  const void* X;        // the gradient (U, I0, I1, I2), only read
  float* Y;             // fp32 output (U, R0, R1, R2)
  const float* M0;      // R0 x I0 (row-major fp32)
  const float* M1;      // R1 x I1
  const float* M2;      // R2 x I2
  const uint64_t* mask;
  const uint32_t* rank;
  const uint32_t* omega;
  float* S;             // gathered S (written)
  uint64_t kS;          // |Omega|; 0: no sparse part
  uint32_t U, I0, I1, I2, R0, R1, R2;
  uint32_t slab_e;      // I1 * I2
  uint32_t lds_wave;    // bytes per wave (two slab buffers)
  uint32_t off_x1;      // second buffer, within a wave's bytes
  uint32_t off_stack;   // two round stacks of WPB3 rows of R1 R2 floats + 64 trash slots
  uint32_t stack_fl;    // floats per round stack
  uint32_t off_m0;      // M0 copy
  uint32_t off_fac;     // per-lane operand tables of passes 1 and 2 (see k_proj3s)
};

// NTW: output tiles (16 x 16) per wave, at most; ND: loads a slab transfer issues
// ((slab bytes / 16 + 63) / 64)
template <typename XT, int NRB1, int NRB2, int NTW, int ND>
__global__ void __launch_bounds__(NT3) __attribute__((amdgpu_waves_per_eu(4, 8))) k_proj3s(S3K k) {
  extern __shared__ float smem[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LDS unsigned char* const lds = (LDS unsigned char*)smem;
  LDS unsigned char* const xb0 = lds + wv * k.lds_wave;
  LDS unsigned char* const xb1 = xb0 + k.off_x1;
  LDS float* const stacks = (LDS float*)(lds + k.off_stack);
  LDS float* const m0s = (LDS float*)(lds + k.off_m0);
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I0 = k.I0, I1 = k.I1, I2 = k.I2, R0 = k.R0, R1 = k.R1, R2 = k.R2;
  const u32x4 keep1 = run_keep(lg, I2);   // pass 1: i2 = 8 lg + e < I2
  const uint32_t RC = R1 * R2;                 // stack row length
  const uint32_t trash = WPB3 * RC;            // float offset of a stack's trash slots
  const uint32_t SF = k.stack_fl;
  const uint32_t slab_e = k.slab_e;
  const uint64_t N = (uint64_t)k.U * I0 * slab_e;
  const uint64_t kS = k.kS;
  const bool sparse = kS > 0;
  // mode d-2 output tiles of this wave: row block jb = wv / (WPB3 / 2), column blocks
  // ct0 + (WPB3 / 2) m, ct0 = wv % (WPB3 / 2)
  const uint32_t nct = (RC + 15) / 16, njb = (R0 + 15) / 16;
  const uint32_t jb = wv / (WPB3 / 2), ct0 = wv % (WPB3 / 2);
  const uint32_t j0 = 16 * jb + li;
  const uint32_t jc = jb < njb && j0 < R0 ? j0 : R0 - 1;   // M0 row this lane reads

  // The factor operands, as every lane supplies them, in LDS tables shared by the
  // workgroup (registers would not leave room for the mode d-2 accumulators):
  //   b1t[part][lane]: pass 1 B[k = i2][col = r2] = M2[r2][i2], i2 = 8 (lane / 16) + e,
  //                    r2 = lane % 16, in three bf16 parts (16 bytes a lane);
  //   a2t[r2][rb][lane]: pass 2 A[row = j1][k] = M1[j1][i1], j1 = 16 r2 + lane % 16,
  //                    i1 = 16 rb + 4 (lane / 16) + v for v = 0..3 (16 bytes a lane).
  LDS u16x8* const b1t = (LDS u16x8*)(lds + k.off_fac);
  LDS f4* const a2t = (LDS f4*)(lds + k.off_fac + 3 * 64 * 16);
  for (uint32_t q = threadIdx.x; q < R0 * I0; q += NT3) m0s[q] = k.M0[q];
  if (wv == 0) {
    u16x8 b1[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t i2 = 8 * lg + e;
      const float v = (li < R2 && i2 < I2) ? k.M2[li * I2 + i2] : 0.0f;
      unsigned short a, b, c;
      split3(v, a, b, c);
      b1[0][e] = a; b1[1][e] = b; b1[2][e] = c;
    }
#pragma unroll
    for (int h = 0; h < 3; ++h) b1t[h * 64 + lane] = b1[h];
  } else if (wv == 1) {
#pragma unroll
    for (int r2 = 0; r2 < NRB2; ++r2)
#pragma unroll
      for (int rb = 0; rb < NRB1; ++rb) {
        f4 a;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t j1 = 16 * r2 + li, i1 = 16 * rb + 4 * lg + v;
          a[v] = (j1 < R1 && i1 < I1) ? k.M1[j1 * I1 + i1] : 0.0f;
        }
        a2t[(r2 * NRB1 + rb) * 64 + lane] = a;
      }
  }
  wait_lgkm0();
  wave_fence();
  __builtin_amdgcn_s_barrier();
  wave_fence();

  // this wave's slabs: round c of unit r (unit blockIdx.x + r * gridDim.x) is slab
  // WPB3 c + wv of the unit; g = r * nch + c
  const uint32_t G = gridDim.x;
  const uint32_t nu = (k.U - 1 - blockIdx.x) / G + 1;
  const uint32_t nch = I0 / WPB3;
  const uint32_t cnt = nu * nch;
  auto slab_at = [&](uint32_t r, uint32_t c) -> uint32_t {
    return (blockIdx.x + r * G) * I0 + WPB3 * c + wv;
  };
  auto step = [&](uint32_t& r, uint32_t& c) {
    if (++c == nch) {
      c = 0;
      ++r;
    }
  };
  const XT* X = (const XT*)k.X;
  const uint32_t xchunks = slab_e * 2 / 16;
  // (the slab index is wave-uniform; readfirstlane keeps the base in scalar registers)
  auto dma = [&](uint32_t s, LDS unsigned char* b) {
    const uint32_t su = __builtin_amdgcn_readfirstlane(s);
    wave_dma_n<ND>(X + (uint64_t)su * slab_e, xchunks, b, lane);
  };
  auto bounds = [&](uint32_t s, BoundsV& b) {
    b = load_bounds(k.mask, k.rank, (uint64_t)s * slab_e, slab_e, N, lane);
  };
  auto range = [&](uint32_t s, const BoundsV& b, uint64_t& lo, uint64_t& hi) {
    lo = rank_at(lane_u64(b.m, 0), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 0),
                 (uint64_t)s * slab_e, N, kS);
    hi = rank_at(lane_u64(b.m, 1), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 1),
                 (uint64_t)(s + 1) * slab_e, N, kS);
  };
  OmegaPipe op;
  {
    const uint32_t s0 = slab_at(0, 0);
    if (sparse) {
      BoundsV w;
      bounds(s0, w);
      wait_vm0();
      range(s0, w, op.lo[0], op.hi[0]);
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = op.lo[0] + lane + 64 * q;
        op.om[0][q] = k.omega[j < kS ? j : kS - 1];
      }
      uint32_t r1 = 0, c1 = 0;
      step(r1, c1);
      if (cnt > 1) bounds(slab_at(r1, c1), op.bw);
    }
    dma(s0, xb0);
    // every slab is followed by exactly one transfer (a copy of slab 0 when there is no
    // second slab), so the waits below can count on it
    uint32_t r1 = 0, c1 = 0;
    step(r1, c1);
    dma(cnt > 1 ? slab_at(r1, c1) : s0, xb1);
  }

  f4 acc3[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) acc3[m] = f4{0.f, 0.f, 0.f, 0.f};
  // a finished unit's tiles are written at the start of the next slab, where every
  // transfer has landed anyway
  uint32_t pend = 0xFFFFFFFFu;
  auto write_unit = [&]() {
    if (pend == 0xFFFFFFFFu) return;
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const uint32_t ct = ct0 + (WPB3 / 2) * m;
      if (jb < njb && ct < nct) {
        const uint32_t col = 16 * ct + li;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t row = 16 * jb + 4 * lg + v;
          if (row < R0 && col < RC) k.Y[((uint64_t)pend * R0 + row) * RC + col] = acc3[m][v];
        }
      }
      acc3[m] = f4{0.f, 0.f, 0.f, 0.f};
    }
    pend = 0xFFFFFFFFu;
  };

  uint32_t r = 0, c = 0;   // the current slab's unit (of this workgroup) and round
  auto slab = [&](uint32_t g, auto slot) {
    constexpr int cur = decltype(slot)::value, nxt = cur ^ 1;
    const uint32_t n = slab_at(r, c);
    uint32_t r1 = r, c1 = c;
    step(r1, c1);
    uint32_t rn2 = r1, cn2 = c1;   // the slab after the next one
    step(rn2, cn2);
    // slab n, its Omega indices and the next slab's bounds have landed; the next slab's
    // transfer, the last ND operations issued, may still be in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | ND);   // vmcnt(ND)
    wave_fence();
    write_unit();
    if (g + 1 < cnt && sparse) {
      range(slab_at(r1, c1), op.bw, op.lo[nxt], op.hi[nxt]);
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = op.lo[nxt] + lane + 64 * q;
        op.om[nxt][q] = k.omega[j < kS ? j : kS - 1];
      }
      if (g + 2 < cnt) bounds(slab_at(rn2, cn2), op.bw);
    }

    LDS unsigned short* const xs = (LDS unsigned short*)(cur ? xb1 : xb0);
    const uint64_t e_lo = (uint64_t)n * slab_e;
    if (sparse) {
      // S[j] = X[omega[j]] and X[omega[j]] <- 0 in the LDS copy (+0 is the zero bit
      // pattern of both 16-bit formats); the gradient in HBM is only read
      const uint64_t jlo = op.lo[cur], jhi = op.hi[cur];
      float sv[NOM];
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = jlo + lane + 64 * q;
        sv[q] = j < jhi ? Bits16<XT>::value(xs[(uint32_t)(op.om[cur][q] - e_lo)]) : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = jlo + lane + 64 * q;
        if (j < jhi) {
          k.S[j] = sv[q];
          xs[(uint32_t)(op.om[cur][q] - e_lo)] = 0;
        }
      }
      for (uint64_t j = jlo + 64 * NOM + lane; j < jhi; j += 64) {
        const uint32_t loc = (uint32_t)(k.omega[j] - e_lo);
        k.S[j] = Bits16<XT>::value(xs[loc]);
        xs[loc] = 0;
      }
      wave_fence();
    }

    // pass 1 (mode d): rows i1, k = i2, columns r2, one 16-row block at a time, and
    // the block's terms of pass 2 (mode d-1: rows j1, k = i1, columns r2) straight from
    // its registers
    f4 acc2[NRB2];
#pragma unroll
    for (int r2 = 0; r2 < NRB2; ++r2) acc2[r2] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) {
      const uint32_t i1 = 16 * rb + li;
      u16x8 xp[Bits16<XT>::NP];
      // (the largest tile shapes keep 16-bit reads: the dword form's registers would spill)
      if constexpr (Bits16<XT>::NP == 1 && NRB1 + NRB2 + NTW <= 8) {
        // row i1 (rows past I1 read row I1 - 1 and are masked to zero), i2 = 8 lg + e;
        // past the last wave's buffers lie the round stacks
        const u32x4 w = lds_run8((const LDS unsigned char*)xs + (min(i1, I1 - 1) * I2 + 8 * lg) * 2);
        xp[0] = __builtin_bit_cast(u16x8, w & (i1 < I1 ? keep1 : u32x4{0u, 0u, 0u, 0u}));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t i2 = 8 * lg + e;
          const unsigned short raw =
              (i1 < I1 && i2 < I2) ? xs[i1 * I2 + i2] : (unsigned short)0;
          unsigned short p[2];
          Bits16<XT>::parts(raw, p);
#pragma unroll
          for (int h = 0; h < Bits16<XT>::NP; ++h) xp[h][e] = p[h];
        }
      }
      u16x8 b1[3];
#pragma unroll
      for (int h = 0; h < 3; ++h) b1[h] = b1t[h * 64 + lane];
      f4 acc1 = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (Bits16<XT>::NP == 1) {
        acc1 = mma(xp[0], b1[2], acc1);
        acc1 = mma(xp[0], b1[1], acc1);
        acc1 = mma(xp[0], b1[0], acc1);
      } else {
        acc1 = mma_2x3(xp[0], xp[1], b1, acc1);
      }
#pragma unroll
      for (int r2 = 0; r2 < NRB2; ++r2) {
        const f4 a = a2t[(r2 * NRB1 + rb) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc2[r2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[v], acc1[v], acc2[r2], 0, 0, 0);
      }
    }
    // this slab's buffer has been read: the slab after the next one goes into it, so two
    // transfers are in flight through the stack write, the barrier and the mode d-2 share
    // (past the last slab, a copy of this one that nothing reads keeps the count fixed)
    wave_fence();
    dma(g + 2 < cnt ? slab_at(rn2, cn2) : n, cur ? xb1 : xb0);
    // round g of the workgroup (every wave is in the same round) uses stack g % 2
    LDS float* const st = stacks + cur * SF;
#pragma unroll
    for (int r2 = 0; r2 < NRB2; ++r2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t j1 = 16 * r2 + 4 * lg + v;
        st[(j1 < R1 && li < R2) ? wv * RC + j1 * R2 + li : trash + lane] = acc2[r2][v];
      }

    // the round's stack is complete; its share of the mode d-2 product (the other stack
    // is written only after the next barrier, which follows these reads)
    wait_lgkm0();
    wave_fence();
    __builtin_amdgcn_s_barrier();
    wave_fence();
    // Every operand read is unconditional and at a fixed offset, so the compiler can
    // issue them without a branch or a register per address (reads under a branch each
    // waited for their own LDS round trip). Rows j0 >= R0 read row R0 - 1 (jc), and
    // tiles past the last column block, like columns RC .. 16 nct - 1, read on into the
    // next rows, the other round stack, the M0 copy or the factor tables (all inside the
    // workgroup's LDS); all of these only reach outputs that are not stored.
#pragma unroll
    for (int h = 0; h < WPB3 / 4; ++h) {
      const uint32_t i0l = 4 * h + lg;               // row of the stack
      const uint32_t i0 = WPB3 * c + i0l;            // mode d-2 index
      const float av = m0s[jc * I0 + i0];
      const LDS float* const brow = st + i0l * RC + 16 * ct0 + li;
#pragma unroll
      for (int m = 0; m < NTW; ++m)
        acc3[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, brow[16 * (WPB3 / 2) * m], acc3[m], 0,
                                                       0, 0);
    }
    if (c == nch - 1) pend = blockIdx.x + r * G;
    step(r, c);
  };
  for (uint32_t g = 0; g < cnt; g += 2) {
    slab(g, Slot<0>{});
    if (g + 1 < cnt) slab(g + 1, Slot<1>{});
  }
  wait_vm0();   // the trailing copies have landed before the workgroup's LDS is released
  write_unit();
}

uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

struct Plan3s {
  S3K k;
  size_t lds;
  int nrb1, nrb2, ntw;
  bool ok;
};

Plan3s plan3s(const ModeProd2& mp) {
  Plan3s p{};
  S3K& k = p.k;
  p.ok = false;
  if (mp.P != 1 || mp.recon) return p;
  if (mp.in_dt != DT_BF16 && mp.in_dt != DT_F16) return p;
  const uint32_t I0 = mp.I0, I1 = mp.I1, I2 = mp.I2, R0 = mp.R0, R1 = mp.R1, R2 = mp.R2;
  if (I0 < (uint32_t)WPB3 || I0 > 64 || I0 % WPB3 != 0 || R0 == 0 || R0 > 32) return p;
  if (I1 > 64 || I2 > 32 || R1 > 32 || R2 > 16 || I1 == 0 || I2 == 0 || R1 == 0 || R2 == 0)
    return p;
  const uint32_t slab_e = I1 * I2;
  if (slab_e % 8 != 0 || mp.A == 0 || mp.A % I0 != 0) return p;
  if ((uintptr_t)mp.X % 16) return p;
  // column blocks per wave (WPB3 / 2 waves per 16-row block of R0 <= 32)
  const uint32_t ntw = ((R1 * R2 + 15) / 16 + WPB3 / 2 - 1) / (WPB3 / 2);
  p.ntw = ntw <= 2 ? 2 : ntw <= 3 ? 3 : ntw <= 4 ? 4 : 0;
  if (!p.ntw) return p;
  k.U = mp.A / I0;
  k.I0 = I0; k.I1 = I1; k.I2 = I2; k.R0 = R0; k.R1 = R1; k.R2 = R2;
  k.slab_e = slab_e;
  p.nrb1 = (int)((I1 + 15) / 16);
  p.nrb2 = (int)((R1 + 15) / 16);
  k.off_x1 = al16(slab_e * 2);
  k.lds_wave = 2 * k.off_x1;
  k.off_stack = WPB3 * k.lds_wave;
  k.stack_fl = al16((WPB3 * R1 * R2 + 64) * 4) / 4;
  k.off_m0 = k.off_stack + 2 * k.stack_fl * 4;
  k.off_fac = k.off_m0 + al16(R0 * I0 * 4);
  p.lds = k.off_fac + 3 * 64 * 16 + (size_t)p.nrb2 * p.nrb1 * 64 * 16;
  p.ok = p.lds <= 160 * 1024;
  return p;
}

template <typename XT, int NRB1, int NRB2, int NTW>
auto proj3_fn(uint32_t nd) {
  // a slab of at most 16 NRB1 rows of at most 32 values needs at most NRB1 loads
  return nd <= 1 || NRB1 == 1   ? k_proj3s<XT, NRB1, NRB2, NTW, 1>
         : nd == 2 || NRB1 == 2 ? k_proj3s<XT, NRB1, NRB2, NTW, (NRB1 >= 2 ? 2 : 1)>
         : nd == 3 || NRB1 == 3 ? k_proj3s<XT, NRB1, NRB2, NTW, (NRB1 >= 3 ? 3 : 1)>
                                : k_proj3s<XT, NRB1, NRB2, NTW, (NRB1 >= 4 ? 4 : 1)>;
}
template <typename XT, int NRB1, int NRB2>
hipError_t proj3_ntw(const Plan3s& p, int num_cu, hipStream_t s) {
  const uint32_t nd = (p.k.slab_e * 2 / 16 + 63) / 64;
  if (nd > (uint32_t)NRB1) return hipErrorInvalidValue;
  auto fn = p.ntw == 2   ? proj3_fn<XT, NRB1, NRB2, 2>(nd)
            : p.ntw == 3 ? proj3_fn<XT, NRB1, NRB2, 3>(nd)
                         : proj3_fn<XT, NRB1, NRB2, 4>(nd);
  if (p.lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT3, p.lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidValue;
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * (uint64_t)per_cu;
  if (grid > p.k.U) grid = p.k.U;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(NT3), p.lds, s, p.k);
  return hipGetLastError();
}
template <typename XT, int NRB1>
hipError_t proj3_nrb2(const Plan3s& p, int num_cu, hipStream_t s) {
  if (p.nrb2 == 1) return proj3_ntw<XT, NRB1, 1>(p, num_cu, s);
  return proj3_ntw<XT, NRB1, 2>(p, num_cu, s);
}
template <typename XT>
hipError_t proj3_go(const Plan3s& p, int num_cu, hipStream_t s) {
  switch (p.nrb1) {
    case 1: return proj3_nrb2<XT, 1>(p, num_cu, s);
    case 2: return proj3_nrb2<XT, 2>(p, num_cu, s);
    case 3: return proj3_nrb2<XT, 3>(p, num_cu, s);
    default: return proj3_nrb2<XT, 4>(p, num_cu, s);
  }
}

struct Plan2s {
  S2K k;
  int num_cu;
  size_t lds;
  int nrb1, nrb2;   // projection: (NRB1, NRB2); reconstruction: (NRB1, NCB2)
  bool ok;
};

Plan2s plan2s(const ModeProd2& mp, int num_cu) {
  Plan2s p{};
  S2K& k = p.k;
  p.ok = false;
  if (mp.P != 1) return p;
  const bool rec = mp.recon != 0;
  const int dt16 = rec ? mp.w_dt : mp.in_dt;
  if (dt16 != DT_BF16 && dt16 != DT_F16) return p;
  if (rec && (!mp.apply || mp.in_dt != DT_F32)) return p;
  // sizes in the kernels' names: I = the full-size side, R = the core side
  const uint32_t I1 = rec ? mp.R1 : mp.I1, I2 = rec ? mp.R2 : mp.I2;
  const uint32_t R1 = rec ? mp.I1 : mp.R1, R2 = rec ? mp.I2 : mp.R2;
  if (I1 > 64 || I2 > 32 || R1 > 32 || R2 > 16 || I1 == 0 || I2 == 0 || R1 == 0 || R2 == 0)
    return p;
  const uint32_t slab_e = I1 * I2;
  if (slab_e % 8 != 0 || (R1 * R2) % 4 != 0) return p;
  const uintptr_t big = (uintptr_t)(rec ? mp.W : mp.X);
  const uintptr_t small = (uintptr_t)(rec ? mp.X : (const void*)mp.Y);
  if (big % 16 || small % 16) return p;
  k.I1 = I1; k.I2 = I2; k.R1 = R1; k.R2 = R2;
  k.slab_e = slab_e;
  k.A = mp.A;
  p.nrb1 = (int)((I1 + 15) / 16);
  if (!rec) {
    p.nrb2 = (int)((R1 + 15) / 16);
    k.ly = 16u * p.nrb1 + 4;
    uint32_t off = al16(slab_e * 2);
    k.off_b1 = off; off += al16(slab_e * 2);
    k.off_y = off; off += al16(16 * k.ly * 4);
    k.off_o = off; off += al16((R1 * R2 + 64) * 4);
    k.trash = R1 * R2;
    k.lds_wave = off;
  } else {
    p.nrb2 = (int)((I2 + 15) / 16);
    k.ly = 20;   // Y rows hold j2 < 16 (R2 <= 16), 16-byte aligned
    const uint32_t i1p = 16u * p.nrb1;
    // O rows of block rb must end before Y's block rb + 1 starts
    int64_t d = 0;
    for (int rb = 0; rb + 1 < p.nrb1; ++rb) {
      const int64_t need = 16ll * (rb + 1) * I2 - 16ll * (rb + 1) * k.ly;
      if (need > d) d = need;
    }
    k.ydelta = (uint32_t)((d + 3) & ~3ll);
    const uint32_t ofl = std::max(slab_e, k.ydelta + i1p * k.ly);
    uint32_t off = al16(R1 * R2 * 4);
    k.off_b1 = off; off += al16(R1 * R2 * 4);
    k.off_w0 = off; off += al16(slab_e * 2);
    k.off_o = off; off += al16((ofl + 64) * 4);
    k.trash = ofl;
    k.lds_wave = off;
  }
  p.lds = (size_t)k.lds_wave * WPB;
  p.num_cu = num_cu > 0 ? num_cu : 256;
  p.ok = p.lds <= 64 * 1024;
  return p;
}

// One resident round of workgroups (as many as the kernel's registers and LDS let a CU
// hold); wave w takes every TW-th slab from slab w.
template <typename F>
hipError_t launch2s(F fn, Plan2s p, hipStream_t s) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, p.lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidValue;
  uint64_t grid = (uint64_t)p.num_cu * (uint64_t)per_cu;
  const uint64_t need = ((uint64_t)p.k.A + WPB - 1) / WPB;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(NT), p.lds, s, p.k);
  return hipGetLastError();
}

template <typename XT, int NRB1>
hipError_t proj_nrb2(const Plan2s& p, hipStream_t s) {
  if (p.nrb2 == 1) return launch2s(k_proj2s<XT, NRB1, 1>, p, s);
  return launch2s(k_proj2s<XT, NRB1, 2>, p, s);
}
template <typename XT>
hipError_t proj_go(const Plan2s& p, hipStream_t s) {
  switch (p.nrb1) {
    case 1: return proj_nrb2<XT, 1>(p, s);
    case 2: return proj_nrb2<XT, 2>(p, s);
    case 3: return proj_nrb2<XT, 3>(p, s);
    default: return proj_nrb2<XT, 4>(p, s);
  }
}
template <typename WT, int NRB1, int NCB2, bool CAP>
hipError_t rec_ks(const Plan2s& p, hipStream_t s) {
  switch ((p.k.R1 + 3) / 4) {
    case 1:
    case 2: return launch2s(k_rec2s<WT, NRB1, NCB2, 2, CAP>, p, s);
    case 3:
    case 4: return launch2s(k_rec2s<WT, NRB1, NCB2, 4, CAP>, p, s);
    case 5:
    case 6: return launch2s(k_rec2s<WT, NRB1, NCB2, 6, CAP>, p, s);
    default: return launch2s(k_rec2s<WT, NRB1, NCB2, 8, CAP>, p, s);
  }
}
template <typename WT, int NRB1, bool CAP>
hipError_t rec_ncb(const Plan2s& p, hipStream_t s) {
  if (p.nrb2 == 1) return rec_ks<WT, NRB1, 1, CAP>(p, s);
  return rec_ks<WT, NRB1, 2, CAP>(p, s);
}
template <typename WT, bool CAP>
hipError_t rec_go(const Plan2s& p, hipStream_t s) {
  switch (p.nrb1) {
    case 1: return rec_ncb<WT, 1, CAP>(p, s);
    case 2: return rec_ncb<WT, 2, CAP>(p, s);
    case 3: return rec_ncb<WT, 3, CAP>(p, s);
    default: return rec_ncb<WT, 4, CAP>(p, s);
  }
}

}  // namespace

bool slab2_supported(const ModeProd2& mp, int num_cu) { return plan2s(mp, num_cu).ok; }

bool slab3_supported(const ModeProd2& mp) { return plan3s(mp).ok; }



hipError_t launch_slab3(const ModeProd2& mp, int num_cu, hipStream_t s) {
  Plan3s p = plan3s(mp);
  if (!p.ok) return hipErrorInvalidValue;
  S3K& k = p.k;
  k.X = mp.X;
  k.Y = mp.Y;
  k.M0 = mp.M0;
  k.M1 = mp.M1;
  k.M2 = mp.M2;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.omega = mp.omega;
  k.S = mp.gather_S;
  k.kS = mp.gather_S ? mp.kS : 0;
  return mp.in_dt == DT_BF16 ? proj3_go<bf16_t>(p, num_cu, s) : proj3_go<_Float16>(p, num_cu, s);
}

hipError_t launch_slab2(const ModeProd2& mp, int num_cu, hipStream_t s) {
  Plan2s p = plan2s(mp, num_cu);
  if (!p.ok) return hipErrorInvalidValue;
  S2K& k = p.k;
  const bool rec = mp.recon != 0;
  k.M1 = mp.M1;
  k.M2 = mp.M2;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.omega = mp.omega;
  k.lr = mp.lr;
  k.decay = mp.decay;
  if (!rec) {
    k.X = mp.X;
    k.Y = mp.Y;
    k.S = mp.gather_S;
    k.kS = mp.gather_S ? mp.kS : 0;
    return mp.in_dt == DT_BF16 ? proj_go<bf16_t>(p, s) : proj_go<_Float16>(p, s);
  }
  k.Zin = (const float*)mp.X;
  k.W = mp.W;
  k.S = const_cast<float*>(mp.uS);
  k.kS = mp.has_sparse ? mp.kS : 0;
  k.delta = mp.delta;
  if (mp.delta)
    return mp.w_dt == DT_BF16 ? rec_go<bf16_t, true>(p, s) : rec_go<_Float16, true>(p, s);
  return mp.w_dt == DT_BF16 ? rec_go<bf16_t, false>(p, s) : rec_go<_Float16, false>(p, s);
}

}  // namespace tg
