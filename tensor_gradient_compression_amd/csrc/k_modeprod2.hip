// Two trailing mode products in one pass: the projection's first two products
// (modes d, then d-1) and the reconstruction's last two (modes d-1, then d, fused with
// the weight update).
//
// Same mathematics as the one-mode kernel (pith.science "What carries the argument":
// projection to the core and reconstruction by mode-wise products; appendix M
// Theorem 2: project, update, project back), reorganised so the intermediate between
// the two products never leaves LDS. The tensor is viewed as A slabs of the last two
// modes, (A, I1, I2, P); a slab is contiguous in memory, so a tile of TA slabs is one
// contiguous block in and one contiguous block out.
//   projection:     Y[a, i1, j2] = sum_i2 M2[j2, i2] X[a, i1, i2]       (mode d)
//                   Z[a, j1, j2] = sum_i1 M1[j1, i1] Y[a, i1, j2]       (mode d-1)
//   reconstruction: Y[a, i1, j2] = sum_j1 M1[i1, j1] Z[a, j1, j2]       (mode d-1)
//                   O[a, i1, i2] = sum_j2 M2[i2, j2] Y[a, i1, j2]       (mode d)
//                   W <- round(W * decay - lr * (O + N_S at Omega))
// (indices include the complex part p, as in the one-mode kernel). Each product is an
// MFMA GEMM over LDS operands (v_mfma_f32_16x16x4_f32, fp32 accumulation). Input tiles
// (and W tiles) move HBM -> LDS with 16-byte global_load_lds transfers, double
// buffered; outputs leave with 16-byte stores. Versus two one-mode launches this skips
// writing and re-reading the fp32 intermediate between the two products (nullthought
// summary section 3: no second full tensor).
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int NTH = 512;
constexpr int NW = NTH / 64;   // waves per workgroup
constexpr int NRBMAX = 8;   // up to 128 output rows per product (16 per block)

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct MP2K {
  const void* X;
  const float* M1;
  const float* M2;
  float* Y;
  void* W;
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;
  const uint32_t* omega;
  float* delta;           // EPI == 2: the fp32 update after the sparse merge, stored too
  uint64_t kS, N;
  uint64_t ntiles;
  uint32_t A, TA;
  uint32_t I1, I2, R1, R2;          // input and output slab sizes (elements)
  float inv_b;                      // 1/B of the pass whose B > 1 (fp32-rounded)
  // GEMM shapes of the two passes (values, complex parts included)
  uint32_t k1, kp1, m1, mp1, k2, kp2, m2, mp2;
  uint32_t dma_in, dma_w, vout;
  uint32_t off_m2, off_x0, off_x1, off_y, off_o, off_w0, off_w1, off_r0, off_r1;
  float lr;
  float decay;            // fp32(1 - lr * weight_decay): 1 exactly without decay
  int has_sparse;
  float* gS;              // projection with the COO gather folded in (else null)
};

// One mode product between LDS buffers over the (A', I, B, P) view: ncols = A' * B
// GEMM columns; dst[a', jj, b] = sum_kk sM[jj, kk] src[a', kk, b]. The (16-column block,
// 16-row block) items are dealt to the waves in turn. The inner loop is one
// A read at a fixed stride, one B read from a strength-reduced pointer and the MFMA:
// sM is zero past Kin, and only the last k-step can hold source rows >= Kin (zeroed
// there). Lanes of columns past ncols read a real column whose result is dropped.
// B1: B == 1 (columns are whole fibres). Otherwise a column splits as col = a' B + b
// with a' = floor((col + 1/2) * invB) in fp32: with col < 2^16 and B <= 128 the
// product is within 2^-10 of (col + 1/2) / B, whose distance to an integer is at
// least 1/(2B), so the floor is exact.
template <typename ST, int P, bool B1>
__device__ __forceinline__ void lds_gemm(const ST* src, uint32_t ncols, uint32_t B, float invB,
                                         uint32_t I, uint32_t R, const float* sM, uint32_t Kin,
                                         uint32_t Kpad, uint32_t Mout, uint32_t Mpad,
                                         float* dst) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t g = lane >> 4, li = lane & 15;
  const uint32_t LDM = Kpad + 1;
  const uint32_t rs = B1 ? P : B * P;
  const uint32_t blk_in = I * rs, blk_out = R * rs;
  const uint32_t ncb = (ncols + 15) / 16;
  const uint32_t nks = Kpad >> 2;
  // row kk = 4*ks + g of a column sits at (kk / P) * rs + kk % P
  const uint32_t goff = (P == 1) ? g * rs : (g >> 1) * rs + (g & 1);
  const uint32_t kstep = (P == 1) ? 4 * rs : 2 * rs;
  const bool last_ok = 4 * (nks - 1) + g < Kin;
  // output rows r0 + 4g + v, v = 0..3, sit at (r0 + 4g) / P * rs + vo(v)
  const uint32_t vo1 = (P == 1) ? rs : 1, vo2 = (P == 1) ? 2 * rs : rs;
  const uint32_t vo3 = (P == 1) ? 3 * rs : rs + 1;
  const uint32_t nrb = Mpad >> 4;
  // item = rb * ncb + cb, this wave's first one: cb = wave mod ncb, rb = wave / ncb
  uint32_t cb = wave, rb = 0;
  while (cb >= ncb) {
    cb -= ncb;
    ++rb;
  }
  while (rb < nrb) {
    const uint32_t c0 = cb * 16 + li;
    const bool valid = c0 < ncols;
    const uint32_t col = valid ? c0 : ncols - 1;
    uint32_t ca, cbb;
    if (B1) {
      ca = col;
      cbb = 0;
    } else {
      ca = (uint32_t)(((float)col + 0.5f) * invB);
      cbb = col - ca * B;
    }
    const uint32_t r0 = rb * 16;
    const ST* b = src + ca * blk_in + cbb * P + goff;
    const float* ap = sM + (r0 + li) * LDM + g;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    for (uint32_t ks = 0; ks + 1 < nks; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ap[4 * ks], to_f32(*b), acc, 0, 0, 0);
      b += kstep;
    }
    const float bl = last_ok ? to_f32(*b) : 0.0f;
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ap[4 * (nks - 1)], bl, acc, 0, 0, 0);
    float* d = dst + ca * blk_out + cbb * P + ((r0 + 4 * g) / P) * rs;
    if (r0 + 16 <= Mout) {
      if (valid) {
        d[0] = acc[0];
        d[vo1] = acc[1];
        d[vo2] = acc[2];
        d[vo3] = acc[3];
      }
    } else if (valid) {
      const uint32_t j0 = r0 + 4 * g;
      if (j0 < Mout) d[0] = acc[0];
      if (j0 + 1 < Mout) d[vo1] = acc[1];
      if (j0 + 2 < Mout) d[vo2] = acc[2];
      if (j0 + 3 < Mout) d[vo3] = acc[3];
    }
    cb += NW;
    while (cb >= ncb) {
      cb -= ncb;
      ++rb;
    }
  }
}

template <typename T>
__device__ __forceinline__ void dma_block(const T* src, uint32_t nvals, unsigned char* dst) {
  constexpr uint32_t V = 16 / sizeof(T);
  const uint32_t total = nvals / V;
  const int tid = threadIdx.x;
  const uint32_t wave_base = (uint32_t)(tid & ~63);
  for (uint32_t q0 = 0; q0 < total; q0 += NTH) {
    const uint32_t q = q0 + tid;
    unsigned char* lds = dst + (size_t)(q0 + wave_base) * 16;   // wave-uniform
    if (q < total)
      __builtin_amdgcn_global_load_lds((const void*)(src + (uint64_t)q * V), (lds_void*)lds, 16, 0, 0);
  }
}

template <typename XT, int P, int REC, int EPI, typename WT>
__global__ void __launch_bounds__(NTH) k_modeprod2(MP2K k) {
  constexpr int VO = (EPI == 0) ? 4 : 16 / (int)sizeof(WT);
  extern __shared__ float smem[];
  unsigned char* lds = (unsigned char*)smem;
  const int tid = threadIdx.x;
  float* sM1 = smem;
  float* sM2 = (float*)(lds + k.off_m2);
  float* sYm = (float*)(lds + k.off_y);
  float* sO = (float*)(lds + k.off_o);
  const XT* __restrict__ X = (const XT*)k.X;

  for (uint32_t idx = tid; idx < k.mp1 * k.kp1; idx += NTH) {
    const uint32_t jj = idx / k.kp1, kk = idx - jj * k.kp1;
    sM1[jj * (k.kp1 + 1) + kk] = (jj < k.m1 && kk < k.k1) ? k.M1[(uint64_t)jj * k.k1 + kk] : 0.0f;
  }
  for (uint32_t idx = tid; idx < k.mp2 * k.kp2; idx += NTH) {
    const uint32_t jj = idx / k.kp2, kk = idx - jj * k.kp2;
    sM2[jj * (k.kp2 + 1) + kk] = (jj < k.m2 && kk < k.k2) ? k.M2[(uint64_t)jj * k.k2 + kk] : 0.0f;
  }

  const uint32_t slab_in = k.I1 * k.I2 * P, slab_out = k.R1 * k.R2 * P;
  // projection: pass 1 is mode d (M = M2), pass 2 mode d-1 (M = M1);
  // reconstruction: pass 1 is mode d-1 (M = M1), pass 2 mode d (M = M2).
  const float* sA = REC ? sM1 : sM2;
  const float* sB = REC ? sM2 : sM1;
  const uint32_t ka = REC ? k.k1 : k.k2, kpa = REC ? k.kp1 : k.kp2;
  const uint32_t ma = REC ? k.m1 : k.m2, mpa = REC ? k.mp1 : k.mp2;
  const uint32_t kb = REC ? k.k2 : k.k1, kpb = REC ? k.kp2 : k.kp1;
  const uint32_t mb = REC ? k.m2 : k.m1, mpb = REC ? k.mp2 : k.mp1;

  auto can_dma_in = [&](uint32_t nta) { return k.dma_in && (nta * slab_in * sizeof(XT)) % 16 == 0; };
  auto can_dma_w = [&](uint32_t nta) {
    return EPI >= 1 && k.dma_w && (nta * slab_out * sizeof(WT)) % 16 == 0;
  };
  auto nta_of = [&](uint64_t tile) -> uint32_t {
    const uint64_t a0 = tile * k.TA;
    return (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
  };
  auto issue = [&](uint64_t tile, int buf) {
    const uint32_t nta = nta_of(tile);
    const uint64_t a0 = tile * k.TA;
    if (can_dma_in(nta))
      dma_block<XT>(X + a0 * slab_in, nta * slab_in, lds + (buf ? k.off_x1 : k.off_x0));
    if (EPI >= 1 && can_dma_w(nta))
      dma_block<WT>((const WT*)k.W + a0 * slab_out, nta * slab_out,
                    lds + (buf ? k.off_w1 : k.off_w0));
  };
  // The tile's Omega entries are the contiguous range [rank(e_lo), rank(e_hi)) of the
  // sorted list, rank(e) = rank[e / 64] + popcount(mask[e / 64] below bit e % 64), over
  // the tile's output elements (reconstruction) or input elements (projection). The
  // two boundary words and ranks travel with the tile's transfer: lanes 0-5 of wave 0
  // bring mask[lo] (2 dwords), rank[lo], mask[hi] (2 dwords), rank[hi] into a 24-byte
  // LDS slot of the same buffer, read after the barrier that publishes the tile.
  const uint32_t slab_e = REC ? slab_out : slab_in;
  auto tile_lo = [&](uint64_t tile) -> uint64_t { return tile * k.TA * slab_e / P; };
  auto tile_hi = [&](uint64_t tile) -> uint64_t {
    return (tile * k.TA + nta_of(tile)) * slab_e / P;
  };
  auto issue_rank = [&](uint64_t tile, int buf) {
    if (tid < 6) {
      const uint64_t e = tid < 3 ? tile_lo(tile) : tile_hi(tile);
      const uint32_t part = tid % 3;
      const uint64_t w = e < k.N ? e >> 6 : 0;
      const void* src = part < 2 ? (const void*)((const uint32_t*)(k.mask + w) + part)
                                 : (const void*)(k.rank + w);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + (buf ? k.off_r1 : k.off_r0)), 4,
                                       0, 0);
    }
  };
  auto rank_from = [&](const uint32_t* r, uint64_t e) -> uint64_t {
    if (e >= k.N) return k.kS;
    const uint64_t word = (uint64_t)r[0] | ((uint64_t)r[1] << 32);
    return r[2] + (uint64_t)__popcll(word & ((1ull << (e & 63)) - 1ull));
  };
  const bool merged = (EPI >= 1) && k.has_sparse;
  // projection: the sparse part leaves the staged input before the first product
  const bool gath = !REC && k.gS != nullptr;
  const bool ranged = merged || gath;
  constexpr int NSR = 2;
  uint64_t jc0 = 0, jc1 = 0;

  uint64_t tile = blockIdx.x;
  int cur = 0;
  if (tile < k.ntiles) {
    issue(tile, cur);
    if (ranged) issue_rank(tile, cur);
  }
  __builtin_amdgcn_s_waitcnt(0);
  for (; tile < k.ntiles; tile += gridDim.x) {
    const uint64_t next = tile + gridDim.x;
    lds_barrier();
    const uint32_t nta = nta_of(tile);
    const uint64_t a0 = tile * k.TA;
    unsigned char* bx = lds + (cur ? k.off_x1 : k.off_x0);
    unsigned char* bw = lds + (cur ? k.off_w1 : k.off_w0);
    if (ranged) {
      const uint32_t* r = (const uint32_t*)(lds + (cur ? k.off_r1 : k.off_r0));
      jc0 = rank_from(r, tile_lo(tile));
      jc1 = rank_from(r + 3, tile_hi(tile));
    }
    if (next < k.ntiles) {
      issue(next, cur ^ 1);
      if (ranged) issue_rank(next, cur ^ 1);
    }
    uint32_t om_r[NSR];
    float us_r[NSR][P];
    if (ranged) {
#pragma unroll
      for (int i = 0; i < NSR; ++i) {
        const uint64_t j = jc0 + tid + (uint64_t)NTH * i;
        if (j < jc1) {
          om_r[i] = k.omega[j];
          if (merged) {
#pragma unroll
            for (int p = 0; p < P; ++p) us_r[i][p] = k.uS[j * P + p];
          }
        }
      }
    }
    bool filled = false;
    if (!can_dma_in(nta)) {
      XT* d = (XT*)bx;
      for (uint32_t idx = tid; idx < nta * slab_in; idx += NTH) d[idx] = X[a0 * slab_in + idx];
      filled = true;
    }
    if (EPI >= 1 && !can_dma_w(nta)) {
      WT* d = (WT*)bw;
      const WT* W = (const WT*)k.W;
      for (uint32_t idx = tid; idx < nta * slab_out; idx += NTH) d[idx] = W[a0 * slab_out + idx];
      filled = true;
    }
    if (filled) lds_barrier();

    if (gath) {
      // S[j] = X[omega[j]] (fp32), then X[omega[j]] <- 0 in the staged tile: the
      // projection runs on the residual; the gradient in HBM is only read
      const uint64_t e_lo = a0 * slab_in / P;
      XT* xs = (XT*)bx;
      const XT z = zero_of<XT>();
      auto take = [&](uint64_t j, uint32_t om) {
        const uint32_t loc = (uint32_t)(om - e_lo) * P;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          k.gS[j * P + p] = to_f32(xs[loc + p]);
          xs[loc + p] = z;
        }
      };
#pragma unroll
      for (int i = 0; i < NSR; ++i) {
        const uint64_t j = jc0 + tid + (uint64_t)NTH * i;
        if (j < jc1) take(j, om_r[i]);
      }
      for (uint64_t j = jc0 + (uint64_t)NTH * NSR + tid; j < jc1; j += NTH) take(j, k.omega[j]);
      lds_barrier();
    }

    if (!REC) {
      // mode d: (A' = nta*I1, I = I2, B = 1) -> (nta*I1, R2, 1)
      lds_gemm<XT, P, true>((const XT*)bx, nta * k.I1, 1, 1.0f, k.I2, k.R2, sA, ka, kpa, ma,
                            mpa, sYm);
      lds_barrier();
      // mode d-1: (A' = nta, I = I1, B = R2) -> (nta, R1, R2)
      lds_gemm<float, P, false>(sYm, nta * k.R2, k.R2, k.inv_b, k.I1, k.R1, sB, kb, kpb, mb,
                                mpb, sO);
    } else {
      // mode d-1: (A' = nta, I = I1, B = I2) -> (nta, R1, I2)
      lds_gemm<XT, P, false>((const XT*)bx, nta * k.I2, k.I2, k.inv_b, k.I1, k.R1, sA, ka, kpa,
                             ma, mpa, sYm);
      lds_barrier();
      // mode d: (A' = nta*R1, I = I2, B = 1) -> (nta*R1, R2, 1)
      lds_gemm<float, P, true>(sYm, nta * k.R1, 1, 1.0f, k.I2, k.R2, sB, kb, kpb, mb, mpb,
                               sO);
    }
    lds_barrier();
    if (merged) {
      const uint64_t e_lo = a0 * slab_out / P;
#pragma unroll
      for (int i = 0; i < NSR; ++i) {
        const uint64_t j = jc0 + tid + (uint64_t)NTH * i;
        if (j < jc1) {
          const uint32_t loc = (uint32_t)(om_r[i] - e_lo) * P;
#pragma unroll
          for (int p = 0; p < P; ++p) sO[loc + p] = sO[loc + p] + us_r[i][p];
        }
      }
      for (uint64_t j = jc0 + (uint64_t)NTH * NSR + tid; j < jc1; j += NTH) {
        const uint32_t loc = (uint32_t)(k.omega[j] - e_lo) * P;
#pragma unroll
        for (int p = 0; p < P; ++p) sO[loc + p] = sO[loc + p] + k.uS[j * P + p];
      }
      lds_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);   // next tile's transfer landed; previous stores done

    const uint32_t len = nta * slab_out;
    const uint64_t gbase = a0 * slab_out;
    if (k.vout && len % VO == 0) {
      for (uint32_t q = tid; q < len / VO; q += NTH) {
        const uint32_t off = q * VO;
        float d[VO];
#pragma unroll
        for (int e = 0; e < VO; e += 4) {
          const float4 t = *(const float4*)(sO + off + e);
          d[e] = t.x; d[e + 1] = t.y; d[e + 2] = t.z; d[e + 3] = t.w;
        }
        if (EPI == 0) {
          *(float4*)&k.Y[gbase + off] = make_float4(d[0], d[1], d[2], d[3]);
        } else {
          const uint4 wraw = *(const uint4*)(bw + (size_t)off * sizeof(WT));
          const WT* ws = (const WT*)&wraw;
          WT wv[VO];
#pragma unroll
          for (int e = 0; e < VO; ++e) wv[e] = from_f32<WT>(to_f32(ws[e]) * k.decay - k.lr * d[e]);
          *(uint4*)((WT*)k.W + gbase + off) = *(const uint4*)wv;
          if (EPI == 2) {
#pragma unroll
            for (int e = 0; e < VO; e += 4)
              *(float4*)&k.delta[gbase + off + e] = make_float4(d[e], d[e + 1], d[e + 2], d[e + 3]);
          }
        }
      }
    } else {
      for (uint32_t q = tid; q < len; q += NTH) {
        if (EPI == 0) {
          k.Y[gbase + q] = sO[q];
        } else {
          const float w = to_f32(((const WT*)bw)[q]);
          ((WT*)k.W)[gbase + q] = from_f32<WT>(w * k.decay - k.lr * sO[q]);
          if (EPI == 2) k.delta[gbase + q] = sO[q];
        }
      }
    }
    cur ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(0);
}

size_t esz(int dt) { return dt == DT_F32 ? 4 : 2; }

struct Geo2 {
  MP2K k;
  size_t lds;
  bool ok;
};

Geo2 plan(const ModeProd2& mp, uint32_t TA) {
  Geo2 g{};
  MP2K& k = g.k;
  const uint32_t P = mp.P;
  k.I1 = mp.I1;
  k.I2 = mp.I2;
  k.R1 = mp.R1;
  k.R2 = mp.R2;
  k.inv_b = 1.0f / (float)(mp.recon ? mp.I2 : mp.R2);
  // pass shapes: M1 is (R1*P) x (I1*P), M2 is (R2*P) x (I2*P)
  k.k1 = mp.I1 * P; k.m1 = mp.R1 * P;
  k.k2 = mp.I2 * P; k.m2 = mp.R2 * P;
  k.kp1 = (k.k1 + 3) & ~3u; k.mp1 = (k.m1 + 15) & ~15u;
  k.kp2 = (k.k2 + 3) & ~3u; k.mp2 = (k.m2 + 15) & ~15u;
  g.ok = k.mp1 <= 16 * NRBMAX && k.mp2 <= 16 * NRBMAX && k.kp1 <= 128 && k.kp2 <= 128;
  // the fp32 column split in lds_gemm needs ncols < 2^16 and B <= 128
  const uint32_t dmax = std::max(std::max(mp.I1, mp.I2), std::max(mp.R1, mp.R2));
  g.ok = g.ok && dmax <= 128 && (uint64_t)TA * dmax * dmax < 65536;
  k.A = mp.A;
  k.TA = TA;
  k.ntiles = ((uint64_t)mp.A + TA - 1) / TA;
  const size_t esx = P == 2 ? 4 : esz(mp.in_dt);
  const size_t esw = mp.apply ? (P == 2 ? 4 : esz(mp.w_dt)) : 4;
  const size_t slab_in = (size_t)mp.I1 * mp.I2 * P, slab_out = (size_t)mp.R1 * mp.R2 * P;
  const size_t slab_mid = mp.recon ? (size_t)mp.R1 * mp.I2 * P : (size_t)mp.I1 * mp.R2 * P;
  auto al = [](size_t x) { return (x + 15) & ~(size_t)15; };
  size_t off = al((size_t)k.mp1 * (k.kp1 + 1) * 4);
  k.off_m2 = (uint32_t)off; off += al((size_t)k.mp2 * (k.kp2 + 1) * 4);
  k.off_x0 = (uint32_t)off; off += al(TA * slab_in * esx);
  k.off_x1 = (uint32_t)off; off += al(TA * slab_in * esx);
  k.off_y = (uint32_t)off; off += al(TA * slab_mid * 4);
  k.off_o = (uint32_t)off; off += al(TA * slab_out * 4);
  k.off_w0 = (uint32_t)off; off += mp.apply ? al(TA * slab_out * esw) : 0;
  k.off_w1 = (uint32_t)off; off += mp.apply ? al(TA * slab_out * esw) : 0;
  const bool ranged = mp.apply || mp.gather_S;
  k.off_r0 = (uint32_t)off; off += ranged ? 32 : 0;
  k.off_r1 = (uint32_t)off; off += ranged ? 32 : 0;
  g.lds = off;
  const auto a16 = [](const void* p) { return ((uintptr_t)p) % 16 == 0; };
  k.dma_in = a16(mp.X) && (TA * slab_in * esx) % 16 == 0;
  k.dma_w = mp.apply && a16(mp.W) && (TA * slab_out * esw) % 16 == 0;
  k.vout = a16(mp.apply ? mp.W : (const void*)mp.Y) && (TA * slab_out * esw) % 16 == 0;
  return g;
}

// `grid` is the number of CUs; the launch puts one resident round of workgroups on
// each (as many as the kernel's registers and LDS let a CU hold), capped by the tiles.
template <typename XT, int P, int REC, int EPI, typename WT>
hipError_t go2(const MP2K& k, size_t lds, unsigned grid, hipStream_t s) {
  auto fn = k_modeprod2<XT, P, REC, EPI, WT>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NTH, lds);
  if (e != hipSuccess) return e;
  uint64_t g = (uint64_t)grid * (uint64_t)(per_cu > 0 ? per_cu : 1);
  if (g > k.ntiles) g = k.ntiles;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(fn, dim3((unsigned)g), dim3(NTH), lds, s, k);
  return hipGetLastError();
}

}  // namespace

// MFMA k-steps the busiest wave spends on one pass of a tile, as lds_gemm splits it:
// (16-column block, 16-row block) items dealt round-robin to the NW waves.
static uint64_t pass_steps(uint64_t ncols, uint32_t kpad, uint32_t mpad) {
  const uint64_t items = (ncols + 15) / 16 * (mpad / 16);
  return (items + NW - 1) / NW * (kpad / 4);
}

// Tile (whole slabs) with LDS <= 52 KB (three or more workgroups per CU) that minimises
// the busiest wave's MFMA k-steps per slab over both passes plus a per-tile fixed cost
// (larger tile on ties); 0
// when not even one slab fits (or a product is too large): the caller then uses two
// one-mode launches.
uint32_t modeprod2_tile(const ModeProd2& mp) {
  uint32_t best = 0;
  double best_cost = 0.0;
  for (uint32_t TA = 1; TA <= 64; ++TA) {
    const Geo2 g = plan(mp, TA);
    if (!g.ok || g.lds > 52 * 1024) break;
    const MP2K& k = g.k;
    const uint64_t steps =
        mp.recon ? pass_steps((uint64_t)TA * mp.I2, k.kp1, k.mp1) +
                       pass_steps((uint64_t)TA * mp.R1, k.kp2, k.mp2)
                 : pass_steps((uint64_t)TA * mp.I1, k.kp2, k.mp2) +
                       pass_steps((uint64_t)TA * mp.R2, k.kp1, k.mp1);
    // + 16: a tile's fixed work (barriers, transfer issue, stream-out) costs about as
    // much as 16 k-steps on this GEMM shape class (measured on bf16 48x25 -> 24x13)
    const double cost = (double)(steps + 16) / TA;
    if (!best || cost <= best_cost) {
      best = TA;
      best_cost = cost;
    }
    if ((uint64_t)TA >= mp.A) break;
  }
  return best;
}

hipError_t launch_modeprod2(const ModeProd2& mp, int num_cu, hipStream_t s) {
  const uint32_t TA = mp.force_ta ? mp.force_ta : modeprod2_tile(mp);
  if (!TA) return hipErrorInvalidValue;
  Geo2 g = plan(mp, TA);
  if (!g.ok || g.lds > 160 * 1024) return hipErrorInvalidValue;
  MP2K& k = g.k;
  k.X = mp.X;
  k.M1 = mp.M1;
  k.M2 = mp.M2;
  k.Y = mp.Y;
  k.W = mp.W;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.uS = mp.uS;
  k.omega = mp.omega;
  k.delta = mp.delta;
  k.kS = mp.kS;
  // elements the Omega ranks count over: the output (reconstruction), the input (projection)
  k.N = (uint64_t)mp.A * (mp.recon ? (uint64_t)mp.R1 * mp.R2 : (uint64_t)mp.I1 * mp.I2);
  k.lr = mp.lr;
  k.decay = mp.decay;
  k.has_sparse = mp.has_sparse;
  k.gS = mp.recon ? nullptr : mp.gather_S;
  // persistent grid: one resident round per CU (sized in go2())
  const unsigned gr = (unsigned)(num_cu > 0 ? num_cu : 256);
  if (!mp.recon) {
    if (mp.P == 2) return go2<float, 2, 0, 0, float>(k, g.lds, gr, s);
    switch (mp.in_dt) {
      case DT_F32: return go2<float, 1, 0, 0, float>(k, g.lds, gr, s);
      case DT_F16: return go2<_Float16, 1, 0, 0, float>(k, g.lds, gr, s);
      case DT_BF16: return go2<bf16_t, 1, 0, 0, float>(k, g.lds, gr, s);
    }
    return hipErrorInvalidValue;
  }
  if (mp.in_dt != DT_F32) return hipErrorInvalidValue;
  if (!mp.apply)
    return mp.P == 2 ? go2<float, 2, 1, 0, float>(k, g.lds, gr, s)
                     : go2<float, 1, 1, 0, float>(k, g.lds, gr, s);
  if (mp.delta) {
    if (mp.P == 2) return go2<float, 2, 1, 2, float>(k, g.lds, gr, s);
    switch (mp.w_dt) {
      case DT_F32: return go2<float, 1, 1, 2, float>(k, g.lds, gr, s);
      case DT_F16: return go2<float, 1, 1, 2, _Float16>(k, g.lds, gr, s);
      case DT_BF16: return go2<float, 1, 1, 2, bf16_t>(k, g.lds, gr, s);
    }
    return hipErrorInvalidValue;
  }
  if (mp.P == 2) return go2<float, 2, 1, 1, float>(k, g.lds, gr, s);
  switch (mp.w_dt) {
    case DT_F32: return go2<float, 1, 1, 1, float>(k, g.lds, gr, s);
    case DT_F16: return go2<float, 1, 1, 1, _Float16>(k, g.lds, gr, s);
    case DT_BF16: return go2<float, 1, 1, 1, bf16_t>(k, g.lds, gr, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
