// Mode-n products of the Tucker projection and reconstruction on MFMA.
//
// Projection C = R x_1 U1^H ... x_d Ud^H and reconstruction Delta_L = N_C x_1 U1 ...
// x_d Ud (pith.science "What carries the argument": the gradient is projected to a
// small core and the update reconstructed by mode-wise products; its appendix M
// excerpt of Theorem 2: project, update states, project back). Each mode product is
// one launch over the tensor viewed as (A, I, B, P): A = product of the sizes before
// mode n, I = size of mode n, B = product of the sizes after it, P = 2 for complex
// (re, im innermost) else 1. Output Y[a, jj, b] = sum_kk M[jj, kk] X[a, kk, b] with
// kk = i*P + p, jj = j*P + q; a complex product is this real GEMM with M built from
// the 2x2 real blocks of each complex factor entry.
//
// Tiling: a tile is 64 GEMM columns (a, b). If B >= 64 the tile is one a and 64
// consecutive b: I rows of 64*P contiguous values. If B < 64 the tile is
// floor(64 / B) consecutive a, i.e. one contiguous block. The tile is copied
// coalesced into LDS (converted to fp32) in its memory order; the operand matrix M
// sits in LDS for the whole persistent workgroup. Four waves each own 16 columns and
// every 16-row block of the output; v_mfma_f32_16x16x4_f32 accumulates in fp32. The
// output tile is staged back into LDS and written out in memory order, so global
// stores are contiguous.
//
// Epilogues: store (fp32 intermediate / core) or apply (last reconstruction): W <-
// round(W - lr * (acc + N_S at Omega)), with Omega membership from the bitmask and
// the position in Omega from the per-word rank (nullthought summary section 3: the
// sparse update is scatter-added after the low-rank reconstruction so that two full
// tensors never coexist; here the full Delta never exists at all).
#include "tg_common.h"

namespace tg {

namespace {

constexpr int TC = 64;      // GEMM columns per tile
constexpr int NTH = 256;    // 4 waves
constexpr int PADW = 4;     // LDS row padding (floats) of wide tiles

typedef float f4 __attribute__((ext_vector_type(4)));

struct MPK {
  const void* X;
  const float* M;
  float* Y;
  void* W;
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;
  uint64_t ntiles;
  uint32_t tiles_per_a;
  uint32_t A, I, B, R;
  uint32_t Kin, Mout, Kpad, Mpad;
  uint32_t TA;
  uint32_t wide;
  float lr;
  int has_sparse;
};

template <typename XT, int P, int NRB, int EPI, typename WT>
__global__ void __launch_bounds__(NTH) k_modeprod(MPK k) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t LDM = k.Kpad + 1;
  float* sM = smem;
  float* sX = smem + ((k.Mpad * LDM + 3u) & ~3u);
  const XT* __restrict__ X = (const XT*)k.X;

  for (uint32_t idx = tid; idx < k.Mpad * k.Kpad; idx += NTH) {
    const uint32_t jj = idx / k.Kpad, kk = idx - jj * k.Kpad;
    sM[jj * LDM + kk] = (jj < k.Mout && kk < k.Kin) ? k.M[(uint64_t)jj * k.Kin + kk] : 0.0f;
  }

  constexpr uint32_t TW = TC * P;                 // floats per wide tile row
  constexpr uint32_t TWSH = (P == 1) ? 6 : 7;     // log2(TW)
  const uint32_t rs_in = k.wide ? TW + PADW : k.B * P;
  const uint32_t rs_out = k.wide ? TW + PADW : k.B * P;
  const uint32_t blk_in = k.I * k.B * P;
  const uint32_t blk_out = k.R * k.B * P;
  const int col = wave * 16 + (lane & 15);

  for (uint64_t tile = blockIdx.x; tile < k.ntiles; tile += gridDim.x) {
    uint64_t a0;
    uint32_t b0, ncol, nta;
    if (k.wide) {
      a0 = tile / k.tiles_per_a;
      b0 = (uint32_t)(tile - a0 * k.tiles_per_a) * TC;
      ncol = k.B - b0 < (uint32_t)TC ? k.B - b0 : (uint32_t)TC;
      nta = 1;
    } else {
      a0 = tile * k.TA;
      b0 = 0;
      nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      ncol = nta * k.B;
    }
    __syncthreads();   // M staged / previous tile fully consumed
    if (k.wide) {
      const uint32_t rowlen = ncol * P;
      for (uint32_t idx = tid; idx < k.I * TW; idx += NTH) {
        const uint32_t i = idx >> TWSH, e = idx & (TW - 1);
        if (e < rowlen)
          sX[i * rs_in + e] = to_f32(X[((a0 * k.I + i) * k.B + b0) * P + e]);
      }
    } else {
      const uint32_t n = nta * blk_in;
      const uint64_t base = a0 * blk_in;
      for (uint32_t idx = tid; idx < n; idx += NTH) sX[idx] = to_f32(X[base + idx]);
    }
    __syncthreads();

    const bool cvalid = (uint32_t)col < ncol;
    uint32_t cb_in = 0, cb_out = 0;
    if (cvalid) {
      if (k.wide) {
        cb_in = col * P;
        cb_out = col * P;
      } else {
        const uint32_t ca = col / k.B, cbb = col - ca * k.B;
        cb_in = ca * blk_in + cbb * P;
        cb_out = ca * blk_out + cbb * P;
      }
    }
    f4 acc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[rb] = f4{0.f, 0.f, 0.f, 0.f};
    const uint32_t nks = k.Kpad >> 2;
    for (uint32_t ks = 0; ks < nks; ++ks) {
      const uint32_t kk = ks * 4 + (lane >> 4);
      float bv = 0.0f;
      if (cvalid && kk < k.Kin) bv = sX[cb_in + (kk / P) * rs_in + (kk % P)];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if ((uint32_t)rb * 16 < k.Mpad) {
          const float av = sM[(rb * 16 + (lane & 15)) * LDM + kk];
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[rb], 0, 0, 0);
        }
      }
    }
    __syncthreads();   // every wave finished reading the input tile
    if (cvalid) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t jj = rb * 16 + 4 * (lane >> 4) + v;
          if (jj < k.Mout) sX[cb_out + (jj / P) * rs_out + (jj % P)] = acc[rb][v];
        }
      }
    }
    __syncthreads();

    // stream the output tile out in memory order
    auto emit = [&](uint64_t g, float val) {
      if (EPI == 0) {
        k.Y[g] = val;
      } else {
        float d = val;
        if (k.has_sparse) {
          const uint64_t e = g / P;
          const uint64_t word = k.mask[e >> 6];
          if ((word >> (e & 63)) & 1ull) {
            const uint64_t j = omega_rank(k.mask, k.rank, e, word);
            d = d + k.uS[j * P + (g % P)];
          }
        }
        WT* W = (WT*)k.W;
        const float w = to_f32(W[g]);
        W[g] = from_f32<WT>(w - k.lr * d);
      }
    };
    if (k.wide) {
      const uint32_t rowlen = ncol * P;
      for (uint32_t idx = tid; idx < k.R * TW; idx += NTH) {
        const uint32_t j = idx >> TWSH, e = idx & (TW - 1);
        if (e < rowlen) emit(((a0 * k.R + j) * k.B + b0) * P + e, sX[j * rs_out + e]);
      }
    } else {
      const uint32_t n = nta * blk_out;
      const uint64_t base = a0 * blk_out;
      for (uint32_t idx = tid; idx < n; idx += NTH) emit(base + idx, sX[idx]);
    }
  }
}

struct Geo {
  uint32_t Kin, Mout, Kpad, Mpad, wide, TA, tiles_per_a;
  uint64_t ntiles;
  size_t lds;
};

Geo geometry(const ModeProd& mp) {
  Geo g;
  g.Kin = mp.I * mp.P;
  g.Mout = mp.R * mp.P;
  g.Kpad = (g.Kin + 3u) & ~3u;
  g.Mpad = (g.Mout + 15u) & ~15u;
  g.wide = mp.B >= (uint32_t)TC;
  if (g.wide) {
    g.tiles_per_a = (mp.B + TC - 1) / TC;
    g.TA = 1;
    g.ntiles = (uint64_t)mp.A * g.tiles_per_a;
  } else {
    g.tiles_per_a = 1;
    g.TA = TC / mp.B;
    g.ntiles = ((uint64_t)mp.A + g.TA - 1) / g.TA;
  }
  const size_t sm = ((size_t)g.Mpad * (g.Kpad + 1) + 3) & ~(size_t)3;
  size_t tin, tout;
  if (g.wide) {
    tin = (size_t)mp.I * (TC * mp.P + PADW);
    tout = (size_t)mp.R * (TC * mp.P + PADW);
  } else {
    tin = (size_t)g.TA * mp.I * mp.B * mp.P;
    tout = (size_t)g.TA * mp.R * mp.B * mp.P;
  }
  g.lds = (sm + (tin > tout ? tin : tout)) * sizeof(float);
  return g;
}

template <typename XT, int P, int NRB, int EPI, typename WT>
hipError_t go(const MPK& k, size_t lds, unsigned grid, hipStream_t s) {
  auto fn = k_modeprod<XT, P, NRB, EPI, WT>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(NTH), lds, s, k);
  return hipGetLastError();
}

template <typename XT, int P, int EPI, typename WT>
hipError_t pick_nrb(const MPK& k, size_t lds, unsigned grid, hipStream_t s) {
  const uint32_t nrb = k.Mpad / 16;
  if (nrb <= 1) return go<XT, P, 1, EPI, WT>(k, lds, grid, s);
  if (nrb <= 2) return go<XT, P, 2, EPI, WT>(k, lds, grid, s);
  if (nrb <= 4) return go<XT, P, 4, EPI, WT>(k, lds, grid, s);
  if (nrb <= 8) return go<XT, P, 8, EPI, WT>(k, lds, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

size_t modeprod_lds_bytes(const ModeProd& mp) { return geometry(mp).lds; }

hipError_t launch_modeprod(const ModeProd& mp, int num_cu, hipStream_t s) {
  const Geo g = geometry(mp);
  if (g.Mpad > 128 || g.Kpad > 128) return hipErrorInvalidValue;
  MPK k;
  k.X = mp.X;
  k.M = mp.M;
  k.Y = mp.Y;
  k.W = mp.W;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.uS = mp.uS;
  k.ntiles = g.ntiles;
  k.tiles_per_a = g.tiles_per_a;
  k.A = mp.A;
  k.I = mp.I;
  k.B = mp.B;
  k.R = mp.R;
  k.Kin = g.Kin;
  k.Mout = g.Mout;
  k.Kpad = g.Kpad;
  k.Mpad = g.Mpad;
  k.TA = g.TA;
  k.wide = g.wide;
  k.lr = mp.lr;
  k.has_sparse = mp.has_sparse;
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * 8;
  if (grid > g.ntiles) grid = g.ntiles;
  if (grid < 1) grid = 1;
  const unsigned gr = (unsigned)grid;
  if (!mp.apply) {
    if (mp.P == 2) return pick_nrb<float, 2, 0, float>(k, g.lds, gr, s);
    switch (mp.in_dt) {
      case DT_F32: return pick_nrb<float, 1, 0, float>(k, g.lds, gr, s);
      case DT_F16: return pick_nrb<_Float16, 1, 0, float>(k, g.lds, gr, s);
      case DT_BF16: return pick_nrb<bf16_t, 1, 0, float>(k, g.lds, gr, s);
    }
    return hipErrorInvalidValue;
  }
  if (mp.P == 2) return pick_nrb<float, 2, 1, float>(k, g.lds, gr, s);
  switch (mp.w_dt) {
    case DT_F32: return pick_nrb<float, 1, 1, float>(k, g.lds, gr, s);
    case DT_F16: return pick_nrb<float, 1, 1, _Float16>(k, g.lds, gr, s);
    case DT_BF16: return pick_nrb<float, 1, 1, bf16_t>(k, g.lds, gr, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
