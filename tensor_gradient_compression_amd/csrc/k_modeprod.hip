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
// The work is HBM-bound (a few flops per byte), so the kernel is built around keeping
// HBM busy:
//  * a tile is TC = 64 * NCB GEMM columns (a, b). If B >= TC the tile is one a and TC
//    consecutive b: I row segments of TC*P contiguous values. Otherwise it is
//    floor(TC / B) consecutive a: one contiguous block.
//  * tiles move HBM -> LDS with global_load_lds_dwordx4 (16 bytes per lane straight
//    into LDS, no registers), double-buffered: the next tile's transfer is issued
//    before the current tile is multiplied and written out. The LDS copy keeps the
//    storage dtype and the tile's memory order; MFMA operand reads convert to fp32.
//  * the operand matrix M stays in LDS for the whole persistent workgroup. Four waves
//    each own NCB blocks of 16 columns and every 16-row block of the output;
//    v_mfma_f32_16x16x4_f32 accumulates in fp32.
//  * the output tile is staged in LDS (fp32) and written out in memory order with
//    16-byte stores.
// Epilogues: store (fp32 intermediate or core) or apply (last reconstruction):
// W <- round(W * decay - lr * (acc + N_S at Omega)); the W tile is transferred with the input
// tile. When the output tile is one contiguous element range its Omega entries are one
// contiguous range of the sorted Omega list, added into the staged tile; otherwise each
// output looks up its membership bit and rank (nullthought summary section 3: the
// sparse update is scatter-added after the low-rank reconstruction so that two full
// tensors never coexist; here the full Delta never exists at all).
// EPI: 0 stores, 1 applies, 2 applies and also stores the fp32 update Delta (after the
// sparse merge, before the weight rounding) to a test buffer.
// Tiles whose transfer is not 16-byte aligned fall back to plain loads and stores.
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int NTH = 256;    // 4 waves
constexpr int PADY = 4;     // LDS row padding (floats) of the staged fp32 output (wide)

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct MPK {
  const void* X;
  const float* M;
  float* Y;
  void* W;
  const uint64_t* mask;
  const uint32_t* rank;
  const float* uS;
  const uint32_t* omega;   // Omega ascending (contiguous-range merge)
  float* delta;            // EPI == 2: the fp32 update (after the sparse merge) is also stored here
  uint64_t kS;             // |Omega|
  uint64_t N;              // elements of the output tensor (apply)
  uint64_t ntiles;
  uint32_t tiles_per_a;
  uint32_t A, I, B, R;
  uint32_t Kin, Mout, Kpad, Mpad;
  uint32_t TA;
  uint32_t wide;
  uint32_t dma_in, dma_w;  // 16-byte transfers usable (alignment checked on the host)
  uint32_t vout;           // 16-byte output stores usable
  uint32_t off_x0, off_x1, off_y, off_w0, off_w1;   // LDS byte offsets of the buffers
  float lr;
  float decay;   // fp32(1 - lr * weight_decay): 1 exactly without decay
  int has_sparse;
};

template <typename T>
__device__ __forceinline__ float lds_ld(const unsigned char* base, uint32_t idx) {
  return to_f32(((const T*)base)[idx]);
}

struct TileGeo {
  uint64_t a0;
  uint32_t b0, ncol, nta;
  uint64_t base_in, base_out;    // value offsets (times P) of the tile's first value
  uint32_t len_in, len_out;      // valid values per row segment (wide) or block (narrow)
};

template <int TC, int P>
__device__ __forceinline__ TileGeo tile_geo(const MPK& k, uint64_t tile) {
  TileGeo g;
  if (k.wide) {
    g.a0 = tile / k.tiles_per_a;
    g.b0 = (uint32_t)(tile - g.a0 * k.tiles_per_a) * TC;
    g.ncol = k.B - g.b0 < (uint32_t)TC ? k.B - g.b0 : (uint32_t)TC;
    g.nta = 1;
    g.base_in = (g.a0 * k.I * k.B + g.b0) * P;
    g.base_out = (g.a0 * k.R * k.B + g.b0) * P;
    g.len_in = g.ncol * P;
    g.len_out = g.ncol * P;
  } else {
    g.a0 = tile * k.TA;
    g.b0 = 0;
    g.nta = (uint64_t)k.A - g.a0 < k.TA ? (uint32_t)((uint64_t)k.A - g.a0) : k.TA;
    g.ncol = g.nta * k.B;
    g.base_in = g.a0 * k.I * k.B * P;
    g.base_out = g.a0 * k.R * k.B * P;
    g.len_in = g.nta * k.I * k.B * P;
    g.len_out = g.nta * k.R * k.B * P;
  }
  return g;
}

// Issue the 16-byte HBM -> LDS transfers of one tile region: nseg segments of
// SEGLEN values (of type T) each, gstride values apart in memory, stored back to back in
// LDS at dst (SEGLEN = 0: one segment of `valid` values); only the first `valid` values
// of each segment are transferred. Each wave instruction writes 64 consecutive 16-byte
// LDS slots from a wave-uniform base; lanes without a granule are masked off.
template <typename T, uint32_t SEGLEN>
__device__ __forceinline__ void dma_tile(const T* src, uint32_t nseg, uint64_t gstride,
                                         uint32_t valid, unsigned char* dst) {
  constexpr uint32_t V = 16 / sizeof(T);
  constexpr uint32_t GPS = SEGLEN / V;             // granules per segment (wide)
  const uint32_t total = SEGLEN ? nseg * GPS : valid / V;
  const uint32_t vgps = valid / V;
  const int tid = threadIdx.x;
  const uint32_t wave_base = (uint32_t)(tid & ~63);
  for (uint32_t q0 = 0; q0 < total; q0 += NTH) {
    const uint32_t q = q0 + tid;
    unsigned char* lds = dst + (size_t)(q0 + wave_base) * 16;   // wave-uniform
    if (q < total) {
      uint32_t seg = 0, c = q;
      if (SEGLEN) {
        seg = q / GPS;
        c = q - seg * GPS;
      }
      if (c < vgps) {
        const T* p = src + seg * gstride + (uint64_t)c * V;
        __builtin_amdgcn_global_load_lds((const void*)p, (lds_void*)lds, 16, 0, 0);
      }
    }
  }
}

template <typename XT, int P, int NRB, int NCB, int EPI, typename WT>
__global__ void __launch_bounds__(NTH) k_modeprod(MPK k) {
  constexpr int TC = 64 * NCB;
  constexpr uint32_t TW = TC * P;                 // values per wide row segment
  constexpr int VO = (EPI == 0) ? 4 : 16 / (int)sizeof(WT);
  extern __shared__ float smem[];
  unsigned char* lds = (unsigned char*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t LDM = k.Kpad + 1;
  float* sM = smem;
  float* sY = (float*)(lds + k.off_y);
  const XT* __restrict__ X = (const XT*)k.X;

  for (uint32_t idx = tid; idx < k.Mpad * k.Kpad; idx += NTH) {
    const uint32_t jj = idx / k.Kpad, kk = idx - jj * k.Kpad;
    sM[jj * LDM + kk] = (jj < k.Mout && kk < k.Kin) ? k.M[(uint64_t)jj * k.Kin + kk] : 0.0f;
  }

  // LDS copies are in memory order without padding: wide rows of TW values.
  const uint32_t rs_in = k.wide ? TW : k.B * P;
  const uint32_t rs_y = k.wide ? TW + PADY : k.B * P;
  const uint32_t rs_w = k.wide ? TW : k.B * P;
  const uint32_t blk_in = k.I * k.B * P;
  const uint32_t blk_out = k.R * k.B * P;

  auto can_dma_in = [&](const TileGeo& g) {
    return k.dma_in && (g.len_in * sizeof(XT)) % 16 == 0;
  };
  auto can_dma_w = [&](const TileGeo& g) {
    return EPI >= 1 && k.dma_w && (g.len_out * sizeof(WT)) % 16 == 0;
  };
  auto issue = [&](const TileGeo& g, int buf) {
    unsigned char* dx = lds + (buf ? k.off_x1 : k.off_x0);
    if (can_dma_in(g)) {
      if (k.wide)
        dma_tile<XT, TW>(X + g.base_in, k.I, (uint64_t)k.B * P, g.len_in, dx);
      else
        dma_tile<XT, 0>(X + g.base_in, 1, 0, g.len_in, dx);
    }
    if (EPI >= 1 && can_dma_w(g)) {
      unsigned char* dw = lds + (buf ? k.off_w1 : k.off_w0);
      const WT* W = (const WT*)k.W;
      if (k.wide)
        dma_tile<WT, TW>(W + g.base_out, k.R, (uint64_t)k.B * P, g.len_out, dw);
      else
        dma_tile<WT, 0>(W + g.base_out, 1, 0, g.len_out, dw);
    }
  };

  // Narrow apply: the tile's outputs are one contiguous element range, so its Omega
  // entries are one contiguous range [j0, j1) of the sorted list. The range of the next
  // tile is looked up when its transfer is issued, and the current tile's (index,
  // update) pairs are loaded into registers before the multiply.
  const bool merged = (EPI >= 1) && k.has_sparse && !k.wide;
  constexpr int NSR = 2;                         // Omega entries per thread in registers
  // Omega rank of element e (how many Omega entries lie below e). e is uniform over the
  // workgroup and mask/rank are read-only here, so the words come in by scalar loads:
  // those retire on lgkmcnt, whereas a vector load would retire on vmcnt behind the
  // next tile's transfer and make the double buffering synchronous.
  auto rank_of = [&](uint64_t e) -> uint64_t {
    if (e >= k.N) return k.kS;
    const uint64_t w = e >> 6;
    const uint64_t word = ((const __attribute__((address_space(4))) uint64_t*)k.mask)[w];
    const uint32_t base = ((const __attribute__((address_space(4))) uint32_t*)k.rank)[w];
    return base + (uint64_t)__popcll(word & ((1ull << (e & 63)) - 1ull));
  };
  uint64_t jc0 = 0, jc1 = 0, jn0 = 0, jn1 = 0;

  uint64_t tile = blockIdx.x;
  int cur = 0;
  TileGeo g = tile_geo<TC, P>(k, tile < k.ntiles ? tile : 0);
  if (tile < k.ntiles) {
    issue(g, cur);
    if (merged) {
      jc0 = rank_of(g.base_out / P);
      jc1 = rank_of((g.base_out + g.len_out) / P);
    }
  }

  // vmcnt counts both the transfers and the stores of this thread. Waiting right
  // before the stream-out (not at the top of the loop) lets the next tile's transfer
  // overlap the multiply and lets this tile's stores drain during the next iteration.
  __builtin_amdgcn_s_waitcnt(0);
  for (; tile < k.ntiles; tile += gridDim.x) {
    const uint64_t next = tile + gridDim.x;
    lds_barrier();                 // every thread's transfers visible; buffers free
    const TileGeo gc = g;
    unsigned char* bx = lds + (cur ? k.off_x1 : k.off_x0);
    unsigned char* bw = lds + (cur ? k.off_w1 : k.off_w0);
    if (next < k.ntiles) {
      g = tile_geo<TC, P>(k, next);
      issue(g, cur ^ 1);
      if (merged) {
        jn0 = rank_of(g.base_out / P);
        jn1 = rank_of((g.base_out + g.len_out) / P);
      }
    }
    uint32_t om_r[NSR];
    float us_r[NSR][P];
    if (merged) {
#pragma unroll
      for (int i = 0; i < NSR; ++i) {
        const uint64_t j = jc0 + tid + (uint64_t)NTH * i;
        if (j < jc1) {
          om_r[i] = k.omega[j];
#pragma unroll
          for (int p = 0; p < P; ++p) us_r[i][p] = k.uS[j * P + p];
        }
      }
    }
    // plain loads for tiles the 16-byte transfer cannot cover
    bool filled = false;
    if (!can_dma_in(gc)) {
      XT* d = (XT*)bx;
      if (k.wide) {
        for (uint32_t idx = tid; idx < k.I * TW; idx += NTH) {
          const uint32_t i = idx / TW, e = idx - i * TW;
          if (e < gc.len_in) d[i * TW + e] = X[gc.base_in + (uint64_t)i * k.B * P + e];
        }
      } else {
        for (uint32_t idx = tid; idx < gc.len_in; idx += NTH) d[idx] = X[gc.base_in + idx];
      }
      filled = true;
    }
    if (EPI >= 1 && !can_dma_w(gc)) {
      WT* d = (WT*)bw;
      const WT* W = (const WT*)k.W;
      if (k.wide) {
        for (uint32_t idx = tid; idx < k.R * TW; idx += NTH) {
          const uint32_t j = idx / TW, e = idx - j * TW;
          if (e < gc.len_out) d[j * TW + e] = W[gc.base_out + (uint64_t)j * k.B * P + e];
        }
      } else {
        for (uint32_t idx = tid; idx < gc.len_out; idx += NTH) d[idx] = W[gc.base_out + idx];
      }
      filled = true;
    }
    if (filled) lds_barrier();

    f4 acc[NCB][NRB];
    uint32_t cb_in[NCB], cb_y[NCB];
    bool cvalid[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const uint32_t col = (wave + 4 * c) * 16 + (lane & 15);
      cvalid[c] = col < gc.ncol;
      cb_in[c] = 0;
      cb_y[c] = 0;
      if (cvalid[c]) {
        if (k.wide) {
          cb_in[c] = col * P;
          cb_y[c] = col * P;
        } else {
          const uint32_t ca = col / k.B, cbb = col - ca * k.B;
          cb_in[c] = ca * blk_in + cbb * P;
          cb_y[c] = ca * blk_out + cbb * P;
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) acc[c][rb] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t nks = k.Kpad >> 2;
    for (uint32_t ks = 0; ks < nks; ++ks) {
      const uint32_t kk = ks * 4 + (lane >> 4);
      const bool kv = kk < k.Kin;
      const uint32_t roff = (kk / P) * rs_in + (kk % P);
      float av[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        av[rb] = ((uint32_t)rb * 16 < k.Mpad) ? sM[(rb * 16 + (lane & 15)) * LDM + kk] : 0.0f;
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const float bv = (cvalid[c] && kv) ? lds_ld<XT>(bx, cb_in[c] + roff) : 0.0f;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          if ((uint32_t)rb * 16 < k.Mpad)
            acc[c][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[rb], bv, acc[c][rb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      if (!cvalid[c]) continue;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t jj = rb * 16 + 4 * (lane >> 4) + v;
          if (jj < k.Mout) sY[cb_y[c] + (jj / P) * rs_y + (jj % P)] = acc[c][rb][v];
        }
      }
    }
    lds_barrier();
    if (merged) {
      const uint64_t e_lo = gc.base_out / P;
#pragma unroll
      for (int i = 0; i < NSR; ++i) {
        const uint64_t j = jc0 + tid + (uint64_t)NTH * i;
        if (j < jc1) {
          const uint32_t loc = (uint32_t)(om_r[i] - e_lo) * P;
#pragma unroll
          for (int p = 0; p < P; ++p) sY[loc + p] = sY[loc + p] + us_r[i][p];
        }
      }
      for (uint64_t j = jc0 + (uint64_t)NTH * NSR + tid; j < jc1; j += NTH) {
        const uint32_t loc = (uint32_t)(k.omega[j] - e_lo) * P;
#pragma unroll
        for (int p = 0; p < P; ++p) sY[loc + p] = sY[loc + p] + k.uS[j * P + p];
      }
      lds_barrier();
    }

    // this thread's transfer of the next tile has landed (it is read after the next
    // barrier), and the previous tile's stores have completed
    __builtin_amdgcn_s_waitcnt(0);

    // stream the output tile out in memory order
    auto merge = [&](uint64_t gi, float d) -> float {
      if (k.has_sparse && !merged) {
        const uint64_t e = gi / P;
        const uint64_t word = k.mask[e >> 6];
        if ((word >> (e & 63)) & 1ull) {
          const uint64_t jpos = omega_rank(k.mask, k.rank, e, word);
          d = d + k.uS[jpos * P + (gi % P)];
        }
      }
      return d;
    };
    const uint32_t nseg_o = k.wide ? k.R : 1u;
    const uint32_t seg_o = k.wide ? TW : gc.len_out;          // values per segment slot
    if (k.vout && (gc.len_out % VO) == 0) {
      constexpr uint32_t VPS_W = TW / VO;                      // vectors per wide row
      const uint32_t nvec = k.wide ? k.R * VPS_W : gc.len_out / VO;
      for (uint32_t q = tid; q < nvec; q += NTH) {
        uint32_t seg = 0, off = q * VO;
        if (k.wide) {
          seg = q / VPS_W;
          off = (q - seg * VPS_W) * VO;
          if (off >= gc.len_out) continue;
        }
        const uint64_t g0 = gc.base_out + (uint64_t)seg * k.B * P + off;
        const float* ys = sY + seg * rs_y + off;               // 16-byte aligned
        float d[VO];
#pragma unroll
        for (int e = 0; e < VO; e += 4) {
          const float4 t = *(const float4*)(ys + e);
          d[e] = t.x; d[e + 1] = t.y; d[e + 2] = t.z; d[e + 3] = t.w;
        }
        if (EPI == 0) {
          *(float4*)&k.Y[g0] = make_float4(d[0], d[1], d[2], d[3]);
        } else {
          const uint4 wraw = *(const uint4*)(bw + (size_t)(seg * rs_w + off) * sizeof(WT));
          const WT* wsrc = (const WT*)&wraw;
          WT wv[VO];
#pragma unroll
          for (int e = 0; e < VO; ++e) {
            d[e] = merge(g0 + e, d[e]);
            wv[e] = from_f32<WT>(to_f32(wsrc[e]) * k.decay - k.lr * d[e]);
          }
          *(uint4*)((WT*)k.W + g0) = *(const uint4*)wv;
          if (EPI == 2) {
#pragma unroll
            for (int e = 0; e < VO; e += 4)
              *(float4*)&k.delta[g0 + e] = make_float4(d[e], d[e + 1], d[e + 2], d[e + 3]);
          }
        }
      }
    } else {
      for (uint32_t q = tid; q < nseg_o * seg_o; q += NTH) {
        const uint32_t seg = q / seg_o, e = q - seg * seg_o;
        if (e >= gc.len_out) continue;
        const uint64_t gi = gc.base_out + (uint64_t)seg * k.B * P + e;
        const float d = sY[seg * rs_y + e];
        if (EPI == 0) {
          k.Y[gi] = d;
        } else {
          const float w = lds_ld<WT>(bw, seg * rs_w + e);
          const float dm = merge(gi, d);
          ((WT*)k.W)[gi] = from_f32<WT>(w * k.decay - k.lr * dm);
          if (EPI == 2) k.delta[gi] = dm;
        }
      }
    }
    cur ^= 1;
    jc0 = jn0;
    jc1 = jn1;
  }
  __builtin_amdgcn_s_waitcnt(0);
}

struct Geo {
  uint32_t Kin, Mout, Kpad, Mpad, wide, TA, tiles_per_a, ncb, dma_in, dma_w, vout;
  uint32_t off_x0, off_x1, off_y, off_w0, off_w1;
  uint64_t ntiles;
  size_t lds;
};

size_t esize_of(int dt) { return dt == DT_F32 ? 4 : 2; }

Geo geometry_for(const ModeProd& mp, uint32_t ncb) {
  Geo g;
  const uint32_t TC = 64 * ncb;
  const uint64_t P = mp.P;
  g.ncb = ncb;
  g.Kin = mp.I * mp.P;
  g.Mout = mp.R * mp.P;
  g.Kpad = (g.Kin + 3u) & ~3u;
  g.Mpad = (g.Mout + 15u) & ~15u;
  g.wide = mp.B >= TC;
  if (g.wide) {
    g.tiles_per_a = (mp.B + TC - 1) / TC;
    g.TA = 1;
    g.ntiles = (uint64_t)mp.A * g.tiles_per_a;
  } else {
    g.tiles_per_a = 1;
    g.TA = TC / mp.B;
    g.ntiles = ((uint64_t)mp.A + g.TA - 1) / g.TA;
  }
  const size_t esx = (mp.P == 2) ? 4 : esize_of(mp.in_dt);
  const size_t esw = mp.apply ? ((mp.P == 2) ? 4 : esize_of(mp.w_dt)) : 4;
  // 16-byte transfers: the buffer, every tile start and every row start 16-byte aligned
  auto aligned = [&](uint64_t rows, size_t es, const void* base) {
    if (((uintptr_t)base) % 16) return false;
    if (g.wide)
      return ((mp.B * P * es) % 16 == 0) && ((rows * mp.B * P * es) % 16 == 0) &&
             ((TC * P * es) % 16 == 0);
    return ((uint64_t)g.TA * rows * mp.B * P * es) % 16 == 0;
  };
  g.dma_in = aligned(mp.I, esx, mp.X) ? 1 : 0;
  g.dma_w = mp.apply ? (aligned(mp.R, esw, mp.W) ? 1 : 0) : 0;
  g.vout = aligned(mp.R, esw, mp.apply ? mp.W : (const void*)mp.Y) ? 1 : 0;
  const size_t sm = ((size_t)g.Mpad * (g.Kpad + 1) * 4 + 15) & ~(size_t)15;
  const size_t tin =
      g.wide ? (size_t)mp.I * TC * P * esx : (size_t)g.TA * mp.I * mp.B * P * esx;
  const size_t ty = g.wide ? (size_t)mp.R * (TC * P + PADY) * 4
                           : (size_t)g.TA * mp.R * mp.B * P * 4;
  const size_t tw = g.wide ? (size_t)mp.R * TC * P * esw : (size_t)g.TA * mp.R * mp.B * P * esw;
  auto up = [](size_t x) { return (x + 15) & ~(size_t)15; };
  size_t off = sm;
  g.off_x0 = (uint32_t)off; off += up(tin);
  g.off_x1 = (uint32_t)off; off += up(tin);
  g.off_y = (uint32_t)off; off += (ty + 15) & ~(size_t)15;
  g.off_w0 = (uint32_t)off; off += mp.apply ? up(tw) : 0;
  g.off_w1 = (uint32_t)off; off += mp.apply ? up(tw) : 0;
  g.lds = off;
  return g;
}

// Widest tile (up to 256 columns) whose LDS footprint stays <= 52 KB (3 workgroups per
// CU) and whose accumulators stay <= 64 registers; else 64 columns.
Geo geometry(const ModeProd& mp) {
  if (mp.force_ncb) return geometry_for(mp, (uint32_t)mp.force_ncb);
  const uint32_t Mpad = ((mp.R * mp.P) + 15u) & ~15u;
  const uint32_t nrb = Mpad / 16;
  for (uint32_t ncb : {4u, 2u}) {
    if (nrb * ncb * 4 > 64) continue;
    Geo g = geometry_for(mp, ncb);
    if (g.lds <= 52 * 1024) return g;
  }
  return geometry_for(mp, 1);
}

// `grid` is the number of CUs; the launch puts one resident round of workgroups on
// each (as many as the kernel's registers and LDS let a CU hold), capped by the tiles.
template <typename XT, int P, int NRB, int NCB, int EPI, typename WT>
hipError_t go(const MPK& k, size_t lds, unsigned grid, hipStream_t s) {
  auto fn = k_modeprod<XT, P, NRB, NCB, EPI, WT>;
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

template <typename XT, int P, int NCB, int EPI, typename WT>
hipError_t pick_nrb(const MPK& k, size_t lds, unsigned grid, hipStream_t s) {
  const uint32_t nrb = k.Mpad / 16;
  if (nrb <= 1) return go<XT, P, 1, NCB, EPI, WT>(k, lds, grid, s);
  if (nrb <= 2) return go<XT, P, 2, NCB, EPI, WT>(k, lds, grid, s);
  if (nrb <= 4) return go<XT, P, 4, NCB, EPI, WT>(k, lds, grid, s);
  if constexpr (NCB <= 2) {
    if (nrb <= 8) return go<XT, P, 8, NCB, EPI, WT>(k, lds, grid, s);
  }
  return hipErrorInvalidValue;
}

template <typename XT, int P, int EPI, typename WT>
hipError_t pick_ncb(const MPK& k, uint32_t ncb, size_t lds, unsigned grid, hipStream_t s) {
  if (ncb == 4) return pick_nrb<XT, P, 4, EPI, WT>(k, lds, grid, s);
  if (ncb == 2) return pick_nrb<XT, P, 2, EPI, WT>(k, lds, grid, s);
  return pick_nrb<XT, P, 1, EPI, WT>(k, lds, grid, s);
}

}  // namespace

size_t modeprod_lds_bytes(const ModeProd& mp) { return geometry(mp).lds; }

hipError_t launch_modeprod(const ModeProd& mp, int num_cu, hipStream_t s) {
  const Geo g = geometry(mp);
  if (g.Mpad > 128 || g.Kpad > 128) return hipErrorInvalidValue;
  if (g.lds > 160 * 1024) return hipErrorInvalidValue;
  MPK k;
  k.X = mp.X;
  k.M = mp.M;
  k.Y = mp.Y;
  k.W = mp.W;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.uS = mp.uS;
  k.omega = mp.omega;
  k.delta = mp.delta;
  k.kS = mp.kS;
  k.N = (uint64_t)mp.A * mp.R * mp.B;
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
  k.dma_in = g.dma_in;
  k.dma_w = g.dma_w;
  k.vout = g.vout;
  k.off_x0 = g.off_x0;
  k.off_x1 = g.off_x1;
  k.off_y = g.off_y;
  k.off_w0 = g.off_w0;
  k.off_w1 = g.off_w1;
  k.lr = mp.lr;
  k.decay = mp.decay;
  k.has_sparse = mp.has_sparse;
  // persistent grid: one resident round per CU (sized in go())
  const unsigned gr = (unsigned)(num_cu > 0 ? num_cu : 256);
  const uint32_t ncb = g.ncb;
  if (!mp.apply) {
    if (mp.P == 2) return pick_ncb<float, 2, 0, float>(k, ncb, g.lds, gr, s);
    switch (mp.in_dt) {
      case DT_F32: return pick_ncb<float, 1, 0, float>(k, ncb, g.lds, gr, s);
      case DT_F16: return pick_ncb<_Float16, 1, 0, float>(k, ncb, g.lds, gr, s);
      case DT_BF16: return pick_ncb<bf16_t, 1, 0, float>(k, ncb, g.lds, gr, s);
    }
    return hipErrorInvalidValue;
  }
  if (mp.delta) {
    if (mp.P == 2) return pick_ncb<float, 2, 2, float>(k, ncb, g.lds, gr, s);
    switch (mp.w_dt) {
      case DT_F32: return pick_ncb<float, 1, 2, float>(k, ncb, g.lds, gr, s);
      case DT_F16: return pick_ncb<float, 1, 2, _Float16>(k, ncb, g.lds, gr, s);
      case DT_BF16: return pick_ncb<float, 1, 2, bf16_t>(k, ncb, g.lds, gr, s);
    }
    return hipErrorInvalidValue;
  }
  if (mp.P == 2) return pick_ncb<float, 2, 1, float>(k, ncb, g.lds, gr, s);
  switch (mp.w_dt) {
    case DT_F32: return pick_ncb<float, 1, 1, float>(k, ncb, g.lds, gr, s);
    case DT_F16: return pick_ncb<float, 1, 1, _Float16>(k, ncb, g.lds, gr, s);
    case DT_BF16: return pick_ncb<float, 1, 1, bf16_t>(k, ncb, g.lds, gr, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
