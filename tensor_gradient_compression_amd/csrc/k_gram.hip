// Mode-n Gram matrices of the residual for the HOSVD refresh.
//
// HOSVD factors are the leading eigenvectors of Gram_n = R_(n) R_(n)^H, R = G with
// Omega zeroed (pith.science "What carries the argument": Tucker (higher-order SVD)
// factors; nullthought summary section 3: Tucker decomposition of the residual left
// after the sparse part is extracted). The Gram does not depend on the column order of
// the unfolding, so each launch works on the (A, I, B, P) view of one mode and sums
// over all (a, b) columns.
//
// Complex data is handled as the real stacked Gram of rows kk = i*P + p (size
// (I*P)^2); the eigen kernel forms the Hermitian Gram from its four I x I blocks.
//
// Each workgroup owns a contiguous range of 64-column tiles (split-K). A tile is
// staged in LDS (fp32; entries in Omega read as zero via the membership bitmask, so
// the gradient is never modified), v_mfma_f32_16x16x4_f32 accumulates the tile's
// 64-term sums in fp32 for the upper-triangle 16 x 16 blocks, and every tile result is
// added to fp64 accumulators. Each workgroup writes its fp64 partial (both triangles);
// a second kernel sums the partials in a fixed order, so the result is deterministic
// run to run.
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int TC = 64;
constexpr int NTH = 256;
constexpr int PADW = 4;

typedef float f4 __attribute__((ext_vector_type(4)));

struct GK {
  const void* X;
  const uint64_t* mask;
  double* partial;
  uint64_t ntiles, tiles_per_blk;
  uint32_t tiles_per_a;
  uint32_t A, I, B;
  uint32_t Kin, nb;   // Kin = I*P; nb = ceil(Kin / 16)
  uint32_t TA, wide;
  uint32_t ob0, ob1;  // the output blocks of this launch: ob0 <= block < ob1 of the
                      // nb (nb + 1) / 2 upper-triangle blocks (row-major)
};

// NOB = output 16x16 blocks per wave (nb (nb + 1) / 2 blocks over 4 waves).
template <typename XT, int P, int NOB>
__global__ void __launch_bounds__(NTH) k_gram(GK k) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t* scol = (uint32_t*)smem;   // LDS offset of each tile column
  float* sX = smem + TC;
  const XT* __restrict__ X = (const XT*)k.X;
  constexpr uint32_t TW = TC * P;
  constexpr uint32_t TWSH = (P == 1) ? 6 : 7;
  const uint32_t rs = k.wide ? TW + PADW : k.B * P;
  const uint32_t blk = k.I * k.B * P;
  f4 acc[NOB];
  double dacc[NOB][4];
  // this wave's upper-triangle output blocks (rb <= cb); rb = -1: none
  int brb[NOB], bcb[NOB];
#pragma unroll
  for (int q = 0; q < NOB; ++q) {
    acc[q] = f4{0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < 4; ++v) dacc[q][v] = 0.0;
    const uint32_t ob = k.ob0 + wave + 4 * q;
    brb[q] = -1;
    bcb[q] = 0;
    if (ob < k.ob1) {
      uint32_t t = ob, rb = 0;
      while (t >= k.nb - rb) {
        t -= k.nb - rb;
        ++rb;
      }
      brb[q] = (int)rb;
      bcb[q] = (int)(rb + t);
    }
  }

  const uint64_t t0 = (uint64_t)blockIdx.x * k.tiles_per_blk;
  uint64_t t1 = t0 + k.tiles_per_blk;
  if (t1 > k.ntiles) t1 = k.ntiles;
  for (uint64_t tile = t0; tile < t1; ++tile) {
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
    __syncthreads();
    if (tid < TC) {
      uint32_t off = 0;
      if ((uint32_t)tid < ncol) {
        if (k.wide) {
          off = tid * P;
        } else {
          const uint32_t ca = tid / k.B;
          off = ca * blk + (tid - ca * k.B) * P;
        }
      }
      scol[tid] = off;
    }
    auto ld = [&](uint64_t g) -> float {
      float v = to_f32(X[g]);
      if (k.mask) {
        const uint64_t e = g / P;
        if ((k.mask[e >> 6] >> (e & 63)) & 1ull) v = 0.0f;
      }
      return v;
    };
    if (k.wide) {
      const uint32_t rowlen = ncol * P;
      for (uint32_t idx = tid; idx < k.I * TW; idx += NTH) {
        const uint32_t i = idx >> TWSH, e = idx & (TW - 1);
        if (e < rowlen) sX[i * rs + e] = ld(((a0 * k.I + i) * k.B + b0) * P + e);
      }
    } else {
      const uint32_t n = nta * blk;
      const uint64_t base = a0 * blk;
      for (uint32_t idx = tid; idx < n; idx += NTH) sX[idx] = ld(base + idx);
    }
    __syncthreads();

    for (uint32_t ks = 0; ks < TC / 4; ++ks) {
      const uint32_t c = ks * 4 + (lane >> 4);
      const bool cv = c < ncol;
      const uint32_t cbase = scol[c];
#pragma unroll
      for (int q = 0; q < NOB; ++q) {
        if (brb[q] >= 0) {
          const uint32_t rb = (uint32_t)brb[q], cb = (uint32_t)bcb[q];
          const uint32_t ka = rb * 16 + (lane & 15), kb = cb * 16 + (lane & 15);
          float av = 0.0f, bv = 0.0f;
          if (cv && ka < k.Kin) av = sX[cbase + (ka / P) * rs + (ka % P)];
          if (cv && kb < k.Kin) bv = sX[cbase + (kb / P) * rs + (kb % P)];
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[q], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NOB; ++q) {
      for (int v = 0; v < 4; ++v) dacc[q][v] += (double)acc[q][v];
      acc[q] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // the partial is written symmetric: block (rb, cb) and its transpose
  double* out = k.partial + (uint64_t)blockIdx.x * k.Kin * k.Kin;
#pragma unroll
  for (int q = 0; q < NOB; ++q) {
    if (brb[q] >= 0) {
      const uint32_t rb = (uint32_t)brb[q], cb = (uint32_t)bcb[q];
      const uint32_t colj = cb * 16 + (lane & 15);
      for (int v = 0; v < 4; ++v) {
        const uint32_t rowi = rb * 16 + 4 * (lane >> 4) + v;
        if (rowi < k.Kin && colj < k.Kin) {
          out[rowi * k.Kin + colj] = dacc[q][v];
          if (rb != cb) out[colj * k.Kin + rowi] = dacc[q][v];
        }
      }
    }
  }
}

// Fixed-order two-stage sum of the workgroup partials: stage 1 sums group g's
// contiguous range of partials for every entry, stage 2 sums the groups in order.
constexpr uint32_t RGROUPS = 32;
__global__ void k_gram_reduce1(const double* __restrict__ partial, uint32_t nblk, uint32_t n2,
                               double* __restrict__ stage) {
  const uint32_t x = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t g = blockIdx.y;
  if (x >= n2) return;
  const uint32_t per = (nblk + RGROUPS - 1) / RGROUPS;
  const uint32_t w0 = g * per, w1 = w0 + per < nblk ? w0 + per : nblk;
  double s = 0.0;
  for (uint32_t w = w0; w < w1; ++w) s += partial[(uint64_t)w * n2 + x];
  stage[(uint64_t)g * n2 + x] = s;
}
__global__ void k_gram_reduce2(const double* __restrict__ stage, uint32_t n2,
                               double* __restrict__ out) {
  const uint32_t x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= n2) return;
  double s = 0.0;
  for (uint32_t g = 0; g < RGROUPS; ++g) s += stage[(uint64_t)g * n2 + x];
  out[x] = s;
}

struct GGeo {
  uint32_t Kin, nb, wide, TA, tiles_per_a;
  uint64_t ntiles;
  size_t lds;
};

GGeo ggeo(const GramArgs& g) {
  GGeo r;
  r.Kin = g.I * g.P;
  r.nb = (r.Kin + 15) / 16;
  r.wide = g.B >= (uint32_t)TC;
  if (r.wide) {
    r.tiles_per_a = (g.B + TC - 1) / TC;
    r.TA = 1;
    r.ntiles = (uint64_t)g.A * r.tiles_per_a;
  } else {
    r.tiles_per_a = 1;
    r.TA = TC / g.B;
    r.ntiles = ((uint64_t)g.A + r.TA - 1) / r.TA;
  }
  const size_t tin = r.wide ? (size_t)g.I * (TC * g.P + PADW) : (size_t)r.TA * g.I * g.B * g.P;
  r.lds = (TC + tin) * sizeof(float);
  return r;
}

template <typename XT, int P, int NOB>
hipError_t gogram(const GK& k, size_t lds, unsigned grid, hipStream_t s) {
  auto fn = k_gram<XT, P, NOB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(NTH), lds, s, k);
  return hipGetLastError();
}

// More than 64 output blocks (I P > 128): launches of 64 blocks each (16 a wave), every
// one re-reading the tiles; each writes its own entries of the same partial sums.
template <typename XT, int P>
hipError_t pick_nob(const GK& k, size_t lds, unsigned grid, hipStream_t s) {
  const uint32_t nblocks = k.nb * (k.nb + 1) / 2;   // upper-triangle blocks
  const uint32_t per_wave = (nblocks + 3) / 4;
  GK kk = k;
  kk.ob0 = 0;
  kk.ob1 = nblocks;
  if (per_wave <= 1) return gogram<XT, P, 1>(kk, lds, grid, s);
  if (per_wave <= 4) return gogram<XT, P, 4>(kk, lds, grid, s);
  for (uint32_t b0 = 0; b0 < nblocks; b0 += 64) {
    kk.ob0 = b0;
    kk.ob1 = b0 + 64 < nblocks ? b0 + 64 : nblocks;
    const hipError_t e = gogram<XT, P, 16>(kk, lds, grid, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- 16-bit real data
// bf16 and fp16 products are exact in fp32, so for these the Gram runs on the
// 16x16x32 MFMAs (v_mfma_f32_16x16x32_bf16 / _f16): lane l supplies row l % 16 of a
// 16-row block at the 8 consecutive k = 8 (l / 16) .. + 7, as both the A and the B
// operand, and block (rb, cb) of the Gram is mfma(fragment rb, fragment cb). Only the
// blocks with rb <= cb are formed; the partial is written symmetric.
//
// Tiles move HBM -> LDS with 16-byte global_load_lds transfers, double buffered, in
// a persistent grid (tile = blockIdx.x, + gridDim.x, ...). Two tile forms:
//   wide   (B % 8 == 0, B >= 32): one a, 128 consecutive b, all I rows. The K index is
//          b. Row r's 16-byte chunk c sits at LDS chunk r * 16 + (c ^ (r % 16)), so the
//          transfer stays contiguous in LDS (each lane fetches the chunk that belongs
//          in its slot) and the 16 rows a fragment read touches fall in distinct banks.
//   narrow (I * B small): TA whole slabs, contiguous. K runs over (a, b), element
//          offset a * I * B + r * B + b; fragments are read 16 bits at a time.
// Both forms move 16-byte pieces that start on a multiple of 8 elements, so each piece
// has one byte of Omega's membership bitmask. With a mask, the wave that transfers a
// piece also transfers the dwords holding its byte into LDS; once both have landed the
// thread clears the piece's Omega entries (+0 is the zero pattern of both formats),
// before the barrier that publishes the tile, so the Gram is that of the residual while
// the gradient is only read.
// Each wave sums 8 k-steps in fp32 (at most 256 exact products per sum) before adding
// into fp64; at the end the waves' fp64 sums are combined in wave order, so results are
// deterministic run to run.
constexpr int G16_NTH = 256;
constexpr uint32_t G16_TB = 128;           // wide tiles: columns (b) per tile
constexpr uint32_t G16_NARROW = 16384;     // narrow tiles: at most this many elements
constexpr uint32_t G16_FLUSH = 8;          // k-steps per fp32 partial sum
constexpr int G16_WGS_PER_CU = 3;
// transfer instructions per thread and tile, at most: wide tiles 64 rows x 16 pieces,
// narrow tiles G16_NARROW / 8 pieces, over G16_NTH threads
constexpr int G16_PIECES = (int)(G16_NARROW / 8 / G16_NTH);
constexpr uint32_t G16_MREG = 80;   // bytes of mask dwords per (instruction, wave)
static_assert(64 * (G16_TB / 8) <= G16_PIECES * G16_NTH, "wide tile pieces");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct G16K {
  const uint16_t* X;
  const uint8_t* mask8;   // Omega's bitmask as bytes (element e: bit e % 8 of byte e / 8), or NULL
  uint32_t mask_off;      // LDS byte offset of the two buffers' mask-byte areas
  double* partial;
  uint64_t ntiles;
  uint32_t A, I, B;
  uint32_t wide;
  uint32_t tiles_per_a;   // wide
  uint32_t TA;            // narrow: slabs per tile
  uint32_t buf_bytes;     // one LDS tile buffer (multiple of 16)
  float invB;             // narrow: 1/B rounded to fp32
};

template <bool BF>
__device__ __forceinline__ f4 mfma32(const u16x8& a, const u16x8& b, const f4& c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Upper-triangle block q (row-major: (0,0), (0,1), ..., (1,1), ...) of an NB x NB grid.
__host__ __device__ constexpr int blk_rb(int NB, int q) {
  int rb = 0;
  while (q >= NB - rb) {
    q -= NB - rb;
    ++rb;
  }
  return rb;
}
__host__ __device__ constexpr int blk_cb(int NB, int q) {
  int rb = 0;
  while (q >= NB - rb) {
    q -= NB - rb;
    ++rb;
  }
  return rb + q;
}

// Work split of the four waves. KS: every wave forms all blocks over every fourth
// k-step (used for NB <= 2, and for NB = 3 on slab tiles, whose fragments are read 16
// bits at a time: the four waves then read each fragment once instead of each reading
// the rows of its own blocks; measured 270 -> 119 us for (48 x 25) slabs). Otherwise
// wave W forms blocks W, W + 4, ... (at most 3) over every k-step, which needs fewer
// registers (three workgroups per CU on the wide tiles).
template <int NB, bool KS>
struct G16Split {
  static constexpr int NBLK = NB * (NB + 1) / 2;
  static constexpr bool KSPLIT = KS;
  static constexpr int MAXB = KSPLIT ? NBLK : (NBLK + 3) / 4;
  __host__ __device__ static constexpr int count(int W) {
    return KSPLIT ? NBLK : (NBLK > W ? (NBLK - W + 3) / 4 : 0);
  }
  __host__ __device__ static constexpr int q(int W, int m) { return KSPLIT ? m : W + 4 * m; }
};

template <int NB, bool KS>
__host__ __device__ constexpr bool row_used(int W, int rb) {
  using S = G16Split<NB, KS>;
  for (int m = 0; m < S::count(W); ++m)
    if (blk_rb(NB, S::q(W, m)) == rb || blk_cb(NB, S::q(W, m)) == rb) return true;
  return false;
}

// One k-step of wave W: read the fragments its blocks use, then one MFMA per block.
// Template recursion keeps every block and fragment index a compile-time constant.
template <int NB, bool KS, int W, int RB, class LD>
__device__ __forceinline__ void g16_load(u16x8* fr, LD& ld) {
  if constexpr (RB < NB) {
    if constexpr (row_used<NB, KS>(W, RB)) fr[RB] = ld(RB);
    g16_load<NB, KS, W, RB + 1>(fr, ld);
  }
}
template <bool BF, int NB, bool KS, int W, int M>
__device__ __forceinline__ void g16_mfma(f4* acc, const u16x8* fr) {
  if constexpr (M < G16Split<NB, KS>::count(W)) {
    constexpr int qq = G16Split<NB, KS>::q(W, M);
    constexpr int rb = blk_rb(NB, qq), cb = blk_cb(NB, qq);
    acc[M] = mfma32<BF>(fr[rb], fr[cb], acc[M]);
    g16_mfma<BF, NB, KS, W, M + 1>(acc, fr);
  }
}
template <bool BF, int NB, bool KS, int W, class LD>
__device__ __forceinline__ void g16_step(f4* acc, LD&& ld) {
  u16x8 fr[NB];
  g16_load<NB, KS, W, 0>(fr, ld);
  g16_mfma<BF, NB, KS, W, 0>(acc, fr);
}

// Clear the elements of a staged 16-byte piece (8 16-bit values) whose bits are set in
// its mask byte b.
__device__ __forceinline__ void clear_piece(unsigned char* piece, uint32_t b) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t keep;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    keep[i] = (((b >> (2 * i)) & 1u) ? 0u : 0x0000FFFFu) |
              (((b >> (2 * i + 1)) & 1u) ? 0u : 0xFFFF0000u);
  *(u32x4_t*)piece = *(const u32x4_t*)piece & keep;
}

template <bool BF, int NB, bool KS>
__global__ void __launch_bounds__(G16_NTH) k_gram16(G16K k) {
  extern __shared__ uint4 smem16[];
  unsigned char* lds = (unsigned char*)smem16;
  using S = G16Split<NB, KS>;
  constexpr int NBLK = S::NBLK, MAXB = S::MAXB;
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t li = lane & 15, kg = lane >> 4;
  const uint32_t IB = k.I * k.B;
  const uint32_t st0 = S::KSPLIT ? wave : 0, dst_ = S::KSPLIT ? 4 : 1;

  f4 acc[MAXB];
  double dacc[MAXB][4];
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    acc[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) dacc[m][v] = 0.0;
  }
  auto flush = [&]() {
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
#pragma unroll
      for (int v = 0; v < 4; ++v) dacc[m][v] += (double)acc[m][v];
      acc[m] = f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto step = [&](auto&& ld) {
    if (S::KSPLIT) {
      g16_step<BF, NB, KS, 0>(acc, ld);
    } else {
      switch (wave) {
        case 0: g16_step<BF, NB, KS, 0>(acc, ld); break;
        case 1: g16_step<BF, NB, KS, 1>(acc, ld); break;
        case 2: g16_step<BF, NB, KS, 2>(acc, ld); break;
        default: g16_step<BF, NB, KS, 3>(acc, ld); break;
      }
    }
  };

  // The transfers of a tile. With a mask, each wave also transfers, per instruction j of
  // its piece transfers, the mask bytes of those 64 pieces: as whole dwords (4-byte
  // transfers land at 4-byte steps per lane) into its own 80-byte region of the
  // buffer's mask area. Narrow tiles: the 64 pieces' bytes are consecutive, 17 dwords
  // cover them from the dword below; wide tiles: 4 rows of 16 consecutive bytes, 5
  // dwords each. The bytes are read back only by lanes of the same wave, after the vmcnt
  // wait that also covers the pieces.
  auto mregion = [&](int buf, uint32_t j) -> unsigned char* {
    return lds + k.mask_off + ((size_t)(buf * G16_PIECES + j) * 4 + wave) * G16_MREG;
  };
  const uint32_t* const mask32 = (const uint32_t*)k.mask8;
  auto issue = [&](uint64_t tile, int buf) {
    unsigned char* dst = lds + (size_t)buf * k.buf_bytes;
    if (k.wide) {
      const uint64_t a = tile / k.tiles_per_a;
      const uint32_t b0 = (uint32_t)(tile - a * k.tiles_per_a) * G16_TB;
      const uint32_t lenc = (k.B - b0 < G16_TB ? k.B - b0 : G16_TB) / 8;
      const uint32_t nchunk = k.I * (G16_TB / 8);
      uint32_t j = 0;
      for (uint32_t q0 = wave * 64; q0 < nchunk; q0 += G16_NTH, ++j) {
        const uint32_t p = q0 + lane;
        const uint32_t r = p >> 4, c = (p & 15) ^ (r & 15);
        if (p < nchunk && c < lenc)
          __builtin_amdgcn_global_load_lds((const void*)(k.X + ((a * k.I + r) * k.B + b0 + c * 8)),
                                           (lds_void_t*)(dst + (size_t)q0 * 16), 16, 0, 0);
        if (k.mask8 && lane < 20) {
          const uint32_t rr = (q0 >> 4) + lane / 5;   // row of this dword
          if (rr < k.I) {
            // clamped to the tensor's last mask dword (bytes past a row are not used)
            const uint64_t byte0 = ((a * k.I + rr) * k.B + b0) >> 3;
            const uint64_t d = (byte0 >> 2) + lane % 5;
            const uint64_t dlast = ((uint64_t)k.A * IB / 8 - 1) >> 2;
            __builtin_amdgcn_global_load_lds((const void*)(mask32 + (d < dlast ? d : dlast)),
                                             (lds_void_t*)mregion(buf, j), 4, 0, 0);
          }
        }
      }
    } else {
      const uint64_t a0 = tile * k.TA;
      const uint32_t nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      const uint32_t len = nta * IB;
      const uint32_t n16 = len / 8;
      const uint64_t e0 = a0 * IB;
      const uint16_t* src = k.X + e0;
      uint32_t j = 0;
      for (uint32_t q0 = wave * 64; q0 < n16; q0 += G16_NTH, ++j) {
        if (q0 + lane < n16)
          __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)(q0 + lane) * 8),
                                           (lds_void_t*)(dst + (size_t)q0 * 16), 16, 0, 0);
        if (k.mask8 && lane < 17) {
          // dwords of the bytes of pieces q0 .. q0 + 63, clamped to the tile's last byte
          const uint64_t first = (e0 >> 3) + q0, last = (e0 >> 3) + n16 - 1;
          const uint64_t d = (first >> 2) + lane;
          __builtin_amdgcn_global_load_lds((const void*)(mask32 + (d < (last >> 2) ? d : (last >> 2))),
                                           (lds_void_t*)mregion(buf, j), 4, 0, 0);
        }
      }
      // the last tile may end inside a 16-byte piece
      if (tid < len - n16 * 8) {
        const uint64_t e = e0 + n16 * 8 + tid;
        const bool om = k.mask8 && ((k.mask8[e >> 3] >> (e & 7)) & 1u);
        ((uint16_t*)dst)[n16 * 8 + tid] = om ? (uint16_t)0 : src[n16 * 8 + tid];
      }
    }
  };
  // clear the Omega entries of this thread's pieces of the tile in `buf` (their transfers
  // and mask bytes have landed: called after a vmcnt wait)
  auto clear = [&](uint64_t tile, int buf) {
    unsigned char* dst = lds + (size_t)buf * k.buf_bytes;
    if (k.wide) {
      const uint64_t a = tile / k.tiles_per_a;
      const uint32_t b0 = (uint32_t)(tile - a * k.tiles_per_a) * G16_TB;
      const uint32_t lenc = (k.B - b0 < G16_TB ? k.B - b0 : G16_TB) / 8;
      const uint32_t nchunk = k.I * (G16_TB / 8);
      uint32_t j = 0;
      for (uint32_t q0 = wave * 64; q0 < nchunk; q0 += G16_NTH, ++j) {
        const uint32_t p = q0 + lane;
        const uint32_t r = p >> 4, c = (p & 15) ^ (r & 15);
        if (p < nchunk && c < lenc) {
          const uint32_t mis = (uint32_t)((((a * k.I + r) * k.B + b0) >> 3) & 3u);
          const uint32_t b = mregion(buf, j)[20 * (lane >> 4) + mis + c];
          if (b) clear_piece(dst + (size_t)p * 16, b);
        }
      }
    } else {
      const uint64_t a0 = tile * k.TA;
      const uint32_t nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      const uint32_t n16 = nta * IB / 8;
      const uint32_t mis = (uint32_t)(((a0 * IB) >> 3) & 3u);
      uint32_t j = 0;
      for (uint32_t q0 = wave * 64; q0 < n16; q0 += G16_NTH, ++j) {
        if (q0 + lane < n16) {
          const uint32_t b = mregion(buf, j)[((mis + q0) & 3u) + lane];
          if (b) clear_piece(dst + (size_t)(q0 + lane) * 16, b);
        }
      }
    }
  };

  uint32_t since = 0;
  uint64_t tile = blockIdx.x;
  int cur = 0;
  if (tile < k.ntiles) issue(tile, cur);
  __builtin_amdgcn_s_waitcnt(0);
  if (k.mask8 && tile < k.ntiles) clear(tile, cur);
  for (; tile < k.ntiles; tile += gridDim.x) {
    const uint64_t next = tile + gridDim.x;
    lds_barrier();                  // tile `cur` landed (Omega cleared) everywhere; `cur ^ 1` free
    if (next < k.ntiles) issue(next, cur ^ 1);
    const unsigned char* buf = lds + (size_t)cur * k.buf_bytes;
    if (k.wide) {
      const uint64_t a = tile / k.tiles_per_a;
      const uint32_t b0 = (uint32_t)(tile - a * k.tiles_per_a) * G16_TB;
      const uint32_t lenc = (k.B - b0 < G16_TB ? k.B - b0 : G16_TB) / 8;
      const uint32_t nsteps = (lenc + 3) / 4;
      for (uint32_t st = st0; st < nsteps; st += dst_) {
        const uint32_t c = st * 4 + kg;
        const bool cok = c < lenc;
        const uint32_t cc = cok ? c : 0;
        step([&](int rb) -> u16x8 {
          // rows >= I only reach Gram entries that are dropped: read row I - 1 instead
          const uint32_t r = rb * 16 + li < k.I ? rb * 16 + li : k.I - 1;
          const u16x8 f = *(const u16x8*)(buf + (size_t)(r * 16 + (cc ^ (r & 15))) * 16);
          return cok ? f : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        });
        if (++since == G16_FLUSH) {
          flush();
          since = 0;
        }
      }
    } else {
      const uint64_t a0 = tile * k.TA;
      const uint32_t nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      const uint32_t K = nta * k.B;
      const uint32_t nsteps = (K + 31) / 32;
      const uint16_t* b16 = (const uint16_t*)buf;
      for (uint32_t st = st0; st < nsteps; st += dst_) {
        const uint32_t kk0 = st * 32 + kg * 8;
        uint32_t off[8];
        bool ok[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t kk = kk0 + j;
          ok[j] = kk < K;
          // a = floor(kk / B): exact in fp32 for kk < 2^22 (error 2^-23 kk / B < 1 / (2B))
          const uint32_t a = (uint32_t)(((float)kk + 0.5f) * k.invB);
          off[j] = a * (IB - k.B) + kk;
        }
        step([&](int rb) -> u16x8 {
          // rows >= I only reach Gram entries that are dropped: read row I - 1 instead;
          // k past the tile reads row start and is zeroed, so every read is in bounds
          const uint32_t r = rb * 16 + li < k.I ? rb * 16 + li : k.I - 1;
          const uint32_t ro = r * k.B;
          u16x8 f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint16_t x = b16[ok[j] ? off[j] + ro : ro];
            f[j] = ok[j] ? x : (uint16_t)0;
          }
          return f;
        });
        if (++since == G16_FLUSH) {
          flush();
          since = 0;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's part of the next tile landed
    if (k.mask8 && next < k.ntiles) clear(next, cur ^ 1);
    cur ^= 1;
  }
  flush();

  // block sums to LDS (k-split: added in wave order), then the symmetric partial
  double* red = (double*)lds;
  lds_barrier();
  if (S::KSPLIT) {
    for (uint32_t w = 0; w < 4; ++w) {
      if (wave == w) {
#pragma unroll
        for (int m = 0; m < MAXB; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t idx = (m * 4 + v) * 64 + lane;
            red[idx] = (w == 0 ? 0.0 : red[idx]) + dacc[m][v];
          }
      }
      lds_barrier();
    }
  } else {
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      const uint32_t q = wave + 4 * m;
      if (q < (uint32_t)NBLK) {
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(q * 4 + v) * 64 + lane] = dacc[m][v];
      }
    }
    lds_barrier();
  }
  double* out = k.partial + (uint64_t)blockIdx.x * k.I * k.I;
  for (int q = 0; q < NBLK; ++q) {
    if (wave != (uint32_t)(q & 3)) continue;
    const int rb = blk_rb(NB, q), cb = blk_cb(NB, q);
    const uint32_t col = cb * 16 + li;
    for (int v = 0; v < 4; ++v) {
      const uint32_t row = rb * 16 + 4 * kg + v;
      if (row < k.I && col < k.I) {
        const double x = red[(q * 4 + v) * 64 + lane];
        out[(size_t)row * k.I + col] = x;
        if (rb != cb) out[(size_t)col * k.I + row] = x;
      }
    }
  }
}

struct G16Geo {
  bool ok;
  G16K k;
  size_t lds;
  uint32_t grid;
};

// The work split for NB row blocks on wide or slab tiles.
constexpr bool g16_ks(int NB, bool wide) { return NB <= 2 || (!wide && NB <= 3); }

// Workgroups of k_gram16<BF, NB, KS> a CU holds with `lds` bytes of LDS each (0 on error).
template <bool BF, int NB, bool KS>
int g16_occ(size_t lds) {
  auto fn = k_gram16<BF, NB, KS>;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds) != hipSuccess)
    return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, G16_NTH, lds) != hipSuccess)
    return 0;
  return per_cu;
}
template <bool BF>
int g16_occ_nb(uint32_t I, bool wide, size_t lds) {
  switch ((I + 15) / 16) {
    case 1: return g16_occ<BF, 1, g16_ks(1, false)>(lds);
    case 2: return g16_occ<BF, 2, g16_ks(2, false)>(lds);
    case 3: return wide ? g16_occ<BF, 3, g16_ks(3, true)>(lds)
                        : g16_occ<BF, 3, g16_ks(3, false)>(lds);
    case 4: return g16_occ<BF, 4, g16_ks(4, false)>(lds);
  }
  return 0;
}

G16Geo g16geo(const GramArgs& g, int num_cu) {
  G16Geo r{};
  r.ok = false;
  if (g.P != 1 || (g.dt != DT_BF16 && g.dt != DT_F16) || g.I > 64 || g.I == 0) return r;
  if (((uintptr_t)g.X) % 16 != 0) return r;
  G16K& k = r.k;
  k.X = (const uint16_t*)g.X;
  k.mask8 = (const uint8_t*)g.mask;
  k.A = g.A;
  k.I = g.I;
  k.B = g.B;
  const uint64_t IB = (uint64_t)g.I * g.B;
  if (g.B >= 32 && g.B % 8 == 0) {
    k.wide = 1;
    k.tiles_per_a = (g.B + G16_TB - 1) / G16_TB;
    k.ntiles = (uint64_t)g.A * k.tiles_per_a;
    k.buf_bytes = g.I * G16_TB * 2;
  } else {
    if (IB > G16_NARROW) return r;
    // tiles start on 16-byte boundaries: TA * I * B a multiple of 8
    uint32_t TA = (uint32_t)(G16_NARROW / IB);
    uint32_t step = 8;
    for (uint32_t t = 1; t <= 8; t <<= 1)
      if ((IB * t) % 8 == 0) {
        step = t;
        break;
      }
    TA -= TA % step;
    if (TA == 0) return r;
    if ((uint64_t)TA > g.A) TA = g.A;   // a single tile; its start is the buffer start
    k.wide = 0;
    k.TA = TA;
    k.ntiles = ((uint64_t)g.A + TA - 1) / TA;
    k.buf_bytes = (uint32_t)((TA * IB * 2 + 15) & ~15ull);
    k.invB = 1.0f / (float)g.B;
  }
  const uint32_t nb = (g.I + 15) / 16;
  const size_t red = (size_t)nb * (nb + 1) / 2 * 4 * 64 * sizeof(double);   // block sums
  // masked: per tile buffer, an 80-byte region per (transfer instruction, wave)
  k.mask_off = 2 * k.buf_bytes;
  const size_t mask_area = g.mask ? (size_t)2 * G16_PIECES * 4 * G16_MREG : 0;
  r.lds = std::max((size_t)2 * k.buf_bytes + mask_area, red);
  // a persistent grid of one resident round (a second, partial round would run alone at
  // the end): as many workgroups as a CU holds with this kernel's registers and LDS, at
  // most G16_WGS_PER_CU (each workgroup writes an I x I fp64 partial)
  const int occ = g.dt == DT_BF16 ? g16_occ_nb<true>(g.I, k.wide != 0, r.lds)
                                  : g16_occ_nb<false>(g.I, k.wide != 0, r.lds);
  if (occ < 1) return r;
  const int per_cu = occ < G16_WGS_PER_CU ? occ : G16_WGS_PER_CU;
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * (uint64_t)per_cu;
  if (grid > k.ntiles) grid = k.ntiles;
  if (g.max_blocks && grid > g.max_blocks) grid = g.max_blocks;
  if (grid < 1) grid = 1;
  r.grid = (uint32_t)grid;
  r.ok = true;
  return r;
}

template <bool BF, int NB, bool KS>
hipError_t go16(const G16Geo& g, hipStream_t s) {
  // g16geo has raised the kernel's LDS limit where it needs more than 64 KiB
  auto fn = k_gram16<BF, NB, KS>;
  hipLaunchKernelGGL(fn, dim3(g.grid), dim3(G16_NTH), g.lds, s, g.k);
  return hipGetLastError();
}

template <bool BF>
hipError_t pick16(const G16Geo& g, hipStream_t s) {
  switch ((g.k.I + 15) / 16) {
    case 1: return go16<BF, 1, g16_ks(1, false)>(g, s);
    case 2: return go16<BF, 2, g16_ks(2, false)>(g, s);
    case 3: return g.k.wide ? go16<BF, 3, g16_ks(3, true)>(g, s)
                            : go16<BF, 3, g16_ks(3, false)>(g, s);
    case 4: return go16<BF, 4, g16_ks(4, false)>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Sum nblk partials of n2 values (stored after them: RGROUPS stage rows) into out.
hipError_t gram_reduce(double* partial, uint32_t nblk, uint32_t n2, double* out, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx) {
  double* stage = partial + (uint64_t)nblk * n2;
  if (mark) mark(mctx, KID_GRAM_REDUCE, true);
  k_gram_reduce1<<<dim3((n2 + 255) / 256, RGROUPS), 256, 0, s>>>(partial, nblk, n2, stage);
  k_gram_reduce2<<<(n2 + 255) / 256, 256, 0, s>>>(stage, n2, out);
  if (mark) mark(mctx, KID_GRAM_REDUCE, false);
  return hipGetLastError();
}

uint32_t gram_reduce_groups() { return RGROUPS; }

uint32_t gram_blocks(const GramArgs& g, int num_cu) {
  const G16Geo f = g16geo(g, num_cu);
  if (f.ok) return f.grid;
  const G32Geo f32 = gram32_geo(g, num_cu);
  if (f32.ok) return f32.grid;
  const GGeo r = ggeo(g);
  uint64_t nb = (uint64_t)(num_cu > 0 ? num_cu : 256) * 4;
  if (nb > r.ntiles) nb = r.ntiles;
  // at most 2^24 doubles (128 MB) of partial sums
  const uint64_t k2 = (uint64_t)r.Kin * r.Kin;
  if (nb * k2 > (1ull << 24)) nb = std::max<uint64_t>(1, (1ull << 24) / k2);
  if (g.max_blocks && nb > g.max_blocks) nb = g.max_blocks;
  if (nb < 1) nb = 1;
  // every block gets at least one tile: recompute from tiles per block
  const uint64_t tpb = (r.ntiles + nb - 1) / nb;
  return (uint32_t)((r.ntiles + tpb - 1) / tpb);
}

size_t gram_lds_bytes(const GramArgs& g) { return ggeo(g).lds; }

hipError_t launch_gram(const GramArgs& g, int num_cu, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx) {
  const GGeo r = ggeo(g);
  if (r.Kin > 256) return hipErrorInvalidValue;
  const uint32_t nblk = gram_blocks(g, num_cu);
  const G16Geo f = g16geo(g, num_cu);
  if (f.ok) {
    G16Geo ff = f;
    ff.k.partial = g.partial;
    if (mark) mark(mctx, KID_GRAM, true);
    const hipError_t e = g.dt == DT_BF16 ? pick16<true>(ff, s) : pick16<false>(ff, s);
    if (mark) mark(mctx, KID_GRAM, false);
    if (e != hipSuccess) return e;
    return gram_reduce(g.partial, nblk, r.Kin * r.Kin, g.out, s, mark, mctx);
  }
  const G32Geo f32 = gram32_geo(g, num_cu);
  if (f32.ok) {
    if (mark) mark(mctx, KID_GRAM, true);
    const hipError_t e = launch_gram32(f32, g.partial, s);
    if (mark) mark(mctx, KID_GRAM, false);
    if (e != hipSuccess) return e;
    return gram_reduce(g.partial, nblk, r.Kin * r.Kin, g.out, s, mark, mctx);
  }
  GK k;
  k.X = g.X;
  k.mask = g.mask;
  k.partial = g.partial;
  k.ntiles = r.ntiles;
  k.tiles_per_blk = (r.ntiles + nblk - 1) / nblk;
  k.tiles_per_a = r.tiles_per_a;
  k.A = g.A;
  k.I = g.I;
  k.B = g.B;
  k.Kin = r.Kin;
  k.nb = r.nb;
  k.TA = r.TA;
  k.wide = r.wide;
  hipError_t e;
  if (mark) mark(mctx, KID_GRAM, true);
  if (g.P == 2) {
    e = pick_nob<float, 2>(k, r.lds, nblk, s);
  } else {
    switch (g.dt) {
      case DT_F32: e = pick_nob<float, 1>(k, r.lds, nblk, s); break;
      case DT_F16: e = pick_nob<_Float16, 1>(k, r.lds, nblk, s); break;
      case DT_BF16: e = pick_nob<bf16_t, 1>(k, r.lds, nblk, s); break;
      default: e = hipErrorInvalidValue;
    }
  }
  if (mark) mark(mctx, KID_GRAM, false);
  if (e != hipSuccess) return e;
  return gram_reduce(g.partial, nblk, r.Kin * r.Kin, g.out, s, mark, mctx);
}

}  // namespace tg
