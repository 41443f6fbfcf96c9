// Mode-n Gram matrices of fp32 and complex64 residuals, for the HOSVD refresh.
//
// Same definition as k_gram.hip (pith.science "What carries the argument": each factor
// is taken from the Gram matrix of its mode's unfolding; nullthought summary section 3:
// the unfolding is that of the residual left after the sparse part): Gram_n =
// R_(n) R_(n)^H over the (A, I, B, P) view of mode n, summed over every (a, b) column.
// Complex data (P = 2) gives the stacked real Gram of rows kk = i P + p, of size
// (I P)^2, from which the eigensolver forms the Hermitian matrix.
//
// This kernel serves fp32 and complex64 tensors with I <= 64 read without a mask (the
// residual copy the top-k pass writes). Tiles move HBM -> LDS with 16-byte
// global_load_lds transfers, double buffered, in a persistent grid of one workgroup
// per CU (tile = blockIdx.x, + gridDim.x, ...):
//   wide   (B >= 64, B P a multiple of 4): one a, 64 consecutive columns b, all I rows.
//          Row r's 16-byte piece c lands at LDS piece r Q + (c ^ (r % 16)) (Q pieces a
//          row), so each transfer instruction fills 64 consecutive LDS pieces and the
//          16 rows a fragment read touches spread over the banks.
//   narrow (B <= 128): TA whole slabs (TA B <= 128 columns), a contiguous region of the
//          tensor copied as is; column c = (slab s, b) sits at s I B P + b P, row r adds
//          r B P (a per-column table in LDS).
// The stacked Gram is formed in component-major order (row block q = p NBI + rb holds
// component p of rows 16 rb .. 16 rb + 15) on v_mfma_f32_16x16x4_f32: in each group of
// 16 columns, lane (li, kg) supplies row 16 rb + li at columns 4 kg .. 4 kg + 3, value t
// to k-step t (a fixed permutation of the columns, the same for both operands), so one
// 8-byte LDS read gives both components of a complex value. Block (qa, qb) of the Gram is
// the sum of mfma(fragment qa, fragment qb); only qa <= qb is formed, dealt round-robin
// to the 8 waves. Products are summed in fp32 over 64 columns, then added into fp64;
// each workgroup writes its fp64 partial (both triangles, in the interleaved order
// i P + p) and gram_reduce sums the partials in a fixed order, so results are
// deterministic run to run.
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int G32_NTH = 512;              // 8 waves: two per SIMD
constexpr int G32_WAVES = G32_NTH / 64;
constexpr uint32_t G32_TCW = 64;          // wide tiles: columns per tile
constexpr uint32_t G32_TCN = 128;         // narrow tiles: at most this many columns
constexpr uint32_t G32_FLUSH = 4;         // 16-column groups per fp32 partial sum

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct G32K {
  const float* X;
  double* partial;
  uint64_t ntiles;
  uint32_t A, I, B;
  uint32_t wide;
  uint32_t tiles_per_a;   // wide: tiles per a
  uint32_t rowq;          // wide: 16-byte pieces per tile row (G32_TCW P / 4)
  uint32_t TA;            // narrow: slabs per tile
  uint32_t buf_bytes;     // one tile buffer (multiple of 16)
  uint32_t colb_off;      // narrow: LDS byte offset of the per-column float offsets
};

__host__ __device__ constexpr int g32_rb(int NB, int q) {
  int rb = 0;
  while (q >= NB - rb) {
    q -= NB - rb;
    ++rb;
  }
  return rb;
}
__host__ __device__ constexpr int g32_cb(int NB, int q) {
  int rb = 0;
  while (q >= NB - rb) {
    q -= NB - rb;
    ++rb;
  }
  return rb + q;
}

// The MFMAs of one k-step t for wave W's blocks (compile-time block indices).
template <int NBK, int W, int M>
__device__ __forceinline__ void g32_mfma(f4* acc, const float (*fr)[4], int t) {
  constexpr int NBLK = NBK * (NBK + 1) / 2;
  constexpr int q = W + G32_WAVES * M;
  if constexpr (q < NBLK) {
    constexpr int qa = g32_rb(NBK, q), qb = g32_cb(NBK, q);
    acc[M] = __builtin_amdgcn_mfma_f32_16x16x4f32(fr[qa][t], fr[qb][t], acc[M], 0, 0, 0);
    g32_mfma<NBK, W, M + 1>(acc, fr, t);
  }
}
template <int NBK, int W>
__device__ __forceinline__ void g32_group(f4* acc, const float (*fr)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) g32_mfma<NBK, W, 0>(acc, fr, t);
}

template <int P, int NBI>
__global__ void __launch_bounds__(G32_NTH) k_gram32(G32K k) {
  extern __shared__ uint4 smem32[];
  unsigned char* const lds = (unsigned char*)smem32;
  constexpr int NBK = P * NBI;                     // stacked row blocks
  constexpr int NBLK = NBK * (NBK + 1) / 2;
  constexpr int MAXB = (NBLK + G32_WAVES - 1) / G32_WAVES;
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t li = lane & 15, kg = lane >> 4;
  const uint32_t I = k.I, B = k.B;
  const uint32_t IBP = I * B * P;

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

  // narrow tiles: float offset of every column of a full tile (the same for every tile)
  uint32_t* const colb = (uint32_t*)(lds + k.colb_off);
  if (!k.wide) {
    for (uint32_t c = tid; c < G32_TCN; c += G32_NTH) {
      const uint32_t s = c / B, b = c - s * B;
      colb[c] = c < k.TA * B ? s * IBP + b * P : 0u;
    }
  }

  // the transfers of a tile into buffer `buf`
  auto issue = [&](uint64_t tile, int buf) {
    unsigned char* dst = lds + (size_t)buf * k.buf_bytes;
    if (k.wide) {
      const uint64_t a = tile / k.tiles_per_a;
      const uint32_t b0 = (uint32_t)(tile - a * k.tiles_per_a) * G32_TCW;
      const uint32_t ncol = B - b0 < G32_TCW ? B - b0 : G32_TCW;
      const uint32_t npc = ncol * P / 4;   // valid pieces of a row
      const uint32_t nq = I * k.rowq;
      for (uint32_t q0 = wave * 64; q0 < nq; q0 += G32_NTH) {
        const uint32_t pq = q0 + lane;
        const uint32_t r = pq / k.rowq, slot = pq - r * k.rowq;
        const uint32_t c = slot ^ (r & 15u);
        if (pq < nq && c < npc)
          __builtin_amdgcn_global_load_lds(
              (const void*)(k.X + ((a * I + r) * (uint64_t)B + b0) * P + (uint64_t)c * 4),
              (lds_void_t*)(dst + (size_t)q0 * 16), 16, 0, 0);
      }
    } else {
      const uint64_t a0 = tile * k.TA;
      const uint32_t nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      const uint32_t len = nta * IBP;
      const uint32_t n16 = len / 4;
      const float* src = k.X + a0 * IBP;
      for (uint32_t q0 = wave * 64; q0 < n16; q0 += G32_NTH)
        if (q0 + lane < n16)
          __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)(q0 + lane) * 4),
                                           (lds_void_t*)(dst + (size_t)q0 * 16), 16, 0, 0);
      // the last tile may end inside a 16-byte piece
      if (tid < len - n16 * 4) ((float*)dst)[n16 * 4 + tid] = src[n16 * 4 + tid];
    }
  };

  // fragments of one group of 16 columns (columns 16 g + 4 kg + t for k-step t)
  auto group = [&](const unsigned char* buf, uint32_t g, uint32_t ncol) {
    float fr[NBK][4];
    if (k.wide) {
      // one 16-byte read per row block gives a lane its columns 4 kg .. 4 kg + 3 (P = 1),
      // or two of them, both components (P = 2: two reads)
#pragma unroll
      for (int rb = 0; rb < NBI; ++rb) {
        // rows >= I only reach Gram entries that are dropped: read row I - 1 instead
        const uint32_t r = 16 * rb + li < I ? 16 * rb + li : I - 1;
        if constexpr (P == 2) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // columns c0 = 16 g + 4 kg + 2 h and c0 + 1: floats 2 c0 .. 2 c0 + 3, one piece
            const uint32_t c0 = 16 * g + 4 * kg + 2 * h;
            const uint32_t cp = 8 * g + 2 * kg + h;
            const f4 v = *(const f4*)(buf + ((r * k.rowq + (cp ^ (r & 15u))) << 4));
            const bool ok0 = c0 < ncol, ok1 = c0 + 1 < ncol;
            fr[rb][2 * h] = ok0 ? v[0] : 0.0f;
            fr[NBI + rb][2 * h] = ok0 ? v[1] : 0.0f;
            fr[rb][2 * h + 1] = ok1 ? v[2] : 0.0f;
            fr[NBI + rb][2 * h + 1] = ok1 ? v[3] : 0.0f;
          }
        } else {
          const uint32_t cp = 4 * g + kg;
          const f4 v = *(const f4*)(buf + ((r * k.rowq + (cp ^ (r & 15u))) << 4));
#pragma unroll
          for (int t = 0; t < 4; ++t) fr[rb][t] = 16 * g + 4 * kg + t < ncol ? v[t] : 0.0f;
        }
      }
    } else {
      const float* bf = (const float*)buf;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t c = 16 * g + 4 * kg + t;
        const bool ok = c < ncol;
        const uint32_t cb = colb[ok ? c : 0];
#pragma unroll
        for (int rb = 0; rb < NBI; ++rb) {
          const uint32_t r = 16 * rb + li < I ? 16 * rb + li : I - 1;
          const uint32_t off = cb + r * B * P;
          if constexpr (P == 2) {
            const f2 v = *(const f2*)(bf + off);
            fr[rb][t] = ok ? v[0] : 0.0f;
            fr[NBI + rb][t] = ok ? v[1] : 0.0f;
          } else {
            const float v = bf[off];
            fr[rb][t] = ok ? v : 0.0f;
          }
        }
      }
    }
    switch (wave) {
      case 0: g32_group<NBK, 0>(acc, fr); break;
      case 1: g32_group<NBK, 1>(acc, fr); break;
      case 2: g32_group<NBK, 2>(acc, fr); break;
      case 3: g32_group<NBK, 3>(acc, fr); break;
      case 4: g32_group<NBK, 4>(acc, fr); break;
      case 5: g32_group<NBK, 5>(acc, fr); break;
      case 6: g32_group<NBK, 6>(acc, fr); break;
      default: g32_group<NBK, 7>(acc, fr); break;
    }
  };

  uint64_t tile = blockIdx.x;
  int cur = 0;
  if (tile < k.ntiles) issue(tile, cur);
  __builtin_amdgcn_s_waitcnt(0);
  for (; tile < k.ntiles; tile += gridDim.x) {
    const uint64_t next = tile + gridDim.x;
    lds_barrier();                  // tile `cur` landed everywhere; `cur ^ 1` is free
    if (next < k.ntiles) issue(next, cur ^ 1);
    const unsigned char* buf = lds + (size_t)cur * k.buf_bytes;
    uint32_t ncol;
    if (k.wide) {
      const uint64_t a = tile / k.tiles_per_a;
      const uint32_t b0 = (uint32_t)(tile - a * k.tiles_per_a) * G32_TCW;
      ncol = B - b0 < G32_TCW ? B - b0 : G32_TCW;
    } else {
      const uint64_t a0 = tile * k.TA;
      const uint32_t nta = (uint64_t)k.A - a0 < k.TA ? (uint32_t)((uint64_t)k.A - a0) : k.TA;
      ncol = nta * B;
    }
    const uint32_t ng = (ncol + 15) / 16;
    for (uint32_t g = 0; g < ng; ++g) {
      group(buf, g, ncol);
      if ((g + 1) % G32_FLUSH == 0) flush();
    }
    flush();
    __builtin_amdgcn_s_waitcnt(0);  // this thread's part of the next tile landed
    cur ^= 1;
  }

  // the symmetric partial, in the interleaved order i P + p
  const uint32_t K = I * P;
  double* out = k.partial + (uint64_t)blockIdx.x * K * K;
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    const int q = (int)wave + G32_WAVES * m;
    if (q >= NBLK) continue;
    const int qa = g32_rb(NBK, q), qb = g32_cb(NBK, q);
    const uint32_t pa = (uint32_t)qa / NBI, pb = (uint32_t)qb / NBI;
    const uint32_t ib = ((uint32_t)qb % NBI) * 16 + li;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t ia = ((uint32_t)qa % NBI) * 16 + 4 * kg + v;
      if (ia < I && ib < I) {
        const uint32_t row = ia * P + pa, col = ib * P + pb;
        out[(size_t)row * K + col] = dacc[m][v];
        if (qa != qb) out[(size_t)col * K + row] = dacc[m][v];
      }
    }
  }
}

template <int P, int NBI>
hipError_t go32(const G32K& k, size_t lds, uint32_t grid, hipStream_t s) {
  auto fn = k_gram32<P, NBI>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute((const void*)fn,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(G32_NTH), lds, s, k);
  return hipGetLastError();
}

}  // namespace

// The geometry of the fp32 / complex64 Gram launch, or ok = false where it does not
// apply (another dtype, I > 64, a mask, a misaligned input, or narrow slabs that do not
// fit a tile).
G32Geo gram32_geo(const GramArgs& g, int num_cu) {
  G32Geo r{};
  r.ok = false;
  if (g.dt != DT_F32 || (g.P != 1 && g.P != 2) || g.I == 0 || g.I > 64 || g.mask) return r;
  if (((uintptr_t)g.X) % 16 != 0 || g.A == 0 || g.B == 0) return r;
  const uint32_t P = g.P;
  G32K k{};
  k.I = g.I;
  k.B = g.B;
  k.A = g.A;
  const uint64_t IBP = (uint64_t)g.I * g.B * P;
  size_t lds;
  if (g.B >= G32_TCW && (g.B * P) % 4 == 0) {
    k.wide = 1;
    k.tiles_per_a = (g.B + G32_TCW - 1) / G32_TCW;
    k.ntiles = (uint64_t)g.A * k.tiles_per_a;
    k.rowq = G32_TCW * P / 4;
    k.buf_bytes = g.I * k.rowq * 16;
    k.colb_off = 2 * k.buf_bytes;
    lds = 2 * (size_t)k.buf_bytes;
  } else {
    if (g.B > G32_TCN) return r;
    // tiles start on 16-byte boundaries: TA I B P a multiple of 4
    uint32_t step = 4;
    for (uint32_t t = 1; t <= 4; t <<= 1)
      if ((IBP * t) % 4 == 0) {
        step = t;
        break;
      }
    uint32_t TA = G32_TCN / g.B;
    TA -= TA % step;
    if (TA == 0) return r;
    if ((uint64_t)TA > g.A) TA = g.A;   // a single tile; its start is the buffer start
    k.wide = 0;
    k.TA = TA;
    k.ntiles = ((uint64_t)g.A + TA - 1) / TA;
    k.buf_bytes = (uint32_t)((TA * IBP * 4 + 15) & ~15ull);
    k.colb_off = 2 * k.buf_bytes;
    lds = 2 * (size_t)k.buf_bytes + G32_TCN * 4;
  }
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256);
  if (grid > k.ntiles) grid = k.ntiles;
  if (g.max_blocks && grid > g.max_blocks) grid = g.max_blocks;
  if (grid < 1) grid = 1;
  k.X = (const float*)g.X;
  r.ok = true;
  r.P = P;
  r.grid = (uint32_t)grid;
  r.lds = lds;
  static_assert(sizeof(G32K) <= sizeof(r.kbytes), "kernel arguments fit the geometry record");
  __builtin_memcpy(r.kbytes, &k, sizeof(G32K));
  return r;
}

hipError_t launch_gram32(const G32Geo& geo, double* partial, hipStream_t s) {
  if (!geo.ok) return hipErrorInvalidValue;
  G32K k;
  __builtin_memcpy(&k, geo.kbytes, sizeof(G32K));
  k.partial = partial;
  const uint32_t nbi = (k.I + 15) / 16;
  const bool cplx = geo.P == 2;
  switch (nbi) {
    case 1: return cplx ? go32<2, 1>(k, geo.lds, geo.grid, s) : go32<1, 1>(k, geo.lds, geo.grid, s);
    case 2: return cplx ? go32<2, 2>(k, geo.lds, geo.grid, s) : go32<1, 2>(k, geo.lds, geo.grid, s);
    case 3: return cplx ? go32<2, 3>(k, geo.lds, geo.grid, s) : go32<1, 3>(k, geo.lds, geo.grid, s);
    case 4: return cplx ? go32<2, 4>(k, geo.lds, geo.grid, s) : go32<1, 4>(k, geo.lds, geo.grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
