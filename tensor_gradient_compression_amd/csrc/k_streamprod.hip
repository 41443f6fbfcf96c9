// One fp32 mode product streamed by independent waves: the leading compressed modes of
// the reconstruction and the projection (any fp32 -> fp32 mode product with I <= 64,
// R <= 64 and a long trailing part, real or complex).
//
// Same product as k_modeprod.hip (pith.science "What carries the argument": projection
// to the core and reconstruction by mode-wise products; appendix M Theorem 2), on the
// tensor viewed as (A, I, B): Y[a, r, b] = sum_i M[r, i] X[a, i, b].
//
// Organisation. The work is a stream: every X value is read once and every Y value
// written once, a few flops apart, so what matters is how many bytes each CU keeps in
// flight. A tile is 64 consecutive columns b of one a; each wave takes tiles strided
// over all waves of the grid and owns every output row of its tile, so each X value it
// loads feeds all NRB row blocks of the product (v_mfma_f32_16x16x4_f32, fp32
// accumulation, k in steps of 4 as in k_modeprod.hip).
//  * Lane (li, lg) loads the four columns 4 li .. 4 li + 3 of row 4 ks + lg in one
//    16-byte load; value j of it is that lane's B operand in the product of column
//    block j (block j holds the columns 4 li + j). The accumulators of the four blocks
//    then hold, per lane and output row, four consecutive columns: one 16-byte store.
//  * The next tile's loads go into a second register set while this tile is
//    multiplied: a wave keeps a tile of loads (8 KB at I = 32) in flight, with no LDS
//    staging and no barrier. A tile's operands are waited for with its predecessor's
//    stores still in flight (they were issued after the operands' loads).
//  * Loads and stores are buffer operations over one a's slice: a per-lane offset past
//    the resource's extent reads zero and drops the store (the range check covers the
//    per-lane offset, not the scalar one, so every row offset goes into the per-lane
//    offset). Rows k >= I read zero and rows r >= R are not stored by that rule; columns
//    past B and tiles past the end get an offset of 2^31 (the extent is below 2^31, and
//    adding a row offset below 2^31 neither wraps nor comes back in range), so every wave
//    issues the same memory instructions and the wait counts are exact.
//  * M's A operands come from a per-lane LDS table (one conflict-free read per MFMA),
//    filled once per workgroup.
// Complex data (CPLX) is taken as the real tensor (A, I, 2B) of its interleaved
// (re, im) values, multiplied by Re M and by Im M (two tables, two accumulator sets):
// a lane's four columns are two complex values, and M X = (Re M) X + i (Im M) X is
// formed in registers before the store: re = (Re M x)_re - (Im M x)_im, im =
// (Re M x)_im + (Im M x)_re.
#include "tg_common.h"

namespace tg {

namespace {

constexpr int SP_WPB = 4;            // waves per workgroup
constexpr int SP_NT = SP_WPB * 64;
constexpr uint32_t SP_TC = 64;       // columns per tile

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

struct SPK {
  const float* X;    // (A, I, B) (complex: B counts the real values, twice the complex)
  float* Y;          // (A, R, B)
  const float* M;    // R x I row-major (complex: Re M)
  const float* Mi;   // complex: Im M, R x I
  uint64_t ntiles;   // A * tpa
  uint32_t A, I, B, R;
  uint32_t tpa;      // tiles per a
};

// NRB: 16-row blocks of R (<= 4); NKS: k-steps of 4 (I <= 4 NKS); CPLX: complex data.
template <int NRB, int NKS, bool CPLX>
__global__ void __launch_bounds__(SP_NT) k_streamprod(SPK k) {
  extern __shared__ float smem[];
  // at[(rb NKS + ks) 64 + lane] = M[16 rb + lane % 16][4 ks + lane / 16] (zero outside);
  // complex: the Im M table follows
  constexpr uint32_t NTAB = NRB * NKS * 64;
  LDS float* const at = (LDS float*)smem;
  LDS float* const ati = at + NTAB;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I = k.I, B = k.B, R = k.R;

  {
    constexpr uint32_t NT2 = CPLX ? 2 * NTAB : NTAB;
    constexpr int IT = (int)((NT2 + SP_NT - 1) / SP_NT);
    float tv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t q2 = threadIdx.x + it * SP_NT;
      const bool im = CPLX && q2 >= NTAB;
      const uint32_t q = im ? q2 - NTAB : q2;
      const uint32_t rk = q >> 6, rb = rk / NKS, ks = rk - rb * NKS;
      const uint32_t row = 16 * rb + (q & 15), kk = 4 * ks + ((q & 63) >> 4);
      const bool ok = q2 < NT2 && row < R && kk < I;
      const float v = (im ? k.Mi : k.M)[ok ? row * I + kk : 0];
      tv[it] = ok ? v : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t q = threadIdx.x + it * SP_NT;
      if (q < NT2) at[q] = tv[it];   // the Im table follows the Re one
    }
  }
  __syncthreads();

  const uint64_t TW = (uint64_t)gridDim.x * SP_WPB;
  const uint64_t t0 = (uint64_t)blockIdx.x * SP_WPB + wv;
  if (t0 >= k.ntiles) return;

  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t xbytes = I * B * 4, ybytes = R * B * 4;
  // the a and first column of tile t (a = 0 for a tile past the end: its accesses are
  // all out of range)
  auto place = [&](uint64_t t, bool valid, uint32_t& a, uint32_t& b0) {
    a = valid ? (uint32_t)(t / k.tpa) : 0u;
    b0 = valid ? (uint32_t)(t - (uint64_t)a * k.tpa) * SP_TC : 0u;
  };
  // B operands of tile t: b[ks] = X[a, 4 ks + lg, b0 + 4 li .. b0 + 4 li + 3]
  auto load = [&](uint64_t t, bool valid, u32x4 (&b)[NKS]) {
    uint32_t a, b0;
    place(t, valid, a, b0);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k.X + (uint64_t)a * I * B), 0, (int)xbytes, 0x00020000);
    const uint32_t col = b0 + 4 * li;
    const uint32_t off = (valid && col < B) ? (lg * B + col) * 4 : OOB;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      b[ks] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16 * ks * B), 0, 0);
  };
  // acc[j][rb]: rows 16 rb + 4 lg + v, column b0 + 4 li + j (complex: acc[j + 4][rb]
  // the same with Im M)
  constexpr int NJ = CPLX ? 8 : 4;
  auto multiply = [&](const u32x4 (&b)[NKS], f4 (&acc)[NJ][NRB]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) acc[j][rb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float a[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) a[rb] = at[(rb * NKS + ks) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[j][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rb], __uint_as_float(b[ks][j]),
                                                           acc[j][rb], 0, 0, 0);
      if constexpr (CPLX) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) a[rb] = ati[(rb * NKS + ks) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            acc[j + 4][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                a[rb], __uint_as_float(b[ks][j]), acc[j + 4][rb], 0, 0, 0);
      }
    }
  };
  auto store = [&](uint64_t t, bool valid, const f4 (&acc)[NJ][NRB]) {
    uint32_t a, b0;
    place(t, valid, a, b0);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k.Y + (uint64_t)a * R * B), 0, (int)ybytes, 0x00020000);
    const uint32_t col = b0 + 4 * li;
    const uint32_t off = (valid && col < B) ? (4 * lg * B + col) * 4 : OOB;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float o[4];
        if constexpr (CPLX) {
          // columns 4 li, 4 li + 1 and 4 li + 2, 4 li + 3 are two complex values
          o[0] = acc[0][rb][v] - acc[5][rb][v];
          o[1] = acc[1][rb][v] + acc[4][rb][v];
          o[2] = acc[2][rb][v] - acc[7][rb][v];
          o[3] = acc[3][rb][v] + acc[6][rb][v];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = acc[j][rb][v];
        }
        const u32x4 val = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                           __float_as_uint(o[3])};
        __builtin_amdgcn_raw_buffer_store_b128(val, ry, (int)(off + (16 * rb + v) * B * 4), 0, 0);
      }
  };

  // Each step: the next tile's loads into the other register set, this tile's product,
  // its stores. The first tile is peeled off so that every wait for a tile's operands
  // has the same memory operations behind it (the loads of the next tile and the
  // stores of the previous one), whichever way the loop was entered. A scheduling
  // barrier keeps the compiler from sinking the loads down to their use.
  f4 acc[NJ][NRB];
  u32x4 bA[NKS], bB[NKS];
  load(t0, true, bA);
  load(t0 + TW, t0 + TW < k.ntiles, bB);
  __builtin_amdgcn_sched_barrier(0);
  multiply(bA, acc);
  store(t0, true, acc);
  for (uint64_t t = t0 + TW; t < k.ntiles;) {
    load(t + TW, t + TW < k.ntiles, bA);
    __builtin_amdgcn_sched_barrier(0);
    multiply(bB, acc);
    store(t, true, acc);
    t += TW;
    if (t >= k.ntiles) break;
    load(t + TW, t + TW < k.ntiles, bB);
    __builtin_amdgcn_sched_barrier(0);
    multiply(bA, acc);
    store(t, true, acc);
    t += TW;
  }
}

struct PlanS {
  SPK k;
  bool cplx;
  int nrb, nks;
  int max_wg;
  size_t lds;
  bool ok;
};

PlanS plan_s(const ModeProd& mp) {
  PlanS p{};
  p.ok = false;
  if (mp.in_dt != DT_F32 || mp.apply || !mp.Y) return p;
  const bool cplx = mp.P == 2;
  if (mp.P != 1 && !(cplx && mp.Mre && mp.Mim)) return p;
  // complex: the real view's rows hold 2 B values
  const uint64_t B = cplx ? 2ull * mp.B : (uint64_t)mp.B;
  // rows of 32 values take half a tile: still ahead of the tiled kernel
  if (mp.A == 0 || mp.I == 0 || mp.I > 64 || mp.R == 0 || mp.R > 64 || B < SP_TC / 2) return p;
  // 16-byte pieces: rows of whole pieces, 16-byte aligned tensors; 32-bit byte offsets
  // within one a (buffer extents below 2^31)
  if (B % 4 != 0 || (uintptr_t)mp.X % 16 != 0 || (uintptr_t)mp.Y % 16 != 0) return p;
  if (B * 64 * 4 >= 0x7FFFFFFFull) return p;
  p.cplx = cplx;
  p.nrb = (int)((mp.R + 15) / 16);
  const int ks = (int)((mp.I + 3) / 4);
  p.nks = ks <= 4 ? 4 : ks <= 6 ? 6 : ks <= 8 ? 8 : ks <= 12 ? 12 : 16;
  SPK& k = p.k;
  k.X = (const float*)mp.X;
  k.Y = mp.Y;
  k.M = cplx ? mp.Mre : mp.M;
  k.Mi = cplx ? mp.Mim : nullptr;
  k.A = mp.A;
  k.I = mp.I;
  k.B = (uint32_t)B;
  k.R = mp.R;
  k.tpa = (k.B + SP_TC - 1) / SP_TC;
  k.ntiles = (uint64_t)mp.A * k.tpa;
  p.lds = (size_t)p.nrb * p.nks * 64 * 4 * (cplx ? 2 : 1);
  p.max_wg = mp.max_wg;
  p.ok = true;
  return p;
}

template <int NRB, int NKS, bool CPLX>
hipError_t sp_launch(const PlanS& p, int num_cu, hipStream_t s) {
  auto fn = k_streamprod<NRB, NKS, CPLX>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, SP_NT, p.lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidValue;
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * (uint64_t)per_cu;
  const uint64_t need = (p.k.ntiles + SP_WPB - 1) / SP_WPB;
  if (grid > need) grid = need;
  if (p.max_wg > 0 && grid > (uint64_t)p.max_wg) grid = (uint64_t)p.max_wg;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(SP_NT), p.lds, s, p.k);
  return hipGetLastError();
}
template <int NRB>
hipError_t sp_nks(const PlanS& p, int num_cu, hipStream_t s) {
  if (p.cplx) {
    switch (p.nks) {
      case 4: return sp_launch<NRB, 4, true>(p, num_cu, s);
      case 6: return sp_launch<NRB, 6, true>(p, num_cu, s);
      case 8: return sp_launch<NRB, 8, true>(p, num_cu, s);
      case 12: return sp_launch<NRB, 12, true>(p, num_cu, s);
      default: return sp_launch<NRB, 16, true>(p, num_cu, s);
    }
  }
  switch (p.nks) {
    case 4: return sp_launch<NRB, 4, false>(p, num_cu, s);
    case 6: return sp_launch<NRB, 6, false>(p, num_cu, s);
    case 8: return sp_launch<NRB, 8, false>(p, num_cu, s);
    case 12: return sp_launch<NRB, 12, false>(p, num_cu, s);
    default: return sp_launch<NRB, 16, false>(p, num_cu, s);
  }
}

}  // namespace

bool streamprod_supported(const ModeProd& mp) { return plan_s(mp).ok; }

hipError_t launch_streamprod(const ModeProd& mp, int num_cu, hipStream_t s) {
  const PlanS p = plan_s(mp);
  if (!p.ok) return hipErrorInvalidValue;
  switch (p.nrb) {
    case 1: return sp_nks<1>(p, num_cu, s);
    case 2: return sp_nks<2>(p, num_cu, s);
    case 3: return sp_nks<3>(p, num_cu, s);
    default: return sp_nks<4>(p, num_cu, s);
  }
}

}  // namespace tg
