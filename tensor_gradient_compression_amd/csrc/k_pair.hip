// Two neighbouring mode products in one launch, for modes followed by a long trailing
// part: the leading compressed modes of the projection (after the trailing modes have
// been contracted) and of the reconstruction (before the trailing ones are expanded).
//
// Same products as one launch per mode (pith.science "What carries the argument":
// projection to the core and reconstruction by mode-wise products; appendix M
// Theorem 2), on the fp32 tensor viewed as (A, I0, I1, C):
//   Y[a, j0, j1, c] = sum_i0 M0[j0, i0] sum_i1 M1[j1, i1] X[a, i0, i1, c]
// with the inner sum Z[i0] = M1 X[a, i0, :, c-block] formed per i0 and never written to
// HBM, so the tensor between the two modes (61 MB for the largest workload) is neither
// written nor read back.
//
// Organisation. A workgroup of 4 waves owns 16 consecutive columns c of one a and all
// rows j0, so it applies where the J0 x J1 x 16 accumulators fit in registers (the
// projection's contracting pairs; an expanding pair would need its rows split over
// workgroups, each repeating the first product: measured slower than one launch per
// mode, so that form is not used). It walks i0 in groups of four. The DMA engine brings
// X[a, i0 .. i0+3, :, c-block] in 16-byte pieces into two LDS buffers. Wave w forms
// Z[i0 + w] = M1 X[i0 + w] on v_mfma_f32_16x16x4_f32, with M1 held in registers, and
// leaves it in LDS; every wave adds a group's rank-4 update Y[j0, (j1, c)] +=
// M0[j0, i0 .. i0+3] Z[.., j1, c] to the 16 x 16 output tiles it owns, one MFMA each.
// The two products are software-pipelined over two Z copies: after the one barrier of
// group g, the waves form group g + 1's Z and add group g's update while group g + 2
// arrives. Accumulation is fp32 throughout, as in the single-mode kernel. The output
// leaves in 64-byte row pieces. Neighbouring column blocks share 128-byte lines and are
// placed on one XCD (see the block mapping). At 57 KB of LDS and 156 + 88 registers two
// workgroups fit a CU, which holds the largest workload's 468 in one round. Its
// transfers alone take 35 us; the fp32 MFMA work is 2.9 GFLOP (19 us at the MFMA peak).
#include <algorithm>

#include "tg_common.h"

namespace tg {

namespace {

constexpr int PW_NT = 256;          // 4 waves
constexpr int PW_CB = 16;           // columns c per workgroup
constexpr int PW_TILES = 16;        // output tiles per wave (at most)

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
#define LDS __attribute__((address_space(3)))

struct PWK {
  const float* X;
  float* Y;
  const float* M0;   // J0 x I0
  const float* M1;   // J1 x I1
  uint64_t C;        // trailing columns
  uint32_t A, I0, I1, J0, J1;
  uint32_t JB;       // rows j0 a workgroup owns (16 or 32, a multiple of 16)
  uint32_t ncb;      // column blocks per a
  uint32_t njb;      // j0 blocks
  uint32_t xbuf;                    // bytes of one X buffer (two, at 0 and xbuf)
  uint32_t off_z, off_m0;           // LDS byte offsets
};

// NRB1 = J1 / 16 row blocks of Z (<= 4); KS1 = I1 / 4 k-steps of the first product.
template <int NRB1, int KS1>
__global__ void __launch_bounds__(PW_NT) k_pair(PWK k) {
  extern __shared__ f4 smem_pw[];
  LDS unsigned char* const lds = (LDS unsigned char*)smem_pw;
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I0 = k.I0, I1 = k.I1, J0 = k.J0, J1 = k.J1, JB = k.JB;

  // block -> (a, column block, j0 block). Two neighbouring column blocks read the two
  // 64-byte halves of the same 128-byte lines: they go to blocks b and b + 8, which the
  // dispatcher places on the same XCD (blocks go round-robin over the 8 XCDs) at about
  // the same time, so the line crosses HBM into that XCD's L2 once. Blocks of the last
  // partial run of 16 keep their own index.
  uint32_t b = blockIdx.x;
  const uint32_t full = gridDim.x & ~15u;
  if (b < full) {
    const uint32_t q = b >> 4, h = (b >> 3) & 1, x = b & 7;
    b = 16 * q + 2 * x + h;
  }
  const uint32_t jb = b % k.njb;
  b /= k.njb;
  const uint32_t cbk = b % k.ncb;
  const uint32_t a = b / k.ncb;
  const uint64_t c0 = (uint64_t)cbk * PW_CB;
  const uint32_t j00 = jb * JB;
  const float* const Xa = k.X + (uint64_t)a * I0 * I1 * k.C + c0;

  // LDS layouts chosen so that the 16-lane groups of a read fall in different banks:
  //   Z[t][j1][c] at t ZT + 16 j1 + c (ZT = 16 J1p + 16); one copy serves every group,
  //   as the barrier that opens group g + 1 follows every read of group g's Z;
  //   M0 transposed, M0[j0][i0] at i0 JB + j0
  constexpr uint32_t J1p = 16 * NRB1, ZR = 16, ZT = J1p * ZR + 16;
  LDS float* const zs = (LDS float*)(lds + k.off_z);
  LDS float* const m0s = (LDS float*)(lds + k.off_m0);
  const uint32_t MS = JB;
  for (uint32_t q = tid; q < JB * I0; q += PW_NT) {
    const uint32_t r = q / I0, i = q - r * I0;
    m0s[i * MS + r] = j00 + r < J0 ? k.M0[(j00 + r) * I0 + i] : 0.0f;
  }
  // M1 as the first product's A operand: lane (li, lg) of k-step s holds
  // M1[16 rb + li][4 s + lg]
  float m1[NRB1][KS1];
#pragma unroll
  for (int rb = 0; rb < NRB1; ++rb)
#pragma unroll
    for (int s = 0; s < KS1; ++s) {
      const uint32_t j1 = 16 * rb + li, i1 = 4 * s + lg;
      m1[rb][s] = (j1 < J1 && i1 < I1) ? k.M1[j1 * I1 + i1] : 0.0f;
    }

  // X[a, i0 .. i0+3, i1, c0 .. c0+15] into buffer `buf`: piece p = (t, i1, quarter);
  // 16 I1 pieces, so every thread issues exactly PER of them (I1 = 4 KS1)
  constexpr int PER = KS1 / 4;
  static_assert(KS1 % 4 == 0, "I1 must be a multiple of 16");
  auto issue = [&](uint32_t g, uint32_t buf) {
    LDS unsigned char* const dst = lds + buf * k.xbuf;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const uint32_t p0 = wv * 64 + PW_NT * m, p = p0 + lane;
      const uint32_t t = p / (4 * I1), rem = p - t * 4 * I1;
      const uint32_t i1 = rem >> 2, qq = rem & 3;
      __builtin_amdgcn_global_load_lds(
          (const void*)(Xa + ((uint64_t)(4 * g + t) * I1 + i1) * k.C + 4 * qq),
          (lds_void*)(dst + (size_t)p0 * 16), 16, 0, 0);
    }
  };

  // output tiles of this wave: tile u = wv + 4 m, row block u / J1, j1 = u % J1 (wave
  // uniform). Tiles past the last one repeat it and are not stored, so the group loop has
  // no branch around its MFMAs.
  const uint32_t ntiles = (JB / 16) * J1;
  uint32_t t_ab[PW_TILES], t_b[PW_TILES];   // LDS float offsets of each tile's operands
#pragma unroll
  for (int m = 0; m < PW_TILES; ++m) {
    const uint32_t u = min(wv + 4 * m, ntiles - 1);
    const uint32_t r = u / J1, j1 = u - r * J1;
    t_ab[m] = __builtin_amdgcn_readfirstlane(16 * r);
    t_b[m] = __builtin_amdgcn_readfirstlane(j1 * 16);
  }
  f4 acc[PW_TILES];
#pragma unroll
  for (int m = 0; m < PW_TILES; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  const uint32_t ng = I0 / 4;
  // first product of group gg: wave wv forms Z[i0 = 4 gg + wv] from X buffer xb into Z copy
  // zb (even and odd k-steps in separate accumulators: twice the independent MFMA chains)
  auto first = [&](uint32_t xb, uint32_t zb) {
    const LDS float* const xt = (const LDS float*)(lds + xb * k.xbuf) + wv * I1 * 16;
    f4 z[NRB1], z2[NRB1];
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) z[rb] = z2[rb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS1; ++s) {
      const float xb2 = xt[(4 * s + lg) * 16 + li];
#pragma unroll
      for (int rb = 0; rb < NRB1; ++rb) {
        if (s & 1) z2[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(m1[rb][s], xb2, z2[rb], 0, 0, 0);
        else z[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(m1[rb][s], xb2, z[rb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) z[rb] += z2[rb];
    // Z[t = wv][j1][c]: the result rows are j1 = 16 rb + 4 lg + v, column c = li
    LDS float* const zw = zs + zb * 4 * ZT + wv * ZT;
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) zw[(16 * rb + 4 * lg + v) * ZR + li] = z[rb][v];
  };
  // second product of group g: tile (row block r, j1) += M0[16 r + li][4 g + lg] Z[lg][j1][li]
  auto second = [&](uint32_t g, uint32_t zb) {
    const LDS float* const zg = zs + zb * 4 * ZT + lg * ZT + li;
    const LDS float* const mg = m0s + (4 * g + lg) * MS + li;
#pragma unroll
    for (int m = 0; m < PW_TILES; ++m)
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(mg[t_ab[m]], zg[t_b[m]], acc[m], 0, 0, 0);
  };

  // Software pipeline, one barrier a group: while the DMA engine brings group g + 2, each
  // wave forms group g + 1's Z (into the other Z copy) and adds group g's update, so the
  // two products' MFMAs interleave. The barrier that opens group g follows every read of
  // X[g] (group g's first product ran a group earlier) and of the Z copy group g + 1
  // writes (group g - 1's second product).
  // the M0 and M1 loads above retire before the first transfer is waited for
  __builtin_amdgcn_s_waitcnt(0);
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  if (ng > 1) issue(1, 1);
  first(0, 0);
  for (uint32_t g = 0; g < ng; ++g) {
    // this thread's pieces of group g + 1 and its Z writes of group g are done; after the
    // barrier everyone's are
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (g + 2 < ng) issue(g + 2, g & 1);
    if (g + 1 < ng) first((g + 1) & 1, (g + 1) & 1);
    second(g, g & 1);
  }
  // Y[a, j0, j1, c0 + li], j0 = j00 + 16 r + 4 lg + v
  float* const Ya = k.Y + (uint64_t)a * J0 * J1 * k.C + c0;
#pragma unroll
  for (int m = 0; m < PW_TILES; ++m) {
    const uint32_t u = wv + 4 * m;
    if (u < ntiles) {
      const uint32_t r = u / J1, j1 = u - r * J1;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t j0 = j00 + 16 * r + 4 * lg + v;
        if (j0 < J0) Ya[((uint64_t)j0 * J1 + j1) * k.C + li] = acc[m][v];
      }
    }
  }
}

struct PairPlan {
  bool ok;
  PWK k;
  size_t lds;
  uint32_t grid;
  int nrb1, ks1;
};

PairPlan pair_plan(const ModePair& mp) {
  PairPlan p{};
  p.ok = false;
  if (mp.A == 0 || mp.C == 0 || mp.C % PW_CB != 0) return p;
  if (mp.I0 == 0 || mp.I1 == 0 || mp.J0 == 0 || mp.J1 == 0) return p;
  // whole groups of four i0 (a partial group would multiply stale staged values by the
  // zero rows of M0, which a NaN there would not survive) and of four i1
  if (mp.I0 > 64 || mp.I1 > 64 || mp.J0 > 64 || mp.J1 > 64 || mp.I0 % 4 || mp.I1 % 16)
    return p;
  if ((uintptr_t)mp.X % 16 != 0 || (uintptr_t)mp.Y % 4 != 0) return p;
  PWK& k = p.k;
  k.X = mp.X;
  k.Y = mp.Y;
  k.M0 = mp.M0;
  k.M1 = mp.M1;
  k.C = mp.C;
  k.A = mp.A;
  k.I0 = mp.I0;
  k.I1 = mp.I1;
  k.J0 = mp.J0;
  k.J1 = mp.J1;
  p.nrb1 = (int)((mp.J1 + 15) / 16);
  p.ks1 = (int)(mp.I1 / 4);
  // rows j0 per workgroup: as many 16-row blocks as keep (JB / 16) * J1 <= 4 PW_TILES
  const uint32_t nj0b = (mp.J0 + 15) / 16;
  uint32_t per = (uint32_t)(4 * PW_TILES) / mp.J1;
  if (per == 0) return p;
  if (per > nj0b) per = nj0b;
  k.JB = 16 * per;
  k.njb = (nj0b + per - 1) / per;
  if (k.njb != 1) return p;   // all rows j0 in one workgroup (see the organisation note)
  k.ncb = (uint32_t)(mp.C / PW_CB);
  const uint64_t grid = (uint64_t)mp.A * k.ncb * k.njb;
  if (grid > 0x7FFFFFFFull) return p;
  p.grid = (uint32_t)grid;
  const uint32_t xbuf = 4 * mp.I1 * PW_CB * 4;          // bytes of one X buffer
  const uint32_t ZT = 16 * (uint32_t)p.nrb1 * 16 + 16;   // floats of one Z slice (k_pair)
  k.xbuf = xbuf;
  k.off_z = 2 * xbuf;
  k.off_m0 = k.off_z + 2 * 4 * ZT * 4;   // two copies of the four Z slices
  p.lds = k.off_m0 + (size_t)mp.I0 * k.JB * 4;
  p.ok = p.lds <= 160 * 1024;
  return p;
}

template <int NRB1, int KS1>
hipError_t go_pair(const PairPlan& p, hipStream_t s) {
  auto fn = k_pair<NRB1, KS1>;
  if (p.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute((const void*)fn,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)p.lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(p.grid), dim3(PW_NT), p.lds, s, p.k);
  return hipGetLastError();
}

template <int NRB1>
hipError_t pick_pair(const PairPlan& p, hipStream_t s) {
  switch (p.ks1) {
    case 4: return go_pair<NRB1, 4>(p, s);
    case 8: return go_pair<NRB1, 8>(p, s);
    case 12: return go_pair<NRB1, 12>(p, s);
    case 16: return go_pair<NRB1, 16>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool pair_supported(const ModePair& mp) {
  const PairPlan p = pair_plan(mp);
  // the first product's k-steps are a kernel parameter: I1 in {16, 32, 48, 64}
  const int ks = p.ks1;
  return p.ok && (ks == 4 || ks == 8 || ks == 12 || ks == 16) && p.nrb1 <= 4;
}

hipError_t launch_pair(const ModePair& mp, hipStream_t s) {
  const PairPlan p = pair_plan(mp);
  if (!p.ok) return hipErrorInvalidValue;
  switch (p.nrb1) {
    case 1: return pick_pair<1>(p, s);
    case 2: return pick_pair<2>(p, s);
    case 3: return pick_pair<3>(p, s);
    case 4: return pick_pair<4>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
