// The reconstruction's last three modes in one launch, with the sparse merge and the
// weight update (16-bit weights).
//
// Same mathematics as the two-mode reconstruction in k_slab2.hip (pith.science "What
// carries the argument": the update is brought back to full size by one factor product
// per mode; appendix M Theorem 2, "project back"), with the sparse update added after the
// low-rank reconstruction (nullthought summary section 3). A unit is one index of the
// leading modes: its core-side block Z[u] (R0 x R1 x R2, fp32, contiguous) expands to I0
// slabs of I1 x I2, contiguous in W. A workgroup of WPR waves takes one unit at a time
// (units strided over the grid):
//   1. with Z[u] in LDS, the waves form the unit's mode d-2 expansion
//      Y[i0, :] = sum_r0 M0[i0, r0] Z[u][r0, :] for every i0 (the R1 R2 columns in
//      16-column blocks dealt to the waves, all row blocks of a column block in one
//      wave; v_mfma_f32_16x16x4_f32, fp32 accumulators) into an LDS stack;
//   2. one barrier; the next unit's Z block starts to arrive in the Z buffer;
//   3. wave w takes slabs i0 = (I0 / WPR) w + c, one after another without workgroup
//      barriers: it finishes its previous slab, W <- round(W * decay - lr * O), from the
//      O it staged and the weights it loaded into registers a slab ago (16-byte stores),
//      loads the weights of this slab, expands row i0 of the stack over modes d-1 and d
//      as the two-mode reconstruction does (fp32 MFMAs, the factors' per-lane operands
//      in LDS tables) into its staged O, and merges the slab's Omega range (indices and
//      N_S prefetched a slab ahead);
//   4. one barrier (the stack is free and the next Z block has arrived).
// The tensor between modes d-2 and d-1 (I0 R1 R2 values a unit) never leaves the CU.
#include <algorithm>

#include "k_slab_common.h"
#include "tg_common.h"

namespace tg {

namespace {

constexpr int WPR = 12;           // waves per workgroup
constexpr int NTR = WPR * 64;

struct R3K {
  const float* Zin;     // (U, R0, R1, R2) fp32
  void* W;              // (U, I0, I1, I2), updated in place
  const float* M0;      // I0 x R0 (row-major fp32)
  const float* M1;      // I1 x R1
  const float* M2;      // I2 x R2
  const uint64_t* mask;
  const uint32_t* rank;
  const uint32_t* omega;
  const float* S;       // N_S (read)
  float* delta;         // test capture: the fp32 update O is stored here too (else NULL)
  uint64_t kS;          // |Omega|; 0: no sparse part
  uint32_t U, I0, R0, I1, I2, R1, R2;
  uint32_t slab_e;      // I1 * I2
  uint32_t zq;          // 16-byte pieces of a unit's Z block
  uint32_t ks0;         // k-steps of the mode d-2 expansion (even; R0 <= 4 ks0)
  uint32_t off_stack;   // the unit's stack: I0 rows of R1 R2 floats, then 64 trash slots
  uint32_t off_m0;      // M0 copy
  uint32_t off_fac;     // per-lane operand tables of the two trailing products
  uint32_t off_o;       // per-wave O regions (o_wave bytes each)
  uint32_t o_wave;
  uint32_t ly, ydelta, trash;   // O region layout, as the two-mode reconstruction's
  float lr, decay;
};

// NRB1: 16-row blocks of I1 (<= 64); NCB2: 16-column blocks of I2 (<= 32); KS1: fp32
// MFMA k-steps of the mode d-1 product (R1 <= 4 KS1 <= 32); R2 <= 16. FULL: I1 = 16 NRB1
// and R1 = 4 KS1, so that only the last column block of a slab and the columns past R2
// of the stack rows need lane tests (every lane test is a mask the compiler keeps in
// scalar registers across the slab loop).
// CAP: the test capture of the fp32 update is on (its stores are issued only then).
template <typename WT, int NRB1, int NCB2, int KS1, bool FULL, bool CAP>
__global__ void __launch_bounds__(NTR) __attribute__((amdgpu_waves_per_eu(3, 8))) k_rec3s(R3K k) {
  // 16-byte weight pieces a lane holds: a slab has at most 16 NRB1 x 16 NCB2 values
  constexpr int WQ = (NRB1 * NCB2 + 1) / 2;
  extern __shared__ float smem[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LDS unsigned char* const lds = (LDS unsigned char*)smem;
  LDS float* const zs = (LDS float*)lds;
  LDS float* const st = (LDS float*)(lds + k.off_stack);
  LDS float* const m0s = (LDS float*)(lds + k.off_m0);
  // per-lane operand tables: a1t[(rb KS1 + t) 64 + lane] = M1[i1 = 16 rb + lane % 16]
  // [j1 = KS1 (lane / 16) + t]; b2t[(cb 4 + t) 64 + lane] = M2[i2 = 16 cb + lane % 16]
  // [j2 = 4 (lane / 16) + t] (zero outside the factors)
  LDS float* const a1t = (LDS float*)(lds + k.off_fac);
  LDS float* const b2t = a1t + NRB1 * KS1 * 64;
  LDS float* const Ob = (LDS float*)(lds + k.off_o + wv * k.o_wave);   // [I1][I2]
  LDS float* const Yb = Ob + k.ydelta;                                   // pass 1 [i1][ly]
  const uint32_t li = lane & 15, lg = lane >> 4;
  const uint32_t I0 = k.I0, R0 = k.R0, I1 = k.I1, I2 = k.I2, R1 = k.R1, R2 = k.R2, LY = k.ly;
  const uint32_t RC = R1 * R2, slab_e = k.slab_e;
  const uint32_t strash = I0 * RC;             // the stack's trash slots
  const uint64_t N = (uint64_t)k.U * I0 * slab_e;
  const uint64_t kS = k.kS;
  const bool sparse = kS > 0;
  // used only by per-lane arithmetic: kept in vector registers
  const float lr = __builtin_bit_cast(float, in_vgpr(__builtin_bit_cast(uint32_t, k.lr)));
  const float decay = __builtin_bit_cast(float, in_vgpr(__builtin_bit_cast(uint32_t, k.decay)));

  // M0 into LDS (4-byte transfers, I0 R0 <= 2048 values), and the operand tables: every
  // load of a thread issued before its first LDS write (one memory latency in all)
  for (uint32_t q0 = wv * 64; q0 < I0 * R0; q0 += NTR)
    if (q0 + lane < I0 * R0)
      __builtin_amdgcn_global_load_lds(k.M0 + q0 + lane, (lds_void*)(m0s + q0), 4, 0, 0);
  {
    constexpr uint32_t NT1 = NRB1 * KS1 * 64, NTAB = NT1 + NCB2 * 4 * 64;
    constexpr int IT = (int)((NTAB + NTR - 1) / NTR);
    float tv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t q = threadIdx.x + it * NTR;
      const uint32_t l = q & 63, lli = l & 15, llg = l >> 4;
      bool ok;
      const float* src;
      if (q < NT1) {
        const uint32_t rb = (q >> 6) / KS1, t = (q >> 6) - rb * KS1;
        const uint32_t i1 = 16 * rb + lli, j1 = KS1 * llg + t;
        ok = i1 < I1 && j1 < R1;
        src = k.M1 + (ok ? i1 * R1 + j1 : 0);
      } else {
        const uint32_t q2 = (q - NT1) >> 6, cb = q2 >> 2, t = q2 & 3;
        const uint32_t i2 = 16 * cb + lli, j2 = 4 * llg + t;
        ok = q < NTAB && i2 < I2 && j2 < R2;
        src = k.M2 + (ok ? i2 * R2 + j2 : 0);
      }
      const float v = *src;
      tv[it] = ok ? v : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t q = threadIdx.x + it * NTR;
      if (q < NTAB) a1t[q] = tv[it];   // b2t follows a1t
    }
  }

  const uint32_t G = gridDim.x;
  const uint32_t nu = (k.U - 1 - blockIdx.x) / G + 1;
  const uint32_t spw = I0 / WPR;               // slabs of a unit per wave
  const uint32_t cnt = nu * spw;               // slabs of this wave
  const WT* Wg = (const WT*)k.W;
  // unit r of this workgroup: its Z block into the Z buffer (all waves)
  auto zdma = [&](uint32_t r) {
    const float* src = k.Zin + (uint64_t)(blockIdx.x + r * G) * R0 * RC;
    for (uint32_t q0 = wv * 64; q0 < k.zq; q0 += NTR)
      if (q0 + lane < k.zq)
        __builtin_amdgcn_global_load_lds((const unsigned char*)src + (size_t)(q0 + lane) * 16,
                                         (lds_void*)(lds + (size_t)q0 * 16), 16, 0, 0);
  };
  // slab i of this wave (row i0 = spw wv + c of unit i / spw)
  auto slab_of = [&](uint32_t i) -> uint32_t {
    const uint32_t r = i / spw, c = i - r * spw;
    return (blockIdx.x + r * G) * I0 + spw * wv + c;
  };
  // bitmask words and ranks at the start and the end of slab s (vector loads into lanes
  // 0 and 1: they retire on vmcnt, at the next slab's wait; scalar loads would retire on
  // lgkmcnt, so every wait for an LDS read after them would wait for them too), and
  // slab s's Omega range from them
  // the Omega structures' addresses are used only by per-lane loads: they live in
  // vector registers (this kernel runs short of scalar ones)
  const auto maskv = in_vgpr_ptr(k.mask);
  const auto rankv = in_vgpr_ptr(k.rank);
  const auto omegav = in_vgpr_ptr(k.omega);
  const auto Sv = in_vgpr_ptr(k.S);
  auto bounds = [&](uint32_t s, BoundsV& b) {
    b = load_bounds(maskv, rankv, (uint64_t)s * slab_e, slab_e, N, lane);
  };
  auto range = [&](uint32_t s, const BoundsV& b, uint64_t& lo, uint64_t& hi) {
    lo = rank_at(lane_u64(b.m, 0), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 0),
                 (uint64_t)s * slab_e, N, kS);
    hi = rank_at(lane_u64(b.m, 1), (uint32_t)__builtin_amdgcn_readlane((int)b.r, 1),
                 (uint64_t)(s + 1) * slab_e, N, kS);
  };
  // A slab's weights (and the test capture of its update) are reached through buffer
  // resources over the slab alone: piece q >= np lies past the extent, so its load
  // reads zero and its store is dropped, without a per-lane branch (each per-lane branch
  // is a mask the compiler keeps in scalar registers across the loop).
  auto wres = [&](uint32_t s) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(Wg + (uint64_t)s * slab_e), 0,
                                             (int)(slab_e * 2), 0x00020000);
  };
  // the weights of slab s into registers (pieces lane + 64 j), kept as loaded: unpacking
  // them here would make the wave wait for the loads at once; they are used a slab later
  const uint32_t vq = lane * 16;   // byte offset of piece lane; piece lane + 64 j adds 1024 j
  u32x4 wr[WQ];
  auto wload = [&](uint32_t s) {
    const __amdgpu_buffer_rsrc_t rw = wres(s);
#pragma unroll
    for (int j = 0; j < WQ; ++j)
      wr[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(vq + 1024 * j), 0, 0);
  };
  // W <- round(W * decay - lr * O) for slab s from the staged O and the loaded weights,
  // one piece at a time (a scheduling barrier keeps the pieces' LDS reads from being
  // hoisted together, which would hold all of them in registers at once). decay is 1
  // exactly without weight decay, and W * 1 is W: one expression serves both. A piece
  // past the slab reads O slots past this wave's region (the allocation extends far
  // enough for the last wave) and its store is dropped. The test capture of the fp32
  // update (CAP) goes through a resource over the slab's capture values.
  auto epilogue = [&](uint32_t s) {
    const __amdgpu_buffer_rsrc_t rw = wres(s);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(CAP ? k.delta + (uint64_t)s * slab_e : (float*)k.W), 0,
        CAP ? (int)(slab_e * 4) : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < WQ; ++j) {
      const LDS float* const ob = Ob + 8 * (lane + 64 * j);
      const f4 o0 = *(const LDS f4*)ob;
      const f4 o1 = *(const LDS f4*)(ob + 4);
      const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = wr[j][e];
        const float lo = wlo<WT>(w) * decay, hi = whi<WT>(w) * decay;
        out[e] = wpack<WT>(lo - lr * ov[2 * e], hi - lr * ov[2 * e + 1]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(out, rw, (int)(vq + 1024 * j), 0, 0);
      if constexpr (CAP) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0), rd,
                                               (int)(2 * vq + 2048 * j), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1), rd,
                                               (int)(2 * vq + 2048 * j + 16), 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  OmegaPipe op;   // op.bw: bounds of the slab after next
  if (sparse) {
    BoundsV w;
    const uint32_t s0 = slab_of(0);
    bounds(s0, w);
    wait_vm0();
    range(s0, w, op.lo[0], op.hi[0]);
#pragma unroll
    for (int q = 0; q < NOM; ++q) {
      const uint64_t j = op.lo[0] + lane + 64 * q;
      const uint64_t jc = j < kS ? j : kS - 1;
      op.om[0][q] = omegav[jc];
      op.us[0][q] = Sv[jc];
    }
    if (cnt > 1) bounds(slab_of(1), op.bw);
  }
  zdma(0);
  wait_vm0();
  wait_lgkm0();
  wave_fence();
  __builtin_amdgcn_s_barrier();   // Z of the first unit, the M0 copy and the tables in LDS
  wave_fence();

  // 1. the unit's mode d-2 expansion into the stack (Z of the unit in LDS, the stack free)
  const uint32_t ncy = (RC + 15) / 16, nrb0 = (I0 + 15) / 16, ks0 = k.ks0;
  auto expand = [&]() {
    for (uint32_t t = wv; t < ncy; t += WPR) {
      const uint32_t col = 16 * t + li;
      f4 acc[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = f4{0.f, 0.f, 0.f, 0.f};
      // two k-steps at a time, their operands read together
      for (uint32_t ks = 0; ks < ks0; ks += 2) {
        float a[4][2], b[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t r0 = 4 * (ks + h) + lg;
          const bool okb = r0 < R0 && col < RC;
          const float bv = zs[okb ? r0 * RC + col : 0];
          b[h] = okb ? bv : 0.0f;
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const uint32_t row = 16 * rb + li;
            const bool oka = (uint32_t)rb < nrb0 && row < I0 && r0 < R0;
            const float av = m0s[oka ? row * R0 + r0 : 0];
            a[rb][h] = oka ? av : 0.0f;
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            if ((uint32_t)rb < nrb0)
              acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rb][h], b[h], acc[rb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        if ((uint32_t)rb < nrb0)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t row = 16 * rb + 4 * lg + v;
            st[(row < I0 && col < RC) ? row * RC + col : strash + lane] = acc[rb][v];
          }
    }
  };

  uint32_t s_prev = 0;
  // slab i of this wave; slot = i % 2 (the Omega slot)
  auto slab = [&](uint32_t i, auto slot) {
    constexpr int cur = decltype(slot)::value, nxt = cur ^ 1;
    const uint32_t c = i % spw;
    if (c == 0) {
      // 2. the stack is complete; every wave is past its reads of this Z block
      wait_lgkm0();
      wave_fence();
      __builtin_amdgcn_s_barrier();
      wave_fence();
    }
    // the previous slab's weights and Omega data, its stores: issued a slab ago
    wait_vm0();
    wave_fence();
    if (c == 0 && i + spw < cnt) zdma(i / spw + 1);   // waited for at the unit's end
    if (i > 0) epilogue(s_prev);
    const uint32_t n = slab_of(i);
    wload(n);
    if (sparse && i + 1 < cnt) {
      const uint32_t n1 = slab_of(i + 1);
      range(n1, op.bw, op.lo[nxt], op.hi[nxt]);
#pragma unroll
      for (int q = 0; q < NOM; ++q) {
        const uint64_t j = op.lo[nxt] + lane + 64 * q;
        const uint64_t jc = j < kS ? j : kS - 1;
        op.om[nxt][q] = omegav[jc];
        op.us[nxt][q] = Sv[jc];
      }
      if (i + 2 < cnt) bounds(slab_of(i + 2), op.bw);
    }
    // 3. modes d-1 and d of row i0 of the stack, then the Omega merge
    const LDS float* const zr = st + (spw * wv + c) * RC;
    float zv[KS1];
    if constexpr (FULL) {
      const bool okc = li < R2;
#pragma unroll
      for (int t = 0; t < KS1; ++t) {
        const float z = zr[okc ? (KS1 * lg + t) * R2 + li : 0];
        zv[t] = okc ? z : 0.0f;
      }
    } else {
#pragma unroll
      for (int t = 0; t < KS1; ++t) {
        const uint32_t j1 = KS1 * lg + t;
        zv[t] = (j1 < R1 && li < R2) ? zr[j1 * R2 + li] : 0.0f;
      }
    }
    f4 acc1[NRB1];
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb) acc1[rb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KS1; ++t)
#pragma unroll
      for (int rb = 0; rb < NRB1; ++rb)
        acc1[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1t[(rb * KS1 + t) * 64 + lane], zv[t],
                                                        acc1[rb], 0, 0, 0);
#pragma unroll
    for (int rb = 0; rb < NRB1; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) Yb[(16 * rb + 4 * lg + v) * LY + li] = acc1[rb][v];
    wave_fence();
    float b2[NCB2][4];
#pragma unroll
    for (int cb = 0; cb < NCB2; ++cb)
#pragma unroll
      for (int t = 0; t < 4; ++t) b2[cb][t] = b2t[(cb * 4 + t) * 64 + lane];
    // Y's block rb is read before O's block rb is written over it (their placement keeps
    // block rb + 1 intact)
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
          if constexpr (FULL) {
            if (cb + 1 < NCB2)
              Ob[i1 * I2 + i2] = acc[cb][v];
            else
              Ob[i2 < I2 ? i1 * I2 + i2 : k.trash + lane] = acc[cb][v];
          } else {
            Ob[(i1 < I1 && i2 < I2) ? i1 * I2 + i2 : k.trash + lane] = acc[cb][v];
          }
        }
    }
    wave_fence();
    if (sparse) {
      // the prefetched entries: all reads, then all writes (distinct elements; lanes past
      // the range use their trash slot)
      const uint64_t e_lo = (uint64_t)n * slab_e;
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
        const uint32_t l = (uint32_t)(omegav[j] - e_lo);
        Ob[l] = Ob[l] + Sv[j];
      }
      wave_fence();
    }
    s_prev = n;
    if (c + 1 == spw && i + 1 < cnt) {
      // 4. every wave is past its reads of the stack; the next Z block has arrived
      wait_vm0();
      wait_lgkm0();
      wave_fence();
      __builtin_amdgcn_s_barrier();
      wave_fence();
      expand();
    }
  };
  expand();
  for (uint32_t i = 0; i < cnt; i += 2) {
    slab(i, Slot<0>{});
    if (i + 1 < cnt) slab(i + 1, Slot<1>{});
  }
  wait_vm0();
  wait_lgkm0();
  epilogue(s_prev);
}

uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

struct Plan3r {
  R3K k;
  size_t lds;
  int nrb1, ncb2, ks1;
  bool ok;
};

// mp: a reconstruction (recon = 1, apply) of the last three modes; I0, I1, I2 are the
// core-side sizes and R0, R1, R2 the full sizes (the fields' convention for recon).
Plan3r plan3r(const ModeProd2& mp) {
  Plan3r p{};
  R3K& k = p.k;
  p.ok = false;
  if (mp.P != 1 || !mp.recon || !mp.apply || mp.in_dt != DT_F32) return p;
  if (mp.w_dt != DT_BF16 && mp.w_dt != DT_F16) return p;
  // kernel names: I = the full-size side, R = the core side
  const uint32_t I0 = mp.R0, I1 = mp.R1, I2 = mp.R2, R0 = mp.I0, R1 = mp.I1, R2 = mp.I2;
  if (I0 == 0 || I0 > 64 || I0 % WPR != 0 || R0 == 0 || R0 > 32) return p;
  // the instantiated tile shapes: I1 in (16, 64], I2 <= 32, R1 in (8, 32], R2 <= 16
  if (I1 <= 16 || I1 > 64 || I2 == 0 || I2 > 32 || R1 <= 8 || R1 > 32 || R2 == 0 || R2 > 16)
    return p;
  const uint32_t slab_e = I1 * I2;
  if (slab_e % 8 != 0) return p;   // 16-byte weight pieces (at most 64 WQ a slab)
  if (((uint64_t)R0 * R1 * R2) % 4 != 0 || mp.A == 0 || mp.A % R0 != 0) return p;
  if ((uintptr_t)mp.X % 16 || (uintptr_t)mp.W % 16) return p;
  k.U = mp.A / R0;
  k.I0 = I0; k.I1 = I1; k.I2 = I2; k.R0 = R0; k.R1 = R1; k.R2 = R2;
  k.slab_e = slab_e;
  k.zq = R0 * R1 * R2 / 4;
  k.ks0 = ((R0 + 7) / 8) * 2;   // even
  p.nrb1 = (int)((I1 + 15) / 16);
  p.ncb2 = (int)((I2 + 15) / 16);
  p.ks1 = (int)((R1 + 3) / 4);
  p.ks1 += p.ks1 & 1;   // 4, 6 or 8
  k.ly = 20;   // pass 1 rows hold j2 < 16 (R2 <= 16), 16-byte aligned
  const uint32_t i1p = 16u * p.nrb1;
  int64_t d = 0;   // O rows of block rb must end before pass 1's block rb + 1 starts
  for (int rb = 0; rb + 1 < p.nrb1; ++rb) {
    const int64_t need = 16ll * (rb + 1) * I2 - 16ll * (rb + 1) * k.ly;
    if (need > d) d = need;
  }
  k.ydelta = (uint32_t)((d + 3) & ~3ll);
  const uint32_t ofl = std::max(slab_e, k.ydelta + i1p * k.ly);
  k.trash = ofl;
  k.o_wave = al16((ofl + 64) * 4);
  k.off_stack = al16(R0 * R1 * R2 * 4);
  k.off_m0 = k.off_stack + al16((I0 * R1 * R2 + 64) * 4);
  k.off_fac = k.off_m0 + al16(I0 * R0 * 4);
  k.off_o = k.off_fac + (uint32_t)(p.nrb1 * p.ks1 + p.ncb2 * 4) * 64 * 4;
  p.lds = (size_t)k.off_o + (size_t)WPR * k.o_wave;
  // the epilogue of the last wave reads up to 8 * 64 WQ floats from its region's start
  const uint32_t wq = (uint32_t)(p.nrb1 * p.ncb2 + 1) / 2;
  const size_t rd_end = (size_t)k.off_o + (size_t)(WPR - 1) * k.o_wave + (size_t)512 * wq * 4;
  if (rd_end > p.lds) p.lds = rd_end;
  p.ok = p.lds <= 160 * 1024;
  return p;
}

template <typename WT, int NRB1, int NCB2, int KS1>
hipError_t rec3_launch(const Plan3r& p, int num_cu, hipStream_t s) {
  const bool full = p.k.I1 == 16u * NRB1 && p.k.R1 == 4u * KS1;
  const bool cap = p.k.delta != nullptr;
  auto fn = full ? (cap ? k_rec3s<WT, NRB1, NCB2, KS1, true, true>
                        : k_rec3s<WT, NRB1, NCB2, KS1, true, false>)
                 : (cap ? k_rec3s<WT, NRB1, NCB2, KS1, false, true>
                        : k_rec3s<WT, NRB1, NCB2, KS1, false, false>);
  if (p.lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NTR, p.lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidValue;
  uint64_t grid = (uint64_t)(num_cu > 0 ? num_cu : 256) * (uint64_t)per_cu;
  if (grid > p.k.U) grid = p.k.U;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(NTR), p.lds, s, p.k);
  return hipGetLastError();
}
template <typename WT, int NRB1, int NCB2>
hipError_t rec3_ks1(const Plan3r& p, int num_cu, hipStream_t s) {
  switch (p.ks1) {
    case 4: return rec3_launch<WT, NRB1, NCB2, 4>(p, num_cu, s);
    case 6: return rec3_launch<WT, NRB1, NCB2, 6>(p, num_cu, s);
    default: return rec3_launch<WT, NRB1, NCB2, 8>(p, num_cu, s);
  }
}
template <typename WT, int NRB1>
hipError_t rec3_ncb(const Plan3r& p, int num_cu, hipStream_t s) {
  if (p.ncb2 == 1) return rec3_ks1<WT, NRB1, 1>(p, num_cu, s);
  return rec3_ks1<WT, NRB1, 2>(p, num_cu, s);
}
template <typename WT>
hipError_t rec3_go(const Plan3r& p, int num_cu, hipStream_t s) {
  switch (p.nrb1) {
    case 2: return rec3_ncb<WT, 2>(p, num_cu, s);
    case 3: return rec3_ncb<WT, 3>(p, num_cu, s);
    default: return rec3_ncb<WT, 4>(p, num_cu, s);
  }
}

}  // namespace

bool rec3_supported(const ModeProd2& mp) { return plan3r(mp).ok; }

hipError_t launch_rec3(const ModeProd2& mp, int num_cu, hipStream_t s) {
  Plan3r p = plan3r(mp);
  if (!p.ok) return hipErrorInvalidValue;
  R3K& k = p.k;
  k.Zin = (const float*)mp.X;
  k.W = mp.W;
  k.M0 = mp.M0;
  k.M1 = mp.M1;
  k.M2 = mp.M2;
  k.mask = mp.mask;
  k.rank = mp.rank;
  k.omega = mp.omega;
  k.S = mp.uS;
  k.delta = mp.delta;
  k.kS = mp.has_sparse ? mp.kS : 0;
  k.lr = mp.lr;
  k.decay = mp.decay;
  return mp.w_dt == DT_BF16 ? rec3_go<bf16_t>(p, num_cu, s) : rec3_go<_Float16>(p, num_cu, s);
}

}  // namespace tg
