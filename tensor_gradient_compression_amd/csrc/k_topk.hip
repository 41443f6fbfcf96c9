// Top-k by magnitude with ties to the lowest linear index, on device, no host sync.
//
// The sparse set Omega of a TensorGRaD refresh is the k largest-|G| entries
// (nullthought summary section 2: top-k gradient elements in COO form; pith.science
// "What carries the argument": Omega chosen by top-k magnitude).
//
// Keys: the storage bit pattern with the sign cleared (an order-preserving integer
// form of |x| for IEEE formats, subnormals kept distinct, NaN above Inf); complex:
// the bits of fl64(re^2 + im^2) (both squares exact in fp64, so one rounding), any
// NaN mapped to the canonical quiet NaN.
//
// Algorithm (all passes re-read G; no key array is stored):
//   1. radix select, most significant 11-bit digit first: per pass, each workgroup
//      builds an LDS histogram of the digit over the elements whose higher digits
//      equal the prefix found so far, and adds it to a global histogram; a one-block
//      kernel walks the bins from the top and fixes the next digit. After the last
//      digit: tau = the k-th largest key, need = how many keys equal to tau are taken.
//   2. count pass: each wave64 counts (key > tau, key == tau) over a unit of 1024
//      consecutive elements.
//   3. scan: one block turns unit counts into each unit's output offset and its
//      number of preceding ties.
//   4. compaction: each wave walks its unit 64 elements at a time; ballots give the
//      in-order rank of every selected element, so Omega comes out ascending. The
//      selection ballot of an aligned 64-element group is also the Omega membership
//      bitmask word, and the running offset its rank word. Optionally the same pass
//      writes the residual (G with Omega zeroed) to a separate buffer.
#include "tg_common.h"

namespace tg {

namespace {

constexpr int DIGIT = 11;
constexpr int NBINS = 1 << DIGIT;
constexpr int UNIT_ITERS = 16;               // 16 x 64 = 1024 elements per wave unit
constexpr uint64_t UNIT = 64ull * UNIT_ITERS;

// state[0] = prefix, state[1] = remaining (ties still to take), state[2] = k
// Per storage type: load the raw element, its key, and store a raw element.
struct KeyF32 {
  static constexpr int BITS = 31;
  typedef uint32_t Raw;
  __device__ static Raw load(const void* G, uint64_t e) { return ((const uint32_t*)G)[e]; }
  __device__ static uint64_t key_of(Raw x) { return (uint64_t)(x & 0x7FFFFFFFu); }
  __device__ static void store(void* R, uint64_t e, Raw x) { ((uint32_t*)R)[e] = x; }
  __device__ static Raw zero() { return 0u; }
  __device__ static uint64_t key(const void* G, uint64_t e) { return key_of(load(G, e)); }
};
struct KeyH16 {
  static constexpr int BITS = 15;
  typedef uint16_t Raw;
  __device__ static Raw load(const void* G, uint64_t e) { return ((const uint16_t*)G)[e]; }
  __device__ static uint64_t key_of(Raw x) { return (uint64_t)(x & 0x7FFFu); }
  __device__ static void store(void* R, uint64_t e, Raw x) { ((uint16_t*)R)[e] = x; }
  __device__ static Raw zero() { return (uint16_t)0; }
  __device__ static uint64_t key(const void* G, uint64_t e) { return key_of(load(G, e)); }
};
struct KeyC64 {
  static constexpr int BITS = 63;
  typedef float2 Raw;
  __device__ static Raw load(const void* G, uint64_t e) { return ((const float2*)G)[e]; }
  __device__ static uint64_t key_of(Raw z) {
    const double re = (double)z.x, im = (double)z.y;
    const double s = re * re + im * im;
    if (s != s) return 0x7FF8000000000000ull;
    return (uint64_t)__double_as_longlong(s) & 0x7FFFFFFFFFFFFFFFull;
  }
  __device__ static void store(void* R, uint64_t e, Raw x) { ((float2*)R)[e] = x; }
  __device__ static Raw zero() { return make_float2(0.0f, 0.0f); }
  __device__ static uint64_t key(const void* G, uint64_t e) { return key_of(load(G, e)); }
};

__global__ void k_topk_init(uint64_t* state, uint32_t* hist, uint32_t k) {
  for (int i = threadIdx.x; i < NBINS; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) {
    state[0] = 0;
    state[1] = k;
    state[2] = k;
    state[3] = 0;
  }
}

template <class K>
__global__ void __launch_bounds__(256) k_topk_hist(const void* __restrict__ G, uint64_t N,
                                                   int shift, int width,
                                                   const uint64_t* __restrict__ state,
                                                   uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[NBINS];
  for (int i = threadIdx.x; i < NBINS; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int hi = shift + width;              // <= 63
  const uint64_t want = state[0] >> hi;
  const uint64_t dmask = (1ull << width) - 1ull;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < N; e += stride) {
    const uint64_t key = K::key(G, e);
    if ((key >> hi) == want) atomicAdd(&h[(key >> shift) & dmask], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (1 << width); i += blockDim.x)
    if (h[i]) atomicAdd(&ghist[i], h[i]);
}

// Fix the next digit; clears the histogram for the next pass.
__global__ void k_topk_select(uint32_t* hist, int shift, int width, uint64_t* state) {
  if (threadIdx.x == 0) {
    const uint64_t rem = state[1];
    uint64_t cum = 0;
    int b = (1 << width) - 1;
    for (; b > 0; --b) {
      const uint64_t c = hist[b];
      if (cum + c >= rem) break;
      cum += c;
    }
    state[0] |= ((uint64_t)b) << shift;
    state[1] = rem - cum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NBINS; i += blockDim.x) hist[i] = 0;
}

template <class K>
__global__ void __launch_bounds__(256) k_topk_count(const void* __restrict__ G, uint64_t N,
                                                    const uint64_t* __restrict__ state,
                                                    uint32_t* __restrict__ ucount,
                                                    uint64_t nunits) {
  const uint64_t unit = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (unit >= nunits) return;   // whole wave exits together
  const uint64_t tau = state[0];
  uint32_t gt = 0, eq = 0;
  for (int it = 0; it < UNIT_ITERS; ++it) {
    const uint64_t e = unit * UNIT + (uint64_t)it * 64 + lane;
    bool pg = false, pe = false;
    typename K::Raw x = K::zero();
    if (e < N) {
      x = K::load(G, e);
      const uint64_t key = K::key_of(x);
      pg = key > tau;
      pe = key == tau;
    }
    gt += (uint32_t)__popcll(__ballot(pg));
    eq += (uint32_t)__popcll(__ballot(pe));
  }
  if (lane == 0) {
    ucount[2 * unit] = gt;
    ucount[2 * unit + 1] = eq;
  }
}

// One block of 1024 threads: exclusive scan of (gt, eq) unit counts.
__global__ void __launch_bounds__(1024) k_topk_scan(const uint32_t* __restrict__ ucount,
                                                    uint64_t nunits,
                                                    const uint64_t* __restrict__ state,
                                                    uint32_t* __restrict__ uoff) {
  __shared__ uint64_t sg[1024], se[1024];
  const int t = threadIdx.x;
  const uint64_t per = (nunits + 1023) / 1024;
  const uint64_t lo = per * t < nunits ? per * t : nunits;
  const uint64_t hi = lo + per < nunits ? lo + per : nunits;
  uint64_t g = 0, q = 0;
  for (uint64_t u = lo; u < hi; ++u) {
    g += ucount[2 * u];
    q += ucount[2 * u + 1];
  }
  sg[t] = g;
  se[t] = q;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    uint64_t ag = 0, aq = 0;
    if (t >= off) {
      ag = sg[t - off];
      aq = se[t - off];
    }
    __syncthreads();
    sg[t] += ag;
    se[t] += aq;
    __syncthreads();
  }
  uint64_t gp = sg[t] - g, qp = se[t] - q;   // exclusive prefixes
  const uint64_t need = state[1];
  for (uint64_t u = lo; u < hi; ++u) {
    uoff[2 * u] = (uint32_t)(gp + (qp < need ? qp : need));
    uoff[2 * u + 1] = (uint32_t)qp;
    gp += ucount[2 * u];
    qp += ucount[2 * u + 1];
  }
}

template <class K>
__global__ void __launch_bounds__(256) k_topk_compact(const void* __restrict__ G, uint64_t N,
                                                      const uint64_t* __restrict__ state,
                                                      const uint32_t* __restrict__ uoff,
                                                      uint64_t nunits, uint64_t k,
                                                      uint32_t* __restrict__ omega,
                                                      uint64_t* __restrict__ mask,
                                                      uint32_t* __restrict__ rank,
                                                      void* __restrict__ resid) {
  const uint64_t unit = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (unit >= nunits) return;
  const uint64_t tau = state[0];
  const uint64_t need = state[1];
  const uint64_t nwords = (N + 63) >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint64_t pos = uoff[2 * unit];
  uint64_t eqrun = uoff[2 * unit + 1];
  for (int it = 0; it < UNIT_ITERS; ++it) {
    const uint64_t w = unit * UNIT_ITERS + it;
    const uint64_t e = w * 64 + lane;
    bool pg = false, pe = false;
    typename K::Raw x = K::zero();
    if (e < N) {
      x = K::load(G, e);
      const uint64_t key = K::key_of(x);
      pg = key > tau;
      pe = key == tau;
    }
    const uint64_t eqb = __ballot(pe);
    const bool take_eq = pe && (eqrun + (uint64_t)__popcll(eqb & lt) < need);
    const bool sel = pg || take_eq;
    const uint64_t selb = __ballot(sel);
    const uint64_t at = pos + (uint64_t)__popcll(selb & lt);
    if (sel && at < k) omega[at] = (uint32_t)e;
    if (resid && e < N) K::store(resid, e, sel ? K::zero() : x);
    if (lane == 0 && w < nwords) {
      mask[w] = selb;
      rank[w] = (uint32_t)pos;
    }
    pos += (uint64_t)__popcll(selb);
    eqrun += (uint64_t)__popcll(eqb);
  }
}

template <class K>
hipError_t run_topk(const void* G, uint64_t N, uint32_t k, const TopkWs& ws, uint32_t* omega,
                    uint64_t* mask, uint32_t* rank, void* resid, hipStream_t s,
                    void (*mark)(void*, int, bool), void* mctx) {
  auto M = [&](int id, bool b) { if (mark) mark(mctx, id, b); };
  hipError_t err;
  M(KID_TOPK_INIT, true);
  k_topk_init<<<1, 256, 0, s>>>(ws.state, ws.hist, k);
  M(KID_TOPK_INIT, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  uint64_t hb = (N + 256ull * 16 - 1) / (256ull * 16);
  if (hb > 4096) hb = 4096;
  if (hb < 1) hb = 1;
  for (int pass = 0;; ++pass) {
    int top = K::BITS - DIGIT * pass;         // bits above this digit already fixed
    if (top <= 0) break;
    int width = top < DIGIT ? top : DIGIT;
    int shift = top - width;
    M(KID_TOPK_HIST, true);
    k_topk_hist<K><<<(unsigned)hb, 256, 0, s>>>(G, N, shift, width, ws.state, ws.hist);
    M(KID_TOPK_HIST, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    M(KID_TOPK_SELECT, true);
    k_topk_select<<<1, 256, 0, s>>>(ws.hist, shift, width, ws.state);
    M(KID_TOPK_SELECT, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const uint64_t nunits = topk_units(N);
  const unsigned ub = (unsigned)((nunits + 3) / 4);
  M(KID_TOPK_COUNT, true);
  k_topk_count<K><<<ub, 256, 0, s>>>(G, N, ws.state, ws.ucount, nunits);
  M(KID_TOPK_COUNT, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  M(KID_TOPK_SCAN, true);
  k_topk_scan<<<1, 1024, 0, s>>>(ws.ucount, nunits, ws.state, ws.uoff);
  M(KID_TOPK_SCAN, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  M(KID_TOPK_COMPACT, true);
  k_topk_compact<K><<<ub, 256, 0, s>>>(G, N, ws.state, ws.uoff, nunits, k, omega, mask, rank,
                                       resid);
  M(KID_TOPK_COMPACT, false);
  return hipGetLastError();
}

__global__ void k_mask_from_omega(const uint32_t* __restrict__ omega, uint32_t k,
                                  uint64_t* __restrict__ mask, uint32_t* __restrict__ rank,
                                  uint64_t nwords) {
  const uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= nwords) return;
  const uint64_t base = w * 64;
  uint32_t lo = 0, hi = k;                  // first j with omega[j] >= base
  while (lo < hi) {
    uint32_t mid = lo + ((hi - lo) >> 1);
    if ((uint64_t)omega[mid] < base) lo = mid + 1; else hi = mid;
  }
  rank[w] = lo;
  uint64_t bits = 0;
  for (uint32_t j = lo; j < k && (uint64_t)omega[j] < base + 64; ++j)
    bits |= 1ull << ((uint64_t)omega[j] - base);
  mask[w] = bits;
}

__global__ void k_fill_u32(uint32_t* p, uint64_t n, uint32_t v) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}
__global__ void k_fill_u64(uint64_t* p, uint64_t n, uint64_t v) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

unsigned fill_blocks(uint64_t n) {
  uint64_t b = (n + 255) / 256;
  if (b > 4096) b = 4096;
  return b ? (unsigned)b : 1u;
}

}  // namespace

uint64_t topk_units(uint64_t N) { return (N + UNIT - 1) / UNIT; }

hipError_t launch_topk(int dt, const void* G, uint64_t N, uint32_t k, const TopkWs& ws,
                       uint32_t* omega, uint64_t* mask, uint32_t* rank, void* resid,
                       hipStream_t s, void (*mark)(void*, int, bool), void* mctx) {
  switch (dt) {
    case DT_F32: return run_topk<KeyF32>(G, N, k, ws, omega, mask, rank, resid, s, mark, mctx);
    case DT_F16:
    case DT_BF16: return run_topk<KeyH16>(G, N, k, ws, omega, mask, rank, resid, s, mark, mctx);
    case DT_C64: return run_topk<KeyC64>(G, N, k, ws, omega, mask, rank, resid, s, mark, mctx);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mask_from_omega(const uint32_t* omega, uint32_t k, uint64_t* mask,
                                  uint32_t* rank, uint64_t nwords, hipStream_t s) {
  const unsigned b = (unsigned)((nwords + 255) / 256);
  k_mask_from_omega<<<b ? b : 1, 256, 0, s>>>(omega, k, mask, rank, nwords);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t v, hipStream_t s) {
  if (!n) return hipSuccess;
  k_fill_u32<<<fill_blocks(n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}
hipError_t launch_fill_u64(uint64_t* p, uint64_t n, uint64_t v, hipStream_t s) {
  if (!n) return hipSuccess;
  k_fill_u64<<<fill_blocks(n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace tg
