// Top-k by magnitude with ties to the lowest linear index, on device, no host sync.
//
// The sparse set Omega of a TensorGRaD refresh is the k largest-|G| entries
// (nullthought summary section 2: top-k gradient elements in COO form; pith.science
// "What carries the argument": Omega chosen by top-k magnitude).
//
// Random sampling, the other choice pith.science names, runs the same selection on
// per-element random keys instead of magnitudes: element e's key is the top 31 bits of
// SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014) applied to the state
// base + 0x9E3779B97F4A7C15 * e, so the k largest keys are a uniform k-subset, and a
// refresh needs no generator state beyond the base (the host derives it from the seed and
// the step). G is then read only to write the residual.
//
// Keys: the storage bit pattern with the sign cleared (an order-preserving integer
// form of |x| for IEEE formats, subnormals kept distinct, NaN above Inf); complex:
// the bits of fl64(re^2 + im^2) (both squares exact in fp64, so one rounding), any
// NaN mapped to the canonical quiet NaN.
//
// Algorithm (all passes re-read G; no key array is stored). Every pass reads G as groups
// of 8 consecutive elements per lane (16 bytes for 16-bit data):
//   1. radix select, most significant 11-bit digit first: per pass, each workgroup
//      builds an LDS histogram of the digit over the elements whose higher digits
//      equal the prefix found so far, and adds it to a global histogram; a one-block
//      kernel walks the bins from the top and fixes the next digit. After the last
//      digit: tau = the k-th largest key, need = how many keys equal to tau are taken.
//      16-bit magnitude keys (15 bits) take one pass instead of two: one workgroup per
//      CU holds the histogram of the whole key (32768 bins, 128 KB of LDS) and adds its
//      nonzero bins to the global one.
//   2. count pass: each wave counts (key > tau, key == tau) over a unit of 1024
//      consecutive elements.
//   3. scan: one block turns unit counts into each unit's output offset and its
//      number of preceding ties, a chunk of units at a time.
//   4. compaction: each wave walks its unit 512 elements at a time; prefix sums of the
//      lanes' counts give the in-order rank of every selected element (ties taken in
//      index order), so Omega comes out ascending. Each lane writes its 8 membership
//      bits as one byte of the bitmask, the lane that starts a 64-element word writes
//      that word's rank, and optionally the residual (G with Omega zeroed) goes to a
//      separate buffer.
// G must be 16-byte aligned.
#include "tg_common.h"

namespace tg {

namespace {

constexpr int DIGIT = 11;
constexpr int NBINS = 1 << DIGIT;
constexpr int NB15 = 1 << 15;                // whole 16-bit magnitude keys
constexpr int NT15 = 1024;                   // threads of the one-pass histogram
static_assert(NB15 <= TOPK_HIST_BINS, "the global histogram holds every 15-bit key");
constexpr int UNIT_ITERS = 2;                // 2 x 64 lanes x 8 = 1024 elements per wave unit
constexpr uint64_t UNIT = 512ull * UNIT_ITERS;

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
  __device__ static void load8(const void* G, uint64_t e0, Raw* x) {
    const uint4 a = ((const uint4*)((const uint32_t*)G + e0))[0];
    const uint4 b = ((const uint4*)((const uint32_t*)G + e0))[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ static void store8(void* R, uint64_t e0, const Raw* x) {
    ((uint4*)((uint32_t*)R + e0))[0] = make_uint4(x[0], x[1], x[2], x[3]);
    ((uint4*)((uint32_t*)R + e0))[1] = make_uint4(x[4], x[5], x[6], x[7]);
  }
};
struct KeyH16 {
  static constexpr int BITS = 15;
  typedef uint16_t Raw;
  __device__ static Raw load(const void* G, uint64_t e) { return ((const uint16_t*)G)[e]; }
  __device__ static uint64_t key_of(Raw x) { return (uint64_t)(x & 0x7FFFu); }
  __device__ static void store(void* R, uint64_t e, Raw x) { ((uint16_t*)R)[e] = x; }
  __device__ static Raw zero() { return (uint16_t)0; }
  __device__ static uint64_t key(const void* G, uint64_t e) { return key_of(load(G, e)); }
  __device__ static void load8(const void* G, uint64_t e0, Raw* x) {
    const uint4 a = *(const uint4*)((const uint16_t*)G + e0);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = (uint16_t)(w[j] & 0xFFFFu);
      x[2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __device__ static void store8(void* R, uint64_t e0, const Raw* x) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)x[2 * j] | ((uint32_t)x[2 * j + 1] << 16);
    *(uint4*)((uint16_t*)R + e0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
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
  __device__ static void load8(const void* G, uint64_t e0, Raw* x) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = ((const float4*)((const float2*)G + e0))[j];
      x[2 * j] = make_float2(v.x, v.y);
      x[2 * j + 1] = make_float2(v.z, v.w);
    }
  }
  __device__ static void store8(void* R, uint64_t e0, const Raw* x) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ((float4*)((float2*)R + e0))[j] =
          make_float4(x[2 * j].x, x[2 * j].y, x[2 * j + 1].x, x[2 * j + 1].y);
  }
};

__device__ __forceinline__ uint64_t rand_key(uint64_t base, uint64_t e) {
  uint64_t z = base + 0x9E3779B97F4A7C15ull * e;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z >> 33;
}

// The 8 consecutive elements e0 .. e0 + 7 (e0 a multiple of 8, G 16-byte aligned);
// past N they read as zero keys and are never selected.
template <class K>
__device__ __forceinline__ void load_group(const void* G, uint64_t N, uint64_t e0,
                                           typename K::Raw* x) {
  if (e0 + 8 <= N) {
    K::load8(G, e0, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = e0 + j < N ? K::load(G, e0 + j) : K::zero();
  }
}

__global__ void k_topk_init(uint64_t* state, uint32_t* hist, uint32_t k) {
  for (int i = threadIdx.x; i < TOPK_HIST_BINS; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) {
    state[0] = 0;
    state[1] = k;
    state[2] = k;
    state[3] = 0;
  }
}

template <class K, bool RK>
__global__ void __launch_bounds__(256) k_topk_hist(const void* __restrict__ G, uint64_t N,
                                                   int shift, int width,
                                                   const uint64_t* __restrict__ state,
                                                   uint32_t* __restrict__ ghist,
                                                   uint64_t rk_base) {
  __shared__ uint32_t h[NBINS];
  for (int i = threadIdx.x; i < NBINS; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int hi = shift + width;              // <= 63
  const uint64_t want = state[0] >> hi;
  const uint64_t dmask = (1ull << width) - 1ull;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t ngroups = (N + 7) / 8;
  for (uint64_t gi = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < ngroups;
       gi += stride) {
    typename K::Raw x[8];
    if constexpr (!RK) load_group<K>(G, N, gi * 8, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t key;
      if constexpr (RK) key = rand_key(rk_base, gi * 8 + j);
      else key = K::key_of(x[j]);
      if (gi * 8 + j < N && (key >> hi) == want) atomicAdd(&h[(key >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (1 << width); i += blockDim.x)
    if (h[i]) atomicAdd(&ghist[i], h[i]);
}

// The whole 15-bit key of every element in one pass (K = KeyH16): the LDS histogram of
// a workgroup per CU, whose nonzero bins are added to the global one. Two groups of 8
// elements per iteration, both loaded before the first LDS atomic (four measured
// slower).
template <class K>
__global__ void __launch_bounds__(NT15) k_topk_hist15(const void* __restrict__ G, uint64_t N,
                                                      uint32_t* __restrict__ ghist) {
  extern __shared__ uint32_t h15[];
  for (int i = threadIdx.x; i < NB15; i += NT15) h15[i] = 0;
  __syncthreads();
  const uint64_t stride = (uint64_t)gridDim.x * NT15;
  const uint64_t ngroups = (N + 7) / 8;
  uint64_t gi = (uint64_t)blockIdx.x * NT15 + threadIdx.x;
  auto add = [&](uint64_t g, const typename K::Raw* x) {
    if (g * 8 + 8 <= N) {
#pragma unroll
      for (int j = 0; j < 8; ++j) atomicAdd(&h15[K::key_of(x[j])], 1u);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (g * 8 + j < N) atomicAdd(&h15[K::key_of(x[j])], 1u);
    }
  };
  for (; gi + stride < ngroups; gi += 2 * stride) {
    typename K::Raw x[8], y[8];
    load_group<K>(G, N, gi * 8, x);
    load_group<K>(G, N, (gi + stride) * 8, y);
    add(gi, x);
    add(gi + stride, y);
  }
  if (gi < ngroups) {
    typename K::Raw x[8];
    load_group<K>(G, N, gi * 8, x);
    add(gi, x);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB15; i += NT15)
    if (h15[i]) atomicAdd(&ghist[i], h15[i]);
}

// Fix the next digit and (CLEAR) clear the histogram for the next pass. The digit is
// the highest bin b whose count, added to the counts of all higher bins, reaches the
// number of keys still to take (bin 0 if none does); NT threads own NB / NT consecutive
// bins each and a suffix scan over the threads (shuffles within a wave, then over the
// waves' totals) locates that bin. Counts fit 32 bits: N < 2^32.
template <int NT, int NB, bool CLEAR>
__global__ void __launch_bounds__(NT) k_topk_select(uint32_t* hist, int shift, int width,
                                                    uint64_t* state) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t wsum[NW + 1];
  __shared__ int found_b;
  __shared__ uint32_t found_cum;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nb = 1 << width;
  constexpr int PER = NB / NT;
  const int b0 = t * PER;
  static_assert(PER % 4 == 0, "bins are read four at a time");
  uint32_t c[PER];
  uint32_t mine = 0;
  if (b0 + PER <= nb) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const uint4 v = *(const uint4*)(hist + b0 + i);   // 16-byte aligned: PER % 4 == 0
      c[i] = v.x; c[i + 1] = v.y; c[i + 2] = v.z; c[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) c[i] = b0 + i < nb ? hist[b0 + i] : 0u;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += c[i];
  // x: the sum over the lanes >= lane of this wave
  uint32_t x = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off, 64);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wsum[w] = x;
  if (t == 0) found_b = -1;
  __syncthreads();
  if (t == 0) {
    uint32_t acc = 0;
    wsum[NW] = 0;
    for (int v = NW - 1; v >= 0; --v) {
      acc += wsum[v];
      wsum[v] = acc;            // the sum over waves >= v
    }
  }
  __syncthreads();
  const uint32_t rem = (uint32_t)state[1];
  const uint32_t above = x - mine + wsum[w + 1];   // bins owned by higher threads
  if (above < rem && above + mine >= rem) {
    uint32_t cum = above;
    for (int i = PER - 1; i >= 0; --i) {
      const int b = b0 + i;
      if (b == 0 || cum + c[i] >= rem) {
        found_b = b;
        found_cum = cum;
        break;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  if (t == 0) {
    int b = found_b;
    uint32_t cum = found_cum;
    if (b < 0) {             // never reached: bin 0, with every higher bin counted
      b = 0;
      cum = wsum[0] - (nb > 0 ? hist[0] : 0u);
    }
    state[0] |= ((uint64_t)b) << shift;
    state[1] = rem - cum;
  }
  if constexpr (CLEAR) {
    __syncthreads();
    for (int i = t; i < NB; i += NT) hist[i] = 0;
  }
}

int cu_count() {
  static int n = 0;
  if (!n) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        c > 0)
      n = c;
    else
      return 256;
  }
  return n;
}

template <class K, bool RK>
__global__ void __launch_bounds__(256) k_topk_count(const void* __restrict__ G, uint64_t N,
                                                    const uint64_t* __restrict__ state,
                                                    uint32_t* __restrict__ ucount,
                                                    uint64_t nunits, uint64_t rk_base) {
  const uint64_t unit = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (unit >= nunits) return;   // whole wave exits together
  const uint64_t tau = state[0];
  uint32_t gt = 0, eq = 0;
  for (int it = 0; it < UNIT_ITERS; ++it) {
    const uint64_t e0 = unit * UNIT + (uint64_t)it * 512 + (uint64_t)lane * 8;
    typename K::Raw x[8];
    if constexpr (!RK) load_group<K>(G, N, e0, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t key;
      if constexpr (RK) key = rand_key(rk_base, e0 + j);
      else key = K::key_of(x[j]);
      const bool in = e0 + j < N;
      gt += (in && key > tau) ? 1u : 0u;
      eq += (in && key == tau) ? 1u : 0u;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off, 64);
    eq += __shfl_xor(eq, off, 64);
  }
  if (lane == 0) {
    ucount[2 * unit] = gt;
    ucount[2 * unit + 1] = eq;
  }
}

// Exclusive scan of the (gt, eq) unit counts in chunks of 1024 x SCAN_V consecutive units
// (each thread SCAN_V of them, loaded as 16-byte pieces), one block of 1024 threads per
// chunk: k_topk_chunk_tot sums each chunk, k_topk_scan adds the totals of the chunks
// before its own and scans it.
// uoff[2u] = selected elements before unit u = gt before + min(eq before, need);
// uoff[2u + 1] = ties before unit u. (N < 2^32, so every count fits in 32 bits.)
constexpr int SCAN_V = 8;
constexpr uint32_t SCAN_CH = 1024u * SCAN_V;
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sw, uint32_t& total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sw[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t y = sw[w];
    before += w < wave ? y : 0u;
    total += y;
  }
  __syncthreads();
  return before + x - v;
}

// this thread's SCAN_V unit counts of the chunk at unit c0 (zeros past the end)
__device__ __forceinline__ void scan_load(const uint32_t* __restrict__ ucount, uint32_t nu,
                                          uint32_t c0, uint4* v) {
  const uint32_t u0 = c0 + (uint32_t)threadIdx.x * SCAN_V;
#pragma unroll
  for (int q = 0; q < SCAN_V / 2; ++q) {
    const uint32_t u = u0 + 2 * q;
    if (u + 2 <= nu) {
      v[q] = *(const uint4*)(ucount + 2 * (uint64_t)u);
    } else {
      v[q] = make_uint4(u < nu ? ucount[2 * (uint64_t)u] : 0u,
                        u < nu ? ucount[2 * (uint64_t)u + 1] : 0u, 0u, 0u);
    }
  }
}

__global__ void __launch_bounds__(1024) k_topk_chunk_tot(const uint32_t* __restrict__ ucount,
                                                         uint64_t nunits,
                                                         uint32_t* __restrict__ ctot) {
  __shared__ uint32_t sw[16];
  uint4 cur[SCAN_V / 2];
  scan_load(ucount, (uint32_t)nunits, blockIdx.x * SCAN_CH, cur);
  uint32_t g = 0, q = 0;
#pragma unroll
  for (int i = 0; i < SCAN_V / 2; ++i) {
    g += cur[i].x + cur[i].z;
    q += cur[i].y + cur[i].w;
  }
  uint32_t gt_tot, eq_tot;
  block_excl_scan(g, sw, gt_tot);
  block_excl_scan(q, sw, eq_tot);
  if (threadIdx.x == 0) {
    ctot[2 * blockIdx.x] = gt_tot;
    ctot[2 * blockIdx.x + 1] = eq_tot;
  }
}

__global__ void __launch_bounds__(1024) k_topk_scan(const uint32_t* __restrict__ ucount,
                                                    uint64_t nunits,
                                                    const uint32_t* __restrict__ ctot,
                                                    const uint64_t* __restrict__ state,
                                                    uint32_t* __restrict__ uoff) {
  __shared__ uint32_t sw[16];
  const int t = threadIdx.x;
  const uint32_t need = (uint32_t)state[1];
  const uint32_t nu = (uint32_t)nunits;
  const uint32_t c0 = blockIdx.x * SCAN_CH;
  uint4 cur[SCAN_V / 2];
  scan_load(ucount, nu, c0, cur);
  // the counts of every earlier chunk
  uint32_t gb = 0, qb = 0;
  for (uint32_t c = t; c < blockIdx.x; c += 1024) {
    gb += ctot[2 * c];
    qb += ctot[2 * c + 1];
  }
  uint32_t gbase, qbase;
  block_excl_scan(gb, sw, gbase);
  block_excl_scan(qb, sw, qbase);
  uint32_t g = 0, q = 0;
#pragma unroll
  for (int i = 0; i < SCAN_V / 2; ++i) {
    g += cur[i].x + cur[i].z;
    q += cur[i].y + cur[i].w;
  }
  uint32_t gt_tot, eq_tot;
  uint32_t gp = gbase + block_excl_scan(g, sw, gt_tot);
  uint32_t qp = qbase + block_excl_scan(q, sw, eq_tot);
  const uint32_t u0 = c0 + (uint32_t)t * SCAN_V;
#pragma unroll
  for (int i = 0; i < SCAN_V / 2; ++i) {
    const uint32_t u = u0 + 2 * i;
    const uint32_t o0 = gp + (qp < need ? qp : need), e0 = qp;
    gp += cur[i].x;
    qp += cur[i].y;
    const uint32_t o1 = gp + (qp < need ? qp : need), e1 = qp;
    gp += cur[i].z;
    qp += cur[i].w;
    if (u + 2 <= nu) {
      *(uint4*)(uoff + 2 * (uint64_t)u) = make_uint4(o0, e0, o1, e1);
    } else if (u < nu) {
      uoff[2 * (uint64_t)u] = o0;
      uoff[2 * (uint64_t)u + 1] = e0;
    }
  }
}

template <class K, bool RK>
__global__ void __launch_bounds__(256) k_topk_compact(const void* __restrict__ G, uint64_t N,
                                                      const uint64_t* __restrict__ state,
                                                      const uint32_t* __restrict__ uoff,
                                                      uint64_t nunits, uint64_t k,
                                                      uint32_t* __restrict__ omega,
                                                      uint64_t* __restrict__ mask,
                                                      uint32_t* __restrict__ rank,
                                                      void* __restrict__ resid,
                                                      uint64_t rk_base) {
  const uint64_t unit = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (unit >= nunits) return;
  const uint64_t tau = state[0];
  const uint64_t need = state[1];
  const uint64_t nwords = (N + 63) >> 6;
  uint64_t pos = uoff[2 * unit];        // selected elements before this group of 512
  uint64_t eqrun = uoff[2 * unit + 1];  // ties before it
  for (int it = 0; it < UNIT_ITERS; ++it) {
    const uint64_t e0 = unit * UNIT + (uint64_t)it * 512 + (uint64_t)lane * 8;
    typename K::Raw x[8];
    if (!RK || resid) load_group<K>(G, N, e0, x);   // rand-k reads G only for the residual
    uint32_t pg = 0, pe = 0;   // bit j: element e0 + j is > tau / == tau
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t key;
      if constexpr (RK) key = rand_key(rk_base, e0 + j);
      else key = K::key_of(x[j]);
      if (e0 + j < N) {
        pg |= (key > tau ? 1u : 0u) << j;
        pe |= (key == tau ? 1u : 0u) << j;
      }
    }
    // ties and strict selections before this lane's group, in element order
    uint32_t ce = (uint32_t)__popc(pe), cg = (uint32_t)__popc(pg);
    uint32_t xe = ce, xg = cg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t ye = __shfl_up(xe, off, 64), yg = __shfl_up(xg, off, 64);
      if (lane >= off) {
        xe += ye;
        xg += yg;
      }
    }
    const uint32_t te = __shfl(xe, 63, 64), tg = __shfl(xg, 63, 64);
    uint64_t eqb = eqrun + (xe - ce);              // ties before this lane's group
    // selected before this lane's group: strict ones plus the ties taken so far
    const uint64_t taken0 = eqrun < need ? eqrun : need;
    const uint64_t takenb = eqb < need ? eqb : need;
    uint64_t at = pos + (xg - cg) + (takenb - taken0);
    uint32_t sel = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bool sj = (pg >> j) & 1u;
      if ((pe >> j) & 1u) {
        sj = eqb < need;
        ++eqb;
      }
      if (sj) {
        if (at < k) omega[at] = (uint32_t)(e0 + j);
        ++at;
        sel |= 1u << j;
      }
    }
    if (e0 < nwords * 64) {
      ((uint8_t*)mask)[e0 >> 3] = (uint8_t)sel;
      if ((lane & 7) == 0) rank[e0 >> 6] = (uint32_t)(pos + (xg - cg) + (takenb - taken0));
    }
    if (resid && e0 < N) {
      if (e0 + 8 <= N) {
        typename K::Raw y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = ((sel >> j) & 1u) ? K::zero() : x[j];
        K::store8(resid, e0, y);
      } else {
        for (int j = 0; j < 8 && e0 + j < N; ++j)
          K::store(resid, e0 + j, ((sel >> j) & 1u) ? K::zero() : x[j]);
      }
    }
    // the group of 512 after this one
    const uint64_t taken1 = (eqrun + te) < need ? (eqrun + te) : need;
    pos += tg + (taken1 - taken0);
    eqrun += te;
  }
}

template <class K, bool RK>
hipError_t run_topk(const void* G, uint64_t N, uint32_t k, const TopkWs& ws, uint32_t* omega,
                    uint64_t* mask, uint32_t* rank, void* resid, uint64_t rk_base,
                    hipStream_t s, void (*mark)(void*, int, bool), void* mctx) {
  auto M = [&](int id, bool b) { if (mark) mark(mctx, id, b); };
  hipError_t err;
  M(KID_TOPK_INIT, true);
  k_topk_init<<<1, 256, 0, s>>>(ws.state, ws.hist, k);
  M(KID_TOPK_INIT, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  uint64_t hb = (N + 256ull * 16 - 1) / (256ull * 16);
  if (hb > 1024) hb = 1024;
  if (hb < 1) hb = 1;
  if constexpr (!RK && K::BITS == 15) {
    // the whole key in one pass
    err = hipFuncSetAttribute((const void*)k_topk_hist15<K>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, NB15 * 4);
    if (err != hipSuccess) return err;
    uint64_t g15 = ((N + 7) / 8 + NT15 - 1) / NT15;
    if (g15 > (uint64_t)cu_count()) g15 = (uint64_t)cu_count();
    if (g15 < 1) g15 = 1;
    M(KID_TOPK_HIST, true);
    k_topk_hist15<K><<<(unsigned)g15, NT15, NB15 * 4, s>>>(G, N, ws.hist);
    M(KID_TOPK_HIST, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    M(KID_TOPK_SELECT, true);
    k_topk_select<1024, NB15, false><<<1, 1024, 0, s>>>(ws.hist, 0, 15, ws.state);
    M(KID_TOPK_SELECT, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  for (int pass = 0; RK || K::BITS != 15; ++pass) {
    constexpr int BITS = RK ? 31 : K::BITS;
    int top = BITS - DIGIT * pass;            // bits above this digit already fixed
    if (top <= 0) break;
    int width = top < DIGIT ? top : DIGIT;
    int shift = top - width;
    M(KID_TOPK_HIST, true);
    k_topk_hist<K, RK><<<(unsigned)hb, 256, 0, s>>>(G, N, shift, width, ws.state, ws.hist,
                                                    rk_base);
    M(KID_TOPK_HIST, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    M(KID_TOPK_SELECT, true);
    k_topk_select<256, NBINS, true><<<1, 256, 0, s>>>(ws.hist, shift, width, ws.state);
    M(KID_TOPK_SELECT, false);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const uint64_t nunits = topk_units(N);
  const unsigned ub = (unsigned)((nunits + 3) / 4);
  M(KID_TOPK_COUNT, true);
  k_topk_count<K, RK><<<ub, 256, 0, s>>>(G, N, ws.state, ws.ucount, nunits, rk_base);
  M(KID_TOPK_COUNT, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned nch = (unsigned)topk_chunks(N);
  M(KID_TOPK_SCAN, true);
  k_topk_chunk_tot<<<nch, 1024, 0, s>>>(ws.ucount, nunits, ws.ctot);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  k_topk_scan<<<nch, 1024, 0, s>>>(ws.ucount, nunits, ws.ctot, ws.state, ws.uoff);
  M(KID_TOPK_SCAN, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  M(KID_TOPK_COMPACT, true);
  k_topk_compact<K, RK><<<ub, 256, 0, s>>>(G, N, ws.state, ws.uoff, nunits, k, omega, mask,
                                           rank, resid, rk_base);
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

template <int P>
__global__ void __launch_bounds__(256) k_remap_moments(const uint64_t* __restrict__ mask_old,
                                                       const uint32_t* __restrict__ rank_old,
                                                       const uint32_t* __restrict__ om_new,
                                                       uint32_t k,
                                                       const float* __restrict__ m_old,
                                                       const float* __restrict__ v_old,
                                                       float* __restrict__ m_new,
                                                       float* __restrict__ v_new) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < k; j += stride) {
    const uint64_t e = om_new[j];
    const uint64_t word = mask_old[e >> 6];
    const bool kept = (word >> (e & 63)) & 1ull;
    const uint64_t i = kept ? omega_rank(mask_old, rank_old, e, word) : 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      m_new[j * P + p] = kept ? m_old[i * P + p] : 0.0f;
      v_new[j * P + p] = kept ? v_old[i * P + p] : 0.0f;
    }
  }
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
uint64_t topk_chunks(uint64_t N) { return (topk_units(N) + SCAN_CH - 1) / SCAN_CH; }

template <class K>
hipError_t topk_dispatch(const void* G, uint64_t N, uint32_t k, const TopkWs& ws,
                         uint32_t* omega, uint64_t* mask, uint32_t* rank, void* resid,
                         int randk, uint64_t rk_base, hipStream_t s,
                         void (*mark)(void*, int, bool), void* mctx) {
  if (randk) return run_topk<K, true>(G, N, k, ws, omega, mask, rank, resid, rk_base, s, mark, mctx);
  return run_topk<K, false>(G, N, k, ws, omega, mask, rank, resid, 0, s, mark, mctx);
}

hipError_t launch_topk(int dt, const void* G, uint64_t N, uint32_t k, const TopkWs& ws,
                       uint32_t* omega, uint64_t* mask, uint32_t* rank, void* resid,
                       int randk, uint64_t rk_base, hipStream_t s,
                       void (*mark)(void*, int, bool), void* mctx) {
  switch (dt) {
    case DT_F32:
      return topk_dispatch<KeyF32>(G, N, k, ws, omega, mask, rank, resid, randk, rk_base, s,
                                   mark, mctx);
    case DT_F16:
    case DT_BF16:
      return topk_dispatch<KeyH16>(G, N, k, ws, omega, mask, rank, resid, randk, rk_base, s,
                                   mark, mctx);
    case DT_C64:
      return topk_dispatch<KeyC64>(G, N, k, ws, omega, mask, rank, resid, randk, rk_base, s,
                                   mark, mctx);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_remap_moments(const uint64_t* mask_old, const uint32_t* rank_old,
                                const uint32_t* omega_new, uint32_t k, uint32_t P,
                                const float* m_old, const float* v_old, float* m_new,
                                float* v_new, hipStream_t s) {
  if (!k) return hipSuccess;
  uint64_t b = ((uint64_t)k + 255) / 256;
  if (b > 8192) b = 8192;
  if (P == 2)
    k_remap_moments<2><<<(unsigned)b, 256, 0, s>>>(mask_old, rank_old, omega_new, k, m_old,
                                                   v_old, m_new, v_new);
  else
    k_remap_moments<1><<<(unsigned)b, 256, 0, s>>>(mask_old, rank_old, omega_new, k, m_old,
                                                   v_old, m_new, v_new);
  return hipGetLastError();
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
