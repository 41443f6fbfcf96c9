// Host side of libtgrad: the handle, state allocation, and the order of launches for
// one TensorGRaD step and refresh. Every launch goes onto the caller's stream; no host
// synchronisation happens inside tgrad_step or tgrad_refresh.
//
// Step order (nullthought summary section 3; pith.science "What carries the argument"
// and its appendix M excerpt of Theorem 2):
//   [refresh when due] -> gather S = G[Omega], zero G[Omega] -> projection, one mode
//   product per compressed mode (last mode first) -> fused Adam on core and S ->
//   reconstruction, one mode product per compressed mode (first mode first), the last
//   one applying W <- round(W * decay - lr * (Delta_L + lambda N_S at Omega)).
// Refresh: top-k -> Omega (+ bitmask, ranks) -> per compressed mode: Gram of the
//   residual (the gradient read with Omega's entries cleared in the staged tiles) ->
//   eigensolver (tridiagonal route for real modes up to 64, else Jacobi) -> U(n) and
//   operand matrices.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <new>
#include <utility>
#include <string>
#include <vector>

#include "tg_common.h"
#include "tgrad.h"

using namespace tg;

namespace {

struct Rec {
  int id;
  hipEvent_t a, b;
};

// The scratch buffers of a refresh's kernels: the top-k workspace, the Gram partial sums
// and the Gram matrices (one gram_stride-double matrix per compressed mode); `masked`:
// the Gram launches read the gradient with Omega cleared through the bitmask rather than
// a residual copy.
struct RefreshWs {
  tg::TopkWs tw;
  double* gram_part;
  double* gram;
  bool masked;
  uint32_t max_gram_blocks;   // 0: no cap on a Gram launch's partial sums
};

}  // namespace

struct tgrad_handle {
  int device = 0;
  int num_cu = 256;
  int d = 0;
  int64_t shape[TGRAD_MAX_NDIM] = {0};
  int64_t ranks[TGRAD_MAX_NDIM] = {0};
  int dtype = 0;
  uint32_t P = 1;
  uint64_t N = 0, k = 0, ncore = 0, nwords = 0;
  int64_t T = 1;
  double lr = 0, b1 = 0, b2 = 0, eps = 0;
  int64_t t = 0, refreshed_for = 0;
  std::vector<int> fmodes;   // compressed modes, ascending
  bool can_fuse = false;     // last two modes compressed and a slab fits in LDS
  bool fuse = false;         // use the two-mode launches
  bool slab2 = true;         // 16-bit data: the wave-per-slab two-mode kernels where they fit
  bool can_slab3 = false;    // the projection's first launch can also take mode d-3
  bool slab3 = true;         // use it
  bool can_rec3 = false;     // the reconstruction's last launch can also take mode d-3
  bool rec3 = true;          // use it (not under set_fusion 4)
  bool can_gram3 = false;    // refresh: the last three modes' Grams from one read
  bool gram3 = true;         // use it
  // refresh: the Gram kernels read the gradient and clear Omega's entries in their staged
  // tiles through the bitmask, instead of reading a residual copy that the top-k pass
  // writes (the copy is the faster default: 0.10 ms per refresh on the bf16
  // (64,64,48,48,25) tensor)
  bool gram_masked = false;
  void* resid = nullptr;     // refresh: G with Omega zeroed (shares buf's memory)
  bool can_pair = false;     // the fused chains hold two neighbouring leading modes
  bool pairs = true;         // launch those as one (k_pair)
  bool stream = true;        // single fp32 mode products on k_streamprod where it applies
  bool rows = true;          // single last-mode products on k_rowprod where it applies
  int stream_wg = 0;         // test hook: cap on its workgroups (0: none)
  // the sparse values' Adam update on a second stream of the handle, forked after the
  // first projection launch (which writes S) and joined before the reconstruction, so it
  // overlaps the projection's later launches and the core's Adam update (default
  // priority; created at init). 0: never; 1: when k P >= kAdamForkMin (the fork and the
  // join cost about 10 us a step, which only a large sparse update repays: bf16
  // (64,64,48,48,25) 0.749 -> 0.740 ms, fp16 (64,64,64,64) 0.179 -> 0.192 ms); 2: always
  int adam_overlap = 1;
  // refresh: the leading modes' eigensolver beside the three-mode Gram launch
  bool eig_overlap = true;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;

  uint32_t* omega = nullptr;
  uint64_t* mask = nullptr;
  uint32_t* rank = nullptr;
  float *S = nullptr, *mS = nullptr, *vS = nullptr;
  float *core = nullptr, *ucore = nullptr, *mC = nullptr, *vC = nullptr;
  float* buf[2] = {nullptr, nullptr};
  void* gcopy = nullptr;         // step without the folded gather: the residual (N elements)
  float* U[TGRAD_MAX_NDIM] = {nullptr};
  float* Mp[TGRAD_MAX_NDIM] = {nullptr};
  float* Mr[TGRAD_MAX_NDIM] = {nullptr};
  // complex modes: Mps holds Re, Im of the projection operand (r x I each), Mrs those of
  // the reconstruction operand (I x r each), for the streaming kernel's complex form.
  // Modes wider than 64 (csplit: their real-block operands exceed the tiled product's
  // 128 rows or columns) run each product as two real products on the interleaved
  // (re, im) view, one with Re M and one with Im M, and a combine pass; ctmp: the Im M
  // product's output (N P floats), then, when the reconstruction's last launch is such a
  // mode, its full update before the dense apply (N P floats)
  bool csplit[TGRAD_MAX_NDIM] = {false};
  float* Mps[TGRAD_MAX_NDIM] = {nullptr};
  float* Mrs[TGRAD_MAX_NDIM] = {nullptr};
  float* ctmp = nullptr;
  double* eig[TGRAD_MAX_NDIM] = {nullptr};
  double* gram_part = nullptr;
  double* gram = nullptr;        // one (I*P)^2 matrix per compressed mode
  uint64_t gram_stride = 0;
  TopkWs tw{};

  // variants (tgrad_options); the defaults are the plain method
  double wd = 0.0, lam = 1.0;
  int selection = TGRAD_SELECT_TOPK;
  bool remap = false;
  uint64_t seed = 0;
  int order = TGRAD_ORDER_SPARSE_FIRST;
  float* lbuf = nullptr;         // low-rank first: L, then G - L (N * P fp32)
  // remapped sparse moments: the previous Omega's bitmask and ranks, and the second
  // moment buffers (allocated when remapping is first enabled)
  uint64_t* mask_prev = nullptr;
  uint32_t* rank_prev = nullptr;
  float *mS_alt = nullptr, *vS_alt = nullptr;
  // test capture (tgrad_debug_capture_delta): the fp32 update of every step is also
  // written here (caller's device buffer, N * P floats) while it is set
  float* delta_cap = nullptr;
  // eigensolver report of the last refresh: per compressed mode, the sweeps it took, or
  // -1 when the sweep cap was reached before the off-diagonal bound (device, 8 ints)
  int* eig_status = nullptr;
  bool refreshed_once = false;

  std::vector<void*> allocs;
  int64_t state_bytes = 0, ws_bytes = 0;
  std::string err;

  // the launches of the last step or refresh call with their algorithmic work
  std::vector<tgrad_launch> launches;

  bool timing = false;
  int timing_only = -1;   // >= 0: only launches of this kernel id are timed
  int max_rec = 0;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipStream_t cur_stream = nullptr;
};

namespace {

struct DevGuard {
  int prev = -1;
  explicit DevGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DevGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Streams and events for tgrad_step_many: per device, created on first use and kept for
// the life of the process; default priority. One mutex serialises the calls.
constexpr int kManyStreams = 4;
struct ManyPool {
  bool ready = false;
  hipStream_t st[kManyStreams] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kManyStreams] = {};
};
std::mutex g_many_mu;
std::vector<ManyPool> g_many;

hipError_t many_pool(int dev, ManyPool** out) {
  if ((int)g_many.size() <= dev) g_many.resize(dev + 1);
  ManyPool& p = g_many[dev];
  if (!p.ready) {
    hipError_t e;
    for (int i = 0; i < kManyStreams; ++i)
      if ((e = hipStreamCreateWithFlags(&p.st[i], hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&p.fork, hipEventDisableTiming)) != hipSuccess) return e;
    for (int i = 0; i < kManyStreams; ++i)
      if ((e = hipEventCreateWithFlags(&p.join[i], hipEventDisableTiming)) != hipSuccess) return e;
    p.ready = true;
  }
  *out = &p;
  return hipSuccess;
}

int fail_hip(tgrad_t* h, hipError_t e, const char* what) {
  if (h) {
    h->err = std::string(what) + ": " + hipGetErrorString(e);
  }
  return TGRAD_EHIP;
}

#define HIPCHK(h, expr)                                  \
  do {                                                   \
    hipError_t _e = (expr);                              \
    if (_e != hipSuccess) return fail_hip((h), _e, #expr); \
  } while (0)

template <typename T>
bool dalloc(tgrad_t* h, T** p, uint64_t n, bool state) {
  *p = nullptr;
  if (n == 0) return true;
  void* q = nullptr;
  const size_t bytes = (size_t)n * sizeof(T);
  if (hipMalloc(&q, bytes) != hipSuccess) return false;
  h->allocs.push_back(q);
  (state ? h->state_bytes : h->ws_bytes) += (int64_t)bytes;
  *p = (T*)q;
  return true;
}

void free_all(tgrad_t* h) {
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
  for (auto& r : h->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  h->recs.clear();
  for (auto e : h->pool) (void)hipEventDestroy(e);
  h->pool.clear();
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  h->side = nullptr;
  h->ev_fork = h->ev_join = nullptr;
}

uint64_t dt_bytes(int dtype) {
  return dtype == TGRAD_C64 ? 8 : (dtype == TGRAD_F32 ? 4 : 2);
}

// (A, I, B) view of mode n of a tensor with the given current sizes.
void view(const int64_t* sz, int d, int n, uint32_t* A, uint32_t* I, uint32_t* B) {
  uint64_t a = 1, b = 1;
  for (int i = 0; i < n; ++i) a *= (uint64_t)sz[i];
  for (int i = n + 1; i < d; ++i) b *= (uint64_t)sz[i];
  *A = (uint32_t)a;
  *I = (uint32_t)sz[n];
  *B = (uint32_t)b;
}

hipEvent_t take_event(tgrad_t* h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void mark_cb(void* ctx, int id, bool begin) {
  tgrad_t* h = (tgrad_t*)ctx;
  if (!h->timing) return;
  if (h->timing_only >= 0 && id != h->timing_only) return;
  if (begin) {
    if ((int)h->recs.size() >= h->max_rec) return;
    Rec r;
    r.id = id;
    r.a = take_event(h);
    r.b = take_event(h);
    if (!r.a || !r.b) return;
    (void)hipEventRecord(r.a, h->cur_stream);
    h->recs.push_back(r);
  } else {
    if (h->recs.empty() || h->recs.back().id != id) return;
    Rec& r = h->recs.back();
    if (r.b == nullptr) return;
    (void)hipEventRecord(r.b, h->cur_stream);
  }
}

struct Mark {
  tgrad_t* h;
  int id;
  Mark(tgrad_t* hh, int i) : h(hh), id(i) { mark_cb(h, id, true); }
  ~Mark() { mark_cb(h, id, false); }
};

void record(tgrad_t* h, int kid, int modes, uint64_t br, uint64_t bw, uint64_t fl) {
  tgrad_launch l;
  l.kernel = kid;
  l.modes = modes;
  l.bytes_read = (int64_t)br;
  l.bytes_written = (int64_t)bw;
  l.flops = (int64_t)fl;
  h->launches.push_back(l);
}

// Record a mode-product launch that contracts `modes` (in order) of a tensor whose
// current sizes are `cur`: towards the ranks (projection) or the full sizes
// (reconstruction). Its algorithmic bytes: the input once (es_in bytes a value) and the
// fp32 output once; with `gather`, the k Omega indices read and the k sparse values
// written; with `apply`, the weights read and written (instead of an output), the k
// indices and k sparse updates read. Flops: 2 K M per column of each product, K and M
// the real sizes (times P) of the contracted and produced mode.
void account_chain(tgrad_t* h, int kid, const int64_t* cur, const std::vector<int>& modes,
                   bool projection, uint64_t es_in, bool gather, bool apply) {
  const uint64_t P = h->P;
  int64_t c[TGRAD_MAX_NDIM];
  uint64_t in = 1;
  for (int i = 0; i < h->d; ++i) {
    c[i] = cur[i];
    in *= (uint64_t)cur[i];
  }
  uint64_t fl = 0, size = in;
  int mbits = 0;
  for (int n : modes) {
    const uint64_t tgt = (uint64_t)(projection ? h->ranks[n] : h->shape[n]);
    fl += 2 * (size / (uint64_t)c[n]) * ((uint64_t)c[n] * P) * (tgt * P);
    size = size / (uint64_t)c[n] * tgt;
    c[n] = (int64_t)tgt;
    mbits |= 1 << n;
  }
  uint64_t br = in * P * es_in, bw = apply ? 0 : size * P * 4;
  if (gather) {
    br += h->k * 4;
    bw += h->k * P * 4;
  }
  if (apply) {
    const uint64_t esw = h->dtype == TGRAD_C64 ? 4 : dt_bytes(h->dtype);
    br += h->N * P * esw + h->k * 4 + h->k * P * 4;
    bw += h->N * P * esw;
  }
  record(h, kid, mbits, br, bw, fl);
}

void host_operands(uint32_t I, uint32_t r, uint32_t P, const float* U, float* Mp, float* Mr) {
  if (P == 1) {
    for (uint32_t i = 0; i < I; ++i)
      for (uint32_t c = 0; c < r; ++c) {
        Mp[(size_t)c * I + i] = U[(size_t)i * r + c];
        Mr[(size_t)i * r + c] = U[(size_t)i * r + c];
      }
    return;
  }
  const size_t KP = 2 * (size_t)I, RP = 2 * (size_t)r;
  for (uint32_t i = 0; i < I; ++i)
    for (uint32_t c = 0; c < r; ++c) {
      const float ur = U[((size_t)i * r + c) * 2], ui = U[((size_t)i * r + c) * 2 + 1];
      Mp[(2 * c) * KP + 2 * i] = ur;
      Mp[(2 * c) * KP + 2 * i + 1] = ui;
      Mp[(2 * c + 1) * KP + 2 * i] = -ui;
      Mp[(2 * c + 1) * KP + 2 * i + 1] = ur;
      Mr[(2 * i) * RP + 2 * c] = ur;
      Mr[(2 * i) * RP + 2 * c + 1] = -ui;
      Mr[(2 * i + 1) * RP + 2 * c] = ui;
      Mr[(2 * i + 1) * RP + 2 * c + 1] = ur;
    }
}

// Launch groups of the projection (applied in order) and the reconstruction: each group
// is one launch, one mode or the two trailing modes together.
// Launch groups of the two chains. fuse: the two trailing modes run as one launch in
// each direction; proj3 (with fuse): the projection's first launch also takes mode d-3.
// The (A, I0, I1, C) view of modes n, n + 1 of a tensor whose sizes are cur.
void pair_view(const int64_t* cur, int d, int n, ModePair* mp) {
  uint64_t A = 1, C = 1;
  for (int i = 0; i < n; ++i) A *= (uint64_t)cur[i];
  for (int i = n + 2; i < d; ++i) C *= (uint64_t)cur[i];
  mp->A = (uint32_t)A;
  mp->I0 = (uint32_t)cur[n];
  mp->I1 = (uint32_t)cur[n + 1];
  mp->C = C;
}

// One mode product runs on the streaming kernel where it applies (and is enabled), else
// on the tiled one; the launch is recorded under the kernel id of the kernel that ran.
bool use_stream(const tgrad_t* h, const ModeProd& mp) {
  return h->stream && streamprod_supported(mp);
}
hipError_t mode_product(const tgrad_t* h, const ModeProd& mp, hipStream_t s) {
  if (use_stream(h, mp)) {
    ModeProd m = mp;
    m.max_wg = h->stream_wg;
    return launch_streamprod(m, h->num_cu, s);
  }
  return launch_modeprod(mp, h->num_cu, s);
}

// Re and Im parts of mode n's operands (a wide complex mode), from its real-block ones.
hipError_t split_operands(const tgrad_t* h, int n, hipStream_t s) {
  const uint32_t I = (uint32_t)h->shape[n], r = (uint32_t)h->ranks[n];
  const size_t ri = (size_t)r * I;
  hipError_t e = launch_split_operand(h->Mp[n], r, I, h->Mps[n], h->Mps[n] + ri, s);
  if (e == hipSuccess) e = launch_split_operand(h->Mr[n], I, r, h->Mrs[n], h->Mrs[n] + ri, s);
  return e;
}

// A single-mode product of a wide complex mode n: mp describes it in the real-block form
// (P = 2, operand (R P) x (I P)); Ms holds Re M then Im M (R x I each). The interleaved
// view of X is a real (A, I, 2B) tensor, so (Re M) X lands in Y and (Im M) X in ctmp as
// (re, im) pairs, and the combine pass leaves M X = (Re M) X + i (Im M) X in Y.
int split_product(tgrad_t* h, const ModeProd& mp, const float* Ms, int n, int kid,
                  int kid_stream, float* Y, hipStream_t s) {
  ModeProd m{};
  m.X = mp.X;
  m.in_dt = DT_F32;
  m.A = mp.A;
  m.I = mp.I;
  m.B = 2 * mp.B;
  m.R = mp.R;
  m.P = 1;
  m.apply = 0;
  const uint64_t in = (uint64_t)mp.A * mp.I * mp.B * 2, out = (uint64_t)mp.A * mp.R * mp.B * 2;
  const uint64_t fl = 2 * ((uint64_t)mp.A * 2 * mp.B) * mp.I * mp.R;
  float* parts[2] = {Y, h->ctmp};
  for (int p = 0; p < 2; ++p) {
    m.M = Ms + (size_t)p * mp.R * mp.I;
    m.Y = parts[p];
    const int k = use_stream(h, m) ? kid_stream : kid;
    Mark mk(h, k);
    HIPCHK(h, mode_product(h, m, s));
    record(h, k, 1 << n, in * 4, out * 4, fl);
  }
  Mark mk(h, KID_CSPLIT_COMBINE);
  HIPCHK(h, launch_csplit_combine(Y, h->ctmp, out / 2, s));
  record(h, KID_CSPLIT_COMBINE, 1 << n, out * 8, out * 4, 2 * out);
  return TGRAD_OK;
}

// A group of two modes that is not the trailing pair: a k_pair launch.
bool is_lead_pair(const tgrad_t* h, const std::vector<int>& g) {
  return g.size() == 2 && std::min(g[0], g[1]) < h->d - 2;
}

void build_chain(const tgrad_t* h, bool fuse, bool proj3, std::vector<std::vector<int>>& proj,
                 std::vector<std::vector<int>>& rec, bool pairs = true, bool rec3 = false) {
  proj.clear();
  rec.clear();
  const int nf = (int)h->fmodes.size();
  const int d = h->d;
  proj3 = proj3 && fuse;
  rec3 = rec3 && fuse;
  if (proj3) proj.push_back({d - 1, d - 2, d - 3});
  else if (fuse) proj.push_back({d - 1, d - 2});
  for (int j = nf - 1; j >= 0; --j) {
    const int n = h->fmodes[j];
    if ((fuse && n >= d - 2) || (proj3 && n == d - 3)) continue;
    proj.push_back({n});
  }
  for (int j = 0; j < nf; ++j) {
    const int n = h->fmodes[j];
    if ((fuse && n >= d - 2) || (rec3 && n == d - 3)) continue;
    rec.push_back({n});
  }
  if (rec3) rec.push_back({d - 3, d - 2, d - 1});
  else if (fuse) rec.push_back({d - 2, d - 1});
  if (!(fuse && pairs && h->pairs && h->P == 1)) return;
  // neighbouring single modes after the first group (projection) and before the last
  // (reconstruction) become one k_pair launch where it applies to their sizes there
  auto merge = [&](std::vector<std::vector<int>>& chain, bool projection) {
    int64_t cur[TGRAD_MAX_NDIM];
    for (int i = 0; i < d; ++i) cur[i] = h->shape[i];
    if (!projection)
      for (int n : h->fmodes) cur[n] = h->ranks[n];
    std::vector<std::vector<int>> out;
    for (size_t j = 0; j < chain.size(); ++j) {
      const bool inner = projection ? j > 0 : j + 1 < chain.size();
      if (inner && j + 1 < chain.size() && (projection || j + 2 < chain.size()) &&
          chain[j].size() == 1 && chain[j + 1].size() == 1 &&
          chain[j + 1][0] == chain[j][0] + (projection ? -1 : 1)) {
        const int n0 = std::min(chain[j][0], chain[j + 1][0]);
        ModePair mp{};
        pair_view(cur, d, n0, &mp);
        mp.J0 = (uint32_t)(projection ? h->ranks[n0] : h->shape[n0]);
        mp.J1 = (uint32_t)(projection ? h->ranks[n0 + 1] : h->shape[n0 + 1]);
        mp.X = (const float*)(uintptr_t)256;
        mp.Y = (float*)(uintptr_t)256;
        if (pair_supported(mp)) {
          out.push_back({chain[j][0], chain[j + 1][0]});
          cur[n0] = mp.J0;
          cur[n0 + 1] = mp.J1;
          ++j;
          continue;
        }
      }
      for (int n : chain[j]) cur[n] = projection ? h->ranks[n] : h->shape[n];
      out.push_back(chain[j]);
    }
    chain = out;
  };
  merge(proj, true);
  merge(rec, false);
}

// The three-mode projection launch for input X0 (16-byte aligned for its transfers).
bool use_proj3(const tgrad_t* h, const void* X0) {
  return h->fuse && h->slab2 && h->slab3 && h->can_slab3 && ((uintptr_t)X0 % 16) == 0;
}
// The three-mode reconstruction + apply launch for the weights W (16-byte aligned).
bool use_rec3(const tgrad_t* h, bool apply, const void* W) {
  return apply && h->fuse && h->slab2 && h->rec3 && h->can_rec3 && ((uintptr_t)W % 16) == 0;
}

int run_projection(tgrad_t* h, const void* X0, bool gather, hipStream_t s,
                   const AdamK* fork_adam = nullptr);
int run_reconstruction(tgrad_t* h, const float* X0, bool apply, void* weight, float* out,
                       hipStream_t s, hipEvent_t wait_last = nullptr);
int step_body(tgrad_t* h, void* weight, const void* grad, int64_t t, hipStream_t s);

// Omega (+ bitmask, ranks) as the k largest keys of `src` (storage type dt), or a random
// k-subset; optionally the residual (src with Omega zeroed) written to `resid`. With
// remapped moments the new bitmask goes to the other buffer, so the old one still
// locates each element's previous moments, which then follow their element.
int select_omega(tgrad_t* h, const TopkWs& tw, const void* src, int dt, void* resid,
                 hipStream_t s) {
  if (h->remap) {
    std::swap(h->mask, h->mask_prev);
    std::swap(h->rank, h->rank_prev);
  }
  const uint64_t gamma = 0x9E3779B97F4A7C15ull;
  const uint64_t serves = (uint64_t)(h->t + 1);
  const uint64_t rk_base = h->seed + gamma * ((serves << 32) + 1ull);
  HIPCHK(h, launch_topk(dt, src, h->N, (uint32_t)h->k, tw, h->omega, h->mask, h->rank, resid,
                        h->selection == TGRAD_SELECT_RANDK, rk_base, s, mark_cb, h));
  {
    // the radix passes read the keys' source (magnitudes: 11 bits a pass, 16-bit
    // magnitudes all 15 bits in one pass), the count pass
    // once more, the compaction once more (rand-k keys need no read, except for the
    // residual); the compaction writes Omega, its bitmask and word ranks, and the residual
    const bool rk = h->selection == TGRAD_SELECT_RANDK;
    const uint64_t es = dt == DT_C64 ? 8 : (dt == DT_F32 ? 4 : 2);
    const int bits = rk ? 31 : (dt == DT_C64 ? 63 : (dt == DT_F32 ? 31 : 15));
    const uint64_t passes = bits == 15 ? 1 : (uint64_t)((bits + 10) / 11);
    const uint64_t src_b = rk ? 0 : h->N * es;
    record(h, KID_TOPK_HIST, 0, passes * src_b, 0, 0);
    record(h, KID_TOPK_COUNT, 0, src_b, 0, 0);
    record(h, KID_TOPK_COMPACT, 0, (rk && !resid) ? 0 : h->N * es,
           h->k * 4 + h->N / 8 + h->N / 16 + (resid ? h->N * es : 0), 0);
  }
  if (h->remap) {
    Mark m(h, KID_REMAP);
    HIPCHK(h, launch_remap_moments(h->mask_prev, h->rank_prev, h->omega, (uint32_t)h->k,
                                   h->P, h->mS, h->vS, h->mS_alt, h->vS_alt, s));
    std::swap(h->mS, h->mS_alt);
    std::swap(h->vS, h->vS_alt);
  }
  return TGRAD_OK;
}

// The one-read Gram launch of the last three modes over X (entries in `mask` read as
// zero), where all three are compressed in a real 16-bit tensor (the caller still asks
// gram3_supported).
bool gram3_args(const tgrad_t* h, const void* X, const uint64_t* mask, double* partial,
                Gram3Args* g) {
  const int d = h->d;
  if (d < 3 || h->P != 1 || (h->dtype != TGRAD_BF16 && h->dtype != TGRAD_F16)) return false;
  for (int i = d - 3; i < d; ++i)
    if (h->ranks[i] >= h->shape[i]) return false;
  uint64_t A = 1;
  for (int i = 0; i < d - 3; ++i) A *= (uint64_t)h->shape[i];
  *g = Gram3Args{};
  g->X = X;
  g->dt = h->dtype;
  g->A = (uint32_t)A;
  g->Ia = (uint32_t)h->shape[d - 3];
  g->Ib = (uint32_t)h->shape[d - 2];
  g->Ic = (uint32_t)h->shape[d - 1];
  g->mask = mask;
  g->partial = partial;
  return true;
}

RefreshWs handle_ws(const tgrad_t* h) {
  RefreshWs ws;
  ws.tw = h->tw;
  ws.gram_part = h->gram_part;
  ws.gram = h->gram;
  ws.masked = h->gram_masked;
  ws.max_gram_blocks = 0;
  return ws;
}

int do_refresh(tgrad_t* h, const void* grad, hipStream_t s, const RefreshWs& ws) {
  // sparse first: Omega from G, then the Grams of the residual (G itself when k = 0):
  // the copy with Omega zeroed that the top-k compaction writes, or (gram_masked) G read
  // with Omega's entries cleared through its bitmask. Low-rank first: the Grams of G,
  // then Omega from the residual G - L of the new factors.
  const bool lowrank_first =
      h->order == TGRAD_ORDER_LOWRANK_FIRST && h->k > 0 && !h->fmodes.empty();
  const void* R = grad;
  const uint64_t* rmask = nullptr;
  int rc;
  if (h->k > 0 && !lowrank_first) {
    void* rw = (h->fmodes.empty() || ws.masked) ? nullptr : h->resid;
    if ((rc = select_omega(h, ws.tw, grad, h->dtype, rw, s)) != TGRAD_OK) return rc;
    if (rw) R = rw;
    else rmask = h->mask;
  }
  const int gdt = (h->dtype == DT_C64) ? DT_F32 : h->dtype;
  EigArgs eig[TGRAD_MAX_NDIM];
  int ne = 0;
  // the last three modes' Grams from one read of R where that launch applies, the other
  // modes one launch each
  Gram3Args g3;
  const bool tail3 = h->gram3 && h->can_gram3 && gram3_args(h, R, rmask, ws.gram_part, &g3) &&
                     gram3_supported(g3, h->num_cu);
  for (int n : h->fmodes) {
    double* const out = ws.gram + (size_t)ne * h->gram_stride;
    if (tail3 && n >= h->d - 3) {
      g3.out[n - (h->d - 3)] = out;
    } else {
      GramArgs g{};
      g.X = R;
      g.max_blocks = ws.max_gram_blocks;
      g.dt = gdt;
      view(h->shape, h->d, n, &g.A, &g.I, &g.B);
      g.P = h->P;
      g.mask = rmask;
      g.partial = ws.gram_part;
      g.out = out;
      HIPCHK(h, launch_gram(g, h->num_cu, s, mark_cb, h));
      record(h, KID_GRAM, 1 << n, h->N * dt_bytes(h->dtype) + (rmask ? h->N / 8 : 0), 0,
             2 * (h->N / g.I) * ((uint64_t)g.I * h->P) * ((uint64_t)g.I * h->P));
    }
    EigArgs& e = eig[ne];
    e.status = h->eig_status + ne;
    ++ne;
    e.gram = out;
    e.I = (uint32_t)h->shape[n];
    e.r = (uint32_t)h->ranks[n];
    e.P = h->P;
    e.U = h->U[n];
    e.Mproj = h->Mp[n];
    e.Mrec = h->Mr[n];
    e.eigvals = h->eig[n];
  }
  // With the last three modes' Grams in one launch, the modes before them have their
  // Gram matrices before that launch starts: their eigensolver (one workgroup a matrix)
  // runs on the handle's second stream, on CUs the three-mode launch leaves free (it
  // takes one workgroup per CU otherwise), and the caller's stream waits for it before
  // the refresh ends. Results do not depend on the overlap.
  int nlead = 0;
  for (int n : h->fmodes)
    if (tail3 && n < h->d - 3) ++nlead;
  const bool eig_fork = tail3 && h->eig_overlap && h->side && nlead > 0 && nlead < ne &&
                        nlead < h->num_cu / 4;
  if (eig_fork) {
    HIPCHK(h, hipEventRecord(h->ev_fork, s));
    HIPCHK(h, hipStreamWaitEvent(h->side, h->ev_fork, 0));
    hipError_t e;
    h->cur_stream = h->side;   // the timing events of this launch go on the side stream
    {
      Mark m(h, KID_EIG);
      e = launch_eig(eig, nlead, h->side);
    }
    h->cur_stream = s;
    if (e != hipSuccess) return fail_hip(h, e, "launch_eig (leading modes)");
    record(h, KID_EIG, 0, 0, 0, 0);
    HIPCHK(h, hipEventRecord(h->ev_join, h->side));
  }
  if (tail3) {
    hipError_t e = launch_gram3(g3, eig_fork ? h->num_cu - nlead : h->num_cu, s, mark_cb, h);
    if (e != hipSuccess) {
      if (eig_fork) (void)hipStreamWaitEvent(s, h->ev_join, 0);
      return fail_hip(h, e, "launch_gram3");
    }
    const uint64_t I3[3] = {g3.Ia, g3.Ib, g3.Ic};
    uint64_t fl = 0;
    for (int m = 0; m < 3; ++m) fl += 2 * (h->N / I3[m]) * I3[m] * I3[m];
    record(h, KID_GRAM3, 7 << (h->d - 3), h->N * dt_bytes(h->dtype) + (rmask ? h->N / 8 : 0), 0,
           fl);
  }
  const int e0 = eig_fork ? nlead : 0;
  if (ne > e0) {
    Mark m(h, KID_EIG);
    const hipError_t e = launch_eig(eig + e0, ne - e0, s);
    if (e != hipSuccess) {
      if (eig_fork) (void)hipStreamWaitEvent(s, h->ev_join, 0);
      return fail_hip(h, e, "launch_eig");
    }
    record(h, KID_EIG, 0, 0, 0, 0);
  }
  if (eig_fork) HIPCHK(h, hipStreamWaitEvent(s, h->ev_join, 0));
  for (int n : h->fmodes)
    if (h->Mps[n]) {
      Mark m(h, KID_CSPLIT_OPERAND);
      HIPCHK(h, split_operands(h, n, s));
      const uint64_t ri = (uint64_t)h->shape[n] * h->ranks[n];
      record(h, KID_CSPLIT_OPERAND, 1 << n, 2 * ri * 4, 4 * ri * 4, 0);
    }
  if (lowrank_first) {
    if (h->selection == TGRAD_SELECT_RANDK) {
      if ((rc = select_omega(h, ws.tw, grad, h->dtype, nullptr, s)) != TGRAD_OK) return rc;
    } else {
      // R = G - (G x_n Un^H ...) x_n Un ... in fp32, then its k largest entries
      if ((rc = run_projection(h, grad, false, s)) != TGRAD_OK) return rc;
      if ((rc = run_reconstruction(h, h->core, false, nullptr, h->lbuf, s)) != TGRAD_OK) return rc;
      {
        Mark m(h, KID_GATHER);
        HIPCHK(h, launch_resid_sub(h->dtype, grad, h->lbuf, h->N * h->P, s));
      }
      if ((rc = select_omega(h, ws.tw, h->lbuf, h->P == 2 ? DT_C64 : DT_F32, nullptr, s)) !=
          TGRAD_OK)
        return rc;
    }
  }
  h->refreshed_for = h->t + 1;
  h->refreshed_once = true;
  return TGRAD_OK;
}
}  // namespace

extern "C" {

const char* tgrad_status_string(int status) {
  switch (status) {
    case TGRAD_OK: return "ok";
    case TGRAD_EINVAL: return "invalid argument";
    case TGRAD_ENOMEM: return "device allocation failed";
    case TGRAD_EHIP: return "HIP call failed";
    case TGRAD_ESTATE: return "invalid state";
  }
  return "unknown status";
}

const char* tgrad_last_error(const tgrad_t* h) { return h ? h->err.c_str() : ""; }

const char* tgrad_kernel_name(int id) {
  static const char* names[KID_COUNT_] = {
      "topk_init", "topk_hist", "topk_select", "topk_count", "topk_scan", "topk_compact",
      "mask_from_omega", "gather_residual", "modeprod_project", "adam_fused",
      "modeprod_reconstruct", "modeprod_reconstruct_apply", "apply_dense", "gram",
      "gram_reduce", "eigensolver", "fill", "modeprod_project_first",
      "modeprod2_project_first", "modeprod2_reconstruct_apply", "modeprod2_reconstruct",
      "remap_moments", "modeprod3_project_first", "gram3_tail", "modeprod_pair_project",
      "modeprod_pair_reconstruct", "modeprod3_reconstruct_apply", "streamprod_project",
      "streamprod_reconstruct", "complex_split_operand", "complex_split_combine",
      "rowprod_project", "rowprod_reconstruct_apply", "adam_sparse"};
  static_assert(KID_COUNT_ <= TGRAD_MAX_KERNEL_IDS, "kernel ids fit the timing arrays");
  if (id < 0 || id >= KID_COUNT_) return "";
  return names[id];
}

int tgrad_init(tgrad_t** out, int ndim, const int64_t* shape, const int64_t* tucker_ranks,
               int dtype, double sparse_ratio, int64_t T, double lr, double beta1, double beta2,
               double eps) {
  if (!out) return TGRAD_EINVAL;
  *out = nullptr;
  if (ndim < 1 || ndim > TGRAD_MAX_NDIM || !shape || !tucker_ranks) return TGRAD_EINVAL;
  if (dtype < TGRAD_F32 || dtype > TGRAD_C64) return TGRAD_EINVAL;
  if (!(sparse_ratio >= 0.0 && sparse_ratio <= 1.0) || T < 1) return TGRAD_EINVAL;
  if (!(lr >= 0.0) || !(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) ||
      !(eps >= 0.0))
    return TGRAD_EINVAL;
  uint64_t N = 1, ncore = 1;
  for (int i = 0; i < ndim; ++i) {
    if (shape[i] < 1 || tucker_ranks[i] < 1 || tucker_ranks[i] > shape[i]) return TGRAD_EINVAL;
    if (tucker_ranks[i] < shape[i] && shape[i] > TGRAD_MAX_FACTOR_DIM) return TGRAD_EINVAL;
    N *= (uint64_t)shape[i];
    ncore *= (uint64_t)tucker_ranks[i];
    if (N >= (1ull << 32)) return TGRAD_EINVAL;
  }
  // a compressed mode's rank cannot exceed the rank of its unfolding, N / I_n: the extra
  // core entries would be zero up to rounding, and Adam turns rounding noise into O(1)
  // updates there
  for (int i = 0; i < ndim; ++i)
    if (tucker_ranks[i] < shape[i] && (uint64_t)tucker_ranks[i] > N / (uint64_t)shape[i])
      return TGRAD_EINVAL;
  tgrad_t* h = new (std::nothrow) tgrad_t();
  if (!h) return TGRAD_ENOMEM;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return TGRAD_EHIP;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, h->device) == hipSuccess &&
      cu > 0)
    h->num_cu = cu;
  h->d = ndim;
  for (int i = 0; i < ndim; ++i) {
    h->shape[i] = shape[i];
    h->ranks[i] = tucker_ranks[i];
    if (tucker_ranks[i] < shape[i]) h->fmodes.push_back(i);
  }
  h->dtype = dtype;
  h->P = dtype == TGRAD_C64 ? 2 : 1;
  h->N = N;
  h->k = (uint64_t)std::floor(sparse_ratio * (double)N);
  if (h->k > N) h->k = N;
  h->ncore = ncore;
  h->nwords = (N + 63) / 64;
  h->T = T;
  h->lr = lr;
  h->b1 = beta1;
  h->b2 = beta2;
  h->eps = eps;
  const uint64_t P = h->P;

  // Two trailing compressed modes can run as one launch in each direction.
  {
    const int d = ndim;
    if (d >= 2 && tucker_ranks[d - 2] < shape[d - 2] && tucker_ranks[d - 1] < shape[d - 1]) {
      uint64_t A = 1;
      for (int i = 0; i < d - 2; ++i) A *= (uint64_t)shape[i];
      ModeProd2 pp{};
      pp.in_dt = dtype == TGRAD_C64 ? DT_F32 : dtype;
      pp.P = h->P;
      pp.A = (uint32_t)A;
      pp.I1 = (uint32_t)shape[d - 2];
      pp.I2 = (uint32_t)shape[d - 1];
      pp.R1 = (uint32_t)tucker_ranks[d - 2];
      pp.R2 = (uint32_t)tucker_ranks[d - 1];
      ModeProd2 rr = pp;
      rr.recon = 1;
      rr.in_dt = DT_F32;
      rr.apply = 1;
      rr.w_dt = pp.in_dt;
      std::swap(rr.I1, rr.R1);
      std::swap(rr.I2, rr.R2);
      h->can_fuse = modeprod2_tile(pp) > 0 && modeprod2_tile(rr) > 0;
      h->fuse = h->can_fuse;
      if (h->can_fuse && d >= 3 && tucker_ranks[d - 3] < shape[d - 3]) {
        ModeProd2 p3 = pp;
        p3.X = (const void*)(uintptr_t)256;   // transfers need a 16-byte aligned input
        p3.I0 = (uint32_t)shape[d - 3];
        p3.R0 = (uint32_t)tucker_ranks[d - 3];
        h->can_slab3 = slab3_supported(p3);
        // the reconstruction's last three modes (core-side sizes in I, full in R)
        ModeProd2 r3{};
        r3.X = (const void*)(uintptr_t)256;
        r3.W = (void*)(uintptr_t)256;
        r3.in_dt = DT_F32;
        r3.w_dt = pp.in_dt;
        r3.P = h->P;
        r3.recon = 1;
        r3.apply = 1;
        r3.A = (uint32_t)(A / shape[d - 3] * tucker_ranks[d - 3]);
        r3.I0 = (uint32_t)tucker_ranks[d - 3];
        r3.I1 = (uint32_t)tucker_ranks[d - 2];
        r3.I2 = (uint32_t)tucker_ranks[d - 1];
        r3.R0 = (uint32_t)shape[d - 3];
        r3.R1 = (uint32_t)shape[d - 2];
        r3.R2 = (uint32_t)shape[d - 1];
        h->can_rec3 = rec3_supported(r3);
      }
    }
  }
  // Largest intermediate of the projection and reconstruction chains (either plan).
  uint64_t inter = 0;
  for (int plan = 0; plan < 2; ++plan) {
    const bool fz = plan == 1;
    if (fz && !h->can_fuse) continue;
    int64_t cur[TGRAD_MAX_NDIM];
    for (int i = 0; i < ndim; ++i) cur[i] = shape[i];
    std::vector<std::vector<int>> proj, rec;
    build_chain(h, fz, false, proj, rec, false);   // pairs only drop intermediates
    uint64_t size = N;
    for (size_t j = 0; j < proj.size(); ++j) {
      for (int n : proj[j]) {
        size = size / (uint64_t)cur[n] * (uint64_t)h->ranks[n];
        cur[n] = h->ranks[n];
      }
      if (j + 1 < proj.size() && size > inter) inter = size;    // not the core
    }
    for (size_t j = 0; j < rec.size(); ++j) {
      for (int n : rec[j]) {
        size = size / (uint64_t)cur[n] * (uint64_t)shape[n];
        cur[n] = shape[n];
      }
      if (j + 1 < rec.size() && size > inter) inter = size;     // not the weight
    }
  }

  bool ok = true;
  ok = ok && dalloc(h, &h->omega, h->k, true);
  ok = ok && dalloc(h, &h->mask, h->nwords, false);
  ok = ok && dalloc(h, &h->rank, h->nwords, false);
  ok = ok && dalloc(h, &h->S, h->k * P, false);
  ok = ok && dalloc(h, &h->mS, h->k * P, true);
  ok = ok && dalloc(h, &h->vS, h->k * P, true);
  ok = ok && dalloc(h, &h->mC, ncore * P, true);
  ok = ok && dalloc(h, &h->vC, ncore * P, true);
  ok = ok && dalloc(h, &h->ucore, ncore * P, false);
  if (!h->fmodes.empty()) ok = ok && dalloc(h, &h->core, ncore * P, false);
  // One block holds the two chain intermediates and, during a refresh (when they are
  // idle), the residual G with Omega zeroed that the Gram kernels read.
  {
    const uint64_t esz = dtype == TGRAD_C64 ? 8 : (dtype == TGRAD_F32 ? 4 : 2);
    const uint64_t rbytes = (h->k > 0 && !h->fmodes.empty()) ? N * esz : 0;
    const uint64_t ib = (inter * P * sizeof(float) + 255) & ~255ull;
    unsigned char* blk = nullptr;
    ok = ok && dalloc(h, &blk, std::max(2 * ib, rbytes), false);
    if (ok && inter) {
      h->buf[0] = (float*)blk;
      h->buf[1] = (float*)(blk + ib);
    }
    if (ok && rbytes) h->resid = blk;
  }
  uint64_t gpart = 0, gmax = 0;
  for (int n : h->fmodes) {
    const uint64_t I = (uint64_t)shape[n], r = (uint64_t)tucker_ranks[n];
    ok = ok && dalloc(h, &h->U[n], I * r * P, true);
    ok = ok && dalloc(h, &h->Mp[n], I * r * P * P, false);
    ok = ok && dalloc(h, &h->Mr[n], I * r * P * P, false);
    ok = ok && dalloc(h, &h->eig[n], I, false);
    if (P == 2) {
      // Re and Im parts of the operands (the streaming kernel's complex form, and the
      // split products of modes wider than 64)
      ok = ok && dalloc(h, &h->Mps[n], 2 * I * r, false);
      ok = ok && dalloc(h, &h->Mrs[n], 2 * I * r, false);
      if (I > 64) {
        h->csplit[n] = true;
        if (!h->ctmp) ok = ok && dalloc(h, &h->ctmp, 2 * N * P, false);
      }
    }
    GramArgs g{};
    view(shape, ndim, n, &g.A, &g.I, &g.B);
    g.P = (uint32_t)P;
    const uint64_t K2 = (I * P) * (I * P);
    // partials for whichever Gram path a refresh takes (the 16-bit one needs an
    // aligned input; the general one takes any)
    g.dt = DT_F32;
    uint64_t nb = gram_blocks(g, h->num_cu);
    g.dt = dtype == TGRAD_C64 ? DT_F32 : dtype;
    nb = std::max<uint64_t>(nb, gram_blocks(g, h->num_cu));
    // and with a mask (the masked Grams take the general kernels where the unmasked
    // ones take the fp32 / complex one)
    g.mask = (const uint64_t*)(uintptr_t)64;
    nb = std::max<uint64_t>(nb, gram_blocks(g, h->num_cu));
    g.dt = DT_F32;
    nb = std::max<uint64_t>(nb, gram_blocks(g, h->num_cu)) + gram_reduce_groups();
    if (nb * K2 > gpart) gpart = nb * K2;
    if (K2 > gmax) gmax = K2;
  }
  {
    Gram3Args g3;
    // with the mask a refresh will pass (the launch then stages mask bytes too)
    const uint64_t* m3 = h->k > 0 ? h->mask : nullptr;
    if (gram3_args(h, (const void*)(uintptr_t)256, m3, nullptr, &g3) &&
        gram3_supported(g3, h->num_cu)) {
      h->can_gram3 = true;
      gpart = std::max<uint64_t>(gpart, gram3_partial_doubles(g3, h->num_cu));
    }
  }
  ok = ok && dalloc(h, &h->gram_part, gpart, false);
  if (h->can_fuse) {
    std::vector<std::vector<int>> pp, rr;
    build_chain(h, true, false, pp, rr);
    for (const auto& g : pp) h->can_pair = h->can_pair || is_lead_pair(h, g);
    for (const auto& g : rr) h->can_pair = h->can_pair || is_lead_pair(h, g);
  }
  // the unfused launch plan projects a residual copy of grad (the fused one zeroes Omega
  // in its staged tiles)
  if (h->k > 0 && !h->can_fuse) {
    unsigned char* gc = nullptr;
    ok = ok && dalloc(h, &gc, N * dt_bytes(dtype), false);
    h->gcopy = gc;
  }
  h->gram_stride = gmax;
  ok = ok && dalloc(h, &h->gram, gmax * h->fmodes.size(), false);
  ok = ok && dalloc(h, &h->eig_status, TGRAD_MAX_NDIM, false);
  const uint64_t units = topk_units(N);
  ok = ok && dalloc(h, &h->tw.hist, TOPK_HIST_BINS, false);
  ok = ok && dalloc(h, &h->tw.state, 4, false);
  ok = ok && dalloc(h, &h->tw.ucount, 2 * units, false);
  ok = ok && dalloc(h, &h->tw.uoff, 2 * units, false);
  ok = ok && dalloc(h, &h->tw.ctot, 2 * topk_chunks(N), false);
  if (!ok) {
    free_all(h);
    delete h;
    return TGRAD_ENOMEM;
  }
  hipError_t e = hipSuccess;
  auto zero = [&](void* p, uint64_t bytes) {
    if (p && bytes && e == hipSuccess) e = hipMemset(p, 0, bytes);
  };
  zero(h->mS, h->k * P * 4);
  zero(h->vS, h->k * P * 4);
  zero(h->mC, ncore * P * 4);
  zero(h->vC, ncore * P * 4);
  zero(h->mask, h->nwords * 8);
  zero(h->rank, h->nwords * 4);
  zero(h->omega, h->k * 4);
  zero(h->eig_status, TGRAD_MAX_NDIM * sizeof(int));
  for (int n : h->fmodes) {
    const uint64_t I = (uint64_t)shape[n], r = (uint64_t)tucker_ranks[n];
    zero(h->U[n], I * r * P * 4);
    zero(h->Mp[n], I * r * P * P * 4);
    zero(h->Mr[n], I * r * P * P * 4);
    zero(h->eig[n], I * 8);
    zero(h->Mps[n], 2 * I * r * 4);
    zero(h->Mrs[n], 2 * I * r * 4);
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_all(h);
    delete h;
    return TGRAD_EHIP;
  }
  *out = h;
  return TGRAD_OK;
}

int tgrad_destroy(tgrad_t* h) {
  if (!h) return TGRAD_OK;
  {
    DevGuard g(h->device);
    free_all(h);
  }
  delete h;
  return TGRAD_OK;
}

int tgrad_step_many(tgrad_t* const* hs, void* const* weights, const void* const* grads, int n,
                    void* stream) {
  if (n < 0 || (n > 0 && (!hs || !weights || !grads))) return TGRAD_EINVAL;
  if (n == 0) return TGRAD_OK;
  for (int i = 0; i < n; ++i) {
    if (!hs[i] || !weights[i] || !grads[i] || ((uintptr_t)grads[i] & 15u) != 0)
      return TGRAD_EINVAL;
    if (hs[i]->device != hs[0]->device) return TGRAD_EINVAL;
    for (int j = 0; j < i; ++j)
      if (hs[j] == hs[i]) return TGRAD_EINVAL;   // one handle's steps must stay ordered
  }
  std::lock_guard<std::mutex> lock(g_many_mu);
  tgrad_t* h0 = hs[0];
  DevGuard gd(h0->device);
  ManyPool* p = nullptr;
  HIPCHK(h0, many_pool(h0->device, &p));
  const hipStream_t s = (hipStream_t)stream;
  const int ns = n < kManyStreams ? n : kManyStreams;
  // fork: every pool stream starts after the work already on the caller's stream
  HIPCHK(h0, hipEventRecord(p->fork, s));
  for (int i = 0; i < ns; ++i) HIPCHK(h0, hipStreamWaitEvent(p->st[i], p->fork, 0));
  int rc = TGRAD_OK;
  int launched = 0;
  for (int i = 0; i < n && rc == TGRAD_OK; ++i, ++launched)
    rc = tgrad_step(hs[i], weights[i], grads[i], p->st[i % ns]);
  // join: the caller's stream waits for every pool stream that received work
  const int used = launched < ns ? launched : ns;
  for (int i = 0; i < used; ++i) {
    HIPCHK(h0, hipEventRecord(p->join[i], p->st[i]));
    HIPCHK(h0, hipStreamWaitEvent(s, p->join[i], 0));
  }
  return rc;
}

int tgrad_refresh(tgrad_t* h, const void* grad, void* stream) {
  if (!h || !grad || ((uintptr_t)grad & 15u) != 0) return TGRAD_EINVAL;
  DevGuard g(h->device);
  h->cur_stream = (hipStream_t)stream;
  h->launches.clear();
  return do_refresh(h, grad, (hipStream_t)stream, handle_ws(h));
}

}  // extern "C"

namespace {

// The Adam update of the k sparse values (S holds them once the first projection launch,
// which takes the COO gather, has run) on the handle's second stream: it waits for the
// work enqueued on s so far and is joined back (ev_join) before the reconstruction. The
// update is element-wise, so its result does not depend on the overlap.
constexpr uint64_t kAdamForkMin = 1ull << 22;

int fork_sparse_adam(tgrad_t* h, const AdamK& a, hipStream_t s) {
  const uint64_t nsv = h->k * h->P;
  HIPCHK(h, hipEventRecord(h->ev_fork, s));
  HIPCHK(h, hipStreamWaitEvent(h->side, h->ev_fork, 0));
  hipError_t e;
  h->cur_stream = h->side;   // the timing events of this launch go on the side stream
  {
    Mark m(h, KID_ADAM_SPARSE);
    e = launch_adam_sparse(h->S, h->mS, h->vS, nsv, a, h->side);
  }
  h->cur_stream = s;
  if (e != hipSuccess) return fail_hip(h, e, "launch_adam (sparse values)");
  // S, m, v read and S, m, v written, fp32
  record(h, KID_ADAM_SPARSE, 0, nsv * 12, nsv * 12, 0);
  HIPCHK(h, hipEventRecord(h->ev_join, h->side));
  return TGRAD_OK;
}

// Projection chain C = X x_n Un^H ... (last compressed mode first) into h->core. X has
// the handle's storage dtype. gather: the first launch is a two-mode one that also takes
// S = X[Omega] and projects its staged tiles with Omega zeroed.
int run_projection(tgrad_t* h, const void* X0, bool gather, hipStream_t s,
                   const AdamK* fork_adam) {
  const uint32_t P = h->P;
  std::vector<std::vector<int>> proj, rec;
  build_chain(h, h->fuse, use_proj3(h, X0), proj, rec);
  int64_t cur[TGRAD_MAX_NDIM];
  for (int i = 0; i < h->d; ++i) cur[i] = h->shape[i];
  const void* X = X0;
  int xdt = (h->dtype == DT_C64) ? DT_F32 : h->dtype;
  int which = 0;
  for (size_t j = 0; j < proj.size(); ++j) {
    float* Y = (j + 1 == proj.size()) ? h->core : h->buf[which];
    if (proj[j].size() == 3) {
      const int d = h->d;
      ModeProd2 mp{};
      mp.X = X;
      mp.in_dt = xdt;
      mp.P = P;
      uint32_t A, I, B;
      view(cur, d, d - 2, &A, &I, &B);
      mp.A = A;
      mp.I0 = (uint32_t)cur[d - 3];
      mp.I1 = (uint32_t)cur[d - 2];
      mp.I2 = (uint32_t)cur[d - 1];
      mp.R0 = (uint32_t)h->ranks[d - 3];
      mp.R1 = (uint32_t)h->ranks[d - 2];
      mp.R2 = (uint32_t)h->ranks[d - 1];
      mp.recon = 0;
      mp.M0 = h->Mp[d - 3];
      mp.M1 = h->Mp[d - 2];
      mp.M2 = h->Mp[d - 1];
      mp.Y = Y;
      if (j == 0 && gather) {
        mp.gather_S = h->S;
        mp.mask = h->mask;
        mp.rank = h->rank;
        mp.omega = h->omega;
        mp.kS = h->k;
        mp.has_sparse = 1;
      }
      Mark m(h, KID_PROJECT_FUSED3);
      HIPCHK(h, launch_slab3(mp, h->num_cu, s));
      account_chain(h, KID_PROJECT_FUSED3, cur, proj[j], true, xdt == DT_F32 ? 4 : 2,
                    j == 0 && gather, false);
      cur[d - 3] = h->ranks[d - 3];
      cur[d - 2] = h->ranks[d - 2];
      cur[d - 1] = h->ranks[d - 1];
    } else if (is_lead_pair(h, proj[j])) {
      const int n0 = std::min(proj[j][0], proj[j][1]);
      ModePair mp{};
      pair_view(cur, h->d, n0, &mp);
      mp.X = (const float*)X;
      mp.Y = Y;
      mp.M0 = h->Mp[n0];
      mp.M1 = h->Mp[n0 + 1];
      mp.J0 = (uint32_t)h->ranks[n0];
      mp.J1 = (uint32_t)h->ranks[n0 + 1];
      Mark m(h, KID_PROJECT_PAIR);
      HIPCHK(h, launch_pair(mp, s));
      account_chain(h, KID_PROJECT_PAIR, cur, proj[j], true, 4, false, false);
      cur[n0] = h->ranks[n0];
      cur[n0 + 1] = h->ranks[n0 + 1];
    } else if (proj[j].size() == 2) {
      const int d = h->d;
      ModeProd2 mp{};
      mp.X = X;
      mp.in_dt = xdt;
      mp.P = P;
      uint32_t A, I, B;
      view(cur, d, d - 2, &A, &I, &B);
      mp.A = A;
      mp.I1 = (uint32_t)cur[d - 2];
      mp.I2 = (uint32_t)cur[d - 1];
      mp.R1 = (uint32_t)h->ranks[d - 2];
      mp.R2 = (uint32_t)h->ranks[d - 1];
      mp.recon = 0;
      mp.M1 = h->Mp[d - 2];
      mp.M2 = h->Mp[d - 1];
      mp.Y = Y;
      if (j == 0 && gather) {
        mp.gather_S = h->S;
        mp.mask = h->mask;
        mp.rank = h->rank;
        mp.omega = h->omega;
        mp.kS = h->k;
        mp.has_sparse = 1;
      }
      Mark m(h, KID_PROJECT_FUSED2);
      if (h->slab2 && slab2_supported(mp, h->num_cu))
        HIPCHK(h, launch_slab2(mp, h->num_cu, s));
      else
        HIPCHK(h, launch_modeprod2(mp, h->num_cu, s));
      account_chain(h, KID_PROJECT_FUSED2, cur, proj[j], true, xdt == DT_F32 ? 4 : 2,
                    j == 0 && gather, false);
      cur[d - 2] = h->ranks[d - 2];
      cur[d - 1] = h->ranks[d - 1];
    } else {
      const int n = proj[j][0];
      ModeProd mp{};
      mp.X = X;
      mp.in_dt = xdt;
      mp.M = h->Mp[n];
      view(cur, h->d, n, &mp.A, &mp.I, &mp.B);
      mp.R = (uint32_t)h->ranks[n];
      mp.P = P;
      mp.apply = 0;
      mp.Y = Y;
      if (h->Mps[n] && !h->csplit[n]) {
        mp.Mre = h->Mps[n];
        mp.Mim = h->Mps[n] + (size_t)mp.R * mp.I;
      }
      if (h->csplit[n]) {
        const int rc = split_product(h, mp, h->Mps[n], n,
                                     j == 0 ? KID_PROJECT_FIRST : KID_PROJECT,
                                     KID_STREAM_PROJECT, Y, s);
        if (rc != TGRAD_OK) return rc;
      } else if (j == 0 && gather) {
        // the last mode (B = 1) with the COO gather: a stream of rows of the gradient
        mp.gather_S = h->S;
        mp.mask = h->mask;
        mp.rank = h->rank;
        mp.kS = h->k;
        if (!rowprod_supported(mp)) {
          h->err = "run_projection: the first single-mode launch cannot take the gather";
          return TGRAD_EHIP;
        }
        Mark m(h, KID_ROW_PROJECT);
        HIPCHK(h, launch_rowprod(mp, h->num_cu, s));
        account_chain(h, KID_ROW_PROJECT, cur, proj[j], true, xdt == DT_F32 ? 4 : 2, true,
                      false);
      } else if (h->rows && rowprod_supported(mp)) {
        // the last mode (B = 1): a stream of rows
        Mark m(h, KID_ROW_PROJECT);
        HIPCHK(h, launch_rowprod(mp, h->num_cu, s));
        account_chain(h, KID_ROW_PROJECT, cur, proj[j], true, xdt == DT_F32 ? 4 : 2, false,
                      false);
      } else {
        const int kid =
            use_stream(h, mp) ? KID_STREAM_PROJECT : j == 0 ? KID_PROJECT_FIRST : KID_PROJECT;
        Mark m(h, kid);
        HIPCHK(h, mode_product(h, mp, s));
        account_chain(h, kid, cur, proj[j], true, xdt == DT_F32 ? 4 : 2, false, false);
      }
      cur[n] = h->ranks[n];
    }
    if (j == 0 && fork_adam) {
      const int rc = fork_sparse_adam(h, *fork_adam, s);
      if (rc != TGRAD_OK) return rc;
    }
    X = Y;
    xdt = DT_F32;
    which ^= 1;
  }
  return TGRAD_OK;
}

// Reconstruction chain X x_1 U1 ... (first compressed mode first) from the core-sized
// fp32 X. apply: the last launch merges N_S at Omega and updates W; otherwise it
// writes the full fp32 tensor to out.
// wait_last: an event the last launch (the one that merges the sparse update) waits for
int run_reconstruction(tgrad_t* h, const float* X0, bool apply, void* weight, float* out,
                       hipStream_t s, hipEvent_t wait_last) {
  const uint32_t P = h->P;
  std::vector<std::vector<int>> proj, rec;
  build_chain(h, h->fuse, false, proj, rec, true, use_rec3(h, apply, weight));
  int64_t cur[TGRAD_MAX_NDIM];
  for (int i = 0; i < h->d; ++i) cur[i] = h->shape[i];
  for (int n : h->fmodes) cur[n] = h->ranks[n];
  const float lr = (float)h->lr;
  const float decay = (float)(1.0 - h->lr * h->wd);
  const void* X = X0;
  int which = 0;
  for (size_t j = 0; j < rec.size(); ++j) {
    const bool last = (j + 1 == rec.size());
    const bool app = last && apply;
    if (last && wait_last) HIPCHK(h, hipStreamWaitEvent(s, wait_last, 0));
    float* Y = last ? (apply ? nullptr : out) : h->buf[which];
    if (rec[j].size() == 3) {
      // the last three modes with the merge and the weight update (last launch, apply)
      const int d = h->d;
      ModeProd2 mp{};
      mp.X = X;
      mp.in_dt = DT_F32;
      mp.P = P;
      uint32_t A, I, B;
      view(cur, d, d - 2, &A, &I, &B);
      mp.A = A;
      mp.I0 = (uint32_t)cur[d - 3];
      mp.I1 = (uint32_t)cur[d - 2];
      mp.I2 = (uint32_t)cur[d - 1];
      mp.R0 = (uint32_t)h->shape[d - 3];
      mp.R1 = (uint32_t)h->shape[d - 2];
      mp.R2 = (uint32_t)h->shape[d - 1];
      mp.recon = 1;
      mp.M0 = h->Mr[d - 3];
      mp.M1 = h->Mr[d - 2];
      mp.M2 = h->Mr[d - 1];
      mp.apply = 1;
      mp.W = weight;
      mp.w_dt = h->dtype;
      mp.mask = h->mask;
      mp.rank = h->rank;
      mp.uS = h->S;
      mp.omega = h->omega;
      mp.kS = h->k;
      mp.lr = lr;
      mp.decay = decay;
      mp.has_sparse = h->k > 0;
      mp.delta = h->delta_cap;
      Mark m(h, KID_RECON_FUSED3_APPLY);
      HIPCHK(h, launch_rec3(mp, h->num_cu, s));
      account_chain(h, KID_RECON_FUSED3_APPLY, cur, rec[j], false, 4, false, true);
      cur[d - 3] = h->shape[d - 3];
      cur[d - 2] = h->shape[d - 2];
      cur[d - 1] = h->shape[d - 1];
    } else if (is_lead_pair(h, rec[j])) {
      const int n0 = std::min(rec[j][0], rec[j][1]);
      ModePair mp{};
      pair_view(cur, h->d, n0, &mp);
      mp.X = (const float*)X;
      mp.Y = Y;
      mp.M0 = h->Mr[n0];
      mp.M1 = h->Mr[n0 + 1];
      mp.J0 = (uint32_t)h->shape[n0];
      mp.J1 = (uint32_t)h->shape[n0 + 1];
      Mark m(h, KID_RECON_PAIR);
      HIPCHK(h, launch_pair(mp, s));
      account_chain(h, KID_RECON_PAIR, cur, rec[j], false, 4, false, false);
      cur[n0] = h->shape[n0];
      cur[n0 + 1] = h->shape[n0 + 1];
    } else if (rec[j].size() == 2) {
      const int d = h->d;
      ModeProd2 mp{};
      mp.X = X;
      mp.in_dt = DT_F32;
      mp.P = P;
      uint32_t A, I, B;
      view(cur, d, d - 2, &A, &I, &B);
      mp.A = A;
      mp.I1 = (uint32_t)cur[d - 2];
      mp.I2 = (uint32_t)cur[d - 1];
      mp.R1 = (uint32_t)h->shape[d - 2];
      mp.R2 = (uint32_t)h->shape[d - 1];
      mp.recon = 1;
      mp.M1 = h->Mr[d - 2];
      mp.M2 = h->Mr[d - 1];
      mp.apply = app ? 1 : 0;
      mp.Y = Y;
      mp.W = weight;
      mp.w_dt = (h->dtype == DT_C64) ? DT_F32 : h->dtype;
      mp.mask = h->mask;
      mp.rank = h->rank;
      mp.uS = h->S;
      mp.omega = h->omega;
      mp.kS = h->k;
      mp.lr = lr;
      mp.decay = decay;
      mp.has_sparse = app && h->k > 0;
      mp.delta = app ? h->delta_cap : nullptr;
      Mark m(h, app ? KID_RECON_FUSED2_APPLY : KID_RECON_FUSED2);
      if (h->slab2 && slab2_supported(mp, h->num_cu))
        HIPCHK(h, launch_slab2(mp, h->num_cu, s));
      else
        HIPCHK(h, launch_modeprod2(mp, h->num_cu, s));
      account_chain(h, app ? KID_RECON_FUSED2_APPLY : KID_RECON_FUSED2, cur, rec[j], false, 4,
                    false, app);
      cur[d - 2] = h->shape[d - 2];
      cur[d - 1] = h->shape[d - 1];
    } else {
      const int n = rec[j][0];
      ModeProd mp{};
      mp.X = X;
      mp.in_dt = DT_F32;
      mp.M = h->Mr[n];
      view(cur, h->d, n, &mp.A, &mp.I, &mp.B);
      mp.R = (uint32_t)h->shape[n];
      mp.P = P;
      mp.apply = app ? 1 : 0;
      mp.Y = Y;
      mp.W = weight;
      mp.w_dt = (h->dtype == DT_C64) ? DT_F32 : h->dtype;
      mp.mask = h->mask;
      mp.rank = h->rank;
      mp.uS = h->S;
      mp.omega = h->omega;
      mp.kS = h->k;
      mp.lr = lr;
      mp.decay = decay;
      mp.has_sparse = app && h->k > 0;
      mp.delta = app ? h->delta_cap : nullptr;
      if (h->Mrs[n] && !h->csplit[n]) {
        mp.Mre = h->Mrs[n];
        mp.Mim = h->Mrs[n] + (size_t)mp.R * mp.I;
      }
      if (h->csplit[n]) {
        // with apply: the full update goes to ctmp's second half, then the dense apply
        float* dst = app ? h->ctmp + h->N * P : Y;
        const int rc = split_product(h, mp, h->Mrs[n], n, KID_RECONSTRUCT,
                                     KID_STREAM_RECONSTRUCT, dst, s);
        if (rc != TGRAD_OK) return rc;
        if (app) {
          Mark m(h, KID_APPLY_DENSE);
          HIPCHK(h, launch_apply_dense(h->dtype, weight, dst, h->mask, h->rank, h->S, h->N, lr,
                                       decay, h->k > 0, h->delta_cap, s));
          record(h, KID_APPLY_DENSE, 0, h->N * (dt_bytes(h->dtype) + P * 4) + h->k * P * 4,
                 h->N * dt_bytes(h->dtype), 0);
        }
      } else if (app && h->rows && rowprod_supported(mp)) {
        // the last mode (B = 1) with the weight update: a stream of rows
        Mark m(h, KID_ROW_RECON_APPLY);
        HIPCHK(h, launch_rowprod(mp, h->num_cu, s));
        account_chain(h, KID_ROW_RECON_APPLY, cur, rec[j], false, 4, false, true);
      } else {
        const int kid =
            use_stream(h, mp) ? KID_STREAM_RECONSTRUCT : app ? KID_RECON_APPLY : KID_RECONSTRUCT;
        Mark m(h, kid);
        HIPCHK(h, mode_product(h, mp, s));
        account_chain(h, kid, cur, rec[j], false, 4, false, app);
      }
      cur[n] = h->shape[n];
    }
    X = Y;
    which ^= 1;
  }
  return TGRAD_OK;
}

}  // namespace

extern "C" {

int tgrad_step(tgrad_t* h, void* weight, const void* grad, void* stream) {
  if (!h || !weight || !grad || ((uintptr_t)grad & 15u) != 0) return TGRAD_EINVAL;
  DevGuard gd(h->device);
  hipStream_t s = (hipStream_t)stream;
  h->cur_stream = s;
  h->launches.clear();
  // the step count advances only when every launch of the step has been enqueued, so a
  // failed call can be repeated (the refresh it needs is then still due)
  const int64_t t = h->t + 1;
  if ((t - 1) % h->T == 0 && h->refreshed_for != t) {
    const int rc = do_refresh(h, grad, s, handle_ws(h));   // serves step h->t + 1 = t
    if (rc != TGRAD_OK) return rc;
  }
  const int rc = step_body(h, weight, grad, t, s);
  if (rc == TGRAD_OK) h->t = t;
  return rc;
}

}  // extern "C"

namespace {

// The one-mode plan's first projection launch is a row stream over the last mode that
// can also take the COO gather (the same ModeProd run_projection builds for it).
bool first_rows_gather(const tgrad_t* h, const void* grad,
                       const std::vector<std::vector<int>>& proj) {
  const int d = h->d;
  if (!h->rows || proj.empty() || proj[0].size() != 1 || proj[0][0] != d - 1) return false;
  if (h->csplit[d - 1]) return false;
  ModeProd mp{};
  mp.X = grad;
  mp.in_dt = (h->dtype == DT_C64) ? DT_F32 : h->dtype;
  mp.M = h->Mp[d - 1];
  view(h->shape, d, d - 1, &mp.A, &mp.I, &mp.B);
  mp.R = (uint32_t)h->ranks[d - 1];
  mp.P = h->P;
  mp.Y = h->core;   // any non-null output: only the shape and alignment are checked
  mp.gather_S = h->S;
  mp.mask = h->mask;
  mp.rank = h->rank;
  return rowprod_supported(mp);
}

int step_body(tgrad_t* h, void* weight, const void* grad, int64_t t, hipStream_t s) {
  const uint32_t P = h->P;
  const size_t nf = h->fmodes.size();
  const bool lowrank_first = h->order == TGRAD_ORDER_LOWRANK_FIRST && h->k > 0;
  const void* G0 = grad;             // the gradient the projection and dense Adam see
  int rc;
  AdamK a;
  a.b1 = (float)h->b1;
  a.c1 = (float)(1.0 - h->b1);
  a.b2 = (float)h->b2;
  a.c2 = (float)(1.0 - h->b2);
  a.eps = (float)h->eps;
  a.bc1 = (float)(1.0 - std::pow(h->b1, (double)t));
  a.bc2 = (float)(1.0 - std::pow(h->b2, (double)t));
  a.lam = (float)h->lam;
  bool forked = false;
  if (lowrank_first) {
    // the low-rank part of the whole gradient, then the sparse part of what it leaves:
    // S = (G - L)[Omega] with L = C x_n Un ... in fp32
    if (nf) {
      if ((rc = run_projection(h, grad, false, s)) != TGRAD_OK) return rc;
      if ((rc = run_reconstruction(h, h->core, false, nullptr, h->lbuf, s)) != TGRAD_OK) return rc;
      Mark m(h, KID_GATHER);
      HIPCHK(h, launch_gather_sub(h->dtype, grad, h->lbuf, h->omega, (uint32_t)h->k, h->S, s));
      // k indices, k values of G and of L read; k fp32 values written
      record(h, KID_GATHER, 0, h->k * (4 + dt_bytes(h->dtype) + 4 * P), h->k * P * 4, 0);
    } else {
      // every mode full rank: L = G, so S = 0
      HIPCHK(h, launch_fill_u32((uint32_t*)h->S, h->k * P, 0u, s));
    }
  } else {
    std::vector<std::vector<int>> proj, rec;
    build_chain(h, h->fuse, use_proj3(h, grad), proj, rec);
    // the COO gather runs on its own unless the first projection launch is a fused
    // multi-mode one, which takes S and zeroes Omega on its staged input, or a row
    // stream over the last mode, which does the same on its loaded rows
    const bool gather_fused =
        h->k > 0 && !proj.empty() && (proj[0].size() >= 2 || first_rows_gather(h, grad, proj));
    // the first projection's input: grad itself, or (when the gather is not folded into
    // it) a copy of grad that the gather turns into the residual; grad is only read
    if (h->k > 0 && !gather_fused) {
      if (!h->gcopy) {
        h->err = "no residual workspace for the unfused launch plan";
        return TGRAD_EHIP;
      }
      HIPCHK(h, hipMemcpyAsync(h->gcopy, grad, (size_t)h->N * dt_bytes(h->dtype),
                               hipMemcpyDeviceToDevice, s));
      Mark m(h, KID_GATHER);
      HIPCHK(h, launch_gather(h->dtype, h->gcopy, h->omega, (uint32_t)h->k, h->S, s));
      // k indices and values read, k fp32 values written and k values zeroed (on the
      // copy of grad, whose device copy is not a kernel launch)
      record(h, KID_GATHER, 0, h->k * (4 + dt_bytes(h->dtype)), h->k * (P * 4 + dt_bytes(h->dtype)),
             0);
      G0 = h->gcopy;
    }
    // the sparse values' Adam update forks to the second stream when the gather is folded
    // into a first projection launch that other launches follow
    forked = h->side && gather_fused && nf && proj.size() >= 2 &&
             (h->adam_overlap == 2 || (h->adam_overlap == 1 && h->k * P >= kAdamForkMin));
    if (nf) {
      rc = run_projection(h, G0, gather_fused, s, forked ? &a : nullptr);
      if (rc != TGRAD_OK) {
        if (forked) (void)hipStreamWaitEvent(s, h->ev_join, 0);
        return rc;
      }
    }
  }
  {
    Mark m(h, KID_ADAM);
    const void* gcore = nf ? (const void*)h->core : G0;
    const int cdt = nf ? DT_F32 : h->dtype;
    const uint64_t nc = h->ncore * P, nsv = forked ? 0 : h->k * P;
    HIPCHK(h, launch_adam(cdt, gcore, h->ucore, h->mC, h->vC, nc, h->S, h->mS, h->vS, nsv, a, s));
    // g, m, v read and u, m, v written, fp32, over the core and the k sparse values (the
    // dense case reads g in its storage type)
    record(h, KID_ADAM, 0, nc * (nf ? 4 : dt_bytes(h->dtype) / P) + nc * 8 + nsv * 12,
           (nc + nsv) * 12, 0);
  }
  if (nf == 0) {
    const float lr = (float)h->lr;
    const float decay = (float)(1.0 - h->lr * h->wd);
    Mark m(h, KID_APPLY_DENSE);
    HIPCHK(h, launch_apply_dense(h->dtype, weight, h->ucore, h->mask, h->rank, h->S, h->N, lr,
                                 decay, h->k > 0, h->delta_cap, s));
    record(h, KID_APPLY_DENSE, 0, h->N * (dt_bytes(h->dtype) + P * 4) + h->k * P * 4,
           h->N * dt_bytes(h->dtype), 0);
    return TGRAD_OK;
  }
  // the sparse update, forked to the second stream, is joined before the launch that
  // merges it (the reconstruction's earlier launches overlap it too)
  rc = run_reconstruction(h, h->ucore, true, weight, nullptr, s, forked ? h->ev_join : nullptr);
  if (rc != TGRAD_OK && forked) (void)hipStreamWaitEvent(s, h->ev_join, 0);
  return rc;
}

}  // namespace

extern "C" {

int tgrad_debug_capture_delta(tgrad_t* h, float* delta) {
  if (!h) return TGRAD_EINVAL;
  if (delta && ((uintptr_t)delta & 15u) != 0) return TGRAD_EINVAL;
  h->delta_cap = delta;
  return TGRAD_OK;
}

int tgrad_get_info(const tgrad_t* h, tgrad_info* out) {
  if (!h || !out) return TGRAD_EINVAL;
  int st[TGRAD_MAX_NDIM] = {0};
  const int nf = (int)h->fmodes.size();
  if (h->refreshed_once && nf) {
    DevGuard g(h->device);
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(st, h->eig_status, nf * sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(const_cast<tgrad_t*>(h), e, "tgrad_get_info");
  }
  std::memset(out, 0, sizeof(*out));
  for (int i = 0; i < nf; ++i) {
    if (st[i] < 0) out->eig_unconverged += 1;
    else if (st[i] > out->eig_sweeps_max) out->eig_sweeps_max = st[i];
  }
  out->ndim = h->d;
  out->dtype = h->dtype;
  out->numel = (int64_t)h->N;
  out->k = (int64_t)h->k;
  out->core_numel = (int64_t)h->ncore;
  out->T = h->T;
  out->t = h->t;
  for (int i = 0; i < h->d; ++i) {
    out->shape[i] = h->shape[i];
    out->ranks[i] = h->ranks[i];
  }
  out->state_bytes = h->state_bytes;
  out->workspace_bytes = h->ws_bytes;
  return TGRAD_OK;
}

int tgrad_get_omega(tgrad_t* h, uint32_t* out, int64_t cap) {
  if (!h || (!out && h->k) || cap < (int64_t)h->k) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  if (h->k) HIPCHK(h, hipMemcpy(out, h->omega, h->k * 4, hipMemcpyDeviceToHost));
  return TGRAD_OK;
}

int tgrad_get_factor(tgrad_t* h, int mode, float* out, int64_t cap) {
  if (!h || !out || mode < 0 || mode >= h->d || !h->U[mode]) return TGRAD_EINVAL;
  const uint64_t n = (uint64_t)h->shape[mode] * h->ranks[mode] * h->P;
  if (cap < (int64_t)n) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  HIPCHK(h, hipMemcpy(out, h->U[mode], n * 4, hipMemcpyDeviceToHost));
  return TGRAD_OK;
}

int tgrad_get_eigvals(tgrad_t* h, int mode, double* out, int64_t cap) {
  if (!h || !out || mode < 0 || mode >= h->d || !h->eig[mode]) return TGRAD_EINVAL;
  if (cap < h->shape[mode]) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  HIPCHK(h, hipMemcpy(out, h->eig[mode], (size_t)h->shape[mode] * 8, hipMemcpyDeviceToHost));
  return TGRAD_OK;
}

int tgrad_get_moments(tgrad_t* h, float* m_core, float* v_core, float* m_sparse,
                      float* v_sparse) {
  if (!h) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  const size_t nc = h->ncore * h->P * 4, ns = h->k * h->P * 4;
  if (m_core && nc) HIPCHK(h, hipMemcpy(m_core, h->mC, nc, hipMemcpyDeviceToHost));
  if (v_core && nc) HIPCHK(h, hipMemcpy(v_core, h->vC, nc, hipMemcpyDeviceToHost));
  if (m_sparse && ns) HIPCHK(h, hipMemcpy(m_sparse, h->mS, ns, hipMemcpyDeviceToHost));
  if (v_sparse && ns) HIPCHK(h, hipMemcpy(v_sparse, h->vS, ns, hipMemcpyDeviceToHost));
  return TGRAD_OK;
}

int tgrad_set_omega(tgrad_t* h, const uint32_t* omega, int64_t k) {
  if (!h || k != (int64_t)h->k || (k && !omega)) return TGRAD_EINVAL;
  for (int64_t j = 0; j < k; ++j) {
    if ((uint64_t)omega[j] >= h->N) return TGRAD_EINVAL;
    if (j && omega[j] <= omega[j - 1]) return TGRAD_EINVAL;
  }
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  if (k) HIPCHK(h, hipMemcpy(h->omega, omega, (size_t)k * 4, hipMemcpyHostToDevice));
  HIPCHK(h, launch_mask_from_omega(h->omega, (uint32_t)k, h->mask, h->rank, h->nwords, nullptr));
  HIPCHK(h, hipDeviceSynchronize());
  return TGRAD_OK;
}

int tgrad_set_factor(tgrad_t* h, int mode, const float* U, int64_t n_floats) {
  if (!h || !U || mode < 0 || mode >= h->d || !h->U[mode]) return TGRAD_EINVAL;
  const uint32_t I = (uint32_t)h->shape[mode], r = (uint32_t)h->ranks[mode];
  const uint64_t n = (uint64_t)I * r * h->P;
  if (n_floats != (int64_t)n) return TGRAD_EINVAL;
  std::vector<float> mp(n * h->P), mr(n * h->P);
  host_operands(I, r, h->P, U, mp.data(), mr.data());
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  HIPCHK(h, hipMemcpy(h->U[mode], U, n * 4, hipMemcpyHostToDevice));
  HIPCHK(h, hipMemcpy(h->Mp[mode], mp.data(), mp.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(h, hipMemcpy(h->Mr[mode], mr.data(), mr.size() * 4, hipMemcpyHostToDevice));
  if (h->Mps[mode]) {
    HIPCHK(h, split_operands(h, mode, nullptr));
    HIPCHK(h, hipDeviceSynchronize());
  }
  return TGRAD_OK;
}

// ---------------------------------------------------------------- checkpoint / resume
// Layout: header, then Omega (k u32), per compressed mode (ascending) U(n) (I r P fp32)
// and its eigenvalues (I fp64), then m_C, v_C (core P fp32 each), m_S, v_S (k P fp32
// each). Membership mask, ranks and the MFMA operand matrices are rebuilt on load.
}  // extern "C"
namespace {
struct CkptHeader {
  char magic[8];
  uint32_t version, dtype;
  int64_t ndim;
  int64_t shape[TGRAD_MAX_NDIM];
  int64_t ranks[TGRAD_MAX_NDIM];
  uint64_t k, ncore;
  int64_t t, refreshed_for;
  // hyper-parameters and options of the saved run (version 2)
  int64_t T;
  double lr, beta1, beta2, eps;
  double weight_decay, sparse_scale;
  uint64_t seed;
  int32_t selection, remap, order, pad;
};
constexpr char kCkptMagic[8] = {'T', 'G', 'R', 'A', 'D', 'C', 'K', '1'};
constexpr uint32_t kCkptVersion = 2;

void ckpt_header(const tgrad_t* h, CkptHeader* c) {
  std::memset(c, 0, sizeof(*c));
  std::memcpy(c->magic, kCkptMagic, 8);
  c->version = kCkptVersion;
  c->dtype = (uint32_t)h->dtype;
  c->ndim = h->d;
  for (int i = 0; i < h->d; ++i) {
    c->shape[i] = h->shape[i];
    c->ranks[i] = h->ranks[i];
  }
  c->k = h->k;
  c->ncore = h->ncore;
  c->t = h->t;
  c->refreshed_for = h->refreshed_for;
  c->T = h->T;
  c->lr = h->lr;
  c->beta1 = h->b1;
  c->beta2 = h->b2;
  c->eps = h->eps;
  c->weight_decay = h->wd;
  c->sparse_scale = h->lam;
  c->seed = h->seed;
  c->selection = h->selection;
  c->remap = h->remap ? 1 : 0;
  c->order = h->order;
}

// The saved run and this handle agree on everything that shapes the steps after the
// resume: tensor layout, Omega size, refresh period, Adam's betas and eps, and every
// option. The learning rate may differ (a schedule may change it between runs).
bool ckpt_compatible(const CkptHeader& a, const CkptHeader& b) {
  return std::memcmp(a.magic, b.magic, 8) == 0 && a.version == b.version && a.dtype == b.dtype &&
         a.ndim == b.ndim && a.k == b.k && a.ncore == b.ncore &&
         std::memcmp(a.shape, b.shape, sizeof(a.shape)) == 0 &&
         std::memcmp(a.ranks, b.ranks, sizeof(a.ranks)) == 0 && a.T == b.T &&
         a.beta1 == b.beta1 && a.beta2 == b.beta2 && a.eps == b.eps &&
         a.weight_decay == b.weight_decay && a.sparse_scale == b.sparse_scale &&
         a.seed == b.seed && a.selection == b.selection && a.remap == b.remap &&
         a.order == b.order;
}

// (device pointer, bytes) of every state array in checkpoint order
std::vector<std::pair<void*, size_t>> ckpt_arrays(tgrad_t* h) {
  std::vector<std::pair<void*, size_t>> a;
  a.push_back({h->omega, (size_t)h->k * 4});
  for (int n : h->fmodes) {
    const size_t I = (size_t)h->shape[n], r = (size_t)h->ranks[n];
    a.push_back({h->U[n], I * r * h->P * 4});
    a.push_back({h->eig[n], I * 8});
  }
  const size_t nc = (size_t)h->ncore * h->P * 4, ns = (size_t)h->k * h->P * 4;
  a.push_back({h->mC, nc});
  a.push_back({h->vC, nc});
  a.push_back({h->mS, ns});
  a.push_back({h->vS, ns});
  return a;
}
}  // namespace
extern "C" {

int64_t tgrad_state_size(tgrad_t* h) {
  if (!h) return -1;
  int64_t n = (int64_t)sizeof(CkptHeader);
  for (auto& a : ckpt_arrays(h)) n += (int64_t)a.second;
  return n;
}

int tgrad_save_state(tgrad_t* h, void* buf, int64_t cap) {
  if (!h || !buf || cap < tgrad_state_size(h)) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  unsigned char* p = (unsigned char*)buf;
  ckpt_header(h, (CkptHeader*)p);
  p += sizeof(CkptHeader);
  for (auto& a : ckpt_arrays(h)) {
    if (a.second) HIPCHK(h, hipMemcpy(p, a.first, a.second, hipMemcpyDeviceToHost));
    p += a.second;
  }
  return TGRAD_OK;
}

int tgrad_load_state(tgrad_t* h, const void* buf, int64_t size) {
  if (!h || !buf || size != tgrad_state_size(h)) return TGRAD_EINVAL;
  CkptHeader mine, theirs;
  ckpt_header(h, &mine);
  std::memcpy(&theirs, buf, sizeof(theirs));
  if (!ckpt_compatible(theirs, mine) || theirs.t < 0) return TGRAD_EINVAL;
  const unsigned char* p = (const unsigned char*)buf + sizeof(CkptHeader);
  // Omega must be ascending and in range, as tgrad_set_omega requires
  const uint32_t* om = (const uint32_t*)p;
  for (uint64_t j = 0; j < h->k; ++j) {
    uint32_t x;
    std::memcpy(&x, om + j, 4);
    uint32_t prev = 0;
    if (j) std::memcpy(&prev, om + j - 1, 4);
    if ((uint64_t)x >= h->N || (j && x <= prev)) return TGRAD_EINVAL;
  }
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  for (auto& a : ckpt_arrays(h)) {
    if (a.second) HIPCHK(h, hipMemcpy(a.first, p, a.second, hipMemcpyHostToDevice));
    p += a.second;
  }
  HIPCHK(h, launch_mask_from_omega(h->omega, (uint32_t)h->k, h->mask, h->rank, h->nwords,
                                   nullptr));
  for (int n : h->fmodes) {
    const uint32_t I = (uint32_t)h->shape[n], r = (uint32_t)h->ranks[n];
    const size_t nu = (size_t)I * r * h->P;
    std::vector<float> U(nu), mp(nu * h->P), mr(nu * h->P);
    HIPCHK(h, hipMemcpy(U.data(), h->U[n], nu * 4, hipMemcpyDeviceToHost));
    host_operands(I, r, h->P, U.data(), mp.data(), mr.data());
    HIPCHK(h, hipMemcpy(h->Mp[n], mp.data(), mp.size() * 4, hipMemcpyHostToDevice));
    HIPCHK(h, hipMemcpy(h->Mr[n], mr.data(), mr.size() * 4, hipMemcpyHostToDevice));
    if (h->Mps[n]) HIPCHK(h, split_operands(h, n, nullptr));
  }
  HIPCHK(h, hipDeviceSynchronize());
  h->t = theirs.t;
  h->refreshed_for = theirs.refreshed_for;
  return TGRAD_OK;
}

void tgrad_default_options(tgrad_options* out) {
  if (!out) return;
  std::memset(out, 0, sizeof(*out));
  out->weight_decay = 0.0;
  out->sparse_scale = 1.0;
  out->selection = TGRAD_SELECT_TOPK;
  out->remap_moments = 0;
  out->seed = 0;
  out->order = TGRAD_ORDER_SPARSE_FIRST;
}

int tgrad_get_options(const tgrad_t* h, tgrad_options* out) {
  if (!h || !out) return TGRAD_EINVAL;
  tgrad_default_options(out);
  out->weight_decay = h->wd;
  out->sparse_scale = h->lam;
  out->selection = h->selection;
  out->remap_moments = h->remap ? 1 : 0;
  out->seed = h->seed;
  out->order = h->order;
  return TGRAD_OK;
}

int tgrad_set_options(tgrad_t* h, const tgrad_options* o) {
  if (!h || !o) return TGRAD_EINVAL;
  if (!std::isfinite(o->weight_decay) || o->weight_decay < 0.0 || !std::isfinite(o->sparse_scale))
    return TGRAD_EINVAL;
  if (o->selection != TGRAD_SELECT_TOPK && o->selection != TGRAD_SELECT_RANDK) return TGRAD_EINVAL;
  if (o->remap_moments != 0 && o->remap_moments != 1) return TGRAD_EINVAL;
  if (o->order != TGRAD_ORDER_SPARSE_FIRST && o->order != TGRAD_ORDER_LOWRANK_FIRST)
    return TGRAD_EINVAL;
  if (o->order == TGRAD_ORDER_LOWRANK_FIRST && h->k > 0 && !h->fmodes.empty() && !h->lbuf) {
    DevGuard g(h->device);
    if (!dalloc(h, &h->lbuf, h->N * h->P, false)) return TGRAD_ENOMEM;
  }
  if (o->remap_moments && h->k > 0 && !h->mask_prev) {
    DevGuard g(h->device);
    const uint64_t ns = h->k * h->P;
    bool ok = dalloc(h, &h->mask_prev, h->nwords, false);
    ok = ok && dalloc(h, &h->rank_prev, h->nwords, false);
    ok = ok && dalloc(h, &h->mS_alt, ns, true);
    ok = ok && dalloc(h, &h->vS_alt, ns, true);
    if (!ok) {
      // keep the handle usable: release what this call got
      struct Part { void** p; int64_t bytes; bool state; };
      const Part parts[4] = {{(void**)&h->mask_prev, (int64_t)h->nwords * 8, false},
                             {(void**)&h->rank_prev, (int64_t)h->nwords * 4, false},
                             {(void**)&h->mS_alt, (int64_t)ns * 4, true},
                             {(void**)&h->vS_alt, (int64_t)ns * 4, true}};
      for (const Part& q : parts) {
        if (!*q.p) continue;
        auto it = std::find(h->allocs.begin(), h->allocs.end(), *q.p);
        if (it != h->allocs.end()) h->allocs.erase(it);
        (void)hipFree(*q.p);
        *q.p = nullptr;
        (q.state ? h->state_bytes : h->ws_bytes) -= q.bytes;
      }
      return TGRAD_ENOMEM;
    }
    HIPCHK(h, hipDeviceSynchronize());
    HIPCHK(h, hipMemset(h->mask_prev, 0, h->nwords * 8));
    HIPCHK(h, hipMemset(h->rank_prev, 0, h->nwords * 4));
    HIPCHK(h, hipDeviceSynchronize());
  }
  h->wd = o->weight_decay;
  h->lam = o->sparse_scale;
  h->selection = o->selection;
  h->remap = o->remap_moments != 0;
  h->seed = o->seed;
  h->order = o->order;
  return TGRAD_OK;
}

int tgrad_set_fusion(tgrad_t* h, int enable) {
  if (!h || enable < 0 || enable > 4) return TGRAD_EINVAL;
  if (enable && !h->can_fuse) return TGRAD_EINVAL;
  if (!enable && h->k > 0 && !h->gcopy) {
    DevGuard g(h->device);
    unsigned char* gc = nullptr;
    if (!dalloc(h, &gc, h->N * dt_bytes(h->dtype), false)) return TGRAD_ENOMEM;
    h->gcopy = gc;
  }
  h->fuse = enable != 0;
  h->slab2 = enable != 2;
  h->slab3 = enable == 1 || enable == 4;
  h->rec3 = enable == 1;
  return TGRAD_OK;
}

int tgrad_set_stream_products(tgrad_t* h, int enable) {
  if (!h || enable < 0) return TGRAD_EINVAL;
  h->stream = enable != 0;
  h->rows = enable != 0;
  h->stream_wg = enable > 1 ? enable - 1 : 0;
  return TGRAD_OK;
}

int tgrad_set_stream_overlap(tgrad_t* h, int adam, int eig) {
  if (!h || adam < 0 || adam > 2 || eig < 0 || eig > 1) return TGRAD_EINVAL;
  h->adam_overlap = adam;
  h->eig_overlap = eig != 0;
  return TGRAD_OK;
}

int tgrad_set_pair_fusion(tgrad_t* h, int enable) {
  if (!h || enable < 0 || enable > 1) return TGRAD_EINVAL;
  if (enable && !h->can_pair) return TGRAD_EINVAL;
  h->pairs = enable != 0;
  return TGRAD_OK;
}

int tgrad_set_gram_fusion(tgrad_t* h, int enable) {
  if (!h || enable < 0 || enable > 3) return TGRAD_EINVAL;
  if ((enable & 1) && !h->can_gram3) return TGRAD_EINVAL;
  h->gram3 = (enable & 1) != 0;
  h->gram_masked = (enable & 2) != 0;
  return TGRAD_OK;
}

int tgrad_mark_refreshed(tgrad_t* h) {
  if (!h) return TGRAD_EINVAL;
  h->refreshed_for = h->t + 1;
  return TGRAD_OK;
}

int tgrad_last_launches(const tgrad_t* h, tgrad_launch* out, int cap) {
  if (!h || cap < 0 || (cap > 0 && !out)) return -1;
  const int n = (int)h->launches.size();
  for (int i = 0; i < n && i < cap; ++i) out[i] = h->launches[i];
  return n;
}

int tgrad_timing_enable(tgrad_t* h, int enable, int max_records) {
  if (!h || max_records < 0) return TGRAD_EINVAL;
  h->timing = enable != 0;
  h->max_rec = max_records;
  return TGRAD_OK;
}

int tgrad_timing_only(tgrad_t* h, int id) {
  if (!h || id < -1 || id >= TGRAD_MAX_KERNEL_IDS) return TGRAD_EINVAL;
  h->timing_only = id;
  return TGRAD_OK;
}

// ---------------------------------------------------------------- refresh without allocation
}  // extern "C"

// The scratch of tgrad_refresh_noalloc: one array per GPU for the life of the process. In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device (g_scratch_ptr), and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[TGRAD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<unsigned char*> g_scratch_ptr;   // per device: scratch's device address

// The device address of this device's scratch array (the device is current).
int scratch_address(tgrad_t* h, unsigned char** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= h->device) g_scratch_ptr.resize(h->device + 1, nullptr);
  if (!g_scratch_ptr[h->device]) {
    void* p = nullptr;
    HIPCHK(h, hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) {
      h->err = "tgrad_refresh_noalloc: no device address for the scratch array";
      return TGRAD_EHIP;
    }
    g_scratch_ptr[h->device] = (unsigned char*)p;
  }
  *out = g_scratch_ptr[h->device];
  return TGRAD_OK;
}

// The refresh's scratch carved from the array at `base`: top-k workspace, Gram matrices,
// then the Gram partial sums with each launch's workgroups capped so that they fit.
// Returns false (with h->err set) when the refresh needs more than the array holds.
bool noalloc_ws(tgrad_t* h, unsigned char* base, RefreshWs* ws) {
  const size_t cap = TGRAD_NOALLOC_SCRATCH_BYTES;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const uint64_t units = topk_units(h->N), chunks = topk_chunks(h->N);
  size_t off = 0;
  const size_t o_hist = off;   off += up(TOPK_HIST_BINS * 4);
  const size_t o_state = off;  off += up(4 * 8);
  const size_t o_ucount = off; off += up(2 * units * 4);
  const size_t o_uoff = off;   off += up(2 * units * 4);
  const size_t o_ctot = off;   off += up(2 * chunks * 4);
  const size_t o_gram = off;   off += up((size_t)h->gram_stride * h->fmodes.size() * 8);
  const size_t o_part = off;
  if (off >= cap) {
    h->err = "tgrad_refresh_noalloc: the top-k workspace for this N exceeds the scratch array";
    return false;
  }
  const size_t avail = (cap - off) / 8;   // doubles for the partial sums
  const uint64_t groups = gram_reduce_groups();
  uint64_t blocks = UINT32_MAX;
  for (int n : h->fmodes) {
    const uint64_t K2 = (uint64_t)h->shape[n] * h->P * h->shape[n] * h->P;
    const uint64_t fit = avail / K2;
    if (fit <= groups) {
      h->err = "tgrad_refresh_noalloc: a Gram partial sum exceeds the scratch array";
      return false;
    }
    blocks = std::min<uint64_t>(blocks, fit - groups);
  }
  Gram3Args g3;
  if (h->gram3 && h->can_gram3 && h->k > 0 &&
      gram3_args(h, (const void*)(uintptr_t)256, h->mask, nullptr, &g3) &&
      gram3_supported(g3, h->num_cu) && gram3_partial_doubles(g3, h->num_cu) > avail) {
    h->err = "tgrad_refresh_noalloc: the three-mode Gram partial sums exceed the scratch array";
    return false;
  }
  ws->tw.hist = (uint32_t*)(base + o_hist);
  ws->tw.state = (uint64_t*)(base + o_state);
  ws->tw.ucount = (uint32_t*)(base + o_ucount);
  ws->tw.uoff = (uint32_t*)(base + o_uoff);
  ws->tw.ctot = (uint32_t*)(base + o_ctot);
  ws->gram = (double*)(base + o_gram);
  ws->gram_part = (double*)(base + o_part);
  ws->masked = true;
  ws->max_gram_blocks = (uint32_t)std::min<uint64_t>(blocks, UINT32_MAX);
  return true;
}

}  // namespace

extern "C" {

int tgrad_refresh_noalloc(tgrad_t* h, const void* grad, void* stream) {
  if (!h || !grad || ((uintptr_t)grad & 15u) != 0) return TGRAD_EINVAL;
  if (h->order == TGRAD_ORDER_LOWRANK_FIRST && h->k > 0 && !h->fmodes.empty()) {
    h->err = "tgrad_refresh_noalloc: the low-rank-first order needs full-size intermediates";
    return TGRAD_EINVAL;
  }
  DevGuard g(h->device);
  unsigned char* base = nullptr;
  int rc = scratch_address(h, &base);
  if (rc != TGRAD_OK) return rc;
  RefreshWs ws{};
  if (!noalloc_ws(h, base, &ws)) return TGRAD_EINVAL;
  h->cur_stream = (hipStream_t)stream;
  h->launches.clear();
  // per-launch timing would create events: off for this call
  const bool timing = h->timing;
  h->timing = false;
  rc = do_refresh(h, grad, (hipStream_t)stream, ws);
  h->timing = timing;
  return rc;
}

int tgrad_timing_read(tgrad_t* h, int64_t* launches, double* ms, int n_ids) {
  if (!h || n_ids < 0 || n_ids > TGRAD_MAX_KERNEL_IDS) return TGRAD_EINVAL;
  DevGuard g(h->device);
  HIPCHK(h, hipDeviceSynchronize());
  for (int i = 0; i < n_ids; ++i) {
    if (launches) launches[i] = 0;
    if (ms) ms[i] = 0.0;
  }
  for (auto& r : h->recs) {
    float el = 0.0f;
    if (r.a && r.b && hipEventElapsedTime(&el, r.a, r.b) == hipSuccess && r.id < n_ids) {
      if (launches) launches[r.id] += 1;
      if (ms) ms[r.id] += el;
    }
    h->pool.push_back(r.a);
    h->pool.push_back(r.b);
  }
  h->recs.clear();
  return TGRAD_OK;
}

}  // extern "C"
