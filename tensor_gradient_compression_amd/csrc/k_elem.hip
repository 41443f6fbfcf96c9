// Element-wise kernels of the TensorGRaD step:
//   gather:       S = G[Omega] in fp32 and G[Omega] <- 0, so G becomes the residual in
//                 place (nullthought summary section 3: the sparse part is extracted
//                 first and the remainder is the residual).
//   adam:         fp32 Adam on the core and on the sparse values in one launch
//                 (nullthought section 3: each part gets its own Adam update; section 3
//                 mixed precision: optimizer state stays fp32; pith.science: Adam
//                 moments live on the core). Operation order, each rounded to fp32:
//                 m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g);
//                 u = (m/bc1) / (sqrt(v/bc2) + eps); the sparse output is then scaled
//                 by lambda (1 for the plain method, an exact identity). The library is built without
//                 floating-point contraction, so no step is fused into an FMA.
//   gather_sub,   low-rank first: S = G[Omega] - L[Omega], and the residual G - L that
//   resid_sub:    its refresh selects Omega from (nullthought summary section 5 and
//                 pith.science free parameters: the decomposition order is a choice).
//   apply_dense:  the update when no mode is compressed (every r_n = I_n): Delta =
//                 N_C, plus N_S at Omega, W <- round(W * decay - lr * Delta), decay =
//                 fp32(1 - lr * weight_decay) (decoupled decay, exactly 1 without it).
//   csplit:       complex mode products wider than the tiled kernel's 128 real rows
//                 and columns run as two real products on the interleaved (re, im)
//                 view of the tensor, one with Re M and one with Im M;
//                 split_operand takes those two parts out of the real-block operand
//                 and combine forms (Re M) x + i (Im M) x from the two outputs.
#include "tg_common.h"

namespace tg {

namespace {

unsigned grid_for(uint64_t n, unsigned per_block, unsigned cap) {
  uint64_t b = (n + per_block - 1) / per_block;
  if (b > cap) b = cap;
  return b ? (unsigned)b : 1u;
}

template <typename ST, int P>
__global__ void __launch_bounds__(256) k_gather(ST* __restrict__ G,
                                                const uint32_t* __restrict__ omega, uint32_t k,
                                                float* __restrict__ S) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < k; j += stride) {
    const uint64_t e = omega[j];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      S[j * P + p] = to_f32(G[e * P + p]);
      G[e * P + p] = zero_of<ST>();
    }
  }
}

template <typename ST, int P>
__global__ void __launch_bounds__(256) k_gather_sub(const ST* __restrict__ G,
                                                    const float* __restrict__ L,
                                                    const uint32_t* __restrict__ omega,
                                                    uint32_t k, float* __restrict__ S) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < k; j += stride) {
    const uint64_t e = omega[j];
#pragma unroll
    for (int p = 0; p < P; ++p) S[j * P + p] = to_f32(G[e * P + p]) - L[e * P + p];
  }
}

// four values per thread per pass (16-byte L accesses when the tail allows)
template <typename ST>
__global__ void __launch_bounds__(256) k_resid_sub(const ST* __restrict__ G, float* __restrict__ L,
                                                   uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 4;
  for (uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      float4 l = *(const float4*)(L + i);
      l.x = to_f32(G[i]) - l.x;
      l.y = to_f32(G[i + 1]) - l.y;
      l.z = to_f32(G[i + 2]) - l.z;
      l.w = to_f32(G[i + 3]) - l.w;
      *(float4*)(L + i) = l;
    } else {
      for (uint64_t q = i; q < n; ++q) L[q] = to_f32(G[q]) - L[q];
    }
  }
}

__device__ __forceinline__ float adam_one(float g, float& m, float& v, const AdamK& a) {
  m = a.b1 * m + a.c1 * g;
  v = a.b2 * v + a.c2 * (g * g);
  return (m / a.bc1) / (sqrtf(v / a.bc2) + a.eps);
}

template <typename CT>
__global__ void __launch_bounds__(256) k_adam(const CT* __restrict__ gc, float* __restrict__ uc,
                                              float* __restrict__ mc, float* __restrict__ vc,
                                              uint64_t nc, float* __restrict__ S,
                                              float* __restrict__ ms, float* __restrict__ vs,
                                              uint64_t ns, AdamK a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t n = nc + ns;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (i < nc) {
      float m = mc[i], v = vc[i];
      uc[i] = adam_one(to_f32(gc[i]), m, v, a);
      mc[i] = m;
      vc[i] = v;
    } else {
      const uint64_t j = i - nc;
      float m = ms[j], v = vs[j];
      S[j] = a.lam * adam_one(S[j], m, v, a);
      ms[j] = m;
      vs[j] = v;
    }
  }
}

// The sparse values' update alone (its own symbol, so that a profile tells it apart from
// the launch that also updates the core)
__global__ void __launch_bounds__(256) k_adam_sparse(float* __restrict__ S,
                                                     float* __restrict__ ms,
                                                     float* __restrict__ vs, uint64_t ns,
                                                     AdamK a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < ns; j += stride) {
    float m = ms[j], v = vs[j];
    S[j] = a.lam * adam_one(S[j], m, v, a);
    ms[j] = m;
    vs[j] = v;
  }
}

// The same updates four values a thread (16-byte accesses; every buffer 16-byte aligned):
// quads of the core, then quads of the sparse values, then the two tails one value a
// thread. Each value sees the operations of the one-value kernels, so results are
// bit-identical to theirs.
__device__ __forceinline__ void adam_quad(const float* g, float* u, float* m, float* v,
                                          const AdamK& a, float scale) {
  const float4 gq = *(const float4*)g;
  float4 mq = *(const float4*)m, vq = *(const float4*)v, uq;
  uq.x = scale * adam_one(gq.x, mq.x, vq.x, a);
  uq.y = scale * adam_one(gq.y, mq.y, vq.y, a);
  uq.z = scale * adam_one(gq.z, mq.z, vq.z, a);
  uq.w = scale * adam_one(gq.w, mq.w, vq.w, a);
  *(float4*)u = uq;
  *(float4*)m = mq;
  *(float4*)v = vq;
}
__device__ __forceinline__ void adam4_body(const float* __restrict__ gc, float* __restrict__ uc,
                                           float* __restrict__ mc, float* __restrict__ vc,
                                           uint64_t nc, float* __restrict__ S,
                                           float* __restrict__ ms, float* __restrict__ vs,
                                           uint64_t ns, const AdamK& a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t qc = nc / 4, qs = ns / 4;
  for (uint64_t i = tid; i < qc + qs; i += stride) {
    if (i < qc) {
      adam_quad(gc + 4 * i, uc + 4 * i, mc + 4 * i, vc + 4 * i, a, 1.0f);
    } else {
      const uint64_t j = 4 * (i - qc);
      // N_S = lam * update; lam = 1 multiplies exactly
      adam_quad(S + j, S + j, ms + j, vs + j, a, a.lam);
    }
  }
  const uint64_t tc = nc - 4 * qc, ts = ns - 4 * qs;
  if (tid < tc) {
    const uint64_t i = 4 * qc + tid;
    float m = mc[i], v = vc[i];
    uc[i] = adam_one(gc[i], m, v, a);
    mc[i] = m;
    vc[i] = v;
  } else if (tid < tc + ts) {
    const uint64_t j = 4 * qs + (tid - tc);
    float m = ms[j], v = vs[j];
    S[j] = a.lam * adam_one(S[j], m, v, a);
    ms[j] = m;
    vs[j] = v;
  }
}

__global__ void __launch_bounds__(256) k_adam4(const float* __restrict__ gc, float* __restrict__ uc,
                                               float* __restrict__ mc, float* __restrict__ vc,
                                               uint64_t nc, float* __restrict__ S,
                                               float* __restrict__ ms, float* __restrict__ vs,
                                               uint64_t ns, AdamK a) {
  adam4_body(gc, uc, mc, vc, nc, S, ms, vs, ns, a);
}
// the sparse values alone (its own symbol, so that a profile tells it apart)
__global__ void __launch_bounds__(256) k_adam_sparse4(float* __restrict__ S,
                                                      float* __restrict__ ms,
                                                      float* __restrict__ vs, uint64_t ns,
                                                      AdamK a) {
  adam4_body(nullptr, nullptr, nullptr, nullptr, 0, S, ms, vs, ns, a);
}

template <typename WT, int P>
__global__ void __launch_bounds__(256) k_apply_dense(WT* __restrict__ W,
                                                     const float* __restrict__ uc,
                                                     const uint64_t* __restrict__ mask,
                                                     const uint32_t* __restrict__ rank,
                                                     const float* __restrict__ us, uint64_t N,
                                                     float lr, float decay,
                                                     int has_sparse, float* __restrict__ delta) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < N; e += stride) {
    float d[P];
#pragma unroll
    for (int p = 0; p < P; ++p) d[p] = uc[e * P + p];
    if (has_sparse) {
      const uint64_t word = mask[e >> 6];
      if ((word >> (e & 63)) & 1ull) {
        const uint64_t j = omega_rank(mask, rank, e, word);
#pragma unroll
        for (int p = 0; p < P; ++p) d[p] = d[p] + us[j * P + p];
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float w = to_f32(W[e * P + p]);
      W[e * P + p] = from_f32<WT>(w * decay - lr * d[p]);
      if (delta) delta[e * P + p] = d[p];   // test capture of the fp32 update
    }
  }
}

}  // namespace

hipError_t launch_gather(int dt, void* G, const uint32_t* omega, uint32_t k, float* S,
                         hipStream_t s) {
  if (!k) return hipSuccess;
  const unsigned b = grid_for(k, 256, 8192);
  switch (dt) {
    case DT_F32: k_gather<float, 1><<<b, 256, 0, s>>>((float*)G, omega, k, S); break;
    case DT_F16: k_gather<_Float16, 1><<<b, 256, 0, s>>>((_Float16*)G, omega, k, S); break;
    case DT_BF16: k_gather<bf16_t, 1><<<b, 256, 0, s>>>((bf16_t*)G, omega, k, S); break;
    case DT_C64: k_gather<float, 2><<<b, 256, 0, s>>>((float*)G, omega, k, S); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gather_sub(int dt, const void* G, const float* L, const uint32_t* omega,
                             uint32_t k, float* S, hipStream_t s) {
  if (!k) return hipSuccess;
  const unsigned b = grid_for(k, 256, 8192);
  switch (dt) {
    case DT_F32: k_gather_sub<float, 1><<<b, 256, 0, s>>>((const float*)G, L, omega, k, S); break;
    case DT_F16: k_gather_sub<_Float16, 1><<<b, 256, 0, s>>>((const _Float16*)G, L, omega, k, S); break;
    case DT_BF16: k_gather_sub<bf16_t, 1><<<b, 256, 0, s>>>((const bf16_t*)G, L, omega, k, S); break;
    case DT_C64: k_gather_sub<float, 2><<<b, 256, 0, s>>>((const float*)G, L, omega, k, S); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_sub(int dt, const void* G, float* L, uint64_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  const unsigned b = grid_for((n + 3) / 4, 256, 16384);
  switch (dt) {
    case DT_F32:
    case DT_C64: k_resid_sub<float><<<b, 256, 0, s>>>((const float*)G, L, n); break;
    case DT_F16: k_resid_sub<_Float16><<<b, 256, 0, s>>>((const _Float16*)G, L, n); break;
    case DT_BF16: k_resid_sub<bf16_t><<<b, 256, 0, s>>>((const bf16_t*)G, L, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_adam(int core_dt, const void* g_core, float* u_core, float* m_core,
                       float* v_core, uint64_t n_core, float* S, float* m_s, float* v_s,
                       uint64_t n_s, AdamK a, hipStream_t s) {
  const uint64_t n = n_core + n_s;
  if (!n) return hipSuccess;
  const unsigned b = grid_for(n, 256, 8192);
  auto al16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  switch (core_dt) {
    case DT_F32:
    case DT_C64:
      if (al16(g_core) && al16(u_core) && al16(m_core) && al16(v_core) && al16(S) && al16(m_s) &&
          al16(v_s)) {
        k_adam4<<<grid_for(n / 4 + 8, 256, 8192), 256, 0, s>>>(
            (const float*)g_core, u_core, m_core, v_core, n_core, S, m_s, v_s, n_s, a);
        break;
      }
      k_adam<float><<<b, 256, 0, s>>>((const float*)g_core, u_core, m_core, v_core, n_core, S,
                                      m_s, v_s, n_s, a);
      break;
    case DT_F16:
      k_adam<_Float16><<<b, 256, 0, s>>>((const _Float16*)g_core, u_core, m_core, v_core,
                                         n_core, S, m_s, v_s, n_s, a);
      break;
    case DT_BF16:
      k_adam<bf16_t><<<b, 256, 0, s>>>((const bf16_t*)g_core, u_core, m_core, v_core, n_core,
                                       S, m_s, v_s, n_s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_adam_sparse(float* S, float* m_s, float* v_s, uint64_t n_s, AdamK a,
                              hipStream_t s) {
  if (!n_s) return hipSuccess;
  if ((((uintptr_t)S | (uintptr_t)m_s | (uintptr_t)v_s) & 15u) == 0) {
    k_adam_sparse4<<<grid_for(n_s / 4 + 8, 256, 8192), 256, 0, s>>>(S, m_s, v_s, n_s, a);
    return hipGetLastError();
  }
  const unsigned b = grid_for(n_s, 256, 8192);
  k_adam_sparse<<<b, 256, 0, s>>>(S, m_s, v_s, n_s, a);
  return hipGetLastError();
}

hipError_t launch_apply_dense(int dt, void* W, const float* u_core, const uint64_t* mask,
                              const uint32_t* rank, const float* u_s, uint64_t N, float lr,
                              float decay, int has_sparse, float* delta, hipStream_t s) {
  const unsigned b = grid_for(N, 256, 8192);
  switch (dt) {
    case DT_F32:
      k_apply_dense<float, 1><<<b, 256, 0, s>>>((float*)W, u_core, mask, rank, u_s, N, lr,
                                                decay, has_sparse, delta);
      break;
    case DT_F16:
      k_apply_dense<_Float16, 1><<<b, 256, 0, s>>>((_Float16*)W, u_core, mask, rank, u_s, N, lr,
                                                   decay, has_sparse, delta);
      break;
    case DT_BF16:
      k_apply_dense<bf16_t, 1><<<b, 256, 0, s>>>((bf16_t*)W, u_core, mask, rank, u_s, N, lr,
                                                 decay, has_sparse, delta);
      break;
    case DT_C64:
      k_apply_dense<float, 2><<<b, 256, 0, s>>>((float*)W, u_core, mask, rank, u_s, N, lr,
                                                decay, has_sparse, delta);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {

// re[r, c] = M[2r, 2c] and im[r, c] = M[2r + 1, 2c] of the (2 rows) x (2 cols) real-block
// form of a complex matrix (each entry a + ib stored as the block [[a, -b], [b, a]])
__global__ void __launch_bounds__(256) k_split_operand(const float* __restrict__ M,
                                                       uint32_t rows, uint32_t cols,
                                                       float* __restrict__ re,
                                                       float* __restrict__ im) {
  const uint64_t n = (uint64_t)rows * cols;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    const uint64_t r = j / cols, c = j % cols;
    re[j] = M[(2 * r) * (2 * (uint64_t)cols) + 2 * c];
    im[j] = M[(2 * r + 1) * (2 * (uint64_t)cols) + 2 * c];
  }
}

// y1 holds (Re M) x and y2 (Im M) x, both as (re, im) pairs; y1 <- M x:
// re = y1.re - y2.im, im = y1.im + y2.re. VEC (both buffers 16-byte aligned): two
// complex values (16 bytes) per thread and pass, and an odd count leaves one pair, done
// on its own; otherwise one pair per thread and pass.
template <bool VEC>
__global__ void __launch_bounds__(256) k_csplit_combine(float* __restrict__ y1,
                                                        const float* __restrict__ y2,
                                                        uint64_t npairs) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t t0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!VEC) {
    for (uint64_t q = t0; q < npairs; q += stride) {
      const float ar = y1[2 * q], ai = y1[2 * q + 1], br = y2[2 * q], bi = y2[2 * q + 1];
      y1[2 * q] = ar - bi;
      y1[2 * q + 1] = ai + br;
    }
    return;
  }
  const uint64_t nq = npairs / 2;
  for (uint64_t q = t0; q < nq; q += stride) {
    const float4 a = reinterpret_cast<const float4*>(y1)[q];
    const float4 b = reinterpret_cast<const float4*>(y2)[q];
    reinterpret_cast<float4*>(y1)[q] = make_float4(a.x - b.y, a.y + b.x, a.z - b.w, a.w + b.z);
  }
  if ((npairs & 1) && t0 == 0) {
    const uint64_t e = 2 * (npairs - 1);
    const float ar = y1[e], ai = y1[e + 1], br = y2[e], bi = y2[e + 1];
    y1[e] = ar - bi;
    y1[e + 1] = ai + br;
  }
}

}  // namespace

hipError_t launch_split_operand(const float* M, uint32_t rows, uint32_t cols, float* re,
                                float* im, hipStream_t s) {
  k_split_operand<<<grid_for((uint64_t)rows * cols, 256, 1024), 256, 0, s>>>(M, rows, cols, re,
                                                                            im);
  return hipGetLastError();
}

hipError_t launch_csplit_combine(float* y1, const float* y2, uint64_t npairs, hipStream_t s) {
  if (!npairs) return hipSuccess;
  if ((((uintptr_t)y1) | ((uintptr_t)y2)) % 16 == 0)
    k_csplit_combine<true><<<grid_for(npairs / 2 + 1, 256, 8192), 256, 0, s>>>(y1, y2, npairs);
  else
    k_csplit_combine<false><<<grid_for(npairs, 256, 8192), 256, 0, s>>>(y1, y2, npairs);
  return hipGetLastError();
}

}  // namespace tg
