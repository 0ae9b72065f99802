// Sparse-buffer reduction and the AdamS update at the masked indices.
//
// Reduction: b_bar[r] = (((b0 + b1) + ...) + b_{K-1}) * fp32(1/K), the
// in-HBM stand-in for the sparse reduce-scatter of the single synchronised
// buffer (technical summary §2).
// AdamS (SCAPE paper §II-C eq. (2), with bias correction): the second
// moment is rebuilt from m_{t-1} and the synchronised buffer alone.
// Every float operation below is rounded on its own: contraction is off for
// this file, and sqrtf and '/' are the correctly rounded forms.
#include "scape_internal.h"

#pragma clang fp contract(off)

namespace scape {
namespace {

struct AdamsK {
  float b1, b2, c1, c2, ibc1, ibc2, eps, wd, lr;
  int64_t n;
};

__device__ __forceinline__ void adams_one(int64_t j, float x, float* __restrict__ w,
                                          float* __restrict__ m, float* __restrict__ v,
                                          const AdamsK& c) {
  if (j >= c.n) return;  // an index list from a malformed mask stays in bounds
  const float mo = m[j];
  const float wo = w[j];
  const float mn = (c.b1 * mo) + (c.c1 * x);
  const float vn = (c.b2 * (mo * mo)) + (c.c2 * (x * x));
  const float mh = mn * c.ibc1;
  const float vh = vn * c.ibc2;
  const float d = sqrtf(vh) + c.eps;
  const float u = mh / d;
  const float wn = wo - (c.lr * (u + (c.wd * wo)));
  m[j] = mn;
  if (v) v[j] = vn;  // optional: AdamS never reads v back
  w[j] = wn;
}

__device__ __forceinline__ float worker_mean(const float* __restrict__ b, int K, int64_t pk,
                                             int64_t r, float invK) {
  float s = b[r];
  for (int i = 1; i < K; ++i) s = s + b[(int64_t)i * pk + r];
  return s * invK;
}

__global__ void __launch_bounds__(kThreads)
reduce_kernel(const float* __restrict__ b, int K, int64_t pk, float invK, float* __restrict__ bbar) {
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < pk; r += (int64_t)gridDim.x * kThreads)
    bbar[r] = worker_mean(b, K, pk, r, invK);
}

__global__ void __launch_bounds__(kThreads)
adams_kernel(const float* __restrict__ bbar, const uint32_t* __restrict__ idx, int64_t pk,
             float* __restrict__ w, float* __restrict__ m, float* __restrict__ v, AdamsK c) {
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < pk; r += (int64_t)gridDim.x * kThreads)
    adams_one(idx[r], bbar[r], w, m, v, c);
}

// Dense AdamS on the worker mean (the baseline the SCAPE step is compared
// with): one streaming pass, x = ((g0 + g1) + ...) * fp32(1/K), AdamS at
// every element, non-temporal.  With K = 2, 4 or 8 a thread takes kDenseU
// vectors of 4 elements per stream per iteration and issues every load of
// the iteration before the first is used (four vectors measured 10% faster
// than one at K = 4); other K take one vector, the rows one after another.
typedef float v4f __attribute__((ext_vector_type(4)));

// Vectors of 4 elements per stream a thread takes per iteration of the
// dense kernel, and its blocks.
constexpr int kDenseU = 4;
constexpr int64_t kDenseBlocks = 8192;

// VEC: 16-byte aligned, n % 4 == 0.  KT > 0: K == KT, every gradient row's
// vector (and m's and w's) loaded before any is used, then added in row
// order as below; KT == 0: any K, one row after another.
template <bool VEC, int KT>
__global__ void __launch_bounds__(kThreads)
dense_adams_kernel(const float* __restrict__ g, int K, int64_t n, float invK, float* __restrict__ w,
                   float* __restrict__ m, float* __restrict__ v, AdamsK c) {
  auto update = [&](const float (&x)[4], const float (&mo)[4], const float (&wo)[4], float (&mn)[4], float (&vn)[4],
                    float (&wn)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mn[q] = (c.b1 * mo[q]) + (c.c1 * x[q]);
      vn[q] = (c.b2 * (mo[q] * mo[q])) + (c.c2 * (x[q] * x[q]));
      const float mh = mn[q] * c.ibc1;
      const float vh = vn[q] * c.ibc2;
      const float d = sqrtf(vh) + c.eps;
      const float u = mh / d;
      wn[q] = wo[q] - (c.lr * (u + (c.wd * wo[q])));
    }
  };
  if constexpr (VEC && KT > 0) {
    constexpr int U = kDenseU;
    const int64_t stride = (int64_t)gridDim.x * kThreads * 4 * U;
    for (int64_t b0 = ((int64_t)blockIdx.x * U * kThreads + threadIdx.x) * 4; b0 < n; b0 += stride) {
      v4f gv[U][KT], mv[U], wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j0 = b0 + (int64_t)u * kThreads * 4;
        if (j0 < n) {
#pragma unroll
          for (int i = 0; i < KT; ++i)
            gv[u][i] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(g + (int64_t)i * n + j0));
          mv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(m + j0));
          wv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(w + j0));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j0 = b0 + (int64_t)u * kThreads * 4;
        if (j0 >= n) break;
        v4f s = gv[u][0];
#pragma unroll
        for (int i = 1; i < KT; ++i) s = s + gv[u][i];
        float x[4], mo[4], wo[4], mn[4], vn[4], wn[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[q] = s[q] * invK;
          mo[q] = mv[u][q];
          wo[q] = wv[u][q];
        }
        update(x, mo, wo, mn, vn, wn);
        __builtin_nontemporal_store((v4f){mn[0], mn[1], mn[2], mn[3]}, reinterpret_cast<v4f*>(m + j0));
        if (v) __builtin_nontemporal_store((v4f){vn[0], vn[1], vn[2], vn[3]}, reinterpret_cast<v4f*>(v + j0));
        __builtin_nontemporal_store((v4f){wn[0], wn[1], wn[2], wn[3]}, reinterpret_cast<v4f*>(w + j0));
      }
    }
    return;
  }
  const int64_t stride = (int64_t)gridDim.x * kThreads * 4;
  for (int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4; j0 < n; j0 += stride) {
    float x[4], mo[4], wo[4];
    if (VEC) {
      v4f s = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(g + j0));
      for (int i = 1; i < K; ++i) s = s + __builtin_nontemporal_load(reinterpret_cast<const v4f*>(g + (int64_t)i * n + j0));
      const v4f mv = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(m + j0));
      const v4f wv = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(w + j0));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] = s[q] * invK;
        mo[q] = mv[q];
        wo[q] = wv[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = j0 + q;
        if (j >= n) break;
        float s = g[j];
        for (int i = 1; i < K; ++i) s = s + g[(int64_t)i * n + j];
        x[q] = s * invK;
        mo[q] = m[j];
        wo[q] = w[j];
      }
    }
    float mn[4], vn[4], wn[4];
    update(x, mo, wo, mn, vn, wn);
    if (VEC) {
      __builtin_nontemporal_store((v4f){mn[0], mn[1], mn[2], mn[3]}, reinterpret_cast<v4f*>(m + j0));
      if (v) __builtin_nontemporal_store((v4f){vn[0], vn[1], vn[2], vn[3]}, reinterpret_cast<v4f*>(v + j0));
      __builtin_nontemporal_store((v4f){wn[0], wn[1], wn[2], wn[3]}, reinterpret_cast<v4f*>(w + j0));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = j0 + q;
        if (j >= n) break;
        m[j] = mn[q];
        if (v) v[j] = vn[q];
        w[j] = wn[q];
      }
    }
  }
}

unsigned grid_for(int64_t count) {
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

// One step of the bias-correction state ([P] §II-C, the remark after
// eq. (2)): beta^t as binary64 products, each step one more multiplication
// by binary64(beta) in the order the host takes them, then the fp32
// reciprocals of 1 - beta^t.  One thread.
__global__ void bias_step_kernel(scape_bias_state* __restrict__ st, float b1, float b2) {
  if (threadIdx.x != 0) return;
  const double p1 = st->beta1_pow * (double)b1;
  const double p2 = st->beta2_pow * (double)b2;
  st->beta1_pow = p1;
  st->beta2_pow = p2;
  st->ibc1 = (float)(1.0 / (1.0 - p1));
  st->ibc2 = (float)(1.0 / (1.0 - p2));
}

}  // namespace

hipError_t launch_reduce(const Geom& g, const float* b, float* bbar, hipStream_t s) {
  const int64_t pk = (int64_t)g.P * g.k;
  const float invK = (float)(1.0 / (double)g.K);
  reduce_kernel<<<grid_for(pk), kThreads, 0, s>>>(b, g.K, pk, invK, bbar);
  return hipGetLastError();
}

hipError_t launch_adams(const Geom& g, const float* bbar, const uint32_t* idx, float* w, float* m,
                        float* v, float b1, float b2, float c1, float c2, float ibc1, float ibc2,
                        float eps, float wd, float lr, hipStream_t s, int64_t count) {
  const int64_t pk = count < 0 ? (int64_t)g.P * g.k : count;
  if (pk < 1) return hipSuccess;
  AdamsK c{b1, b2, c1, c2, ibc1, ibc2, eps, wd, lr, g.n};
  adams_kernel<<<grid_for(pk), kThreads, 0, s>>>(bbar, idx, pk, w, m, v, c);
  return hipGetLastError();
}

hipError_t launch_bias_step(scape_bias_state* st, float b1, float b2, hipStream_t s) {
  bias_step_kernel<<<1, 64, 0, s>>>(st, b1, b2);
  return hipGetLastError();
}

hipError_t launch_dense_adams(const Geom& g, const float* grads, float* w, float* m, float* v, float b1,
                              float b2, float c1, float c2, float ibc1, float ibc2, float eps, float wd,
                              float lr, bool vec, hipStream_t s) {
  const float invK = (float)(1.0 / (double)g.K);
  AdamsK c{b1, b2, c1, c2, ibc1, ibc2, eps, wd, lr, g.n};
  int64_t blocks = (g.n / 4 + kThreads - 1) / kThreads;
  if (blocks > kDenseBlocks) blocks = kDenseBlocks;
  if (blocks < 1) blocks = 1;
  const unsigned nb = (unsigned)blocks;
  if (!vec)
    dense_adams_kernel<false, 0><<<nb, kThreads, 0, s>>>(grads, g.K, g.n, invK, w, m, v, c);
  else if (g.K == 2)
    dense_adams_kernel<true, 2><<<nb, kThreads, 0, s>>>(grads, g.K, g.n, invK, w, m, v, c);
  else if (g.K == 4)
    dense_adams_kernel<true, 4><<<nb, kThreads, 0, s>>>(grads, g.K, g.n, invK, w, m, v, c);
  else if (g.K == 8)
    dense_adams_kernel<true, 8><<<nb, kThreads, 0, s>>>(grads, g.K, g.n, invK, w, m, v, c);
  else
    dense_adams_kernel<true, 0><<<nb, kThreads, 0, s>>>(grads, g.K, g.n, invK, w, m, v, c);
  return hipGetLastError();
}

}  // namespace scape
