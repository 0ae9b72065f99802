// Streaming passes over the flat buffer: the error-feedback compression of
// every worker's gradient at the current mask (SCAPE paper §II-B, at the
// shared index set of the technical summary §2), fused with the owner's
// first-moment statistic and the level-1 histogram of its keys; and the
// statistic-only passes used by the mask call and the step-1 bootstrap.
//
// Work decomposition: grid (G, P).  Block (b, p) walks tiles b, b+G, ... of
// partition p; a tile is 4096 elements = 64 mask words; thread `tid` owns
// the 4 consecutive elements 4*tid .. 4*tid+3 of each 1024-element chunk, so
// every global access is a 16-byte-per-lane coalesced load or store when the
// layout allows vector access (n_p % 4 == 0 and 16-byte aligned bases).
#include "scape_internal.h"

#pragma clang fp contract(off)

namespace scape {
namespace {

__device__ __forceinline__ uint32_t stat_key(float m, float a, float b1, float c1) {
  // s = (b1*m) + (c1*a), each operation rounded on its own; key = |s| bits.
  const float s = (b1 * m) + (c1 * a);
  return __float_as_uint(s) & 0x7fffffffu;
}

__device__ __forceinline__ void load4(const float* p, int64_t lj, int64_t n_p, bool vec, float out[4]) {
  if (vec) {
    const float4 v = *reinterpret_cast<const float4*>(p + lj);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = (lj + q < n_p) ? p[lj + q] : 0.0f;
  }
}

__device__ __forceinline__ void store4(float* p, int64_t lj, int64_t n_p, bool vec, const float v[4]) {
  if (vec) {
    *reinterpret_cast<float4*>(p + lj) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lj + q < n_p) p[lj + q] = v[q];
  }
}

__device__ __forceinline__ void store4u(uint32_t* p, int64_t lj, int64_t n_p, bool vec, const uint32_t v[4]) {
  if (vec) {
    *reinterpret_cast<uint4*>(p + lj) = make_uint4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lj + q < n_p) p[lj + q] = v[q];
  }
}

__device__ __forceinline__ void hist_zero(uint32_t* sh) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) sh[i] = 0;
}

__device__ __forceinline__ void hist_merge(const uint32_t* sh, uint32_t* gh) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// MODE 0: key from stat[].  MODE 1: key from b1*m + c1*(g^o + e^o).
template <int MODE, bool VEC>
__global__ void __launch_bounds__(kThreads)
keys_kernel(Geom g, const float* __restrict__ stat, const float* __restrict__ m,
            const float* __restrict__ grads, const float* __restrict__ e, float b1, float c1,
            uint32_t* __restrict__ keys, uint32_t* __restrict__ hist) {
  __shared__ uint32_t sh[kBins];
  hist_zero(sh);
  __syncthreads();
  const int p = blockIdx.y;
  const int64_t pbase = (int64_t)p * g.n_p;
  const int o = (int)(((int64_t)p * g.K) / g.P);
  const float* gp = grads + (int64_t)o * g.n + pbase;
  const float* ep = e + (int64_t)o * g.n + pbase;
  for (int64_t t = blockIdx.x; t < g.tpp; t += gridDim.x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t lj = t * kTile + c * 1024 + 4 * threadIdx.x;
      if (lj >= g.n_p) break;
      uint32_t kk[4];
      if (MODE == 0) {
        float s[4];
        load4(stat + pbase, lj, g.n_p, VEC, s);
#pragma unroll
        for (int q = 0; q < 4; ++q) kk[q] = __float_as_uint(s[q]) & 0x7fffffffu;
      } else {
        float mm[4], gg[4], ee[4];
        load4(m + pbase, lj, g.n_p, VEC, mm);
        load4(gp, lj, g.n_p, VEC, gg);
        load4(ep, lj, g.n_p, VEC, ee);
#pragma unroll
        for (int q = 0; q < 4; ++q) kk[q] = stat_key(mm[q], gg[q] + ee[q], b1, c1);
      }
      store4u(keys + pbase, lj, g.n_p, VEC, kk);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (VEC || lj + q < g.n_p) atomicAdd(&sh[kk[q] >> kL1Shift], 1u);
    }
  }
  __syncthreads();
  hist_merge(sh, hist + (int64_t)p * kBins);
}

// Loads the tile's 64 mask words into LDS with their exclusive popcount
// prefix (one wave scans).
__device__ __forceinline__ void load_tile_words(const uint64_t* __restrict__ bits, int64_t wbase,
                                                int64_t wpp, int64_t t, uint64_t* sw, uint32_t* spre) {
  if (threadIdx.x < kWordsPerTile) {
    const int64_t w = t * kWordsPerTile + threadIdx.x;
    const uint64_t word = (w < wpp) ? bits[wbase + w] : 0ull;
    sw[threadIdx.x] = word;
    uint32_t c = (uint32_t)__popcll(word);
    // inclusive scan across the 64 lanes of wave 0
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(c, d, 64);
      if ((int)threadIdx.x >= d) c += y;
    }
    spre[threadIdx.x] = c - (uint32_t)__popcll(word);
  }
}

template <bool STAT, bool VEC>
__global__ void __launch_bounds__(kThreads)
compress_kernel(Geom g, const float* __restrict__ grads, float* __restrict__ e,
                const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                float* __restrict__ b, const float* __restrict__ m, float b1, float c1,
                uint32_t* __restrict__ keys, uint32_t* __restrict__ hist) {
  __shared__ uint64_t sw[kWordsPerTile];
  __shared__ uint32_t spre[kWordsPerTile];
  __shared__ uint32_t sh[STAT ? kBins : 1];
  if (STAT) hist_zero(sh);
  const int p = blockIdx.y;
  const int64_t pbase = (int64_t)p * g.n_p;
  const int64_t wbase = (int64_t)p * g.wpp;
  const int64_t pk = (int64_t)g.P * g.k;
  const int owner = (int)(((int64_t)p * g.K) / g.P);
  const int lane16 = threadIdx.x & 15;
  const int sh4 = 4 * lane16;
  const uint64_t below = (sh4 == 0) ? 0ull : ((1ull << sh4) - 1ull);

  for (int64_t t = blockIdx.x; t < g.tpp; t += gridDim.x) {
    __syncthreads();  // previous tile's words no longer in use
    load_tile_words(bits, wbase, g.wpp, t, sw, spre);
    __syncthreads();
    const int64_t rbase = (int64_t)p * g.k + tile_off[(int64_t)p * g.tpp + t];
    const int64_t rend = (int64_t)(p + 1) * g.k;

    // Per chunk: the lane's 4 mask bits and the rank of its first element.
    uint32_t nib[4];
    int64_t rank0[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = c * 16 + (threadIdx.x >> 4);
      const uint64_t word = sw[q];
      nib[c] = (uint32_t)(word >> sh4) & 0xfu;
      rank0[c] = rbase + spre[q] + (uint32_t)__popcll(word & below);
    }

    for (int i = 0; i < g.K; ++i) {
      const float* gi = grads + (int64_t)i * g.n + pbase;
      float* ei = e + (int64_t)i * g.n + pbase;
      float* bi = b + (int64_t)i * pk;
      float ga[4][4], ea[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t lj = t * kTile + c * 1024 + 4 * threadIdx.x;
        if (lj < g.n_p) {
          load4(gi, lj, g.n_p, VEC, ga[c]);
          load4(ei, lj, g.n_p, VEC, ea[c]);
        }
      }
      const bool own = STAT && (i == owner);
      float ma[4][4];
      if (own) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t lj = t * kTile + c * 1024 + 4 * threadIdx.x;
          if (lj < g.n_p) load4(m + pbase, lj, g.n_p, VEC, ma[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t lj = t * kTile + c * 1024 + 4 * threadIdx.x;
        if (lj >= g.n_p) continue;
        float a[4], eo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[q] = ga[c][q] + ea[c][q];
          eo[q] = ((nib[c] >> q) & 1u) ? 0.0f : a[q];
        }
        store4(ei, lj, g.n_p, VEC, eo);
        if (nib[c]) {
          // ranks stay inside partition p's k entries for any mask with k
          // bits per partition; the bound keeps a malformed mask in bounds
          int64_t r = rank0[c];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((nib[c] >> q) & 1u) {
              if (r < rend) bi[r] = a[q];
              ++r;
            }
        }
        if (own) {
          uint32_t kk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) kk[q] = stat_key(ma[c][q], a[q], b1, c1);
          store4u(keys + pbase, lj, g.n_p, VEC, kk);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (VEC || lj + q < g.n_p) atomicAdd(&sh[kk[q] >> kL1Shift], 1u);
        }
      }
    }
  }
  if (STAT) {
    __syncthreads();
    hist_merge(sh, hist + (int64_t)p * kBins);
  }
}

}  // namespace

hipError_t launch_keys_from_stat(const Geom& g, const float* stat, uint32_t* keys, uint32_t* hist,
                                 bool vec, hipStream_t s) {
  dim3 grid(g.G, g.P);
  if (vec)
    keys_kernel<0, true><<<grid, kThreads, 0, s>>>(g, stat, nullptr, nullptr, nullptr, 0.f, 0.f, keys, hist);
  else
    keys_kernel<0, false><<<grid, kThreads, 0, s>>>(g, stat, nullptr, nullptr, nullptr, 0.f, 0.f, keys, hist);
  return hipGetLastError();
}

hipError_t launch_keys_from_state(const Geom& g, const float* m, const float* grads, const float* e,
                                  float b1, float c1, uint32_t* keys, uint32_t* hist, bool vec,
                                  hipStream_t s) {
  dim3 grid(g.G, g.P);
  if (vec)
    keys_kernel<1, true><<<grid, kThreads, 0, s>>>(g, nullptr, m, grads, e, b1, c1, keys, hist);
  else
    keys_kernel<1, false><<<grid, kThreads, 0, s>>>(g, nullptr, m, grads, e, b1, c1, keys, hist);
  return hipGetLastError();
}

hipError_t launch_compress(const Geom& g, const float* grads, float* e, const uint64_t* bits,
                           const uint32_t* tile_off, float* b, bool stat, const float* m, float b1,
                           float c1, uint32_t* keys, uint32_t* hist, bool vec, hipStream_t s) {
  dim3 grid(g.G, g.P);
  if (stat) {
    if (vec)
      compress_kernel<true, true><<<grid, kThreads, 0, s>>>(g, grads, e, bits, tile_off, b, m, b1, c1, keys, hist);
    else
      compress_kernel<true, false><<<grid, kThreads, 0, s>>>(g, grads, e, bits, tile_off, b, m, b1, c1, keys, hist);
  } else {
    if (vec)
      compress_kernel<false, true><<<grid, kThreads, 0, s>>>(g, grads, e, bits, tile_off, b, nullptr, 0.f, 0.f, nullptr, nullptr);
    else
      compress_kernel<false, false><<<grid, kThreads, 0, s>>>(g, grads, e, bits, tile_off, b, nullptr, 0.f, 0.f, nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace scape
