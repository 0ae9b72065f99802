// Exact partitioned top-k (technical summary §2, partitioned mask
// synchronisation; ties to the lower index) and the packed forms of the mask
// (single-bit words, ascending index list, per-tile offsets).
//
// Method: radix select on the unique 64-bit composite
//     c = (key << 32) | (idx_mask - local_index)
// so that "the k largest composites" is exactly "the k largest keys, ties to
// the lower index".  Level 1 (key bits 30..19) is histogrammed by the
// streaming pass that produces the keys.  The select pass then reads every
// key once: keys above the level-1 threshold digit are selected outright and
// written as mask words (one ballot per 64 elements), keys equal to it are
// compacted as composites into per-block candidate segments (no global
// atomics).  The remaining levels (key bits 18..7, 6..0, then the index
// bits) run on the candidates only; the last step sets the candidates'
// bits.  Emission turns the words into the ascending index list.
#include "scape_internal.h"

namespace scape {
namespace {

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive scan over a block of kThreads (4 waves); `wtot` is LDS [4].
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t* total) {
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if ((int)lane >= d) x += y;
  }
  __syncthreads();
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < (int)wave) off += wtot[w];
    tot += wtot[w];
  }
  *total = tot;
  return off + x - v;
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// One level of the threshold search for partition blockIdx.x: find the
// digit d (scanning from the largest) whose bin holds the r-th largest
// composite among those matching the current prefix; narrow the prefix.
// Level 1 starts from r = k and an empty prefix.  Leaves the bins zeroed.
__global__ void __launch_bounds__(kThreads)
level_scan_kernel(Geom g, uint32_t* __restrict__ hist, PartSel* __restrict__ state, int shift,
                  int nbits, int first) {
  __shared__ uint32_t wtot[kThreads / 64];
  __shared__ int found;
  const int p = blockIdx.x;
  uint32_t* h = hist + (int64_t)p * kBins;
  const int nb = 1 << nbits;
  PartSel st;
  if (first) {
    st.prefix = 0; st.mask = 0; st.r = (uint32_t)g.k; st.done = 0; st.bin1 = 0; st.fault = 0;
  } else {
    st = state[p];
  }
  if (!st.done) {
    const int per = (nb + kThreads - 1) / kThreads;
    // thread t owns descending positions [t*per, (t+1)*per): bin = nb-1-pos
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) {
      const int pos = threadIdx.x * per + q;
      if (pos < nb) s += h[nb - 1 - pos];
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0) found = 0;
    __syncthreads();
    if (above < st.r && st.r <= above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int pos = threadIdx.x * per + q;
        if (pos >= nb) break;
        const int d = nb - 1 - pos;
        const uint32_t c = h[d];
        if (acc + c >= st.r) {
          PartSel o = st;
          o.r = st.r - acc;
          o.prefix = st.prefix | ((uint64_t)d << shift);
          uint64_t dm = ((1ull << nbits) - 1ull) << shift;
          if (first) dm |= (1ull << 63);  // bit 63 of every composite is zero
          o.mask = st.mask | dm;
          o.done = (c == o.r) ? 1u : 0u;
          if (first) o.bin1 = (uint32_t)d;
          state[p] = o;
          found = 1;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && !found) {
      st.fault = 1;
      st.done = 1;
      state[p] = st;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0u;
}

// Reads every key of the partition once.  Words of definite selections are
// written whole; threshold-digit keys go to the block's candidate segment.
__global__ void __launch_bounds__(kThreads)
select_pass_kernel(Geom g, const uint32_t* __restrict__ keys, const PartSel* __restrict__ state,
                   uint64_t* __restrict__ bits, uint64_t* __restrict__ cand,
                   uint32_t* __restrict__ segcnt) {
  __shared__ uint32_t fill;
  const int p = blockIdx.y;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) fill = 0;
  __syncthreads();
  const PartSel st = state[p];
  const uint32_t B1 = st.bin1;
  const bool done = st.done != 0;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t pbase = (int64_t)p * g.n_p;
  uint64_t* seg = cand + ((int64_t)p * g.G + b) * g.seg_cap;

  for (int64_t t = b; t < g.tpp; t += g.G) {
    const int64_t w0 = t * kWordsPerTile + 16 * wave;
    uint32_t kv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t j = (w0 + q) * 64 + lane;
      kv[q] = (j < g.n_p) ? keys[pbase + j] : 0u;
    }
    uint64_t myword = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t j = (w0 + q) * 64 + lane;
      const bool valid = j < g.n_p;
      const uint32_t bin = kv[q] >> kL1Shift;
      const bool def = valid && (bin > B1 || (done && bin == B1));
      const bool cnd = valid && !done && bin == B1;
      const uint64_t wb = __ballot(def);
      if (lane == (uint32_t)q) myword = wb;
      const uint64_t cb = __ballot(cnd);
      if (cb) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&fill, (uint32_t)__popcll(cb));
        base = __shfl(base, 0, 64);
        if (cnd) {
          const uint64_t c = ((uint64_t)kv[q] << 32) | (uint64_t)(g.idx_mask - (uint32_t)j);
          seg[base + mbcnt(cb)] = c;
        }
      }
    }
    if (lane < 16) {
      const int64_t w = w0 + lane;
      if (w < g.wpp) bits[(int64_t)p * g.wpp + w] = myword;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) segcnt[(int64_t)p * g.G + b] = fill;
}

// Histogram of one digit over the candidates that match the prefix.
__global__ void __launch_bounds__(kThreads)
cand_hist_kernel(Geom g, const uint64_t* __restrict__ cand, const uint32_t* __restrict__ segcnt,
                 const PartSel* __restrict__ state, uint32_t* __restrict__ hist, int shift,
                 int nbits) {
  __shared__ uint32_t sh[kBins];
  const int p = blockIdx.y;
  const PartSel st = state[p];
  if (st.done) return;
  const int nb = 1 << nbits;
  for (int i = threadIdx.x; i < nb; i += kThreads) sh[i] = 0;
  __syncthreads();
  for (int s = blockIdx.x; s < g.G; s += gridDim.x) {
    const uint32_t cnt = segcnt[(int64_t)p * g.G + s];
    const uint64_t* seg = cand + ((int64_t)p * g.G + s) * g.seg_cap;
    for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) {
      const uint64_t c = seg[i];
      if ((c & st.mask) == st.prefix) atomicAdd(&sh[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* h = hist + (int64_t)p * kBins;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(h + i, c);
  }
}

// Sets the bits of the candidates at or above the threshold composite.
__global__ void __launch_bounds__(kThreads)
mark_kernel(Geom g, const uint64_t* __restrict__ cand, const uint32_t* __restrict__ segcnt,
            const PartSel* __restrict__ state, uint64_t* __restrict__ bits) {
  const int p = blockIdx.y;
  const uint64_t T = state[p].prefix;
  uint64_t* wb = bits + (int64_t)p * g.wpp;
  for (int s = blockIdx.x; s < g.G; s += gridDim.x) {
    const uint32_t cnt = segcnt[(int64_t)p * g.G + s];
    const uint64_t* seg = cand + ((int64_t)p * g.G + s) * g.seg_cap;
    for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) {
      const uint64_t c = seg[i];
      if (c >= T) {
        const uint32_t j = g.idx_mask - (uint32_t)c;
        atomicOr(reinterpret_cast<unsigned long long*>(wb + (j >> 6)), 1ull << (j & 63));
      }
    }
  }
}

// One wave per tile: number of selected elements in the tile.
__global__ void __launch_bounds__(kThreads)
tile_count_kernel(Geom g, const uint64_t* __restrict__ bits, uint32_t* __restrict__ tilecnt) {
  const int p = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= g.tpp) return;
  const uint32_t lane = lane_id();
  const int64_t w = t * kWordsPerTile + lane;
  uint32_t c = (w < g.wpp) ? (uint32_t)__popcll(bits[(int64_t)p * g.wpp + w]) : 0u;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
  if (lane == 0) tilecnt[(int64_t)p * g.tpp + t] = c;
}

// Exclusive scan of the tile counts of partition blockIdx.x -> tile_off.
__global__ void __launch_bounds__(kThreads)
scan_tiles_kernel(Geom g, const uint32_t* __restrict__ tilecnt, uint32_t* __restrict__ tile_off,
                  PartSel* __restrict__ state) {
  __shared__ uint32_t wtot[kThreads / 64];
  const int p = blockIdx.x;
  const int64_t per = (g.tpp + kThreads - 1) / kThreads;
  const int64_t lo = threadIdx.x * per;
  const int64_t hi = (lo + per < g.tpp) ? lo + per : g.tpp;
  const uint32_t* tc = tilecnt + (int64_t)p * g.tpp;
  uint32_t s = 0;
  for (int64_t t = lo; t < hi; ++t) s += tc[t];
  uint32_t tot;
  uint32_t run = block_excl_scan(s, wtot, &tot);
  uint32_t* to = tile_off + (int64_t)p * g.tpp;
  for (int64_t t = lo; t < hi; ++t) {
    to[t] = run;
    run += tc[t];
  }
  if (threadIdx.x == 0 && tot != (uint32_t)g.k) state[p].fault |= 2u;
}

// One wave per tile: write the tile's selected global indices in order.
__global__ void __launch_bounds__(kThreads)
write_idx_kernel(Geom g, const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                 uint32_t* __restrict__ idx) {
  const int p = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= g.tpp) return;
  const uint32_t lane = lane_id();
  const int64_t w = t * kWordsPerTile + lane;
  uint64_t word = (w < g.wpp) ? bits[(int64_t)p * g.wpp + w] : 0ull;
  const uint32_t c = (uint32_t)__popcll(word);
  uint32_t x = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if ((int)lane >= d) x += y;
  }
  int64_t pos = (int64_t)tile_off[(int64_t)p * g.tpp + t] + (x - c);
  uint32_t* out = idx + (int64_t)p * g.k;
  const uint32_t jbase = (uint32_t)((int64_t)p * g.n_p + w * 64);
  while (word) {
    if (pos < g.k) out[pos] = jbase + (uint32_t)__builtin_ctzll(word);  // bound: malformed mask
    ++pos;
    word &= word - 1ull;
  }
}

__global__ void __launch_bounds__(kThreads)
overlap_kernel(const uint64_t* __restrict__ a, const uint64_t* __restrict__ b, int64_t nwords,
               unsigned long long* __restrict__ out) {
  uint64_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * kThreads)
    acc += (uint64_t)__popcll(a[i] & b[i]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane_id() == 0 && acc) atomicAdd(out, (unsigned long long)acc);
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  zero_u32_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(p, count);
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const uint32_t* keys, uint32_t* hist, uint32_t* segcnt,
                         uint64_t* cand, PartSel* state, uint32_t* tilecnt, uint64_t* bits,
                         uint32_t* idx, uint32_t* tile_off, hipStream_t s,
                         void (*mark)(void*, int), void* ctx) {
  level_scan_kernel<<<g.P, kThreads, 0, s>>>(g, hist, state, 32 + kL1Shift, kDigitBits, 1);
  select_pass_kernel<<<dim3(g.G, g.P), kThreads, 0, s>>>(g, keys, state, bits, cand, segcnt);
  if (mark) mark(ctx, 1);
  for (int l = 0; l < g.nlevels; ++l) {
    cand_hist_kernel<<<dim3(g.R, g.P), kThreads, 0, s>>>(g, cand, segcnt, state, hist,
                                                         g.levels[l].shift, g.levels[l].nbits);
    level_scan_kernel<<<g.P, kThreads, 0, s>>>(g, hist, state, g.levels[l].shift, g.levels[l].nbits, 0);
  }
  mark_kernel<<<dim3(g.R, g.P), kThreads, 0, s>>>(g, cand, segcnt, state, bits);
  if (mark) mark(ctx, 2);
  const unsigned tblocks = (unsigned)((g.tpp + 3) / 4);
  tile_count_kernel<<<dim3(tblocks, g.P), kThreads, 0, s>>>(g, bits, tilecnt);
  scan_tiles_kernel<<<g.P, kThreads, 0, s>>>(g, tilecnt, tile_off, state);
  write_idx_kernel<<<dim3(tblocks, g.P), kThreads, 0, s>>>(g, bits, tile_off, idx);
  return hipGetLastError();
}

hipError_t launch_overlap(const Geom& g, const uint64_t* a, const uint64_t* b, uint64_t* out,
                          hipStream_t s) {
  zero_u64_kernel<<<1, 1, 0, s>>>(reinterpret_cast<unsigned long long*>(out));
  const int64_t nwords = (int64_t)g.P * g.wpp;
  int64_t blocks = (nwords + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  overlap_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(a, b, nwords, reinterpret_cast<unsigned long long*>(out));
  return hipGetLastError();
}

}  // namespace scape
