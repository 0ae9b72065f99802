// Exact partitioned top-k (technical summary §2, partitioned mask
// synchronisation; ties to the lower index) and the packed forms of the mask
// (single-bit words, ascending index list, per-tile offsets).
//
// Method: radix select on the unique 64-bit composite
//     c = (key << 32) | (idx_mask - local_index)
// so that "the k largest composites" is exactly "the k largest keys, ties to
// the lower index".  The streaming pass that produces the keys captures,
// per tile, every key at or above a bound `lo` together with a level-1
// histogram (key bits 30..19) of the captured keys.  If a partition captured
// at least k keys, its top k lie among the captures; otherwise an exact
// fallback recounts all its keys to find the level-1 digit and recaptures
// from there.  A first capture, with no previous bound, takes its bound
// from a histogram of a sample of tiles (kScanSample).  The candidate select pass then reads only the captures:
// digits above the threshold digit are selected and written as whole mask
// words, the threshold digit's captures are compacted in place and
// histogrammed on the next digit.  The remaining levels (key bits 6..0, then
// the index bits) run on those few; marking sets their bits; emission turns
// the words into the ascending index list and per-tile offsets.
#include "scape_internal.h"

namespace scape {
namespace {

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

// Chunks of 64 candidates a wave loads per round when it walks a slot.
constexpr int kCandChunks = 4;

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

__device__ __forceinline__ PartSel fresh_sel(uint32_t k) {
  PartSel s;
  s.prefix = 0; s.mask = 0; s.r = k; s.done = 0; s.bin1 = 0; s.fault = 0; s.fb = 0; s.lo_fb = 0;
  s.kth = 0xffffffffu; s.c1 = 0; s.lo_next = 0; s.pad = 0;
  return s;
}

// Block-wide minimum folded into *dst with one atomic per block.
__device__ __forceinline__ void block_min_into(uint32_t v, uint32_t* smin, uint32_t* dst) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t y = __shfl_xor(v, d, 64);
    v = y < v ? y : v;
  }
  if ((threadIdx.x & 63) == 0) atomicMin(smin, v);
  __syncthreads();
  if (threadIdx.x == 0 && *smin != 0xffffffffu) atomicMin(dst, *smin);
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void init_state_kernel(PartSel* state, int P, uint32_t k) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p < P) {
    PartSel s = fresh_sel(k);
    s.fb = 1;
    state[p] = s;
  }
}

// One level of the threshold search for partition blockIdx.x: find the
// digit d (scanning from the largest) whose bin holds the r-th largest
// composite among those matching the current prefix, and narrow the prefix.
// Level-1 modes start from r = k and an empty prefix (see kScan*).  Always
// leaves the partition's bins zeroed.
__global__ void __launch_bounds__(kThreads)
level_scan_kernel(Geom g, uint32_t* __restrict__ hist, PartSel* __restrict__ state, int shift,
                  int nbits, int mode, uint32_t target) {
  __shared__ uint32_t wtot[kThreads / 64];
  __shared__ int found;
  __shared__ uint32_t s_lo;
  __shared__ int s_dmin;
  const int p = blockIdx.x;
  uint32_t* h = hist + (int64_t)p * kBins;
  const int nb = 1 << nbits;
  const PartSel cur = state[p];
  bool active;
  if (mode == kScanCheck) active = true;
  else if (mode == kScanLevel) active = !cur.done && !cur.fb;
  else active = cur.fb != 0;  // kScanBound, kScanFinal, kScanSample
  const bool first = mode != kScanLevel;
  const PartSel st = first ? fresh_sel((uint32_t)g.k) : cur;
  if (active && mode == kScanSample) {
    // The bound for a first capture: the digit at which the count of the
    // sampled keys from the top reaches `target` (scaled to the sample), or
    // 0 (capture every key) if the sample holds fewer.
    const int per = (nb + kThreads - 1) / kThreads;
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) {
      const int pos = threadIdx.x * per + q;
      if (pos < nb) s += h[nb - 1 - pos];
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0 && tot < target) state[p].lo_fb = 0u;
    if (tot >= target && above < target && target <= above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int pos = threadIdx.x * per + q;
        if (pos >= nb) break;
        const int d = nb - 1 - pos;
        acc += h[d];
        if (acc >= target) {
          state[p].lo_fb = (uint32_t)d << kL1Shift;
          break;
        }
      }
    }
  } else if (active) {
    const int per = (nb + kThreads - 1) / kThreads;
    // thread t owns descending positions [t*per, (t+1)*per): bin = nb-1-pos
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) {
      const int pos = threadIdx.x * per + q;
      if (pos < nb) s += h[nb - 1 - pos];
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0) {
      found = 0;
      s_lo = 0xffffffffu;
      s_dmin = nb;
    }
    __syncthreads();
    // Capture bound for the next step: the digit at which the count of keys
    // from the top reaches `need` (level 1: target; level 2: the part of the
    // target that falls inside the threshold bin).
    const bool bound_l1 = (mode == kScanCheck || mode == kScanFinal);
    const bool bound_l2 = (mode == kScanLevel && shift == g.levels[0].shift);
    int64_t need = -1;
    if (bound_l1) need = (tot >= target) ? (int64_t)target : -2;
    if (bound_l2) {
      const int64_t above_bin = (int64_t)g.k - (int64_t)cur.r;  // selected above the threshold bin
      const int64_t in_bin = (int64_t)target - above_bin;
      if (in_bin > 0 && in_bin <= (int64_t)tot) need = in_bin;
    }
    if (need >= 1 && above < (uint64_t)need && (uint64_t)need <= (uint64_t)above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int pos = threadIdx.x * per + q;
        if (pos >= nb) break;
        const int d = nb - 1 - pos;
        acc += h[d];
        if (acc >= (uint32_t)need) {
          s_lo = (uint32_t)(((st.prefix & ~(((1ull << nbits) - 1ull) << shift)) | ((uint64_t)d << shift)) >> 32);
          break;
        }
      }
    }
    if (bound_l1 && need == -2) {
      // fewer keys than the target were captured: one bin below the lowest
      // captured digit
      for (int q = per - 1; q >= 0; --q) {
        const int pos = threadIdx.x * per + q;
        if (pos < nb && h[nb - 1 - pos]) {
          atomicMin(&s_dmin, nb - 1 - pos);
          break;
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) s_lo = (uint32_t)(s_dmin >= 1 && s_dmin < nb ? s_dmin - 1 : 0) << kL1Shift;
    }
    __syncthreads();
    if (mode == kScanCheck && tot < st.r) {
      if (threadIdx.x == 0) {
        PartSel o = st;
        o.fb = 1;
        state[p] = o;
        found = 1;
      }
    } else if (above < st.r && st.r <= above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int pos = threadIdx.x * per + q;
        if (pos >= nb) break;
        const int d = nb - 1 - pos;
        const uint32_t c = h[d];
        if (acc + c >= st.r) {
          if (mode == kScanBound) {
            PartSel o = cur;
            o.lo_fb = (uint32_t)d << kL1Shift;
            state[p] = o;
          } else {
            PartSel o = st;
            o.r = st.r - acc;
            o.prefix = st.prefix | ((uint64_t)d << shift);
            uint64_t dm = ((1ull << nbits) - 1ull) << shift;
            if (first) dm |= (1ull << 63);  // bit 63 of every composite is zero
            o.mask = st.mask | dm;
            o.done = (c == o.r) ? 1u : 0u;
            if (first) {
              o.bin1 = (uint32_t)d;
              o.c1 = c;
            }
            o.fb = 0;
            state[p] = o;
          }
          found = 1;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && !found) {
      PartSel o = cur;
      o.fault |= 1u;
      o.done = 1;
      o.fb = 0;
      state[p] = o;
    }
    __syncthreads();
    // record the bound (level 1 sets it; level 2 may raise it inside the bin)
    if (threadIdx.x == 0 && (bound_l1 || bound_l2) && mode != kScanBound) {
      if (bound_l1) state[p].lo_next = (s_lo == 0xffffffffu) ? 0u : s_lo;
      else if (s_lo != 0xffffffffu && s_lo > state[p].lo_next) state[p].lo_next = s_lo;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0u;
}

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Orders this wave's LDS accesses before its next ones.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per tile: reads the tile's captured candidates in rounds of
// kCandChunks chunks of 64; selects the digits above the level-1 threshold
// digit into the tile's 64 mask words (written whole, so every word of the
// partition is written); compacts the threshold digit's candidates in
// place, in order (a write position never passes the candidates already
// read), and histograms their level-2 digit.
__global__ void __launch_bounds__(kThreads)
cand_select_kernel(Geom g, PartSel* __restrict__ state, uint64_t* __restrict__ cand,
                   const uint32_t* __restrict__ cnt1, uint32_t* __restrict__ cnt2,
                   uint32_t* __restrict__ hist, uint64_t* __restrict__ bits,
                   uint32_t* __restrict__ tilecnt) {
  __shared__ unsigned long long words[kThreads / 64][kWordsPerTile];
  __shared__ uint32_t sh[kBins];
  __shared__ uint32_t smin;
  const int p = blockIdx.y;
  const PartSel st = state[p];
  const uint32_t B1 = st.bin1;
  const bool done = st.done != 0;
  const int l2shift = g.levels[0].shift;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  unsigned long long* wd = words[wave];
  uint32_t kmin = 0xffffffffu;  // smallest key selected whole from the threshold digit
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh[i] = 0;
  if (threadIdx.x == 0) smin = 0xffffffffu;
  __syncthreads();
  // The wave takes tiles t0, t0 + nw, ... in batches of up to 64: lane i
  // loads the capture count of the batch's i-th tile, and the first 64
  // captures of the next tile are loaded while a tile is processed, so that
  // a tile costs no dependent global load of its own.
  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t t0 = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  const uint32_t* c1p = cnt1 + (int64_t)p * g.tpp;
  for (int64_t tb = t0; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t cv = (tl < g.tpp) ? c1p[tl] : 0u;
    if (cv > (uint32_t)kTile) cv = (uint32_t)kTile;  // a slot holds at most one tile
    const int64_t left = (g.tpp - tb + nw - 1) / nw;
    const int nb = left < 64 ? (int)left : 64;
    uint64_t cnext = 0ull;
    {
      const uint32_t nn = (uint32_t)__shfl((int)cv, 0, 64);
      const uint64_t* ns = cand + ((int64_t)p * g.tpp + tb) * kTile;
      if (lane < nn) cnext = ns[lane];
    }
    for (int j = 0; j < nb; ++j) {
      const int64_t t = tb + (int64_t)j * nw;
      const uint32_t n1 = (uint32_t)__shfl((int)cv, j, 64);
      const uint64_t c0 = cnext;
      if (j + 1 < nb) {
        const uint32_t nn = (uint32_t)__shfl((int)cv, j + 1, 64);
        const uint64_t* ns = cand + ((int64_t)p * g.tpp + t + nw) * kTile;
        cnext = (lane < nn) ? ns[lane] : 0ull;
      }
      wd[lane] = 0ull;
      wave_lds_sync();
      uint64_t* slot = cand + ((int64_t)p * g.tpp + t) * kTile;
      const uint32_t tile_lo = (uint32_t)(t * kTile);
      uint32_t n2 = 0;
      // rounds of kCandChunks chunks of 64, all loaded before any is used
      for (uint32_t base = 0; base < n1; base += 64 * kCandChunks) {
        uint64_t cc[kCandChunks];
#pragma unroll
        for (int u = 0; u < kCandChunks; ++u) {
          const uint32_t i = base + 64 * u + lane;
          cc[u] = (base == 0 && u == 0) ? c0 : ((i < n1) ? slot[i] : 0ull);
        }
#pragma unroll
        for (int u = 0; u < kCandChunks; ++u) {
          if (base + 64 * u >= n1) break;  // wave-uniform
          const uint64_t c = cc[u];
          const bool valid = base + 64 * u + lane < n1;
          const uint32_t d1 = (uint32_t)(c >> (32 + kL1Shift)) & (kBins - 1);
          const uint32_t jl = g.idx_mask - (uint32_t)c - tile_lo;
          const bool ok = valid && jl < (uint32_t)kTile;  // false only for a corrupted slot
          const bool sel = ok && (d1 > B1 || (done && d1 == B1));
          const bool keep = ok && !done && d1 == B1;
          if (sel) {
            atomicOr(&wd[jl >> 6], 1ull << (jl & 63));
            if (d1 == B1) {
              const uint32_t key = (uint32_t)(c >> 32);
              kmin = key < kmin ? key : kmin;
            }
          }
          // in-place compaction: a write lands at a position already read
          // (n2 never passes the candidates read so far)
          const uint64_t kb = __ballot(keep);
          if (keep) {
            slot[n2 + mbcnt(kb)] = c;
            atomicAdd(&sh[(uint32_t)(c >> l2shift) & (kBins - 1)], 1u);
          }
          n2 += (uint32_t)__popcll(kb);
        }
      }
      wave_lds_sync();
      const int64_t w = t * kWordsPerTile + lane;
      const unsigned long long word = wd[lane];
      if (w < g.wpp) bits[(int64_t)p * g.wpp + w] = word;
      uint32_t pc = (uint32_t)__popcll(word);
#pragma unroll
      for (int dd = 32; dd >= 1; dd >>= 1) pc += __shfl_xor(pc, dd, 64);
      if (lane == 0) {
        cnt2[(int64_t)p * g.tpp + t] = n2;
        tilecnt[(int64_t)p * g.tpp + t] = pc;
      }
      wave_lds_sync();
    }
  }
  __syncthreads();
  uint32_t* h = hist + (int64_t)p * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(h + i, c);
  }
  if (done) block_min_into(kmin, &smin, &state[p].kth);  // block-uniform
}

// The compacted candidate lists are walked one wave per tile (each wave
// takes tiles wave_id, wave_id + nwaves, ...).
// Candidates 0 .. ct-1 of a slot, read by the wave in rounds of
// kCandChunks chunks of 64 (all loaded before any is used); f(c) runs on
// the lanes that hold a candidate.
template <typename F>
__device__ __forceinline__ void for_each_cand(const uint64_t* __restrict__ slot, uint32_t ct, uint32_t lane,
                                              F&& f) {
  for (uint32_t base = 0; base < ct; base += 64 * kCandChunks) {
    uint64_t cc[kCandChunks];
#pragma unroll
    for (int u = 0; u < kCandChunks; ++u) {
      const uint32_t i = base + 64 * u + lane;
      cc[u] = (i < ct) ? slot[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kCandChunks; ++u)
      if (base + 64 * u + lane < ct) f(cc[u]);
  }
}

// The counts are loaded 64 tiles at a time (lane i: the batch's i-th tile)
// and only tiles with candidates are visited, in ascending order.
template <typename F>
__device__ __forceinline__ void for_each_tile(const Geom& g, int p, const uint32_t* __restrict__ cnt2,
                                              F&& f) {
  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t t0 = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t lane = lane_id();
  for (int64_t tb = t0; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t ct = (tl < g.tpp) ? cnt2[(int64_t)p * g.tpp + tl] : 0u;
    if (ct > (uint32_t)kTile) ct = (uint32_t)kTile;  // a slot holds at most one tile
    uint64_t nz = __ballot(ct != 0u);
    while (nz) {  // wave-uniform
      const int j = __builtin_ctzll(nz);
      nz &= nz - 1;
      f(tb + (int64_t)j * nw, (uint32_t)__shfl((int)ct, j, 64));
    }
  }
}

// Histogram of one digit over the compacted candidates matching the prefix.
__global__ void __launch_bounds__(kThreads)
cand_hist_kernel(Geom g, const uint64_t* __restrict__ cand, const uint32_t* __restrict__ cnt2,
                 const PartSel* __restrict__ state, uint32_t* __restrict__ hist, int shift, int nbits) {
  __shared__ uint32_t sh[kBins];
  const int p = blockIdx.y;
  const PartSel st = state[p];
  if (st.done || st.fb) return;
  const int nb = 1 << nbits;
  for (int i = threadIdx.x; i < nb; i += kThreads) sh[i] = 0;
  __syncthreads();
  const uint32_t lane = lane_id();
  for_each_tile(g, p, cnt2, [&](int64_t t, uint32_t ct) {
    const uint64_t* slot = cand + ((int64_t)p * g.tpp + t) * kTile;
    for_each_cand(slot, ct, lane, [&](uint64_t c) {
      if ((c & st.mask) == st.prefix) atomicAdd(&sh[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
    });
  });
  __syncthreads();
  uint32_t* h = hist + (int64_t)p * kBins;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(h + i, c);
  }
}

// Sets the bits of the compacted candidates at or above the threshold: the
// wave of a tile assembles the tile's words in LDS and ORs each non-zero
// word into the mask (it is the only writer of its tile's words here, so a
// plain read-modify-write suffices), and adds their count to the tile's.
__global__ void __launch_bounds__(kThreads)
mark_kernel(Geom g, const uint64_t* __restrict__ cand, const uint32_t* __restrict__ cnt2,
            PartSel* __restrict__ state, uint64_t* __restrict__ bits, uint32_t* __restrict__ tilecnt) {
  __shared__ unsigned long long words[kThreads / 64][kWordsPerTile];
  __shared__ uint32_t smin;
  const int p = blockIdx.y;
  const uint64_t T = state[p].prefix;
  uint64_t* wb = bits + (int64_t)p * g.wpp;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  unsigned long long* wd = words[wave];
  uint32_t kmin = 0xffffffffu;
  if (threadIdx.x == 0) smin = 0xffffffffu;
  for_each_tile(g, p, cnt2, [&](int64_t t, uint32_t ct) {
    const uint64_t* slot = cand + ((int64_t)p * g.tpp + t) * kTile;
    const uint32_t tile_lo = (uint32_t)(t * kTile);
    const int64_t w = t * kWordsPerTile + lane;
    const uint64_t old = (w < g.wpp) ? wb[w] : 0ull;  // in flight while the candidates are read
    wd[lane] = 0ull;
    wave_lds_sync();
    for_each_cand(slot, ct, lane, [&](uint64_t c) {
      const uint32_t jl = g.idx_mask - (uint32_t)c - tile_lo;
      if (c >= T && jl < (uint32_t)kTile) {
        atomicOr(&wd[jl >> 6], 1ull << (jl & 63));
        const uint32_t key = (uint32_t)(c >> 32);
        kmin = key < kmin ? key : kmin;
      }
    });
    wave_lds_sync();
    const unsigned long long word = wd[lane];
    if (word && w < g.wpp) wb[w] = old | word;
    // these elements were not selected by the candidate select pass, so the
    // tile's count grows by exactly their number
    uint32_t pc = (uint32_t)__popcll(word);
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) pc += __shfl_xor(pc, dd, 64);
    if (lane == 0 && pc) tilecnt[(int64_t)p * g.tpp + t] += pc;
    wave_lds_sync();
  });
  __syncthreads();
  block_min_into(kmin, &smin, &state[p].kth);
}

// Exclusive scan of the tile counts of partition blockIdx.x -> tile_off;
// then the slot's threshold record: the k-th key and the capture bound
// proposed by the level scans for the next step.
__global__ void __launch_bounds__(kThreads)
scan_tiles_kernel(Geom g, const uint32_t* __restrict__ tilecnt, uint32_t* __restrict__ tile_off,
                  PartSel* __restrict__ state, uint32_t* __restrict__ meta_out) {
  __shared__ uint32_t wtot[kThreads / 64];
  const int p = blockIdx.x;
  const int64_t per = (g.tpp + kThreads - 1) / kThreads;
  const int64_t lo = threadIdx.x * per;
  const int64_t hi = (lo + per < g.tpp) ? lo + per : g.tpp;
  const uint32_t* tc = tilecnt + (int64_t)p * g.tpp;
  // a thread's counts are read in batches, all loads of a batch issued
  // before any is used
  constexpr int kBatch = 16;
  uint32_t s = 0;
  for (int64_t t0 = lo; t0 < hi; t0 += kBatch) {
    uint32_t x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = (t0 + u < hi) ? tc[t0 + u] : 0u;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) s += x[u];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan(s, wtot, &tot);
  uint32_t* to = tile_off + (int64_t)p * g.tpp;
  for (int64_t t0 = lo; t0 < hi; t0 += kBatch) {
    uint32_t x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = (t0 + u < hi) ? tc[t0 + u] : 0u;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (t0 + u < hi) to[t0 + u] = run;
      run += x[u];
    }
  }
  if (threadIdx.x == 0) {
    if (tot != (uint32_t)g.k) state[p].fault |= 2u;
    if (meta_out) {
      meta_out[p] = state[p].kth;
      meta_out[g.P + p] = state[p].lo_next;
      meta_out[2 * g.P + p] = state[p].fault;
    }
  }
}

// Position of the r-th set bit (from 0) of a word with more than r set bits.
__device__ __forceinline__ uint32_t select_bit(uint64_t word, uint32_t r) {
  uint32_t pos = 0;
  uint32_t half = (uint32_t)word;
  const uint32_t c32 = (uint32_t)__popc(half);
  if (r >= c32) {
    r -= c32;
    pos = 32;
    half = (uint32_t)(word >> 32);
  }
#pragma unroll
  for (int sh = 16; sh >= 1; sh >>= 1) {
    const uint32_t c = (uint32_t)__popc(half & ((1u << sh) - 1u));
    if (r >= c) {
      r -= c;
      pos += sh;
      half >>= sh;
    }
  }
  return pos;
}

// One wave per tile: write the tile's selected global indices in order.
// RANKS false (sparse masks): each lane walks the set bits of its own word.
// RANKS true (denser masks, where a lane's word holds several indices): the
// lanes take ranks r, r + 64, ... within the tile, so consecutive lanes
// write consecutive entries of the index list; rank r lies in the last word
// whose exclusive popcount prefix is at most r (a binary search over the
// tile's 64 prefixes in LDS), at that word's (r - prefix)-th set bit.
template <bool RANKS>
__global__ void __launch_bounds__(kThreads)
write_idx_kernel(Geom g, const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                 uint32_t* __restrict__ idx) {
  __shared__ unsigned long long swords[RANKS ? kThreads / 64 : 1][kWordsPerTile];
  __shared__ uint32_t spre[RANKS ? kThreads / 64 : 1][kWordsPerTile];
  const int p = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= g.tpp) return;  // wave-uniform; the waves synchronise only among their own lanes
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t w = t * kWordsPerTile + lane;
  uint64_t word = (w < g.wpp) ? bits[(int64_t)p * g.wpp + w] : 0ull;
  const uint32_t c = (uint32_t)__popcll(word);
  uint32_t x = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if ((int)lane >= d) x += y;
  }
  const int64_t base = (int64_t)tile_off[(int64_t)p * g.tpp + t];
  uint32_t* out = idx + (int64_t)p * g.k;
  if (!RANKS) {
    int64_t pos = base + (x - c);
    const uint32_t jbase = (uint32_t)((int64_t)p * g.n_p + w * 64);
    while (word) {
      if (pos < g.k) out[pos] = jbase + (uint32_t)__builtin_ctzll(word);  // bound: malformed mask
      ++pos;
      word &= word - 1ull;
    }
    return;
  }
  const uint32_t sw = RANKS ? wave : 0u;  // this wave's rows of the LDS arrays
  swords[sw][lane] = word;
  spre[sw][lane] = x - c;
  const uint32_t total = (uint32_t)__shfl((int)x, 63, 64);
  wave_lds_sync();
  const uint32_t tbase = (uint32_t)((int64_t)p * g.n_p + t * kTile);
  for (uint32_t r = lane; r < total; r += 64) {
    uint32_t q = 0;
#pragma unroll
    for (uint32_t step = 32; step >= 1; step >>= 1)
      if (spre[sw][q + step] <= r) q += step;
    const uint32_t j = select_bit(swords[sw][q], r - spre[sw][q]);
    if (base + r < g.k) out[base + r] = tbase + q * 64 + j;  // bound: malformed mask
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

// acc |= m over all mask words; *out += popcount of the result.
__global__ void __launch_bounds__(kThreads)
union_kernel(uint64_t* __restrict__ acc, const uint64_t* __restrict__ m, int64_t nwords,
             unsigned long long* __restrict__ out) {
  uint64_t c = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * kThreads) {
    const uint64_t u = acc[i] | m[i];
    acc[i] = u;
    c += (uint64_t)__popcll(u);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
  if (lane_id() == 0 && c) atomicAdd(out, (unsigned long long)c);
}

// ---- validation of a mask against the partitioned top-k contract ----
// One wave per tile: the tile's selected count must equal the step between
// its offset and the next tile's (k after the last tile; the first offset
// is 0), so the offsets are right and the partition holds exactly k bits;
// bits past n_p must be clear; the selection's fault word must be 0.
__global__ void __launch_bounds__(kThreads)
check_tiles_kernel(Geom g, const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                   const uint32_t* __restrict__ meta, uint32_t* __restrict__ res) {
  const int p = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= g.tpp) return;  // wave-uniform
  const uint32_t lane = lane_id();
  const int64_t w = t * kWordsPerTile + lane;
  const uint64_t word = (w < g.wpp) ? bits[(int64_t)p * g.wpp + w] : 0ull;
  uint32_t bad = 0;
  const int tail = (int)(g.n_p & 63);
  if (w == g.wpp - 1 && tail && (word >> tail)) bad |= kMaskBadPad;
  uint32_t c = (uint32_t)__popcll(word);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
  if (lane == 0) {
    const uint32_t* to = tile_off + (int64_t)p * g.tpp;
    const uint32_t here = to[t];
    const uint32_t next = (t + 1 < g.tpp) ? to[t + 1] : (uint32_t)g.k;
    if ((t == 0 && here != 0u) || next < here || next - here != c) bad |= kMaskBadCount;
    if (t == 0 && meta && meta[2 * g.P + p] != 0u) bad |= kMaskBadFault;
  }
  if (bad) atomicOr(res + p, bad);
}

// Every index entry lies in its partition, ascends, and sits on a set bit
// (with exactly k bits per partition this makes the list the set bits).
__global__ void __launch_bounds__(kThreads)
check_idx_kernel(Geom g, const uint64_t* __restrict__ bits, const uint32_t* __restrict__ idx,
                 uint32_t* __restrict__ res) {
  const int64_t total = (int64_t)g.P * g.k;
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < total; r += (int64_t)gridDim.x * kThreads) {
    const int64_t p = r / g.k;
    const int64_t lo = p * g.n_p;
    const int64_t j = (int64_t)idx[r];
    bool ok = j >= lo && j < lo + g.n_p;
    if (ok) {
      const int64_t loc = j - lo;
      ok = ((bits[p * g.wpp + (loc >> 6)] >> (loc & 63)) & 1ull) != 0ull;
    }
    if (ok && r % g.k != 0) ok = (int64_t)idx[r - 1] < j;
    if (!ok) atomicOr(res + p, kMaskBadIdx);
  }
}

// kCaptureMargin * k, at most n_p.
uint32_t capture_target(const Geom& g) {
  double t = kCaptureMargin * (double)g.k;
  if (t > (double)g.n_p) t = (double)g.n_p;
  return (uint32_t)(t + 0.5);
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  zero_u32_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(p, count);
  return hipGetLastError();
}

hipError_t launch_init_state(const Geom& g, PartSel* state, hipStream_t s) {
  init_state_kernel<<<(g.P + kThreads - 1) / kThreads, kThreads, 0, s>>>(state, g.P, (uint32_t)g.k);
  return hipGetLastError();
}

hipError_t launch_level1(const Geom& g, const SelectBufs& w, int mode, hipStream_t s, uint32_t target) {
  level_scan_kernel<<<g.P, kThreads, 0, s>>>(g, w.hist, w.state, 32 + kL1Shift, kDigitBits, mode,
                                             target ? target : capture_target(g));
  return hipGetLastError();
}

hipError_t launch_select_tail(const Geom& g, const SelectBufs& w, uint64_t* bits, uint32_t* idx,
                              uint32_t* tile_off, uint32_t* meta_out, hipStream_t s,
                              void (*mark)(void*, int), void* ctx) {
  const unsigned sblocks = (unsigned)((g.tpp + 4 * kSelectTilesPerWave - 1) / (4 * kSelectTilesPerWave));
  cand_select_kernel<<<dim3(sblocks, g.P), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt1, w.cnt2, w.hist, bits,
                                                              w.tilecnt);
  if (mark) mark(ctx, 1);
  level_scan_kernel<<<g.P, kThreads, 0, s>>>(g, w.hist, w.state, g.levels[0].shift, g.levels[0].nbits,
                                             kScanLevel, capture_target(g));
  for (int l = 1; l < g.nlevels; ++l) {
    cand_hist_kernel<<<dim3(sblocks, g.P), kThreads, 0, s>>>(g, w.cand, w.cnt2, w.state, w.hist,
                                                             g.levels[l].shift, g.levels[l].nbits);
    level_scan_kernel<<<g.P, kThreads, 0, s>>>(g, w.hist, w.state, g.levels[l].shift, g.levels[l].nbits,
                                               kScanLevel, capture_target(g));
  }
  mark_kernel<<<dim3(sblocks, g.P), kThreads, 0, s>>>(g, w.cand, w.cnt2, w.state, bits, w.tilecnt);
  if (mark) mark(ctx, 2);
  const unsigned tblocks = (unsigned)((g.tpp + 3) / 4);
  scan_tiles_kernel<<<g.P, kThreads, 0, s>>>(g, w.tilecnt, tile_off, w.state, meta_out);
  // rank-parallel emission pays from a mask density of about 5% on
  if (g.k * 20 >= g.n_p)
    write_idx_kernel<true><<<dim3(tblocks, g.P), kThreads, 0, s>>>(g, bits, tile_off, idx);
  else
    write_idx_kernel<false><<<dim3(tblocks, g.P), kThreads, 0, s>>>(g, bits, tile_off, idx);
  return hipGetLastError();
}

hipError_t launch_mask_check(const Geom& g, const uint64_t* bits, const uint32_t* idx, const uint32_t* tile_off,
                             const uint32_t* meta, uint32_t* res, hipStream_t s) {
  hipError_t e = launch_zero_u32(res, g.P, s);
  if (e != hipSuccess) return e;
  check_tiles_kernel<<<dim3((unsigned)((g.tpp + 3) / 4), g.P), kThreads, 0, s>>>(g, bits, tile_off, meta, res);
  int64_t blocks = ((int64_t)g.P * g.k + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  check_idx_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(g, bits, idx, res);
  return hipGetLastError();
}

hipError_t launch_union(const Geom& g, uint64_t* acc, const uint64_t* m, uint64_t* out, hipStream_t s) {
  zero_u64_kernel<<<1, 1, 0, s>>>(reinterpret_cast<unsigned long long*>(out));
  const int64_t nwords = (int64_t)g.P * g.wpp;
  int64_t blocks = (nwords + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  union_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(acc, m, nwords, reinterpret_cast<unsigned long long*>(out));
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
