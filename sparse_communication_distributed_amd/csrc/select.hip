// Exact partitioned top-k (technical summary §2, partitioned mask
// synchronisation; ties to the lower index) and the packed forms of the mask
// (single-bit words, ascending index list, per-tile offsets).
//
// Method: radix select on the unique 64-bit composite
//     c = (key << 32) | (idx_mask - local_index)
// so that "the k largest composites" is exactly "the k largest keys, ties to
// the lower index".  The streaming pass that produces the keys captures,
// per tile, every key at or above a bound `lo` (with the element's offset
// in the tile) together with a level-1
// histogram (key bits 30..19) of the captured keys.  If a partition captured
// at least k keys, its top k lie among the captures; otherwise an exact
// fallback recounts all its keys to find the level-1 digit and recaptures
// from there.  A first capture, with no previous bound, takes its bound
// from a histogram of a sample of tiles (kScanSample).  The candidate
// select pass then reads only the captures: digits above the threshold
// digit are selected and written as whole mask words, the threshold
// digit's captures are compacted in place, as 32-bit entries (the key bits
// below the level-1 digit and the offset in the tile), and histogrammed on
// the level-2 digit (key bits 18..7): merged per block with atomics, or, at sparse
// masks on large layouts, by a pass of its own that stores partial
// histograms.  One block per partition resolves level 2; a
// pass over the compacted candidates counts those above the level-2 digit
// per tile and keeps the few at it; one block per partition then resolves
// the remaining levels (key bits 6..0, then the index bits) on those few
// and scans the per-tile counts into tile offsets.  The emission marks the
// threshold bin's selected candidates in the words and writes the
// ascending index list.
#include "level1.h"

namespace scape {
namespace {


// Chunks of 64 candidates a wave loads per round when it walks a slot.
constexpr int kCandChunks = 4;
// Tiles each wave of the sparse-mask emission takes, their loads issued
// together (the rank-parallel emission of denser masks takes one: there a
// tile's index writes dominate and more waves pay).
constexpr int kEmitTiles = 4;
__host__ __device__ constexpr int emit_tiles(bool ranks) { return ranks ? 1 : kEmitTiles; }
// Entries of a wave's LDS index list in the emission of denser masks.
constexpr int kEmitList = 1024;

// The threshold bin's candidates, once compacted by the candidate select
// pass, are 32-bit entries in the keys' place of their tile's slot: the
// key's bits below the level-1 digit (18..0) over the element's offset in
// the tile (12 bits).  The partition's level-1 digit, the tile and idx_mask give the
// composite back.
constexpr int kOffBits = 12;
static_assert((int64_t(1) << kOffBits) == kTile && kL1Shift + kOffBits <= 32, "a bin entry fits 32 bits");
__device__ __forceinline__ uint32_t bin_entry(uint32_t key, uint32_t jl) {
  return ((key & ((1u << kL1Shift) - 1u)) << kOffBits) | jl;
}
// hi: the level-1 digit in place (bin1 << kL1Shift); tile_lo: the tile's
// first local index
__device__ __forceinline__ uint64_t bin_composite(uint32_t e, uint32_t hi, uint32_t tile_lo, uint32_t idx_mask) {
  const uint32_t key = hi | (e >> kOffBits);
  return ((uint64_t)key << 32) | (uint64_t)(idx_mask - (tile_lo + (e & (uint32_t)(kTile - 1))));
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

__global__ void init_state_kernel(PartSel* state, uint32_t* arrive, int p0, int np, uint32_t k) {
  const int p = p0 + blockIdx.x * blockDim.x + threadIdx.x;
  if (p < p0 + np) {
    PartSel s = fresh_sel(k);
    s.fb = 1;
    state[p] = s;
    arrive[p] = 0u;
  }
}

// Level 1 of the threshold search for partition blockIdx.x (level1_block),
// then the partition's bins zeroed.
__global__ void __launch_bounds__(kThreads)
level_scan_kernel(Geom g, uint32_t* __restrict__ hist, PartSel* __restrict__ state, uint32_t* __restrict__ arrive,
                  int mode, uint32_t target) {
  const int p = g.sp0 + blockIdx.x;
  uint32_t* h = hist + (int64_t)p * kBins;
  // the fallback's statistic passes count their blocks' arrivals from zero
  if (mode == kScanCheck && threadIdx.x == 0) arrive[p] = 0u;
  level1_block(g, p, h, state, mode, target);
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
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

// Tiles whose first 64 captured candidates cand_select loads together.
constexpr int kPreTiles = 4;

// One wave per tile: reads the tile's captured keys and offsets (the first
// 64 with those of the next kPreTiles - 1 tiles of the wave, the rest in
// rounds of kCandChunks chunks of 64); selects the digits above the level-1
// threshold digit into the tile's 64 mask words (written whole, so every
// word of the partition is written) and counts them; compacts the threshold
// digit's candidates in place, in order, as bin entries over the keys (a
// write never passes the keys already read), and (HIST) histograms their
// level-2 digit, merging the block's histogram into the partition's with
// atomics.
template <bool HIST>
__global__ void __launch_bounds__(kThreads)
cand_select_kernel(Geom g, PartSel* __restrict__ state, uint32_t* __restrict__ cand,
                   const uint32_t* __restrict__ cnt1, uint32_t* __restrict__ cnt2,
                   uint32_t* __restrict__ hist, uint64_t* __restrict__ bits,
                   uint32_t* __restrict__ tilecnt) {
  __shared__ unsigned long long words[kThreads / 64][kWordsPerTile];
  __shared__ uint32_t sh[HIST ? kBins : 1];
  __shared__ uint32_t smin;
  const int p = g.sp0 + blockIdx.y;
  const PartSel st = state[p];
  const uint32_t B1 = st.bin1;
  const bool done = st.done != 0;
  const int l2shift = g.levels[0].shift - 32;  // the level-2 digit in a key
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  unsigned long long* wd = words[wave];
  uint32_t kmin = 0xffffffffu;  // smallest key selected whole from the threshold digit
  if (HIST)
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh[i] = 0;
  if (threadIdx.x == 0) smin = 0xffffffffu;
  __syncthreads();
  // The wave takes tiles t0, t0 + nw, ... in batches of up to 64: lane i
  // loads the capture count of the batch's i-th tile.  The first 64
  // captures of kPreTiles tiles are loaded together before the first of
  // them is processed, so a group of tiles costs one dependent global load
  // rather than one per tile.
  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t t0 = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  const uint32_t* c1p = cnt1 + (int64_t)p * g.tpp;
  uint32_t* cpart = cand + (int64_t)p * g.tpp * kSlotWords;
  for (int64_t tb = t0; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t cv = (tl < g.tpp) ? c1p[tl] : 0u;
    if (cv > (uint32_t)kTile) cv = (uint32_t)kTile;  // a slot holds at most one tile
    const int64_t left = (g.tpp - tb + nw - 1) / nw;
    const int nb = left < 64 ? (int)left : 64;
    for (int j0 = 0; j0 < nb; j0 += kPreTiles) {
      uint32_t kpre[kPreTiles], opre[kPreTiles];
#pragma unroll
      for (int u = 0; u < kPreTiles; ++u) {
        const int j = j0 + u;
        const uint32_t nn = (uint32_t)__shfl((int)cv, j & 63, 64);
        const uint32_t* sj = cpart + (tb + (int64_t)j * nw) * kSlotWords;
        const bool in = j < nb && lane < nn;
        kpre[u] = in ? sj[lane] : 0u;
        opre[u] = in ? reinterpret_cast<const uint16_t*>(sj + kTile)[lane] : 0u;
      }
      // Wait for the group's loads here, once: the tiles' own code then
      // has no load to wait for (unless a tile holds more than 64
      // captures), so it never waits for the stores of the tiles before it.
#pragma unroll
      for (int u = 0; u < kPreTiles; ++u) asm volatile("" ::"v"(kpre[u]), "v"(opre[u]));
#pragma unroll
      for (int u = 0; u < kPreTiles; ++u) {
        const int j = j0 + u;
        if (j >= nb) break;  // wave-uniform
        const int64_t t = tb + (int64_t)j * nw;
        const uint32_t n1 = (uint32_t)__shfl((int)cv, j, 64);
        wd[lane] = 0ull;
        wave_lds_sync();
        uint32_t* slot = cpart + t * kSlotWords;
        const uint16_t* offs = reinterpret_cast<const uint16_t*>(slot + kTile);
        uint32_t n2 = 0;
        auto take = [&](uint32_t key, uint32_t jl, bool valid) {
          const uint32_t d1 = (key >> kL1Shift) & (kBins - 1);
          const bool sel = valid && (d1 > B1 || (done && d1 == B1));
          const bool keep = valid && !done && d1 == B1;
          if (sel) {
            atomicOr(&wd[jl >> 6], 1ull << (jl & 63));
            if (d1 == B1) kmin = key < kmin ? key : kmin;
          }
          // in-place compaction into bin entries: a write lands on a key
          // already read (n2 never passes the candidates read so far)
          const uint64_t kb = __ballot(keep);
          if (keep) {
            slot[n2 + mbcnt(kb)] = bin_entry(key, jl);
            if (HIST) atomicAdd(&sh[(key >> l2shift) & (kBins - 1)], 1u);
          }
          n2 += (uint32_t)__popcll(kb);
        };
        if (n1) take(kpre[u], opre[u] & (uint32_t)(kTile - 1), lane < n1);  // wave-uniform
        // the rest in rounds of kCandChunks chunks of 64, all loaded before
        // any is used
        for (uint32_t base = 64; base < n1; base += 64 * kCandChunks) {
          uint32_t kc[kCandChunks], oc[kCandChunks];
#pragma unroll
          for (int q = 0; q < kCandChunks; ++q) {
            const uint32_t i = base + 64 * q + lane;
            kc[q] = (i < n1) ? slot[i] : 0u;
            oc[q] = (i < n1) ? offs[i] : 0u;
          }
#pragma unroll
          for (int q = 0; q < kCandChunks; ++q) {
            if (base + 64 * q >= n1) break;  // wave-uniform
            take(kc[q], oc[q] & (uint32_t)(kTile - 1), base + 64 * q + lane < n1);
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
  }
  __syncthreads();
  if (HIST) {
    uint32_t* h = hist + (int64_t)p * kBins;
    for (int i = threadIdx.x; i < kBins; i += kThreads) {
      const uint32_t c = sh[i];
      if (c) atomicAdd(h + i, c);
    }
  }
  if (done) block_min_into(kmin, &smin, &state[p].kth);  // block-uniform
}

// Bin entries 0 .. ct-1 of a tile (the compacted threshold bin), read by
// the wave in rounds of kCandChunks chunks of 64 (all loaded before any is
// used); f(e) runs on the lanes that hold an entry.  Every load of a round
// is waited for at once, so none is left outstanding after the loop (code
// after it then has no reason to wait for the stores issued since).
template <typename F>
__device__ __forceinline__ void for_each_entry(const uint32_t* __restrict__ ent, uint32_t ct, uint32_t lane,
                                               F&& f) {
  for (uint32_t base = 0; base < ct; base += 64 * kCandChunks) {
    uint32_t cc[kCandChunks];
#pragma unroll
    for (int u = 0; u < kCandChunks; ++u) {
      const uint32_t i = base + 64 * u + lane;
      cc[u] = (i < ct) ? ent[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kCandChunks; ++u) asm volatile("" ::"v"(cc[u]));
#pragma unroll
    for (int u = 0; u < kCandChunks; ++u)
      if (base + 64 * u + lane < ct) f(cc[u]);
  }
}

// ---- the threshold search inside the level-1 threshold bin ----
// One block of kResolveThreads per partition.
constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;

// Exclusive scan over a block of kResolveThreads; `wtot` is LDS [waves].
__device__ __forceinline__ uint32_t resolve_excl_scan(uint32_t v, uint32_t* wtot, uint32_t* total) {
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
  for (int w = 0; w < kResolveWaves; ++w) {
    if (w < (int)wave) off += wtot[w];
    tot += wtot[w];
  }
  *total = tot;
  return off + x - v;
}

struct DigitFind {
  int d;           // digit holding the rank, -1 if none
  uint32_t c;      // its count
  uint32_t above;  // count above it
  uint32_t tot;    // count of all bins
};

// In bins h[0 .. nb) scanned from the largest digit, the digit in which the
// cumulative count first reaches `rank` (1-based).  Block-wide; every
// thread gets the result.
__device__ DigitFind find_digit(const uint32_t* h, int nb, uint32_t rank, uint32_t* wtot, DigitFind* out) {
  const int per = (nb + kResolveThreads - 1) / kResolveThreads;
  uint32_t s = 0;
  for (int q = 0; q < per; ++q) {
    const int pos = threadIdx.x * per + q;
    if (pos < nb) s += h[nb - 1 - pos];
  }
  uint32_t tot;
  const uint32_t above = resolve_excl_scan(s, wtot, &tot);
  if (threadIdx.x == 0) *out = DigitFind{-1, 0u, 0u, tot};
  __syncthreads();
  if (rank >= 1 && above < rank && rank <= above + s) {
    uint32_t acc = above;
    for (int q = 0; q < per; ++q) {
      const int pos = threadIdx.x * per + q;
      if (pos >= nb) break;
      const int d = nb - 1 - pos;
      const uint32_t c = h[d];
      if (acc + c >= rank) {
        *out = DigitFind{d, c, acc, tot};
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const DigitFind r = *out;
  __syncthreads();
  return r;
}

// The threshold bin's candidates of partition p (the bin entries at the
// start of the tile slots), walked by the block's waves.  A wave takes 64 tiles at a
// time (wave w: tiles w, w + W, ..., W waves), scans their counts and walks
// the 64 slots as one flattened sequence: lane i takes entries i, i + 64,
// ... and finds its tile by a binary search over the 64 prefixes in LDS, so
// kWalkBatch loads per lane are in flight at once whatever the tiles' sizes.
// f(c, j) runs for each candidate's composite c (hi: the level-1 digit in
// place) of the batch's tile j; after a batch, end(t, j) runs on the lane of
// each tile t with candidates (j = the lane).
constexpr int kWalkBatch = 8;
template <typename F, typename E>
__device__ __forceinline__ void walk_bin(const Geom& g, int p, uint32_t hi, const uint32_t* __restrict__ cand,
                                         const uint32_t* __restrict__ cnt2, uint32_t* spre, F&& f, E&& end) {
  const uint32_t* cp = cand + (int64_t)p * g.tpp * kSlotWords;
  const int64_t nw = kResolveWaves;
  const uint32_t lane = lane_id();
  for (int64_t tb = threadIdx.x >> 6; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t ct = (tl < g.tpp) ? cnt2[(int64_t)p * g.tpp + tl] : 0u;
    if (ct > (uint32_t)kTile) ct = (uint32_t)kTile;  // a slot holds at most one tile
    uint32_t x = ct;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(x, d, 64);
      if ((int)lane >= d) x += y;
    }
    const uint32_t total = (uint32_t)__shfl((int)x, 63, 64);
    if (total == 0) continue;  // wave-uniform
    spre[lane] = x - ct;
    wave_lds_sync();
    for (uint32_t i0 = 0; i0 < total; i0 += 64 * kWalkBatch) {
      uint32_t cc[kWalkBatch];
      uint32_t jj[kWalkBatch];
#pragma unroll
      for (int u = 0; u < kWalkBatch; ++u) {
        const uint32_t i = i0 + 64 * u + lane;
        uint32_t j = 0;
#pragma unroll
        for (uint32_t step = 32; step >= 1; step >>= 1)
          if (spre[j + step] <= i) j += step;  // the last tile whose prefix is at most i
        jj[u] = j;
        cc[u] = (i < total) ? cp[(tb + (int64_t)j * nw) * kSlotWords + (i - spre[j])] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kWalkBatch; ++u)
        if (i0 + 64 * u + lane < total)
          f(bin_composite(cc[u], hi, (uint32_t)((tb + (int64_t)jj[u] * nw) * kTile), g.idx_mask), jj[u]);
    }
    wave_lds_sync();
    if (ct) end(tl, lane);
    wave_lds_sync();
  }
}

// The level-2 histogram of the threshold bin's compacted candidates as a
// pass of its own (layouts with g.hparts > 0): block (h, p) walks its share
// of partition p's tiles, as walk_bin walks a partition's (the batch's bin
// entries as one flattened sequence), histograms their level-2 digit
// (key bits 18..7, which a bin entry holds whole) in LDS and stores the kBins counts whole to part
// [p][h][*], so no atomics leave the block.  Partitions whose search level
// 1 finished have no candidates compacted and get zero counts.
constexpr int kHistThreads = 1024;
constexpr int kHistWaves = kHistThreads / 64;
__global__ void __launch_bounds__(kHistThreads)
l2_hist_kernel(Geom g, const uint32_t* __restrict__ cand, const uint32_t* __restrict__ cnt2,
               uint32_t* __restrict__ part) {
  __shared__ uint32_t sh[kBins];
  __shared__ uint32_t spre[kHistWaves][64];
  const int p = g.sp0 + blockIdx.y;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) sh[i] = 0u;
  __syncthreads();
  const int shift = g.levels[0].shift - 32 + kOffBits;  // the level-2 digit in a bin entry
  uint32_t* pre = spre[wave];
  const uint32_t* c2p = cnt2 + (int64_t)p * g.tpp;
  const uint32_t* cp = cand + (int64_t)p * g.tpp * kSlotWords;
  const int64_t nw = (int64_t)gridDim.x * kHistWaves;
  const int64_t t0 = (int64_t)blockIdx.x * kHistWaves + wave;
  for (int64_t tb = t0; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t ct = (tl < g.tpp) ? c2p[tl] : 0u;
    if (ct > (uint32_t)kTile) ct = (uint32_t)kTile;  // a slot holds at most one tile
    uint32_t x = ct;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(x, d, 64);
      if ((int)lane >= d) x += y;
    }
    const uint32_t total = (uint32_t)__shfl((int)x, 63, 64);
    if (total == 0) continue;  // wave-uniform
    pre[lane] = x - ct;
    wave_lds_sync();
    for (uint32_t i0 = 0; i0 < total; i0 += 64 * kWalkBatch) {
      uint32_t cc[kWalkBatch];
#pragma unroll
      for (int u = 0; u < kWalkBatch; ++u) {
        const uint32_t i = i0 + 64 * u + lane;
        uint32_t j = 0;
#pragma unroll
        for (uint32_t step = 32; step >= 1; step >>= 1)
          if (pre[j + step] <= i) j += step;  // the last tile whose prefix is at most i
        cc[u] = (i < total) ? cp[(tb + (int64_t)j * nw) * kSlotWords + (i - pre[j])] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kWalkBatch; ++u)
        if (i0 + 64 * u + lane < total) atomicAdd(&sh[(uint32_t)(cc[u] >> shift) & (uint32_t)(kBins - 1)], 1u);
    }
    wave_lds_sync();
  }
  __syncthreads();
  uint32_t* out = part + ((int64_t)p * gridDim.x + blockIdx.x) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) out[i] = sh[i];
}

constexpr int kScanBatch = 16;

// ---- the threshold search inside the level-1 bin, and the tile offsets ----
// Level 2 (key bits 18..7) for partition blockIdx.x, on the histogram of
// the threshold bin's candidates that the candidate select pass built:
// the digit holding the remaining rank narrows the prefix (the search is
// done when that digit's candidates are exactly the rank still needed),
// and the next step's capture bound is refined to the level-2 digit at
// which the count from the top reaches the part of the target inside the
// bin.  Leaves the partition's histogram bins zeroed and its survivor
// count at zero (or, when the candidates left at the level-2 digit cannot
// fit the survivor list, at their number).
template <bool PARTS>
__global__ void __launch_bounds__(kThreads)
l2_scan_kernel(Geom g, uint32_t* __restrict__ hist, const uint32_t* __restrict__ part, PartSel* __restrict__ state,
               uint32_t* __restrict__ nsurv, uint32_t target) {
  __shared__ uint32_t wtot[kThreads / 64];
  __shared__ uint32_t s_d, s_c, s_above, s_lo;
  __shared__ uint32_t hs[PARTS ? kBins : 1];
  const int p = g.sp0 + blockIdx.x;
  uint32_t* gh = hist + (int64_t)p * kBins;
  const PartSel cur = state[p];
  if (threadIdx.x == 0) nsurv[p] = 0u;
  if (!cur.done && !cur.fb) {
    if constexpr (PARTS) {
      // the sum of the partition's g.hparts parts: thread i adds bins
      // 4i .. 4i+3 (and the same 1024 bins on) of every part, with 16-byte
      // loads, four parts at a time
      typedef uint32_t v4u __attribute__((ext_vector_type(4)));
      const int H = g.hparts;
      const v4u* pp = reinterpret_cast<const v4u*>(part + (int64_t)p * H * kBins);
      constexpr int R = kBins / (4 * kThreads), stride = kBins / 4;
      v4u acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = v4u{0u, 0u, 0u, 0u};
      int q = 0;
      for (; q + 4 <= H; q += 4) {
        v4u x[4][R];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < R; ++r) x[a][r] = pp[(int64_t)(q + a) * stride + r * kThreads + threadIdx.x];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] += x[a][r];
      }
      for (; q < H; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += pp[(int64_t)q * stride + r * kThreads + threadIdx.x];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int b = 4 * (r * kThreads + threadIdx.x);
        hs[b] = acc[r].x;
        hs[b + 1] = acc[r].y;
        hs[b + 2] = acc[r].z;
        hs[b + 3] = acc[r].w;
      }
      __syncthreads();
    }
    const uint32_t* h = PARTS ? hs : gh;
    const int shift = g.levels[0].shift;
    constexpr int nb = kBins, per = kBins / kThreads;
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) s += h[nb - 1 - (threadIdx.x * per + q)];
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0) {
      s_d = 0xffffffffu;
      s_lo = 0xffffffffu;
    }
    __syncthreads();
    const int64_t in_bin = (int64_t)target - ((int64_t)g.k - (int64_t)cur.r);
    uint32_t acc = above;
    for (int q = 0; q < per; ++q) {
      const int d = nb - 1 - (threadIdx.x * per + q);
      const uint32_t c = h[d];
      if (acc < cur.r && acc + c >= cur.r) {
        s_d = (uint32_t)d;
        s_c = c;
        s_above = acc;
      }
      if (in_bin > 0 && in_bin <= (int64_t)tot && (int64_t)acc < in_bin && (int64_t)(acc + c) >= in_bin)
        s_lo = (uint32_t)d;
      acc += c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      PartSel o = cur;
      const uint64_t dmask = (uint64_t)(kBins - 1) << shift;
      if (s_lo != 0xffffffffu) {
        const uint32_t lo = (uint32_t)(((cur.prefix & ~dmask) | ((uint64_t)s_lo << shift)) >> 32);
        if (lo > o.lo_next) o.lo_next = lo;
      }
      if (s_d == 0xffffffffu) {  // the rank lies in no bin: corrupted input
        o.fault |= 1u;
        o.done = 1;
      } else {
        o.r = cur.r - s_above;
        o.prefix = cur.prefix | ((uint64_t)s_d << shift);
        o.mask = cur.mask | dmask;
        o.bin2 = s_d;
        o.done2 = (s_c == o.r) ? 1u : 0u;
        // more candidates at the level-2 digit than the survivor list
        // holds (ties): the walk keeps no list, and the count says so
        if (!o.done2 && s_c > (uint32_t)kSurvivorCap) nsurv[p] = s_c;
      }
      state[p] = o;
    }
  }
  __syncthreads();
  if (!PARTS)
    for (int i = threadIdx.x; i < kBins; i += kThreads) gh[i] = 0u;
}

// Survivors a bin_walk block stages in LDS before it reserves their range of
// the partition's list with one atomic.
constexpr int kWalkStage = 512;
// Tiles each wave of bin_walk's flattened walk takes, at most (fewer where
// the layout has fewer than kSelectWaves * kFlatTilesPerWave tiles).
constexpr int kFlatTilesPerWave = 32;

// One wave per tile, or per batch of tiles, over the threshold bin's
// compacted candidates, after level 2: adds to each tile's count the
// candidates above the level-2 threshold digit (and those at it, when that
// digit decides the search); when it does not, histograms the level-3 digit
// (key bits 6..0) of the candidates at it and, when level 2 counted no more
// of them than the survivor list holds, appends them to the list.  When the
// level-2 digit decides, the smallest key at it is folded into the state's
// k-th key.  Each wave takes tiles wave_id, wave_id + nwaves, ... in
// batches of 64 (lane i: the batch's i-th tile, its candidate count and its
// tile count).  FLAT (waves with several tiles of few candidates each): the
// wave walks the batch's candidates as one flattened sequence, as walk_bin
// does, so that kWalkBatch loads per lane are in flight whatever the tiles'
// sizes.  Otherwise it walks the tiles with candidates one by one, and the
// first 64 candidates of a tile are loaded while the tile before it is
// walked.
template <bool FLAT>
__global__ void __launch_bounds__(kThreads)
bin_walk_kernel(Geom g, PartSel* __restrict__ state, const uint32_t* __restrict__ cand,
                const uint32_t* __restrict__ cnt2, uint32_t* __restrict__ tilecnt, uint32_t* __restrict__ hist,
                uint64_t* __restrict__ surv, uint32_t* __restrict__ nsurv) {
  __shared__ uint32_t sh[1 << (kL1Shift - kDigitBits)];
  __shared__ unsigned long long sstage[kWalkStage];
  __shared__ uint32_t spre[FLAT ? kThreads / 64 : 1][64];
  __shared__ uint32_t sadd[FLAT ? kThreads / 64 : 1][64];
  __shared__ uint32_t smin, sn, sfill, sbase;
  constexpr int nb3 = 1 << (kL1Shift - kDigitBits);
  const int p = g.sp0 + blockIdx.y;
  const PartSel st = state[p];
  if (st.fb || !st.mask || st.done) return;  // block-uniform: nothing left in the bin to walk
  const bool done2 = st.done2 != 0;
  const int sh2 = g.levels[0].shift, sh3 = g.levels[1].shift;
  const uint32_t d2 = st.bin2;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < nb3; i += kThreads) sh[i] = 0u;
  if (FLAT) sadd[wave][lane] = 0u;
  if (threadIdx.x == 0) {
    smin = 0xffffffffu;
    sn = 0u;     // stage positions handed out
    sfill = 0u;  // stage entries written: a prefix of the stage
  }
  __syncthreads();
  uint32_t kmin = 0xffffffffu;
  uint64_t* sl = surv + (int64_t)p * kSurvivorCap;
  uint32_t* tc = tilecnt + (int64_t)p * g.tpp;
  const uint32_t* c2p = cnt2 + (int64_t)p * g.tpp;
  const uint32_t* cp = cand + (int64_t)p * g.tpp * kSlotWords;
  const uint32_t hi = st.bin1 << kL1Shift;
  // false when level 2 found more candidates at its digit than the list
  // holds: then no wave appends (the walks of the later levels take over)
  const bool listed = nsurv[p] <= (uint32_t)kSurvivorCap;

  // One candidate per lane, called by the whole wave (valid: the lane holds
  // one).  Returns whether it adds to its tile's count.
  auto take = [&](uint64_t c, bool valid) -> bool {
    const uint32_t dd = (uint32_t)(c >> sh2) & (uint32_t)(kBins - 1);
    const bool at = valid && dd == d2;
    if (at && done2) {
      const uint32_t key = (uint32_t)(c >> 32);
      kmin = key < kmin ? key : kmin;
    }
    const bool keep = at && !done2;
    const uint64_t kb = __ballot(keep);
    if (kb && !listed) {  // wave-uniform
      if (keep) atomicAdd(&sh[(uint32_t)(c >> sh3) & (uint32_t)(nb3 - 1)], 1u);
    } else if (kb) {  // wave-uniform
      // Level 2 counted these candidates, no more than the list holds, so
      // each has a place in it.  They go to the block's LDS stage; a chunk
      // that no longer fits there reserves its own range of the list at once
      // (positions are handed out in order, so the chunks that fit form a
      // prefix of the stage).
      const uint32_t nk = (uint32_t)__popcll(kb);
      uint32_t pos = 0u;
      if (lane == 0) pos = atomicAdd(&sn, nk);
      pos = (uint32_t)__shfl((int)pos, 0, 64);
      const bool staged = pos + nk <= (uint32_t)kWalkStage;  // wave-uniform
      if (staged) {
        if (lane == 0) atomicAdd(&sfill, nk);
      } else {
        if (lane == 0) pos = atomicAdd(nsurv + p, nk);
        pos = (uint32_t)__shfl((int)pos, 0, 64);
      }
      pos += mbcnt(kb);
      if (keep) {
        atomicAdd(&sh[(uint32_t)(c >> sh3) & (uint32_t)(nb3 - 1)], 1u);
        if (staged)
          sstage[pos] = c;
        else if (pos < (uint32_t)kSurvivorCap)
          sl[pos] = c;
      }
    }
    return valid && (dd > d2 || (done2 && at));
  };

  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t t0 = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  for (int64_t tb = t0; tb < g.tpp; tb += 64 * nw) {
    const int64_t tl = tb + (int64_t)lane * nw;
    uint32_t ct = (tl < g.tpp) ? c2p[tl] : 0u;
    const uint32_t tv = (tl < g.tpp) ? tc[tl] : 0u;
    if (ct > (uint32_t)kTile) ct = (uint32_t)kTile;  // a slot holds at most one tile
    if constexpr (FLAT) {
      uint32_t* pre = spre[wave];
      uint32_t* ad = sadd[wave];
      uint32_t x = ct;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if ((int)lane >= d) x += y;
      }
      const uint32_t total = (uint32_t)__shfl((int)x, 63, 64);
      if (total == 0) continue;  // wave-uniform
      pre[lane] = x - ct;
      wave_lds_sync();
      for (uint32_t i0 = 0; i0 < total; i0 += 64 * kWalkBatch) {
        uint32_t cc[kWalkBatch];
        uint32_t jj[kWalkBatch];
#pragma unroll
        for (int u = 0; u < kWalkBatch; ++u) {
          const uint32_t i = i0 + 64 * u + lane;
          uint32_t j = 0;
#pragma unroll
          for (uint32_t step = 32; step >= 1; step >>= 1)
            if (pre[j + step] <= i) j += step;  // the last tile whose prefix is at most i
          jj[u] = j;
          cc[u] = (i < total) ? cp[(tb + (int64_t)j * nw) * kSlotWords + (i - pre[j])] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kWalkBatch; ++u) {
          if (i0 + 64 * u >= total) break;  // wave-uniform
          const bool valid = i0 + 64 * u + lane < total;
          const uint32_t tile_lo = (uint32_t)((tb + (int64_t)jj[u] * nw) * kTile);
          const bool up = take(bin_composite(cc[u], hi, tile_lo, g.idx_mask), valid);
          // the chunk's lanes hold consecutive entries, so each tile's
          // entries are a run of lanes: the run's first lane adds its count
          const uint32_t j = jj[u];
          const uint32_t jp = (uint32_t)__shfl_up((int)j, 1, 64);
          const uint64_t heads = __ballot(valid && (lane == 0 || j != jp));
          const uint64_t ups = __ballot(up);
          if ((heads >> lane) & 1ull) {
            const uint64_t later = lane == 63 ? 0ull : heads & (~0ull << (lane + 1));
            const uint64_t below_end = later ? (1ull << __builtin_ctzll(later)) - 1ull : ~0ull;
            const uint32_t n = (uint32_t)__popcll(ups & below_end & (~0ull << lane));
            if (n) atomicAdd(&ad[j], n);
          }
        }
      }
      wave_lds_sync();
      const uint32_t a = ad[lane];
      if (a) tc[tl] = tv + a;  // this wave alone walks tile tl here
      ad[lane] = 0u;
      wave_lds_sync();
    } else {
      uint64_t nz = __ballot(ct != 0u);
      uint32_t cnext = 0u;
      if (nz) {  // wave-uniform
        const int j = __builtin_ctzll(nz);
        const uint32_t nn = (uint32_t)__shfl((int)ct, j, 64);
        if (lane < nn) cnext = cp[(tb + (int64_t)j * nw) * kSlotWords + lane];
      }
      while (nz) {  // wave-uniform
        const int j = __builtin_ctzll(nz);
        nz &= nz - 1;
        const int64_t t = tb + (int64_t)j * nw;
        const uint32_t n1 = (uint32_t)__shfl((int)ct, j, 64);
        const uint32_t tvj = (uint32_t)__shfl((int)tv, j, 64);
        const uint32_t c0 = cnext;
        if (nz) {
          const int jn = __builtin_ctzll(nz);
          const uint32_t nn = (uint32_t)__shfl((int)ct, jn, 64);
          cnext = (lane < nn) ? cp[(tb + (int64_t)jn * nw) * kSlotWords + lane] : 0u;
        }
        const uint32_t* ent = cp + t * kSlotWords;
        const uint32_t tile_lo = (uint32_t)(t * kTile);
        uint32_t add = 0;
        for (uint32_t base = 0; base < n1; base += 64 * kCandChunks) {
          uint32_t cc[kCandChunks];
#pragma unroll
          for (int u = 0; u < kCandChunks; ++u) {
            const uint32_t i = base + 64 * u + lane;
            cc[u] = (base == 0 && u == 0) ? c0 : ((i < n1) ? ent[i] : 0u);
          }
#pragma unroll
          for (int u = 0; u < kCandChunks; ++u) {
            if (base + 64 * u >= n1) break;  // wave-uniform
            add += take(bin_composite(cc[u], hi, tile_lo, g.idx_mask), base + 64 * u + lane < n1) ? 1u : 0u;
          }
        }
#pragma unroll
        for (int dd = 32; dd >= 1; dd >>= 1) add += __shfl_xor(add, dd, 64);
        if (lane == 0 && add) tc[t] = tvj + add;  // this wave alone walks tile t here
      }
    }
  }
  __syncthreads();
  uint32_t* h = hist + (int64_t)p * kBins;
  for (int i = threadIdx.x; i < nb3; i += kThreads) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(h + i, c);
  }
  const uint32_t fill = sfill;
  if (fill) {  // block-uniform: the staged survivors take one range of the list
    if (threadIdx.x == 0) sbase = atomicAdd(nsurv + p, fill);
    __syncthreads();
    const uint32_t b0 = sbase;
    for (uint32_t i = threadIdx.x; i < fill; i += kThreads)
      if (b0 + i < (uint32_t)kSurvivorCap) sl[b0 + i] = sstage[i];
  }
  if (done2) block_min_into(kmin, &smin, &state[p].kth);  // block-uniform
}

// The remaining levels for partition blockIdx.x (after level 2: key bits
// 6..0 from the walk's histogram, then the index bits) on the survivors, or
// by walks over the tile slots when the survivors overflowed their list;
// then the tile counts of the selected survivors (composite >= T), and the
// exclusive scan of the partition's tile counts into tile_off.  Writes the
// partition's search state and the slot's threshold record (k-th key, next
// capture bound, fault word: bit 1 if the total is not k), and leaves the
// partition's histogram bins zeroed.
__global__ void __launch_bounds__(kResolveThreads)
finish_kernel(Geom g, uint32_t* __restrict__ hist, PartSel* __restrict__ state,
              const uint32_t* __restrict__ cand, const uint32_t* __restrict__ cnt2,
              const uint64_t* __restrict__ surv, const uint32_t* __restrict__ nsurv,
              uint32_t* __restrict__ tilecnt, uint32_t* __restrict__ tile_off, uint32_t* __restrict__ meta_out) {
  __shared__ uint32_t sh[kBins];
  __shared__ unsigned long long ls[kSurvivorCap];
  __shared__ uint32_t wtot[kResolveWaves];
  __shared__ uint32_t spre[kResolveWaves][65];
  __shared__ uint32_t scnt[kResolveWaves][64];
  __shared__ DigitFind sfind;
  const int p = g.sp0 + blockIdx.x;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t* tc = tilecnt + (int64_t)p * g.tpp;
  PartSel st = state[p];
  if (lane == 0) spre[wave][64] = 0xffffffffu;  // above every index: ends the binary search
  scnt[wave][lane] = 0u;
  if (!st.done && !st.fb && st.mask && !st.done2) {
    const uint32_t ns = nsurv[p];
    const bool kept = ns <= (uint32_t)kSurvivorCap;
    for (uint32_t i = threadIdx.x; kept && i < ns; i += kResolveThreads) ls[i] = surv[(int64_t)p * kSurvivorCap + i];
    uint32_t* gh = hist + (int64_t)p * kBins;
    const int nb3 = 1 << g.levels[1].nbits;
    for (int i = threadIdx.x; i < nb3; i += kResolveThreads) {
      sh[i] = gh[i];
      gh[i] = 0u;
    }
    __syncthreads();
    for (int l = 1; l < g.nlevels; ++l) {
      const int shift = g.levels[l].shift, nb = 1 << g.levels[l].nbits;
      const uint64_t dmask = (uint64_t)(nb - 1) << shift;
      if (l > 1) {
        for (int i = threadIdx.x; i < nb; i += kResolveThreads) sh[i] = 0u;
        __syncthreads();
        const uint64_t pm = st.mask, pv = st.prefix;
        if (kept) {
          for (uint32_t i = threadIdx.x; i < ns; i += kResolveThreads) {
            const uint64_t c = ls[i];
            if ((c & pm) == pv) atomicAdd(&sh[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
          }
        } else {
          walk_bin(g, p, st.bin1 << kL1Shift, cand, cnt2, spre[wave],
                   [&](uint64_t c, uint32_t) {
                     if ((c & pm) == pv) atomicAdd(&sh[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
                   },
                   [&](int64_t, uint32_t) {});
        }
        __syncthreads();
      }
      const DigitFind f = find_digit(sh, nb, st.r, wtot, &sfind);
      if (f.d < 0) {  // corrupted input
        st.fault |= 1u;
        break;
      }
      st.r -= f.above;
      st.prefix |= (uint64_t)f.d << shift;
      st.mask |= dmask;
      if (f.c == st.r) break;  // every composite matching the prefix is selected
      __syncthreads();
    }
    st.kth = (uint32_t)(st.prefix >> 32);  // both key levels are resolved here
    // tile counts of the selected candidates at the level-2 digit
    const uint64_t T = st.prefix;
    const uint32_t d2 = st.bin2;
    const int sh2 = g.levels[0].shift;
    if (kept) {
      for (uint32_t i = threadIdx.x; i < ns; i += kResolveThreads) {
        const uint64_t c = ls[i];
        const uint32_t jl = g.idx_mask - (uint32_t)c;
        if (c >= T && jl < (uint32_t)g.n_p) atomicAdd(tc + jl / kTile, 1u);
      }
    } else {
      walk_bin(g, p, st.bin1 << kL1Shift, cand, cnt2, spre[wave],
               [&](uint64_t c, uint32_t j) {
                 if (((uint32_t)(c >> sh2) & (uint32_t)(kBins - 1)) == d2 && c >= T) atomicAdd(&scnt[wave][j], 1u);
               },
               [&](int64_t t, uint32_t j) {
                 const uint32_t add = scnt[wave][j];
                 if (add) atomicAdd(tc + t, add);
                 scnt[wave][j] = 0u;
               });
    }
  }
  st.done = 1;
  __syncthreads();
  // ---- tile offsets: each thread sums a contiguous run of tile counts, the
  // block scans the run sums, and each thread writes its run's offsets.  The
  // counts may have been updated above by atomics, so they are read at
  // device scope (not from a cache line another block of this CU loaded).
  const int64_t per = (g.tpp + kResolveThreads - 1) / kResolveThreads;
  const int64_t lo = threadIdx.x * per;
  const int64_t hi = (lo + per < g.tpp) ? lo + per : g.tpp;
  uint32_t s = 0;
  for (int64_t t0 = lo; t0 < hi; t0 += kScanBatch) {
    uint32_t x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u)
      x[u] = (t0 + u < hi) ? __hip_atomic_load(tc + t0 + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) s += x[u];
  }
  uint32_t tot;
  uint32_t run = resolve_excl_scan(s, wtot, &tot);
  uint32_t* to = tile_off + (int64_t)p * g.tpp;
  for (int64_t t0 = lo; t0 < hi; t0 += kScanBatch) {
    uint32_t x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u)
      x[u] = (t0 + u < hi) ? __hip_atomic_load(tc + t0 + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (t0 + u < hi) to[t0 + u] = run;
      run += x[u];
    }
  }
  if (threadIdx.x == 0) {
    if (tot != (uint32_t)g.k) st.fault |= 2u;
    state[p] = st;
    if (meta_out) {
      meta_out[p] = st.kth;
      meta_out[g.P + p] = st.lo_next;
      meta_out[2 * g.P + p] = st.fault;
    }
  }
}

// Position of the r-th set bit (from 0) of a word with more than r set bits.
// Each wave takes emit_tiles(RANKS) consecutive tiles (with the loads they
// need issued together), and for each completes the tile's mask words and writes
// its global indices in order.  The threshold bin's candidates of the tile
// at or above
// T (the resolved threshold composite) are assembled in LDS and ORed into
// the words (written back only where bits were added; this wave is the only
// writer of its tile's words).  Then, with the tile's offset:
// RANKS false (sparse masks): each lane walks the set bits of its own word.
// RANKS true (denser masks, where a lane's word holds several indices): the
// lanes write their indices into an LDS list at their ranks, and the wave
// copies it out with consecutive lanes on consecutive entries of the index
// list.
template <bool RANKS>
__global__ void __launch_bounds__(kThreads)
emit_kernel(Geom g, const PartSel* __restrict__ state, const uint32_t* __restrict__ cand,
            const uint32_t* __restrict__ cnt2, uint64_t* __restrict__ bits,
            const uint32_t* __restrict__ tile_off, uint32_t* __restrict__ idx) {
  __shared__ unsigned long long swords[kThreads / 64][kWordsPerTile];
  __shared__ uint32_t slist[RANKS ? kThreads / 64 : 1][RANKS ? kEmitList : 1];
  constexpr int ET = emit_tiles(RANKS);
  const int p = g.sp0 + blockIdx.y;
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  // the wave's tiles tw .. tw + ET - 1
  const int64_t tw = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * ET;
  if (tw >= g.tpp) return;  // wave-uniform; the waves synchronise only among their own lanes
  unsigned long long* wd = swords[wave];
  uint64_t* wb = bits + (int64_t)p * g.wpp;
  uint32_t* out = idx + (int64_t)p * g.k;
  const uint64_t T = state[p].prefix;
  const uint32_t hi = state[p].bin1 << kL1Shift;
  // Every load the wave's tiles need before their words are complete is
  // issued up front: the words, the candidate counts and offsets (lane j:
  // tile j), then the first 64 candidates of each tile.
  uint64_t words[ET];
#pragma unroll
  for (int j = 0; j < ET; ++j) {
    const int64_t w = (tw + j) * kWordsPerTile + lane;
    words[j] = (tw + j < g.tpp && w < g.wpp) ? wb[w] : 0ull;
  }
  // one tile: wave-uniform (scalar) loads; several: lane j loads tile j's
  const int64_t tl = tw + (ET == 1 ? 0 : lane);
  const bool lt = (ET == 1 || lane < (uint32_t)ET) && tl < g.tpp;
  uint32_t ctl = lt ? cnt2[(int64_t)p * g.tpp + tl] : 0u;
  if (ctl > (uint32_t)kTile) ctl = (uint32_t)kTile;  // a slot holds at most one tile
  const uint32_t bl = lt ? tile_off[(int64_t)p * g.tpp + tl] : 0u;
  auto of_tile = [&](uint32_t v, int j) { return ET == 1 ? v : (uint32_t)__shfl((int)v, j, 64); };
  uint32_t c0[ET];
#pragma unroll
  for (int j = 0; j < ET; ++j) {
    const uint32_t ct = of_tile(ctl, j);
    const uint32_t* ent = cand + ((int64_t)p * g.tpp + tw + j) * kSlotWords;
    c0[j] = (lane < ct) ? ent[lane] : 0u;
  }
  // Wait for these loads here, once, before the first store: a wait placed
  // between the tiles would also wait for the stores of the tiles before.
#pragma unroll
  for (int j = 0; j < ET; ++j) asm volatile("" ::"v"(words[j]), "v"(c0[j]));
  asm volatile("" ::"v"(bl));
#pragma unroll
  for (int j = 0; j < ET; ++j) {
    const int64_t t = tw + j;
    if (t >= g.tpp) break;  // wave-uniform
    const int64_t w = t * kWordsPerTile + lane;
    const uint32_t ct = of_tile(ctl, j);
    const int64_t base = (int64_t)of_tile(bl, j);
    uint64_t word = words[j];
    if (ct) {  // wave-uniform
      wd[lane] = 0ull;
      wave_lds_sync();
      const uint32_t* ent = cand + ((int64_t)p * g.tpp + t) * kSlotWords;
      const uint32_t tile_lo = (uint32_t)(t * kTile);
      auto take = [&](uint32_t e) {
        const uint32_t jl = e & (uint32_t)(kTile - 1);
        if (bin_composite(e, hi, tile_lo, g.idx_mask) >= T) atomicOr(&wd[jl >> 6], 1ull << (jl & 63));
      };
      if (lane < ct) take(c0[j]);
      if (ct > 64u) for_each_entry(ent + 64, ct - 64u, lane, take);  // wave-uniform
      wave_lds_sync();
      const uint64_t add = wd[lane];
      if (add && w < g.wpp) {
        word |= add;
        wb[w] = word;
      }
      wave_lds_sync();
    }
    const uint32_t c = (uint32_t)__popcll(word);
    uint32_t x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(x, d, 64);
      if ((int)lane >= d) x += y;
    }
    if (!RANKS) {
      int64_t pos = base + (x - c);
      const uint32_t jbase = (uint32_t)((int64_t)p * g.n_p + w * 64);
      while (word) {
        if (pos < g.k) out[pos] = jbase + (uint32_t)__builtin_ctzll(word);  // bound: malformed mask
        ++pos;
        word &= word - 1ull;
      }
      continue;
    }
    // Denser masks: the lanes write their words' indices into the wave's
    // LDS list at their ranks, kEmitList ranks a round, and the wave copies
    // each round's list out with consecutive lanes on consecutive entries.
    uint32_t* sl = slist[RANKS ? wave : 0u];
    const uint32_t total = (uint32_t)__shfl((int)x, 63, 64);
    const uint32_t first = x - c;  // rank of this lane's first index
    const uint32_t jbase = (uint32_t)((int64_t)p * g.n_p + w * 64);
    for (uint32_t r0 = 0; r0 < total; r0 += kEmitList) {  // wave-uniform
      uint64_t wv = word;
      uint32_t r = first;
      if (first + c > r0 && first < r0 + kEmitList) {
        for (; wv && r < r0; ++r) wv &= wv - 1ull;  // ranks of earlier rounds
        for (; wv && r < r0 + kEmitList; ++r) {
          sl[r - r0] = jbase + (uint32_t)__builtin_ctzll(wv);
          wv &= wv - 1ull;
        }
      }
      wave_lds_sync();
      const uint32_t cnt = (total - r0 < (uint32_t)kEmitList) ? total - r0 : (uint32_t)kEmitList;
      for (uint32_t i = lane; i < cnt; i += 64)
        if (base + r0 + i < g.k) out[base + r0 + i] = sl[i];  // bound: malformed mask
      wave_lds_sync();  // the next round or tile rewrites the list
    }
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

}  // namespace

uint32_t capture_target(const Geom& g) {
  double t = kCaptureMargin * (double)g.k;
  if (t > (double)g.n_p) t = (double)g.n_p;
  return (uint32_t)(t + 0.5);
}

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  zero_u32_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(p, count);
  return hipGetLastError();
}

hipError_t launch_init_state(const Geom& g, const SelectBufs& w, hipStream_t s) {
  if (g.snp < 1) return hipSuccess;
  init_state_kernel<<<(g.snp + kThreads - 1) / kThreads, kThreads, 0, s>>>(w.state, w.arrive, g.sp0, g.snp,
                                                                            (uint32_t)g.k);
  return hipGetLastError();
}

hipError_t launch_level1(const Geom& g, const SelectBufs& w, int mode, hipStream_t s, uint32_t target) {
  if (g.snp < 1) return hipSuccess;
  level_scan_kernel<<<g.snp, kThreads, 0, s>>>(g, w.hist, w.state, w.arrive, mode,
                                               target ? target : capture_target(g));
  return hipGetLastError();
}

hipError_t launch_select_tail(const Geom& g, const SelectBufs& w, uint64_t* bits, uint32_t* idx,
                              uint32_t* tile_off, uint32_t* meta_out, hipStream_t s,
                              void (*mark)(void*, int), void* ctx) {
  if (g.snp < 1) return hipSuccess;
  // tiles per wave of the passes over candidate slots: kSelectTilesPerWave
  // on large layouts, fewer where that would leave too few waves
  int64_t tpw = ((int64_t)g.snp * g.tpp + kSelectWaves - 1) / kSelectWaves;
  tpw = tpw < 1 ? 1 : (tpw > kSelectTilesPerWave ? kSelectTilesPerWave : tpw);
  const unsigned sblocks = (unsigned)((g.tpp + 4 * tpw - 1) / (4 * tpw));
  if (g.hparts) {
    cand_select_kernel<false><<<dim3(sblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt1, w.cnt2, w.hist,
                                                                       bits, w.tilecnt);
    l2_hist_kernel<<<dim3(g.hparts, g.snp), kHistThreads, 0, s>>>(g, w.cand, w.cnt2, w.part);
  } else {
    cand_select_kernel<true><<<dim3(sblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt1, w.cnt2, w.hist,
                                                                      bits, w.tilecnt);
  }
  if (mark) mark(ctx, 1);
  if (g.hparts)
    l2_scan_kernel<true><<<g.snp, kThreads, 0, s>>>(g, w.hist, w.part, w.state, w.nsurv, capture_target(g));
  else
    l2_scan_kernel<false><<<g.snp, kThreads, 0, s>>>(g, w.hist, w.part, w.state, w.nsurv, capture_target(g));
  // rank-parallel emission, and the per-tile bin walk, pay from a mask
  // density of about 5% on (many candidates per tile)
  const bool ranks = g.k * 20 >= g.n_p;
  // the bin walk flattens a wave's tiles at sparser masks, where it takes
  // up to kFlatTilesPerWave of them
  int64_t wpw = tpw;
  if (!ranks) {
    wpw = ((int64_t)g.snp * g.tpp + kSelectWaves - 1) / kSelectWaves;
    wpw = wpw < 1 ? 1 : (wpw > kFlatTilesPerWave ? kFlatTilesPerWave : wpw);
  }
  const unsigned wblocks = (unsigned)((g.tpp + 4 * wpw - 1) / (4 * wpw));
  if (!ranks && wpw > 1)
    bin_walk_kernel<true><<<dim3(wblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt2, w.tilecnt, w.hist,
                                                                    w.surv, w.nsurv);
  else
    bin_walk_kernel<false><<<dim3(wblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt2, w.tilecnt, w.hist,
                                                                     w.surv, w.nsurv);
  finish_kernel<<<g.snp, kResolveThreads, 0, s>>>(g, w.hist, w.state, w.cand, w.cnt2, w.surv, w.nsurv, w.tilecnt,
                                                tile_off, meta_out);
  if (mark) mark(ctx, 2);
  const int et = 4 * emit_tiles(ranks);  // tiles per block
  const unsigned tblocks = (unsigned)((g.tpp + et - 1) / et);
  if (ranks)
    emit_kernel<true><<<dim3(tblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt2, bits, tile_off, idx);
  else
    emit_kernel<false><<<dim3(tblocks, g.snp), kThreads, 0, s>>>(g, w.state, w.cand, w.cnt2, bits, tile_off, idx);
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
