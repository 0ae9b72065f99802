// Level 1 of the threshold search on one partition's level-1 histogram,
// shared by its own kernel and by the exact fallback's statistic passes
// (whose last block per partition runs it), and the block helpers it uses.
#pragma once

#include "scape_internal.h"

namespace scape {

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

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
  s.kth = 0xffffffffu; s.c1 = 0; s.lo_next = 0; s.bin2 = 0; s.done2 = 0; s.pad = 0;
  return s;
}

// Level 1 of the threshold search for partition p, on its level-1
// histogram h (key bits 30..19; global or LDS; see kScan* for the modes),
// by a block of kThreads: find the digit (scanning from the largest) whose
// bin holds the k-th largest key, and record the capture bound of the next
// step (the digit at which the count from the top reaches `target`).  The
// caller zeroes the bins afterwards.
__device__ __forceinline__ void level1_block(const Geom& g, int p, const uint32_t* h, PartSel* __restrict__ state,
                                             int mode, uint32_t target) {
  __shared__ uint32_t wtot[kThreads / 64];
  __shared__ int found;
  __shared__ uint32_t s_lo;
  __shared__ int s_dmin;
  constexpr int nb = kBins;
  constexpr int shift = 32 + kL1Shift;
  const PartSel cur = state[p];
  const bool active = (mode == kScanCheck) || cur.fb != 0;  // the other modes: fallback partitions only
  const PartSel st = fresh_sel((uint32_t)g.k);
  constexpr int per = (nb + kThreads - 1) / kThreads;
  if (active && mode == kScanSample) {
    // The bound for a first capture: the digit at which the count of the
    // sampled keys from the top reaches `target` (scaled to the sample), or
    // 0 (capture every key) if the sample holds fewer.
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) s += h[nb - 1 - (threadIdx.x * per + q)];
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0 && tot < target) state[p].lo_fb = 0u;
    if (tot >= target && above < target && target <= above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int d = nb - 1 - (threadIdx.x * per + q);
        acc += h[d];
        if (acc >= target) {
          state[p].lo_fb = (uint32_t)d << kL1Shift;
          break;
        }
      }
    }
  } else if (active) {
    // thread t owns descending positions [t*per, (t+1)*per): bin = nb-1-pos
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) s += h[nb - 1 - (threadIdx.x * per + q)];
    uint32_t tot;
    const uint32_t above = block_excl_scan(s, wtot, &tot);
    if (threadIdx.x == 0) {
      found = 0;
      s_lo = 0xffffffffu;
      s_dmin = nb;
    }
    __syncthreads();
    // Capture bound for the next step: the digit at which the count of keys
    // from the top reaches the target.
    const bool bound = (mode == kScanCheck || mode == kScanFinal);
    const int64_t need = bound ? ((tot >= target) ? (int64_t)target : -2) : -1;
    if (need >= 1 && above < (uint64_t)need && (uint64_t)need <= (uint64_t)above + s) {
      uint32_t acc = above;
      for (int q = 0; q < per; ++q) {
        const int d = nb - 1 - (threadIdx.x * per + q);
        acc += h[d];
        if (acc >= (uint32_t)need) {
          s_lo = (uint32_t)d << kL1Shift;
          break;
        }
      }
    }
    if (need == -2) {
      // fewer keys than the target were captured: one bin below the lowest
      // captured digit
      for (int q = per - 1; q >= 0; --q) {
        const int pos = threadIdx.x * per + q;
        if (h[nb - 1 - pos]) {
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
        const int d = nb - 1 - (threadIdx.x * per + q);
        const uint32_t c = h[d];
        if (acc + c >= st.r) {
          if (mode == kScanBound) {
            state[p].lo_fb = (uint32_t)d << kL1Shift;
          } else {
            PartSel o = st;
            o.r = st.r - acc;
            o.prefix = (uint64_t)d << shift;
            o.mask = ((uint64_t)(nb - 1) << shift) | (1ull << 63);  // bit 63 of every composite is zero
            o.done = (c == o.r) ? 1u : 0u;
            o.bin1 = (uint32_t)d;
            o.c1 = c;
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
      state[p].fault = cur.fault | 1u;
      state[p].done = 1u;
      state[p].fb = 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0 && bound) state[p].lo_next = (s_lo == 0xffffffffu) ? 0u : s_lo;
  }
}

}  // namespace scape
