// Internal declarations of libscape: geometry of the flat buffer, mask slots
// and workspace, and the launch wrappers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace scape {

// Compaction / work tile: 4096 elements = 64 mask words.
constexpr int64_t kTile = 4096;
constexpr int kWordsPerTile = 64;
// Radix digit width and histogram size for the threshold search.
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
// Level-1 digit: key bits [30:19] (bit 31 of a key is always zero).
constexpr int kL1Shift = 19;
// Target number of blocks for streaming passes (>> 256 CUs).
constexpr int kTargetBlocks = 4096;
// Blocks per partition for the passes over candidate lists.
constexpr int kRefineBlocks = 16;
constexpr int kThreads = 256;

// Per-partition state of the threshold search.  The search runs on the
// 64-bit composite  c = (key << 32) | (idx_mask - local_index),  unique per
// element, so "k largest composites" is exactly "k largest keys, ties to the
// lower index".  `prefix` holds the determined high bits of the k-th largest
// composite (undetermined bits zero); an element is selected iff c >= prefix
// once the search ends.
struct PartSel {
  uint64_t prefix;
  uint64_t mask;    // bits of prefix that are determined
  uint32_t r;       // rank still needed among composites matching prefix
  uint32_t done;    // 1: every composite matching prefix is selected
  uint32_t bin1;    // level-1 digit of the threshold
  uint32_t fault;   // 1: rank not found (internal invariant broken)
};

struct Level {
  int shift;  // bit position of the digit in the composite
  int nbits;  // digit width (<= kDigitBits)
};

struct Geom {
  int64_t n, n_p, k;
  int P, K;
  int64_t wpp;        // mask words per partition
  int64_t tpp;        // tiles per partition
  int G;              // blocks per partition of the streaming passes
  int64_t seg_tiles;  // tiles handled by one streaming block (upper bound)
  int64_t seg_cap;    // candidate capacity of one block segment
  int R;              // blocks per partition over candidate lists
  int idx_bits;       // bits of (n_p - 1), >= 1
  uint32_t idx_mask;  // (1 << idx_bits) - 1
  int nlevels;        // levels after level 1
  Level levels[8];
  // mask slot: offsets inside one slot, slot size
  size_t off_bits, off_idx, off_toff, slot_bytes;
  // workspace offsets and total
  size_t ws_keys, ws_b, ws_hist, ws_segcnt, ws_cand, ws_state, ws_tilecnt, ws_total;
};

// Returns false if dims/k are outside the limits.
bool make_geom(int64_t n, int P, int K, int64_t k, Geom* g);

// ---- launch wrappers (each returns hipGetLastError() of its launches) ----

// Keys + level-1 histogram from a statistic array: key = bits(stat) & 0x7fffffff.
hipError_t launch_keys_from_stat(const Geom& g, const float* stat, uint32_t* keys, uint32_t* hist,
                                 bool vec, hipStream_t s);
// Keys + level-1 histogram from the statistic b1*m + c1*(g^o + e^o) (step-1 bootstrap).
hipError_t launch_keys_from_state(const Geom& g, const float* m, const float* grads, const float* e,
                                  float b1, float c1, uint32_t* keys, uint32_t* hist, bool vec,
                                  hipStream_t s);
// Error-feedback compression at a mask; optionally fused owner statistic.
hipError_t launch_compress(const Geom& g, const float* grads, float* e, const uint64_t* bits,
                           const uint32_t* tile_off, float* b, bool stat, const float* m, float b1,
                           float c1, uint32_t* keys, uint32_t* hist, bool vec, hipStream_t s);

// Selection pipeline: level-1 threshold from hist, select pass, candidate
// levels, marking and emission of idx / tile_off.  hist must hold the
// level-1 histogram of keys; it is left zeroed.
hipError_t launch_select(const Geom& g, const uint32_t* keys, uint32_t* hist, uint32_t* segcnt,
                         uint64_t* cand, PartSel* state, uint32_t* tilecnt, uint64_t* bits,
                         uint32_t* idx, uint32_t* tile_off, hipStream_t s,
                         void (*mark)(void*, int), void* mark_ctx);

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s);

hipError_t launch_reduce(const Geom& g, const float* b, float* bbar, hipStream_t s);
hipError_t launch_adams(const Geom& g, const float* bbar, const uint32_t* idx, float* w, float* m,
                        float* v, float b1, float b2, float c1, float c2, float ibc1, float ibc2,
                        float eps, float wd, float lr, hipStream_t s);
hipError_t launch_reduce_adams(const Geom& g, const float* b, const uint32_t* idx, float* w,
                               float* m, float* v, float b1, float b2, float c1, float c2,
                               float ibc1, float ibc2, float eps, float wd, float lr,
                               hipStream_t s);
hipError_t launch_overlap(const Geom& g, const uint64_t* a, const uint64_t* b, uint64_t* out,
                          hipStream_t s);

}  // namespace scape
