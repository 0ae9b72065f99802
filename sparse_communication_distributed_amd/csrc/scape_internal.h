// Internal declarations of libscape: geometry of the flat buffer, mask slots
// and workspace, and the launch wrappers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "scape.h"

namespace scape {

// Compaction / work tile: 4096 elements = 64 mask words.
constexpr int64_t kTile = 4096;
constexpr int kWordsPerTile = 64;
// A tile's candidate slot, in 32-bit words: the captured keys u32[kTile],
// then their offsets in the tile u16[kTile].  After the candidate select
// pass, the keys' place holds the threshold bin's 32-bit entries.
constexpr int64_t kSlotWords = kTile + kTile / 2;
// Radix digit width and histogram size for the threshold search.
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
// Level-1 digit: key bits [30:19] (bit 31 of a key is always zero).
constexpr int kL1Shift = 19;
// The step pass and the compression run one block per tile (grid: tiles x
// partitions): the hardware dispatcher then balances tiles of uneven cost
// (dense mask or capture regions) across the 256 CUs, and no block holds
// the end of the pass back by more than one tile.
// Target number of blocks of the statistic passes (the bootstrap, and the
// fallback, which usually has nothing to do and should cost little).
constexpr int kStatBlocks = 8192;
// Tiles each wave of the passes over candidate slots walks, at most; fewer
// where the layout has fewer than kSelectWaves * kSelectTilesPerWave tiles.
constexpr int kSelectTilesPerWave = 8;
constexpr int64_t kSelectWaves = 8192;
constexpr int kThreads = 256;
// At sparse masks on such layouts, the level-2 histogram of the threshold
// bin has a pass of its own: about kHistBlocks blocks in all, each writing
// its partial histogram with plain stores.  (Merged with atomics by every
// block of the candidate select pass, it costs millions of device-scope
// atomics per step at the largest layouts.)
constexpr int kHistBlocks = 512;

// Statistic sources and phases of stat_kernel.
constexpr int kSrcStat = 0;    // key of a given array
constexpr int kSrcState = 1;   // b1*m + c1*(g^o + e^o), before compression
constexpr int kSrcMasked = 2;  // b1*m + c1*a^o, a^o rebuilt from e' and b^o
constexpr int kPhaseHist = 0;
constexpr int kPhaseCapture = 1;

// Modes of the level-1 scan.
constexpr int kScanCheck = 1;  // level 1 on captured keys; flags a fallback if fewer than k
constexpr int kScanBound = 2;  // fallback: level 1 on all keys -> capture bound
constexpr int kScanFinal = 3;  // fallback: level 1 on the recaptured keys
constexpr int kScanSample = 4;  // level 1 on a sample of tiles -> capture bound for a first capture

// Per-partition state of the threshold search.  The search runs on the
// 64-bit composite  c = (key << 32) | (idx_mask - local_index),  unique per
// element, so "k largest composites" is exactly "k largest keys, ties to the
// lower index".  `prefix` holds the determined high bits of the k-th largest
// composite (undetermined bits zero); an element is selected iff c >= prefix
// once the search ends.
struct PartSel {
  uint64_t prefix;
  uint64_t mask;   // bits of prefix that are determined
  uint32_t r;      // rank still needed among composites matching prefix
  uint32_t done;   // 1: every composite matching prefix is selected
  uint32_t bin1;   // level-1 digit of the threshold
  uint32_t fault;  // bit 0: rank not found; bit 1: emitted count != k (recorded in the slot's meta)
  uint32_t fb;     // 1: the captured candidates cannot hold the top k
  uint32_t lo_fb;  // capture bound of the fallback (lowest key of bin1)
  uint32_t kth;      // smallest selected key (the k-th largest key)
  uint32_t c1;       // captured keys in the level-1 threshold bin
  uint32_t lo_next;  // capture bound proposed for the next step
  uint32_t bin2;     // level-2 digit of the threshold (once level 2 is resolved)
  uint32_t done2;    // 1: every candidate at the level-2 digit is selected
  uint32_t pad;
};

// The next step's capture bound sits where this step counted
// kCaptureMargin * k keys at or above it (first on the level-1 digit, then
// refined inside the threshold bin on the level-2 digit).
constexpr double kCaptureMargin = 1.25;
// A first capture (no previous bound) estimates its bound from every
// kSampleStep-th tile, aiming at kSampleMargin * k keys above it.
constexpr int kSampleStep = 16;
constexpr double kSampleMargin = 1.5;
// Candidates of the threshold bin that still match the prefix after level 2
// (ties and near-ties at the threshold): at most this many are kept per
// partition for the later levels; beyond it those levels walk the tile
// slots again (exact, slower).
constexpr int kSurvivorCap = 4096;

struct Level {
  int shift;  // bit position of the digit in the composite
  int nbits;  // digit width (<= kDigitBits)
};

struct Geom {
  int64_t n, n_p, k;
  int P, K;
  int64_t wpp;        // mask words per partition
  int64_t tpp;        // tiles per partition
  int G;              // blocks per partition of the streaming step pass
  int Gs;             // blocks per partition of the statistic passes
  int idx_bits;       // bits of (n_p - 1), >= 1
  uint32_t idx_mask;  // (1 << idx_bits) - 1
  int nlevels;        // levels after level 1 (level 2 first)
  int sp0, snp;       // partitions the selection kernels work on: [sp0, sp0 + snp)
  int hparts;         // level-2 histogram parts per partition (0: merged by the select pass)
  Level levels[8];
  // mask slot: offsets inside one slot, slot size
  size_t off_bits, off_idx, off_toff, off_meta, slot_bytes;
  // workspace offsets and total
  size_t ws_b, ws_mold, ws_hist, ws_cand, ws_cnt1, ws_cnt2, ws_state, ws_tilecnt, ws_surv, ws_nsurv, ws_arrive,
      ws_part, ws_total;
};

// Returns false if dims/k are outside the limits.
bool make_geom(int64_t n, int P, int K, int64_t k, Geom* g);

struct StatArgs {
  PartSel* state;
  int only_fb;
  const float* stat;
  const float* m;
  const float* grads;
  const float* e;
  const float* b;
  const float* mold;  // m_{t-1} of the masked elements, by rank (SRC masked)
  const uint64_t* bits;
  const uint32_t* tile_off;
  float b1, c1;
  uint32_t* cand;  // candidate slots, kSlotWords per tile
  uint32_t* cnt1;
  uint32_t* hist;
  int tile_step;  // visit tiles 0, tile_step, 2*tile_step, ... (a sample when > 1)
  bool single_row;  // grads, e, b are the owner's rows alone (a rank's share), not [K] rows
  // The fallback's passes (only_fb): after a partition's blocks have all
  // merged their histograms, the last to arrive runs level 1 in this mode
  // (kScanBound or kScanFinal; 0: none) with `target`, counting arrivals in
  // arrive[p] (zero before the pass, and left zero).
  int then_mode;
  uint32_t target;
  uint32_t* arrive;
};

// Buffers of the selection pipeline (workspace views).
struct SelectBufs {
  uint32_t* hist;
  uint32_t* cand;  // candidate slots, kSlotWords per tile
  uint32_t* cnt1;
  uint32_t* cnt2;
  PartSel* state;
  uint32_t* tilecnt;  // [P][tiles] selected elements per tile
  uint64_t* surv;     // [P][kSurvivorCap] candidates at the level-2 threshold digit
  uint32_t* nsurv;    // [P] their counts
  uint32_t* arrive;   // [P] blocks arrived in a fallback pass
  uint32_t* part;     // [P][hparts][kBins] level-2 histogram parts
};

// ---- launch wrappers (each returns hipGetLastError() of its launches) ----

// Arguments of the fused step pass.
struct StepArgs {
  const float* grads;
  float* e;
  const uint64_t* bits;      // M_t
  const uint32_t* tile_off;  // M_t
  float* b;                  // [K][P*k] sparse buffers
  float *m, *v, *w;
  float* mold;               // [P*k] pre-update m of the masked elements
  float b1, b2, c1, c2, ibc1, ibc2, eps, wd, lr;
  const uint32_t* lo;        // [P] capture bounds
  uint32_t* cand;  // candidate slots, kSlotWords per tile
  uint32_t* cnt1;
  uint32_t* hist;
  int p0, nparts;            // partitions of this launch
  int64_t e_stride;          // elements between the worker rows of e
  const float* ibc_dev;      // if set: ibc1, ibc2 read from device memory here
};

hipError_t launch_stat(const Geom& g, int src, int phase, const StatArgs& a, bool vec, hipStream_t s);
// Error-feedback compression at a mask (the component call).
hipError_t launch_compress(const Geom& g, const float* grads, float* e, const uint64_t* bits,
                           const uint32_t* tile_off, float* b, hipStream_t s, bool vec);
// The fused step pass: compression, owner statistic with candidate capture,
// worker-sum reduction and AdamS at M_t.
// seg: w, m, v rows 64-byte aligned and n_p % 16 == 0 (whole-segment AdamS writes)
hipError_t launch_step_pass(const Geom& g, const StepArgs& a, bool vec, bool seg, hipStream_t s);
// The step over the resident buffers (all partitions, p0 = 0), as the
// single pass above or, where multi_pass_pays(g), as K passes: K - 1 passes
// each compress one non-owner worker per partition into its sparse buffer,
// then the owner pass (statistic, capture, worker sum from the sparse
// buffers in worker order, AdamS).  Both forms give the same results, bit
// for bit.
bool multi_pass_pays(const Geom& g);
// One rank's pass of the sharded step: compression of the rank's rows
// (grads, e: [n]; b: [P*k]) over every partition, statistic and capture on
// the partitions the rank owns.
hipError_t launch_shard_pass(const Geom& g, int rank, const float* grads, float* e, const uint64_t* bits,
                             const uint32_t* tile_off, float* b, const float* m, float b1, float c1,
                             const uint32_t* lo, uint32_t* cand, uint32_t* cnt1, uint32_t* hist, bool vec,
                             hipStream_t s);
hipError_t launch_step_passes(const Geom& g, const StepArgs& a, bool vec, bool seg, hipStream_t s);

hipError_t launch_init_state(const Geom& g, const SelectBufs& w, hipStream_t s);
// kCaptureMargin * k, at most n_p.
uint32_t capture_target(const Geom& g);
// target 0: the capture target of a step (kCaptureMargin * k)
hipError_t launch_level1(const Geom& g, const SelectBufs& w, int mode, hipStream_t s, uint32_t target = 0);
// From level-1 digits to the mask: candidate select pass (writes every mask
// word, counts each tile's selection, compacts the threshold bin's
// candidates), level 2, a pass over the bin's candidates (tile counts, the
// next histogram, the few candidates left at the threshold digit), the
// later levels and the tile offsets, and the emission (the bin's selected
// candidates ORed into the words, the index list), plus the slot's
// threshold record.
hipError_t launch_select_tail(const Geom& g, const SelectBufs& w, uint64_t* bits, uint32_t* idx,
                              uint32_t* tile_off, uint32_t* meta_out, hipStream_t s,
                              void (*mark)(void*, int), void* mark_ctx);

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s);

hipError_t launch_reduce(const Geom& g, const float* b, float* bbar, hipStream_t s);
// AdamS at idx[0 .. count) with x = bbar[0 .. count) (count < 0: all P*k entries).
hipError_t launch_adams(const Geom& g, const float* bbar, const uint32_t* idx, float* w, float* m,
                        float* v, float b1, float b2, float c1, float c2, float ibc1, float ibc2,
                        float eps, float wd, float lr, hipStream_t s, int64_t count = -1);
// Advances the device-resident bias-correction state by one step.
hipError_t launch_bias_step(scape_bias_state* st, float b1, float b2, hipStream_t s);
hipError_t launch_dense_adams(const Geom& g, const float* grads, float* w, float* m, float* v, float b1,
                              float b2, float c1, float c2, float ibc1, float ibc2, float eps, float wd,
                              float lr, bool vec, hipStream_t s);
// Reason bits of the mask check, per partition.
constexpr uint32_t kMaskBadFault = 1;  // the selection's fault word is set
constexpr uint32_t kMaskBadCount = 2;  // bit count != k, or tile offsets off
constexpr uint32_t kMaskBadIdx = 4;    // index list off the bits, out of order or range
constexpr uint32_t kMaskBadPad = 8;    // bits set past n_p
// res: u32[P], per-partition reason bits (zeroed first).
hipError_t launch_mask_check(const Geom& g, const uint64_t* bits, const uint32_t* idx, const uint32_t* tile_off,
                             const uint32_t* meta, uint32_t* res, hipStream_t s);
hipError_t launch_union(const Geom& g, uint64_t* acc, const uint64_t* m, uint64_t* out, hipStream_t s);
// *out += the number of NaN and +-inf values among x[0 .. n-1].
hipError_t launch_count_nonfinite(const float* x, int64_t n, uint64_t* out, hipStream_t s);
hipError_t launch_overlap(const Geom& g, const uint64_t* a, const uint64_t* b, uint64_t* out,
                          hipStream_t s);

}  // namespace scape
