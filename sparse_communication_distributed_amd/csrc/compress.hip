// Streaming passes over the flat buffer.
//
//  * compress_kernel: error-feedback compression of every worker's gradient
//    at the current mask (SCAPE paper §II-B, at the shared index set of the
//    technical summary §2), fused with the owner's first-moment statistic
//    (technical summary §2, lagged mask built from first-moment statistics)
//    and the capture of the selection candidates: owner keys at or above a
//    per-partition bound `lo` are written, each with its offset in the tile
//    (key and offset identify the element), to a per-tile candidate slot,
//    and a level-1 histogram of the captured keys is kept.  The step runs it as one pass over all
//    workers, or as one pass per non-owner worker followed by the owner's
//    pass (MODE below).
//  * stat_kernel: the statistic alone, for the step-1 bootstrap (from
//    m, g^o, e^o), for scape_mask_topk (from a given array), and for the
//    exact fallback when a partition captured fewer than k candidates (from
//    m and the compressed state e', b of the owner).  Phase HIST counts every
//    key; phase CAPTURE captures keys at or above the partition's bound.
//
// Work decomposition: grid (G, P).  Block (b, p) walks tiles b, b+G, ... of
// partition p (the step pass has G = tiles per partition, one tile per
// block); a tile is 4096 elements = 64 mask words; thread `tid` owns
// elements 4*tid .. 4*tid+3 of each 1024-element chunk, so every global
// access is a 16-byte-per-lane coalesced load or store when vector access
// is possible (n_p % 4 == 0 and 16-byte aligned bases).
#include "level1.h"

#pragma clang fp contract(off)

namespace scape {
namespace {

__device__ __forceinline__ uint32_t stat_key(float m, float a, float b1, float c1) {
  // s = (b1*m) + (c1*a), each operation rounded on its own; key = |s| bits.
  const float s = (b1 * m) + (c1 * a);
  return __float_as_uint(s) & 0x7fffffffu;
}

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Streaming accesses are non-temporal: every byte of g, e and m is touched
// once per pass, and keeping them out of the caches leaves those to the
// scattered w / m / v updates and the candidate slots.
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load4(const float* p, int64_t lj, int64_t n_p, bool vec, float out[4]) {
  if (vec) {
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p + lj));
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = (lj + q < n_p) ? p[lj + q] : 0.0f;
  }
}

__device__ __forceinline__ void store4(float* p, int64_t lj, int64_t n_p, bool vec, const float v[4]) {
  if (vec) {
    const v4f t = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f*>(p + lj));
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lj + q < n_p) p[lj + q] = v[q];
  }
}

// Ordinary (cached) 16-byte access to elements o .. o+3 of a 16-byte-aligned row.
__device__ __forceinline__ void load4t(const float* p, uint32_t o, float out[4]) {
  const v4f t = *reinterpret_cast<const v4f*>(p + o);
  out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
}

__device__ __forceinline__ void store4t(float* p, uint32_t o, const float v[4]) {
  *reinterpret_cast<v4f*>(p + o) = v4f{v[0], v[1], v[2], v[3]};
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

// Loads the tile's 64 mask words into LDS with their exclusive popcount
// prefix (wave 0 scans).
__device__ __forceinline__ void load_tile_words(const uint64_t* __restrict__ bits, int64_t wbase,
                                                int64_t wpp, int64_t t, uint64_t* sw, uint32_t* spre) {
  if (threadIdx.x < kWordsPerTile) {
    const int64_t w = t * kWordsPerTile + threadIdx.x;
    const uint64_t word = (w < wpp) ? bits[wbase + w] : 0ull;
    sw[threadIdx.x] = word;
    uint32_t c = (uint32_t)__popcll(word);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(c, d, 64);
      if ((int)threadIdx.x >= d) c += y;
    }
    spre[threadIdx.x] = c - (uint32_t)__popcll(word);
  }
}

// Wave-cooperative capture of the lane's 4 keys (elements lj .. lj+3 of
// the partition): flagged keys are appended to the tile's candidate slot,
// the key and its offset in the tile at positions handed out by the LDS
// counter `tcnt`, and counted in the LDS histogram.  Every lane of the wave
// must call this (ballots and a lane-0 broadcast).
__device__ __forceinline__ void capture4(const uint32_t kk[4], const bool f[4], uint32_t lj,
                                         uint32_t* __restrict__ slot, uint32_t* tcnt, uint32_t* sh) {
  uint64_t B[4];
  uint32_t pre[4], tot = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    B[q] = __ballot(f[q]);
    pre[q] = tot;
    tot += (uint32_t)__popcll(B[q]);
  }
  if (tot == 0) return;  // wave-uniform
  uint32_t base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(tcnt, tot);
  base = __shfl(base, 0, 64);
  uint16_t* offs = reinterpret_cast<uint16_t*>(slot + kTile);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (f[q]) {
      const uint32_t pos = base + pre[q] + mbcnt(B[q]);
      slot[pos] = kk[q];
      offs[pos] = (uint16_t)((lj + q) & (uint32_t)(kTile - 1));
      atomicAdd(&sh[kk[q] >> kL1Shift], 1u);
    }
  }
}

// The lanes that write this lane's 64-byte line of w / m / v as one
// segment.  A line is 4 lanes x 4 elements; where the partition's first
// element is not 16-aligned, the lines start `sl` lanes before the
// partition's 4-lane groups (sl = (partition base mod 16) / 4).  A line that
// crosses the wave's 256 elements is written by each of its lanes alone.
__device__ __forceinline__ uint64_t seg_lanes(uint32_t lane, uint32_t sl) {
  const int l0 = (int)((lane + sl) & ~3u) - (int)sl;
  return (l0 >= 0 && l0 <= 60) ? (0xfull << l0) : (1ull << lane);
}

// Grid of the streaming passes: (G, partitions); the dispatcher fills the
// device partition by partition, G blocks each.
__device__ __forceinline__ int block_part() { return blockIdx.y; }
__device__ __forceinline__ int block_in_part() { return blockIdx.x; }
__device__ __forceinline__ int blocks_per_part() { return gridDim.x; }
inline dim3 stream_grid(int nparts, int G) { return dim3(G, nparts); }

struct AdamsC {
  float b1, b2, c1, c2, ibc1, ibc2, eps, wd, lr, invK;
};

// STEP false: error-feedback compression only (the component call).
// STEP true: the fused step pass.  Besides compressing, it keeps each masked
// element's worker sum S = ((a^0 + a^1) + ...) + a^{K-1} in registers (the
// single synchronised buffer of the technical summary §2: on one device all
// K workers' entries of an element are in the same thread), so of the
// sparse buffers only the owner's is written (the exact recount of the
// selection rebuilds the owner's a from it), applies AdamS
// there with x = S * fp32(1/K) (SCAPE paper §II-C eq. (2)), and saves the
// pre-update m of masked elements to mold[rank] for the exact fallback;
// the owner's statistic reads m before its update.
// Chunks of 1024 elements processed together per pass over the workers:
// the tile's 4 chunks are walked in groups of kChunkGroup, so that the
// registers held across the worker loop (m, the worker sum, the loads in
// flight) stay within an occupancy of 4+ waves per SIMD.
constexpr int kChunkGroup = 2;
// Minimum waves per SIMD the step pass is compiled for (caps its VGPRs at
// 128, which the chunk group of 2 fits without spilling).
constexpr int kStepMinWaves = 4;

// Which workers a block walks (MODE):
//  kModeAll     every worker: the component compression (STEP false) and
//               the single-pass fused step (STEP true).
//  kModeWorker  STEP false, one worker per partition, (owner + 1 + rot) % K:
//               one of the K - 1 non-owner passes of the multi-pass step.
//               It compresses that worker's row and writes its sparse buffer.
//  kModeOwner   STEP true, the owner alone: the last pass of the multi-pass
//               step.  The worker sum at a masked element is formed here, in
//               worker order, from the other workers' sparse buffers and the
//               owner's own value.
// A pass over one worker streams three rows (g, e read; e written) where
// the single pass streams 3K + 1 at once; HBM serves the narrower mix
// faster.
// Minimum waves per SIMD the owner and worker passes are compiled for, and
// their chunk groups.
constexpr int kOwnerMinWaves = 8;
constexpr int kOwnerChunkGroup = 1;
constexpr int kWorkerMinWaves = 4;
constexpr int kWorkerChunkGroup = 2;
constexpr int kModeAll = 0;
constexpr int kModeWorker = 1;
constexpr int kModeOwner = 2;
//  kModeAllPre  the single-pass fused step for exactly kPreWorkers workers
//               on layouts of few tiles (one block per CU or so), where
//               each block's chain of dependent loads is the step's time:
//               the whole tile is one chunk group, and both workers' g and e
//               are loaded before any is used.
constexpr int kModeAllPre = 3;
constexpr int kPreWorkers = 2;
constexpr int kPreMinWaves = 2;
// Tiles (over all partitions) up to which the step takes kModeAllPre.
constexpr int64_t kPreMaxTiles = 2048;

// VOUT: v_t is stored at the masked elements (v non-null).  AdamS never
// reads v back, so a caller may leave it out.
template <bool STEP, bool VEC, bool SEG, bool VOUT, int MODE>
__global__ void __launch_bounds__(kThreads, MODE == kModeOwner    ? kOwnerMinWaves
                                           : MODE == kModeWorker ? kWorkerMinWaves
                                           : MODE == kModeAllPre ? kPreMinWaves
                                                                 : kStepMinWaves)
compress_kernel(Geom g, const float* __restrict__ grads, float* __restrict__ e,
                const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                float* __restrict__ b, float* __restrict__ m, float* __restrict__ v,
                float* __restrict__ w, float* __restrict__ mold, AdamsC ac,
                const uint32_t* __restrict__ lo_in, uint32_t* __restrict__ cand,
                uint32_t* __restrict__ cnt1, uint32_t* __restrict__ hist, int p0, int64_t e_stride,
                const float* __restrict__ ibc_dev, int rot) {
  static_assert(MODE == kModeAll || (MODE == kModeWorker && !STEP) || (MODE == kModeOwner && STEP) ||
                    (MODE == kModeAllPre && STEP),
                "worker passes compress only; the owner pass is a step pass");
  constexpr int CG = (MODE == kModeOwner)    ? kOwnerChunkGroup
                     : (MODE == kModeWorker) ? kWorkerChunkGroup
                     : (MODE == kModeAllPre) ? 4
                                             : kChunkGroup;
  __shared__ uint64_t sw[kWordsPerTile];
  __shared__ uint32_t spre[kWordsPerTile];
  __shared__ uint32_t sh[STEP ? kBins : 1];
  // bias-correction reciprocals: kernel arguments, or the device-resident
  // state of a graph-capturable step
  const float ibc1 = (STEP && ibc_dev) ? ibc_dev[0] : ac.ibc1;
  const float ibc2 = (STEP && ibc_dev) ? ibc_dev[1] : ac.ibc2;
  __shared__ uint32_t tcnt;
  if (STEP) hist_zero(sh);
  // partitions p0 .. p0 + nparts - 1; e holds their rows [K][nparts * n_p]
  // with rows e_stride apart (e_stride = n and p0 = 0 for the resident buffer)
  const int p = p0 + block_part();
  const int64_t ebase = (int64_t)(p - p0) * g.n_p;
  const int64_t pbase = (int64_t)p * g.n_p;
  const uint32_t sl = (uint32_t)(pbase & 15) >> 2;  // line shift of SEG (w, m, v 64-byte aligned)
  const int64_t wbase = (int64_t)p * g.wpp;
  const int64_t pk = (int64_t)g.P * g.k;
  const int owner = (int)(((int64_t)p * g.K) / g.P);
  // the one worker of a worker or owner pass
  const int wsel = (MODE == kModeWorker) ? (owner + 1 + rot) % g.K : owner;
  const int nwork = (MODE == kModeAll) ? g.K : (MODE == kModeAllPre) ? kPreWorkers : 1;
  const uint32_t lo = STEP ? lo_in[p] : 0u;
  const int lane16 = threadIdx.x & 15;
  const int sh4 = 4 * lane16;
  const uint64_t below = (sh4 == 0) ? 0ull : ((1ull << sh4) - 1ull);

  for (int64_t t = block_in_part(); t < g.tpp; t += blocks_per_part()) {
    __syncthreads();  // previous tile's LDS words and counter no longer in use
    load_tile_words(bits, wbase, g.wpp, t, sw, spre);
    if (threadIdx.x == 0) tcnt = 0;
    __syncthreads();
    // Addresses are a block-uniform tile base (scalar registers) plus a
    // 32-bit lane offset: element o of the tile, rank rr of the tile's
    // first masked element.
    const int64_t tb = t * kTile;
    const uint32_t tn = (uint32_t)min<int64_t>(kTile, g.n_p - tb);  // elements in this tile
    const int64_t rbase = (int64_t)p * g.k + tile_off[(int64_t)p * g.tpp + t];
    // ranks stay inside partition p's k entries for any mask with k bits per
    // partition; the bound keeps a malformed mask in bounds
    const int64_t rlim = (int64_t)(p + 1) * g.k - rbase;
    uint32_t* slot = cand + ((int64_t)p * g.tpp + t) * kSlotWords;
    const float* mt = m + pbase + tb;

    for (int cg = 0; cg < 4; cg += CG) {
      uint32_t nib[CG], rr0[CG], o[CG];
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const int c = cg + u;
        const int q = c * 16 + (threadIdx.x >> 4);
        const uint64_t word = sw[q];
        nib[u] = (uint32_t)(word >> sh4) & 0xfu;
        rr0[u] = spre[q] + (uint32_t)__popcll(word & below);
        o[u] = c * 1024 + 4 * threadIdx.x;
      }
      float ma[CG][4], S[CG][4];
      (void)S;
      if (STEP) {
#pragma unroll
        for (int u = 0; u < CG; ++u)
          if (o[u] < tn) load4(mt, o[u], tn, VEC, ma[u]);
      }
      // The owner pass streams too few rows to hide the latency of the w
      // gather behind them, so it loads w at the group's masked elements
      // (their segments, with SEG) here, together with m.
      float wpre[CG][4];
      (void)wpre;
      if (MODE == kModeOwner) {
        const float* wt0 = w + pbase + tb;
#pragma unroll
        for (int u = 0; u < CG; ++u) {
          if (SEG) {
            const uint32_t lane = threadIdx.x & 63u;
            const uint64_t act = __ballot(nib[u] != 0u);
            if ((act & seg_lanes(lane, sl)) && o[u] < tn) load4t(wt0, o[u], wpre[u]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (((nib[u] >> q) & 1u) && o[u] + q < tn) wpre[u][q] = wt0[o[u] + q];
          }
        }
      }
      if constexpr (MODE == kModeAllPre) {
        // one worker's compression, its part of the worker sum and the
        // owner's capture, from its loaded g and e (the same steps as the
        // loop over workers below)
        auto work = [&](int i, const float* gt, float* et, float (&ga)[CG][4], float (&ea)[CG][4]) {
          (void)gt;
          float* bt = b + (int64_t)i * pk + rbase;
          const bool own = STEP && (i == owner);  // block-uniform
#pragma unroll
          for (int u = 0; u < CG; ++u) {
            float a[4];
            if (o[u] < tn) {
              float eo[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                a[q] = ga[u][q] + ea[u][q];
                eo[q] = ((nib[u] >> q) & 1u) ? 0.0f : a[q];
              }
              store4(et, o[u], tn, VEC, eo);
              if (nib[u]) {
                uint32_t rr = rr0[u];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  if ((nib[u] >> q) & 1u) {
                    if ((!STEP || own) && (int64_t)rr < rlim) bt[rr] = a[q];
                    ++rr;
                    // the worker sum so far (the owner pass: the owner's value)
                    if (STEP) S[u][q] = (MODE == kModeOwner || i == 0) ? a[q] : S[u][q] + a[q];
                  }
              }
            }
            if (own) {  // all lanes of the wave take part in the capture
              uint32_t kk[4];
              bool f[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const bool valid = o[u] + q < tn;
                kk[q] = valid ? stat_key(ma[u][q], a[q], ac.b1, ac.c1) : 0u;
                f[q] = valid && kk[q] >= lo;
              }
              capture4(kk, f, (uint32_t)tb + o[u], slot, &tcnt, sh);
            }
          }
        };
        // both workers' g and e loaded before either is used
        float ga[kPreWorkers][CG][4], ea[kPreWorkers][CG][4];
#pragma unroll
        for (int i = 0; i < kPreWorkers; ++i)
#pragma unroll
          for (int u = 0; u < CG; ++u)
            if (o[u] < tn) {
              load4(grads + (int64_t)i * g.n + pbase + tb, o[u], tn, VEC, ga[i][u]);
              load4(e + (int64_t)i * e_stride + ebase + tb, o[u], tn, VEC, ea[i][u]);
            }
#pragma unroll
        for (int i = 0; i < kPreWorkers; ++i)
          work(i, grads + (int64_t)i * g.n + pbase + tb, e + (int64_t)i * e_stride + ebase + tb, ga[i], ea[i]);
      } else {
        for (int ii = 0; ii < nwork; ++ii) {
          const int i = (MODE == kModeAll) ? ii : wsel;
          const float* gt = grads + (int64_t)i * g.n + pbase + tb;
          float* et = e + (int64_t)i * e_stride + ebase + tb;
          float* bt = b + (int64_t)i * pk + rbase;
          float ga[CG][4], ea[CG][4];
#pragma unroll
          for (int u = 0; u < CG; ++u) {
            if (o[u] < tn) {
              load4(gt, o[u], tn, VEC, ga[u]);
              load4(et, o[u], tn, VEC, ea[u]);
            }
          }
          const bool own = STEP && (i == owner);  // block-uniform
#pragma unroll
          for (int u = 0; u < CG; ++u) {
            float a[4];
            if (o[u] < tn) {
              float eo[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                a[q] = ga[u][q] + ea[u][q];
                eo[q] = ((nib[u] >> q) & 1u) ? 0.0f : a[q];
              }
              store4(et, o[u], tn, VEC, eo);
              if (nib[u]) {
                uint32_t rr = rr0[u];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  if ((nib[u] >> q) & 1u) {
                    if ((!STEP || own) && (int64_t)rr < rlim) bt[rr] = a[q];
                    ++rr;
                    // the worker sum so far (the owner pass: the owner's value)
                    if (STEP) S[u][q] = (MODE == kModeOwner || i == 0) ? a[q] : S[u][q] + a[q];
                  }
              }
            }
            if (own) {  // all lanes of the wave take part in the capture
              uint32_t kk[4];
              bool f[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const bool valid = o[u] + q < tn;
                kk[q] = valid ? stat_key(ma[u][q], a[q], ac.b1, ac.c1) : 0u;
                f[q] = valid && kk[q] >= lo;
              }
              capture4(kk, f, (uint32_t)tb + o[u], slot, &tcnt, sh);
            }
          }
        }
      }
      if (STEP) {
        // AdamS at the group's masked elements.
        float* wt = w + pbase + tb;
        float* mw = m + pbase + tb;
        float* vt = VOUT ? v + pbase + tb : nullptr;  // v may be null without VOUT
        float* ot = mold + rbase;
#pragma unroll
        for (int u = 0; u < CG; ++u) {
          float wo[4], vo[4], mn4[4], wn4[4];
          if (SEG) {
            // w, m (and v) are written as whole 64-byte segments (4 lanes x
            // 4 elements) wherever a segment holds a masked element, the
            // unmasked elements with the values just read.  A 4-byte write
            // still occupies a whole memory burst; aligned whole segments
            // measured faster than scattered element writes.
            const uint32_t lane = threadIdx.x & 63u;
            const uint64_t act = __ballot(nib[u] != 0u);
            if (!(act & seg_lanes(lane, sl)) || o[u] >= tn) continue;
            if (MODE == kModeOwner) {
#pragma unroll
              for (int q = 0; q < 4; ++q) wo[q] = wpre[u][q];
            } else {
              load4t(wt, o[u], wo);
            }
            if (VOUT) load4t(vt, o[u], vo);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              mn4[q] = ma[u][q];
              wn4[q] = wo[q];
            }
          } else {
            if (!nib[u]) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (((nib[u] >> q) & 1u) && o[u] + q < tn) wo[q] = (MODE == kModeOwner) ? wpre[u][q] : wt[o[u] + q];
          }
          uint32_t rr = rr0[u];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (!((nib[u] >> q) & 1u) || o[u] + q >= tn) continue;
            float sum = S[u][q];
            if (MODE == kModeOwner) {  // ((x^0 + x^1) + ...) + x^{K-1}, x^owner in registers
              // the other workers' values are loaded 8 at a time before
              // they are added, so their loads overlap
              const float* bp = b + rbase + rr;
              const bool inb = (int64_t)rr < rlim;
              for (int i0 = 0; i0 < g.K; i0 += 8) {
                float xs[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                  const int i2 = i0 + j;
                  xs[j] = (i2 == owner) ? S[u][q] : ((i2 < g.K && inb) ? bp[(int64_t)i2 * pk] : 0.0f);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                  if (i0 + j < g.K) sum = (i0 + j == 0) ? xs[j] : sum + xs[j];
              }
            }
            const float x = sum * ac.invK;
            const float mo = ma[u][q];
            const float mn = (ac.b1 * mo) + (ac.c1 * x);
            const float vn = (ac.b2 * (mo * mo)) + (ac.c2 * (x * x));
            const float mh = mn * ibc1;
            const float vh = vn * ibc2;
            const float d = sqrtf(vh) + ac.eps;
            const float uu = mh / d;
            const float wn = wo[q] - (ac.lr * (uu + (ac.wd * wo[q])));
            if (SEG) {
              mn4[q] = mn;
              vo[q] = vn;
              wn4[q] = wn;
            } else {
              mw[o[u] + q] = mn;
              if (VOUT) vt[o[u] + q] = vn;
              wt[o[u] + q] = wn;
            }
            if ((int64_t)rr < rlim) ot[rr] = mo;
            ++rr;
          }
          if (SEG) {
            store4t(mw, o[u], mn4);
            if (VOUT) store4t(vt, o[u], vo);
            store4t(wt, o[u], wn4);
          }
        }
      }
    }
    if (STEP) {
      __syncthreads();
      if (threadIdx.x == 0) cnt1[(int64_t)p * g.tpp + t] = tcnt;
    }
  }
  if (STEP) {
    __syncthreads();
    hist_merge(sh, hist + (int64_t)p * kBins);
  }
}

// One rank's pass in the sharded step (SCAPE paper abstract and §I: the
// mask generation is distributed like the optimizer's shards): the rank is
// one worker, so it compresses its own gradient row g^r with its own
// error-feedback row e^r at the shared mask M_t over every partition, and
// writes its sparse buffer b^r (the non-owner workers' job in the one-device
// step).  On the partitions it owns it also forms the statistic
// b1*m + c1*a^r from m before any update and captures the selection
// candidates, as the step pass's owner does.  The AdamS update waits for the
// synchronised buffer b_bar of the owned partitions (after the reduction
// across ranks), so it is a call of its own.  grads, e: [n] (the rank's
// rows); b: [P*k].
template <bool VEC>
__global__ void __launch_bounds__(kThreads, kWorkerMinWaves)
shard_pass_kernel(Geom g, int rank, const float* __restrict__ grads, float* __restrict__ e,
                  const uint64_t* __restrict__ bits, const uint32_t* __restrict__ tile_off,
                  float* __restrict__ b, const float* __restrict__ m, float b1, float c1,
                  const uint32_t* __restrict__ lo_in, uint32_t* __restrict__ cand,
                  uint32_t* __restrict__ cnt1, uint32_t* __restrict__ hist) {
  constexpr int CG = kWorkerChunkGroup;
  __shared__ uint64_t sw[kWordsPerTile];
  __shared__ uint32_t spre[kWordsPerTile];
  __shared__ uint32_t sh[kBins];
  __shared__ uint32_t tcnt;
  const int p = block_part();
  const bool own = (int)(((int64_t)p * g.K) / g.P) == rank;  // block-uniform
  if (own) hist_zero(sh);
  const int64_t pbase = (int64_t)p * g.n_p;
  const int64_t wbase = (int64_t)p * g.wpp;
  const uint32_t lo = own ? lo_in[p] : 0u;
  const int lane16 = threadIdx.x & 15;
  const int sh4 = 4 * lane16;
  const uint64_t below = (sh4 == 0) ? 0ull : ((1ull << sh4) - 1ull);

  for (int64_t t = block_in_part(); t < g.tpp; t += blocks_per_part()) {
    __syncthreads();  // previous tile's LDS words and counter no longer in use
    load_tile_words(bits, wbase, g.wpp, t, sw, spre);
    if (threadIdx.x == 0) tcnt = 0;
    __syncthreads();
    const int64_t tb = t * kTile;
    const uint32_t tn = (uint32_t)min<int64_t>(kTile, g.n_p - tb);
    const int64_t rbase = (int64_t)p * g.k + tile_off[(int64_t)p * g.tpp + t];
    const int64_t rlim = (int64_t)(p + 1) * g.k - rbase;  // a malformed mask stays in bounds
    uint32_t* slot = cand + ((int64_t)p * g.tpp + t) * kSlotWords;
    const float* gt = grads + pbase + tb;
    float* et = e + pbase + tb;
    const float* mt = m + pbase + tb;
    float* bt = b + rbase;
    for (int cg = 0; cg < 4; cg += CG) {
      uint32_t nib[CG], rr0[CG], o[CG];
      float ga[CG][4], ea[CG][4], ma[CG][4];
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const int c = cg + u;
        const int q = c * 16 + (threadIdx.x >> 4);
        const uint64_t word = sw[q];
        nib[u] = (uint32_t)(word >> sh4) & 0xfu;
        rr0[u] = spre[q] + (uint32_t)__popcll(word & below);
        o[u] = c * 1024 + 4 * threadIdx.x;
        if (o[u] < tn) {
          load4(gt, o[u], tn, VEC, ga[u]);
          load4(et, o[u], tn, VEC, ea[u]);
          if (own) load4(mt, o[u], tn, VEC, ma[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        float a[4];
        if (o[u] < tn) {
          float eo[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a[q] = ga[u][q] + ea[u][q];
            eo[q] = ((nib[u] >> q) & 1u) ? 0.0f : a[q];
          }
          store4(et, o[u], tn, VEC, eo);
          if (nib[u]) {
            uint32_t rr = rr0[u];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if ((nib[u] >> q) & 1u) {
                if ((int64_t)rr < rlim) bt[rr] = a[q];
                ++rr;
              }
          }
        }
        if (own) {  // all lanes of the wave take part in the capture
          uint32_t kk[4];
          bool f[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool valid = o[u] + q < tn;
            kk[q] = valid ? stat_key(ma[u][q], a[q], b1, c1) : 0u;
            f[q] = valid && kk[q] >= lo;
          }
          capture4(kk, f, (uint32_t)tb + o[u], slot, &tcnt, sh);
        }
      }
    }
    if (own) {
      __syncthreads();
      if (threadIdx.x == 0) cnt1[(int64_t)p * g.tpp + t] = tcnt;
    }
  }
  if (own) {
    __syncthreads();
    hist_merge(sh, hist + (int64_t)p * kBins);
  }
}

// SRC 0: key from stat[].  SRC 1: from b1*m + c1*(g^o + e^o).  SRC 2: from
// b1*m + c1*a^o with a^o rebuilt from the compressed state: b^o at the
// element's rank on the mask, e'^o off it.
// PHASE 0 (HIST): histogram of every key.  PHASE 1 (CAPTURE): capture keys
// >= state.lo_fb.  With only_fb, partitions whose fallback flag is clear
// are skipped.
template <int SRC, int PHASE, bool VEC>
__global__ void __launch_bounds__(kThreads)
stat_kernel(Geom g, PartSel* __restrict__ state, int only_fb, const float* __restrict__ stat,
            const float* __restrict__ m, const float* __restrict__ grads, const float* __restrict__ e,
            const float* __restrict__ b, const float* __restrict__ mold, const uint64_t* __restrict__ bits,
            const uint32_t* __restrict__ tile_off, float b1, float c1, uint32_t* __restrict__ cand,
            uint32_t* __restrict__ cnt1, uint32_t* __restrict__ hist, int tile_step, int64_t g_stride,
            int64_t e_stride, int64_t b_stride, int then_mode, uint32_t target, uint32_t* __restrict__ arrive) {
  __shared__ uint64_t sw[kWordsPerTile];
  __shared__ uint32_t spre[kWordsPerTile];
  __shared__ uint32_t sh[kBins];
  __shared__ uint32_t tcnt;
  const int p = g.sp0 + block_part();
  const PartSel st = state[p];
  if (only_fb && !st.fb) return;  // block-uniform
  hist_zero(sh);
  const int64_t pbase = (int64_t)p * g.n_p;
  const int64_t wbase = (int64_t)p * g.wpp;
  const int o = (int)(((int64_t)p * g.K) / g.P);
  // the owner's rows (a row stride of 0: the arrays are that one row)
  const float* go = grads + (int64_t)o * g_stride + pbase;
  const float* eo = e + (int64_t)o * e_stride + pbase;
  const float* bo = b + (int64_t)o * b_stride;
  const uint32_t lo = st.lo_fb;
  const int lane16 = threadIdx.x & 15;
  const int sh4 = 4 * lane16;
  const uint64_t below = (sh4 == 0) ? 0ull : ((1ull << sh4) - 1ull);

  const int64_t tstride = (int64_t)blocks_per_part() * tile_step;
  for (int64_t t = (int64_t)block_in_part() * tile_step; t < g.tpp; t += tstride) {
    __syncthreads();
    if (SRC == 2) load_tile_words(bits, wbase, g.wpp, t, sw, spre);
    if (threadIdx.x == 0) tcnt = 0;
    __syncthreads();
    const int64_t rbase = (SRC == 2) ? (int64_t)p * g.k + tile_off[(int64_t)p * g.tpp + t] : 0;
    const int64_t rend = (int64_t)(p + 1) * g.k;
    uint32_t* slot = cand + ((int64_t)p * g.tpp + t) * kSlotWords;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t lj = t * kTile + c * 1024 + 4 * threadIdx.x;
      uint32_t kk[4] = {0u, 0u, 0u, 0u};
      if (lj < g.n_p) {
        if (SRC == 0) {
          float s[4];
          load4(stat + pbase, lj, g.n_p, VEC, s);
#pragma unroll
          for (int q = 0; q < 4; ++q) kk[q] = __float_as_uint(s[q]) & 0x7fffffffu;
        } else {
          float mm[4], a[4];
          load4(m + pbase, lj, g.n_p, VEC, mm);
          if (SRC == 1) {
            float gg[4], ee[4];
            load4(go, lj, g.n_p, VEC, gg);
            load4(eo, lj, g.n_p, VEC, ee);
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] = gg[q] + ee[q];
          } else {
            load4(eo, lj, g.n_p, VEC, a);
            const int qw = c * 16 + (threadIdx.x >> 4);
            const uint64_t word = sw[qw];
            const uint32_t nib = (uint32_t)(word >> sh4) & 0xfu;
            if (nib) {
              int64_t r = rbase + spre[qw] + (uint32_t)__popcll(word & below);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if ((nib >> q) & 1u) {
                  if (r < rend) {
                    a[q] = bo[r];
                    if (mold) mm[q] = mold[r];
                  }
                  ++r;
                }
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) kk[q] = stat_key(mm[q], a[q], b1, c1);
        }
      }
      if (PHASE == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (lj + q < g.n_p) atomicAdd(&sh[kk[q] >> kL1Shift], 1u);
      } else {
        bool f[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = (lj + q < g.n_p) && kk[q] >= lo;
        capture4(kk, f, (uint32_t)lj, slot, &tcnt, sh);
      }
    }
    if (PHASE == 1) {
      __syncthreads();
      if (threadIdx.x == 0) cnt1[(int64_t)p * g.tpp + t] = tcnt;
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)p * kBins;
  hist_merge(sh, gh);
  if (!then_mode) return;  // kernel-uniform
  // The last of the partition's blocks to arrive (its histogram now holds
  // every block's counts) runs level 1 on it, zeroes its bins and resets
  // the arrival count.
  __shared__ int last;
  __threadfence();  // this block's histogram atomics before its arrival
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(arrive + p, 1u) == (uint32_t)blocks_per_part() - 1u;
  __syncthreads();
  if (!last) return;  // block-uniform
  __threadfence();
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    sh[i] = __hip_atomic_load(gh + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  level1_block(g, p, sh, state, then_mode, target);
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads) gh[i] = 0u;
  if (threadIdx.x == 0) arrive[p] = 0u;
}

template <int SRC, int PHASE>
void launch_stat_t(const Geom& g, const StatArgs& a, bool vec, hipStream_t s) {
  if (g.snp < 1) return;
  const dim3 grid = stream_grid(g.snp, g.Gs);
  const int ts = a.tile_step < 1 ? 1 : a.tile_step;
  const int64_t pk = (int64_t)g.P * g.k;
  const int64_t gs = a.single_row ? 0 : g.n, es = a.single_row ? 0 : g.n, bs = a.single_row ? 0 : pk;
  if (vec)
    stat_kernel<SRC, PHASE, true><<<grid, kThreads, 0, s>>>(g, a.state, a.only_fb, a.stat, a.m, a.grads, a.e, a.b,
                                                           a.mold, a.bits, a.tile_off, a.b1, a.c1, a.cand, a.cnt1, a.hist,
                                                           ts, gs, es, bs, a.then_mode, a.target, a.arrive);
  else
    stat_kernel<SRC, PHASE, false><<<grid, kThreads, 0, s>>>(g, a.state, a.only_fb, a.stat, a.m, a.grads, a.e, a.b,
                                                            a.mold, a.bits, a.tile_off, a.b1, a.c1, a.cand, a.cnt1, a.hist,
                                                            ts, gs, es, bs, a.then_mode, a.target, a.arrive);
}

}  // namespace

hipError_t launch_stat(const Geom& g, int src, int phase, const StatArgs& a, bool vec, hipStream_t s) {
  if (src == kSrcStat && phase == kPhaseHist) launch_stat_t<kSrcStat, kPhaseHist>(g, a, vec, s);
  else if (src == kSrcStat) launch_stat_t<kSrcStat, kPhaseCapture>(g, a, vec, s);
  else if (src == kSrcState && phase == kPhaseHist) launch_stat_t<kSrcState, kPhaseHist>(g, a, vec, s);
  else if (src == kSrcState) launch_stat_t<kSrcState, kPhaseCapture>(g, a, vec, s);
  else if (phase == kPhaseHist) launch_stat_t<kSrcMasked, kPhaseHist>(g, a, vec, s);
  else launch_stat_t<kSrcMasked, kPhaseCapture>(g, a, vec, s);
  return hipGetLastError();
}

template <int MODE>
void launch_compress_t(const Geom& g, const float* grads, float* e, const uint64_t* bits, const uint32_t* tile_off,
                       float* b, bool vec, int rot, hipStream_t s) {
  const dim3 grid = stream_grid(g.P, g.G);
  AdamsC ac{};
  if (vec)
    compress_kernel<false, true, false, false, MODE><<<grid, kThreads, 0, s>>>(
        g, grads, e, bits, tile_off, b, nullptr, nullptr, nullptr, nullptr, ac, nullptr, nullptr, nullptr, nullptr,
        0, g.n, nullptr, rot);
  else
    compress_kernel<false, false, false, false, MODE><<<grid, kThreads, 0, s>>>(
        g, grads, e, bits, tile_off, b, nullptr, nullptr, nullptr, nullptr, ac, nullptr, nullptr, nullptr, nullptr,
        0, g.n, nullptr, rot);
}

hipError_t launch_compress(const Geom& g, const float* grads, float* e, const uint64_t* bits,
                           const uint32_t* tile_off, float* b, hipStream_t s, bool vec) {
  launch_compress_t<kModeAll>(g, grads, e, bits, tile_off, b, vec, 0, s);
  return hipGetLastError();
}

template <bool VEC, bool SEG, bool VOUT, int MODE>
void launch_step_t(const Geom& g, const StepArgs& a, const AdamsC& ac, hipStream_t s) {
  compress_kernel<true, VEC, SEG, VOUT, MODE><<<stream_grid(a.nparts, g.G), kThreads, 0, s>>>(
      g, a.grads, a.e, a.bits, a.tile_off, a.b, a.m, a.v, a.w, a.mold, ac, a.lo, a.cand, a.cnt1, a.hist, a.p0,
      a.e_stride, a.ibc_dev, 0);
}

template <int MODE>
void launch_step_mode(const Geom& g, const StepArgs& a, bool vec, bool seg, hipStream_t s) {
  AdamsC ac{a.b1, a.b2, a.c1, a.c2, a.ibc1, a.ibc2, a.eps, a.wd, a.lr, (float)(1.0 / (double)g.K)};
  const bool vout = a.v != nullptr;
  if (vec && seg) {
    if (vout) launch_step_t<true, true, true, MODE>(g, a, ac, s);
    else launch_step_t<true, true, false, MODE>(g, a, ac, s);
  } else if (vec) {
    if (vout) launch_step_t<true, false, true, MODE>(g, a, ac, s);
    else launch_step_t<true, false, false, MODE>(g, a, ac, s);
  } else {
    if (vout) launch_step_t<false, false, true, MODE>(g, a, ac, s);
    else launch_step_t<false, false, false, MODE>(g, a, ac, s);
  }
}

hipError_t launch_step_pass(const Geom& g, const StepArgs& a, bool vec, bool seg, hipStream_t s) {
  // two workers on few tiles: the latency form (kModeAllPre)
  if (g.K == kPreWorkers && (int64_t)g.P * g.tpp <= kPreMaxTiles) launch_step_mode<kModeAllPre>(g, a, vec, seg, s);
  else launch_step_mode<kModeAll>(g, a, vec, seg, s);
  return hipGetLastError();
}

hipError_t launch_shard_pass(const Geom& g, int rank, const float* grads, float* e, const uint64_t* bits,
                             const uint32_t* tile_off, float* b, const float* m, float b1, float c1,
                             const uint32_t* lo, uint32_t* cand, uint32_t* cnt1, uint32_t* hist, bool vec,
                             hipStream_t s) {
  const dim3 grid = stream_grid(g.P, g.G);
  if (vec)
    shard_pass_kernel<true><<<grid, kThreads, 0, s>>>(g, rank, grads, e, bits, tile_off, b, m, b1, c1, lo, cand, cnt1,
                                                      hist);
  else
    shard_pass_kernel<false><<<grid, kThreads, 0, s>>>(g, rank, grads, e, bits, tile_off, b, m, b1, c1, lo, cand,
                                                       cnt1, hist);
  return hipGetLastError();
}

bool multi_pass_pays(const Geom& g) {
  // Measured on the model-shaped workloads: at K = 8 and 1% density the K
  // passes ran 6.5% faster than the single pass on average; at K = 4, and
  // at K = 8 with 10% density (the sparse buffers' round trip, 8(K-1)Pk
  // bytes, at 5.6% of the streams), they ran 1-2% slower on average.
  const double trip = 8.0 * (g.K - 1) * (double)g.P * (double)g.k;
  const double streams = (12.0 * g.K + 4.0) * (double)g.n;
  return g.K >= 8 && trip <= 0.02 * streams;
}

hipError_t launch_step_passes(const Geom& g, const StepArgs& a, bool vec, bool seg, hipStream_t s) {
  if (!multi_pass_pays(g)) return launch_step_pass(g, a, vec, seg, s);
  // K - 1 non-owner passes (pass j: worker (owner + 1 + j) % K of every
  // partition), then the owner pass; stream order makes every sparse buffer
  // complete before the owner pass reads it
  for (int j = 0; j + 1 < g.K; ++j) {
    launch_compress_t<kModeWorker>(g, a.grads, a.e, a.bits, a.tile_off, a.b, vec, j, s);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  launch_step_mode<kModeOwner>(g, a, vec, seg, s);
  return hipGetLastError();
}

}  // namespace scape
