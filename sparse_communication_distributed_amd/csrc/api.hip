// C ABI of libscape (declared in include/scape.h): argument validation,
// geometry of masks and workspace, and the order of launches of one SCAPE
// optimizer step.
#include "scape.h"
#include "scape_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

namespace scape {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int bit_width_u64(uint64_t x) {
  int b = 0;
  while (x) {
    ++b;
    x >>= 1;
  }
  return b;
}

bool make_geom(int64_t n, int P, int K, int64_t k, Geom* g) {
  if (P < 1 || P > 65535 || K < 1 || n < 1 || n % P != 0 || n >= (int64_t(1) << 32)) return false;
  const int64_t n_p = n / P;
  if (k < 1 || k > n_p) return false;
  Geom r{};
  r.n = n;
  r.n_p = n_p;
  r.k = k;
  r.P = P;
  r.K = K;
  r.wpp = (n_p + 63) / 64;
  r.tpp = (n_p + kTile - 1) / kTile;
  r.G = (int)r.tpp;  // one block per tile (tpp < 2^21: n < 2^32)
  int64_t Gs = (kStatBlocks + P - 1) / P;
  if (Gs > r.tpp) Gs = r.tpp;
  r.Gs = (int)(Gs < 1 ? 1 : Gs);
  r.idx_bits = bit_width_u64((uint64_t)(n_p - 1));
  if (r.idx_bits < 1) r.idx_bits = 1;
  r.idx_mask = (uint32_t)((uint64_t(1) << r.idx_bits) - 1);
  // levels after level 1: key bits 18..7, 6..0, then the index bits
  int nl = 0;
  r.levels[nl++] = Level{32 + kL1Shift - kDigitBits, kDigitBits};
  r.levels[nl++] = Level{32, kL1Shift - kDigitBits};
  for (int rem = r.idx_bits; rem > 0;) {
    const int nb = rem < kDigitBits ? rem : kDigitBits;
    r.levels[nl++] = Level{rem - nb, nb};
    rem -= nb;
  }
  r.nlevels = nl;
  r.sp0 = 0;
  r.snp = P;
  // the level-2 histogram in a pass of its own: masks under 5% density on
  // layouts of more than kSelectWaves tiles, about kHistBlocks blocks in
  // all, no more than one per 64 tiles of a partition
  r.hparts = 0;
  if (k * 20 < n_p && (int64_t)P * r.tpp > kSelectWaves) {
    int64_t h = kHistBlocks / P;
    const int64_t hmax = (r.tpp + 63) / 64;
    if (h > hmax) h = hmax;
    r.hparts = (int)(h < 1 ? 1 : h);
  }
  // mask slot: bits, idx, tile_off, then the threshold record u32[3P]
  r.off_bits = 0;
  r.off_idx = align256((size_t)P * r.wpp * 8);
  r.off_toff = align256(r.off_idx + (size_t)P * k * 4);
  r.off_meta = align256(r.off_toff + (size_t)P * r.tpp * 4);
  r.slot_bytes = align256(r.off_meta + (size_t)P * 3 * 4);
  // workspace
  size_t o = 0;
  r.ws_b = o;       o = align256(o + (size_t)K * P * k * 4);
  r.ws_mold = o;    o = align256(o + (size_t)P * k * 4);
  r.ws_hist = o;    o = align256(o + (size_t)P * kBins * 4);
  r.ws_cand = o;    o = align256(o + (size_t)P * r.tpp * kSlotWords * 4);
  r.ws_cnt1 = o;    o = align256(o + (size_t)P * r.tpp * 4);
  r.ws_cnt2 = o;    o = align256(o + (size_t)P * r.tpp * 4);
  r.ws_state = o;   o = align256(o + (size_t)P * sizeof(PartSel));
  r.ws_tilecnt = o; o = align256(o + (size_t)P * r.tpp * 4);
  r.ws_surv = o;    o = align256(o + (size_t)P * kSurvivorCap * 8);
  r.ws_nsurv = o;   o = align256(o + (size_t)P * 4);
  r.ws_arrive = o;  o = align256(o + (size_t)P * 4);
  r.ws_part = o;    o = align256(o + (size_t)P * r.hparts * kBins * 4);
  r.ws_total = o;
  *g = r;
  return true;
}

}  // namespace scape

using namespace scape;

namespace {

thread_local char g_err[512] = "";

scape_status fail(scape_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

scape_status hip_check(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(SCAPE_EHIP, "%s: %s", where, hipGetErrorString(e));
  return SCAPE_OK;
}

scape_status check_dims(const scape_dims* d, int64_t k, Geom* g) {
  if (!d) return fail(SCAPE_EINVAL, "dims is null");
  if (!make_geom(d->n, d->num_partitions, d->num_workers, k, g))
    return fail(SCAPE_ESHAPE, "invalid shape: n=%lld P=%d K=%d k=%lld (need 1<=P<=65535, K>=1, n%%P==0, n<2^32, 1<=k<=n/P)",
                (long long)d->n, d->num_partitions, d->num_workers, (long long)k);
  return SCAPE_OK;
}

scape_status check_betas(const scape_betas& b, float lr) {
  if (!(b.beta1 >= 0.0f && b.beta1 < 1.0f) || !(b.beta2 >= 0.0f && b.beta2 < 1.0f))
    return fail(SCAPE_EINVAL, "betas must lie in [0, 1)");
  if (!(b.eps > 0.0f) || !std::isfinite(b.eps)) return fail(SCAPE_EINVAL, "eps must be positive and finite");
  if (!std::isfinite(b.weight_decay)) return fail(SCAPE_EINVAL, "weight_decay must be finite");
  if (!std::isfinite(lr)) return fail(SCAPE_EINVAL, "lr must be finite");
  return SCAPE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// Whole 64-byte lines of w, m (and v) per 16 elements: needs 64-byte
// aligned rows (the lines follow the rows' alignment, whatever a
// partition's first element).  A line costs the read of w's line, which the
// update reads anyway, so without v it pays at any density; with v it also
// reads v's line, which pays only where masked elements are not too rare (at
// a density of 0.1% that read costs more than the whole writes save).
bool seg_ok(const Geom& g, const void* w, const void* m, const void* v) {
  return (((uintptr_t)w | (uintptr_t)m | (uintptr_t)v) & 63u) == 0 && (v == nullptr || g.k * 200 >= g.n_p);
}

// fp32(1 / (1 - beta^t)), beta^t formed by t binary64 multiplications by
// binary64(beta) starting from 1.  A product of a previous call with the same
// beta and at most t steps is resumed (the same multiplications in the same
// order), so consecutive steps cost one multiplication each.
float bias_reciprocal(float beta, int64_t t) {
  struct Entry {
    uint32_t bits;
    int64_t t;  // 0: empty
    double p;
  };
  thread_local Entry cache[4] = {};
  thread_local int next = 0;
  uint32_t bits;
  std::memcpy(&bits, &beta, sizeof bits);
  double p = 1.0;
  int64_t from = 0;
  Entry* mine = nullptr;
  for (Entry& c : cache) {
    if (c.t == 0 || c.bits != bits) continue;
    mine = &c;
    if (c.t <= t) {
      from = c.t;
      p = c.p;
    }
  }
  for (int64_t i = from; i < t; ++i) p = p * (double)beta;
  if (!mine) {
    mine = &cache[next];
    next = (next + 1) % 4;
  }
  *mine = Entry{bits, t, p};
  return (float)(1.0 / (1.0 - p));
}

scape_mask_view slot_view(const Geom& g, void* blob, int slot) {
  char* base = static_cast<char*>(blob) + (size_t)slot * g.slot_bytes;
  return scape_mask_view{reinterpret_cast<uint64_t*>(base + g.off_bits),
                         reinterpret_cast<uint32_t*>(base + g.off_idx),
                         reinterpret_cast<uint32_t*>(base + g.off_toff),
                         reinterpret_cast<uint32_t*>(base + g.off_meta)};
}

struct Ws {
  float* b;
  float* mold;
  SelectBufs sel;
};

Ws ws_view(const Geom& g, void* ws) {
  char* c = static_cast<char*>(ws);
  Ws w;
  w.b = reinterpret_cast<float*>(c + g.ws_b);
  w.mold = reinterpret_cast<float*>(c + g.ws_mold);
  w.sel.hist = reinterpret_cast<uint32_t*>(c + g.ws_hist);
  w.sel.cand = reinterpret_cast<uint32_t*>(c + g.ws_cand);
  w.sel.cnt1 = reinterpret_cast<uint32_t*>(c + g.ws_cnt1);
  w.sel.cnt2 = reinterpret_cast<uint32_t*>(c + g.ws_cnt2);
  w.sel.state = reinterpret_cast<PartSel*>(c + g.ws_state);
  w.sel.tilecnt = reinterpret_cast<uint32_t*>(c + g.ws_tilecnt);
  w.sel.surv = reinterpret_cast<uint64_t*>(c + g.ws_surv);
  w.sel.nsurv = reinterpret_cast<uint32_t*>(c + g.ws_nsurv);
  w.sel.arrive = reinterpret_cast<uint32_t*>(c + g.ws_arrive);
  w.sel.part = reinterpret_cast<uint32_t*>(c + g.ws_part);
  return w;
}

// ------------------------------------------------------------- profiling

enum Stage { ST_BOOT = 0, ST_PASS, ST_SELECT, ST_REFINE, ST_EMIT, ST_COUNT };
const char* kStageNames[ST_COUNT] = {"bootstrap_select", "step_pass", "select_pass", "refine", "emit"};

struct Rec {
  int stage;
  hipEvent_t a, b;
};

struct Profiler {
  bool on = false;
  bool bad = false;  // an event call failed; the next collect reports it
  std::vector<Rec> recs;
  int open = -1;
  hipStream_t stream = nullptr;
  void begin(int stage, hipStream_t s) {
    if (!on) return;
    end();
    Rec r{stage, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
      bad = true;
      return;
    }
    if (hipEventRecord(r.a, s) != hipSuccess) bad = true;
    recs.push_back(r);
    open = (int)recs.size() - 1;
    stream = s;
  }
  void end() {
    if (!on || open < 0) return;
    if (hipEventRecord(recs[open].b, stream) != hipSuccess) bad = true;
    open = -1;
  }
};
Profiler g_prof;

// Sub-stage boundaries inside the selection pipeline.
struct SelectMarks {
  hipStream_t s;
};
void select_mark(void* ctx, int id) {
  SelectMarks* m = static_cast<SelectMarks*>(ctx);
  if (id == 1) g_prof.begin(ST_REFINE, m->s);
  if (id == 2) g_prof.begin(ST_EMIT, m->s);
}

// Level 1 with the exact fallback: for partitions flagged in the state,
// count every key (source `src`) and bound the capture at the threshold
// digit (the pass's last block per partition), then recapture and redo
// level 1 on the recaptured keys (likewise): two launches, which do nothing
// but read the state where no partition is flagged.
scape_status run_fallback(const Geom& g, const Ws& w, int src, StatArgs a, bool vec, hipStream_t s) {
  scape_status st;
  a.state = w.sel.state;
  a.only_fb = 1;
  a.cand = w.sel.cand;
  a.cnt1 = w.sel.cnt1;
  a.hist = w.sel.hist;
  a.arrive = w.sel.arrive;
  a.target = capture_target(g);
  a.then_mode = kScanBound;
  if ((st = hip_check(launch_stat(g, src, kPhaseHist, a, vec, s), "fallback count"))) return st;
  a.then_mode = kScanFinal;
  return hip_check(launch_stat(g, src, kPhaseCapture, a, vec, s), "fallback capture");
}

scape_status run_tail(const Geom& g, const Ws& w, scape_mask_view out, hipStream_t s, bool prof) {
  SelectMarks marks{s};
  hipError_t e = launch_select_tail(g, w.sel, out.bits, out.idx, out.tile_off, out.meta, s,
                                    prof ? select_mark : nullptr, &marks);
  return hip_check(e, "select launch");
}

// Mask from scratch (no capture bound known).  With enough tiles per
// partition, a histogram of every kSampleStep-th tile gives each partition
// the level-1 digit above which about kSampleMargin * k keys lie; one
// capture pass at that bound follows and is checked as after a step pass,
// and a partition that captured fewer than k keys takes the exact two-pass
// route of the fallback (every partition does, without the sample).
scape_status run_fresh_select(const Geom& g, const Ws& w, int src, const StatArgs& a, bool vec,
                              scape_mask_view out, hipStream_t s) {
  scape_status st;
  if ((st = hip_check(launch_zero_u32(w.sel.hist + (int64_t)g.sp0 * kBins, (int64_t)g.snp * kBins, s), "zero")))
    return st;
  if ((st = hip_check(launch_init_state(g, w.sel, s), "init"))) return st;
  if (g.tpp >= 4 * kSampleStep) {
    StatArgs b = a;
    b.state = w.sel.state;
    b.only_fb = 1;
    b.cand = w.sel.cand;
    b.cnt1 = w.sel.cnt1;
    b.hist = w.sel.hist;
    b.tile_step = kSampleStep;
    const int64_t sampled = (g.tpp + kSampleStep - 1) / kSampleStep;
    const double frac = (double)(sampled * kTile) / (double)(g.tpp * kTile);
    double tgt = std::ceil(kSampleMargin * (double)g.k * frac);
    if (tgt < 1.0) tgt = 1.0;
    if ((st = hip_check(launch_stat(g, src, kPhaseHist, b, vec, s), "sample count"))) return st;
    if ((st = hip_check(launch_level1(g, w.sel, kScanSample, s, (uint32_t)tgt), "sample bound"))) return st;
    b.tile_step = 1;
    if ((st = hip_check(launch_stat(g, src, kPhaseCapture, b, vec, s), "first capture"))) return st;
    if ((st = hip_check(launch_level1(g, w.sel, kScanCheck, s), "level 1"))) return st;
  }
  if ((st = run_fallback(g, w, src, a, vec, s))) return st;
  return run_tail(g, w, out, s, false);
}

}  // namespace

extern "C" {

int64_t scape_tile_elems(void) { return kTile; }

int32_t scape_step_pass_count(const scape_dims* dims, int64_t k) {
  Geom g;
  if (!dims || !make_geom(dims->n, dims->num_partitions, dims->num_workers, k, &g)) return -1;
  return multi_pass_pays(g) ? g.K : 1;
}

size_t scape_mask_bytes(const scape_dims* dims, int64_t k) {
  Geom g;
  if (!dims || !make_geom(dims->n, dims->num_partitions, dims->num_workers, k, &g)) return 0;
  return 2 * g.slot_bytes;
}

scape_status scape_mask_slot(const scape_dims* dims, int64_t k, void* mask_blob, int slot,
                             scape_mask_view* out) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!mask_blob || !out) return fail(SCAPE_EINVAL, "mask_blob or out is null");
  if (slot != 0 && slot != 1) return fail(SCAPE_EINVAL, "slot must be 0 or 1");
  *out = slot_view(g, mask_blob, slot);
  return SCAPE_OK;
}

size_t scape_workspace_bytes(const scape_dims* dims, int64_t k) {
  Geom g;
  if (!dims || !make_geom(dims->n, dims->num_partitions, dims->num_workers, k, &g)) return 0;
  return g.ws_total;
}

scape_status scape_mask_topk(const scape_dims* dims, int64_t k, const float* stat,
                             scape_mask_view out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!stat || !out.bits || !out.idx || !out.tile_off || !workspace)
    return fail(SCAPE_EINVAL, "null pointer argument");
  if (workspace_bytes < g.ws_total)
    return fail(SCAPE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, g.ws_total);
  Ws w = ws_view(g, workspace);
  const bool vec = (g.n_p % 4 == 0) && aligned16(stat);
  StatArgs a{};
  a.stat = stat;
  return run_fresh_select(g, w, kSrcStat, a, vec, out, stream);
}

scape_status scape_compress(const scape_dims* dims, int64_t k, const float* grads, float* e,
                            scape_mask_view cur, float* b, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!grads || !e || !cur.bits || !cur.tile_off || !b) return fail(SCAPE_EINVAL, "null pointer argument");
  const bool vec = (g.n_p % 4 == 0) && aligned16(grads) && aligned16(e);
  return hip_check(launch_compress(g, grads, e, cur.bits, cur.tile_off, b, stream, vec), "compress");
}

scape_status scape_reduce_sparse(const scape_dims* dims, int64_t k, const float* b, float* b_bar,
                                 hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!b || !b_bar) return fail(SCAPE_EINVAL, "null pointer argument");
  return hip_check(launch_reduce(g, b, b_bar, stream), "reduce");
}

scape_status scape_adams_update(const scape_dims* dims, int64_t k, float* params, float* m,
                                float* v, const float* b_bar, scape_mask_view cur,
                                scape_betas betas, float lr, int64_t step, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!params || !m || !b_bar || !cur.idx) return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = check_betas(betas, lr))) return st;
  if (step < 1) return fail(SCAPE_EINVAL, "step must be >= 1");
  const float b1 = betas.beta1, b2 = betas.beta2;
  const float c1 = 1.0f - b1, c2 = 1.0f - b2;
  return hip_check(launch_adams(g, b_bar, cur.idx, params, m, v, b1, b2, c1, c2,
                                bias_reciprocal(b1, step), bias_reciprocal(b2, step), betas.eps,
                                betas.weight_decay, lr, stream),
                   "adams");
}

}  // extern "C"

namespace {

// Everything of one step except the pass over the error-feedback buffers:
// validation, the step-1 bootstrap, and (after the pass) level 1, the exact
// fallback and the selection of M_{t+1}.  `e` is where the fallback and the
// bootstrap read the error-feedback rows ([K][n]).
struct StepCtx {
  Geom g;
  Ws w;
  scape_mask_view cur, nxt;
  StatArgs a;
  StepArgs sa;
  bool vec;
  bool prof;  // stage timing records this call
};

// `bias` null: step t = `step` from the host (slots (t-1)&1 -> t&1, host
// bias reciprocals, bootstrap at t = 1).  `bias` set: the graph-capturable
// form, M_t in slot cur_slot, the bias state advanced on the device, no
// bootstrap and no stage timing.
scape_status step_begin(StepCtx& c, const scape_dims* dims, float* params, const float* grads, float* m,
                        float* v, float* e, void* mask_blob, int64_t k, scape_betas betas, float lr,
                        int64_t step, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        scape_bias_state* bias = nullptr, int cur_slot = 0, bool timing = true) {
  scape_status st = check_dims(dims, k, &c.g);
  if (st) return st;
  const Geom& g = c.g;
  if (!params || !grads || !m || !e || !mask_blob || !workspace)  // v is optional
    return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = check_betas(betas, lr))) return st;
  if (!bias && step < 1) return fail(SCAPE_EINVAL, "step must be >= 1");
  if (bias && cur_slot != 0 && cur_slot != 1) return fail(SCAPE_EINVAL, "cur_slot must be 0 or 1");
  if (bias && ((uintptr_t)bias & 7u)) return fail(SCAPE_EINVAL, "bias state must be 8-byte aligned");
  if (workspace_bytes < g.ws_total)
    return fail(SCAPE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, g.ws_total);

  c.prof = g_prof.on && !bias && timing;
  c.w = ws_view(g, workspace);
  const int cs = bias ? cur_slot : (int)((step - 1) & 1);
  c.cur = slot_view(g, mask_blob, cs);
  c.nxt = slot_view(g, mask_blob, 1 - cs);
  c.vec = (g.n_p % 4 == 0) && aligned16(grads) && aligned16(e) && aligned16(m);
  const float b1 = betas.beta1, b2 = betas.beta2;
  const float c1 = 1.0f - b1, c2 = 1.0f - b2;
  StatArgs& a = c.a;
  a = StatArgs{};
  a.m = m;
  a.grads = grads;
  a.e = e;
  a.b = c.w.b;
  a.mold = c.w.mold;  // the step pass updates m at M_t before the selection runs
  a.bits = c.cur.bits;
  a.tile_off = c.cur.tile_off;
  a.b1 = b1;
  a.c1 = c1;
  StepArgs& sa = c.sa;
  sa = StepArgs{};
  sa.grads = grads;
  sa.e = e;
  sa.bits = c.cur.bits;
  sa.tile_off = c.cur.tile_off;
  sa.b = c.w.b;
  sa.m = m;
  sa.v = v;
  sa.w = params;
  sa.mold = c.w.mold;
  sa.b1 = b1;
  sa.b2 = b2;
  sa.c1 = c1;
  sa.c2 = c2;
  sa.ibc1 = bias ? 0.0f : bias_reciprocal(b1, step);
  sa.ibc2 = bias ? 0.0f : bias_reciprocal(b2, step);
  sa.ibc_dev = bias ? &bias->ibc1 : nullptr;  // ibc2 follows ibc1
  sa.eps = betas.eps;
  sa.wd = betas.weight_decay;
  sa.lr = lr;
  sa.lo = c.cur.meta + g.P;
  sa.cand = c.w.sel.cand;
  sa.cnt1 = c.w.sel.cnt1;
  sa.hist = c.w.sel.hist;
  sa.p0 = 0;
  sa.nparts = g.P;
  sa.e_stride = g.n;

  if (bias && (st = hip_check(launch_bias_step(bias, b1, b2, stream), "bias step"))) return st;
  if (!bias && step == 1) {  // bootstrap: M_1 = top-k of the step-1 statistic
    if (c.prof) g_prof.begin(ST_BOOT, stream);
    StatArgs boot = a;
    boot.mold = nullptr;
    if ((st = run_fresh_select(g, c.w, kSrcState, boot, c.vec, c.cur, stream))) return st;
  }
  if (c.prof) g_prof.begin(ST_PASS, stream);
  return hip_check(launch_zero_u32(c.w.sel.hist + (int64_t)g.sp0 * kBins, (int64_t)g.snp * kBins, stream), "zero");
}

scape_status step_end(StepCtx& c, hipStream_t stream) {
  const Geom& g = c.g;
  scape_status st;
  if (c.prof) g_prof.begin(ST_SELECT, stream);
  if ((st = hip_check(launch_level1(g, c.w.sel, kScanCheck, stream), "level 1"))) return st;
  if ((st = run_fallback(g, c.w, kSrcMasked, c.a, c.vec, stream))) return st;
  st = run_tail(g, c.w, c.nxt, stream, c.prof);
  if (c.prof) g_prof.end();
  return st;
}

// Events of the offload pipeline, created once per device on first use:
// per stage buffer, "copied in", "pass done" and "copied out", plus the
// call's start.  A call holds g_oev_lock while it enqueues, so that every
// wait it enqueues refers to a record of the same call (a wait takes the
// event's latest record at the time it is enqueued).
constexpr int kMaxDevices = 64;
struct OffloadEvents {
  bool ready = false;
  hipEvent_t in[2], pass[2], out[2], start;
};
OffloadEvents g_oev[kMaxDevices];
std::mutex g_oev_lock;

scape_status offload_events(OffloadEvents** out) {
  int dev = -1;
  scape_status st = hip_check(hipGetDevice(&dev), "offload device");
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(SCAPE_EHIP, "offload: device %d out of range", dev);
  OffloadEvents& ev = g_oev[dev];
  if (!ev.ready) {
    hipEvent_t* all[7] = {&ev.in[0], &ev.in[1], &ev.pass[0], &ev.pass[1], &ev.out[0], &ev.out[1], &ev.start};
    for (hipEvent_t* e : all)
      if ((st = hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "offload events"))) return st;
    ev.ready = true;
  }
  *out = &ev;
  return SCAPE_OK;
}

// Scratch of scape_step_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  Host code never passes `scratch`
// itself (a host-side stand-in for the symbol) to a kernel: each device's
// address is looked up once, with that device current, and kept.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_lock;

scape_status static_scratch(void** out) {
  int dev = -1;
  scape_status st = hip_check(hipGetDevice(&dev), "static scratch device");
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(SCAPE_EHIP, "static scratch: device %d out of range", dev);
  std::lock_guard<std::mutex> hold(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((st = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "static scratch address"))) return st;
    if (!ptr) return fail(SCAPE_EHIP, "static scratch address: null on device %d", dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SCAPE_OK;
}

int64_t chunk_parts_of(const Geom& g, int32_t chunk_parts) {
  return chunk_parts < 1 ? 0 : (chunk_parts > g.P ? g.P : chunk_parts);
}

}  // namespace

extern "C" {

scape_status scape_step(const scape_dims* dims, float* params, const float* grads, float* m,
                        float* v, float* e, void* mask_blob, int64_t k, scape_betas betas, float lr,
                        int64_t step, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  StepCtx c;
  scape_status st = step_begin(c, dims, params, grads, m, v, e, mask_blob, k, betas, lr, step, workspace,
                               workspace_bytes, stream);
  if (st) return st;
  const bool vec = c.vec && aligned16(params) && aligned16(v);
  const bool seg = vec && seg_ok(c.g, params, m, v);
  if ((st = hip_check(launch_step_passes(c.g, c.sa, vec, seg, stream), "step pass"))) return st;
  return step_end(c, stream);
}

size_t scape_step_noalloc_max_bytes(void) { return kStaticScratchBytes; }

scape_status scape_step_noalloc(const scape_dims* dims, float* params, const float* grads, float* m,
                                float* v, float* e, void* mask_blob, int64_t k, scape_betas betas, float lr,
                                int64_t step, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (g.ws_total > kStaticScratchBytes)
    return fail(SCAPE_EWORKSPACE,
                "scape_step_noalloc: n=%lld P=%d K=%d k=%lld needs %zu bytes of scratch, more than the %zu bytes "
                "of static scratch; call scape_step with a workspace",
                (long long)g.n, g.P, g.K, (long long)g.k, g.ws_total, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws))) return st;
  StepCtx c;
  if ((st = step_begin(c, dims, params, grads, m, v, e, mask_blob, k, betas, lr, step, ws, g.ws_total, stream,
                       nullptr, 0, false)))
    return st;
  const bool vec = c.vec && aligned16(params) && aligned16(v);
  const bool seg = vec && seg_ok(c.g, params, m, v);
  if ((st = hip_check(launch_step_passes(c.g, c.sa, vec, seg, stream), "step pass"))) return st;
  return step_end(c, stream);
}

scape_status scape_bias_state_at(scape_betas betas, int64_t steps_done, scape_bias_state* out) {
  scape_status st = check_betas(betas, 1.0f);
  if (st) return st;
  if (!out) return fail(SCAPE_EINVAL, "out is null");
  if (steps_done < 0) return fail(SCAPE_EINVAL, "steps_done must be >= 0");
  double p1 = 1.0, p2 = 1.0;
  for (int64_t i = 0; i < steps_done; ++i) {
    p1 = p1 * (double)betas.beta1;
    p2 = p2 * (double)betas.beta2;
  }
  out->beta1_pow = p1;
  out->beta2_pow = p2;
  out->ibc1 = steps_done ? bias_reciprocal(betas.beta1, steps_done) : 0.0f;
  out->ibc2 = steps_done ? bias_reciprocal(betas.beta2, steps_done) : 0.0f;
  return SCAPE_OK;
}

scape_status scape_step_graph(const scape_dims* dims, float* params, const float* grads, float* m, float* v,
                              float* e, void* mask_blob, int64_t k, scape_betas betas, float lr, int32_t cur_slot,
                              scape_bias_state* bias, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!bias) return fail(SCAPE_EINVAL, "null pointer argument");
  StepCtx c;
  scape_status st = step_begin(c, dims, params, grads, m, v, e, mask_blob, k, betas, lr, 2, workspace,
                               workspace_bytes, stream, bias, cur_slot);
  if (st) return st;
  const bool vec = c.vec && aligned16(params) && aligned16(v);
  const bool seg = vec && seg_ok(c.g, params, m, v);
  if ((st = hip_check(launch_step_passes(c.g, c.sa, vec, seg, stream), "step pass"))) return st;
  return step_end(c, stream);
}

size_t scape_offload_stage_bytes(const scape_dims* dims, int64_t k, int32_t chunk_parts) {
  Geom g;
  if (!dims || !make_geom(dims->n, dims->num_partitions, dims->num_workers, k, &g)) return 0;
  const int64_t cp = chunk_parts_of(g, chunk_parts);
  return cp ? 2 * (size_t)g.K * (size_t)cp * (size_t)g.n_p * 4 : 0;
}

scape_status scape_step_offload(const scape_dims* dims, float* params, const float* grads, float* m,
                                float* v, float* e_host, void* mask_blob, int64_t k, scape_betas betas,
                                float lr, int64_t step, void* workspace, size_t workspace_bytes, void* stage,
                                size_t stage_bytes, int32_t chunk_parts, hipStream_t stream,
                                hipStream_t copy_in, hipStream_t copy_out) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  const int64_t cp = chunk_parts_of(g, chunk_parts);
  if (cp == 0) return fail(SCAPE_EINVAL, "chunk_parts must be >= 1");
  if (!stage) return fail(SCAPE_EINVAL, "null pointer argument");
  const size_t need = scape_offload_stage_bytes(dims, k, chunk_parts);
  if (stage_bytes < need) return fail(SCAPE_EWORKSPACE, "stage has %zu bytes, needs %zu", stage_bytes, need);
  if (copy_in == copy_out || copy_in == stream || copy_out == stream)
    return fail(SCAPE_EINVAL, "stream, copy_in and copy_out must be three distinct streams");
  StepCtx c;
  if ((st = step_begin(c, dims, params, grads, m, v, e_host, mask_blob, k, betas, lr, step, workspace,
                       workspace_bytes, stream)))
    return st;
  std::lock_guard<std::mutex> hold(g_oev_lock);
  OffloadEvents* ev = nullptr;
  if ((st = offload_events(&ev))) return st;
  OffloadEvents& oev = *ev;
  const int64_t n_p = g.n_p, chunk = cp * n_p;
  float* sbuf[2] = {static_cast<float*>(stage), static_cast<float*>(stage) + (size_t)g.K * chunk};
  const bool vec = c.vec && aligned16(params) && aligned16(v) && aligned16(stage) && (chunk % 4 == 0);
  const bool seg = vec && seg_ok(g, params, m, v);
  // the copies of this call follow everything already on the compute stream
  if ((st = hip_check(hipEventRecord(oev.start, stream), "offload record"))) return st;
  if ((st = hip_check(hipStreamWaitEvent(copy_in, oev.start, 0), "offload wait"))) return st;
  const int64_t nchunks = (g.P + cp - 1) / cp;
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int b = (int)(ci & 1);
    const int64_t p0 = ci * cp;
    const int64_t np = (p0 + cp <= g.P) ? cp : g.P - p0;
    // stage buffer b is free once the copy-out of chunk ci - 2 is done
    if (ci >= 2 && (st = hip_check(hipStreamWaitEvent(copy_in, oev.out[b], 0), "offload wait"))) return st;
    for (int i = 0; i < g.K; ++i) {
      st = hip_check(hipMemcpyAsync(sbuf[b] + (size_t)i * chunk, e_host + (size_t)i * g.n + (size_t)p0 * n_p,
                                    (size_t)np * n_p * 4, hipMemcpyHostToDevice, copy_in),
                     "offload copy in");
      if (st) return st;
    }
    if ((st = hip_check(hipEventRecord(oev.in[b], copy_in), "offload record"))) return st;
    if ((st = hip_check(hipStreamWaitEvent(stream, oev.in[b], 0), "offload wait"))) return st;
    StepArgs sa = c.sa;
    sa.e = sbuf[b];
    sa.p0 = (int)p0;
    sa.nparts = (int)np;
    sa.e_stride = chunk;
    if ((st = hip_check(launch_step_pass(g, sa, vec, seg, stream), "step pass"))) return st;
    if ((st = hip_check(hipEventRecord(oev.pass[b], stream), "offload record"))) return st;
    if ((st = hip_check(hipStreamWaitEvent(copy_out, oev.pass[b], 0), "offload wait"))) return st;
    for (int i = 0; i < g.K; ++i) {
      st = hip_check(hipMemcpyAsync(e_host + (size_t)i * g.n + (size_t)p0 * n_p, sbuf[b] + (size_t)i * chunk,
                                    (size_t)np * n_p * 4, hipMemcpyDeviceToHost, copy_out),
                     "offload copy out");
      if (st) return st;
    }
    if ((st = hip_check(hipEventRecord(oev.out[b], copy_out), "offload record"))) return st;
  }
  // the selection's fallback reads e_host: wait for every copy-out
  for (int b = 0; b < 2 && b < nchunks; ++b)
    if ((st = hip_check(hipStreamWaitEvent(stream, oev.out[b], 0), "offload wait"))) return st;
  return step_end(c, stream);
}

}  // extern "C"

namespace {

// The partitions rank r owns, floor(p*K/P) == r: [ceil(r*P/K), ceil((r+1)*P/K)).
void owned_range(const Geom& g, int r, int* lo, int* hi) {
  *lo = (int)(((int64_t)r * g.P + g.K - 1) / g.K);
  *hi = (int)(((int64_t)(r + 1) * g.P + g.K - 1) / g.K);
}

// Validation shared by the shard calls; on success g holds the geometry with
// the selection restricted to the rank's partitions.
scape_status shard_geom(const scape_dims* dims, int64_t k, int32_t rank, Geom* g) {
  scape_status st = check_dims(dims, k, g);
  if (st) return st;
  if (rank < 0 || rank >= g->K) return fail(SCAPE_EINVAL, "rank %d outside [0, %d)", rank, g->K);
  int lo, hi;
  owned_range(*g, rank, &lo, &hi);
  g->sp0 = lo;
  g->snp = hi - lo;
  return SCAPE_OK;
}

}  // namespace

extern "C" {

scape_status scape_shard_partitions(const scape_dims* dims, int32_t rank, int32_t* first, int32_t* count) {
  Geom g;
  scape_status st = shard_geom(dims, 1, rank, &g);
  if (st) return st;
  if (!first || !count) return fail(SCAPE_EINVAL, "null pointer argument");
  *first = g.sp0;
  *count = g.snp;
  return SCAPE_OK;
}

scape_status scape_shard_select_initial(const scape_dims* dims, int64_t k, int32_t rank, const float* grads,
                                        const float* e, const float* m, void* mask_blob, scape_betas betas,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Geom g;
  scape_status st = shard_geom(dims, k, rank, &g);
  if (st) return st;
  if (!grads || !e || !m || !mask_blob || !workspace) return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = check_betas(betas, 1.0f))) return st;
  if (workspace_bytes < g.ws_total)
    return fail(SCAPE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, g.ws_total);
  if (g.snp < 1) return SCAPE_OK;  // this rank owns no partition
  Ws w = ws_view(g, workspace);
  StatArgs a{};
  a.m = m;
  a.grads = grads;
  a.e = e;
  a.b1 = betas.beta1;
  a.c1 = 1.0f - betas.beta1;
  a.single_row = true;
  const bool vec = (g.n_p % 4 == 0) && aligned16(grads) && aligned16(e) && aligned16(m);
  return run_fresh_select(g, w, kSrcState, a, vec, slot_view(g, mask_blob, 0), stream);
}

scape_status scape_shard_compress(const scape_dims* dims, int64_t k, int32_t rank, const float* grads, float* e,
                                  const float* m, float* b, void* mask_blob, scape_betas betas, int64_t step,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Geom g;
  scape_status st = shard_geom(dims, k, rank, &g);
  if (st) return st;
  if (!grads || !e || !m || !b || !mask_blob || !workspace) return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = check_betas(betas, 1.0f))) return st;
  if (step < 1) return fail(SCAPE_EINVAL, "step must be >= 1");
  if (workspace_bytes < g.ws_total)
    return fail(SCAPE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, g.ws_total);
  Ws w = ws_view(g, workspace);
  const scape_mask_view cur = slot_view(g, mask_blob, (int)((step - 1) & 1));
  const scape_mask_view nxt = slot_view(g, mask_blob, (int)(step & 1));
  const float b1 = betas.beta1, c1 = 1.0f - betas.beta1;
  const bool vec = (g.n_p % 4 == 0) && aligned16(grads) && aligned16(e) && aligned16(m);
  const bool prof = g_prof.on;
  if (g.snp > 0 &&
      (st = hip_check(launch_zero_u32(w.sel.hist + (int64_t)g.sp0 * kBins, (int64_t)g.snp * kBins, stream), "zero")))
    return st;
  if (prof) g_prof.begin(ST_PASS, stream);
  if ((st = hip_check(launch_shard_pass(g, rank, grads, e, cur.bits, cur.tile_off, b, m, b1, c1, cur.meta + g.P,
                                        w.sel.cand, w.sel.cnt1, w.sel.hist, vec, stream),
                      "shard pass")))
    return st;
  if (g.snp < 1) {  // this rank owns no partition: nothing to select
    if (prof) g_prof.end();
    return SCAPE_OK;
  }
  if (prof) g_prof.begin(ST_SELECT, stream);
  if ((st = hip_check(launch_level1(g, w.sel, kScanCheck, stream), "level 1"))) return st;
  StatArgs a{};
  a.m = m;  // not yet updated: the update of this step comes after the reduction across ranks
  a.grads = grads;
  a.e = e;
  a.b = b;
  a.bits = cur.bits;
  a.tile_off = cur.tile_off;
  a.b1 = b1;
  a.c1 = c1;
  a.single_row = true;
  if ((st = run_fallback(g, w, kSrcMasked, a, vec, stream))) return st;
  st = run_tail(g, w, nxt, stream, prof);
  if (prof) g_prof.end();
  return st;
}

scape_status scape_shard_update(const scape_dims* dims, int64_t k, int32_t rank, float* params, float* m, float* v,
                                const float* b_bar, void* mask_blob, scape_betas betas, float lr, int64_t step,
                                hipStream_t stream) {
  Geom g;
  scape_status st = shard_geom(dims, k, rank, &g);
  if (st) return st;
  // v is optional, and b_bar may be null for a rank that owns no partition
  if (!params || !m || !mask_blob || (g.snp > 0 && !b_bar)) return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = check_betas(betas, lr))) return st;
  if (step < 1) return fail(SCAPE_EINVAL, "step must be >= 1");
  if (g.snp < 1) return SCAPE_OK;
  const scape_mask_view cur = slot_view(g, mask_blob, (int)((step - 1) & 1));
  const float b1 = betas.beta1, b2 = betas.beta2;
  return hip_check(launch_adams(g, b_bar, cur.idx + (int64_t)g.sp0 * g.k, params, m, v, b1, b2, 1.0f - b1, 1.0f - b2,
                                bias_reciprocal(b1, step), bias_reciprocal(b2, step), betas.eps, betas.weight_decay,
                                lr, stream, (int64_t)g.snp * g.k),
                   "shard update");
}

scape_status scape_dense_adams_step(const scape_dims* dims, float* params, const float* grads, float* m,
                                   float* v, scape_betas betas, float lr, int64_t step, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, 1, &g);
  if (st) return st;
  if (!params || !grads || !m) return fail(SCAPE_EINVAL, "null pointer argument");  // v is optional
  if ((st = check_betas(betas, lr))) return st;
  if (step < 1) return fail(SCAPE_EINVAL, "step must be >= 1");
  const float b1 = betas.beta1, b2 = betas.beta2;
  const bool vec = (g.n % 4 == 0) && aligned16(params) && aligned16(grads) && aligned16(m) && aligned16(v);
  return hip_check(launch_dense_adams(g, grads, params, m, v, b1, b2, 1.0f - b1, 1.0f - b2,
                                      bias_reciprocal(b1, step), bias_reciprocal(b2, step), betas.eps,
                                      betas.weight_decay, lr, vec, stream),
                   "dense adams");
}

scape_status scape_mask_overlap(const scape_dims* dims, int64_t k, scape_mask_view a,
                                scape_mask_view b, uint64_t* count_out, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!a.bits || !b.bits || !count_out) return fail(SCAPE_EINVAL, "null pointer argument");
  return hip_check(launch_overlap(g, a.bits, b.bits, count_out, stream), "overlap");
}

scape_status scape_mask_union(const scape_dims* dims, int64_t k, uint64_t* acc_bits, scape_mask_view m,
                              uint64_t* count_out, hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!acc_bits || !m.bits || !count_out) return fail(SCAPE_EINVAL, "null pointer argument");
  return hip_check(launch_union(g, acc_bits, m.bits, count_out, stream), "union");
}

scape_status scape_count_nonfinite(const float* x, int64_t count, uint64_t* nonfinite_out, hipStream_t stream) {
  if (count < 0) return fail(SCAPE_EINVAL, "count must be >= 0");
  if (count == 0) return SCAPE_OK;
  if (!x || !nonfinite_out) return fail(SCAPE_EINVAL, "null pointer argument");
  return hip_check(launch_count_nonfinite(x, count, nonfinite_out, stream), "count non-finite");
}

scape_status scape_mask_check(const scape_dims* dims, int64_t k, scape_mask_view m, uint32_t* result,
                              hipStream_t stream) {
  Geom g;
  scape_status st = check_dims(dims, k, &g);
  if (st) return st;
  if (!m.bits || !m.idx || !m.tile_off || !result) return fail(SCAPE_EINVAL, "null pointer argument");
  if ((st = hip_check(launch_mask_check(g, m.bits, m.idx, m.tile_off, m.meta, result, stream), "mask check")))
    return st;
  std::vector<uint32_t> res((size_t)g.P);
  if ((st = hip_check(hipMemcpyAsync(res.data(), result, (size_t)g.P * 4, hipMemcpyDeviceToHost, stream),
                      "mask check copy")))
    return st;
  if ((st = hip_check(hipStreamSynchronize(stream), "mask check sync"))) return st;
  int64_t nbad = 0, first = -1;
  for (int p = 0; p < g.P; ++p)
    if (res[p]) {
      if (first < 0) first = p;
      ++nbad;
    }
  if (!nbad) return SCAPE_OK;
  const uint32_t r = res[first];
  return fail(SCAPE_EMASK,
              "%lld of %d partitions violate the partitioned top-k contract; first: partition %lld:%s%s%s%s",
              (long long)nbad, g.P, (long long)first, (r & kMaskBadFault) ? " selection fault recorded;" : "",
              (r & kMaskBadCount) ? " bit count or tile offsets differ from k;" : "",
              (r & kMaskBadIdx) ? " index list does not match the bits;" : "",
              (r & kMaskBadPad) ? " bits set past the partition end;" : "");
}

const char* scape_status_string(scape_status s) {
  switch (s) {
    case SCAPE_OK: return "ok";
    case SCAPE_EINVAL: return "invalid argument";
    case SCAPE_ESHAPE: return "invalid shape";
    case SCAPE_EWORKSPACE: return "workspace too small";
    case SCAPE_EHIP: return "HIP error";
    case SCAPE_EMASK: return "mask violates the partitioned top-k contract";
  }
  return "unknown status";
}

const char* scape_last_error(void) { return g_err; }

int scape_profile_stages(void) { return ST_COUNT; }

const char* scape_profile_stage_name(int stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "";
}

scape_status scape_profile_enable(int on) {
  g_prof.end();
  g_prof.on = on != 0;
  return SCAPE_OK;
}

scape_status scape_profile_collect(double* ms_out, int64_t* count_out) {
  if (!ms_out || !count_out) return fail(SCAPE_EINVAL, "null pointer argument");
  g_prof.end();
  for (int i = 0; i < ST_COUNT; ++i) {
    ms_out[i] = 0.0;
    count_out[i] = 0;
  }
  scape_status st = SCAPE_OK;
  for (Rec& r : g_prof.recs) {
    float ms = 0.f;
    if (st == SCAPE_OK) {
      hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess) st = hip_check(e, "profile events");
    }
    ms_out[r.stage] += ms;
    count_out[r.stage] += 1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.recs.clear();
  if (g_prof.bad && st == SCAPE_OK) st = fail(SCAPE_EHIP, "profile: an event could not be created or recorded");
  g_prof.bad = false;
  return st;
}

}  // extern "C"
