/*
 * scape.h — C ABI of libscape.so: SCAPE's per-step sparse optimizer path on
 * one MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [P] SCAPE paper (Zheng, Chen, Xie, Zhang; arXiv 2607.01678, Chinese
 *       translation): §II-A sharded data parallelism, §II-B top-k with error
 *       feedback, §II-C AdamS eq. (2) and the bias-correction remark.
 *   [S] "Sintesi Tecnica: SCAPE" (technical summary), §2 "Componenti del
 *       Design del Sistema": partitioned mask synchronisation, one-step
 *       mask lag, single-buffer second-moment rebuild, single-bit packed
 *       masks ("Ottimizzazione della Memoria").
 *
 * Model.  The optimizer state is one flat fp32 buffer of n parameters cut
 * into P equal contiguous partitions of n_p = n / P elements (the even
 * optimizer shards of [P] §II-A).  K data-parallel workers are simulated on
 * the one device: worker i's gradient and error-feedback buffer are rows i
 * of [K][n] arrays.  Partition p is owned by worker floor(p*K/P).  In every
 * partition the mask selects exactly k elements (k = per-partition count).
 *
 * Common rules for every call:
 *   - Pointers are DEVICE pointers unless stated; the caller allocates and
 *     owns every buffer, including workspaces and mask blobs.  The library
 *     never allocates or frees device memory and keeps no state between
 *     calls, except the HIP events that scape_step_offload creates once
 *     per device and the stage timing creates while it is on.
 *   - Arguments are validated synchronously before anything is enqueued; a
 *     failed check returns a status and touches no buffer.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Calls on the same buffers must use one stream.  A launch failure
 *     returns SCAPE_EHIP; device faults surface at the caller's next sync.
 *   - Limits: 1 <= P <= 65535, 1 <= K, n % P == 0, n < 2^32, 1 <= k <= n_p.
 *   - Arithmetic: IEEE binary32, each operation rounded separately (no
 *     contraction), correctly rounded sqrt and division, subnormals kept.
 *     Results are deterministic and match the CPU oracle bit for bit.
 */
#ifndef SCAPE_H
#define SCAPE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SCAPE_OK = 0,
  SCAPE_EINVAL = 1,     /* null pointer, bad hyper-parameter, step < 1     */
  SCAPE_ESHAPE = 2,     /* n, P, K or k outside the limits above           */
  SCAPE_EWORKSPACE = 3, /* workspace smaller than scape_workspace_bytes()  */
  SCAPE_EHIP = 4,       /* a HIP launch or event call failed               */
  SCAPE_EMASK = 5       /* scape_mask_check: a mask breaks the partitioned
                           top-k contract (k bits per partition, index list
                           and tile offsets on the bits, no selection fault) */
} scape_status;

/* n = total parameters, num_partitions = P, num_workers = K. */
typedef struct {
  int64_t n;
  int32_t num_partitions;
  int32_t num_workers;
} scape_dims;

/* AdamS hyper-parameters ([P] §II-C eq. (2)): beta1, beta2 in [0, 1),
 * eps > 0 and finite, weight_decay finite (lambda of eq. (2)). */
typedef struct {
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} scape_betas;

/*
 * One mask M (k selected elements per partition), three views of it:
 *   bits     u64[P * W], W = ceil(n_p / 64): partition p's bit j (local
 *            index j) is bit (j % 64) of word p*W + j/64; bits past n_p are
 *            zero.  This is the single-bit packed form of [S] §2.
 *   idx      u32[P * k]: global indices (p*n_p + j) in ascending order;
 *            partition p's k entries are idx[p*k .. p*k + k).
 *   tile_off u32[P * T], T = ceil(n_p / scape_tile_elems()): for tile t of
 *            partition p, the number of selected elements of p that lie
 *            before local index t*scape_tile_elems().
 *   meta     u32[3 * P] threshold record (may be null where a call does not
 *            need it): meta[p] = the k-th largest key of partition p in the
 *            selection that produced this mask; meta[P + p] = the key bound
 *            at which the next step captures selection candidates (any
 *            value is safe: a bound that captures fewer than k keys of a
 *            partition sends it through an exact recount, so it only
 *            affects speed, never the result); meta[2P + p] = fault bits of
 *            that selection, 0 when it selected exactly k elements (bit 0:
 *            the threshold search found no digit holding the k-th key; bit
 *            1: the emitted count was not k).  A nonzero fault word only
 *            arises from corrupted inputs or workspace; scape_mask_check
 *            reports it.
 * The sparse buffers b are laid out like idx: entry r of a buffer belongs to
 * element idx[r].
 */
typedef struct {
  uint64_t* bits;
  uint32_t* idx;
  uint32_t* tile_off;
  uint32_t* meta;
} scape_mask_view;

/* ---------------------------------------------------------------- layout */

/* Elements per compaction tile (the granularity of tile_off). */
int64_t scape_tile_elems(void);

/* Passes over the flat buffer that scape_step and scape_step_graph make
 * for these dims and k: 1 (every worker's rows in one pass) or K (one pass
 * per non-owner worker of each partition, then the owner's pass), chosen
 * by measured speed; the results are the same bit for bit.  -1 if dims/k
 * are invalid. */
int32_t scape_step_pass_count(const scape_dims* dims, int64_t k);

/* Bytes of a mask blob holding TWO mask slots (the current mask M_t and the
 * next one, for the one-step lag of [S] §2).  0 if dims/k are invalid. */
size_t scape_mask_bytes(const scape_dims* dims, int64_t k);

/* Fills *out with the views of slot 0 or 1 inside a blob of
 * scape_mask_bytes() bytes starting at mask_blob (device pointer, 256-byte
 * aligned).  Pure pointer arithmetic: nothing is read or written on the
 * device. */
scape_status scape_mask_slot(const scape_dims* dims, int64_t k, void* mask_blob, int slot,
                             scape_mask_view* out);

/* Bytes of scratch that scape_mask_topk and scape_step need (256-byte
 * aligned device memory; contents undefined before and after a call). */
size_t scape_workspace_bytes(const scape_dims* dims, int64_t k);

/* ------------------------------------------------------------ components */

/*
 * Partitioned top-k mask ([S] §2, partitioned mask synchronisation; [P]
 * abstract and §I): in each partition, select the k elements of stat[n]
 * with the largest |stat|, ties going to the lower index (|x| is ranked by
 * the binary32 pattern with the sign bit cleared, so -0 == +0 and NaN ranks
 * above +inf).  Writes bits, idx and tile_off of `out`, and meta when it is
 * not null; reads stat only.
 */
scape_status scape_mask_topk(const scape_dims* dims, int64_t k, const float* stat,
                             scape_mask_view out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Error-feedback compression at a fixed index set ([P] §II-B, with the
 * shared mask of [S] §2): for every worker i and element j,
 *   a = grads[i][j] + e[i][j];
 *   if j is in `cur`:  b[i][r] = a (r = position of j in cur.idx), e[i][j] = 0
 *   else:              e[i][j] = a.
 * grads [K][n] is read-only; e [K][n] is updated in place; b is [K][P*k].
 * Reads cur.bits and cur.tile_off (not cur.idx).
 */
scape_status scape_compress(const scape_dims* dims, int64_t k, const float* grads, float* e,
                            scape_mask_view cur, float* b, hipStream_t stream);

/*
 * Reduction of the K workers' sparse buffers ([S] §2, the single
 * synchronised sparse buffer): b_bar[r] = (((b[0][r] + b[1][r]) + ...) +
 * b[K-1][r]) * fp32(1/K), for r < P*k.  In a multi-GPU run this is the
 * sparse reduce-scatter; here the K buffers sit in the one device's HBM.
 */
scape_status scape_reduce_sparse(const scape_dims* dims, int64_t k, const float* b, float* b_bar,
                                 hipStream_t stream);

/*
 * AdamS at the masked indices ([P] §II-C eq. (2) with bias correction; [S]
 * §2, second moment rebuilt from the single buffer): for r < P*k with
 * j = cur.idx[r], x = b_bar[r], mo = m[j], wo = params[j]:
 *   mn = b1*mo + (1-b1)*x;  vn = b2*mo*mo + (1-b2)*x*x
 *   mh = mn / (1 - b1^step); vh = vn / (1 - b2^step)   (host-computed fp32
 *                                                        reciprocals)
 *   params[j] = wo - lr*(mh/(sqrt(vh) + eps) + weight_decay*wo)
 *   m[j] = mn; v[j] = vn (if v is not NULL).
 * Entries off the mask are untouched.  AdamS keeps no second moment: v_t is
 * rebuilt from m_{t-1} and the step's gradient every step ([P] §II-C), so
 * v is an optional output (NULL: not stored), written and never read.
 */
scape_status scape_adams_update(const scape_dims* dims, int64_t k, float* params, float* m,
                                float* v, const float* b_bar, scape_mask_view cur,
                                scape_betas betas, float lr, int64_t step, hipStream_t stream);

/* ------------------------------------------------------------ fused step */

/*
 * One SCAPE optimizer step t = `step` (>= 1) ([P] abstract, §II-B, §II-C;
 * [S] §2).  mask_blob holds two slots (scape_mask_bytes): the step applies
 * M_t from slot (t-1)&1 and writes M_{t+1} to slot t&1.
 *   t == 1: slot 0 is ignored and filled first with the top-k of the
 *           statistic below (bootstrap), so M_1 = M_2.
 *   The selection of M_{t+1} reads the threshold record of slot (t-1)&1
 *   (see scape_mask_view) to bound its candidate capture, and writes the
 *   record of slot t&1.
 *   1. a^i = grads[i] + e[i]; error-feedback compression at M_t; e updated
 *      in place.  The step makes one pass or K passes over the flat buffer
 *      (scape_step_pass_count; the same results bit for bit).  One pass
 *      walks every worker's rows of a tile together, sums the workers'
 *      values of each masked element in registers and writes only the
 *      owner's sparse buffer.  K passes compress, for every partition, one
 *      non-owner worker per pass into its sparse buffer in the workspace,
 *      then the owner's pass (steps 2 and 3) reads those buffers back.
 *   2. statistic per partition p with owner o: s = b1*m + (1-b1)*a^o, using
 *      m before this step's update; M_{t+1} = per-partition top-k of |s|.
 *   3. b_bar = worker mean of the sparse buffers; AdamS at M_t.
 * params, m [n], e [K][n] and mask_blob are in/out; grads [K][n] is
 * read-only; workspace as scape_workspace_bytes().  v [n] is an optional
 * output (NULL: not stored): the uncorrected v_t at the masked entries, as
 * in scape_adams_update.
 */
scape_status scape_step(const scape_dims* dims, float* params, const float* grads, float* m,
                        float* v, float* e, void* mask_blob, int64_t k, scape_betas betas, float lr,
                        int64_t step, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * scape_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments minus the
 * workspace, same results bit for bit.  The scratch is a static device
 * array inside the library: scape_step_noalloc_max_bytes() bytes (64 MiB)
 * per device, held from the library's first use on that device until the
 * process ends; its address is looked up on the first call on each device
 * (`stream` must belong to the current device).  Dims whose workspace
 * (scape_workspace_bytes) exceeds it are rejected with SCAPE_EWORKSPACE
 * before anything is enqueued.  The call allocates nothing; its scratch
 * needs no clearing between calls (the step initialises what it reads).
 * Every call on a device shares that device's scratch: calls that overlap
 * on one device (several streams or host threads) race and must not be
 * issued.  Stage timing records nothing for these calls.
 */
size_t scape_step_noalloc_max_bytes(void);
scape_status scape_step_noalloc(const scape_dims* dims, float* params, const float* grads, float* m,
                                float* v, float* e, void* mask_blob, int64_t k, scape_betas betas, float lr,
                                int64_t step, hipStream_t stream);

/*
 * Bias-correction state of the graph-capturable step, in DEVICE memory
 * (8-byte aligned): beta1_pow = beta1^t and beta2_pow = beta2^t after t
 * steps, as binary64 products of binary64(beta) taken one step at a time
 * (the same roundings as scape_step's host computation), and the fp32
 * reciprocals ibc1 = 1/(1 - beta1^t), ibc2 = 1/(1 - beta2^t) that step t
 * uses ([P] §II-C, the bias-correction remark).
 */
typedef struct {
  double beta1_pow;
  double beta2_pow;
  float ibc1;
  float ibc2;
} scape_bias_state;

/* The state after `steps_done` (>= 0) steps, computed on the host into *out
 * (host memory); copy it to the device before the first scape_step_graph.
 * For steps_done == 0 the reciprocals are 0 (unused). */
scape_status scape_bias_state_at(scape_betas betas, int64_t steps_done, scape_bias_state* out);

/*
 * One step t >= 2 of scape_step in a form a HIP graph can capture and
 * replay: nothing of it depends on host-side values that change from step
 * to step.  The mask of this step, M_t, is read from slot `cur_slot` (0 or
 * 1; scape_step's slot (t-1)&1) and M_{t+1} is written to slot 1-cur_slot.
 * `bias` (device) holds the state after t-1 steps on entry; the call's
 * first kernel advances it to step t, and the step uses its reciprocals.
 * There is no step-1 bootstrap: run step 1 with scape_step, then copy
 * scape_bias_state_at(betas, 1) to `bias`.  Stage timing records nothing
 * for these calls.  A graph of two calls (cur_slot 1, then 0) replays
 * steps t, t+1 for even t; the caller refills `grads` between replays.
 * Results equal scape_step's bit for bit.
 */
scape_status scape_step_graph(const scape_dims* dims, float* params, const float* grads, float* m, float* v,
                              float* e, void* mask_blob, int64_t k, scape_betas betas, float lr, int32_t cur_slot,
                              scape_bias_state* bias, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense AdamS on the worker mean: the baseline the pages compare SCAPE's
 * per-step time with ([P] abstract; [S] §4).  For every element j:
 *   x = (((grads[0][j] + grads[1][j]) + ...) + grads[K-1][j]) * fp32(1/K)
 *   then the AdamS update of scape_adams_update at j ([P] §II-C eq. (2)).
 * params, m [n] in/out; v [n] an optional output (NULL: not stored);
 * grads [K][n] read-only.  No error feedback, no mask, no workspace.
 * dims->num_partitions only has to divide n.
 */
scape_status scape_dense_adams_step(const scape_dims* dims, float* params, const float* grads, float* m,
                                   float* v, scape_betas betas, float lr, int64_t step, hipStream_t stream);

/*
 * ---- One rank's share of the sharded step ----
 * In a run over K GPUs each rank is one worker and the owner of the
 * partitions p with floor(p*K/P) == rank; the mask generation is
 * distributed like the optimizer's shards ([P] abstract and §I; [S] §2,
 * partitioned mask synchronisation).  Per step t a rank calls, in order:
 *   scape_shard_compress  its own rows at M_t over every partition, and the
 *                         selection of M_{t+1} on its own partitions;
 *   (the caller reduces the ranks' sparse buffers b over the K ranks, a
 *    sparse reduce-scatter: each rank receives b_bar for its partitions)
 *   scape_shard_update    AdamS on its partitions from that b_bar;
 *   (the caller all-gathers the updated parameters at M_t, and the ranks'
 *    parts of M_{t+1} (bits, idx, tile_off, meta) into every rank's blob,
 *    before step t+1's compression reads M_{t+1})
 * At t = 1 every rank first calls scape_shard_select_initial, and the
 * ranks' parts of M_1 are all-gathered, before the compression.  The
 * arithmetic equals scape_step's bit for bit: on one device, K ranks called
 * in turn on shared params/m/v/mask blob, with b_bar from
 * scape_reduce_sparse, reproduce scape_step.
 * grads and e are the rank's rows ([n] each; e in/out); b is the rank's
 * sparse buffer [P*k] (laid out like idx); m and params are [n] (a rank
 * reads and writes only its partitions' entries of m, params and v); the
 * workspace is scape_workspace_bytes() (a rank uses its partitions' parts).
 * A rank that owns no partition (K > P) only compresses.
 */

/* The partitions rank `rank` owns: *first, *count (possibly 0). */
scape_status scape_shard_partitions(const scape_dims* dims, int32_t rank, int32_t* first, int32_t* count);

/* Step-1 mask M_1 on the rank's partitions, written to slot 0: the top-k of
 * |b1*m + (1-b1)*(grads + e)| (the bootstrap of scape_step). */
scape_status scape_shard_select_initial(const scape_dims* dims, int64_t k, int32_t rank, const float* grads,
                                        const float* e, const float* m, void* mask_blob, scape_betas betas,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step t (>= 1): a = grads + e; at M_t (slot (t-1)&1, every partition):
 * b[r] = a at idx[r], e <- 0 there and a elsewhere.  On the rank's
 * partitions: statistic b1*m + (1-b1)*a with m before this step's update,
 * and M_{t+1} written to slot t&1 (those partitions only).  Stage timing,
 * while on, records its pass and its selection like scape_step's. */
scape_status scape_shard_compress(const scape_dims* dims, int64_t k, int32_t rank, const float* grads, float* e,
                                  const float* m, float* b, void* mask_blob, scape_betas betas, int64_t step,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step t: AdamS at M_t on the rank's partitions (scape_adams_update's rule)
 * with x = b_bar[r - first*k] for entries r in [first*k, (first+count)*k)
 * of the index list: b_bar holds count*k entries, the synchronised buffer
 * of the rank's partitions (NULL allowed when count is 0).  v is an
 * optional output (NULL: not stored). */
scape_status scape_shard_update(const scape_dims* dims, int64_t k, int32_t rank, float* params, float* m, float* v,
                                const float* b_bar, void* mask_blob, scape_betas betas, float lr, int64_t step,
                                hipStream_t stream);

/*
 * Error-feedback buffers offloaded to pinned host memory, with double
 * buffering ([P] §I: the EF buffers live in CPU memory, moved over the
 * CPU-GPU link; [S] §2 "Ottimizzazione della Memoria": CPU offload with
 * double buffering).  Same step and results as scape_step, except that
 * e_host ([K][n] fp32) is pinned host memory (hipHostMalloc, device
 * accessible).  The pass over e runs on chunks of chunk_parts partitions:
 * chunk c+1 is copied in on copy_in and chunk c-1 copied out on copy_out
 * while chunk c is processed on `stream`, through `stage`, a device buffer
 * of scape_offload_stage_bytes() bytes (two chunks).  The step-1 bootstrap
 * and the exact recount of the selection read e_host directly.  The three
 * streams must be distinct; `stream` waits for the last copy-out before
 * the call's selection work, so later work on `stream` sees the new e_host.
 * `stream`, copy_in and copy_out belong to the current device.  The
 * pipeline's HIP events are created once per device on first use and
 * shared by every call on that device; a call holds a process-wide lock
 * while it enqueues, so calls from several host threads are safe.
 */
size_t scape_offload_stage_bytes(const scape_dims* dims, int64_t k, int32_t chunk_parts);
scape_status scape_step_offload(const scape_dims* dims, float* params, const float* grads, float* m,
                                float* v, float* e_host, void* mask_blob, int64_t k, scape_betas betas,
                                float lr, int64_t step, void* workspace, size_t workspace_bytes, void* stage,
                                size_t stage_bytes, int32_t chunk_parts, hipStream_t stream,
                                hipStream_t copy_in, hipStream_t copy_out);

/*
 * Overlap of two masks: *count_out (device u64) = |A ∩ B| summed over all
 * partitions (the consecutive-step mask stability the [P] §I insight
 * rests on; divide by P*k for the fraction).  Reads a.bits and b.bits.
 */
scape_status scape_mask_overlap(const scape_dims* dims, int64_t k, scape_mask_view a,
                                scape_mask_view b, uint64_t* count_out, hipStream_t stream);

/*
 * Union of masks, for the fill-in effect of per-worker top-k ([P] §II-B:
 * when each worker keeps its own top-k indices, the synchronised global mask
 * is their union and fills in as workers are added; [S] §2, partitioned
 * mask synchronisation avoids it): acc_bits (device, words laid out like a
 * mask's bits) |= m.bits, then *count_out (device u64) = popcount(acc_bits).
 */
scape_status scape_mask_union(const scape_dims* dims, int64_t k, uint64_t* acc_bits, scape_mask_view m,
                              uint64_t* count_out, hipStream_t stream);

/*
 * Validation of one mask against the partitioned top-k contract ([S] §2:
 * exactly k selected elements per partition, one mask shared by every
 * worker): in every partition the bits hold exactly k elements and none
 * past n_p, tile_off matches the bits, idx lists the set bits in ascending
 * order, and (when m.meta is not null) the selection's fault word is 0.
 * result is a device buffer of u32[P] that receives per-partition reason
 * bits (1: fault word set; 2: bit count or tile offsets differ from k; 4:
 * idx does not match the bits; 8: bits past n_p).  Reads m.bits, m.idx,
 * m.tile_off and m.meta; SYNCHRONOUS: it waits for `stream` (and so for
 * any step that wrote the mask on it) and returns SCAPE_OK, or SCAPE_EMASK
 * with the first offending partition named in scape_last_error().
 */
scape_status scape_mask_check(const scape_dims* dims, int64_t k, scape_mask_view m, uint32_t* result,
                              hipStream_t stream);

/*
 * Debug count of non-finite inputs: *nonfinite_out (device u64) += the
 * number of NaN and +-inf values among x[0 .. count-1] (device fp32, any
 * alignment).  The pages' workloads are finite; the step computes on
 * whatever it is given (a NaN statistic sorts above +inf in the selection,
 * NaN and inf propagate through the compression and AdamS), so a caller
 * that wants its gradients checked calls this on them before the step, on
 * the same stream.  It accumulates: the caller zeroes the counter, and one
 * counter can cover several arrays.  count 0 launches nothing; count < 0,
 * or a null x or counter with count > 0, is SCAPE_EINVAL.
 */
scape_status scape_count_nonfinite(const float* x, int64_t count, uint64_t* nonfinite_out, hipStream_t stream);

/* -------------------------------------------------------------- utility */

const char* scape_status_string(scape_status s);
/* Detail of the last failing call on this thread (static storage). */
const char* scape_last_error(void);

/*
 * Stage timing with HIP events recorded on the caller's stream.  While
 * enabled, scape_step records an event pair around each of its stages.
 * scape_profile_collect waits for the recorded events, writes per-stage
 * total milliseconds and launch counts (arrays of scape_profile_stages()
 * entries, host memory) and clears the record.  Stage names come from
 * scape_profile_stage_name().  Not thread-safe: enable it only while a
 * single host thread makes calls.
 */
int scape_profile_stages(void);
const char* scape_profile_stage_name(int stage);
scape_status scape_profile_enable(int on);
scape_status scape_profile_collect(double* ms_out, int64_t* count_out);

#ifdef __cplusplus
}
#endif

#endif /* SCAPE_H */
