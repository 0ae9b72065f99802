"""Benchmark of the SCAPE optimizer step on one MI355X.

    python bench.py [--config llama1.8b] [--steps 5] [--warmup 2]

A step is one call of scape_step: error-feedback compression of all K
workers' gradients with the fused owner statistic, the partitioned top-k of
the next mask, the sparse reduction and AdamS at the current mask.  Inputs
(parameters, a pool of per-step gradient sets) are generated on the device
before the timed region; the timed region is bracketed by synchronisations
and holds exactly --steps calls.  Prints one JSON line.

Algorithmic bytes per step (what the method must move, independent of this
implementation):  B = (12K + 4 + (K+1)/8) * n + (8K + 24) * P * k, and
4 * P * k more where v_t is also stored (--store-v).  AdamS keeps no second
moment (it is rebuilt from m_{t-1} every step), so by default the step
stores none; the bench line also times the step that stores it.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CPU_WAIT_S = 600.0  # bound on every wait of the CPU baseline
# the other workloads measured after the headline one (each at most this many
# timed and warmup steps)
EXTRA_STEPS = 10
EXTRA_WARMUP = 3
# Workloads this small run in tens of microseconds a step: they are timed
# over SMALL_STEPS steps, so that the timed region is milliseconds long.
SMALL_N = 1 << 22
SMALL_STEPS = 200
# Device memory left free when the placement of e is chosen.
PLACE_MARGIN = 8 << 30
CPU_SHARE = 16  # host cores per GPU on the benchmark host
METRIC = "optimizer-step params/s + HBM GB/s (% peak), Llama-1.8B shape, 99% sparsity"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes_step(n, P, K, k, v_out=False):
    return (12 * K + 4 + (K + 1) / 8) * n + (8 * K + 24 + (4 if v_out else 0)) * P * k


def alg_bytes_step_pass(n, P, K, k, v_out=False, passes=1):
    """The step pass: every worker reads g and e and writes e, the owner
    statistic reads m, the owner's sparse buffer is written (the exact
    recount of the selection needs it), and AdamS reads w and writes w and m
    (and v, if stored) at the P*k masked elements (its m read is the
    statistic's).  As one pass (passes = 1) the mask words are read once and
    the workers' values are summed in registers, so the other K - 1 sparse
    buffers are not needed.  As K passes (one per non-owner worker, then the
    owner's) every pass reads the mask words, and each non-owner worker
    writes its sparse buffer, which the owner pass reads back.  Candidate
    captures and the saved pre-update m are implementation traffic, not
    counted."""
    per_masked = (16 if v_out else 12) + 4
    if passes > 1:
        return (12 * K + 4) * n + K * n / 8 + (8 * (K - 1) + per_masked) * P * k
    return (12 * K + 4) * n + n / 8 + per_masked * P * k


def _oracle_partition(name, p, seed, barrier, results):
    """One process: generate partition p's step-1 inputs with the host
    generator, wait for the others, then time one oracle step."""
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import scape_oracle as O
    from sparse_communication_distributed_amd import workload as W
    cfg = W.CONFIGS[name]
    g = np.stack([W.grads_partition(cfg, 1, i, p, seed) for i in range(cfg.K)])
    st = O.PartitionState.fresh(W.init_params_partition(cfg, p, seed), cfg.K)
    hp = O.Hyper.make(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.lr)
    barrier.wait(timeout=CPU_WAIT_S)
    t0 = time.perf_counter()
    O.step_partition(st, g, cfg.k, O.owner(p, cfg.P, cfg.K), hp, 1)
    results.put((p, time.perf_counter() - t0))


def cpu_baseline(cfg, seed, workers, log_fn):
    """The CPU oracle as it stands, on the host's cores: one process per
    partition (partitions are independent), `workers` partitions stepped at
    once.  The processes are fresh interpreters (spawned), since this runs
    after the GPU measurements, in a process that has initialised the GPU."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    parts = list(range(min(workers, cfg.P)))
    barrier = ctx.Barrier(len(parts) + 1)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_partition, args=(cfg.name, p, seed, barrier, results)) for p in parts]
    for pr in procs:
        pr.start()
    log_fn(f"cpu baseline: {len(parts)} oracle processes generating inputs")
    try:  # a process that dies breaks the barrier or starves the queue: no wait is unbounded
        barrier.wait(timeout=CPU_WAIT_S)
        t0 = time.perf_counter()
        times = [results.get(timeout=CPU_WAIT_S) for _ in parts]
        wall = time.perf_counter() - t0
    except Exception as exc:
        for pr in procs:
            pr.terminate()
        raise RuntimeError(f"cpu baseline: an oracle process failed or stalled ({type(exc).__name__})") from exc
    for pr in procs:
        pr.join()
    n = len(parts) * cfg.n_p
    log_fn(f"cpu baseline: {n} params in {wall:.1f} s wall")
    return {"value": n / wall, "unit": "params/s", "cores": len(parts), "kind": "oracle",
            "ms_per_step_equiv": cfg.n / (n / wall) * 1e3,
            "sample": f"step 1 of {len(parts)} of the {cfg.P} partitions ({n} params, {cfg.K} workers), "
                      f"one single-threaded numpy process per partition, inputs from the host generator, "
                      f"{wall:.1f} s wall (per-process {min(t for _, t in times):.1f}-{max(t for _, t in times):.1f} s)"}


def cpu_tiny_single_core(seed, log_fn, steps=3):
    """The whole tiny workload (n = 2^20, P = 4, K = 2) stepped by the oracle
    in this one process: median ms per step over steps 1..steps, inputs
    generated before each timed step."""
    from oracle import scape_oracle as O
    from sparse_communication_distributed_amd import workload as W
    cfg = W.CONFIGS["tiny"]
    hp = O.Hyper.make(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.lr)
    opt = O.OracleOptimizer(W.init_params(cfg, seed), cfg.P, cfg.K, cfg.k, hp)
    times = []
    for t in range(1, steps + 1):
        g = W.grads(cfg, t, seed)
        t0 = time.perf_counter()
        opt.step(g)
        times.append((time.perf_counter() - t0) * 1e3)
    ms = float(np.median(times))
    log_fn(f"cpu baseline: tiny workload on one core {ms:.1f} ms/step")
    return {"workload": "tiny", "n_params": cfg.n, "ms_per_step": ms, "params_per_s": cfg.n / (ms * 1e-3),
            "cores": 1, "steps": steps}


def stream_calibration(torch, dev, log_fn):
    """A plain copy of 1 GiB (read 1 GiB, write 1 GiB), five times: the
    known-size kernel that scales the HBM byte counters, and the streaming
    rate this device reaches."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    gbps = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    log_fn(f"calibration copy 1 GiB: {ms:.3f} ms, {gbps:.0f} GB/s (read+write)")
    del src, dst
    return {"kernel": "torch copy_ fp32 1 GiB", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
            "ms": ms, "GBps": gbps}


def fillin_study(S, W, cfg, seed, steps, log_fn):
    """Fill-in of per-worker top-k: after `steps` SCAPE steps, each worker i
    selects its own top-k of |g^i + e^i| per partition (the per-worker
    selection the pages contrast with the shared partitioned mask); the
    union of the first K' workers' masks is the global mask such a scheme
    must synchronise.  Reports |union| / (P k) for K' = 1..K; SCAPE's shared
    mask is exactly 1 by construction.  (The elementwise g + e for the study
    is a torch add: it is analysis glue, not the optimizer path.)"""
    import torch
    n, P, K, k = cfg.n, cfg.P, cfg.K, cfg.k
    dev = torch.device("cuda:0")
    params = torch.empty(n, dtype=torch.float32, device=dev)
    W.device_init_params(cfg, seed, params)
    opt = S.ScapeOptimizer(params, P, K, k, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.lr)
    sigma = W.device_sigma(cfg, seed, dev)
    g = torch.empty((K, n), dtype=torch.float32, device=dev)
    for t in range(1, steps + 1):
        W.device_grads(cfg, t, seed, sigma, g)
        opt.step(g)
    W.device_grads(cfg, steps + 1, seed, sigma, g)
    d = opt.d
    blob = torch.zeros(S.mask_bytes(d, k), dtype=torch.uint8, device=dev)
    mv = S.mask_slot(d, k, blob, 0)
    acc = torch.zeros_like(S.mask_slot_tensors(d, k, blob, 0)[0])
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    stat = torch.empty(n, dtype=torch.float32, device=dev)
    dens = []
    for i in range(K):
        torch.add(g[i], opt.e[i], out=stat)
        S.mask_topk(d, k, stat, mv, opt.ws)
        S.mask_union(d, k, acc, mv, cnt)
        dens.append(cnt.item() / (P * k))
        log_fn(f"fill-in: workers 1..{i + 1}: union density {dens[-1]:.3f} x (P k)")
    return {"metric": "fill-in of per-worker top-k masks: |union of K' workers' masks| / (P k)",
            "workload": cfg.name, "after_steps": steps, "union_density": dens,
            "shared_partitioned_mask_density": 1.0,
            "data": "synthetic: independent gradients per worker (the no-correlation case)"}


def offload_bench(S, W, cfg, args, log_fn):
    """The step with the error-feedback buffers in pinned host memory,
    staged through the device in chunks of partitions (two copy streams,
    double buffered).  Timed like the main benchmark, once per chunk size
    of --offload (comma-separated), in this one process on the same pinned
    buffer; `value` is the fastest."""
    import torch
    n, P, K, k = cfg.n, cfg.P, cfg.K, cfg.k
    chunks = [int(x) for x in str(args.offload).split(",") if x.strip()]
    dev = torch.device("cuda:0")
    d = S.dims(n, P, K)
    bt = S.betas(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay)
    params = torch.empty(n, dtype=torch.float32, device=dev)
    W.device_init_params(cfg, args.seed, params)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev) if args.store_v else None
    log_fn(f"pinning {K * n * 4 / 1e9:.1f} GB of host memory for e")
    e_host = torch.zeros((K, n), dtype=torch.float32, pin_memory=True)
    mask = torch.zeros(S.mask_bytes(d, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(S.workspace_bytes(d, k), dtype=torch.uint8, device=dev)
    sigma = W.device_sigma(cfg, args.seed, dev)
    pool = []
    for s_ in range(args.pool):
        gset = torch.empty((K, n), dtype=torch.float32, device=dev)
        W.device_grads(cfg, s_ + 1, args.seed, sigma, gset)
        pool.append(gset)
    del sigma
    stream = torch.cuda.current_stream()
    cin, cout = torch.cuda.Stream(), torch.cuda.Stream()
    t = 0
    runs = []
    for cp in chunks:
        stage = torch.empty(S.offload_stage_bytes(d, k, cp), dtype=torch.uint8, device=dev)

        def one_step():
            nonlocal t
            t += 1
            S.step_offload(d, params, pool[(t - 1) % len(pool)], m, v, e_host, mask, k, bt, cfg.lr, t, ws, stage,
                           cp, stream, cin, cout)

        for _ in range(args.warmup):
            one_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            one_step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        link = 2 * K * n * 4 / (ms * 1e-3) / 1e9
        log_fn(f"offload ({cp} partitions per chunk): {ms:.2f} ms/step, {link:.1f} GB/s over the host link")
        runs.append({"chunk_parts": cp, "ms_per_step": ms, "host_link_gbps_both_directions": link})
        del stage
    best = min(runs, key=lambda r: r["ms_per_step"])
    return {"metric": "optimizer-step params/s with e offloaded to pinned host memory",
            "value": n / (best["ms_per_step"] * 1e-3), "unit": "params/s", "ms_per_step": best["ms_per_step"],
            "steps": args.steps, "warmup": args.warmup, "chunk_parts": best["chunk_parts"], "runs": runs,
            "host_link_gbps_both_directions": best["host_link_gbps_both_directions"],
            "bytes_over_link_per_step": 2 * K * n * 4, "dtype": "f32", "data": "synthetic",
            "config": {"workload": cfg.name, "n_params": n, "partitions": P, "workers": K, "k_per_partition": k}}


def graph_bench(S, torch, d, params, pool, m, v, e, mask, k, bt, lr, steps_done, ws, steps, log_fn):
    """Two consecutive steps recorded once into a HIP graph through
    scape_step_graph (the step's slot and bias state on the device), then
    replayed: ms per step over `steps` replays of two steps each."""
    bias = S.bias_state_tensor(bt, steps_done, params.device)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        for j in range(2):
            S.step_graph(d, params, pool[j % len(pool)], m, v, e, mask, k, bt, lr, (steps_done + j) & 1, bias, ws)
    graph.replay()  # warm
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (2 * steps)
    log_fn(f"graph replay: {ms:.3f} ms/step ({steps} replays of 2 steps)")
    return {"ms_per_step": ms, "replays": steps, "steps_per_replay": 2}


def shard_bench(S, W, torch, cfg, args, log_fn):
    """One rank's share of the sharded step at the workload's layout with
    --shard ranks: the rank's compression of its own rows over every
    partition with the statistic and selection on its own partitions
    (scape_shard_compress), then AdamS on those partitions
    (scape_shard_update).  The reduction of the ranks' sparse buffers and
    the all-gathers run over the network in a multi-GPU run and are not
    timed; here the rank's own values stand in for the reduced buffer, and
    the other ranks' parts of the next mask are the current mask's (copied
    outside the timed region).  Rank 0 is timed."""
    K = args.shard
    cfg = cfg.with_(num_workers=K)
    n, P, k, n_p = cfg.n, cfg.P, cfg.k, cfg.n_p
    dev = torch.device("cuda:0")
    d = S.dims(n, P, K)
    bt = S.betas(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay)
    rank = 0
    first, count = S.shard_partitions(d, rank)
    log_fn(f"shard: {cfg.name} layout, {K} ranks: rank {rank} owns partitions {first}..{first + count - 1}")
    params = torch.empty(n, dtype=torch.float32, device=dev)
    W.device_init_params(cfg, args.seed, params)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    b = torch.zeros(P * k, dtype=torch.float32, device=dev)
    mask = torch.zeros(S.mask_bytes(d, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(S.workspace_bytes(d, k), dtype=torch.uint8, device=dev)
    sigma = W.device_sigma(cfg, args.seed, dev)
    rows = torch.empty((K, n), dtype=torch.float32, device=dev)
    pool = []
    for s_ in range(args.pool):  # the rank's gradient row of steps 1, 2, ...
        W.device_grads(cfg, s_ + 1, args.seed, sigma, rows)
        pool.append(rows[rank].clone())
    del rows, sigma
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    # M_1 for every partition (each rank's part from the same row)
    for r in range(K):
        S.shard_select_initial(d, k, r, pool[0], e, m, mask, bt, ws, stream)
    views = [S.mask_slot_tensors(d, k, mask, sl) + (S.mask_slot_meta(d, k, mask, sl),) for sl in (0, 1)]
    Wp, T = (n_p + 63) // 64, (n_p + 4095) // 4096

    def gather_other_parts(t):
        """The other ranks' parts of M_{t+1}: those of M_t (stand-in)."""
        src, dst = views[(t - 1) & 1], views[t & 1]
        for lo, hi in ((0, first), (first + count, P)):
            if hi <= lo:
                continue
            for (a_, b_), per in zip(zip(src[:3], dst[:3]), (Wp, k, T)):
                b_[lo * per:hi * per].copy_(a_[lo * per:hi * per])
            for j in range(3):
                dst[3][j * P + lo:j * P + hi].copy_(src[3][j * P + lo:j * P + hi])

    t = 0
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    c_ms, u_ms = [], []

    def one(timed):
        nonlocal t
        t += 1
        evs[0].record(stream)
        S.shard_compress(d, k, rank, pool[(t - 1) % len(pool)], e, m, b, mask, bt, t, ws, stream)
        evs[1].record(stream)
        S.shard_update(d, k, rank, params, m, None, b[first * k:(first + count) * k], mask, bt, cfg.lr, t, stream)
        evs[2].record(stream)
        gather_other_parts(t)
        if timed:
            torch.cuda.synchronize()
            c_ms.append(evs[0].elapsed_time(evs[1]))
            u_ms.append(evs[1].elapsed_time(evs[2]))

    for _ in range(args.warmup):
        one(False)
    torch.cuda.synchronize()
    S.profile_enable(True)
    for _ in range(args.steps):
        one(True)
    stages = S.profile_collect()
    S.profile_enable(False)
    stage_ms = {name: tot / c for name, (tot, c) in stages.items() if c}
    S.mask_check(d, k, S.mask_slot(d, k, mask, t & 1))
    cm, um = float(np.median(c_ms)), float(np.median(u_ms))
    n_own = count * n_p
    # the rank's pass: its rows (g read, e read and written), the mask
    # words, its sparse buffer written, m read on its partitions
    b_pass = 12 * n + n / 8 + 4 * P * k + 4 * n_own
    # the update: per entry of its partitions, b_bar and the index read, w
    # and m read and written
    b_upd = 24 * count * k
    pass_ms = stage_ms.get("step_pass", float("nan"))
    log_fn(f"shard: compress+select {cm:.3f} ms (pass {pass_ms:.3f} ms), update {um:.3f} ms")
    return {"metric": "one rank's share of the sharded SCAPE step (compression of its rows, selection and AdamS "
                      "on its partitions), ms per step",
            "value": cm + um, "unit": "ms", "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": cfg.name, "n_params": n, "partitions": P, "ranks": K, "rank": rank,
                       "owned_partitions": [first, count], "k_per_partition": k, "sparsity": cfg.sparsity},
            "compress_select_ms": cm, "update_ms": um, "stage_ms": stage_ms,
            "roofline": {"bound": "hbm", "kernel": "shard_pass_kernel", "achieved": b_pass / (pass_ms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": b_pass / (pass_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "bytes_alg_per_launch": b_pass, "ms_per_launch": pass_ms, "traffic": None},
            "update": {"bytes_alg": b_upd, "GBps_alg": b_upd / (um * 1e-3) / 1e9},
            "dtype": "f32", "data": "synthetic",
            "note": "local work only: the reduce-scatter of the sparse buffers and the all-gathers of "
                    "parameters and mask bits run over the network in a multi-GPU run"}


def counters_traffic(name, store_v):
    """HBM bytes per step pass from the committed counter summary of this
    workload, while it was taken from the step-pass code as it stands (the
    summary carries a hash of that code); None otherwise."""
    prof_path = os.path.join(ROOT, "profiles", f"step_pass_{name}_counters.json")
    if store_v or not os.path.exists(prof_path):  # the counters come from the v-less step
        return None
    from sparse_communication_distributed_amd.prof_summary import step_pass_source_hash
    with open(prof_path) as f:
        doc = json.load(f)
    if doc.get("source_hash") != step_pass_source_hash():
        return None
    return doc.get("hbm_bytes_per_step_pass")


def measure_workload(S, W, torch, cfg, args, steps, warmup, full, log_fn):
    """One workload on cuda:0: state and a pool of gradient sets generated on
    the device, `warmup` untimed steps, `steps` timed steps between two
    synchronisations, then a second (profiled) pass of `steps` steps with
    HIP-event stage timing on the launch stream and, for the stress law,
    the mask overlap of every step.  With `full`, also the dense AdamS
    baseline, the steps storing v, the graph replay (--graph), a step-1 call
    and the torch stream reference on the same tensors.  Everything is freed
    before returning."""
    n, P, K, k = cfg.n, cfg.P, cfg.K, cfg.k
    dev = torch.device("cuda:0")
    overlap = args.overlap or cfg.grad_law == "stress_t3"
    log_fn(f"config {cfg.name}: n={n} P={P} K={K} k={k} pool={args.pool} steps={steps} warmup={warmup}")
    d = S.dims(n, P, K)
    bt = S.betas(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay)

    def alloc_state():
        params = torch.empty(n, dtype=torch.float32, device=dev)
        W.device_init_params(cfg, args.seed, params)
        m = torch.zeros(n, dtype=torch.float32, device=dev)
        v = torch.zeros(n, dtype=torch.float32, device=dev) if args.store_v else None
        e = torch.zeros((K, n), dtype=torch.float32, device=dev)
        mask = torch.zeros(S.mask_bytes(d, k), dtype=torch.uint8, device=dev)
        ws = torch.empty(S.workspace_bytes(d, k), dtype=torch.uint8, device=dev)
        return params, m, v, e, mask, ws

    def alloc_grads():
        sigma = W.device_sigma(cfg, args.seed, dev)
        pool = []
        for s in range(args.pool):
            gset = torch.empty((K, n), dtype=torch.float32, device=dev)
            W.device_grads(cfg, s + 1, args.seed, sigma, gset)
            pool.append(gset)
            log_fn(f"{cfg.name}: gradient set {s + 1}/{args.pool} generated")
        del sigma
        return pool

    if args.grads_first:
        pool = alloc_grads()
        params, m, v, e, mask, ws = alloc_state()
    else:
        params, m, v, e, mask, ws = alloc_state()
        pool = alloc_grads()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    rec = {}
    if args.calib and full:
        rec["stream_calibration"] = stream_calibration(torch, dev, log_fn)

    t = 0

    def one_step(v_out=v):
        nonlocal t
        t += 1
        S.step(d, params, pool[(t - 1) % len(pool)], m, v_out, e, mask, k, bt, cfg.lr, t, ws, stream)

    # Placement of e (the error-feedback rows), chosen at setup: up to
    # --place - 1 more allocations of e, as free memory allows, each taking
    # e's role for two ordinary steps per round (S.choose_placement); the
    # fastest keeps it.  Untimed, before the warmup.
    if args.place > 1 and n > SMALL_N:
        # The gradient sets after the first lend their memory to more
        # allocations of e while the placement is chosen, so its steps all
        # take the first set.  Afterwards the state is put back to its
        # initial values (no step has run yet), the sets are generated
        # again, and the same number of ordinary steps runs over all of
        # them: the steps that follow are those of a run that cycled every
        # set from the start.
        assert t == 0
        lent = len(pool) - 1
        del pool[1:]
        torch.cuda.empty_cache()
        free, _ = torch.cuda.mem_get_info()
        ncand = int(min(args.place - 1, (free - PLACE_MARGIN) // (e.numel() * 4)))
        if ncand >= 1:
            cands = [torch.empty_like(e) for _ in range(ncand)]

            def run(x):
                nonlocal e
                e = x
                one_step()
                one_step()

            e, place_ms = S.choose_placement(e, cands, run, rounds=2)
            del cands
            torch.cuda.empty_cache()
            best = place_ms.index(min(place_ms))
            rec["e_placement"] = {"allocations": ncand + 1, "ms_per_2_steps": place_ms, "chosen": best,
                                  "steps": 4 * (ncand + 1), "gradient_sets_lent": lent}
            log_fn(f"{cfg.name}: e placement: {ncand + 1} allocations, two steps each "
                   f"{', '.join(f'{x:.2f}' for x in place_ms)} ms, kept #{best}")
        if lent:
            placed = t
            W.device_init_params(cfg, args.seed, params)
            for x in (m, v, e, mask):
                if x is not None:
                    x.zero_()
            t = 0
            sigma = W.device_sigma(cfg, args.seed, dev)
            for s in range(1, lent + 1):
                gset = torch.empty((K, n), dtype=torch.float32, device=dev)
                W.device_grads(cfg, s + 1, args.seed, sigma, gset)
                pool.append(gset)
            del sigma
            for _ in range(placed):
                one_step()
            torch.cuda.synchronize()

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    log_fn(f"{cfg.name}: warmup done ({warmup} steps)")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        one_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    log_fn(f"{cfg.name}: timed {steps} steps: {ms:.3f} ms/step")

    # per-stage durations of the same steps, recorded with HIP events on the
    # stream the kernels run on (a second, profiled pass of `steps` steps)
    S.profile_enable(True)
    overlaps = []
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        step_ev[i].record(stream)
        one_step()
        step_ev[i + 1].record(stream)
        if overlap:  # |M_t ∩ M_{t+1}| / (P k), outside the timed region
            S.mask_overlap(d, k, S.mask_slot(d, k, mask, (t - 1) & 1), S.mask_slot(d, k, mask, t & 1), cnt, stream)
            overlaps.append(cnt.item() / (P * k))
    torch.cuda.synchronize()
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(steps)]
    stages = S.profile_collect()
    S.profile_enable(False)
    stage_ms = {name: tot / c for name, (tot, c) in stages.items() if c}
    log_fn(f"{cfg.name}: stage ms: " + ", ".join(f"{kk}={vv:.3f}" for kk, vv in stage_ms.items()))
    # the masks the steps left are valid partitioned top-k masks (synchronous check)
    S.mask_check(d, k, S.mask_slot(d, k, mask, t & 1))
    S.mask_check(d, k, S.mask_slot(d, k, mask, (t - 1) & 1))

    b_step = alg_bytes_step(n, P, K, k, args.store_v)
    passes = S.step_pass_count(d, k)
    b_pass = alg_bytes_step_pass(n, P, K, k, args.store_v, passes)
    gbps = b_step / (ms * 1e-3) / 1e9
    pass_ms = stage_ms.get("step_pass", float("nan"))
    pass_gbps = b_pass / (pass_ms * 1e-3) / 1e9
    traffic = counters_traffic(cfg.name, args.store_v)
    rec.update({
        "workload": cfg.name, "n_params": n, "tensors": len(cfg.tensors), "partitions": P, "workers": K,
        "k_per_partition": k, "sparsity": cfg.sparsity, "gradient_law": cfg.grad_law,
        "steps": steps, "warmup": warmup, "ms_per_step": ms, "params_per_s": n / (ms * 1e-3),
        "hbm_gbps_alg": gbps, "hbm_frac_alg": gbps / HBM_PEAK_GBPS, "bytes_alg_per_step": b_step,
        "stage_ms": stage_ms, "profiled_step_ms": step_ms,
        "step_pass": {"kernel": "compress_kernel (step pass" + (": K - 1 worker passes, then the owner pass)"
                                                                 if passes > 1 else ")"),
                      "achieved": pass_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": pass_gbps / HBM_PEAK_GBPS,
                      "traffic": traffic, "bytes_alg_per_step_pass": b_pass, "ms_per_step_pass": pass_ms,
                      "launches_per_step_pass": passes,
                      "traffic_gbps": None if traffic is None else traffic / (pass_ms * 1e-3) / 1e9},
    })
    if overlaps:
        rec["mask_overlap"] = overlaps

    if full:
        # the pages' comparison point: dense AdamS on the worker mean, same
        # tensors, same number of steps (after the SCAPE measurements)
        ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev2.record(stream)
        for s_ in range(steps):
            S.dense_adams_step(d, params, pool[s_ % len(pool)], m, v, bt, cfg.lr, t + 1 + s_, stream)
        ev3.record(stream)
        torch.cuda.synchronize()
        dense_ms = ev2.elapsed_time(ev3) / steps
        log_fn(f"dense AdamS: {dense_ms:.3f} ms/step")
        b_dense = (4 * K + (20 if args.store_v else 16)) * n
        rec["dense_adams"] = {"ms_per_step": dense_ms, "params_per_s": n / (dense_ms * 1e-3),
                              "hbm_gbps_alg": b_dense / (dense_ms * 1e-3) / 1e9,
                              "hbm_frac_alg": b_dense / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "bytes_alg_per_step": b_dense, "note": "local cost only: no collective runs on one GPU"}

        # the same steps storing v_t as well (an output AdamS never reads back)
        if v is None:
            v_keep = torch.zeros(n, dtype=torch.float32, device=dev)
            one_step(v_keep)
            torch.cuda.synchronize()
            ev2.record(stream)
            for _ in range(steps):
                one_step(v_keep)
            ev3.record(stream)
            torch.cuda.synchronize()
            vs_ms = ev2.elapsed_time(ev3) / steps
            del v_keep
            log_fn(f"steps storing v: {vs_ms:.3f} ms/step")
            rec["step_storing_v"] = {"ms_per_step": vs_ms, "params_per_s": n / (vs_ms * 1e-3),
                                     "hbm_gbps_alg": alg_bytes_step(n, P, K, k, True) / (vs_ms * 1e-3) / 1e9}

        if args.graph:  # continues the SCAPE steps: t steps done, M_{t+1} in slot t & 1
            rec["graph"] = graph_bench(S, torch, d, params, pool, m, v, e, mask, k, bt, cfg.lr, t, ws, steps, log_fn)

        # a step-1 call (the bootstrap: statistic pass and fresh select of M_1
        # before the step pass), timed warm on the same tensors after
        # everything else, since its state afterwards is no longer used
        S.profile_enable(True)
        ev2.record(stream)
        S.step(d, params, pool[0], m, v, e, mask, k, bt, cfg.lr, 1, ws, stream)
        ev3.record(stream)
        torch.cuda.synchronize()
        boot_ms = ev2.elapsed_time(ev3)
        boot_stages = {name: tot for name, (tot, c) in S.profile_collect().items() if c}
        S.profile_enable(False)
        log_fn(f"bootstrap step (t = 1): {boot_ms:.3f} ms")
        rec["bootstrap_step"] = {"ms": boot_ms, "stage_ms": boot_stages}

        # a reference rate for the same allocations: torch's own elementwise
        # kernel adding every worker's gradient row into its error-feedback
        # row (read g, read e, write e: the step pass's 12K bytes per
        # element); last, since it changes e
        for i in range(K):
            e[i].add_(pool[0][i])
        ev2.record(stream)
        for _ in range(2):
            for i in range(K):
                e[i].add_(pool[0][i])
        ev3.record(stream)
        torch.cuda.synchronize()
        ref_ms = ev2.elapsed_time(ev3) / 2
        rec["stream_reference"] = {"kernel": "torch add_: e[i] += g[i] for every worker", "bytes": 12 * K * n,
                                   "ms": ref_ms, "GBps": 12 * K * n / (ref_ms * 1e-3) / 1e9}
        log_fn(f"reference stream (torch add_ over the e and g rows): {ref_ms:.3f} ms, "
               f"{rec['stream_reference']['GBps']:.0f} GB/s")
    del params, m, v, e, mask, ws, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def extra_workloads(spec, head, names):
    """The workloads --extra-configs names, in the order of `names`, without
    the headline one."""
    if spec == "none":
        return []
    if spec == "all":
        return [n for n in names if n != head]
    want = [x.strip() for x in spec.split(",") if x.strip()]
    bad = [x for x in want if x not in names]
    if bad:
        raise SystemExit(f"unknown workload(s) in --extra-configs: {', '.join(bad)}")
    return [n for n in names if n in want and n != head]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama1.8b")
    ap.add_argument("--pool", type=int, default=3, help="distinct gradient sets cycled through")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle processes for the CPU baseline (default: the usable cores, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-configs", default="all", metavar="all|none|NAME[,NAME...]",
                    help="workloads measured after --config, at most "
                         f"{EXTRA_STEPS} steps each ({SMALL_STEPS} for workloads of at most {SMALL_N} "
                         "parameters), reported under 'configs' (default: all the others)")
    ap.add_argument("--overlap", action="store_true",
                    help="report |M_t ∩ M_{t+1}| / (P k) per step (untimed; on by default for the stress workload)")
    ap.add_argument("--offload", default="", metavar="CHUNK_PARTS[,CHUNK_PARTS...]",
                    help="keep e in pinned host memory, staged in chunks of this many partitions "
                         "(several sizes: each timed in turn, in this process)")
    ap.add_argument("--graph", action="store_true",
                    help="also time two steps captured in a HIP graph (scape_step_graph) and replayed")
    ap.add_argument("--study", choices=["fillin"], default=None,
                    help="run a study instead of the step benchmark")
    ap.add_argument("--grads-first", action="store_true",
                    help="allocate the gradient sets before the optimizer state")
    ap.add_argument("--store-v", action="store_true",
                    help="the timed steps also store v_t at the masked entries (AdamS never reads it back)")
    ap.add_argument("--place", type=int, default=17, metavar="N",
                    help="choose the placement of e among up to N allocations (as free memory allows) at setup, "
                         "by timing ordinary steps (S.choose_placement; 1: keep the first)")
    ap.add_argument("--calib", action="store_true",
                    help="also time a plain device copy of 1 GiB (the counter calibration kernel)")
    ap.add_argument("--shard", type=int, default=0, metavar="RANKS",
                    help="time one rank's share of the sharded step at --config's layout with this many ranks")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the simulated workers share one device and no "
              "collective runs; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_communication_distributed_amd import scape as S
    from sparse_communication_distributed_amd import workload as W

    cfg = W.CONFIGS[args.config]
    if args.study == "fillin":
        S.lib()
        print(json.dumps(fillin_study(S, W, cfg, args.seed, args.warmup + args.steps, log)), flush=True)
        return
    if args.offload:
        S.lib()
        print(json.dumps(offload_bench(S, W, cfg, args, log)), flush=True)
        return
    if args.shard:
        S.lib()
        print(json.dumps(shard_bench(S, W, torch, cfg, args, log)), flush=True)
        return
    torch.cuda.set_device(torch.device("cuda:0"))
    S.lib()
    head = measure_workload(S, W, torch, cfg, args, args.steps, args.warmup, True, log)
    extras = {}
    for name in extra_workloads(args.extra_configs, cfg.name, W.CONFIGS):
        cfg_x = W.CONFIGS[name]
        steps_x = min(args.steps, EXTRA_STEPS) if cfg_x.n > SMALL_N else max(args.steps, SMALL_STEPS)
        extras[name] = measure_workload(S, W, torch, cfg_x, args, steps_x, min(args.warmup, EXTRA_WARMUP), False, log)

    # the oracle on the host's cores, after every GPU measurement: run
    # before them (forked, ahead of the GPU's initialisation), it left the
    # Llama-1.8B step pass at 17.64-17.73 ms in six processes of six, where
    # processes without it, and with it afterwards, ran 15.95-17.70 ms
    cpu = None
    if not args.no_cpu_baseline:
        # at most CPU_SHARE processes: the CPU share of one GPU on the
        # benchmark host, whatever the affinity mask shows (an oracle process
        # at the Llama-1.8B shape holds 3-4 GB)
        affinity = len(os.sched_getaffinity(0))
        workers = args.cpu_workers or min(CPU_SHARE, affinity)
        cpu = cpu_baseline(cfg, args.seed, workers, log)
        cpu["affinity_cores"] = affinity
        cpu["tiny_single_core"] = cpu_tiny_single_core(args.seed, log)

    sp = head["step_pass"]
    out = {
        "metric": METRIC,
        "value": head["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_params": cfg.n, "tensors": len(cfg.tensors), "partitions": cfg.P,
                   "workers": cfg.K, "k_per_partition": cfg.k, "sparsity": cfg.sparsity,
                   "gradient_law": cfg.grad_law, "gradient_sets": args.pool, "v_stored": bool(args.store_v)},
        "hbm_gbps_alg": head["hbm_gbps_alg"],
        "hbm_frac_alg": head["hbm_frac_alg"],
        "bytes_alg_per_step": head["bytes_alg_per_step"],
        "stage_ms": head["stage_ms"],
        "profiled_step_ms": head["profiled_step_ms"],
        "roofline": {"bound": "hbm", "kernel": sp["kernel"], "achieved": sp["achieved"], "peak": sp["peak"],
                     "unit": "GB/s", "frac": sp["frac"], "traffic": sp["traffic"],
                     "bytes_alg_per_step_pass": sp["bytes_alg_per_step_pass"],
                     "ms_per_step_pass": sp["ms_per_step_pass"],
                     "launches_per_step_pass": sp["launches_per_step_pass"],
                     # counter-measured bytes over the same launch time
                     "traffic_gbps": sp["traffic_gbps"]},
        "cpu_baseline": None,
    }
    for key in ("e_placement", "bootstrap_step", "dense_adams", "step_storing_v", "stream_reference",
                "stream_calibration", "mask_overlap", "graph"):
        if key in head:
            out[key] = head[key]
    if extras:
        out["configs"] = extras
    if cpu is not None:
        cpu["gpu_over_cpu"] = out["value"] / cpu["value"]
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
