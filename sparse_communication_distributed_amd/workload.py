"""Workload definitions and seeded synthetic inputs.

This module is shared by the tests, the benchmark and the smoke check: it
builds the parameter layouts and draws the inputs (initial parameters and the
per-worker gradients) that both the CPU oracle and the HIP library consume.
It holds none of the optimizer's arithmetic: no statistic, no selection, no
error feedback and no update rule live here.

Layouts follow the models the SCAPE paper trains (GPT-345M, Llama-500M,
Llama-1.8B; SCAPE paper, abstract and §I).  The optimizer sees one flat fp32
buffer that the distributed optimizer splits into equal contiguous shards
(SCAPE paper §II-A, sharded data parallelism), so a layout is a list of tensor
sizes in forward order concatenated into that buffer.

Randomness:
  * host generator: numpy ``Philox`` seeded by ``SeedSequence(seed,
    spawn_key=(config_id, stream, step, worker, partition))``; one stream per
    (step, worker, partition) so that any partition can be regenerated alone.
    Streams: 0 = initial parameters, 1 = per-tensor / per-partition scales,
    2 = gradients, 3 = duplicate-magnitude positions (stress law).
  * device generator (large layouts only): torch's CUDA Philox seeded from the
    same tuple.  It produces different numbers than the host generator; a test
    that needs oracle inputs for a device-generated workload copies the slices
    it checks back to the host.  The stress law's duplicate positions and
    donor picks come from the host stream 3 in both generators.
"""

from __future__ import annotations

import dataclasses
import math
from fractions import Fraction
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# layouts
# --------------------------------------------------------------------------


def llama_tensors(layers: int, hidden: int, ffn: int, vocab: int) -> List[Tuple[str, int]]:
    """Llama-style tensor list in forward order: embedding, per layer
    (attention norm, q/k/v/o, FFN norm, SwiGLU gate/up/down), final norm and an
    untied output head.  Multi-head attention, no biases."""
    t = [("tok_embeddings", vocab * hidden)]
    for i in range(layers):
        t += [
            (f"layers.{i}.attention_norm", hidden),
            (f"layers.{i}.wq", hidden * hidden),
            (f"layers.{i}.wk", hidden * hidden),
            (f"layers.{i}.wv", hidden * hidden),
            (f"layers.{i}.wo", hidden * hidden),
            (f"layers.{i}.ffn_norm", hidden),
            (f"layers.{i}.w_gate", ffn * hidden),
            (f"layers.{i}.w_up", ffn * hidden),
            (f"layers.{i}.w_down", hidden * ffn),
        ]
    t += [("norm", hidden), ("output", vocab * hidden)]
    return t


def gpt_tensors(layers: int, hidden: int, ffn: int, vocab: int, seq: int) -> List[Tuple[str, int]]:
    """GPT-2-style tensor list in forward order with a tied output head."""
    t = [("wte", vocab * hidden), ("wpe", seq * hidden)]
    for i in range(layers):
        t += [
            (f"h.{i}.ln_1.weight", hidden), (f"h.{i}.ln_1.bias", hidden),
            (f"h.{i}.attn.c_attn.weight", 3 * hidden * hidden), (f"h.{i}.attn.c_attn.bias", 3 * hidden),
            (f"h.{i}.attn.c_proj.weight", hidden * hidden), (f"h.{i}.attn.c_proj.bias", hidden),
            (f"h.{i}.ln_2.weight", hidden), (f"h.{i}.ln_2.bias", hidden),
            (f"h.{i}.mlp.c_fc.weight", ffn * hidden), (f"h.{i}.mlp.c_fc.bias", ffn),
            (f"h.{i}.mlp.c_proj.weight", hidden * ffn), (f"h.{i}.mlp.c_proj.bias", hidden),
        ]
    t += [("ln_f.weight", hidden), ("ln_f.bias", hidden)]
    return t


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

GRAD_LAWS = ("partition_scale", "tensor_sigma", "stress_t3")


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload.

    ``sparsity`` is a decimal string ("0.99") so that the per-partition count
    ``k = max(1, floor(n_p * (1 - sparsity)))`` is computed exactly.
    """

    name: str
    config_id: int
    tensors: Tuple[Tuple[str, int], ...]
    num_partitions: int
    num_workers: int
    sparsity: str
    steps: int
    grad_law: str = "tensor_sigma"
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.0
    lr: float = 1e-3

    def __post_init__(self):
        if self.grad_law not in GRAD_LAWS:
            raise ValueError(f"unknown gradient law {self.grad_law!r}")
        if self.n % self.num_partitions:
            raise ValueError("n must be a multiple of the number of partitions")

    @property
    def n(self) -> int:
        return sum(s for _, s in self.tensors)

    @property
    def n_p(self) -> int:
        return self.n // self.num_partitions

    @property
    def k(self) -> int:
        dens = 1 - Fraction(self.sparsity)
        return max(1, math.floor(self.n_p * dens))

    @property
    def P(self) -> int:
        return self.num_partitions

    @property
    def K(self) -> int:
        return self.num_workers

    def tensor_offsets(self) -> np.ndarray:
        sizes = np.array([s for _, s in self.tensors], dtype=np.int64)
        return np.concatenate([[0], np.cumsum(sizes)])

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def flat_config(name: str, n: int, P: int, K: int, sparsity: str, steps: int = 3,
                grad_law: str = "tensor_sigma", config_id: int = 100, **kw) -> Config:
    """A single flat tensor of n parameters (used for small parity cases)."""
    return Config(name=name, config_id=config_id, tensors=(("flat", n),),
                  num_partitions=P, num_workers=K, sparsity=sparsity, steps=steps,
                  grad_law=grad_law, **kw)


# Tensor sizes cycled by mixed_config: small and large, odd and even, so
# that every partition of a small layout spans several tensors (several
# gradient scales) and the tensor boundaries fall at every alignment.
_MIXED_SIZES = (1531, 64, 2903, 1, 777, 4099, 250, 17, 1024, 3)


def mixed_config(name: str, n: int, P: int, K: int, sparsity: str, steps: int = 3,
                 grad_law: str = "tensor_sigma", config_id: int = 101, **kw) -> Config:
    """n parameters as a list of many tensors of mixed sizes (each with its
    own gradient scale), for small parity cases in which one partition holds
    several scales, as the model layouts' partitions do."""
    tensors, left, i = [], n, 0
    while left > 0:
        sz = min(_MIXED_SIZES[i % len(_MIXED_SIZES)], left)
        tensors.append((f"t{i}", sz))
        left -= sz
        i += 1
    return Config(name=name, config_id=config_id, tensors=tuple(tensors), num_partitions=P,
                  num_workers=K, sparsity=sparsity, steps=steps, grad_law=grad_law, **kw)


def partition_tensor_count(cfg: Config, p: int) -> int:
    """How many tensors partition p spans."""
    off = cfg.tensor_offsets()
    first = int(np.searchsorted(off, p * cfg.n_p, side="right")) - 1
    last = int(np.searchsorted(off, (p + 1) * cfg.n_p - 1, side="right")) - 1
    return last - first + 1


def _cfgs():
    tiny = Config("tiny", 0, (("flat", 1 << 20),), 4, 2, "0.9", 20, grad_law="partition_scale")
    gpt = Config("gpt345m", 1, tuple(gpt_tensors(24, 1024, 4096, 50257, 1024)), 32, 8, "0.9", 10)
    l500 = Config("llama500m", 2, tuple(llama_tensors(24, 1280, 3456, 32000)), 32, 8, "0.99", 10)
    l18 = Config("llama1.8b", 3, tuple(llama_tensors(32, 2048, 5632, 32000)), 32, 4, "0.99", 5)
    stress = Config("stress", 4, tuple(llama_tensors(32, 2048, 5632, 32000)), 64, 4, "0.999", 5,
                    grad_law="stress_t3")
    return {c.name: c for c in (tiny, gpt, l500, l18, stress)}


CONFIGS = _cfgs()

# --------------------------------------------------------------------------
# host generator
# --------------------------------------------------------------------------

STREAM_PARAMS, STREAM_SCALES, STREAM_GRADS, STREAM_DUPS = 0, 1, 2, 3


def rng(seed: int, config_id: int, stream: int, step: int = 0, worker: int = 0,
        partition: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(config_id, stream, step, worker, partition))
    return np.random.Generator(np.random.Philox(ss))


def tensor_sigmas(cfg: Config, seed: int = 0) -> np.ndarray:
    """Per-tensor gradient std, 10**U(-5,-2) drawn in float64, cast to fp32."""
    u = rng(seed, cfg.config_id, STREAM_SCALES).uniform(-5.0, -2.0, size=len(cfg.tensors))
    return (10.0 ** u).astype(np.float32)


def partition_scales(cfg: Config, seed: int = 0) -> np.ndarray:
    """Per-partition scale s_p, log-uniform in [0.1, 10] (small flat workload)."""
    u = rng(seed, cfg.config_id, STREAM_SCALES).uniform(-1.0, 1.0, size=cfg.P)
    return 10.0 ** u


def sigma_per_element(cfg: Config, seed: int, lo: int, hi: int) -> np.ndarray:
    """fp32 gradient std for flat elements [lo, hi)."""
    if cfg.grad_law == "partition_scale":
        s = partition_scales(cfg, seed)
        part = np.arange(lo, hi, dtype=np.int64) // cfg.n_p
        return np.asarray([np.float32(x * 1e-3) for x in s], dtype=np.float32)[part]
    sig = tensor_sigmas(cfg, seed)
    off = cfg.tensor_offsets()
    tid = np.searchsorted(off, np.arange(lo, hi, dtype=np.int64), side="right") - 1
    return sig[tid]


def init_params_partition(cfg: Config, p: int, seed: int = 0) -> np.ndarray:
    """Initial fp32 master parameters of partition p, N(0, 0.02)."""
    g = rng(seed, cfg.config_id, STREAM_PARAMS, partition=p)
    return (g.standard_normal(cfg.n_p, dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def init_params(cfg: Config, seed: int = 0, partitions: Optional[Iterable[int]] = None) -> np.ndarray:
    parts = range(cfg.P) if partitions is None else partitions
    return np.concatenate([init_params_partition(cfg, p, seed) for p in parts])


def donor_count(cfg: Config) -> int:
    """Number of donor magnitudes of the stress law: the |g| values ranked
    k-8 .. k+7 of a partition (fewer where that range leaves the partition)."""
    return min(cfg.n_p, cfg.k + 8) - max(0, cfg.k - 8)


def duplicate_draws(cfg: Config, seed: int, step: int, worker: int, p: int):
    """Stress law's random choices for one (step, worker, partition), from
    the host stream STREAM_DUPS: floor(1% n_p) distinct positions (drawn
    without replacement) and, for each, which donor it copies.  Both the
    host and the device generator plant duplicates from these draws."""
    ndup = cfg.n_p // 100
    r = rng(seed, cfg.config_id, STREAM_DUPS, step, worker, p)
    pos = r.choice(cfg.n_p, size=ndup, replace=False)
    pick = r.integers(0, donor_count(cfg), size=ndup)
    return pos.astype(np.int64), pick.astype(np.int64)


def _duplicate_magnitudes(cfg: Config, g: np.ndarray, seed: int, step: int, worker: int, p: int) -> None:
    """Stress law: floor(1% n_p) positions, chosen without replacement, take
    sign-preserving copies of 16 donor magnitudes (the |g| values ranked
    k-8 .. k+7 in the partition) so that exact key ties straddle the
    selection boundary."""
    n_p, k = g.shape[0], cfg.k
    if n_p // 100 == 0:
        return
    mag = np.abs(g)
    order = np.argsort(-mag.astype(np.float64), kind="stable")
    donors = mag[order[max(0, k - 8):min(n_p, k + 8)]]
    pos, pick = duplicate_draws(cfg, seed, step, worker, p)
    g[pos] = np.where(g[pos] < 0, -donors[pick], donors[pick]).astype(np.float32)


def grads_partition(cfg: Config, step: int, worker: int, p: int, seed: int = 0) -> np.ndarray:
    """fp32 gradient of worker `worker` at step `step` for partition p."""
    r = rng(seed, cfg.config_id, STREAM_GRADS, step, worker, p)
    lo = p * cfg.n_p
    sig = sigma_per_element(cfg, seed, lo, lo + cfg.n_p)
    if cfg.grad_law == "stress_t3":
        z = r.standard_t(3, size=cfg.n_p).astype(np.float32)
    else:
        z = r.standard_normal(cfg.n_p, dtype=np.float32)
    g = (sig * z).astype(np.float32)
    if cfg.grad_law == "stress_t3":
        _duplicate_magnitudes(cfg, g, seed, step, worker, p)
    return g


def grads(cfg: Config, step: int, seed: int = 0, partitions: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp32 [K][n] gradients (or [K][len(partitions)*n_p] for a subset)."""
    parts = list(range(cfg.P)) if partitions is None else list(partitions)
    out = np.empty((cfg.K, len(parts) * cfg.n_p), dtype=np.float32)
    for i in range(cfg.K):
        for q, p in enumerate(parts):
            out[i, q * cfg.n_p:(q + 1) * cfg.n_p] = grads_partition(cfg, step, i, p, seed)
    return out


# --------------------------------------------------------------------------
# device generator (large layouts)
# --------------------------------------------------------------------------


def _torch_seed(seed: int, config_id: int, stream: int, step: int, worker: int) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(config_id, stream, step, worker, 1 << 20))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def device_sigma(cfg: Config, seed: int, device) -> "torch.Tensor":
    """fp32 per-element gradient std as a device tensor (built once per layout)."""
    import torch
    out = torch.empty(cfg.n, dtype=torch.float32, device=device)
    if cfg.grad_law == "partition_scale":
        s = partition_scales(cfg, seed)
        for p in range(cfg.P):
            out[p * cfg.n_p:(p + 1) * cfg.n_p].fill_(float(np.float32(s[p] * 1e-3)))
        return out
    sig = tensor_sigmas(cfg, seed)
    off = cfg.tensor_offsets()
    for t in range(len(cfg.tensors)):
        out[int(off[t]):int(off[t + 1])].fill_(float(sig[t]))
    return out


def device_init_params(cfg: Config, seed: int, out) -> None:
    import torch
    gen = torch.Generator(device=out.device)
    gen.manual_seed(_torch_seed(seed, cfg.config_id, STREAM_PARAMS, 0, 0))
    out.normal_(0.0, 1.0, generator=gen).mul_(0.02)


def device_base_grads(cfg: Config, step: int, seed: int, sigma, out) -> None:
    """Fill out[K][n] (fp32, on out's device) with the step's gradients
    before any duplicate planting: sigma * z for the normal laws, sigma * t_3
    with t_3 = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) for the stress law."""
    import torch
    for i in range(cfg.K):
        gen = torch.Generator(device=out.device)
        gen.manual_seed(_torch_seed(seed, cfg.config_id, STREAM_GRADS, step, i))
        row = out[i]
        row.normal_(0.0, 1.0, generator=gen)
        if cfg.grad_law == "stress_t3":
            chi = torch.zeros_like(row)
            tmp = torch.empty_like(row)
            for _ in range(3):
                tmp.normal_(0.0, 1.0, generator=gen)
                chi.addcmul_(tmp, tmp)
            row.div_(chi.div_(3.0).sqrt_())
            del chi, tmp
        row.mul_(sigma)


def device_grads(cfg: Config, step: int, seed: int, sigma, out) -> None:
    """Fill out[K][n] (fp32, on out's device) with the step's gradients:
    device_base_grads, then for the stress law the duplicate-magnitude
    planting of the host law, per (worker, partition), at the positions and
    donor picks of duplicate_draws (drawn on the host)."""
    device_base_grads(cfg, step, seed, sigma, out)
    if cfg.grad_law == "stress_t3":
        for i in range(cfg.K):
            _device_duplicates(cfg, out[i], seed, step, i)


def _device_duplicates(cfg: Config, row, seed: int, step: int, worker: int) -> None:
    import torch
    n_p, k = cfg.n_p, cfg.k
    if n_p // 100 == 0:
        return
    for p in range(cfg.P):
        seg = row[p * n_p:(p + 1) * n_p]
        top = torch.topk(seg.abs(), min(n_p, k + 8), largest=True, sorted=True).values
        donors = top[max(0, k - 8):]
        pos_h, pick_h = duplicate_draws(cfg, seed, step, worker, p)
        pos = torch.from_numpy(pos_h).to(row.device)
        pick = donors[torch.from_numpy(pick_h).to(row.device)]
        seg[pos] = torch.where(seg[pos] < 0, -pick, pick)
        del top, donors, pos, pick
