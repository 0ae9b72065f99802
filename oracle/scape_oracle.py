"""CPU oracle for SCAPE's per-step sparse optimizer path (numpy, fp32).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call this module.  The product
path (the HIP library under ``sparse_communication_distributed_amd/`` and its
binding) never imports, calls or links it, and this module imports nothing
from the product: inputs arrive as plain numpy arrays.

Sources (the pages, cited by title and section):
  [P]  SCAPE paper (Zheng, Chen, Xie, Zhang; arXiv 2607.01678, Chinese
       translation): abstract, §I, §II-A (sharded data parallelism, FP32
       optimizer state), §II-B (top-k sparsification with error feedback),
       §II-C eq. (2) (AdamS) and the bias-correction remark after it.
  [S]  "Sintesi Tecnica: SCAPE" (technical summary), §2 "Componenti del
       Design del Sistema": partitioned mask synchronisation, one-step mask
       lag, second-moment rebuild from a single synchronised buffer; and
       "Ottimizzazione della Memoria" (single-bit packed masks).

Arithmetic.  Every floating-point value is IEEE binary32 and every operation is
rounded on its own (round to nearest even; no fused multiply-add; correctly
rounded sqrt and division; subnormals kept).  [P] §II-A states that optimizer
state is kept in full precision FP32 and §II-B that the error-feedback buffer
is FP32, so the oracle computes in fp32 rather than fp64; numpy float32
ufuncs with float32 scalars do exactly this.

One step t >= 1 (state at entry: w, m = m_{t-1}, v, e^i and the mask M_t,
absent at t = 1; inputs: the K workers' gradients g^i):
  O1  a^i = g^i + e^i                                          [P] §II-B
  O2  per partition p with owner o(p) = floor(p*K/P):
      s = (b1*m) + (c1*a^o); key = bits(s) with the sign bit cleared
                                     [P] abstract, §I; [S] §2 (lagged mask)
  O3  M_{t+1} on p = the k indices first in (key descending, index
      ascending); at t = 1 also M_1 := M_{t+1}      [S] §2 (partitioned mask)
  O4  b^i = a^i restricted to M_t (ascending index order);
      e^i <- 0 on M_t, a^i elsewhere          [P] §II-B, fixed index set
  O5  S = ((b^0 + b^1) + ...) + b^{K-1};  bbar = S * fp32(1/K)   [S] §2
  O6  AdamS at the indices of M_t with x = bbar:       [P] §II-C eq. (2)
        mn = (b1*m) + (c1*x)
        vn = (b2*(m*m)) + (c2*(x*x))
        mh = mn*ibc1; vh = vn*ibc2        (bias correction after eq. (2))
        u  = mh / (sqrt(vh) + eps)
        wn = w - (lr*(u + (wd*w)))
  O7  off the mask, w, m and v are left unchanged.
  O8  overlap_t = |M_t ∩ M_{t+1}| / (P*k)   (a reported statistic, [P] §I)

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository): the statistic of O2 (owner's
error-compensated first-moment estimate), the step-1 bootstrap, raw gradient
values in the sparse buffer, the worker-mean order, global-step bias
correction with host-computed fp32 reciprocals, eps = 1e-8 and weight decay 0
by default, equal contiguous partitions, owner = floor(p*K/P), and v holding
the last uncorrected v_t at masked indices.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against brute force, closed forms and invariants.  The statistic of O2 is
pinned where the pages fix it: at one worker and sparsity 0 it is the dense
first moment m_t of §II-C eq. (2) bit for bit (also when a residual is
carried into that regime), its residual term is pinned by a worked example
of error-feedback re-injection (§II-B), and its owner mapping, sign
handling and ordering are pinned.  Its general form for several workers
(the owner's own error-compensated gradient) is a reading of the pages that
no page value can check: parity unpinned for that choice alone.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

F32 = np.float32
SIGN_CLEAR = np.uint32(0x7FFFFFFF)


@dataclasses.dataclass(frozen=True)
class Hyper:
    """fp32 hyper-parameters; c1 = 1 - b1 and c2 = 1 - b2 are fp32 differences."""

    b1: np.float32
    b2: np.float32
    c1: np.float32
    c2: np.float32
    eps: np.float32
    wd: np.float32
    lr: np.float32

    @classmethod
    def make(cls, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, lr=1e-3) -> "Hyper":
        b1, b2 = F32(beta1), F32(beta2)
        return cls(b1=b1, b2=b2, c1=F32(1) - b1, c2=F32(1) - b2, eps=F32(eps),
                   wd=F32(weight_decay), lr=F32(lr))


def bias_reciprocal(beta: np.float32, t: int) -> np.float32:
    """fp32(1 / (1 - beta**t)), with beta**t formed by t multiplications in
    float64 starting from 1.0 ([P] §II-C, remark after eq. (2))."""
    p = 1.0
    for _ in range(t):
        p = p * float(beta)
    return F32(1.0 / (1.0 - p))


def owner(p: int, P: int, K: int) -> int:
    """Worker that owns partition p: contiguous blocks of partitions per
    worker, as in sharded data parallelism ([P] §II-A)."""
    return (p * K) // P


def magnitude_keys(x: np.ndarray) -> np.ndarray:
    """u32 ranking key of |x|: the binary32 bit pattern with the sign bit
    cleared (+0 and -0 map to 0; NaN ranks above +inf)."""
    x = np.ascontiguousarray(x, dtype=F32)
    return x.view(np.uint32) & SIGN_CLEAR


def accumulate(g: np.ndarray, e: np.ndarray) -> np.ndarray:
    """O1: error-compensated gradient a = g + e ([P] §II-B)."""
    return (g.astype(F32, copy=False) + e.astype(F32, copy=False)).astype(F32, copy=False)


def statistic_keys(m_prev: np.ndarray, a_owner: np.ndarray, hp: Hyper) -> np.ndarray:
    """O2: keys of the first-moment statistic b1*m_{t-1} + c1*a^o."""
    s = (hp.b1 * m_prev) + (hp.c1 * a_owner)
    return magnitude_keys(s)


def topk_indices(keys: np.ndarray, k: int) -> np.ndarray:
    """O3: the k indices that come first in the order (key descending, index
    ascending), returned in ascending index order ([S] §2, partitioned mask;
    ties go to the lower index)."""
    n = keys.shape[0]
    if not 1 <= k <= n:
        raise ValueError("k must lie in [1, n]")
    order = np.argsort(-(keys.astype(np.int64)), kind="stable")
    return np.sort(order[:k]).astype(np.int64)


def compress(a: np.ndarray, idx: np.ndarray):
    """O4: b = a at idx (ascending), e' = 0 at idx and a elsewhere.
    g~ = TopK(g+e) at the fixed index set, e' = g + e - g~ ([P] §II-B)."""
    b = a[idx].astype(F32, copy=True)
    e_new = a.astype(F32, copy=True)
    e_new[idx] = F32(0.0)
    return b, e_new


def reduce_mean(bs: Sequence[np.ndarray]) -> np.ndarray:
    """O5: left-to-right sum over workers, then times fp32(1/K)."""
    s = bs[0].astype(F32, copy=True)
    for b in bs[1:]:
        s = s + b
    return s * F32(1.0 / len(bs))


def adams_update(w: np.ndarray, m: np.ndarray, v: np.ndarray, idx: np.ndarray,
                 x: np.ndarray, hp: Hyper, t: int) -> None:
    """O6 in place at idx, with x the synchronised sparse buffer; v_t is
    rebuilt from m_{t-1} and x alone ([P] §II-C eq. (2); [S] §2,
    single-buffer second-moment rebuild).  O7: other entries untouched."""
    ibc1 = bias_reciprocal(hp.b1, t)
    ibc2 = bias_reciprocal(hp.b2, t)
    mo = m[idx]
    wo = w[idx]
    mn = (hp.b1 * mo) + (hp.c1 * x)
    vn = (hp.b2 * (mo * mo)) + (hp.c2 * (x * x))
    mh = mn * ibc1
    vh = vn * ibc2
    d = np.sqrt(vh) + hp.eps
    u = mh / d
    wn = wo - (hp.lr * (u + (hp.wd * wo)))
    m[idx] = mn
    v[idx] = vn
    w[idx] = wn


def dense_adams_step(w: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray, hp: Hyper, t: int) -> None:
    """Dense AdamS on the worker mean, in place: the baseline the pages
    measure SCAPE against ([P] abstract; [S] §4, per-step speedup over dense
    AdamS).  x = O5's mean of the K gradients, then O6 at every index."""
    x = reduce_mean([g[i] for i in range(g.shape[0])])
    adams_update(w, m, v, np.arange(w.shape[0]), x, hp, t)


def mask_overlap(prev: Sequence[np.ndarray], nxt: Sequence[np.ndarray], k: int) -> float:
    """O8: |M_t ∩ M_{t+1}| / (P*k) over per-partition index lists."""
    common = sum(np.intersect1d(a, b, assume_unique=True).size for a, b in zip(prev, nxt))
    return common / (len(prev) * k)


# --------------------------------------------------------------------------
# whole step
# --------------------------------------------------------------------------


@dataclasses.dataclass
class PartitionState:
    """Optimizer state of one partition: w, m, v [n_p]; e [K][n_p]; idx = M_t
    as ascending local indices (None before step 1)."""

    w: np.ndarray
    m: np.ndarray
    v: np.ndarray
    e: np.ndarray
    idx: Optional[np.ndarray] = None

    @classmethod
    def fresh(cls, w0: np.ndarray, K: int) -> "PartitionState":
        n = w0.shape[0]
        return cls(w=w0.astype(F32, copy=True), m=np.zeros(n, F32), v=np.zeros(n, F32),
                   e=np.zeros((K, n), F32))

    def copy(self) -> "PartitionState":
        return PartitionState(self.w.copy(), self.m.copy(), self.v.copy(), self.e.copy(),
                              None if self.idx is None else self.idx.copy())


def step_partition(st: PartitionState, g: np.ndarray, k: int, own: int, hp: Hyper, t: int) -> dict:
    """One SCAPE step on one partition, O1-O7 in order; updates st in place.

    g: [K][n_p] gradients of this partition; own: the owner worker.
    Returns the intermediates (keys, cur = M_t, nxt = M_{t+1}, b, bbar)."""
    if t < 1:
        raise ValueError("steps count from 1")
    K = g.shape[0]
    a = [accumulate(g[i], st.e[i]) for i in range(K)]            # O1
    keys = statistic_keys(st.m, a[own], hp)                       # O2 (m_{t-1})
    nxt = topk_indices(keys, k)                                   # O3
    if t == 1 or st.idx is None:
        cur = nxt                                                 # bootstrap M_1
    else:
        cur = st.idx
    bs = []
    for i in range(K):                                            # O4
        b, st.e[i] = compress(a[i], cur)
        bs.append(b)
    bbar = reduce_mean(bs)                                        # O5
    adams_update(st.w, st.m, st.v, cur, bbar, hp, t)              # O6, O7
    st.idx = nxt
    return {"keys": keys, "cur": cur, "nxt": nxt, "b": bs, "bbar": bbar}


class OracleOptimizer:
    """The whole flat buffer: P partitions stepped independently."""

    def __init__(self, w0: np.ndarray, P: int, K: int, k: int, hp: Hyper):
        n = w0.shape[0]
        if n % P:
            raise ValueError("n must be a multiple of P")
        self.P, self.K, self.k, self.hp, self.n_p = P, K, k, hp, n // P
        self.parts: List[PartitionState] = [
            PartitionState.fresh(w0[p * self.n_p:(p + 1) * self.n_p], K) for p in range(P)]
        self.t = 0

    def step(self, g: np.ndarray) -> List[dict]:
        """g: [K][n].  Returns the per-partition intermediates."""
        self.t += 1
        out = []
        for p, st in enumerate(self.parts):
            sl = slice(p * self.n_p, (p + 1) * self.n_p)
            out.append(step_partition(st, g[:, sl], self.k, owner(p, self.P, self.K), self.hp, self.t))
        return out

    def gather(self, name: str) -> np.ndarray:
        if name == "e":
            return np.concatenate([s.e for s in self.parts], axis=1)
        return np.concatenate([getattr(s, name) for s in self.parts])

    def mask_global_idx(self) -> np.ndarray:
        """M_{t+1} (the mask the next step applies) as ascending global indices."""
        return np.concatenate([s.idx + p * self.n_p for p, s in enumerate(self.parts)])
