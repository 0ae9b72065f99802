"""Seeded random sweep of shapes and value distributions against the oracle:
the partitioned top-k (mask_topk) on 48 random cases and the fused step in
lockstep on 12 random configurations."""

import numpy as np
import pytest

from oracle import scape_oracle as O
from sparse_communication_distributed_amd import workload as W
from tests.gpu_util import check_mask
from tests.test_gpu_parity import _stat_case, dev, oracle_topk_local, run_lockstep

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
KINDS = ("normal", "ties", "const", "wide", "special")


@pytest.fixture(scope="module")
def S():
    from sparse_communication_distributed_amd import scape
    scape.lib()
    return scape


def _mask_cases(count=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        P = int(rng.integers(1, 10))
        n_p = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 9000)),
                              int(rng.integers(9000, 40000))]))
        k = int(rng.integers(1, n_p + 1)) if rng.random() < 0.5 else max(1, int(n_p * rng.choice([0.01, 0.1, 0.5])))
        out.append((KINDS[int(rng.integers(0, len(KINDS)))], P, n_p, k, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("kind,P,n_p,k,seed", _mask_cases())
def test_random_mask_topk(S, kind, P, n_p, k, seed):
    stat = _stat_case(kind, P, n_p, seed)
    d = S.dims(P * n_p, P, 1)
    blob = torch.zeros(S.mask_bytes(d, k), dtype=torch.uint8, device=DEV)
    ws = torch.full((S.workspace_bytes(d, k),), 0x5A, dtype=torch.uint8, device=DEV)
    S.mask_topk(d, k, dev(stat), S.mask_slot(d, k, blob, 0), ws)
    torch.cuda.synchronize()
    check_mask(*S.mask_slot_tensors(d, k, blob, 0), oracle_topk_local(stat, P, n_p, k), n_p)


def _step_cases(count=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        P = int(rng.integers(1, 7))
        K = int(rng.integers(1, 7))
        n_p = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 20000))]))
        sp = str(rng.choice(["0", "0.5", "0.9", "0.99", "0.999"]))
        law = str(rng.choice(["tensor_sigma", "partition_scale", "stress_t3"]))
        wd = float(rng.choice([0.0, 0.01]))
        out.append((P, K, n_p, sp, law, wd, 200 + i))
    return out


@pytest.mark.parametrize("P,K,n_p,sp,law,wd,cid", _step_cases())
def test_random_step_lockstep(S, P, K, n_p, sp, law, wd, cid):
    cfg = W.flat_config("random", P * n_p, P, K, sp, steps=3, grad_law=law, config_id=cid, weight_decay=wd)
    run_lockstep(S, cfg, cfg.steps)


def _hyper_cases(count=8, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        b1 = float(rng.choice([0.0, 0.5, 0.9, 0.99]))
        b2 = float(rng.choice([0.0, 0.9, 0.95, 0.999, 0.9999]))
        eps = float(10.0 ** rng.uniform(-12, -4))
        lr = float(10.0 ** rng.uniform(-5, -1))
        wd = float(rng.choice([0.0, 1e-4, 0.1]))
        out.append((b1, b2, eps, lr, wd, 300 + i))
    return out


@pytest.mark.parametrize("b1,b2,eps,lr,wd,cid", _hyper_cases())
def test_random_hyper_parameters_lockstep(S, b1, b2, eps, lr, wd, cid):
    """The fused step under random AdamS hyper-parameters (beta1 = 0 makes
    the statistic the owner's residual-compensated gradient alone; beta2
    near 1 makes the bias correction large), bit for bit against the oracle."""
    cfg = W.flat_config("hyper", 3 * 9_000, 3, 2, "0.95", steps=4, config_id=cid,
                        beta1=b1, beta2=b2, eps=eps, lr=lr, weight_decay=wd)
    run_lockstep(S, cfg, cfg.steps)
