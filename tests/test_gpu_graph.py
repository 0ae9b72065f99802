"""The graph-capturable step (scape_step_graph) recorded once into a HIP
graph and replayed: every replay must give what eager scape_step calls give
on the same inputs, bit for bit, and what the oracle gives."""

import numpy as np
import pytest

from oracle import scape_oracle as O
from sparse_communication_distributed_amd import workload as W
from tests.gpu_util import check_mask

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def S():
    from sparse_communication_distributed_amd import scape
    scape.lib()
    return scape


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits_of(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,n_p,P,K,sp", [
    ("tiny", None, None, None, None),
    ("ragged", 10_007, 3, 3, "0.99"),  # scalar path, odd K
    ("kpass", 4096 * 4, 32, 8, "0.99"),  # the step as K passes: 8 launches per step in the graph
])
def test_step_graph_replays_match_eager(S, name, n_p, P, K, sp):
    cfg = W.CONFIGS["tiny"] if name == "tiny" else W.flat_config(name, P * n_p, P, K, sp, steps=7,
                                                                  weight_decay=0.01)
    n, P, K, k = cfg.n, cfg.P, cfg.K, cfg.k
    print(f"[graph] {name} n={n} P={P} K={K} k={k}", flush=True)
    assert S.step_pass_count(S.dims(n, P, K), k) == (K if name == "kpass" else 1)
    w0 = W.init_params(cfg, 0)
    args = (P, K, k, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.lr)
    eager = S.ScapeOptimizer(dev(w0), *args)
    graphed = S.ScapeOptimizer(dev(w0), *args)
    hp = O.Hyper.make(cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.lr)
    ora = O.OracleOptimizer(w0, P, K, k, hp)

    g1 = W.grads(cfg, 1, 0)
    eager.step(dev(g1))
    graphed.step(dev(g1))  # step 1 (the bootstrap) runs eagerly
    ora.step(g1)
    bias = S.bias_state_tensor(graphed.bt, 1, DEV)
    gin = [torch.zeros((K, n), dtype=torch.float32, device=DEV) for _ in range(2)]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        # steps t (even; M_t in slot 1) and t + 1 (M_{t+1} in slot 0)
        for j, slot in enumerate((1, 0)):
            S.step_graph(graphed.d, graphed.params, gin[j], graphed.m, graphed.v, graphed.e, graphed.mask, k,
                         graphed.bt, graphed.lr, slot, bias, graphed.ws)

    for r in range(3):
        t0 = 2 + 2 * r
        ga, gb = W.grads(cfg, t0, 0), W.grads(cfg, t0 + 1, 0)
        gin[0].copy_(dev(ga))
        gin[1].copy_(dev(gb))
        graph.replay()
        eager.step(dev(ga))
        eager.step(dev(gb))
        torch.cuda.synchronize()
        ora.step(ga)
        ora.step(gb)
        print(f"[graph] {name} replay {r}: steps {t0}, {t0 + 1}", flush=True)
        for nm in ("params", "m", "v", "e"):
            got, want = bits_of(getattr(graphed, nm)), bits_of(getattr(eager, nm))
            assert np.array_equal(got, want), f"replay {r}: {nm} differs from the eager step"
        assert torch.equal(graphed.mask, eager.mask), f"replay {r}: mask blob differs from the eager step"
        for nm, o in (("params", "w"), ("m", "m"), ("v", "v"), ("e", "e")):
            assert np.array_equal(bits_of(getattr(graphed, nm)).reshape(-1),
                                  ora.gather(o).view(np.uint32).reshape(-1)), f"replay {r}: {nm} differs from the oracle"
        outs_next = [st.idx for st in ora.parts]
        # after an even number of graph steps, M_{t+2} sits in slot 1 again
        check_mask(*S.mask_slot_tensors(graphed.d, k, graphed.mask, 1), outs_next, cfg.n_p)
        want_bias = bytes(S.bias_state_at(graphed.bt, t0 + 1))
        assert bytes(bias.cpu().numpy().tobytes()) == want_bias, f"replay {r}: bias state differs from the host's"
