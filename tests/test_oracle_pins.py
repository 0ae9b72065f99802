"""Pins of the CPU oracle against brute force, closed forms and invariants.

The pages print no worked example with numbers, so each pin below is a
property that the pages' definitions fix (SCAPE paper §II-B and §II-C eq. (2),
technical summary §2), written so that a plausible slip in the oracle (a tie
broken the wrong way, the wrong worker's gradient in the statistic, m_t in
place of m_{t-1} in the second moment, swapped or missing bias corrections, eps
inside the square root, a different summation order, a missing one-step lag,
a statistic keyed on the gradient without its error-feedback residual) fails
at least one of them.

The statistic that keys the mask is pinned twice: at one worker and sparsity
0 it must be the dense first moment of AdamS (§II-C eq. (2)) bit for bit,
also when a residual is carried into that regime; and a worked example shows
error feedback (§II-B) raising an element whose own gradient never ranks
into the mask, which then sends its whole accumulated residual.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import scape_oracle as O

F32 = np.float32


def brute_topk(keys, k):
    order = sorted(range(len(keys)), key=lambda j: (-int(keys[j]), j))
    return sorted(order[:k])


# ---------------------------------------------------------------- top-k (O3)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 31, 64])
@pytest.mark.parametrize("span", [3, 1 << 31])
def test_topk_matches_brute_force_for_every_k(n, span):
    rng = np.random.default_rng(n * 7 + span % 11)
    keys = rng.integers(0, span, size=n, dtype=np.int64).astype(np.uint32)
    for k in range(1, n + 1):
        assert O.topk_indices(keys, k).tolist() == brute_topk(keys, k)


@pytest.mark.parametrize("k", [1, 17, 1000, 99_999, 200_003])
def test_topk_characterisation_large(k):
    """The selected set is the unique set of size k whose smallest key is at
    least the largest unselected key, and whose members with the threshold key
    all precede (by index) the unselected members with that key."""
    rng = np.random.default_rng(k)
    n = 200_003
    keys = rng.integers(0, 500, size=n).astype(np.uint32)
    sel = O.topk_indices(keys, k)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    chosen = np.zeros(n, bool)
    chosen[sel] = True
    T = keys[chosen].min()
    if k < n:
        assert T >= keys[~chosen].max()
        tie_sel = np.flatnonzero(chosen & (keys == T))
        tie_un = np.flatnonzero(~chosen & (keys == T))
        if tie_un.size:
            assert tie_sel.max() < tie_un.min()


def test_topk_special_cases():
    keys = np.full(100, 7, np.uint32)
    assert O.topk_indices(keys, 13).tolist() == list(range(13))
    r = np.random.default_rng(0).integers(0, 9, 50).astype(np.uint32)
    assert O.topk_indices(r, 50).tolist() == list(range(50))
    assert O.topk_indices(r, 1).tolist() == [int(np.argmax(r))]
    with pytest.raises(ValueError):
        O.topk_indices(r, 0)
    with pytest.raises(ValueError):
        O.topk_indices(r, 51)


# ------------------------------------------------------------- keys (O2, R5)


def test_magnitude_keys_order_sign_zero_nan():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(5000).astype(F32) * F32(10.0) ** rng.integers(-40, 38, 5000).astype(F32),
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38], F32),
    ]).astype(F32)
    x = x[np.isfinite(x)]
    k = O.magnitude_keys(x)
    assert np.array_equal(k, O.magnitude_keys(-x))
    assert O.magnitude_keys(np.array([0.0, -0.0], F32)).tolist() == [0, 0]
    mag = np.abs(x.astype(np.float64))
    i, j = rng.integers(0, x.size, (2, 20000))
    assert np.array_equal(k[i] < k[j], mag[i] < mag[j])
    assert np.array_equal(k[i] == k[j], mag[i] == mag[j])
    special = O.magnitude_keys(np.array([np.inf, -np.nan, np.nan, 3.0e38], F32))
    assert special[1] > special[0] and special[2] > special[0] and special[0] > special[3]


def test_statistic_formula_worked_example():
    """Hand-worked ranking: the key is |b1*m + c1*a|, not |a| or |m|.
    element 0: m=1, a=-9 -> 0.9 - 0.9 ~ 0;  element 1: m=0, a=2 -> 0.2;
    element 2: m=0.1, a=0.1 -> 0.1;        element 3: m=-2, a=0 -> 1.8."""
    hp = O.Hyper.make()
    m = np.array([1.0, 0.0, 0.1, -2.0], F32)
    a = np.array([-9.0, 2.0, 0.1, 0.0], F32)
    keys = O.statistic_keys(m, a, hp)
    assert O.topk_indices(keys[:3], 1).tolist() == [1]
    assert O.topk_indices(keys, 1).tolist() == [3]
    assert O.topk_indices(keys, 3).tolist() == [1, 2, 3]
    s = keys.view(F32)
    assert abs(float(s[0])) < 1e-6 and abs(float(s[3]) - 1.8) < 1e-6


@pytest.mark.parametrize("P,n_p,T,residual", [(1, 700, 12, False), (3, 257, 8, False), (2, 300, 6, True)])
def test_statistic_is_dense_first_moment_at_one_worker_sparsity_zero(P, n_p, T, residual):
    """K = 1 and k = n_p: every element is sent every step and the
    synchronised buffer is the worker's own error-compensated gradient, so
    the statistic that keys M_{t+1} is the dense first moment m_t of AdamS
    (SCAPE paper §II-C eq. (2)).  Its keys must equal bits(|m_t|) bit for bit
    at every step, with m_t taken from the state after the step's update
    (two different code paths of the oracle: O2 and O6).  With `residual`
    the state enters the dense regime carrying a nonzero error-feedback
    residual (as after a change of density): the first dense step sends it,
    so the first moment, and with it the key, includes it."""
    rng = np.random.default_rng(P * 100 + n_p)
    hp = O.Hyper.make(weight_decay=0.01)
    w0 = (rng.standard_normal(P * n_p) * 0.02).astype(F32)
    opt = O.OracleOptimizer(w0, P, 1, n_p, hp)
    if residual:  # enter at step 2 with M_2 = everything and e != 0
        for st in opt.parts:
            st.e[:] = (rng.standard_normal((1, n_p)) * 1e-2).astype(F32)
            st.idx = np.arange(n_p)
        opt.t = 1
    for t in range(opt.t + 1, opt.t + T + 1):
        e_in = opt.gather("e").copy()
        g = (rng.standard_normal((1, P * n_p)) * 10.0 ** rng.integers(-6, -1, (1, P * n_p))).astype(F32)
        outs = opt.step(g)
        for p in range(P):
            st = opt.parts[p]
            assert np.all(st.e == 0)
            assert outs[p]["cur"].size == n_p
            assert np.array_equal(outs[p]["keys"], O.magnitude_keys(st.m)), f"step {t} partition {p}"
        if residual and t == 2:  # m_1 = 0 here: a key of the gradient alone would be |c1*g|
            assert np.any(e_in != 0)
            assert not np.array_equal(outs[0]["keys"], O.magnitude_keys(hp.c1 * g[0, :n_p]))


def test_residual_reinjection_worked_example():
    """Error feedback re-injects what was not sent (SCAPE paper §II-B: the
    dropped part is added back into later communication), and the mask is
    keyed on the owner's error-compensated gradient.  One partition, one
    worker, k = 1.  Element 0 receives a constant gradient c = 0.25 every
    step and element 3 a constant h = 0.5 > c; the rest receive 0.  Element
    3 takes the mask at step 1 and keeps it while element 0's residual
    grows by c per step.  With m_0 = 0 off the mask, element 0's statistic
    at step t is c1 * (t*c); element 3's is its dense first moment
    h * (1 - b1^t).  Element 0 enters M_{T+1} at the first step T at which
    the former exceeds the latter (found here from the float64 closed forms:
    the margins are ~1e-2, far above fp32 rounding), although its own
    gradient never would.  At step T + 1 it sends its whole accumulated
    residual plus the step's gradient, (T + 1) * c exactly (multiples of
    1/4 are exact in fp32), and its residual returns to 0."""
    n = 8
    hp = O.Hyper.make()
    c, h = F32(0.25), F32(0.5)
    b1, c1 = float(hp.b1), float(hp.c1)
    T = next(t for t in range(1, 100) if c1 * t * float(c) > float(h) * (1 - b1 ** t))
    assert T == 17
    assert all(c1 * float(c) < float(h) * (1 - b1 ** t) for t in range(1, 100))  # never on its own
    w0 = np.linspace(0.1, 0.8, n).astype(F32)
    opt = O.OracleOptimizer(w0, 1, 1, 1, hp)
    st = opt.parts[0]
    for t in range(1, T + 3):
        g = np.zeros(n, F32)
        g[0], g[3] = c, h
        out = opt.step(g[None])[0]
        s = out["keys"].view(F32).astype(np.float64)
        if t <= T:
            assert out["cur"].tolist() == [3], f"step {t}"
            assert st.e[0, 0] == F32(t * 0.25) and st.w[0] == w0[0], f"step {t}"
            assert abs(s[0] - c1 * t * 0.25) < 1e-6 and abs(s[3] - 0.5 * (1 - b1 ** t)) < 1e-6, f"step {t}"
            assert out["nxt"].tolist() == ([0] if t == T else [3]), f"step {t}"
        if t == T + 1:
            assert out["cur"].tolist() == [0]
            assert out["bbar"][0] == F32((T + 1) * 0.25)  # the whole accumulated residual
            assert st.e[0, 0] == 0 and st.w[0] != w0[0]
            assert st.e[0, 3] == h                        # element 3 now accumulates


@pytest.mark.parametrize("P,K", [(8, 4), (4, 4), (6, 4), (2, 4), (4, 2), (5, 3)])
def test_step1_mask_is_owner_gradient_topk(P, K):
    """At t = 1 (m = 0, e = 0) the key is fl(c1*|g^o|): the mask of partition p
    is the top-k of the owner's gradient magnitudes, owner = floor(p*K/P)."""
    n_p, k = 257, 19
    rng = np.random.default_rng(P * 10 + K)
    g = rng.standard_normal((K, P * n_p)).astype(F32)
    hp = O.Hyper.make()
    opt = O.OracleOptimizer(np.zeros(P * n_p, F32), P, K, k, hp)
    outs = opt.step(g)
    for p in range(P):
        o = (p * K) // P
        gp = g[o, p * n_p:(p + 1) * n_p]
        mag = np.abs(gp.astype(np.float64))
        assert np.unique(mag).size == n_p
        scaled = np.abs((hp.c1 * gp).astype(np.float64))
        assert np.unique(scaled).size == n_p
        want = sorted(np.argsort(-mag, kind="stable")[:k].tolist())
        assert outs[p]["nxt"].tolist() == want
        assert outs[p]["cur"].tolist() == want  # bootstrap: M_1 = M_2
        for i in range(K):
            if i != o:
                other = sorted(np.argsort(-np.abs(g[i, p * n_p:(p + 1) * n_p].astype(np.float64)),
                                          kind="stable")[:k].tolist())
                assert other != want


# ------------------------------------------------------------ error feedback


def test_error_feedback_identity_exact():
    """g~ + e' = fl(g + e) bitwise; e' = 0 on the mask; b = a at the mask."""
    rng = np.random.default_rng(2)
    n = 10_000
    g = (rng.standard_normal(n) * 10.0 ** rng.integers(-8, 3, n)).astype(F32)
    e = (rng.standard_normal(n) * 10.0 ** rng.integers(-8, 3, n)).astype(F32)
    idx = np.sort(rng.choice(n, 777, replace=False))
    a = O.accumulate(g, e)
    assert np.array_equal(a.view(np.uint32), (g + e).view(np.uint32))
    b, e2 = O.compress(a, idx)
    gt = np.zeros(n, F32)
    gt[idx] = b
    assert np.array_equal((gt + e2).view(np.uint32), a.view(np.uint32))
    assert np.all(e2[idx].view(np.uint32) == 0)
    off = np.ones(n, bool)
    off[idx] = False
    assert np.array_equal(e2[off].view(np.uint32), a[off].view(np.uint32))
    assert math.isclose(float(np.sum(gt, dtype=np.float64) + np.sum(e2, dtype=np.float64)),
                        float(np.sum(a, dtype=np.float64)), rel_tol=0, abs_tol=1e-9)


# ------------------------------------------------------------------- reduce


def test_reduce_special_cases_and_order():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000).astype(F32)
    assert np.array_equal(O.reduce_mean([x]), x)
    assert np.array_equal(O.reduce_mean([x, x]), x)
    ints = [rng.integers(-1000, 1000, 500).astype(F32) for _ in range(4)]
    exact = [Fraction(int(sum(int(b[j]) for b in ints)), 4) for j in range(500)]
    got = O.reduce_mean(ints)
    assert all(Fraction(float(got[j])) == exact[j] for j in range(500))
    # left-to-right: ((1e8 + -1e8) + 1) = 1, whereas 1e8 + (-1e8 + 1) = 0 in fp32
    b = [np.array([1e8], F32), np.array([-1e8], F32), np.array([1.0], F32)]
    assert float(O.reduce_mean(b)[0]) == float(F32(1.0) * F32(1.0 / 3.0))
    three = [rng.standard_normal(200).astype(F32) for _ in range(3)]
    got3 = O.reduce_mean(three).astype(np.float64)
    ref = (three[0].astype(np.float64) + three[1] + three[2]) / 3.0
    assert np.allclose(got3, ref, rtol=1e-6, atol=1e-7)


# -------------------------------------------------------------------- AdamS


@pytest.mark.parametrize("beta", [0.9, 0.95, 0.999])
def test_bias_reciprocal_closed_form(beta):
    b = F32(beta)
    for t in range(1, 60):
        exact = 1 / (1 - Fraction(float(b)) ** t)
        got = Fraction(float(O.bias_reciprocal(b, t)))
        ulp = Fraction(float(np.spacing(F32(float(exact)))))
        assert abs(got - exact) <= ulp


def test_first_step_is_sign_like():
    """m_0 = v_0 = 0: after bias correction mh = x and vh = x^2, so
    w_1 = w_0 - lr * x / (|x| + eps) (Adam's first step)."""
    rng = np.random.default_rng(4)
    n = 4096
    hp = O.Hyper.make(lr=1e-3)
    w0 = (rng.standard_normal(n) * 0.02).astype(F32)
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-5, -1, n)).astype(F32)
    w, m, v = w0.copy(), np.zeros(n, F32), np.zeros(n, F32)
    O.adams_update(w, m, v, np.arange(n), x, hp, 1)
    xd = x.astype(np.float64)
    want = w0.astype(np.float64) - 1e-3 * xd / (np.abs(xd) + 1e-8)
    tol = 1e-3 * 2e-6 + 2 * np.spacing(np.abs(w0)).astype(np.float64)
    assert np.all(np.abs(w.astype(np.float64) - want) <= tol)
    assert np.allclose(m, float(hp.c1) * xd, rtol=1e-6)
    assert np.allclose(v, float(hp.c2) * xd * xd, rtol=1e-6)


def test_constant_gradient_closed_form_dense():
    """Sparsity 0, one worker, constant gradient g:
    m_t = (1 - b1^t) g;  v_t = g^2 (b2 (1 - b1^(t-1))^2 + (1 - b2));
    w_t = w_{t-1} - lr * g / (|g| sqrt(v_t / (g^2 (1 - b2^t))) + eps)."""
    n, T = 64, 30
    rng = np.random.default_rng(5)
    g = (rng.standard_normal(n) * 1e-2).astype(F32)
    w0 = (rng.standard_normal(n) * 0.02).astype(F32)
    hp = O.Hyper.make()
    opt = O.OracleOptimizer(w0, 1, 1, n, hp)
    b1, b2 = float(hp.b1), float(hp.b2)
    gd = g.astype(np.float64)
    w_ref = w0.astype(np.float64)
    for t in range(1, T + 1):
        opt.step(g[None, :])
        m_ref = (1 - b1 ** t) * gd
        v_ref = gd * gd * (b2 * (1 - b1 ** (t - 1)) ** 2 + (1 - b2))
        vh = v_ref / (1 - b2 ** t)
        w_ref = w_ref - 1e-3 * gd / (np.sqrt(vh) + 1e-8)
        st = opt.parts[0]
        assert np.allclose(st.m, m_ref, rtol=4e-6 * t, atol=0)
        assert np.allclose(st.v, v_ref, rtol=8e-6 * t, atol=0)
        assert np.allclose(st.w, w_ref, rtol=0, atol=1e-3 * 4e-6 * t + 4e-8)
        assert np.all(st.e == 0)


def test_weight_decay_closed_form():
    """g = 0: u = 0 / eps = 0 and w_t = w_0 (1 - lr*wd)^t."""
    n, T = 128, 12
    w0 = np.linspace(-1, 1, n).astype(F32)
    hp = O.Hyper.make(weight_decay=0.1, lr=1e-2)
    opt = O.OracleOptimizer(w0, 2, 2, n // 2, hp)
    for t in range(1, T + 1):
        opt.step(np.zeros((2, n), F32))
        ref = w0.astype(np.float64) * (1 - 1e-2 * 0.1) ** t
        assert np.allclose(opt.gather("w"), ref, rtol=3e-7 * t, atol=1e-12)
        assert np.all(opt.gather("m") == 0) and np.all(opt.gather("v") == 0)


def test_off_mask_state_untouched():
    P, K, n_p, k = 3, 2, 1000, 10
    rng = np.random.default_rng(6)
    w0 = rng.standard_normal(P * n_p).astype(F32)
    opt = O.OracleOptimizer(w0, P, K, k, O.Hyper.make())
    for t in range(1, 4):
        before = [s.copy() for s in opt.parts]
        outs = opt.step(rng.standard_normal((K, P * n_p)).astype(F32))
        for p in range(P):
            off = np.ones(n_p, bool)
            off[outs[p]["cur"]] = False
            for name in ("w", "m", "v"):
                a = getattr(before[p], name)[off].view(np.uint32)
                b = getattr(opt.parts[p], name)[off].view(np.uint32)
                assert np.array_equal(a, b)


# ----------------------------------------------------- whole step / the lag


def test_one_step_lag_worked_example():
    """Hand-built: the mask built at step t is applied at step t+1, and the
    residual carries an unsent gradient into the next statistic."""
    n = 8
    hp = O.Hyper.make()
    small = (np.arange(n, dtype=F32) + F32(1)) * F32(1e-3)
    w0 = np.linspace(0.1, 0.8, n).astype(F32)
    opt = O.OracleOptimizer(w0, 1, 1, 1, hp)
    g1 = small.copy(); g1[2] = 1.0
    g2 = small.copy(); g2[5] = 1.0
    g3 = small.copy()
    o1 = opt.step(g1[None])[0]
    assert o1["cur"].tolist() == [2] and o1["nxt"].tolist() == [2]
    o2 = opt.step(g2[None])[0]
    st = opt.parts[0]
    assert o2["cur"].tolist() == [2]               # M_2 = M_1: the spike at 5 waits
    assert st.w[5] == w0[5]                         # not updated at step 2
    assert st.e[0, 5] == F32(g2[5] + F32(g1[5]))    # residual holds g1 + g2
    assert o2["nxt"].tolist() == [5]               # ... and enters M_3
    o3 = opt.step(g3[None])[0]
    assert o3["cur"].tolist() == [5]
    assert st.e[0, 5] == 0
    assert o3["bbar"][0] == F32(g3[5] + F32(g2[5] + F32(g1[5])))
    assert st.w[5] != w0[5]


def test_sparsity_zero_is_dense_adams_on_worker_mean():
    """k = n_p and e = 0: every index is sent every step, e stays 0 and the
    update is dense AdamS ([P] §II-C eq. (2)) on the worker-mean gradient."""
    P, K, n_p, T = 2, 3, 300, 4
    rng = np.random.default_rng(7)
    w0 = rng.standard_normal(P * n_p).astype(F32)
    hp = O.Hyper.make(weight_decay=0.01)
    opt = O.OracleOptimizer(w0, P, K, n_p, hp)
    w, m = w0.copy(), np.zeros_like(w0)
    for t in range(1, T + 1):
        g = (rng.standard_normal((K, P * n_p)) * 1e-2).astype(F32)
        opt.step(g)
        x = g[0].copy()
        for i in range(1, K):
            x = x + g[i]
        x = x * F32(1.0 / K)
        mn = hp.b1 * m + hp.c1 * x
        vn = hp.b2 * (m * m) + hp.c2 * (x * x)
        u = (mn * O.bias_reciprocal(hp.b1, t)) / (np.sqrt(vn * O.bias_reciprocal(hp.b2, t)) + hp.eps)
        w = w - hp.lr * (u + hp.wd * w)
        m = mn
        assert np.array_equal(opt.gather("w").view(np.uint32), w.view(np.uint32))
        assert np.array_equal(opt.gather("m").view(np.uint32), m.view(np.uint32))
        assert np.all(opt.gather("e") == 0)


def test_mask_overlap_worked_example():
    prev = [np.array([0, 2, 4]), np.array([1, 3, 5])]
    nxt = [np.array([0, 2, 6]), np.array([7, 8, 9])]
    assert O.mask_overlap(prev, nxt, 3) == pytest.approx(2 / 6)


def test_dense_adams_equals_scape_at_sparsity_zero():
    """Dense AdamS on the worker mean equals the SCAPE step with every index
    selected (e stays 0, so a = g), bit for bit, over several steps."""
    P, K, n_p, T = 3, 4, 500, 5
    rng = np.random.default_rng(11)
    w0 = rng.standard_normal(P * n_p).astype(F32)
    hp = O.Hyper.make(weight_decay=0.02)
    opt = O.OracleOptimizer(w0, P, K, n_p, hp)
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t in range(1, T + 1):
        g = (rng.standard_normal((K, P * n_p)) * 1e-2).astype(F32)
        g[g == 0] = F32(1e-9)  # no signed zeros: g + (+0) is g bitwise
        opt.step(g)
        O.dense_adams_step(w, m, v, g, hp, t)
        for name, a in (("w", w), ("m", m), ("v", v)):
            assert np.array_equal(opt.gather(name).view(np.uint32), a.view(np.uint32)), name
