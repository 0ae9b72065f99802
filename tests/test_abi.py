"""C ABI checks that need no GPU: the library loads, exports every function
include/scape.h declares, sizes its layouts, and rejects invalid arguments
synchronously (validation happens before any HIP call)."""

import ctypes
import os
import re
import subprocess

import pytest

from sparse_communication_distributed_amd import scape as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scape.h")

pytestmark = pytest.mark.skipif(not os.path.exists(S.LIB_PATH), reason="libscape.so not built")

FAKE = 0x10000  # a non-null address that is never dereferenced by a rejected call


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(scape_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported_and_bound():
    L = S.lib()
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert sorted(S.exported_names()) == names
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_layout_sizes():
    d = S.dims(1 << 20, 4, 2)
    k = 26214
    T = S.tile_elems()
    assert T == 4096
    P, n_p = 4, (1 << 20) // 4
    slot_min = P * (n_p // 64) * 8 + P * k * 4 + P * (n_p // T) * 4
    mb = S.mask_bytes(d, k)
    assert mb >= 2 * slot_min and mb % 256 == 0
    ws = S.workspace_bytes(d, k)
    assert ws >= 4 * (1 << 20) + 2 * P * k * 4
    mv0 = S.MaskView()
    mv1 = S.MaskView()
    L = S.lib()
    assert L.scape_mask_slot(ctypes.byref(d), k, FAKE, 0, ctypes.byref(mv0)) == 0
    assert L.scape_mask_slot(ctypes.byref(d), k, FAKE, 1, ctypes.byref(mv1)) == 0
    assert mv0.bits == FAKE and mv1.bits == FAKE + mb // 2
    assert mv0.idx - mv0.bits >= P * (n_p // 64) * 8 and mv0.idx % 256 == 0
    assert mv0.tile_off - mv0.idx >= P * k * 4
    assert L.scape_mask_slot(ctypes.byref(d), k, FAKE, 2, ctypes.byref(mv0)) == 1


def test_step_pass_count():
    """K passes only where they measured faster: K >= 8 with the sparse
    buffers' round trip at most 2% of the streams (Llama-500M at 99%), one
    pass elsewhere (Llama-1.8B at K = 4, GPT-345M at 10% density)."""
    assert S.step_pass_count(S.dims(557_774_080, 32, 8), 174_304) == 8
    assert S.step_pass_count(S.dims(1_775_372_288, 32, 4), 554_803) == 1
    assert S.step_pass_count(S.dims(354_823_168, 32, 8), 1_108_822) == 1
    assert S.step_pass_count(S.dims(1 << 20, 4, 8), 2621) == 8   # 1% density, K = 8
    assert S.step_pass_count(S.dims(1 << 20, 4, 8), 26214) == 1  # 10% density
    assert S.step_pass_count(S.dims(100, 3, 1), 1) == -1


@pytest.mark.parametrize("n,P,K,k", [(100, 3, 1, 1), (100, 4, 0, 1), (100, 0, 1, 1), (100, 4, 1, 0),
                                     (100, 4, 1, 26), (1 << 32, 1, 1, 1), (0, 1, 1, 1)])
def test_invalid_shapes(n, P, K, k):
    L = S.lib()
    d = S.dims(n, P, K)
    assert S.mask_bytes(d, k) == 0
    assert S.workspace_bytes(d, k) == 0
    st = L.scape_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k, S.betas(), 1e-3, 1, FAKE,
                      1 << 40, None)
    assert st == 2
    assert b"invalid shape" in L.scape_last_error()


def _step(d, k, ptrs=None, bt=None, lr=1e-3, step=1, wsb=None):
    L = S.lib()
    p = dict(params=FAKE, grads=FAKE, m=FAKE, v=FAKE, e=FAKE, mask=FAKE, ws=FAKE)
    p.update(ptrs or {})
    return L.scape_step(ctypes.byref(d), p["params"], p["grads"], p["m"], p["v"], p["e"], p["mask"], k,
                        bt or S.betas(), lr, step, p["ws"],
                        S.workspace_bytes(d, k) if wsb is None else wsb, None)


# v is optional (NULL: the second moment is not stored), so it is not here:
# with fake addresses a call that passes validation would launch kernels.
@pytest.mark.parametrize("which", ["params", "grads", "m", "e", "mask", "ws"])
def test_step_rejects_null_pointers(which):
    d = S.dims(4096, 2, 2)
    assert _step(d, 10, {which: None}) == 1


@pytest.mark.parametrize("bt,lr", [
    (S.betas(beta1=1.0), 1e-3), (S.betas(beta1=-0.1), 1e-3), (S.betas(beta2=1.5), 1e-3),
    (S.betas(eps=0.0), 1e-3), (S.betas(eps=float("inf")), 1e-3), (S.betas(weight_decay=float("nan")), 1e-3),
    (S.betas(), float("nan")), (S.betas(), float("inf")), (S.betas(beta1=float("nan")), 1e-3),
])
def test_step_rejects_bad_hyper_parameters(bt, lr):
    d = S.dims(4096, 2, 2)
    assert _step(d, 10, bt=bt, lr=lr) == 1


def test_step_rejects_step_zero_and_small_workspace():
    d = S.dims(4096, 2, 2)
    assert _step(d, 10, step=0) == 1
    assert _step(d, 10, wsb=S.workspace_bytes(d, 10) - 1) == 3
    assert b"workspace" in S.lib().scape_last_error()


def _step_graph(d, k, cur_slot=1, bias=FAKE, ptrs=None, bt=None, wsb=None):
    L = S.lib()
    p = dict(params=FAKE, grads=FAKE, m=FAKE, v=FAKE, e=FAKE, mask=FAKE, ws=FAKE)
    p.update(ptrs or {})
    return L.scape_step_graph(ctypes.byref(d), p["params"], p["grads"], p["m"], p["v"], p["e"], p["mask"], k,
                              bt or S.betas(), 1e-3, cur_slot, bias, p["ws"],
                              S.workspace_bytes(d, k) if wsb is None else wsb, None)


def test_step_graph_validation():
    """Rejected before anything is enqueued (no device needed)."""
    d = S.dims(4096, 2, 2)
    assert _step_graph(d, 10, cur_slot=2) == 1
    assert b"cur_slot" in S.lib().scape_last_error()
    assert _step_graph(d, 10, cur_slot=-1) == 1
    assert _step_graph(d, 10, bias=None) == 1
    assert _step_graph(d, 10, bias=FAKE + 4) == 1
    assert b"aligned" in S.lib().scape_last_error()
    assert _step_graph(d, 10, ptrs={"e": None}) == 1
    assert _step_graph(d, 10, bt=S.betas(beta2=1.0)) == 1
    assert _step_graph(d, 10, wsb=S.workspace_bytes(d, 10) - 1) == 3
    assert _step_graph(S.dims(4096, 3, 2), 10) == 2


def test_bias_state_matches_stepwise_binary64_products():
    """beta^t is formed one multiplication per step in binary64 from the
    fp32 beta, and the reciprocal 1/(1 - beta^t) is rounded once to fp32:
    the values the host-side step uses ([P] §II-C, bias correction)."""
    import numpy as np
    bt = S.betas(0.9, 0.95, 1e-8, 0.0)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.95))
    for t in (0, 1, 2, 7, 1000, 7, 1001, 2, 1):  # forward, back, forward: products are resumed only from below
        st = S.bias_state_at(bt, t)
        p1 = p2 = 1.0
        for _ in range(t):
            p1, p2 = p1 * b1, p2 * b2
        assert st.beta1_pow == p1 and st.beta2_pow == p2
        if t:
            assert st.ibc1 == np.float32(1.0 / (1.0 - p1)) and st.ibc2 == np.float32(1.0 / (1.0 - p2))
        else:
            assert st.ibc1 == 0.0 and st.ibc2 == 0.0
    assert S.bias_state_at(bt, 1).ibc1 == np.float32(9.999998)
    with pytest.raises(S.ScapeError):
        S.bias_state_at(bt, -1)
    with pytest.raises(S.ScapeError):
        S.bias_state_at(S.betas(beta1=1.0), 3)


def test_component_validation():
    L = S.lib()
    d = S.dims(4096, 2, 2)
    mv = S.MaskView(FAKE, FAKE, FAKE)
    nul = S.MaskView(FAKE, None, FAKE)
    ws = S.workspace_bytes(d, 10)
    assert L.scape_mask_topk(ctypes.byref(d), 10, None, mv, FAKE, ws, None) == 1
    assert L.scape_mask_topk(ctypes.byref(d), 10, FAKE, nul, FAKE, ws, None) == 1
    assert L.scape_mask_topk(ctypes.byref(d), 10, FAKE, mv, FAKE, ws - 1, None) == 3
    assert L.scape_mask_topk(ctypes.byref(d), 2049, FAKE, mv, FAKE, ws, None) == 2
    assert L.scape_compress(ctypes.byref(d), 10, FAKE, None, mv, FAKE, None) == 1
    assert L.scape_compress(ctypes.byref(d), 10, FAKE, FAKE, S.MaskView(None, FAKE, FAKE), FAKE, None) == 1
    assert L.scape_reduce_sparse(ctypes.byref(d), 10, FAKE, None, None) == 1
    assert L.scape_adams_update(ctypes.byref(d), 10, FAKE, FAKE, FAKE, FAKE, mv, S.betas(), 1e-3, 0, None) == 1
    assert L.scape_adams_update(ctypes.byref(d), 10, FAKE, FAKE, FAKE, FAKE, nul, S.betas(), 1e-3, 1, None) == 1
    assert L.scape_adams_update(ctypes.byref(d), 10, FAKE, FAKE, FAKE, FAKE, mv, S.betas(beta2=1.0), 1e-3, 1,
                                None) == 1
    assert L.scape_mask_overlap(ctypes.byref(d), 10, mv, mv, None, None) == 1
    assert L.scape_dense_adams_step(ctypes.byref(d), FAKE, None, FAKE, FAKE, S.betas(), 1e-3, 1, None) == 1
    assert L.scape_dense_adams_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, S.betas(eps=-1.0), 1e-3, 1, None) == 1
    assert L.scape_dense_adams_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, S.betas(), 1e-3, 0, None) == 1
    assert L.scape_dense_adams_step(ctypes.byref(S.dims(4097, 2, 1)), FAKE, FAKE, FAKE, FAKE, S.betas(), 1e-3, 1,
                                    None) == 2
    assert L.scape_mask_topk(None, 10, FAKE, mv, FAKE, ws, None) == 1


def test_count_nonfinite_validation():
    """The debug count of non-finite inputs checks its arguments before any
    HIP call: a negative count, or a null array or counter with elements to
    count, is EINVAL; an empty array launches nothing."""
    L = S.lib()
    assert L.scape_count_nonfinite(FAKE, -1, FAKE, None) == 1
    assert L.scape_count_nonfinite(None, 5, FAKE, None) == 1
    assert L.scape_count_nonfinite(FAKE, 5, None, None) == 1
    assert L.scape_count_nonfinite(None, 0, None, None) == 0


def test_offload_validation():
    L = S.lib()
    d = S.dims(4096, 4, 2)
    assert S.offload_stage_bytes(d, 10, 0) == 0
    assert S.offload_stage_bytes(d, 10, 3) == 2 * 2 * 3 * 1024 * 4
    assert S.offload_stage_bytes(d, 10, 9) == 2 * 2 * 4 * 1024 * 4   # at most P partitions per chunk
    wsb = S.workspace_bytes(d, 10)
    sb = S.offload_stage_bytes(d, 10, 2)
    def call(chunk=2, stage=FAKE, stage_bytes=sb, e=FAKE, streams=(0x100, 0x200, 0x300)):
        return L.scape_step_offload(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, e, FAKE, 10, S.betas(), 1e-3, 1, FAKE,
                                    wsb, stage, stage_bytes, chunk, *streams)
    assert call(chunk=0) == 1
    assert call(stage=None) == 1
    assert call(stage_bytes=sb - 1) == 3
    assert call(e=None) == 1
    for streams in ((None, None, None), (0x100, 0x100, 0x300), (0x100, 0x200, 0x100), (0x100, 0x300, 0x300)):
        assert call(streams=streams) == 1
        assert b"distinct" in L.scape_last_error()


def test_status_strings_and_profile_names():
    L = S.lib()
    assert L.scape_status_string(0) == b"ok"
    assert L.scape_status_string(3) == b"workspace too small"
    names = S.profile_stage_names()
    assert names == ["bootstrap_select", "step_pass", "select_pass", "refine", "emit"]
    assert L.scape_profile_collect(None, None) == 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(S, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        S.lib()


def test_binding_checks_tensor_arguments_before_the_device_sees_them():
    """Host tensors, wrong dtypes and short buffers are refused by the
    binding (they would be device memory faults, not errors, in the library)."""
    torch = pytest.importorskip("torch")
    d = S.dims(4096, 2, 2)
    cpu = torch.zeros(4096)
    with pytest.raises(ValueError, match="device tensor"):
        S.step(d, cpu, None, None, None, None, None, 10, S.betas(), 1e-3, 1, None)
    with pytest.raises(ValueError, match="pinned host memory"):
        S._need(torch.zeros(4), "e", 4, pinned=True)
    meta = torch.device("meta")
    with pytest.raises(ValueError, match="device tensor"):
        S._need(torch.zeros(4, device=meta), "x", 4)
    # dtype, contiguity and size are checked on device tensors; a fake stand-in
    # for one is enough here (no GPU in this test)
    class Fake:
        is_cuda = True
        def __init__(self, dtype, n, contiguous=True, esize=4):
            self.dtype, self._n, self._c, self._e = dtype, n, contiguous, esize
        def numel(self): return self._n
        def element_size(self): return self._e
        def is_contiguous(self): return self._c
        def is_pinned(self): return False
    with pytest.raises(ValueError, match="float32"):
        S._need(Fake(torch.float16, 4096, esize=2), "params", 4096)
    with pytest.raises(ValueError, match="contiguous"):
        S._need(Fake(torch.float32, 4096, contiguous=False), "params", 4096)
    with pytest.raises(ValueError, match="too small"):
        S._need(Fake(torch.float32, 4095), "params", 4096)
    with pytest.raises(ValueError, match="too small"):
        S._need(Fake(torch.uint8, 99, esize=1), "workspace", 100, dtype=None)
    S._need(Fake(torch.float32, 4096), "params", 4096)
    S._need(Fake(torch.uint8, 100, esize=1), "workspace", 100, dtype=None)


def test_optimizer_step_count_unchanged_by_a_rejected_call():
    """A step the binding refuses (host tensors here: no GPU in this test)
    leaves ScapeOptimizer's step count, and so its mask slot choice, as it
    was."""
    torch = pytest.importorskip("torch")
    opt = S.ScapeOptimizer(torch.zeros(4096), P=2, K=2, k=10, device="cpu")
    with pytest.raises(ValueError, match="device tensor"):
        opt.step(torch.zeros((2, 4096)))
    assert opt.t == 0


def test_step_noalloc_rejects_dims_beyond_its_static_scratch():
    """scape_step_noalloc refuses, before any HIP call, dims whose workspace
    exceeds the static scratch, and names both sizes; dims that fit pass
    that check (they then need a device, so are not called here)."""
    L = S.lib()
    cap = S.step_noalloc_max_bytes()
    assert cap == 64 << 20
    big = S.dims(1 << 24, 4, 2)  # candidate slots alone: 8 bytes per element
    assert S.workspace_bytes(big, 1000) > cap
    st = L.scape_step_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1000, S.betas(), 1e-3, 1, None)
    assert st == 3
    msg = L.scape_last_error().decode()
    assert "static scratch" in msg and str(cap) in msg
    assert S.workspace_bytes(S.dims(4 * 60_000, 4, 3), 600) < cap
    # argument checks come first, as in scape_step
    assert L.scape_step_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1000, S.betas(), 1e-3, 1, None) == 1
    assert L.scape_step_noalloc(ctypes.byref(S.dims(100, 3, 1)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                S.betas(), 1e-3, 1, None) == 2


@pytest.mark.parametrize("P,K", [(32, 8), (6, 4), (5, 3), (3, 5), (1, 1), (7, 7)])
def test_shard_partitions_are_the_owners(P, K):
    """Rank r owns exactly the partitions p with floor(p*K/P) == r, as one
    contiguous range; the ranges tile [0, P)."""
    d = S.dims(P * 64, P, K)
    seen = []
    for r in range(K):
        first, count = S.shard_partitions(d, r)
        assert list(range(first, first + count)) == [p for p in range(P) if (p * K) // P == r]
        seen += list(range(first, first + count))
    assert seen == list(range(P))
    with pytest.raises(S.ScapeError):
        S.shard_partitions(d, K)
    with pytest.raises(S.ScapeError):
        S.shard_partitions(d, -1)


def test_shard_calls_validate_before_any_hip_call():
    L = S.lib()
    d = S.dims(4096, 4, 2)
    bt = S.betas()
    assert L.scape_shard_compress(ctypes.byref(d), 10, 2, FAKE, FAKE, FAKE, FAKE, FAKE, bt, 1, FAKE, 1 << 30,
                                  None) == 1  # rank out of range
    assert L.scape_shard_compress(ctypes.byref(d), 10, 0, FAKE, FAKE, FAKE, FAKE, FAKE, bt, 0, FAKE, 1 << 30,
                                  None) == 1  # step 0
    assert L.scape_shard_compress(ctypes.byref(d), 10, 0, FAKE, FAKE, FAKE, FAKE, FAKE, bt, 1, FAKE, 16,
                                  None) == 3  # workspace too small
    assert L.scape_shard_select_initial(ctypes.byref(d), 2000, 0, FAKE, FAKE, FAKE, FAKE, bt, FAKE, 1 << 30,
                                        None) == 2  # k > n_p
    assert L.scape_shard_update(ctypes.byref(d), 10, 1, FAKE, FAKE, None, None, FAKE, bt, 1e-3, 1, None) == 1
    # a rank that owns no partition (K > P) may pass no b_bar
    d3 = S.dims(300, 3, 5)
    assert S.shard_partitions(d3, 2) == (2, 0)
    assert L.scape_shard_update(ctypes.byref(d3), 10, 2, FAKE, FAKE, None, None, FAKE, bt, 1e-3, 1, None) == 0
