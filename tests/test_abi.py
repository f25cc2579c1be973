"""The C-ABI library loads, exports every declared symbol and validates arguments on the
host before touching a GPU (CPU only: every call here fails validation, so nothing launches)."""
import ctypes
import os
import re
import subprocess

import pytest

import contextual_activation_sparsity_amd as dv
from contextual_activation_sparsity_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dejavu_hip.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"dv_predict", "dv_topk", "dv_sparse_mlp", "dv_sparse_attn", "dv_layer_step"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dv_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = _lib.lib()
    for n in names:
        assert getattr(L, n) is not None
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings_and_version():
    L = _lib.lib()
    assert L.dv_status_str(0) == b"ok"
    assert L.dv_status_str(7) == b"workspace too small"
    assert b"gfx950" in L.dv_version()


def dims(**kw):
    base = dict(d_model=768, d_ffn=3072, n_heads=12, head_dim=64, rank_mlp=128, rank_head=128, t_max=129,
                dtype="f32")
    base.update(kw)
    return dv.Dims(**base)


def test_workspace_bytes():
    n1 = dv.dv_workspace_bytes(dims(), 1, 307, 3)
    n2 = dv.dv_workspace_bytes(dims(), 4, 307, 3)
    assert 0 < n1 < n2
    assert dv.dv_workspace_bytes(dims(d_model=700), 1, 10, 3) == 0   # d != H*dh
    assert dv.dv_stack_workspace_bytes(dims(), 1, 307, 3) > 2 * n1


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def layer_struct(ptr=FAKE):
    return _lib.DvLayer(*([ptr] * 10))


def call_mlp(d, B=1, k=10, xn=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30, L=None, idx=FAKE):
    L = L if L is not None else layer_struct()
    dd = d.c()
    return _lib.lib().dv_sparse_mlp(ctypes.byref(dd), ctypes.byref(L), xn, B, idx, k, y, ws, ws_bytes, None)


def test_validation_codes_mlp():
    assert call_mlp(dims(d_model=700)) == 2                  # DV_ERR_DIMS
    assert call_mlp(dims(head_dim=32, n_heads=24)) == 2      # unsupported head_dim
    assert call_mlp(dims(dtype="f16", d_model=772, n_heads=4, head_dim=193)) in (2, 5)
    assert call_mlp(dims(), k=3073) == 3                     # DV_ERR_K
    assert call_mlp(dims(), k=-1) == 3
    assert call_mlp(dims(), B=0) == 2
    assert call_mlp(dims(), xn=None) == 1                    # DV_ERR_NULL
    assert call_mlp(dims(), xn=FAKE + 4) == 5                # DV_ERR_ALIGN
    assert call_mlp(dims(), L=layer_struct(None)) == 1
    assert call_mlp(dims(), ws=FAKE + 16) == 7               # DV_ERR_WORKSPACE (alignment)
    assert call_mlp(dims(), ws_bytes=16) == 7
    assert b"workspace" in _lib.lib().dv_last_error()
    dd = dims().c()
    bad = _lib.DvDims(dd.d_model, dd.d_ffn, dd.n_heads, dd.head_dim, dd.rank_mlp, dd.rank_head, dd.t_max, 9)
    L = layer_struct()
    assert _lib.lib().dv_sparse_mlp(ctypes.byref(bad), ctypes.byref(L), FAKE, 1, FAKE, 1, FAKE, FAKE, 1 << 30,
                                    None) == 4            # DV_ERR_DTYPE
    assert _lib.lib().dv_sparse_mlp(None, ctypes.byref(L), FAKE, 1, FAKE, 1, FAKE, FAKE, 1 << 30, None) == 1


def test_validation_codes_attn_and_layer():
    d = dims().c()
    L = layer_struct()
    f = _lib.lib().dv_sparse_attn
    assert f(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 3, FAKE, FAKE, 128, FAKE, FAKE, 16, None) == 7
    assert f(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 3, FAKE, FAKE, 129, FAKE, FAKE, 1 << 30, None) == 6
    assert f(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 3, FAKE, FAKE, -1, FAKE, FAKE, 1 << 30, None) == 6
    assert f(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 13, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30, None) == 3
    g = _lib.lib().dv_layer_step
    P = _lib.DvPredictor(FAKE, FAKE, FAKE, FAKE)
    # only one of idx_in / heads_in given
    assert g(ctypes.byref(d), ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, 1, 10, 3, FAKE, None, FAKE, FAKE, 0,
             FAKE, None, None, FAKE, 1 << 30, None) == 1
    # inline prediction without predictor
    assert g(ctypes.byref(d), ctypes.byref(L), None, FAKE, FAKE, 1, 10, 3, None, None, FAKE, FAKE, 0,
             FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert g(ctypes.byref(d), ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, 1, 10, 3, None, None, FAKE, FAKE, 0,
             FAKE, None, None, FAKE, 8, None) == 7


def test_validation_codes_topk():
    f = _lib.lib().dv_topk
    assert f(FAKE, 1, 100, 101, FAKE, None, 0, None) == 3
    assert f(FAKE, 1, 70000, 5, FAKE, None, 0, None) == 2
    assert f(None, 1, 100, 5, FAKE, None, 0, None) == 1
    assert f(FAKE, 0, 100, 5, FAKE, None, 0, None) == 2
    assert f(FAKE, 1, 100, 0, None, None, 0, None) == 0       # k = 0: nothing to do, nothing launched
    need = _lib.lib().dv_topk_workspace_bytes(1, 100)
    assert need > 0 and need % 256 == 0
    assert f(FAKE, 1, 100, 5, FAKE, None, 0, None) == 7       # k > 0 needs the workspace
    assert f(FAKE, 1, 100, 5, FAKE, FAKE, need - 1, None) == 7


def test_topk_workspace_size():
    g = _lib.lib().dv_topk_workspace_bytes
    assert g(0, 100) == 0 and g(1, 0) == 0 and g(1, 65537) == 0
    one, two = g(1, 49152), g(2, 49152)
    # per row at least: 12 chunk histograms of 2048 counts, the candidate keys and positions
    assert one >= 4 * (12 * 2048 + 2 * 49152) and two >= 2 * one - 2048


def test_python_raises_with_status_name():
    with pytest.raises(_lib.DejavuError) as e:
        _lib.check("dv_sparse_mlp", 3)
    assert e.value.status_name == "DV_ERR_K"


def test_validation_codes_blocked():
    f = _lib.lib().dv_block_scores
    assert f(FAKE, 1, 100, 8, FAKE, None) == 2        # 8 does not divide 100
    assert f(FAKE, 1, 100, 0, FAKE, None) == 2
    assert f(None, 1, 100, 4, FAKE, None) == 1
    assert f(FAKE, 0, 100, 4, FAKE, None) == 2
    assert f(FAKE + 4, 1, 100, 4, FAKE, None) == 5   # scores not 16-byte aligned
    g = _lib.lib().dv_sparse_mlp_blocked
    d, L = dims().c(), layer_struct()
    assert g(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 4, 7, FAKE, FAKE, 1 << 30, None) == 2   # 7 does not divide d_ffn
    assert g(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 3073, 1, FAKE, FAKE, 1 << 30, None) == 3
    assert g(ctypes.byref(d), ctypes.byref(L), FAKE, 1, None, 4, 8, FAKE, FAKE, 1 << 30, None) == 1
    assert g(ctypes.byref(d), ctypes.byref(L), FAKE, 1, FAKE, 4, 8, FAKE, FAKE, 16, None) == 7


def test_validation_codes_decode_step():
    f = _lib.lib().dv_decode_step
    d = dims().c()
    Ls = (_lib.DvLayer * 1)(layer_struct())
    Ps = (_lib.DvPredictor * 1)(_lib.DvPredictor(FAKE, FAKE, FAKE, FAKE))
    kc = (ctypes.c_void_p * 1)(FAKE)
    vc = (ctypes.c_void_p * 1)(FAKE)

    def call(t_rows, n=1, k=10, ws_bytes=1 << 30):
        return f(ctypes.byref(d), Ls, Ps, n, FAKE, 1, k, 3, kc, vc, t_rows, 1, FAKE, None, None, None, FAKE,
                 ws_bytes, None, None)

    assert call(None) == 1                 # per-row lengths are required
    assert call(FAKE + 2) == 5             # not 4-byte aligned
    assert call(FAKE, n=0) == 2            # no layers
    assert call(FAKE, k=3073) == 3         # k above d_ffn
    assert call(FAKE, ws_bytes=16) == 7    # workspace too small


def test_validation_codes_training():
    f = _lib.lib().dv_predictor_train_step
    g = _lib.lib().dv_predictor_train_workspace_bytes
    assert g(0, 8, 8, 2) == 0 and g(8, 8, 8, -1) == 0
    need = g(64, 32, 16, 4)
    assert need > 4 * (64 * 16 + 2 * 64 * 4) and need % 256 == 0

    def call(M=64, d=32, N=16, r=4, lr=0.1, mu=0.9, x=FAKE, loss=FAKE, ws_bytes=1 << 30):
        return f(x, M, d, FAKE, N, r, FAKE, FAKE, FAKE, FAKE, lr, mu, loss, FAKE, ws_bytes, None)

    assert call(M=0) == 2
    assert call(lr=float("nan")) == 2
    assert call(mu=-0.5) == 2
    assert call(x=None) == 1
    assert call(x=FAKE + 4) == 5
    assert call(loss=FAKE + 2) == 5       # the loss slot needs 4-byte alignment only
    assert call(ws_bytes=need - 1) == 7
    h = _lib.lib().dv_layer_labels
    d = dims().c()
    L = layer_struct()
    assert h(ctypes.byref(d), ctypes.byref(L), FAKE, 2, FAKE, FAKE, 0, None, None, None, FAKE, 1 << 30, None) == 1
    assert h(ctypes.byref(d), ctypes.byref(L), FAKE, 0, FAKE, FAKE, 0, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert h(ctypes.byref(d), ctypes.byref(L), FAKE, 2, FAKE, FAKE, 129, FAKE, None, None, FAKE, 1 << 30, None) == 6
    assert h(ctypes.byref(d), ctypes.byref(L), FAKE, 2, FAKE, FAKE, 0, FAKE, None, None, FAKE, 64, None) == 7


def test_validation_codes_check_indices():
    f = _lib.lib().dv_check_indices
    assert f(FAKE, 0, 4, 10, FAKE, None) == 2        # B <= 0: DV_ERR_DIMS
    assert f(FAKE, 1, 4, 0, FAKE, None) == 2         # n <= 0
    assert f(FAKE, 1, 11, 10, FAKE, None) == 3       # k > n: DV_ERR_K
    assert f(FAKE, 1, -1, 10, FAKE, None) == 3
    assert f(FAKE, 1, 4, 10, None, None) == 1        # status NULL: DV_ERR_NULL
    assert f(None, 1, 4, 10, FAKE, None) == 1        # idx NULL with k > 0
    assert f(FAKE + 2, 1, 4, 10, FAKE, None) == 5    # misaligned idx: DV_ERR_ALIGN
    assert f(FAKE, 1, 4, 10, FAKE + 1, None) == 5    # misaligned status
    assert b"status" in _lib.lib().dv_last_error()


def test_noalloc_refuses_oversized_scratch_before_any_launch():
    """The allocation-free step refuses shapes whose workspace exceeds its fixed array, with
    DV_ERR_WORKSPACE, before any HIP call (so this runs without a GPU)."""
    d = dims(d_model=12288, d_ffn=49152, n_heads=96, head_dim=128, rank_mlp=1000, rank_head=1000, t_max=1025,
             dtype="f16")
    assert dv.dv_workspace_bytes(d, 32, 2458, 19) > 32 << 20
    dd, L = d.c(), layer_struct()
    P = _lib.DvPredictor(FAKE, FAKE, FAKE, FAKE)
    st = _lib.lib().dv_layer_step_noalloc(ctypes.byref(dd), ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, 32, 2458, 19,
                                          None, None, FAKE, FAKE, 100, FAKE, None, None, None)
    assert st == 7
    assert b"DV_NOALLOC_SCRATCH_BYTES" in _lib.lib().dv_last_error()
    st = _lib.lib().dv_layer_step_noalloc(ctypes.byref(dd), ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, 0, 2458, 19,
                                          None, None, FAKE, FAKE, 100, FAKE, None, None, None)
    assert st == 2   # invalid arguments: dv_layer_step's own check (B <= 0)
