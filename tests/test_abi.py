"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments before any HIP call (fake device addresses are
never dereferenced because every call here fails validation)."""
import ctypes
import os
import re

import pytest

import diffusion_transformer_image_amd as dit
from diffusion_transformer_image_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x7F0000000000  # a 16-byte aligned fake device address, never touched


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "dit.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = dit.lib()
    syms = declared_symbols()
    assert len(syms) >= 14
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(dit.EXPORTS)


def cfg(**kw):
    base = dict(batch=2, seq_len=80, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=688,
                eps=1e-6, dtype="f32")
    base.update(kw)
    return dit.make_config(**base)


def test_status_strings():
    L = dit.lib()
    for code in range(8):
        assert L.dit_status_str(code)
    assert L.dit_status_str(0) == b"ok"


@pytest.mark.parametrize("kw,expect", [
    (dict(batch=0), "DIT_ERR_SHAPE"),
    (dict(seq_len=-1), "DIT_ERR_SHAPE"),
    (dict(hidden=255), "DIT_ERR_SHAPE"),          # != H * d
    (dict(n_kv_heads=3), "DIT_ERR_SHAPE"),        # H % Hkv != 0
    (dict(n_heads=8, head_dim=32, n_kv_heads=1), "DIT_ERR_UNSUPPORTED"),  # group 8
    (dict(n_heads=6, head_dim=64, hidden=384, n_kv_heads=2), "DIT_ERR_UNSUPPORTED"),  # group 3
    (dict(n_heads=3, head_dim=64, hidden=192, n_kv_heads=1), "DIT_ERR_UNSUPPORTED"),  # group 3
    (dict(head_dim=32, n_heads=8, n_kv_heads=4), "DIT_ERR_UNSUPPORTED"),  # d = 32
    (dict(dtype="bf16"), "DIT_ERR_UNSUPPORTED"),  # bf16 needs d = 128
    (dict(ffn=690), "DIT_ERR_UNSUPPORTED"),       # ffn % 8
    (dict(eps=-1.0), "DIT_ERR_SHAPE"),
])
def test_bad_config_is_rejected(kw, expect):
    c = cfg(**kw)
    assert dit.workspace_size(c) == 0
    w = _lib.BlockWeights(P, P, P, P, P, P, P)
    st = dit.lib().dit_block_fwd(ctypes.byref(c), ctypes.byref(w), P, P + (1 << 30), P + (2 << 30),
                                 P + (3 << 30), 1 << 40, None)
    assert _lib.STATUS[st] == expect


@pytest.mark.parametrize("heads,kv", [(6, 2), (3, 1), (12, 4)])
def test_group_without_attention_kernel_is_rejected_everywhere(heads, kv):
    """Only 1, 2 and 4 query heads per KV head have attention kernels: any
    other group is refused by every entry point before anything is enqueued."""
    c = cfg(n_heads=heads, n_kv_heads=kv, head_dim=64, hidden=64 * heads)
    L = dit.lib()
    assert L.dit_workspace_size(ctypes.byref(c)) == 0
    assert L.dit_stack_workspace_size(ctypes.byref(c)) == 0
    w = _lib.BlockWeights(P, P, P, P, P, P, P)
    st = L.dit_block_fwd(ctypes.byref(c), ctypes.byref(w), P, P + (1 << 30), P + (2 << 30),
                         P + (3 << 30), 1 << 40, None)
    assert _lib.STATUS[st] == "DIT_ERR_UNSUPPORTED"
    st = L.dit_attention(ctypes.byref(c), P, P + (1 << 30), P + (2 << 30), 1 << 40, None)
    assert _lib.STATUS[st] == "DIT_ERR_UNSUPPORTED"
    st = L.dit_stack_fwd(ctypes.byref(c), 1, ctypes.byref(w), P, P + (1 << 30), P + (2 << 30),
                         P + (3 << 30), 1 << 40, None)
    assert _lib.STATUS[st] == "DIT_ERR_UNSUPPORTED"


def test_bad_dtype_code():
    c = cfg()
    c.dtype = 7
    assert dit.lib().dit_workspace_size(ctypes.byref(c)) == 0
    st = dit.lib().dit_gemm(5, 16, 16, 16, P, P + 4096, P + 8192, None)
    assert _lib.STATUS[st] == "DIT_ERR_DTYPE"


def call_block(c, w, x_in, x_out, mod, ws, ws_bytes):
    return _lib.STATUS[dit.lib().dit_block_fwd(ctypes.byref(c), ctypes.byref(w) if w else None,
                                               x_in, x_out, mod, ws, ws_bytes, None)]


def test_block_argument_checks():
    c = cfg()
    need = dit.workspace_size(c)
    assert need > 0
    w = _lib.BlockWeights(P, P, P, P, P, 0, 0)
    G = 1 << 30
    X, Y, M, WS = P + G, P + 2 * G, P + 3 * G, P + 4 * G
    assert call_block(c, None, X, Y, M, WS, need) == "DIT_ERR_NULL"
    assert call_block(c, _lib.BlockWeights(0, P, P, P, P, 0, 0), X, Y, M, WS, need) == "DIT_ERR_NULL"
    assert call_block(c, w, 0, Y, M, WS, need) == "DIT_ERR_NULL"
    assert call_block(c, w, X, Y, 0, WS, need) == "DIT_ERR_NULL"
    assert call_block(c, w, X, Y, M, 0, need) == "DIT_ERR_WORKSPACE"
    assert call_block(c, w, X, Y, M, WS, need - 1) == "DIT_ERR_WORKSPACE"
    assert call_block(c, w, X + 8, Y, M, WS, need) == "DIT_ERR_ALIGN"
    assert call_block(c, _lib.BlockWeights(P + 4, P, P, P, P, 0, 0), X, Y, M, WS, need) == "DIT_ERR_ALIGN"
    assert call_block(c, w, X, X + 64, M, WS, need) == "DIT_ERR_SHAPE"  # x_out overlaps x_in
    assert call_block(c, w, X, Y, M, X, need) == "DIT_ERR_SHAPE"  # workspace overlaps x_in
    # the workspace must not overlap any weight buffer either
    for i in range(7):
        ptrs = [P, P, P, P, P, 0, 0]
        ptrs[i] = WS + need - 256  # inside the workspace's last bytes
        assert call_block(c, _lib.BlockWeights(*ptrs), X, Y, M, WS, need) == "DIT_ERR_SHAPE", i
    assert call_block(c, _lib.BlockWeights(P, P, P, P, P, 0, 0, WS, 0), X, Y, M, WS, need) == "DIT_ERR_SHAPE"


def test_stack_argument_checks():
    c = cfg()
    need = dit.stack_workspace_size(c)
    assert need > dit.workspace_size(c)
    arr = (_lib.BlockWeights * 2)(_lib.BlockWeights(P, P, P, P, P, 0, 0), _lib.BlockWeights(P, P, 0, P, P, 0, 0))
    G = 1 << 30
    L = dit.lib()
    st = L.dit_stack_fwd(ctypes.byref(c), 0, arr, P + G, P + 2 * G, P + 3 * G, P + 4 * G, need, None)
    assert _lib.STATUS[st] == "DIT_ERR_SHAPE"
    st = L.dit_stack_fwd(ctypes.byref(c), 2, arr, P + G, P + 2 * G, P + 3 * G, P + 4 * G, need, None)
    assert _lib.STATUS[st] == "DIT_ERR_NULL"  # block 1 lacks w_13
    st = L.dit_stack_fwd(ctypes.byref(c), 1, arr, P + G, P + 2 * G, P + 3 * G, P + 4 * G, need - 16, None)
    assert _lib.STATUS[st] == "DIT_ERR_WORKSPACE"


def test_step_argument_checks():
    L = dit.lib()
    c = cfg()
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    assert S(L.dit_gemm(0, 0, 16, 16, P, P + G, P + 2 * G, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_gemm(0, 16, 16, 12, P, P + G, P + 2 * G, None)) == "DIT_ERR_UNSUPPORTED"  # K % 8
    assert S(L.dit_gemm(1, 16, 16, 16, P + 2, P + G, P + 2 * G, None)) == "DIT_ERR_ALIGN"
    assert S(L.dit_gemm(1, 16, 16, 16, P, P + G, P + 64, None)) == "DIT_ERR_SHAPE"  # C overlaps A
    assert S(L.dit_gemm_swiglu(1, 16, 16, 16, 0, P + G, P + 2 * G, None)) == "DIT_ERR_NULL"
    assert S(L.dit_gemm_variant(1, 2, 0, 0, 16, 16, 16, P, P + G, P + 2 * G, None)) == "DIT_ERR_UNSUPPORTED"
    assert S(L.dit_gemm_variant(1, 0, 65, 0, 16, 16, 16, P, P + G, P + 2 * G, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_gemm_variant(1, 0, -1, 0, 16, 16, 16, P, P + G, P + 2 * G, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_gemm_variant(1, 0, 4, 2, 16, 16, 16, P, P + G, P + 2 * G, None)) == "DIT_ERR_SHAPE"
    # split-K tail: dtype, tile / segment ranges, workspace size and overlap
    sk = lambda *a: S(L.dit_gemm_splitk(*a))
    assert sk(0, 0, 512, 512, 256, P, P + G, P + 2 * G, 1, 2, P + 3 * G, 1 << 20, None) == "DIT_ERR_UNSUPPORTED"
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 5, 2, P + 3 * G, 1 << 24, None) == "DIT_ERR_SHAPE"  # 4 tiles
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 2, 5, P + 3 * G, 1 << 24, None) == "DIT_ERR_SHAPE"  # 4 stages
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 2, 0, P + 3 * G, 1 << 24, None) == "DIT_ERR_SHAPE"
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 2, 2, P + 3 * G, 4 * 65536 * 4 - 4, None) == "DIT_ERR_WORKSPACE"
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 2, 2, 0, 1 << 24, None) == "DIT_ERR_WORKSPACE"
    assert sk(1, 0, 512, 512, 256, P, P + G, P + 2 * G, 2, 2, P + 2 * G + 64, 1 << 24, None) == "DIT_ERR_SHAPE"
    assert sk(1, 2, 512, 512, 256, P, P + G, P + 2 * G, 0, 1, 0, 0, None) == "DIT_ERR_SHAPE"
    assert S(L.dit_attention(ctypes.byref(c), P, 0, P + 2 * G, 1 << 30, None)) == "DIT_ERR_NULL"
    assert S(L.dit_attention(ctypes.byref(c), P, P + 64, P + 2 * G, 1 << 30, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_attention(ctypes.byref(c), P, P + G, P + 2 * G, 16, None)) == "DIT_ERR_WORKSPACE"
    assert S(L.dit_attention(ctypes.byref(c), P, P + G, 0, 1 << 30, None)) == "DIT_ERR_WORKSPACE"
    assert S(L.dit_attention_ex(ctypes.byref(c), P, P + G, P + 2 * G, 1 << 30, 2, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_attention_ex(ctypes.byref(c), P, P + G, P + 2 * G, 1 << 30, 1, None)) == "DIT_ERR_UNSUPPORTED"
    cq = cfg(dtype="bf16", hidden=512, n_heads=4, n_kv_heads=1, head_dim=128)
    assert S(L.dit_attention_ex(ctypes.byref(cq), P, 0, P + 2 * G, 1 << 30, 1, None)) == "DIT_ERR_NULL"
    assert S(L.dit_modnorm(ctypes.byref(c), P, 0, P + G, P + 2 * G, P + 3 * G, 0, 2, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_modnorm(ctypes.byref(c), P, 9, P + G, P + 2 * G, P + 3 * G, 0, 0, None)) == "DIT_ERR_DTYPE"
    cb = cfg(dtype="f32")
    assert S(L.dit_gated_residual(ctypes.byref(cb), P, 0, P + G, P + 2 * G, 0, 0, P + 3 * G, 0, None)) == "DIT_ERR_NULL"
    assert S(L.dit_timestep_mod(ctypes.byref(c), 255, P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, 1 << 20, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_timestep_mod(ctypes.byref(c), 256, P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, 16, None)) == "DIT_ERR_WORKSPACE"
    assert S(L.dit_timer_start(99, 4)) == "DIT_ERR_SHAPE"


def test_workspace_sizes_cover_the_buffers():
    import datagen
    for name in ("c0", "c1", "c3", "c4"):
        dc = datagen.get_config(name)
        c = dit.config_of(dc)
        es = 2 if dc.dtype == "bf16" else 4
        T, D = dc.tokens, dc.hidden
        need = T * D * es * 3 + T * D * 4 + T * max(dc.n_qkvg, dc.ffn) * es
        assert dit.workspace_size(c) >= need
        assert dit.stack_workspace_size(c) >= dit.workspace_size(c) + T * D * 4


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libdit.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_gemm_plan_choices():
    """The block's GEMM choices at the 1024 px shapes: the W13 and W2 tails
    are split along K, QKVG runs whole 256-row tiles, O whole 192-row tiles;
    a split always fits its stated partial buffer."""
    T, D, F = 9216, 4096, 11008
    w13 = dit.gemm_plan(T, F, D, swiglu=True)
    assert (w13["sk_tiles"], w13["segs"]) == (24, 6) and w13["part_bytes"] == 24 * 6 * 65536 * 4
    assert (dit.gemm_plan(T, D, F)["sk_tiles"], dit.gemm_plan(T, D, F)["segs"]) == (64, 4)
    # B = 1: the O product splits its 32 tail tiles 5 ways (8 would write more partials than it saves)
    assert (dit.gemm_plan(T // 2, D, D)["sk_tiles"], dit.gemm_plan(T // 2, D, D)["segs"]) == (32, 5)
    assert dit.gemm_plan(T, 10240, D) == {"variant": 0, "sk_tiles": 0, "segs": 1, "part_bytes": 0}
    assert dit.gemm_plan(T, D, D)["variant"] == 1 and dit.gemm_plan(T, D, D)["sk_tiles"] == 0
    for m in (80, 1000, 4608, 9088, 16384):
        for n, k, sw in ((10240, 4096, False), (4096, 11008, False), (11008, 4096, True)):
            p = dit.gemm_plan(m, n, k, swiglu=sw)
            assert p["part_bytes"] == p["sk_tiles"] * p["segs"] * 65536 * 4
            assert p["sk_tiles"] == 0 or 2 <= p["segs"] <= 8
    with pytest.raises(dit.DitError):
        dit.gemm_plan(0, 16, 16)


def test_prologue_argument_checks():
    """dit_prologue validation happens before anything is enqueued."""
    L = dit.lib()
    c = cfg()
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    good = dit.make_prologue(grid_h=2, grid_w=3, axes=(16, 24, 24))  # head_dim 64
    assert S(L.dit_qk_prologue(ctypes.byref(c), None, 0, 0, P, None)) == "DIT_ERR_NULL"
    assert S(L.dit_qk_prologue(ctypes.byref(c), ctypes.byref(good), 0, 0, 0, None)) == "DIT_ERR_NULL"
    assert S(L.dit_qk_prologue(ctypes.byref(c), ctypes.byref(good), P + 4, 0, P + G, None)) == "DIT_ERR_ALIGN"
    for bad in (dit.make_prologue(grid_h=2, grid_w=3, axes=(16, 24, 16)),        # sum != head_dim
                dit.make_prologue(grid_h=2, grid_w=3, axes=(15, 25, 24)),        # odd
                dit.make_prologue(grid_h=0, grid_w=3, axes=(16, 24, 24)),        # empty grid
                dit.make_prologue(grid_h=2, grid_w=3, axes=(16, 24, 24), theta=0.0),
                dit.make_prologue(grid_h=9, grid_w=9, axes=(16, 24, 24)),        # more tokens than seq_len
                _lib.Prologue(2, 0, 0, 0, (ctypes.c_int32 * 3)(0, 0, 0), 1.0)):
        assert S(L.dit_qk_prologue(ctypes.byref(c), ctypes.byref(bad), 0, 0, P, None)) == "DIT_ERR_SHAPE"
        assert S(L.dit_block_fwd_ex(ctypes.byref(c), ctypes.byref(bad), None, P, P + G, P + 2 * G, P + 3 * G,
                                    1 << 40, None)) == "DIT_ERR_SHAPE"
    # rope off: the grid and axes are not looked at
    off = _lib.Prologue(1, 0, 0, 0, (ctypes.c_int32 * 3)(0, 0, 0), 0.0)
    assert S(L.dit_qk_prologue(ctypes.byref(c), ctypes.byref(off), 0, 0, 0, None)) == "DIT_ERR_NULL"


def test_model_argument_checks():
    """dit_model_velocity / dit_sample reject bad shapes before any launch."""
    L = dit.lib()
    c = cfg()  # seq_len 80
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    mc = dit.make_model_config(4, 8, 8, 16, 32, 256)
    assert dit.model_workspace_size(c, mc) > 0
    mw = _lib.ModelWeights(P, P, P, P, P, 0, P)
    bw = (_lib.BlockWeights * 1)(_lib.BlockWeights(P, P, P, P, P, 0, 0, 0, 0))
    ws_need = dit.model_workspace_size(c, mc)
    args = lambda mcx, mwx, nb=1: (ctypes.byref(c), ctypes.byref(mcx), None, ctypes.byref(mwx), nb, bw,
                                   P + G, ctypes.c_float(0.5), P + 2 * G, P + 3 * G, P + 4 * G, ws_need, None)
    assert S(L.dit_model_velocity(*args(dit.make_model_config(4, 8, 8, 15, 32, 256), mw))) == "DIT_ERR_SHAPE"  # 64+15 != 80
    assert S(L.dit_model_velocity(*args(dit.make_model_config(3, 8, 8, 16, 32, 256), mw))) == "DIT_ERR_SHAPE"  # odd C
    assert S(L.dit_model_velocity(*args(dit.make_model_config(4, 8, 8, 16, 12, 256), mw))) == "DIT_ERR_SHAPE"  # txt_dim
    assert S(L.dit_model_velocity(*args(dit.make_model_config(4, 8, 8, 16, 32, 255), mw))) == "DIT_ERR_SHAPE"  # t_dim
    assert S(L.dit_model_velocity(*args(mc, _lib.ModelWeights(P, 0, P, P, P, 0, P)))) == "DIT_ERR_NULL"  # w_txt
    assert S(L.dit_model_velocity(*args(mc, mw, nb=0))) == "DIT_ERR_SHAPE"
    a = list(args(mc, mw))
    a[-2] = ws_need - 16
    assert S(L.dit_model_velocity(*a)) == "DIT_ERR_WORKSPACE"
    assert S(L.dit_sample(ctypes.byref(c), ctypes.byref(mc), None, ctypes.byref(mw), 1, bw, P + G, 0,
                          ctypes.c_float(3.0), P + 2 * G, P + 4 * G, ws_need, None)) == "DIT_ERR_SHAPE"  # 0 steps
    assert S(L.dit_sample(ctypes.byref(c), ctypes.byref(mc), None, ctypes.byref(mw), 1, bw, P + G, 4,
                          ctypes.c_float(0.0), P + 2 * G, P + 4 * G, ws_need, None)) == "DIT_ERR_SHAPE"  # shift 0
    assert S(L.dit_sample(ctypes.byref(c), ctypes.byref(mc), None, ctypes.byref(mw), 1, bw, P + G, 4,
                          ctypes.c_float(3.0), P + G + 256, P + 4 * G, ws_need, None)) == "DIT_ERR_SHAPE"  # txt on z


def test_sample_cfg_argument_checks():
    """dit_sample_cfg checks its model call at 2B samples on B-sample inputs
    and rejects a bad guidance, a missing unconditional text, a short
    workspace and overlaps before any launch."""
    L = dit.lib()
    c = cfg()  # seq_len 80
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    mc = dit.make_model_config(4, 8, 8, 16, 32, 256)
    need = dit.sample_cfg_workspace_size(c, mc)
    assert need > dit.model_workspace_size(c, mc)
    assert dit.sample_cfg_workspace_size(c, dit.make_model_config(0, 8, 8, 16, 32, 256)) == 0
    mw = _lib.ModelWeights(P, P, P, P, P, 0, P)
    bw = (_lib.BlockWeights * 1)(_lib.BlockWeights(P, P, P, P, P, 0, 0, 0, 0))

    def call(steps=2, shift=3.0, g=4.0, txt=P + 2 * G, txt_null=P + 3 * G, ws=P + 4 * G, nbytes=need):
        return S(L.dit_sample_cfg(ctypes.byref(c), ctypes.byref(mc), None, ctypes.byref(mw), 1, bw, P + G, steps,
                                  ctypes.c_float(shift), ctypes.c_float(g), txt, txt_null, ws, nbytes, None))
    assert call(steps=0) == "DIT_ERR_SHAPE"
    assert call(shift=0.0) == "DIT_ERR_SHAPE"
    assert call(g=float("nan")) == "DIT_ERR_SHAPE" and call(g=float("inf")) == "DIT_ERR_SHAPE"
    assert call(txt_null=0) == "DIT_ERR_NULL"
    assert call(txt_null=P + 3 * G + 4) == "DIT_ERR_ALIGN"
    assert call(nbytes=need - 16) == "DIT_ERR_WORKSPACE"
    assert call(ws=0) == "DIT_ERR_WORKSPACE"
    assert call(txt_null=P + 4 * G + 1024) == "DIT_ERR_SHAPE"  # inside the workspace
    assert call(txt_null=P + G) == "DIT_ERR_SHAPE"  # on z


def test_stack_fp8_argument_checks():
    L = dit.lib()
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    c = dit.make_config(batch=2, seq_len=128, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, ffn=1376,
                        eps=1e-6, dtype="bf16")
    need = dit.stack_workspace_size_fp8(c)
    assert need > dit.workspace_size_fp8(c) > 0
    bw = (_lib.BlockWeightsFp8 * 2)(*[_lib.BlockWeightsFp8(P + 5 * G, P + 5 * G, P + 5 * G, P + 5 * G, P + 6 * G,
                                                           P + 6 * G, P + 6 * G, P + 6 * G, P + 6 * G, 0, 0)] * 2)
    call = lambda nb=2, ws=P + 3 * G, nbytes=need, xo=P + G: S(L.dit_stack_fwd_fp8(
        ctypes.byref(c), nb, bw, P, xo, P + 2 * G, ws, nbytes, None))
    assert call(nb=0) == "DIT_ERR_SHAPE"
    assert call(nbytes=need - 16) == "DIT_ERR_WORKSPACE"
    assert call(xo=P) == "DIT_ERR_SHAPE"              # x_out on x_in
    assert call(ws=P + 5 * G - 1024) == "DIT_ERR_SHAPE"  # workspace over a weight
    f32 = dit.make_config(batch=2, seq_len=128, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, ffn=1376,
                          eps=1e-6, dtype="f32")
    assert dit.stack_workspace_size_fp8(f32) == 0


def test_fp8_argument_checks():
    L = dit.lib()
    G = 1 << 30
    S = lambda st: _lib.STATUS[st]
    assert S(L.dit_quantize_fp8(1, 16, 24, P, P + G, P + 2 * G, None)) == "DIT_ERR_UNSUPPORTED"  # k % 16
    assert S(L.dit_quantize_fp8(7, 16, 32, P, P + G, P + 2 * G, None)) == "DIT_ERR_DTYPE"
    assert S(L.dit_quantize_fp8(1, 16, 32, P, P + 64, P + 2 * G, None)) == "DIT_ERR_SHAPE"  # q overlaps x
    assert S(L.dit_quantize_fp8(1, 16, 32, P, P + G, 0, None)) == "DIT_ERR_NULL"
    assert S(L.dit_gemm_fp8(2, 16, 16, 32, P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None)) == "DIT_ERR_SHAPE"
    assert S(L.dit_gemm_fp8(0, 16, 16, 40, P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None)) == "DIT_ERR_UNSUPPORTED"
    assert S(L.dit_gemm_fp8(0, 16, 16, 32, P, P + G, P + 2 * G, P + 3 * G, P + 2, None)) == "DIT_ERR_ALIGN"
    assert S(L.dit_gemm_fp8(0, 16, 16, 32, P, P + G, P + 2 * G, P + 3 * G, P + 64, None)) == "DIT_ERR_SHAPE"
