"""Host-side checks of the C-ABI library (no GPU needed).

* libdg.so loads and exports every function that include/dg.h declares;
* every argument error that the library detects on the host is reported
  with its status code before anything touches the device.  The pointers
  handed in are non-NULL dummies that the library never dereferences: each
  case here fails validation before the device check, so no case can reach
  a kernel launch even on a machine with a GPU;
* the workspace-size queries behave as documented.
"""
import ctypes as C
import os
import re

import pytest

from block_discrete_diffusion_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
DUMMY = 0x1000        # non-NULL, never dereferenced by a host-side check


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from block_discrete_diffusion_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(dg_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("dg_canvas_init", "dg_denoise_step", "dg_run_canvas", "dg_append_canvas_kv"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTS) == names


def test_kernel_kind_names(L):
    got = [L.dg_kernel_kind_name(i).decode() for i in range(B.DG_NUM_KERNEL_KINDS)]
    assert got == B.KIND_NAMES
    assert got[7] == "lmhead_sampler"
    assert L.dg_kernel_kind_name(B.DG_NUM_KERNEL_KINDS).decode() == "?"
    assert L.dg_kernel_kind_name(-1).decode() == "?"


def model(dtype=B.DG_BF16, V=32768, d=2048, Hq=16, Hkv=4, hd=128, **kw):
    m = B.dg_model(vocab=V, d_model=d, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=hd, mask_id=V - 1, eos_id=-1,
                   dtype=dtype, rope_base=1e4, norm_eps=1e-6, embed=DUMMY, wq=DUMMY, wk=DUMMY, wv=DUMMY,
                   wo=DUMMY, lm_head=DUMMY)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def ws_bytes(L, m, batch=1, C_=256, P=1024):
    return L.dg_workspace_bytes(C.byref(m), batch, C_, P)


def test_workspace_bytes(L):
    m = model()
    w = ws_bytes(L, m)
    assert w > 0
    # grows with the prefix (attention partials), the batch and the vocabulary
    assert ws_bytes(L, m, P=65536) >= w
    assert ws_bytes(L, m, batch=8) > w
    assert ws_bytes(L, model(V=262144)) > w
    assert ws_bytes(L, model(dtype=B.DG_F32, V=256, d=64, Hq=4, Hkv=2, hd=16), C_=16, P=32) > 0
    # unsupported shapes report 0
    assert ws_bytes(L, m, batch=0) == 0
    assert ws_bytes(L, m, batch=B.DG_MAX_BATCH + 1) == 0
    assert ws_bytes(L, m, C_=0) == 0
    assert ws_bytes(L, m, C_=B.DG_MAX_CANVAS + 1) == 0
    assert ws_bytes(L, m, P=-1) == 0
    assert ws_bytes(L, model(d=2000)) == 0
    assert ws_bytes(L, model(hd=96)) == 0
    assert ws_bytes(L, model(Hq=6, Hkv=4)) == 0
    assert ws_bytes(L, model(dtype=7)) == 0
    assert L.dg_workspace_bytes(None, 1, 256, 0) == 0
    assert L.dg_prefill_workspace_bytes(C.byref(m), 512) > 0
    assert L.dg_prefill_workspace_bytes(C.byref(m), 0) == 0


class InitArgs:
    """A complete, valid-looking set of dg_canvas_init arguments made of dummies."""

    def __init__(self, L, batch=1, C_=256, P=1024, cap=None, dtype=B.DG_BF16, **mkw):
        if dtype == B.DG_F32:
            mkw = dict(dict(V=256, d=64, Hq=4, Hkv=2, hd=16), **mkw)
        self.m = model(dtype=dtype, **mkw)
        self.smp = B.dg_sampler(n_steps=48, adaptive_stop=0, stop_conf=0.9)
        cap = P + C_ if cap is None else cap
        self.caches = (B.dg_kv_cache * batch)(*[B.dg_kv_cache(DUMMY, DUMMY, cap, P) for _ in range(batch)])
        self.state = B.dg_canvas_state(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY)
        self.batch, self.C = batch, C_
        self.ws = DUMMY
        self.ws_bytes = L.dg_workspace_bytes(C.byref(self.m), batch, C_, max(cap - C_, 0)) if cap >= C_ else 0

    def call(self, L, out=True, m=True, smp=True, caches=True, state=True):
        h = C.c_void_p()
        st = L.dg_canvas_init(C.byref(h) if out else None, C.byref(self.m) if m else None,
                              C.byref(self.smp) if smp else None, self.caches if caches else None,
                              self.batch, self.C, C.byref(self.state) if state else None, None, None, 0,
                              self.ws, self.ws_bytes, None)
        assert not h.value, "no handle may be returned on failure"
        return st, L.dg_last_error().decode()


def expect(L, a, status, words, **kw):
    st, msg = a.call(L, **kw)
    assert st == status, (st, msg)
    assert words in msg, msg


def test_init_null_arguments(L):
    a = InitArgs(L)
    expect(L, a, B.DG_ERR_NULL, "out is NULL", out=False)
    expect(L, a, B.DG_ERR_NULL, "model is NULL", m=False)
    expect(L, a, B.DG_ERR_NULL, "sampler", smp=False)
    expect(L, a, B.DG_ERR_NULL, "sampler", caches=False)
    expect(L, a, B.DG_ERR_NULL, "sampler", state=False)
    a = InitArgs(L); a.ws = None
    expect(L, a, B.DG_ERR_NULL, "workspace")
    a = InitArgs(L); a.m.wo = None
    expect(L, a, B.DG_ERR_NULL, "weight pointer")
    a = InitArgs(L); a.state.done = None
    expect(L, a, B.DG_ERR_NULL, "canvas-state buffer")
    a = InitArgs(L); a.caches[0].v = None
    expect(L, a, B.DG_ERR_NULL, "cache 0 has a NULL buffer")


def test_init_shape_errors(L):
    expect(L, InitArgs(L, d=2000), B.DG_ERR_SHAPE, "d_model")
    expect(L, InitArgs(L, hd=96), B.DG_ERR_SHAPE, "head_dim")
    expect(L, InitArgs(L, Hq=6, Hkv=4), B.DG_ERR_SHAPE, "n_q_heads")
    expect(L, InitArgs(L, mask_id=32768), B.DG_ERR_SHAPE, "mask_id")
    expect(L, InitArgs(L, eos_id=40000), B.DG_ERR_SHAPE, "eos_id")
    expect(L, InitArgs(L, eos_id=32767), B.DG_ERR_SHAPE, "eos_id == mask_id")
    expect(L, InitArgs(L, rope_base=0.0), B.DG_ERR_SHAPE, "rope_base")
    expect(L, InitArgs(L, dtype=B.DG_F32, hd=15), B.DG_ERR_SHAPE, "even head_dim")
    expect(L, InitArgs(L, dtype=B.DG_F32, hd=258), B.DG_ERR_SHAPE, "even head_dim")
    a = InitArgs(L, batch=1); a.batch = 0
    expect(L, a, B.DG_ERR_SHAPE, "batch 0")
    a = InitArgs(L, batch=1); a.batch = B.DG_MAX_BATCH + 1
    expect(L, a, B.DG_ERR_SHAPE, f"batch {B.DG_MAX_BATCH + 1}")
    a = InitArgs(L); a.C = B.DG_MAX_CANVAS + 1
    expect(L, a, B.DG_ERR_SHAPE, "canvas_len 257")
    a = InitArgs(L); a.smp.n_steps = 0
    expect(L, a, B.DG_ERR_SHAPE, "n_steps")
    a = InitArgs(L); a.smp.adaptive_stop = 1; a.smp.stop_conf = float("nan")
    expect(L, a, B.DG_ERR_SHAPE, "stop_conf")
    a = InitArgs(L); a.m.lm_format = 2
    expect(L, a, B.DG_ERR_UNSUPPORTED, "lm_format")
    a = InitArgs(L); a.m.lm_format = B.DG_LM_FP8
    expect(L, a, B.DG_ERR_NULL, "lm_scale")
    a = InitArgs(L, dtype=B.DG_F32); a.m.lm_format = B.DG_LM_FP8; a.m.lm_scale = DUMMY
    expect(L, a, B.DG_ERR_UNSUPPORTED, "bf16 model")
    a = InitArgs(L); a.smp.adaptive_stop = 3
    expect(L, a, B.DG_ERR_SHAPE, "adaptive_stop must be")
    a = InitArgs(L); a.smp.adaptive_stop = 2; a.smp.stop_entropy = float("inf")
    expect(L, a, B.DG_ERR_SHAPE, "stop_entropy")
    a = InitArgs(L); a.smp.commit_rule = 2
    expect(L, a, B.DG_ERR_SHAPE, "commit_rule")
    a = InitArgs(L); a.smp.commit_rule = 1; a.smp.commit_conf = float("inf")
    expect(L, a, B.DG_ERR_SHAPE, "commit_conf")
    a = InitArgs(L); a.smp.canvas_fill = -1
    expect(L, a, B.DG_ERR_SHAPE, "canvas_fill")
    # the fp32 path keeps a query's scores in LDS: at most 8192 keys
    expect(L, InitArgs(L, dtype=B.DG_F32, C_=16, P=8192 - 8), B.DG_ERR_SHAPE, "8192 keys")


def test_init_unknown_dtype(L):
    expect(L, InitArgs(L, dtype=5), B.DG_ERR_UNSUPPORTED, "unknown dtype")


def test_init_capacity_errors(L):
    expect(L, InitArgs(L, P=1024, cap=1024 + 255 + 1 - 8), B.DG_ERR_CAPACITY, "capacity")
    expect(L, InitArgs(L, P=1024, cap=1024 + 256 + 4), B.DG_ERR_CAPACITY, "multiple of 8")
    a = InitArgs(L, batch=3)
    a.caches[2].len = a.caches[2].capacity - 255
    expect(L, a, B.DG_ERR_CAPACITY, "cache 2")
    a = InitArgs(L); a.caches[0].len = -1
    expect(L, a, B.DG_ERR_CAPACITY, "cache 0")


def test_init_workspace_too_small(L):
    a = InitArgs(L)
    a.ws_bytes -= 1
    expect(L, a, B.DG_ERR_WORKSPACE, "workspace")
    # the workspace is sized for the largest capacity, not the current length
    a = InitArgs(L, batch=2, P=0, cap=65536)
    a.ws_bytes = L.dg_workspace_bytes(C.byref(a.m), 2, 256, 0)
    assert ws_bytes(L, a.m, batch=2, P=65536 - 256) > a.ws_bytes
    expect(L, a, B.DG_ERR_WORKSPACE, "workspace")


def test_handle_calls_reject_null(L):
    for name in ("dg_denoise_step", "dg_run_canvas", "dg_append_canvas_kv", "dg_canvas_reset",
                 "dg_canvas_resume", "dg_profile_enable", "dg_canvas_destroy", "dg_run_steps",
                 "dg_append_request_kv", "dg_canvas_admit", "dg_canvas_set_graph"):
        fn = getattr(L, name)
        args = [0 if t in (C.c_uint32, C.c_int32) else None for t in fn.argtypes]
        st = fn(*args)
        assert st == B.DG_ERR_NULL, name
        assert "NULL" in L.dg_last_error().decode()
    ms = (C.c_double * B.DG_NUM_KERNEL_KINDS)()
    n = (C.c_int64 * B.DG_NUM_KERNEL_KINDS)()
    assert L.dg_profile_read(None, ms, n) == B.DG_ERR_NULL
    assert not L.dg_error_word(None)
    assert not L.dg_done_flags(None)


def test_prefill_host_errors(L):
    m = model()
    cache = B.dg_kv_cache(DUMMY, DUMMY, 1024, 0)
    need = L.dg_prefill_workspace_bytes(C.byref(m), 512)

    def call(m_=m, cache_=cache, ids=DUMMY, n=512, ws=DUMMY, wsb=need):
        return L.dg_prefill_kv(C.byref(m_) if m_ is not None else None, C.byref(cache_) if cache_ is not None
                               else None, ids, n, ws, wsb, None)

    assert call(cache_=None) == B.DG_ERR_NULL
    assert call(ids=None) == B.DG_ERR_NULL
    assert call(ws=None) == B.DG_ERR_NULL
    assert call(m_=None) == B.DG_ERR_NULL
    assert call(n=0) == B.DG_ERR_SHAPE
    assert call(n=1025) == B.DG_ERR_CAPACITY
    assert call(cache_=B.dg_kv_cache(DUMMY, DUMMY, 1020, 0)) == B.DG_ERR_CAPACITY
    assert call(cache_=B.dg_kv_cache(DUMMY, None, 1024, 0)) == B.DG_ERR_NULL
    assert call(cache_=B.dg_kv_cache(DUMMY, DUMMY, 1024, 600)) == B.DG_ERR_CAPACITY
    assert call(wsb=need - 1) == B.DG_ERR_WORKSPACE
    assert call(m_=model(hd=100)) == B.DG_ERR_SHAPE


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        B._need(torch.zeros(4), torch.float32, (4,), "x")


def test_static_init_host_errors(L):
    """dg_canvas_init_static validates like dg_canvas_init and refuses shapes
    whose workspace exceeds the library's static scratch, before any device
    call."""
    def call(a, out=True, m=True):
        h = C.c_void_p()
        st = L.dg_canvas_init_static(C.byref(h) if out else None, C.byref(a.m) if m else None, C.byref(a.smp),
                                     a.caches, a.batch, a.C, C.byref(a.state), None, None, 0, None)
        assert not h.value
        return st, L.dg_last_error().decode()

    a = InitArgs(L)
    assert call(a, out=False)[0] == B.DG_ERR_NULL
    assert call(a, m=False)[0] == B.DG_ERR_NULL
    big = InitArgs(L, batch=16, P=16384, V=65536)
    assert big.ws_bytes > 64 * 2 ** 20
    st, msg = call(big)
    assert st == B.DG_ERR_WORKSPACE and "static scratch" in msg, msg
    a = InitArgs(L, hd=96)
    assert call(a)[0] == B.DG_ERR_SHAPE


def test_deep_model_host_errors(L):
    """Stacked layers / FFN arguments are validated on the host."""
    layers = (B.dg_layer * 3)(*[B.dg_layer(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY) for _ in range(3)])
    a = InitArgs(L); a.m.n_layers = 17; a.m.layers = layers
    expect(L, a, B.DG_ERR_SHAPE, "n_layers")
    a = InitArgs(L); a.m.n_layers = 2
    expect(L, a, B.DG_ERR_NULL, "layers is NULL")
    a = InitArgs(L); a.m.d_ff = 512
    expect(L, a, B.DG_ERR_SHAPE, "FFN needs n_layers")
    a = InitArgs(L); a.m.n_layers = 3; a.m.layers = layers; a.m.d_ff = 300
    expect(L, a, B.DG_ERR_SHAPE, "d_ff")
    bad = (B.dg_layer * 2)(B.dg_layer(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY),
                           B.dg_layer(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY))
    a = InitArgs(L); a.m.n_layers = 2; a.m.layers = bad; a.m.d_ff = 512
    expect(L, a, B.DG_ERR_NULL, "layer 1: an FFN weight")
    a = InitArgs(L, dtype=B.DG_F32); a.m.n_layers = 2; a.m.layers = layers
    expect(L, a, B.DG_ERR_UNSUPPORTED, "bf16 model")
    # the workspace grows with the FFN (activation planes, residual planes)
    m = model()
    m1 = model(); m1.n_layers = 2; m1.layers = layers; m1.d_ff = 8192
    assert L.dg_workspace_bytes(C.byref(m1), 1, 256, 1024) > L.dg_workspace_bytes(C.byref(m), 1, 256, 1024)
    # prefill of a deep model is refused
    cache = B.dg_kv_cache(DUMMY, DUMMY, 1024, 0)
    st = L.dg_prefill_kv(C.byref(m1), C.byref(cache), DUMMY, 16, DUMMY, 1 << 30, None)
    assert st == B.DG_ERR_UNSUPPORTED


def test_fp8_projection_host_errors(L):
    """e4m3 projection arguments are validated on the host."""
    full = lambda: B.dg_layer(*([DUMMY] * 14))
    layers = (B.dg_layer * 2)(full(), full())
    a = InitArgs(L); a.m.n_layers = 2; a.m.layers = layers; a.m.proj_format = 5
    expect(L, a, B.DG_ERR_UNSUPPORTED, "proj_format")
    a = InitArgs(L); a.m.proj_format = B.DG_LM_FP8          # the one top-level layer: no scales there
    expect(L, a, B.DG_ERR_UNSUPPORTED, "layers[]")
    a = InitArgs(L, dtype=B.DG_F32); a.m.n_layers = 2; a.m.layers = layers; a.m.proj_format = B.DG_LM_FP8
    expect(L, a, B.DG_ERR_UNSUPPORTED, "bf16 model")
    no_scale = (B.dg_layer * 2)(full(), B.dg_layer(*([DUMMY] * 8 + [None] + [DUMMY] * 5)))
    a = InitArgs(L); a.m.n_layers = 2; a.m.layers = no_scale; a.m.proj_format = B.DG_LM_FP8
    expect(L, a, B.DG_ERR_NULL, "layer 1: an attention weight scale")
    no_ffn_scale = (B.dg_layer * 2)(full(), B.dg_layer(*([DUMMY] * 12 + [None, DUMMY])))
    a = InitArgs(L); a.m.n_layers = 2; a.m.layers = no_ffn_scale; a.m.d_ff = 512; a.m.proj_format = B.DG_LM_FP8
    expect(L, a, B.DG_ERR_NULL, "layer 1: an FFN weight scale")


def test_expert_host_errors(L):
    """Routed-expert arguments are validated on the host."""
    full = lambda: B.dg_layer(*([DUMMY] * 18))
    layers = (B.dg_layer * 2)(full(), full())

    def moe_args(**kw):
        a = InitArgs(L, **{k: v for k, v in kw.items() if k == "dtype"})
        a.m.n_layers = 2; a.m.layers = layers; a.m.d_ff = 512
        a.m.n_experts = kw.get("E", 16); a.m.top_k = kw.get("k", 2); a.m.d_expert = kw.get("de", 256)
        return a
    expect(L, moe_args(E=300), B.DG_ERR_SHAPE, "n_experts")
    expect(L, moe_args(k=0), B.DG_ERR_SHAPE, "top_k")
    expect(L, moe_args(k=17, E=32), B.DG_ERR_SHAPE, "top_k")
    expect(L, moe_args(k=5, E=4), B.DG_ERR_SHAPE, "top_k")
    expect(L, moe_args(de=100), B.DG_ERR_SHAPE, "d_expert")
    a = moe_args(); a.m.d_ff = 0
    expect(L, a, B.DG_ERR_SHAPE, "shared FFN")
    a = moe_args(); a.m.n_layers = 0; a.m.d_ff = 0
    expect(L, a, B.DG_ERR_UNSUPPORTED, "layers[]")
    no_router = (B.dg_layer * 2)(full(), B.dg_layer(*([DUMMY] * 14 + [None] + [DUMMY] * 3)))
    a = moe_args(); a.m.layers = no_router
    expect(L, a, B.DG_ERR_NULL, "layer 1: an expert weight")
    a = InitArgs(L); a.m.n_experts = -1
    expect(L, a, B.DG_ERR_SHAPE, "n_experts")
    # experts need workspace of their own
    m0 = model(); m0.n_layers = 2; m0.layers = layers; m0.d_ff = 512
    m1 = model(); m1.n_layers = 2; m1.layers = layers; m1.d_ff = 512
    m1.n_experts, m1.top_k, m1.d_expert = 16, 2, 256
    assert L.dg_workspace_bytes(C.byref(m1), 1, 256, 1024) > L.dg_workspace_bytes(C.byref(m0), 1, 256, 1024)
