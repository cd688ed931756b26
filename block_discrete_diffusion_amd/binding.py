"""ctypes binding of libdg.so (the C-ABI declared in include/dg.h).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity and handed over as raw device pointers; every step of
the computation runs in the HIP library.  If the library has not been built
(``python -m block_discrete_diffusion_amd.build``) every entry point raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

DG_OK, DG_ERR_NULL, DG_ERR_SHAPE, DG_ERR_CAPACITY, DG_ERR_STATE, DG_ERR_DEVICE, DG_ERR_UNSUPPORTED, \
    DG_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7
DG_F32, DG_BF16 = 0, 1
DG_LM_NATIVE, DG_LM_FP8 = 0, 1
DG_INIT_RESUME = 1
DG_MAX_BATCH, DG_MAX_CANVAS = 32, 256
DG_NUM_KERNEL_KINDS = 13
KIND_NAMES = ["reset", "prep_rows", "qkv_rope", "attention", "attn_merge", "out_proj", "rowscale_h",
              "lmhead_sampler", "sample_commit", "append", "debug_copy", "ffn", "moe"]

STATUS_NAMES = {0: "DG_OK", -1: "DG_ERR_NULL", -2: "DG_ERR_SHAPE", -3: "DG_ERR_CAPACITY",
                -4: "DG_ERR_STATE", -5: "DG_ERR_DEVICE", -6: "DG_ERR_UNSUPPORTED", -7: "DG_ERR_WORKSPACE"}


class dg_layer(C.Structure):
    _fields_ = [("wq", C.c_void_p), ("wk", C.c_void_p), ("wv", C.c_void_p), ("wo", C.c_void_p),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("wq_scale", C.c_void_p), ("wk_scale", C.c_void_p), ("wv_scale", C.c_void_p),
                ("wo_scale", C.c_void_p), ("w_gate_scale", C.c_void_p), ("w_up_scale", C.c_void_p),
                ("w_down_scale", C.c_void_p), ("w_router", C.c_void_p), ("w_expert_gate", C.c_void_p),
                ("w_expert_up", C.c_void_p), ("w_expert_down", C.c_void_p)]


class dg_model(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("mask_id", C.c_int32),
                ("eos_id", C.c_int32), ("dtype", C.c_int32), ("rope_base", C.c_float),
                ("norm_eps", C.c_float), ("embed", C.c_void_p), ("wq", C.c_void_p), ("wk", C.c_void_p),
                ("wv", C.c_void_p), ("wo", C.c_void_p), ("lm_head", C.c_void_p), ("lm_format", C.c_int32),
                ("lm_scale", C.c_void_p), ("n_layers", C.c_int32), ("d_ff", C.c_int32),
                ("layers", C.POINTER(dg_layer)), ("proj_format", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("d_expert", C.c_int32)]


class dg_kv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int64), ("len", C.c_int64)]


class dg_sampler(C.Structure):
    _fields_ = [("n_steps", C.c_int32), ("adaptive_stop", C.c_int32), ("stop_conf", C.c_float),
                ("commit_rule", C.c_int32), ("commit_conf", C.c_float), ("canvas_fill", C.c_int32),
                ("stop_entropy", C.c_float), ("temperature", C.c_float), ("temperature_end", C.c_float),
                ("seed", C.c_uint64)]


class dg_canvas_state(C.Structure):
    _fields_ = [("ids", C.c_void_p), ("committed", C.c_void_p), ("step", C.c_void_p),
                ("n_steps_done", C.c_void_p), ("n_valid", C.c_void_p), ("done", C.c_void_p)]


class dg_canvas_stats(C.Structure):
    _fields_ = [("n_steps_done", C.c_int32), ("n_valid", C.c_int32)]


class dg_debug(C.Structure):
    _fields_ = [("q", C.c_void_p), ("o", C.c_void_p), ("h", C.c_void_p), ("row_stats", C.c_void_p),
                ("logits", C.c_void_p), ("entropy", C.c_void_p), ("moe_sel", C.c_void_p)]


EXPORTS = [
    "dg_workspace_bytes", "dg_canvas_init", "dg_canvas_init_static", "dg_denoise_step", "dg_run_canvas", "dg_append_canvas_kv",
    "dg_canvas_reset", "dg_canvas_resume", "dg_prefill_workspace_bytes", "dg_prefill_kv", "dg_error_word",
    "dg_kernel_kind_name", "dg_profile_enable", "dg_profile_read", "dg_canvas_destroy", "dg_last_error",
    "dg_run_steps", "dg_append_request_kv", "dg_canvas_admit", "dg_done_flags", "dg_canvas_set_graph",
]

_lib = None


class DGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib() -> C.CDLL:
    """Load libdg.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m block_discrete_diffusion_amd.build")
    L = C.CDLL(LIB_PATH)
    P = C.c_void_p
    L.dg_workspace_bytes.argtypes = [C.POINTER(dg_model), C.c_int32, C.c_int32, C.c_int64]
    L.dg_workspace_bytes.restype = C.c_size_t
    L.dg_canvas_init.argtypes = [C.POINTER(P), C.POINTER(dg_model), C.POINTER(dg_sampler), C.POINTER(dg_kv_cache),
                                 C.c_int32, C.c_int32, C.POINTER(dg_canvas_state), P, P, C.c_uint32, P, C.c_size_t, P]
    L.dg_canvas_init_static.argtypes = [C.POINTER(P), C.POINTER(dg_model), C.POINTER(dg_sampler),
                                        C.POINTER(dg_kv_cache), C.c_int32, C.c_int32, C.POINTER(dg_canvas_state),
                                        P, P, C.c_uint32, P]
    L.dg_denoise_step.argtypes = [P, C.POINTER(dg_debug)]
    L.dg_run_canvas.argtypes = [P, C.POINTER(dg_canvas_stats)]
    L.dg_append_canvas_kv.argtypes = [P]
    L.dg_run_steps.argtypes = [P, C.c_int32, C.c_uint32, C.POINTER(C.c_int32), C.POINTER(C.c_uint32)]
    L.dg_append_request_kv.argtypes = [P, C.c_int32, P, P]
    L.dg_canvas_admit.argtypes = [P, C.c_int32, C.POINTER(dg_kv_cache), P, P]
    L.dg_done_flags.argtypes = [P]
    L.dg_done_flags.restype = C.POINTER(C.c_int32)
    L.dg_canvas_set_graph.argtypes = [P, C.c_int32]
    L.dg_canvas_reset.argtypes = [P, P, P]
    L.dg_canvas_resume.argtypes = [P]
    L.dg_prefill_workspace_bytes.argtypes = [C.POINTER(dg_model), C.c_int32]
    L.dg_prefill_workspace_bytes.restype = C.c_size_t
    L.dg_prefill_kv.argtypes = [C.POINTER(dg_model), C.POINTER(dg_kv_cache), P, C.c_int32, P, C.c_size_t, P]
    L.dg_error_word.argtypes = [P]
    L.dg_error_word.restype = P
    L.dg_kernel_kind_name.argtypes = [C.c_int32]
    L.dg_kernel_kind_name.restype = C.c_char_p
    L.dg_profile_enable.argtypes = [P, C.c_uint32]
    L.dg_profile_read.argtypes = [P, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
    L.dg_canvas_destroy.argtypes = [P]
    L.dg_last_error.argtypes = []
    L.dg_last_error.restype = C.c_char_p
    for name in ("dg_canvas_init", "dg_canvas_init_static", "dg_denoise_step", "dg_run_canvas", "dg_append_canvas_kv", "dg_canvas_reset",
                 "dg_canvas_resume", "dg_prefill_kv", "dg_profile_enable", "dg_profile_read", "dg_canvas_destroy",
                 "dg_run_steps", "dg_append_request_kv", "dg_canvas_admit", "dg_canvas_set_graph"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


_hiprt = None


def _hip() -> C.CDLL:
    """The HIP runtime this process already loaded (same soname as the one
    libdg.so links), for plain copies of library-owned device words."""
    global _hiprt
    if _hiprt is None:
        _hiprt = C.CDLL("libamdhip64.so.7")
        _hiprt.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
        _hiprt.hipMemcpy.restype = C.c_int
    return _hiprt


def _check(status: int):
    if status != DG_OK:
        raise DGError(status, lib().dg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, shape, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------------------------
# model / caches / state as torch tensors
# ----------------------------------------------------------------------------

@dataclass
class Model:
    """Device weights plus the dg_model struct that points at them."""
    V: int
    d: int
    Hq: int
    Hkv: int
    hd: int
    mask_id: int
    eos_id: int
    dtype: int
    rope_base: float
    norm_eps: float
    embed: torch.Tensor
    wq: torch.Tensor
    wk: torch.Tensor
    wv: torch.Tensor
    wo: torch.Tensor
    lm_head: torch.Tensor
    lm_scale: Optional[torch.Tensor] = None    # float32 [V]: lm_head holds e4m3 bytes (uint8 [V, d])
    layers: Optional[list] = None              # per layer dict of wq, wk, wv, wo[, wg, wu, wd] device tensors
    d_ff: int = 0
    proj_fp8: bool = False                     # layer weights are e4m3 bytes (uint8) with <name>_scale rows
    n_experts: int = 0                         # routed experts per layer (layer dicts hold wr, wge, wue, wde)
    top_k: int = 0
    d_expert: int = 0

    @property
    def n_layers(self) -> int:
        return len(self.layers) if self.layers else 1

    @property
    def tdtype(self):
        return torch.bfloat16 if self.dtype == DG_BF16 else torch.float32

    def struct(self) -> dg_model:
        fp8 = self.lm_scale is not None
        for name, shp in (("embed", (self.V, self.d)), ("wq", (self.Hq * self.hd, self.d)),
                          ("wk", (self.Hkv * self.hd, self.d)), ("wv", (self.Hkv * self.hd, self.d)),
                          ("wo", (self.d, self.Hq * self.hd)), ("lm_head", (self.V, self.d))):
            _need(getattr(self, name), torch.uint8 if (fp8 and name == "lm_head") else self.tdtype, shp, name)
        if fp8:
            _need(self.lm_scale, torch.float32, (self.V,), "lm_scale")
        n_layers, arr = 0, None
        if self.layers:
            n_layers = len(self.layers)
            arr = (dg_layer * n_layers)()
            wt = torch.uint8 if self.proj_fp8 else self.tdtype
            for l, Ly in enumerate(self.layers):
                shapes = [("wq", (self.Hq * self.hd, self.d)), ("wk", (self.Hkv * self.hd, self.d)),
                          ("wv", (self.Hkv * self.hd, self.d)), ("wo", (self.d, self.Hq * self.hd))]
                if self.d_ff:
                    shapes += [("wg", (self.d_ff, self.d)), ("wu", (self.d_ff, self.d)), ("wd", (self.d, self.d_ff))]
                for name, shp in shapes:
                    _need(Ly[name], wt, shp, f"layer {l} {name}")
                    if self.proj_fp8:
                        _need(Ly[name + "_scale"], torch.float32, (shp[0],), f"layer {l} {name}_scale")
                sc = (lambda n: _ptr(Ly.get(n + "_scale"))) if self.proj_fp8 else (lambda n: None)
                if self.n_experts:
                    E, de = self.n_experts, self.d_expert
                    for name, shp in (("wr", (E, self.d)), ("wge", (E, de, self.d)), ("wue", (E, de, self.d)),
                                      ("wde", (E, self.d, de))):
                        _need(Ly[name], self.tdtype, shp, f"layer {l} {name}")
                arr[l] = dg_layer(_ptr(Ly["wq"]), _ptr(Ly["wk"]), _ptr(Ly["wv"]), _ptr(Ly["wo"]),
                                  _ptr(Ly.get("wg")), _ptr(Ly.get("wu")), _ptr(Ly.get("wd")),
                                  sc("wq"), sc("wk"), sc("wv"), sc("wo"), sc("wg"), sc("wu"), sc("wd"),
                                  _ptr(Ly.get("wr")), _ptr(Ly.get("wge")), _ptr(Ly.get("wue")), _ptr(Ly.get("wde")))
        self._layer_array = arr                 # the struct points into it: keep it alive
        return dg_model(self.V, self.d, self.Hq, self.Hkv, self.hd, self.mask_id, self.eos_id, self.dtype,
                        self.rope_base, self.norm_eps, _ptr(self.embed), _ptr(self.wq), _ptr(self.wk),
                        _ptr(self.wv), _ptr(self.wo), _ptr(self.lm_head), DG_LM_FP8 if fp8 else DG_LM_NATIVE,
                        _ptr(self.lm_scale), n_layers, self.d_ff, arr,
                        DG_LM_FP8 if self.proj_fp8 else DG_LM_NATIVE, self.n_experts, self.top_k, self.d_expert)


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array (bf16 bit patterns as uint16, or float32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def model_from_inputs(inp, device="cuda") -> Model:
    wl = inp.wl
    dt = wl.dtype
    emb = to_device(inp.embed, dt, device)
    scale = None
    if wl.lm_fp8:
        lm = torch.from_numpy(np.ascontiguousarray(inp.lm_head, dtype=np.uint8)).to(device)
        scale = torch.from_numpy(np.ascontiguousarray(inp.lm_scale, dtype=np.float32)).to(device)
    else:
        lm = emb if wl.tied else to_device(inp.lm_head, dt, device)
    layers = None
    fp8 = getattr(wl, "proj_fp8", False)
    if getattr(inp, "layers", None):
        def dev(k, v):
            if fp8 and k not in ("wr", "wge", "wue", "wde"):   # e4m3 codes and fp32 row scales, as they are
                return torch.from_numpy(np.ascontiguousarray(v)).to(device)
            return to_device(v, dt, device)
        layers = [{k: dev(k, v) for k, v in Ly.items()} for Ly in inp.layers]
    return Model(wl.vocab, wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.mask_id, wl.eos_id,
                 DG_BF16 if dt == "bf16" else DG_F32, wl.rope_base, wl.norm_eps, emb,
                 to_device(inp.wq, dt, device), to_device(inp.wk, dt, device), to_device(inp.wv, dt, device),
                 to_device(inp.wo, dt, device), lm, scale, layers, getattr(wl, "d_ff", 0), fp8,
                 getattr(wl, "n_experts", 0), getattr(wl, "top_k", 0), getattr(wl, "d_expert", 0))


class KVCache:
    """k: [L, Hkv, capacity, hd]; v: [L, Hkv, hd, capacity] (position fastest),
    one plane per layer (L = 1 for a one-layer model)."""

    def __init__(self, model: Model, capacity: int, device="cuda"):
        if capacity % 8:
            capacity += 8 - capacity % 8
        self.capacity = capacity
        L = model.n_layers
        self.k = torch.zeros((L, model.Hkv, capacity, model.hd), dtype=model.tdtype, device=device)
        self.v = torch.zeros((L, model.Hkv, model.hd, capacity), dtype=model.tdtype, device=device)
        self.len = 0

    def fill_prefix(self, K, V, layer: int = 0):
        """K, V: [Hkv, P, hd] device tensors of the model dtype."""
        P = K.shape[1]
        self.k[layer, :, :P, :] = K
        self.v[layer, :, :, :P] = V.transpose(1, 2)
        self.len = P

    def rows(self, start: int, stop: int, layer: int = 0):
        """(K, V) rows [start, stop) of a layer as [Hkv, n, hd]."""
        return self.k[layer, :, start:stop, :], self.v[layer, :, :, start:stop].transpose(1, 2)


class State:
    def __init__(self, B: int, C: int, device="cuda"):
        self.ids = torch.zeros((B, C), dtype=torch.int32, device=device)
        self.committed = torch.zeros((B, C), dtype=torch.uint8, device=device)
        self.step = torch.zeros(B, dtype=torch.int32, device=device)
        self.n_steps_done = torch.zeros(B, dtype=torch.int32, device=device)
        self.n_valid = torch.zeros(B, dtype=torch.int32, device=device)
        self.done = torch.zeros(B, dtype=torch.int32, device=device)

    def struct(self) -> dg_canvas_state:
        return dg_canvas_state(_ptr(self.ids), _ptr(self.committed), _ptr(self.step), _ptr(self.n_steps_done),
                               _ptr(self.n_valid), _ptr(self.done))


# ----------------------------------------------------------------------------
# entry points, same names as the C-ABI
# ----------------------------------------------------------------------------

def dg_workspace_bytes(model: Model, batch: int, canvas_len: int, max_prefix: int) -> int:
    m = model.struct()
    return int(lib().dg_workspace_bytes(C.byref(m), batch, canvas_len, max_prefix))


def dg_prefill_workspace_bytes(model: Model, n: int) -> int:
    m = model.struct()
    return int(lib().dg_prefill_workspace_bytes(C.byref(m), n))


def dg_prefill_kv(model: Model, cache: KVCache, ids: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                  stream=None):
    n = ids.numel()
    _need(ids, torch.int32, (n,), "ids")
    m = model.struct()
    need = int(lib().dg_prefill_workspace_bytes(C.byref(m), n))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=ids.device)
    kc = dg_kv_cache(_ptr(cache.k), _ptr(cache.v), cache.capacity, cache.len)
    _check(lib().dg_prefill_kv(C.byref(m), C.byref(kc), _ptr(ids), n, _ptr(workspace), workspace.numel(),
                               _stream(stream)))
    cache.len = int(kc.len)


class Canvas:
    """A dg_canvas handle with the buffers it points at kept alive."""

    def __init__(self, model: Model, caches: Sequence[KVCache], canvas_len: int, n_steps: int,
                 stop_conf: Optional[float] = None, init_ids: Optional[torch.Tensor] = None,
                 init_committed: Optional[torch.Tensor] = None, state: Optional[State] = None,
                 flags: int = 0, stream=None, device="cuda", commit_conf: Optional[float] = None,
                 fill: int = 0, stop_entropy: Optional[float] = None, static_scratch: bool = False,
                 temperature: Optional[tuple] = None):
        """static_scratch: the handle of dg_canvas_init_static (library-owned
        device scratch, no workspace tensor).  temperature: (T0, T1, seed)
        for temperature sampling with annealing."""
        self.model = model
        self.caches = list(caches)
        B = len(self.caches)
        self.B, self.C = B, canvas_len
        self.state = state or State(B, canvas_len, device)
        self._m = model.struct()
        if stop_conf is not None and stop_entropy is not None:
            raise ValueError("stop_conf and stop_entropy select different adaptive stops; give one")
        adaptive = 1 if stop_conf is not None else (2 if stop_entropy is not None else 0)
        self._smp = dg_sampler(n_steps, adaptive,
                               float(stop_conf) if stop_conf is not None else 0.0,
                               1 if commit_conf is not None else 0,
                               float(commit_conf) if commit_conf is not None else 0.0, int(fill),
                               float(stop_entropy) if stop_entropy is not None else 0.0,
                               float(temperature[0]) if temperature else 0.0,
                               float(temperature[1]) if temperature else 0.0,
                               int(temperature[2]) if temperature else 0)
        self._kc = (dg_kv_cache * B)(*[dg_kv_cache(_ptr(c.k), _ptr(c.v), c.capacity, c.len) for c in self.caches])
        self._slot_kc = [self._kc[b] for b in range(B)]     # the struct each slot's cache length lives in
        self._st = self.state.struct()
        for name, t in (("init_ids", init_ids), ("init_committed", init_committed)):
            if t is not None:
                _need(t, torch.int32 if name == "init_ids" else torch.uint8, (B, canvas_len), name)
        self._init_refs = (init_ids, init_committed)
        self._h = C.c_void_p()
        self.stream = _stream(stream)
        if static_scratch:
            self.workspace = None
            _check(lib().dg_canvas_init_static(C.byref(self._h), C.byref(self._m), C.byref(self._smp), self._kc,
                                               B, canvas_len, C.byref(self._st), _ptr(init_ids),
                                               _ptr(init_committed), flags, self.stream))
            return
        maxp = max(c.capacity for c in self.caches) - canvas_len
        need = int(lib().dg_workspace_bytes(C.byref(self._m), B, canvas_len, max(maxp, 0)))
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        _check(lib().dg_canvas_init(C.byref(self._h), C.byref(self._m), C.byref(self._smp), self._kc, B,
                                    canvas_len, C.byref(self._st), _ptr(init_ids), _ptr(init_committed), flags,
                                    _ptr(self.workspace), self.workspace.numel(), self.stream))

    # -- calls --
    def dg_denoise_step(self, q=None, o=None, h=None, row_stats=None, logits=None, entropy=None, moe_sel=None):
        """Optional float32 stage dumps: q, o [B*C, Hq*hd], h [B*C, d],
        row_stats [B*C, 4], logits [B*C, V], entropy [B*C]; int32 moe_sel
        [n_layers, B*C, top_k] (models with experts)."""
        if any(x is not None for x in (q, o, h, row_stats, logits, entropy, moe_sel)):
            m, M = self.model, self.B * self.C
            for name, t, shp in (("q", q, (M, m.Hq * m.hd)), ("o", o, (M, m.Hq * m.hd)), ("h", h, (M, m.d)),
                                 ("row_stats", row_stats, (M, 4)), ("logits", logits, (M, m.V)),
                                 ("entropy", entropy, (M,))):
                if t is not None:
                    _need(t, torch.float32, shp, name)
            if moe_sel is not None:
                _need(moe_sel, torch.int32, (m.n_layers, M, m.top_k), "moe_sel")
            dbg = dg_debug(_ptr(q), _ptr(o), _ptr(h), _ptr(row_stats), _ptr(logits), _ptr(entropy), _ptr(moe_sel))
            _check(lib().dg_denoise_step(self._h, C.byref(dbg)))
        else:
            _check(lib().dg_denoise_step(self._h, None))

    def dg_run_canvas(self, stats: bool = True):
        if not stats:
            _check(lib().dg_run_canvas(self._h, None))
            return None
        out = (dg_canvas_stats * self.B)()
        _check(lib().dg_run_canvas(self._h, out))
        return [(o.n_steps_done, o.n_valid) for o in out]

    def dg_append_canvas_kv(self):
        _check(lib().dg_append_canvas_kv(self._h))
        for c, kc in zip(self.caches, self._slot_kc):
            c.len = int(kc.len)

    # -- continuous batching --
    def dg_run_steps(self, max_steps: int, stop_mask: int = 0):
        """Returns (steps enqueued, mask of done requests)."""
        n = C.c_int32()
        m = C.c_uint32()
        _check(lib().dg_run_steps(self._h, max_steps, stop_mask, C.byref(n), C.byref(m)))
        return int(n.value), int(m.value)

    def _slot_rows(self, init_ids, init_committed):
        if init_ids is not None:
            _need(init_ids, torch.int32, (self.C,), "init_ids")
        if init_committed is not None:
            _need(init_committed, torch.uint8, (self.C,), "init_committed")

    def dg_append_request_kv(self, b: int, init_ids=None, init_committed=None):
        self._slot_rows(init_ids, init_committed)
        _check(lib().dg_append_request_kv(self._h, b, _ptr(init_ids), _ptr(init_committed)))
        self.caches[b].len = int(self._slot_kc[b].len)

    def dg_canvas_admit(self, b: int, cache: "KVCache", init_ids=None, init_committed=None):
        self._slot_rows(init_ids, init_committed)
        if not 0 <= b < self.B:
            raise ValueError(f"slot {b} outside [0, {self.B})")
        kc = dg_kv_cache(_ptr(cache.k), _ptr(cache.v), cache.capacity, cache.len)
        _check(lib().dg_canvas_admit(self._h, b, C.byref(kc), _ptr(init_ids), _ptr(init_committed)))
        self._slot_kc[b] = kc
        self.caches[b] = cache

    def dg_canvas_set_graph(self, on: bool):
        """Steps as one recorded HIP graph launch each (on) or as separate
        kernel launches (off)."""
        _check(lib().dg_canvas_set_graph(self._h, 1 if on else 0))

    def dg_done_flags(self):
        """The pinned done flags as a list (None for a handle without them)."""
        p = lib().dg_done_flags(self._h)
        if not p:
            return None
        return [int(p[b]) for b in range(self.B)]

    def dg_canvas_reset(self, init_ids=None, init_committed=None):
        self._init_refs = (init_ids, init_committed)
        _check(lib().dg_canvas_reset(self._h, _ptr(init_ids), _ptr(init_committed)))

    def dg_canvas_resume(self):
        """After writing the state buffers between steps."""
        _check(lib().dg_canvas_resume(self._h))

    def set_cache_len(self, b: int, length: int):
        """Caller-side cache length, read by the next dg_canvas_reset."""
        self._slot_kc[b].len = length
        self.caches[b].len = length

    def error_word(self) -> torch.Tensor:
        """Device error counters: [appends skipped (canvas not done), invalid ids,
        vocabulary-head groups over the open-row bound (not computed), unused]
        (a copy; waits for the device)."""
        p = lib().dg_error_word(self._h)
        out = torch.empty(4, dtype=torch.int32)
        torch.cuda.synchronize()
        st = _hip().hipMemcpy(C.c_void_p(out.data_ptr()), C.c_void_p(p), C.c_size_t(16), 2)   # device to host
        if st != 0:
            raise RuntimeError(f"hipMemcpy of the error word failed ({st})")
        return out

    def dg_profile_enable(self, kinds=None):
        """kinds: iterable of kernel-kind names (None = all, [] = off)."""
        if kinds is None:
            mask = (1 << DG_NUM_KERNEL_KINDS) - 1
        else:
            mask = 0
            for k in kinds:
                mask |= 1 << KIND_NAMES.index(k)
        _check(lib().dg_profile_enable(self._h, mask))

    def dg_profile_read(self) -> dict:
        ms = (C.c_double * DG_NUM_KERNEL_KINDS)()
        n = (C.c_int64 * DG_NUM_KERNEL_KINDS)()
        _check(lib().dg_profile_read(self._h, ms, n))
        return {lib().dg_kernel_kind_name(k).decode(): (ms[k], n[k]) for k in range(DG_NUM_KERNEL_KINDS) if n[k]}

    def dg_canvas_destroy(self):
        if self._h:
            _check(lib().dg_canvas_destroy(self._h))
            self._h = C.c_void_p()

    def __del__(self):
        try:
            if self._h and _lib is not None:
                _lib.dg_canvas_destroy(self._h)
        except Exception:
            pass


# ----------------------------------------------------------------------------
# materialising a synthetic workload on the device
# ----------------------------------------------------------------------------

@dataclass
class DeviceWorkload:
    model: Model
    caches: List[KVCache]
    init_ids: torch.Tensor
    init_committed: torch.Tensor
    extra_capacity: int = 0


def device_workload(inp, extra_canvases: int = 0, device="cuda") -> DeviceWorkload:
    """Copy synthetic inputs to the device.  Caches get room for the canvas
    plus ``extra_canvases`` more appended canvases.  Prompt workloads are
    prefilled through dg_prefill_kv."""
    wl = inp.wl
    model = model_from_inputs(inp, device)
    caches = []
    for b in range(wl.batch):
        P = inp.prefix_len[b]
        cap = P + wl.canvas * (1 + max(extra_canvases, wl.n_canvases - 1 + extra_canvases))
        kc = KVCache(model, cap, device)
        if inp.prompt is not None:
            dg_prefill_kv(model, kc, torch.from_numpy(inp.prompt).to(device))
        else:
            pk, pv = inp.prefix_k[b], inp.prefix_v[b]
            if not isinstance(pk, (list, tuple)):
                pk, pv = [pk], [pv]
            for l, (k, v) in enumerate(zip(pk, pv)):
                kc.fill_prefix(to_device(k, wl.dtype, device), to_device(v, wl.dtype, device), layer=l)
        caches.append(kc)
    return DeviceWorkload(model, caches, torch.from_numpy(inp.init_ids).to(device),
                          torch.from_numpy(inp.init_committed).to(device))
