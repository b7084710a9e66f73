"""ctypes binding of ``libsmd.so`` (the C ABI in include/sparse_moe_decode.h).

Argument marshalling only: every entry point forwards torch tensors' device
pointers and the current HIP stream to the library, where all of the decode
arithmetic runs. Import fails loudly when the library has not been built;
there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m sparse_moe_decode_amd.build` (hipcc, gfx950)")
_lib = C.CDLL(LIB_PATH)

E0_OK = 0
E0_ERR_ARG = -1
E0_ERR_SHAPE = -2
E0_ERR_ALIGN = -3
E0_ERR_HIP = -4
E0_ERR_RANGE = -5
E0_ERR_SYNC = -6
E0_ERR_STATE = -7
E0_ERR_IO = -8
ROUTER_SOFTMAX_TOPK = 0
ROUTER_SIGMOID_GROUP = 1

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_f = C.c_float


class e0_spec(C.Structure):
    _fields_ = [("d_model", _i32), ("n_experts", _i32), ("top_k", _i32), ("inter", _i32),
                ("shared_inter", _i32), ("head_hidden", _i32), ("group", _i32),
                ("lora_rank", _i32), ("lora_alpha", _f), ("router_kind", _i32),
                ("norm_topk", _i32), ("n_groups", _i32), ("topk_groups", _i32),
                ("route_scale", _f), ("rms_eps", _f), ("quant", _i32)]


class e0_q4(C.Structure):
    _fields_ = [("q", _p), ("s", _p), ("b", _p)]


class e0_experts(C.Structure):
    _fields_ = [("gate", e0_q4), ("up", e0_q4), ("down", e0_q4), ("stride_q", _i64),
                ("stride_s", _i64), ("count", _i32)]


class e0_lora(C.Structure):
    _fields_ = [("a", _p), ("b", _p)]


class e0_shared(C.Structure):
    _fields_ = [("gate", e0_q4), ("up", e0_q4), ("down", e0_q4), ("lgate", e0_lora),
                ("lup", e0_lora), ("ldown", e0_lora)]


class e0_head(C.Structure):
    _fields_ = [("fc1", _p), ("fc2", _p), ("lin", _p), ("bias", _p)]


class e0_layer(C.Structure):
    _fields_ = [("experts", e0_experts), ("slot_of", _p), ("shared", e0_shared),
                ("router", _p), ("router_bias", _p), ("head", e0_head), ("attn", _p)]


class e0_state(C.Structure):
    _fields_ = [("route_idx", _p), ("route_w", _p), ("exec_idx", _p), ("exec_w", _p),
                ("head_logits", _p), ("x_trace", _p), ("n_layers", _i32)]


_lib.e0_create.argtypes = [C.POINTER(e0_spec), _i32, C.POINTER(_p)]
_lib.e0_destroy.argtypes = [_p]
_lib.e0_last_error.restype = C.c_char_p
_lib.e0_device_status.argtypes = [_p, _p]
_lib.moe_int4_decode.argtypes = [_p, C.POINTER(e0_experts), _p, C.POINTER(e0_shared), _p, _p,
                                 _p, _i32, _p, _p]
_lib.moe_int4_decode_static.argtypes = [C.POINTER(e0_spec), C.POINTER(e0_experts), _p,
                                        C.POINTER(e0_shared), _p, _p, _p, _i32, _p, _p, _p]
_lib.lora_delta.argtypes = [_p, _p, _p, _i32, _i32, _i32, _f, _p, _p, _i32, _p]
_lib.prerouter_forward.argtypes = [_p, C.POINTER(e0_head), _p, _p, _p, _i32, _p, _p, _p, _p]
_lib.e0_model_create.argtypes = [_p, C.POINTER(e0_layer), _i32, C.POINTER(_p)]
_lib.e0_model_destroy.argtypes = [_p]
_lib.e0_model_set_path.argtypes = [_p, _i32]
_lib.e0_model_set_grid.argtypes = [_p, _i32]
_lib.e0_model_set_roles.argtypes = [_p, _i32, _i32]
_lib.e0_model_set_trace.argtypes = [_p, _p]
_lib.e0_model_trace_shape.argtypes = [_p, C.POINTER(_i32), C.POINTER(_i32), C.POINTER(_i32)]
_lib.layer_step.argtypes = [_p, _p, _i32, _i32, C.POINTER(e0_state), _i32, _p, _p]
_lib.e0_bundle_bytes.argtypes = [C.POINTER(e0_spec)]
_lib.e0_bundle_bytes.restype = _i64
_lib.e0_stager_create.argtypes = [_p, _p, _i32, _i32, _p, _p, _p, C.POINTER(_p)]
_lib.e0_stager_destroy.argtypes = [_p]
_lib.stage_experts.argtypes = [_p, _i32, _p, _p, _p, _p]
_lib.stage_experts_n.argtypes = [_p, _i32, _i32, _p, _p, _p, _p]
_lib.stage_layer.argtypes = [_p, _p, _p, _p, _p]
_lib.e0_cache_create.argtypes = [_p, _p, _i32, _i32, _p, _p, _p, _p, C.POINTER(_p)]
_lib.e0_cache_destroy.argtypes = [_p]
_lib.e0_cache_copies.argtypes = [_p]
_lib.e0_cache_copies.restype = _i64
_lib.stage_experts_cached.argtypes = [_p, _i32, _i32, _p, _i32, _p, _p]
_lib.e0_store_open.argtypes = [C.POINTER(C.c_char_p), _i32, _i32, _i64, _i32, _i32, C.POINTER(_p)]
_lib.e0_store_close.argtypes = [_p]
_lib.e0_store_read.argtypes = [_p, _i32, C.POINTER(_i32), _i32, C.POINTER(_p), C.POINTER(_i64)]
_lib.e0_store_wait.argtypes = [_p, _i64, C.POINTER(C.c_double), C.POINTER(C.c_double)]
_lib.e0_store_bytes.argtypes = [_p]
_lib.e0_store_bytes.restype = _i64
_lib.e0_stager_copies.argtypes = [_p, C.POINTER(C.c_int64)]

EXPORTS = ["e0_create", "e0_destroy", "e0_last_error", "e0_device_status", "moe_int4_decode",
           "lora_delta", "prerouter_forward", "e0_model_create", "e0_model_destroy",
           "layer_step", "e0_bundle_bytes", "e0_stager_create", "e0_stager_destroy",
           "stage_experts", "stage_experts_n", "e0_stager_copies", "stage_layer",
           "e0_cache_create", "e0_cache_destroy", "e0_cache_copies", "stage_experts_cached",
           "e0_store_open", "e0_store_close", "e0_store_read", "e0_store_wait", "e0_store_bytes", "e0_model_set_path", "e0_model_set_grid", "e0_model_set_trace", "e0_model_trace_shape",
           "e0_model_set_roles", "moe_int4_decode_static"]

PATH_AUTO, PATH_PHASES, PATH_PERSISTENT, PATH_FLOW, PATH_CHAIN = 0, 1, 2, 3, 4
QUANT_SYMMETRIC, QUANT_AFFINE = 0, 1


class E0Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _check(rc):
    if rc != E0_OK:
        raise E0Error(rc, _lib.e0_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_contiguous(), "tensors passed to the library must be contiguous"
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_spec(dims: dict) -> e0_spec:
    s = e0_spec()
    s.d_model, s.n_experts, s.top_k = dims["d"], dims["E"], dims["K"]
    s.inter, s.shared_inter, s.head_hidden = dims["I"], dims.get("Is", 0), dims.get("P", 0)
    s.group, s.lora_rank, s.lora_alpha = dims["G"], dims.get("r", 0), dims.get("alpha", 0.0)
    s.router_kind = dims.get("router_kind", ROUTER_SOFTMAX_TOPK)
    s.norm_topk = int(dims.get("norm_topk", 1))
    s.n_groups, s.topk_groups = dims.get("n_groups", 1), dims.get("topk_groups", 1)
    s.route_scale, s.rms_eps = dims.get("route_scale", 1.0), dims.get("eps", 1e-6)
    s.quant = int(dims.get("quant", QUANT_SYMMETRIC))
    return s


def bundle_bytes_of(dims: dict) -> int:
    """e0_bundle_bytes of a tier (host only, no context)."""
    return int(_lib.e0_bundle_bytes(C.byref(make_spec(dims))))


class Context:
    """e0_ctx: one tier's dimensions plus the shared device scratch."""

    def __init__(self, dims: dict, max_tokens: int = 64):
        self.dims = dict(dims)
        self.spec = make_spec(dims)
        h = _p()
        _check(_lib.e0_create(C.byref(self.spec), max_tokens, C.byref(h)))
        self.handle = h.value
        self.max_tokens = max_tokens

    def close(self):
        # at interpreter exit the module globals may already be gone
        if getattr(self, "handle", None) and _lib is not None:
            _lib.e0_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    def bundle_bytes(self) -> int:
        return int(_lib.e0_bundle_bytes(C.byref(self.spec)))


def device_status(ctx: Context, stream=None) -> int:
    """Synchronise and return the device error flags as an E0 code (0 = none)."""
    return _lib.e0_device_status(ctx.handle, _stream(stream))


def experts_struct(pool: dict, count: int, stride_q: int = 0, stride_s: int = 0) -> e0_experts:
    """pool: tensors gate_q/gate_s/up_q/up_s/down_q/down_s (or ints = device addresses)."""
    ex = e0_experts()
    for name in ("gate", "up", "down"):
        setattr(ex, name, e0_q4(_ptr(pool[f"{name}_q"]), _ptr(pool[f"{name}_s"]),
                                _ptr(pool.get(f"{name}_b"))))
    ex.stride_q, ex.stride_s, ex.count = stride_q, stride_s, count
    return ex


def shared_struct(sh: dict | None) -> e0_shared | None:
    if sh is None:
        return None
    s = e0_shared()
    for name in ("gate", "up", "down"):
        setattr(s, name, e0_q4(_ptr(sh[f"{name}_q"]), _ptr(sh[f"{name}_s"]),
                               _ptr(sh.get(f"{name}_b"))))
    for lname, key in (("lgate", "gate"), ("lup", "up"), ("ldown", "down")):
        setattr(s, lname, e0_lora(_ptr(sh.get(f"a_{key}")), _ptr(sh.get(f"b_{key}"))))
    return s


def head_struct(hd: dict | None) -> e0_head:
    h = e0_head()
    if hd is not None:
        h.fc1, h.fc2, h.lin = _ptr(hd["fc1"]), _ptr(hd["fc2"]), _ptr(hd["lin"])
        h.bias = _ptr(hd.get("bias"))
    return h


def moe_int4_decode(ctx: Context, routed: dict, x, idx, w, y=None, shared: dict | None = None,
                    slot_of=None, count=None, stride: int = 0, stream=None):
    """y[b] = sum_k w[b,k] E_{idx[b,k]}(x[b]) + S(x[b]); x fp16 [B, d] on the GPU.
    stride: bytes between pool entries (0 = stacked per projection)."""
    B = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    ex = experts_struct(routed, count if count is not None else ctx.dims["E"], stride, stride)
    sh = shared_struct(shared)
    _check(_lib.moe_int4_decode(ctx.handle, C.byref(ex), _ptr(slot_of),
                                C.byref(sh) if sh is not None else None, _ptr(x), _ptr(idx),
                                _ptr(w), B, _ptr(y), _stream(stream)))
    return y


def moe_int4_decode_static(dims: dict, routed: dict, x, idx, w, y=None,
                           shared: dict | None = None, slot_of=None, count=None, stride: int = 0,
                           flags=None, stream=None):
    """moe_int4_decode on the library's static workspace (no context, no
    allocation inside the call). flags: device int32 [4] receiving error bits."""
    B = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    spec = make_spec(dims)
    ex = experts_struct(routed, count if count is not None else dims["E"], stride, stride)
    sh = shared_struct(shared)
    _check(_lib.moe_int4_decode_static(C.byref(spec), C.byref(ex), _ptr(slot_of),
                                       C.byref(sh) if sh is not None else None, _ptr(x),
                                       _ptr(idx), _ptr(w), B, _ptr(y), _ptr(flags),
                                       _stream(stream)))
    return y


def lora_delta(ctx: Context, A, Bm, scale: float, x, y_acc, stream=None):
    """y_acc[b] += scale * Bm (A x[b]); A [r, in] fp16, Bm [out, r] fp16, y_acc fp32."""
    r, in_dim = A.shape
    out_dim = Bm.shape[0]
    _check(_lib.lora_delta(ctx.handle, _ptr(A), _ptr(Bm), in_dim, out_dim, r, float(scale),
                           _ptr(x), _ptr(y_acc), x.shape[0], _stream(stream)))
    return y_acc


def prerouter_forward(ctx: Context, head: dict, x, cur_idx, prev_idx=None, logits=None,
                      out_idx=None, out_w=None, stream=None):
    """Head logits on [x; onehot(cur); onehot(prev)] and the routed top-K."""
    B = x.shape[0]
    K, E = ctx.dims["K"], ctx.dims["E"]
    dev = x.device
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_w is None:
        out_w = torch.empty((B, K), dtype=torch.float32, device=dev)
    hs = head_struct(head)
    _check(_lib.prerouter_forward(ctx.handle, C.byref(hs), _ptr(x), _ptr(cur_idx),
                                  _ptr(prev_idx), B, _ptr(logits), _ptr(out_idx), _ptr(out_w),
                                  _stream(stream)))
    return out_idx, out_w


class Model:
    """e0_model: the per-layer weight table of a stack."""

    def __init__(self, ctx: Context, layers: list[dict]):
        arr = (e0_layer * len(layers))()
        for i, L in enumerate(layers):
            arr[i].experts = experts_struct(L["routed"], L.get("count", ctx.dims["E"]),
                                            L.get("stride_q", 0), L.get("stride_s", 0))
            arr[i].slot_of = _ptr(L.get("slot_of"))
            sh = shared_struct(L.get("shared"))
            if sh is not None:
                arr[i].shared = sh
            arr[i].router = _ptr(L.get("router"))
            arr[i].router_bias = _ptr(L.get("router_bias"))
            arr[i].head = head_struct(L.get("head"))
            arr[i].attn = _ptr(L.get("attn"))
        h = _p()
        _check(_lib.e0_model_create(ctx.handle, arr, len(layers), C.byref(h)))
        self.handle = h.value
        self.ctx = ctx
        self.n_layers = len(layers)
        self._keep = layers

    def enable_trace(self, on: bool = True):
        """Allocate (or drop) the phase-trace buffer; returns it ([grid, L + 1, points])."""
        if not on:
            _check(_lib.e0_model_set_trace(self.handle, None))
            self.trace = None
            return None
        g, rows, pts = _i32(), _i32(), _i32()
        _check(_lib.e0_model_trace_shape(self.handle, C.byref(g), C.byref(rows), C.byref(pts)))
        self.trace = torch.zeros((max(g.value, 1), rows.value, pts.value), dtype=torch.int64,
                                 device="cuda")
        _check(_lib.e0_model_set_trace(self.handle, self.trace.data_ptr()))
        return self.trace

    def set_path(self, path: int):
        """PATH_AUTO, PATH_PHASES (one kernel per phase), PATH_CHAIN (the
        persistent kernel with a layer-ahead weight slot), PATH_PERSISTENT (the
        whole-token kernel) or PATH_FLOW (the wave-specialised streaming kernel)."""
        _check(_lib.e0_model_set_path(self.handle, path))

    def set_grid(self, grid: int):
        """Workgroups of the persistent kernels (0 = one per compute unit)."""
        _check(_lib.e0_model_set_grid(self.handle, grid))

    def set_roles(self, n_gate_up: int, n_down: int):
        """Split of the streaming kernel's grid (0, 0 = automatic)."""
        _check(_lib.e0_model_set_roles(self.handle, n_gate_up, n_down))

    def close(self):
        # at interpreter exit the module globals may already be gone
        if getattr(self, "handle", None) and _lib is not None:
            _lib.e0_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


class State:
    """Device-resident decode state (e0_state) for a stack of L layers."""

    def __init__(self, dims: dict, n_layers: int, device="cuda", head_logits: bool = True,
                 x_trace: bool = True):
        K, E = dims["K"], dims["E"]
        self.route_idx = torch.zeros((2, n_layers, K), dtype=torch.int32, device=device)
        self.route_w = torch.zeros((2, n_layers, K), dtype=torch.float32, device=device)
        self.exec_idx = torch.zeros((2, n_layers, K), dtype=torch.int32, device=device)
        self.exec_w = torch.zeros((2, n_layers, K), dtype=torch.float32, device=device)
        self.head_logits = (torch.zeros((n_layers, E), dtype=torch.float32, device=device)
                            if head_logits else None)
        self.x_trace = (torch.zeros((n_layers, dims["d"]), dtype=torch.float16, device=device)
                        if x_trace else None)
        self.n_layers = n_layers
        self.dims = dims
        self.struct = e0_state(_ptr(self.route_idx), _ptr(self.route_w), _ptr(self.exec_idx),
                               _ptr(self.exec_w), _ptr(self.head_logits), _ptr(self.x_trace),
                               n_layers)


def layer_step(ctx: Context, model: Model, layer_begin: int, layer_end: int, state: State,
               token: int, h, stream=None):
    """One token through layers [layer_begin, layer_end); h fp16 [n+1, d] (h[0] input)."""
    if state.n_layers != model.n_layers:
        raise ValueError(f"state sized for {state.n_layers} layers, the model has {model.n_layers}")
    n = layer_end - layer_begin
    d = ctx.dims["d"]
    if (h.dtype != torch.float16 or not h.is_cuda or not h.is_contiguous()
            or h.numel() < (n + 1) * d):
        raise ValueError("h must be a contiguous fp16 CUDA tensor of at least "
                         f"{n + 1} x {d} elements")
    _check(_lib.layer_step(ctx.handle, model.handle, layer_begin, layer_end,
                           C.byref(state.struct), token, _ptr(h), _stream(stream)))
    return h


def bundle_parts(dims: dict) -> list[tuple[str, int]]:
    """(name, bytes) of one expert bundle in the ABI's order: gate q, up q,
    down q (packed u32), gate s, up s, down s (16-bit), then for the affine
    codec gate b, up b, down b (bf16)."""
    qb = dims["I"] * dims["d"] // 2
    sb = dims["I"] * dims["d"] // dims["G"] * 2
    parts = [("gate_q", qb), ("up_q", qb), ("down_q", qb), ("gate_s", sb), ("up_s", sb),
             ("down_s", sb)]
    if dims.get("quant", 0) == 1:
        parts += [("gate_b", sb), ("up_b", sb), ("down_b", sb)]
    return parts


def pack_bundles(pool: dict, dims: dict):
    """Host numpy pool (gate_q [n, I, d/8] u32 ... down_s [n, d, I/G] fp16) ->
    uint8 [n, bundle] in the ABI's bundle layout (a byte re-arrangement)."""
    import numpy as np
    n = pool["gate_q"].shape[0]
    cols = [np.ascontiguousarray(pool[name]).view(np.uint8).reshape(n, nb)
            for name, nb in bundle_parts(dims)]
    return np.concatenate(cols, axis=1)


def bundle_view(base: int, dims: dict) -> dict:
    """Device addresses of the six parts of bundle 0 of a bundle pool at
    `base`; with stride = bundle bytes this is an e0_experts view."""
    view, off = {}, 0
    for name, nb in bundle_parts(dims):
        view[name] = base + off
        off += nb
    return view


class Stager:
    """e0_stager: pinned host pool of expert bundles -> HBM slot pool."""

    def __init__(self, ctx: Context, host_pool, n_layers: int, n_slots: int, hbm_slots,
                 slot_of, slot_expert):
        h = _p()
        _check(_lib.e0_stager_create(ctx.handle, _ptr(host_pool), n_layers, n_slots,
                                     _ptr(hbm_slots), _ptr(slot_of), _ptr(slot_expert),
                                     C.byref(h)))
        self.handle = h.value
        self.ctx = ctx
        self._keep = (host_pool, hbm_slots, slot_of, slot_expert)

    def copies(self) -> int:
        """Bundles copied since creation (synchronises the device)."""
        n = C.c_int64(0)
        _check(_lib.e0_stager_copies(self.handle, C.byref(n)))
        return int(n.value)

    def close(self):
        # at interpreter exit the module globals may already be gone
        if getattr(self, "handle", None) and _lib is not None:
            _lib.e0_stager_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def _event_handle(ev, stream):
    """hipEvent_t of `ev` (a torch.cuda.Event or a raw handle). torch creates
    the underlying event on its first record(), and a wait on an event never
    created is a no-op; so a fresh torch event is recorded once on `stream`
    to create it before the library records it."""
    if ev is None:
        return None
    if not hasattr(ev, "cuda_event"):
        return ev
    if not ev.cuda_event:
        ev.record(stream if stream is not None else torch.cuda.current_stream())
    handle = ev.cuda_event
    assert handle, "event has no HIP handle"
    return handle


def stage_experts(stager: Stager, layer: int, new_idx, in_use_idx=None, side_stream=None,
                  done_event=None):
    ev = _event_handle(done_event, side_stream)
    _check(_lib.stage_experts(stager.handle, layer, _ptr(new_idx), _ptr(in_use_idx),
                              _stream(side_stream), ev))


class HotCache:
    """e0_cache: pinned host pool of expert bundles -> one cross-layer HBM
    pool of n_entries bundles with least-recently-staged replacement."""

    def __init__(self, ctx: Context, host_pool, n_layers: int, n_entries: int, hbm_cache,
                 slot_of, owner, stamp):
        h = _p()
        _check(_lib.e0_cache_create(ctx.handle, _ptr(host_pool), n_layers, n_entries,
                                    _ptr(hbm_cache), _ptr(slot_of), _ptr(owner), _ptr(stamp),
                                    C.byref(h)))
        self.handle = h.value
        self.ctx = ctx
        self.n_entries = n_entries
        self._keep = (host_pool, hbm_cache, slot_of, owner, stamp)

    def copies(self) -> int:
        return int(_lib.e0_cache_copies(self.handle))

    def close(self):
        if self.handle:
            _lib.e0_cache_destroy(self.handle)
            self.handle = None


def stage_experts_cached(cache: HotCache, layer: int, n_layers: int, new_idx, tick: int,
                         side_stream=None, done_event=None):
    """Stage the sets new_idx (device int32 [n_layers, K]) of layers
    [layer, layer + n_layers) for token `tick` through the hot cache."""
    ev = _event_handle(done_event, side_stream)
    _check(_lib.stage_experts_cached(cache.handle, layer, n_layers, _ptr(new_idx), tick,
                                     _stream(side_stream), ev))


class Store:
    """e0_store: per-layer stacked bundle files read by byte range on a pool
    of host I/O threads (host only, no GPU)."""

    def __init__(self, paths: list[str], n_experts: int, bundle_bytes: int, io_threads: int = 16,
                 direct: bool = True):
        arr = (C.c_char_p * len(paths))(*[p.encode() for p in paths])
        h = _p()
        _check(_lib.e0_store_open(arr, len(paths), n_experts, bundle_bytes, io_threads,
                                  1 if direct else 0, C.byref(h)))
        self.handle = h.value

    def read(self, layer: int, ids, dst_ptrs) -> int:
        """Queue reads of bundles `ids` of `layer` into host addresses
        dst_ptrs; returns a ticket."""
        n = len(ids)
        ida = (_i32 * max(n, 1))(*[int(i) for i in ids])
        dsa = (_p * max(n, 1))(*[int(p) for p in dst_ptrs])
        tk = _i64()
        _check(_lib.e0_store_read(self.handle, layer, ida, n, dsa, C.byref(tk)))
        return tk.value

    def wait(self, ticket: int):
        """Block until the ticket's reads are done; returns (blocked_s, read_s)."""
        b, r = C.c_double(), C.c_double()
        _check(_lib.e0_store_wait(self.handle, ticket, C.byref(b), C.byref(r)))
        return b.value, r.value

    def bytes_read(self) -> int:
        return int(_lib.e0_store_bytes(self.handle))

    def close(self):
        if self.handle:
            _lib.e0_store_close(self.handle)
            self.handle = None


def stage_layer(ctx: Context, host_layer, hbm_layer, stream=None, done_event=None):
    """Copy one layer's E expert bundles (pinned host uint8 [E * bundle]) into
    hbm_layer (device, same size) as one DMA transfer on `stream`."""
    ev = _event_handle(done_event, stream)
    _check(_lib.stage_layer(ctx.handle, _ptr(host_layer), _ptr(hbm_layer), _stream(stream), ev))


def stage_experts_n(stager: Stager, layer: int, n_layers: int, new_idx, in_use_idx=None,
                    side_stream=None, done_event=None):
    """stage_experts for layers [layer, layer + n_layers); new_idx / in_use_idx
    device int32 [n_layers, K] (contiguous rows)."""
    ev = _event_handle(done_event, side_stream)
    _check(_lib.stage_experts_n(stager.handle, layer, n_layers, _ptr(new_idx), _ptr(in_use_idx),
                                _stream(side_stream), ev))
