"""ctypes wrapper of the scalar oracle (``oracle.cpp``).

Test infrastructure: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` only. Every array crossing this wrapper is
a numpy array; nothing here touches a GPU.

Page tags used in docstrings:
  [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
       Trained Routing Prediction" (arXiv 2609.18063).
  [CB] "Edge0 streams a 35B MoE off SSD. I counted the bytes it can't stream."
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ROUTER_SOFTMAX_TOPK = 0
ROUTER_SIGMOID_GROUP = 1


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` with g++ (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i = C.c_int
_d = C.c_double
_i64 = C.c_int64


class OrcMoe(C.Structure):
    _fields_ = [("d", _i), ("E", _i), ("K", _i), ("I", _i), ("Is", _i), ("group", _i),
                ("r", _i), ("alpha", _d),
                ("gate_q", _p), ("up_q", _p), ("down_q", _p),
                ("gate_s", _p), ("up_s", _p), ("down_s", _p),
                ("sh_gate_q", _p), ("sh_up_q", _p), ("sh_down_q", _p),
                ("sh_gate_s", _p), ("sh_up_s", _p), ("sh_down_s", _p),
                ("a_gate", _p), ("b_gate", _p), ("a_up", _p), ("b_up", _p),
                ("a_down", _p), ("b_down", _p)]


class OrcRouting(C.Structure):
    _fields_ = [("kind", _i), ("E", _i), ("K", _i), ("norm_topk", _i), ("n_groups", _i),
                ("topk_groups", _i), ("scale", _d)]


class OrcLayer(C.Structure):
    _fields_ = [("moe", OrcMoe), ("rt", OrcRouting), ("eps", _d), ("attn", _p),
                ("router", _p), ("router_bias", _p), ("fc1", _p), ("fc2", _p), ("lin", _p),
                ("head_bias", _p), ("P", _i)]


def _declare(lib):
    lib.orc_f16_round.argtypes = [_p, _i64, _p]
    lib.orc_f16_decode.argtypes = [_p, _i64, _p]
    lib.orc_q4_dequant.argtypes = [_p, _p, _i, _i, _i, _p]
    lib.orc_q4_matvec.argtypes = [_p, _p, _i, _i, _i, _p, _p]
    lib.orc_silu.argtypes = [_p, _i64, _p]
    lib.orc_gelu_erf.argtypes = [_p, _i64, _p]
    lib.orc_rmsnorm.argtypes = [_p, _i, _d, _p]
    lib.orc_topk.argtypes = [_p, _p, _i, _i, _p]
    lib.orc_topk.restype = _i
    lib.orc_route_softmax_topk.argtypes = [_p, _i, _i, _i, _p, _p]
    lib.orc_route_softmax_topk.restype = _i
    lib.orc_route_sigmoid_group.argtypes = [_p, _p, _i, _i, _i, _i, _d, _p, _p, _p, _p]
    lib.orc_route_sigmoid_group.restype = _i
    lib.orc_expert.argtypes = [_p] * 6 + [_i, _i, _i, _p, _p]
    lib.orc_lora_delta.argtypes = [_p, _p, _i, _i, _i, _d, _p, _p]
    lib.orc_shared_expert.argtypes = [_p] * 12 + [_i, _i, _i, _i, _d, _p, _p]
    lib.orc_moe_decode.argtypes = [C.POINTER(OrcMoe), _p, _p, _p, _p]
    lib.orc_moe_decode.restype = _i
    lib.orc_head_logits.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _i, _p]
    lib.orc_head_logits.restype = _i
    lib.orc_route.argtypes = [C.POINTER(OrcRouting), _p, _p, _p, _p]
    lib.orc_route.restype = _i
    lib.orc_layer_step.argtypes = [C.POINTER(OrcLayer)] + [_p] * 13
    lib.orc_layer_step.restype = _i
    lib.orc_slot_policy.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p]
    lib.orc_slot_policy.restype = _i


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_p)


def _c(a, dtype):
    """Contiguous array of `dtype` (a copy only when needed)."""
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _f64(a):
    return _c(a, np.float64)


def _u16(a):
    """fp16 data travels as raw uint16 bit patterns."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


def _u32(a):
    return _c(a, np.uint32)


def _i32(a):
    return _c(a, np.int32)


# ---------------------------------------------------------------- helpers --

def f16_round(x) -> np.ndarray:
    """Round float64 values to binary16 (round-to-nearest-even); returns uint16 bits."""
    x = _f64(x)
    out = np.empty(x.shape, np.uint16)
    load().orc_f16_round(_ptr(x), x.size, _ptr(out))
    return out


def f16_decode(bits) -> np.ndarray:
    b = _u16(bits)
    out = np.empty(b.shape, np.float64)
    load().orc_f16_decode(_ptr(b), b.size, _ptr(out))
    return out


def q4_dequant(q, s, rows, cols, group) -> np.ndarray:
    q, s = _u32(q), _u16(s)
    out = np.empty((rows, cols), np.float64)
    load().orc_q4_dequant(_ptr(q), _ptr(s), rows, cols, group, _ptr(out))
    return out


def q4_matvec(q, s, rows, cols, group, x) -> np.ndarray:
    q, s, x = _u32(q), _u16(s), _f64(x)
    y = np.empty(rows, np.float64)
    load().orc_q4_matvec(_ptr(q), _ptr(s), rows, cols, group, _ptr(x), _ptr(y))
    return y


def silu(z) -> np.ndarray:
    z = _f64(z)
    out = np.empty(z.shape, np.float64)
    load().orc_silu(_ptr(z), z.size, _ptr(out))
    return out


def gelu_erf(z) -> np.ndarray:
    z = _f64(z)
    out = np.empty(z.shape, np.float64)
    load().orc_gelu_erf(_ptr(z), z.size, _ptr(out))
    return out


def rmsnorm(h, eps=1e-6) -> np.ndarray:
    h = _f64(h)
    out = np.empty(h.shape, np.float64)
    load().orc_rmsnorm(_ptr(h), h.size, eps, _ptr(out))
    return out


def topk(score, k, allowed=None) -> np.ndarray:
    score = _f64(score)
    al = None if allowed is None else np.ascontiguousarray(allowed, dtype=np.uint8)
    idx = np.full(k, -1, np.int32)
    n = load().orc_topk(_ptr(score), _ptr(al), score.size, k, _ptr(idx))
    return idx[:n]


def route_softmax_topk(logits, K, norm=True):
    """Softmax-top-K routing [MW App. A]; returns (idx int32[K], w float64[K])."""
    lg = _f64(logits)
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    rc = load().orc_route_softmax_topk(_ptr(lg), lg.size, K, int(norm), _ptr(idx), _ptr(w))
    if rc != 0:
        raise ValueError("bad softmax-top-K arguments")
    return idx, w


def route_sigmoid_group(logits, bias, K, n_groups, topk_groups, scale, return_scores=False):
    """Sigmoid-group routing [MW App. A]; returns (idx, w[, biased scores, group scores])."""
    lg = _f64(logits)
    E = lg.size
    b = None if bias is None else _f64(bias)
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    sel = np.empty(E, np.float64)
    grp = np.empty(n_groups, np.float64)
    rc = load().orc_route_sigmoid_group(_ptr(lg), _ptr(b), E, K, n_groups, topk_groups,
                                        float(scale), _ptr(idx), _ptr(w), _ptr(sel), _ptr(grp))
    if rc != 0:
        raise ValueError("bad sigmoid-group arguments")
    if return_scores:
        return idx, w, sel, grp
    return idx, w


def expert(gate_q, gate_s, up_q, up_s, down_q, down_s, d, I, group, x) -> np.ndarray:
    arrs = [_u32(gate_q), _u16(gate_s), _u32(up_q), _u16(up_s), _u32(down_q), _u16(down_s)]
    x = _f64(x)
    y = np.empty(d, np.float64)
    load().orc_expert(*[_ptr(a) for a in arrs], d, I, group, _ptr(x), _ptr(y))
    return y


def lora_delta(A, B, in_dim, out_dim, r, scale, x, y_acc=None) -> np.ndarray:
    A, B, x = _u16(A), _u16(B), _f64(x)
    y = np.zeros(out_dim, np.float64) if y_acc is None else np.array(y_acc, np.float64)
    load().orc_lora_delta(_ptr(A), _ptr(B), in_dim, out_dim, r, float(scale), _ptr(x), _ptr(y))
    return y


def shared_expert(sh: dict, d, Is, group, r, alpha, x) -> np.ndarray:
    """sh: dict with gate_q/gate_s/up_q/up_s/down_q/down_s and optional a_*/b_* LoRA."""
    keys_q = ["gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"]
    keys_l = ["a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down"]
    arrs = [(_u32 if k.endswith("_q") else _u16)(sh[k]) for k in keys_q]
    arrs += [_u16(sh.get(k)) for k in keys_l]
    x = _f64(x)
    y = np.empty(d, np.float64)
    load().orc_shared_expert(*[_ptr(a) for a in arrs], d, Is, group, r, float(alpha),
                             _ptr(x), _ptr(y))
    return y


class _Keep:
    """Holds the numpy arrays a ctypes struct points into."""

    def __init__(self):
        self.refs = []

    def __call__(self, a):
        if a is not None:
            self.refs.append(a)
        return _ptr(a)


def _moe_struct(dims: dict, routed: dict, shared: dict | None, keep: _Keep) -> OrcMoe:
    m = OrcMoe()
    m.d, m.E, m.K = dims["d"], dims["E"], dims["K"]
    m.I, m.Is, m.group = dims["I"], dims["Is"], dims["G"]
    m.r, m.alpha = dims.get("r", 0), float(dims.get("alpha", 0.0))
    m.gate_q, m.up_q, m.down_q = (keep(_u32(routed[k])) for k in ("gate_q", "up_q", "down_q"))
    m.gate_s, m.up_s, m.down_s = (keep(_u16(routed[k])) for k in ("gate_s", "up_s", "down_s"))
    if shared is not None:
        m.sh_gate_q, m.sh_up_q, m.sh_down_q = (keep(_u32(shared[k]))
                                               for k in ("gate_q", "up_q", "down_q"))
        m.sh_gate_s, m.sh_up_s, m.sh_down_s = (keep(_u16(shared[k]))
                                               for k in ("gate_s", "up_s", "down_s"))
        for k in ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down"):
            setattr(m, k, keep(_u16(shared.get(k))))
    return m


def moe_decode(dims: dict, routed: dict, shared: dict | None, x16, idx, w) -> np.ndarray:
    """Routed combine + shared expert for one token; x16 fp16 bits or float16 array."""
    keep = _Keep()
    m = _moe_struct(dims, routed, shared, keep)
    x16, idx, w = _u16(x16), _i32(idx), _f64(w)
    y = np.empty(dims["d"], np.float64)
    rc = load().orc_moe_decode(C.byref(m), _ptr(x16), _ptr(idx), _ptr(w), _ptr(y))
    if rc != 0:
        raise ValueError("expert id out of range")
    return y


def head_logits(fc1, fc2, lin, d, E, P, K, x16, cur, prev, form=1) -> np.ndarray:
    """Prerouter head logits [MW §3.2 Head]; prev None means the all-zero one-hot."""
    fc1, fc2, lin, x16 = _u16(fc1), _u16(fc2), _u16(lin), _u16(x16)
    cur, prev = _i32(cur), _i32(prev)
    out = np.empty(E, np.float64)
    rc = load().orc_head_logits(_ptr(fc1), _ptr(fc2), _ptr(lin), d, E, P, K, _ptr(x16),
                                _ptr(cur), _ptr(prev), form, _ptr(out))
    if rc != 0:
        raise ValueError("bad or repeated expert id in head input")
    return out


def routing_struct(dims: dict) -> OrcRouting:
    rt = OrcRouting()
    rt.kind = dims.get("router_kind", ROUTER_SOFTMAX_TOPK)
    rt.E, rt.K = dims["E"], dims["K"]
    rt.norm_topk = int(dims.get("norm_topk", 1))
    rt.n_groups = dims.get("n_groups", 1)
    rt.topk_groups = dims.get("topk_groups", 1)
    rt.scale = float(dims.get("route_scale", 1.0))
    return rt


def route(dims: dict, logits, bias=None):
    """Route logits with the tier's routing family; returns (idx, w)."""
    rt = routing_struct(dims)
    lg = _f64(logits)
    b = _c(bias, np.float32)
    idx = np.empty(dims["K"], np.int32)
    w = np.empty(dims["K"], np.float64)
    if load().orc_route(C.byref(rt), _ptr(lg), _ptr(b), _ptr(idx), _ptr(w)) != 0:
        raise ValueError("routing failed")
    return idx, w


def route_scores(dims: dict, logits, bias=None) -> np.ndarray:
    """The score the tier's routing ranks experts by [MW App. A]: the logit for
    softmax-top-K (softmax is monotone in it), the biased sigmoid sigma + bias
    for sigmoid-group."""
    lg = np.asarray(logits, np.float64)
    if dims.get("router_kind", ROUTER_SOFTMAX_TOPK) == ROUTER_SOFTMAX_TOPK:
        return lg.copy()
    sig = 1.0 / (1.0 + np.exp(-lg))
    return sig + (0.0 if bias is None else np.asarray(bias, np.float64))


def route_set_weights(dims: dict, logits, idx, bias=None) -> np.ndarray:
    """Routing weights [MW App. A] that the tier's routing function gives a
    set `idx` (in its order), whichever set that is: softmax-top-K takes the
    softmax over all E logits and, when normalised, renormalises it over the
    set; sigmoid-group takes scale * sigma / (sum of sigma over the set +
    1e-20) on the raw sigmoid (the selection bias only ranks). Used to hold a
    set that differs from the oracle's own under a near tie to the weights
    the routing function assigns that set."""
    lg = np.asarray(logits, np.float64)
    idx = np.asarray(idx, np.int64)
    if dims.get("router_kind", ROUTER_SOFTMAX_TOPK) == ROUTER_SOFTMAX_TOPK:
        g = np.exp(lg - lg.max())
        g = g / g.sum()
        sel = g[idx]
        return sel / sel.sum() if dims.get("norm_topk", 1) else sel
    sig = 1.0 / (1.0 + np.exp(-lg))
    sel = sig[idx]
    return float(dims.get("route_scale", 1.0)) * sel / (sel.sum() + 1e-20)


class LayerOracle:
    """One MoE layer for the oracle: weights are held as numpy arrays.

    ``layer`` keys: routed (dict), shared (dict or None), attn, router,
    router_bias, head (dict fc1/fc2/lin/bias or None).
    """

    def __init__(self, dims: dict, layer: dict):
        self.dims = dims
        self.keep = _Keep()
        k = self.keep
        L = OrcLayer()
        L.moe = _moe_struct(dims, layer["routed"], layer.get("shared"), k)
        L.rt = routing_struct(dims)
        L.eps = float(dims.get("eps", 1e-6))
        L.attn = k(_u16(layer.get("attn")))
        L.router = k(_u16(layer.get("router")))
        L.router_bias = k(_c(layer.get("router_bias"), np.float32))
        head = layer.get("head")
        if head is not None:
            L.fc1, L.fc2, L.lin = (k(_u16(head[n])) for n in ("fc1", "fc2", "lin"))
            L.head_bias = k(_c(head.get("bias"), np.float32))
            L.P = dims["P"]
        self.L = L
        self.has_head = head is not None
        self.has_router = layer.get("router") is not None

    def step(self, h16, route_idx=None, route_w=None, prev_idx=None, x16=None) -> dict:
        """One layer-step. x16 (optional) replaces the oracle's own fp16 rounding of
        the normed activation (out['x16'] is always the oracle's own)."""
        d, E, K = self.dims["d"], self.dims["E"], self.dims["K"]
        h16 = _u16(h16)
        xin = _u16(x16)
        ri = _i32(route_idx) if route_idx is not None else np.zeros(K, np.int32)
        rw = _c(route_w, np.float32) if route_w is not None else np.zeros(K, np.float32)
        pv = _i32(prev_idx)
        out = dict(h_out=np.empty(d, np.float64), x16=np.empty(d, np.uint16),
                   exec_idx=np.empty(K, np.int32), exec_w=np.empty(K, np.float64),
                   router_logits=np.full(E, np.nan), head_logits=np.full(E, np.nan),
                   pred_idx=np.full(K, -1, np.int32), pred_w=np.full(K, np.nan))
        rc = load().orc_layer_step(C.byref(self.L), _ptr(h16), _ptr(xin), _ptr(ri), _ptr(rw),
                                   _ptr(pv),
                                   _ptr(out["h_out"]), _ptr(out["x16"]), _ptr(out["exec_idx"]),
                                   _ptr(out["exec_w"]), _ptr(out["router_logits"]),
                                   _ptr(out["head_logits"]), _ptr(out["pred_idx"]),
                                   _ptr(out["pred_w"]))
        if rc != 0:
            raise ValueError(f"oracle layer step failed ({rc})")
        return out


def slot_policy(E, n_slots, K, slot_of, slot_expert, in_use, nxt):
    """Staged slot policy (see oracle.cpp); mutates slot_of / slot_expert in place.

    Returns the list of (expert, slot) copies.
    """
    assert slot_of.dtype == np.int32 and slot_expert.dtype == np.int32
    iu = _i32(in_use)
    nx = _i32(nxt)
    ce = np.empty(K, np.int32)
    cs = np.empty(K, np.int32)
    n = load().orc_slot_policy(E, n_slots, K, _ptr(slot_of), _ptr(slot_expert), _ptr(iu),
                               _ptr(nx), _ptr(ce), _ptr(cs))
    if n < 0:
        raise ValueError("slot pool overflow or bad id")
    return list(zip(ce[:n].tolist(), cs[:n].tolist()))


def cache_policy(E, C, slot_of, owner, stamp, layer0, new_sets, tick):
    """Cross-layer hot-expert cache of C bundles in HBM ([MW] §3.1 Executor
    paths, "hot": LRU-resident hot experts; Table 1: a shared LRU of expert
    bundles across layers; "Inside Edge0-35B", The Streaming Subsystem: a hit
    skips the read from the slower tier). The pages give no replacement
    detail beyond LRU; this is the reading used:

      * slot_of int32 [L, E]: cache entry of (layer, expert), or -1;
        owner int32 [C]: layer * E + expert held by an entry, or -1 (empty);
        stamp int32 [C]: the last tick at which the entry was staged for a
        set (-1: never). All three are mutated in place.
      * staging the sets of layers layer0 .. layer0 + len(new_sets) - 1 at
        tick T (the sets of token T): every id already cached is a hit and
        its entry's stamp becomes T; the misses, in ascending (layer, id)
        order, take the entries that are empty or were last staged before
        T - 1 (the running token T - 1 and the sets already staged for T
        keep theirs), least recently staged first, ties to the lower entry
        index. The previous owner of a taken entry loses it.

    Returns the copies as (layer - layer0, expert, entry), in miss order.
    Raises ValueError on an id outside [0, E) or when too few entries are
    free (nothing is changed then beyond the hit stamps)."""
    sets = [np.asarray(s).astype(np.int64).ravel() for s in new_sets]
    for s in sets:
        if np.any(s < 0) or np.any(s >= E):
            raise ValueError("expert id out of range")
    misses = []
    for i, s in enumerate(sets):
        l = layer0 + i
        for e in sorted(set(int(v) for v in s)):
            c = int(slot_of[l, e])
            if c >= 0:
                stamp[c] = tick
            else:
                misses.append((l, e))
    free = [c for c in range(C) if owner[c] < 0 or stamp[c] < tick - 1]
    free.sort(key=lambda c: (int(stamp[c]), c))
    if len(free) < len(misses):
        raise ValueError("cache too small for the staged sets")
    copies = []
    for (l, e), c in zip(misses, free):
        if owner[c] >= 0:
            slot_of[owner[c] // E, owner[c] % E] = -1
        owner[c] = l * E + e
        slot_of[l, e] = c
        stamp[c] = tick
        copies.append((l - layer0, e, c))
    return copies


# --------------------------------------------------------------- affine int4
# The pages' own codec ([MW] §3.1: "int4 affine group-64", each projection
# with its scales and biases; bf16 scales and biases in the MLX layout):
# unsigned nibbles, w = s q + b. Plain numpy in fp64, written from that
# definition; it shares nothing with the symmetric C++ path above.

def bf16_decode(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: sign, 8-bit biased exponent,
    7-bit fraction (subnormals at exponent 0)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    expo = (b >> 7) & 0xFF
    frac = b & 0x7F
    normal = np.ldexp((128 + frac).astype(np.float64), (expo - 134).astype(np.int64))
    sub = np.ldexp(frac.astype(np.float64), -133)
    val = np.where(expo == 0, sub, normal)
    val = np.where(expo == 255, np.where(frac == 0, np.inf, np.nan), val)
    return sign * val


def q4_affine_dequant(q, s_bits, b_bits, rows, cols, group) -> np.ndarray:
    """fp64 [rows, cols]: element i of row o is the unsigned nibble at bits
    4 (i % 8) of word i / 8 of the row; w = s[o][i / G] * nibble + b[o][i / G]."""
    words = np.asarray(q, np.uint32).reshape(rows, cols // 8).astype(np.int64)
    nib = np.empty((rows, cols), np.float64)
    for j in range(8):
        nib[:, j::8] = (words >> (4 * j)) & 0xF
    s = bf16_decode(s_bits).reshape(rows, cols // group)
    b = bf16_decode(b_bits).reshape(rows, cols // group)
    g = np.arange(cols) // group
    return s[:, g] * nib + b[:, g]


def _silu64(z):
    return z / (1.0 + np.exp(-z))


def expert_affine(mats: dict, d, I, group, x) -> np.ndarray:
    """down(silu(gate x) * up x) of one affine expert ([MW] §3.1 Math
    contract); mats holds gate_q/_s/_b [I, ...], up_*, down_* [d, ...]."""
    Wg = q4_affine_dequant(mats["gate_q"], mats["gate_s"], mats["gate_b"], I, d, group)
    Wu = q4_affine_dequant(mats["up_q"], mats["up_s"], mats["up_b"], I, d, group)
    Wd = q4_affine_dequant(mats["down_q"], mats["down_s"], mats["down_b"], d, I, group)
    return Wd @ (_silu64(Wg @ x) * (Wu @ x))


def moe_decode_affine(dims: dict, routed: dict, shared: dict | None, x16, idx, w) -> np.ndarray:
    """sum_k w_k E_idx[k](x) + S(x) with affine experts; S carries the
    unmerged LoRA deltas (alpha / r) B (A v) on its gate, up and down ([MW]
    §3.3). x16: fp16 activations."""
    d, I, G = dims["d"], dims["I"], dims["G"]
    x = np.asarray(x16, np.float16).astype(np.float64)
    y = np.zeros(d)
    names = ("gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b", "down_q", "down_s", "down_b")
    for k, e in enumerate(np.asarray(idx).ravel()):
        mats = {n: routed[n][int(e)] for n in names}
        y += float(w[k]) * expert_affine(mats, d, I, G, x)
    if shared is not None:
        Is, r = dims["Is"], dims.get("r", 0)
        Wg = q4_affine_dequant(shared["gate_q"], shared["gate_s"], shared["gate_b"], Is, d, G)
        Wu = q4_affine_dequant(shared["up_q"], shared["up_s"], shared["up_b"], Is, d, G)
        Wd = q4_affine_dequant(shared["down_q"], shared["down_s"], shared["down_b"], d, Is, G)
        g, u = Wg @ x, Wu @ x
        lora = r > 0 and shared.get("a_gate") is not None
        f = lambda a: np.asarray(a, np.float16).astype(np.float64)
        c = dims.get("alpha", 0.0) / r if r else 0.0
        if lora:
            g = g + c * (f(shared["b_gate"]) @ (f(shared["a_gate"]) @ x))
            u = u + c * (f(shared["b_up"]) @ (f(shared["a_up"]) @ x))
        h = _silu64(g) * u
        ys = Wd @ h
        if lora:
            ys = ys + c * (f(shared["b_down"]) @ (f(shared["a_down"]) @ h))
        y += ys
    return y


class LayerOracleAffine:
    """One layer-step with affine routed and shared experts, same interface
    and outputs as LayerOracle.step. The codec changes only the experts'
    weights ([MW] §3.1), so the step is the same sequence: h_attn = h + attn
    stand-in, x = fp16(rmsnorm(h_attn)), routing from the layer's router
    (or the consumed prediction), h_out = h_attn + moe_decode_affine(x), and
    the head's logits and top-K on x (the helpers above)."""

    def __init__(self, dims: dict, layer: dict):
        self.dims = dims
        self.layer = layer
        self.has_head = layer.get("head") is not None
        self.has_router = layer.get("router") is not None

    def step(self, h16, route_idx=None, route_w=None, prev_idx=None, x16=None) -> dict:
        dm, lw = self.dims, self.layer
        d, E, K = dm["d"], dm["E"], dm["K"]
        ha = f16_decode(h16)
        if lw.get("attn") is not None:
            ha = ha + f16_decode(lw["attn"])
        own = f16_round(rmsnorm(ha, float(dm.get("eps", 1e-6))))
        x = own if x16 is None else _u16(x16)
        out = dict(x16=own, router_logits=np.full(E, np.nan), head_logits=np.full(E, np.nan),
                   pred_idx=np.full(K, -1, np.int32), pred_w=np.full(K, np.nan))
        if self.has_router:
            lg = f16_decode(lw["router"]).reshape(E, d) @ f16_decode(x)
            out["router_logits"] = lg
            idx, w = route(dm, lg, lw.get("router_bias"))
        else:
            idx = np.asarray(route_idx, np.int32).copy()
            w = np.asarray(route_w, np.float32).astype(np.float64)
        out["exec_idx"], out["exec_w"] = idx, w
        xf = f16_decode(x).astype(np.float16)
        out["h_out"] = ha + moe_decode_affine(dm, lw["routed"], lw.get("shared"), xf, idx, w)
        if self.has_head:
            hd = lw["head"]
            lg = head_logits(hd["fc1"], hd["fc2"], hd["lin"], d, E, dm["P"], K, x, idx, prev_idx)
            out["head_logits"] = lg
            out["pred_idx"], out["pred_w"] = route(dm, lg, hd.get("bias"))
        return out
