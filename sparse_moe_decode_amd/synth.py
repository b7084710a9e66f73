"""Seeded synthetic inputs shaped like the two tiers of the streaming-MoE decode step.

This module only draws random numbers and lays them out as bytes. It holds no
step of the decode arithmetic (no GEMV, norm, routing or activation), so both
the HIP path and the CPU oracle can take their inputs from it.

Shapes and distributions follow the method's two published tiers ("The Other
Half of the Memory Wall", §3.1 and §3.2; the byte audit "I counted the bytes
it can't stream", MoESpec listing):

* int4 weights: random 32-bit words, i.e. eight independent uniform nibbles,
  read as two's-complement values in [-8, 7]; fp16 group scales drawn as
  |N(0, 0.02)| + 1e-3.
* fp16 dense weights (head, router) ~ N(0, 0.02); LoRA A, B ~ N(0, 0.01).
* hidden / activation vectors ~ N(0, 1) in fp16.
* routing: random K-subsets, or a Markov chain where each id of the previous
  set is kept with probability 0.7 and the rest is refilled uniformly from the
  other ids; routing weights are Dirichlet(1, ..., 1) draws.

All arrays are numpy; fp16 data is returned as ``np.float16``.
"""

from __future__ import annotations

import numpy as np

ROUTER_SOFTMAX_TOPK = 0
ROUTER_SIGMOID_GROUP = 1

# Tier dimensions. d = d_model, E = experts, K = top-K, I / Is = routed /
# shared intermediate, P = head hidden width, G = quant group, r / alpha = LoRA.
TIERS = {
    "tiny": dict(d=64, E=8, K=2, I=32, Is=32, P=16, G=32, r=4, alpha=8.0,
                 router_kind=ROUTER_SOFTMAX_TOPK, norm_topk=1, n_groups=1, topk_groups=1,
                 route_scale=1.0, eps=1e-6),
    "8b": dict(d=1536, E=128, K=8, I=512, Is=512, P=512, G=64, r=16, alpha=32.0,
               router_kind=ROUTER_SIGMOID_GROUP, norm_topk=1, n_groups=8, topk_groups=4,
               route_scale=2.5, eps=1e-6),
    "35b": dict(d=2048, E=256, K=4, I=512, Is=512, P=512, G=64, r=16, alpha=32.0,
                router_kind=ROUTER_SOFTMAX_TOPK, norm_topk=1, n_groups=1, topk_groups=1,
                route_scale=1.0, eps=1e-6),
}

# Layer roles of the full stacks: which layers own a prerouter head and which
# layers are routed by their own router (the rest consume a prediction).
# 35B: heads on layers 6..38, predictions consumed on 7..38, so layers 0..6 and
# 39 run their router. 8B: heads on 7..22, consumers 8..23.
STACKS = {
    "35b": dict(n_layers=40, head_layers=tuple(range(6, 39)),
                consumer_layers=tuple(range(7, 39))),
    "8b": dict(n_layers=24, head_layers=tuple(range(7, 23)),
               consumer_layers=tuple(range(8, 24))),
}


def dims(tier: str, **over) -> dict:
    d = dict(TIERS[tier])
    d.update(over)
    return d


def stack_roles(tier: str) -> list[dict]:
    """Per-layer roles: {'head': bool, 'router': bool}."""
    s = STACKS[tier]
    heads, cons = set(s["head_layers"]), set(s["consumer_layers"])
    return [dict(head=l in heads, router=l not in cons) for l in range(s["n_layers"])]


def rng_for(seed: int, *path: int) -> np.random.Generator:
    """Independent generator (SFC64 bit stream) for a (seed, layer, ...) path."""
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, *path])))


# ------------------------------------------------------------ primitives --

def random_words(rng, shape) -> np.ndarray:
    """uint32 words with eight independent uniform nibbles each."""
    n = int(np.prod(shape))
    raw = rng.bit_generator.random_raw((n + 1) // 2).view(np.uint32)
    return (raw if raw.size == n else raw[:n].copy()).reshape(shape)


def fold_min_code(words: np.ndarray) -> np.ndarray:
    """In place: every nibble holding code 0b1000 (-8) becomes 0.

    Uniform nibbles read as two's complement have mean -0.5; after the fold
    the codes are symmetric in [-7, 7] with mean 0. A nibble is 0b1000 when
    its top bit is set and its low three bits are zero; adding 0b0111 to the
    low three bits sets bit 3 exactly when they are non-zero (no carry leaves
    the nibble), which gives a per-nibble test with whole-word operations.
    """
    lo = np.bitwise_and(words, np.uint32(0x77777777))
    np.add(lo, np.uint32(0x77777777), out=lo)
    np.bitwise_and(lo, np.uint32(0x88888888), out=lo)       # bit 3 set: low bits != 0
    np.bitwise_xor(lo, np.uint32(0x88888888), out=lo)       # bit 3 set: low bits == 0
    np.bitwise_and(lo, words, out=lo)                       # ... and top bit set
    np.bitwise_xor(words, lo, out=words)                    # clear it: 0b1000 -> 0
    return words


def group_scales(rng, shape) -> np.ndarray:
    return (np.abs(rng.normal(0.0, 0.02, size=shape)) + 1e-3).astype(np.float16)


def f16_normal(rng, shape, std=1.0) -> np.ndarray:
    return rng.normal(0.0, std, size=shape).astype(np.float16)


def q4_matrix(rng, rows, cols, G, lead=(), zero_mean=False):
    """Packed int4 matrix: (uint32 [*lead, rows, cols/8], fp16 [*lead, rows, cols/G]).

    zero_mean folds the -8 code to 0 (see fold_min_code)."""
    assert cols % 8 == 0 and cols % G == 0
    q = random_words(rng, (*lead, rows, cols // 8))
    if zero_mean:
        fold_min_code(q)
    return q, group_scales(rng, (*lead, rows, cols // G))


def bf16_bits(x) -> np.ndarray:
    """fp32 values -> bfloat16 bit patterns (round to nearest, ties to even)."""
    f = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def q4_matrix_affine(rng, rows, cols, G, lead=()):
    """Affine int4 matrix: (uint32 [*lead, rows, cols/8] of unsigned nibbles,
    bf16 scales and bf16 biases [*lead, rows, cols/G] as uint16 bits). The
    biases sit near -7.5 scales, so the weights s q + b are about zero-mean."""
    assert cols % 8 == 0 and cols % G == 0
    q = random_words(rng, (*lead, rows, cols // 8))
    shape = (*lead, rows, cols // G)
    s = np.abs(rng.normal(0.0, 0.02, size=shape)) + 1e-3
    b = -7.5 * s + rng.normal(0.0, 0.002, size=shape)
    return q, bf16_bits(s), bf16_bits(b)


def _q4(rng, rows, cols, G, lead, zero_mean, affine):
    if affine:
        return q4_matrix_affine(rng, rows, cols, G, lead)
    return (*q4_matrix(rng, rows, cols, G, lead, zero_mean), None)


# ----------------------------------------------------------- layer parts --

def routed_pool(rng, dm: dict, n: int | None = None, zero_mean: bool = False) -> dict:
    """n experts (default E) stacked: gate/up [n, I, d/8], down [n, d, I/8].
    With dm["quant"] == 1 (the affine codec) the scales are bf16 bits and
    gate_b / up_b / down_b hold the bf16 biases."""
    n = dm["E"] if n is None else n
    d, I, G = dm["d"], dm["I"], dm["G"]
    af = dm.get("quant", 0) == 1
    gq, gs, gb = _q4(rng, I, d, G, (n,), zero_mean, af)
    uq, us, ub = _q4(rng, I, d, G, (n,), zero_mean, af)
    dq, ds, db = _q4(rng, d, I, G, (n,), zero_mean, af)
    out = dict(gate_q=gq, gate_s=gs, up_q=uq, up_s=us, down_q=dq, down_s=ds)
    if af:
        out.update(gate_b=gb, up_b=ub, down_b=db)
    return out


def shared_expert(rng, dm: dict, lora: bool = True, zero_mean: bool = False) -> dict:
    d, Is, G, r = dm["d"], dm["Is"], dm["G"], dm["r"]
    af = dm.get("quant", 0) == 1
    gq, gs, gb = _q4(rng, Is, d, G, (), zero_mean, af)
    uq, us, ub = _q4(rng, Is, d, G, (), zero_mean, af)
    dq, ds, db = _q4(rng, d, Is, G, (), zero_mean, af)
    out = dict(gate_q=gq, gate_s=gs, up_q=uq, up_s=us, down_q=dq, down_s=ds)
    if af:
        out.update(gate_b=gb, up_b=ub, down_b=db)
    if lora and r > 0:
        out.update(a_gate=f16_normal(rng, (r, d), 0.01), b_gate=f16_normal(rng, (Is, r), 0.01),
                   a_up=f16_normal(rng, (r, d), 0.01), b_up=f16_normal(rng, (Is, r), 0.01),
                   a_down=f16_normal(rng, (r, Is), 0.01), b_down=f16_normal(rng, (d, r), 0.01))
    return out


def head(rng, dm: dict) -> dict:
    """Prerouter head weights: fc1 [P, d+2E], fc2 [E, P], lin [E, d+2E] ~ N(0, 0.02)."""
    d, E, P = dm["d"], dm["E"], dm["P"]
    F = d + 2 * E
    out = dict(fc1=f16_normal(rng, (P, F), 0.02), fc2=f16_normal(rng, (E, P), 0.02),
               lin=f16_normal(rng, (E, F), 0.02))
    if dm["router_kind"] == ROUTER_SIGMOID_GROUP:
        out["bias"] = rng.normal(0.0, 0.02, size=E).astype(np.float32)
    return out


def router(rng, dm: dict):
    """fp16 router [E, d] ~ N(0, 0.02) and (sigmoid-group) fp32 bias ~ N(0, 0.02)."""
    W = f16_normal(rng, (dm["E"], dm["d"]), 0.02)
    b = (rng.normal(0.0, 0.02, size=dm["E"]).astype(np.float32)
         if dm["router_kind"] == ROUTER_SIGMOID_GROUP else None)
    return W, b


def layer(seed: int, l: int, dm: dict, role: dict, lora: bool = True,
          zero_mean: bool = False) -> dict:
    """All weights of layer l of a stack (or of a single layer with l = 0).

    zero_mean=True draws zero-mean int4 codes; the stacked workloads use it so
    the residual stream does not drift through the layers (uniform codes have
    mean -0.5, which RMSNorm feeds back as a growing common mode)."""
    rng = rng_for(seed, l)
    out = dict(routed=routed_pool(rng, dm, zero_mean=zero_mean),
               shared=shared_expert(rng, dm, lora, zero_mean=zero_mean),
               attn=f16_normal(rng, dm["d"], 1.0), router=None, router_bias=None, head=None)
    rrng = rng_for(seed, l, 1)
    if role.get("router"):
        out["router"], out["router_bias"] = router(rrng, dm)
    if role.get("head"):
        out["head"] = head(rng_for(seed, l, 2), dm)
    return out


# --------------------------------------------------------------- routing --

def random_set(rng, E: int, K: int) -> np.ndarray:
    return rng.choice(E, size=K, replace=False).astype(np.int32)


def random_weights(rng, K: int) -> np.ndarray:
    return rng.dirichlet(np.ones(K)).astype(np.float32)


def markov_sets(rng, E: int, K: int, steps: int, keep: float = 0.7) -> np.ndarray:
    """[steps, K] routing sets; each id of the previous set survives with prob `keep`."""
    out = np.empty((steps, K), np.int32)
    cur = random_set(rng, E, K)
    out[0] = cur
    for t in range(1, steps):
        kept = cur[rng.random(K) < keep]
        pool = np.setdiff1d(np.arange(E), cur)
        fresh = rng.choice(pool, size=K - kept.size, replace=False)
        cur = np.concatenate([kept, fresh]).astype(np.int32)
        rng.shuffle(cur)
        out[t] = cur
    return out


def ar1_tokens(rng, T: int, d: int, rho: float) -> np.ndarray:
    """[T, d] fp16 token inputs with AR(1) correlation rho between tokens."""
    out = np.empty((T, d), np.float64)
    out[0] = rng.normal(size=d)
    s = np.sqrt(1.0 - rho * rho)
    for t in range(1, T):
        out[t] = rho * out[t - 1] + s * rng.normal(size=d)
    return out.astype(np.float16)
