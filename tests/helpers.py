"""Test-side helpers: an independent int4 packer/unpacker and the parity rules.

The packer and unpacker restate the int4 layout reading (element i of a row
in 32-bit word i/8 at bits 4*(i%8), two's-complement nibble) with numpy bit
operations, independently of both the oracle and the HIP library.
"""

from __future__ import annotations

import itertools

import numpy as np

# Output tolerance for fp16 results against the fp64 oracle:
# |gpu - ref| <= ATOL + RTOL * |ref| element-wise.
ATOL = 2e-3
RTOL = 1e-2
# Routing weights and near-tie gap.
W_TOL = 1e-4
TIE_GAP = 1e-3


def pack_q4(Q: np.ndarray) -> np.ndarray:
    """int matrix [..., cols] in [-8, 7] -> uint32 words [..., cols/8]."""
    Q = np.asarray(Q)
    assert Q.min() >= -8 and Q.max() <= 7 and Q.shape[-1] % 8 == 0
    nib = (Q.astype(np.int64) & 15).astype(np.uint32)
    nib = nib.reshape(*Q.shape[:-1], Q.shape[-1] // 8, 8)
    words = np.zeros(nib.shape[:-1], np.uint32)
    for j in range(8):
        words |= nib[..., j] << np.uint32(4 * j)
    return words


def unpack_q4(words: np.ndarray) -> np.ndarray:
    """uint32 words [..., cols/8] -> int8 values [..., cols]."""
    w = np.asarray(words, np.uint32)
    shifts = (np.arange(8, dtype=np.uint32) * 4)
    nib = ((w[..., None] >> shifts) & np.uint32(15)).astype(np.int16)
    q = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8)


def dequant_ref(words, scales, G) -> np.ndarray:
    """Dense fp64 weights from packed int4 + fp16 group scales."""
    q = unpack_q4(words).astype(np.float64)
    s = np.asarray(scales).astype(np.float64)
    return q * np.repeat(s, G, axis=-1)


def out_err(gpu, ref):
    """Worst ratio |gpu-ref| / (ATOL + RTOL |ref|); <= 1 passes."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref) / (ATOL + RTOL * np.abs(ref))))


def assert_out_close(gpu, ref, what=""):
    r = out_err(gpu, ref)
    assert r <= 1.0, f"{what}: worst error ratio {r:.3f} (atol {ATOL}, rtol {RTOL})"


def topk_set_ok(score: np.ndarray, got: np.ndarray, K: int, allowed=None, gap=TIE_GAP) -> bool:
    """A K-set is acceptable if it is a top-K of `score` up to gap-wide near ties.

    Every chosen id must be allowed, ids must be distinct, and the smallest
    chosen score must be >= the largest unchosen allowed score - gap.
    """
    got = np.asarray(got)
    if got.size != K or np.unique(got).size != K:
        return False
    mask = np.ones(score.size, bool) if allowed is None else np.asarray(allowed, bool).copy()
    if not mask[got].all():
        return False
    chosen = np.zeros(score.size, bool)
    chosen[got] = True
    rest = score[mask & ~chosen]
    if rest.size == 0:
        return True
    return float(score[got].min()) >= float(rest.max()) - gap


def routing_set_ok(dims: dict, logits: np.ndarray, got: np.ndarray, bias=None,
                   gap=TIE_GAP) -> bool:
    """Near-tie acceptance for a routed set, given the oracle's fp64 logits.

    Softmax-top-K: a top-K of the logits up to `gap`. Sigmoid-group: there
    must be a choice S of topk_groups groups that holds every group the set
    touches and is a top-topk_groups of the group scores up to `gap` (its
    lowest score at least the highest score outside S minus `gap`), such that
    the set is a top-K of the biased scores within S up to `gap`. Every such
    S is tried (C(8, 4) = 70 at most for the tiers here).
    """
    K, E = dims["K"], dims["E"]
    if dims["router_kind"] == 0:
        return topk_set_ok(np.asarray(logits, np.float64), got, K, gap=gap)
    n, Gk = dims["n_groups"], dims["topk_groups"]
    per = E // n
    sig = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    sel = sig + (0.0 if bias is None else np.asarray(bias, np.float64))
    gs = np.sort(sel.reshape(n, per), axis=1)[:, -2:].sum(axis=1)
    touched = sorted(set((np.asarray(got) // per).tolist()))
    if len(touched) > Gk:
        return False
    others = [g for g in range(n) if g not in touched]
    for extra in itertools.combinations(others, Gk - len(touched)):
        S = set(touched) | set(extra)
        outside = [g for g in range(n) if g not in S]
        if outside and gs[list(S)].min() < gs[outside].max() - gap:
            continue
        allowed = np.zeros(E, bool)
        for g in S:
            allowed[g * per:(g + 1) * per] = True
        if topk_set_ok(sel, got, K, allowed=allowed, gap=gap):
            return True
    return False
