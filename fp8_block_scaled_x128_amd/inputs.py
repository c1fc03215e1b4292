"""Seeded synthetic inputs for the block-wise FP8 linear layer.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it only draws
random tensors, rounds them to bf16 (the input precision of the layer) and
builds MoE routing.  Shapes follow the Qwen3-4B dense MLP and the
Qwen3-30B-A3B MoE layer, the two models the pages run the block-wise FP8
recipe on ("Low Precision RL", table "Choose a precision").

Random numbers: ``numpy.random.Generator(PCG64(child))`` where ``child`` is
the i-th of ``SeedSequence(seed).spawn(n)``, one child per tensor, in the
order listed by each workload.  Normal draws are float32 ``standard_normal``
times sigma; outliers are ``round(p * numel)`` positions drawn without
replacement from the same child and multiplied by the stated factor before
the single round-to-nearest-even conversion to bf16.

All tensors are returned as numpy ``uint16`` arrays of bf16 bit patterns (or
float32 / int32 for routing).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def _children(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(seed).spawn(n)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(rng: np.random.Generator, shape, sigma: float, outlier_frac: float = 0.0,
                outlier_mult: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outlier_frac > 0.0:
        n = x.size
        k = int(round(outlier_frac * n))
        if k:
            pos = rng.choice(n, size=k, replace=False)
            flat = x.reshape(-1)
            flat[pos] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


# ---------------------------------------------------------------------------
# dense workloads
# ---------------------------------------------------------------------------
def tiny_linear(seed: int = 0):
    """Tiny block-wise FP8 linear: X [256, 512] N(0,1) with 0.5% x50 outliers,
    W [512, 512] N(0, 0.02).  Children: X, W."""
    rx, rw = _children(seed, 2)
    x = normal_bf16(rx, (256, 512), 1.0, 0.005, 50.0)
    w = normal_bf16(rw, (512, 512), 0.02)
    return {"x": x, "w": w}


def qwen3_4b_mlp(seed: int = 1, parts=("up", "down")):
    """Qwen3-4B MLP forward: up X [4096, 2560], W_up [9728, 2560]; down
    X [4096, 9728], W_down [2560, 9728].  X ~ N(0,1) with 0.1% x100 outliers,
    W ~ N(0, 0.02).  Children, in order: X_up, W_up, X_down, W_down."""
    r = _children(seed, 4)
    out = {}
    if "up" in parts:
        out["x_up"] = normal_bf16(r[0], (4096, 2560), 1.0, 0.001, 100.0)
        out["w_up"] = normal_bf16(r[1], (9728, 2560), 0.02)
    if "down" in parts:
        out["x_down"] = normal_bf16(r[2], (4096, 9728), 1.0, 0.001, 100.0)
        out["w_down"] = normal_bf16(r[3], (2560, 9728), 0.02)
    return out


def qwen3_4b_mlp_backward(seed: int = 2, mlp_seed: int = 1):
    """Backward GEMM operands for the same MLP: dY [4096, 9728] ~ N(0, 1e-3)
    (no outliers) from `seed`; X [4096, 2560] and W [9728, 2560] are the
    up-projection tensors of the forward workload (`mlp_seed`)."""
    (rd,) = _children(seed, 1)
    dy = normal_bf16(rd, (4096, 9728), 1e-3)
    fwd = qwen3_4b_mlp(mlp_seed, parts=("up",))
    return {"dy": dy, "x": fwd["x_up"], "w": fwd["w_up"]}


# ---------------------------------------------------------------------------
# MoE workload
# ---------------------------------------------------------------------------
@dataclass
class MoERouting:
    """Token -> expert assignments sorted by (expert, token).

    ``row_token[r]`` is the source token of grouped row r; rows of expert g
    are ``offsets[g]:offsets[g+1]`` (empty groups allowed)."""
    offsets: np.ndarray          # int32 [G+1]
    row_token: np.ndarray        # int32 [tokens * top_k]
    topk_experts: np.ndarray     # int32 [tokens, top_k]
    counts: np.ndarray = field(default=None)
    token_rows: np.ndarray = field(default=None)   # int32 [tokens, top_k]: grouped row of (token, slot)
    weights: np.ndarray = field(default=None)      # float32 [tokens, top_k]: routing weights


def route_topk(logits: np.ndarray, top_k: int) -> MoERouting:
    """Top-k experts per token by router logit (the softmax is monotone, so
    ranking logits ranks probabilities); ties go to the lower expert index.
    Assignments are then stably sorted by (expert, token).  The routing
    weights are the softmax of the token's selected logits in float32 (the
    router's probabilities renormalized over the top k); they are inputs of
    the combine, computed here like any other synthetic input."""
    T, G = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    experts = order.reshape(-1)
    tokens = np.repeat(np.arange(T, dtype=np.int32), top_k)
    perm = np.lexsort((tokens, experts))            # primary key: expert, then token
    counts = np.bincount(experts, minlength=G).astype(np.int64)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    token_rows = np.empty(T * top_k, np.int32)
    token_rows[perm] = np.arange(T * top_k, dtype=np.int32)
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float32)
    e = np.exp(sel - sel[:, :1])                    # order[:, 0] holds the largest logit
    weights = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return MoERouting(offsets=offsets, row_token=tokens[perm].astype(np.int32),
                      topk_experts=order, counts=counts, token_rows=token_rows.reshape(T, top_k),
                      weights=weights)


def qwen3_30b_a3b_moe(seed: int = 3, tokens: int = 16384, hidden: int = 2048, experts: int = 128,
                      inter: int = 768, top_k: int = 8, skewed: bool = False, weights: bool = True,
                      empty_mod: int = 16):
    """Qwen3-30B-A3B-shaped MoE layer.  Children, in order: router logits
    [tokens, experts] fp32 N(0,1); X [tokens, hidden] N(0,1) bf16;
    W_gu [experts, 2*inter, hidden] N(0, 0.02) (rows [0, inter) gate, rows
    [inter, 2*inter) up); W_d [experts, inter, hidden] N(0, 0.02) (the down
    projection contracts over `inter`).

    ``skewed=True`` is a parity-only variant: logits of experts e with
    e % empty_mod == empty_mod - 1 are set to -inf (those groups are empty) and every other
    expert's logit gets a bias -ln(1 + e), giving group sizes from tens to
    thousands that are not multiples of 128."""
    r = _children(seed, 4)
    logits = r[0].standard_normal(size=(tokens, experts), dtype=np.float32)
    if skewed:
        e = np.arange(experts)
        bias = -np.log1p(e).astype(np.float32)
        bias[e % empty_mod == empty_mod - 1] = -np.inf
        logits = logits + bias[None, :]
    routing = route_topk(logits, top_k)
    out = {"logits": logits, "routing": routing,
           "x": normal_bf16(r[1], (tokens, hidden), 1.0)}
    if weights:
        out["w_gu"] = normal_bf16(r[2], (experts, 2 * inter, hidden), 0.02)
        out["w_d"] = normal_bf16(r[3], (experts, inter, hidden), 0.02)
    return out


def small_moe(seed: int = 3, tokens: int = 512, hidden: int = 256, experts: int = 8, inter: int = 128,
              top_k: int = 2, skewed: bool = True, empty_mod: int = 4):
    """Scaled-down MoE layer with the same recipe (for oracle-sized parity)."""
    return qwen3_30b_a3b_moe(seed, tokens, hidden, experts, inter, top_k, skewed,
                             empty_mod=empty_mod)
