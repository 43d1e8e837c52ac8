"""Seeded synthetic inputs for the DDTree tree-verify step.

This module only draws random numbers and lays them out; it holds none of the
verify step's arithmetic (no tree build, attention, vocabulary reduction or
walk). It is the one module that both the CPU oracle's tests and the GPU path's
tests, smoke run and benchmark read their inputs from.

Workloads (one entry per configuration; sizes are those of one tensor-parallel
shard's attention heads on one GPU):

  tiny      B=1,  ctx 256,            4/4 heads, Dh 64,  fp32; D 8,  budget 8,  K 2; V 1024;   greedy
  single    B=1,  ctx 8192,           8/8 heads, Dh 128, bf16; D 8,  budget 32, K 4; V 163840; greedy
  batched   B=16, ctx 4096 each,      8/8 heads, Dh 128, bf16; D 8,  budget 32, K 8; V 163840; T 0.7
  long      B=1,  ctx 65536,          8/8 heads, Dh 128, bf16; D 16, budget 64, K 4; V 163840; greedy
  ragged    B=64, ctx U[512, 16384],  8/8 heads, Dh 128, bf16; D 8,  budget 32, K 4; V 163840; T 1.0,
            target argmax planted on the draft's top-1 with p=0.6 per node

Distributions (the standard deviation is the second argument of N(0, s)):
  * Q, context K/V and tree K/V ~ N(0, 1), rounded to bf16 (RNE) or kept fp32.
  * Draft logits: D+1 rows per request, row d (0-based) is the drafter's
    prediction for tree depth d+1; N(0, s_draft) in fp32.  The drafter is
    block-diffusion style, so row d does not depend on the path (The Tree That
    Couldn't Branch, "Hypothesis 4: The Block-Diffusion Fundamental
    Limitation").
  * Per-depth top-K (the harness stand-in for the draft head): tokens ordered
    by (logit desc, id asc); log-probs are the full-vocabulary log-softmax at
    temperature 1, computed in float64 and rounded to fp32.
  * Target logits of a node at depth d: draft row d plus independent
    N(0, s_target) noise per node, then rounded to bf16 (fp32 for "tiny").
  * Per-node uniforms: raw 64-bit words of a Philox stream, two per node.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "ctx_lengths", "make_inputs", "make_target_logits",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "uniforms_for",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    ctx: object              # int (every request) or (lo, hi) inclusive uniform range
    Hq: int
    Hkv: int
    Dh: int
    dtype: str               # "f32" or "bf16"
    D: int                   # draft depth
    budget: int
    K: int                   # per-node top-k cap
    V: int                   # vocabulary size
    temperature: float       # 0 => greedy verify
    sigma_draft: float
    sigma_target: float
    plant: bool = False      # plant the target argmax (ragged workload)
    seed_index: int = 0

    @property
    def N(self) -> int:
        return self.budget + 1

    @property
    def seed(self) -> int:
        return 20261200 + self.seed_index


CONFIGS = {
    "tiny": Config("tiny", 1, 256, 4, 4, 64, "f32", 8, 8, 2, 1024, 0.0, 2.0, 1.0, seed_index=1),
    "single": Config("single", 1, 8192, 8, 8, 128, "bf16", 8, 32, 4, 163840, 0.0, 3.0, 1.5,
                     seed_index=2),
    "batched": Config("batched", 16, 4096, 8, 8, 128, "bf16", 8, 32, 8, 163840, 0.7, 3.0, 1.5,
                      seed_index=3),
    "long": Config("long", 1, 65536, 8, 8, 128, "bf16", 16, 64, 4, 163840, 0.0, 3.0, 1.5,
                   seed_index=4),
    "ragged": Config("ragged", 64, (512, 16384), 8, 8, 128, "bf16", 8, 32, 4, 163840, 1.0, 3.0,
                     1.5, plant=True, seed_index=5),
}


def config(name: str, **overrides) -> Config:
    """Named workload, optionally with fields replaced (smaller test variants)."""
    return dataclasses.replace(CONFIGS[name], **overrides)


# --- random streams -----------------------------------------------------------------------

_TAGS = {"q": 1, "k_ctx": 2, "v_ctx": 3, "k_tree": 4, "v_tree": 5, "draft": 6, "noise": 7,
         "root": 8, "ctx_len": 9, "plant": 10}


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=np.array([seed, _TAGS[tag]], dtype=np.uint64)))


def uniforms_for(seed: int, b: int, N: int) -> np.ndarray:
    """Two raw 64-bit Philox words per node for request b: [N, 2] uint64.

    Slot 0 is the accept test used when the node is tested as a child; slot 1
    is the bonus draw used if the walk stops at the node."""
    g = np.random.Philox(key=np.array([seed, 1000 + b], dtype=np.uint64))
    return g.random_raw(2 * N).astype(np.uint64).reshape(N, 2)


# --- bf16 bit handling (storage format only) ----------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _normal(gen: np.random.Generator, shape, sigma: float, dtype: str,
            chunk: int = 1 << 25) -> np.ndarray:
    """N(0, sigma) samples in the storage dtype (bf16 -> uint16 bits), drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = gen.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[s:e] = f32_to_bf16_bits(v) if dtype == "bf16" else v
    return out.reshape(shape)


# --- workload inputs ----------------------------------------------------------------------

def ctx_lengths(cfg: Config) -> np.ndarray:
    if isinstance(cfg.ctx, tuple):
        lo, hi = cfg.ctx
        return _rng(cfg.seed, "ctx_len").integers(lo, hi + 1, size=cfg.B).astype(np.int32)
    return np.full(cfg.B, int(cfg.ctx), dtype=np.int32)


def make_inputs(cfg: Config, with_kv: bool = True) -> dict:
    """Everything the step needs except the target logits (which depend on the tree).

    Returns numpy arrays; bf16 tensors are uint16 bit patterns.
      ctx_lens [B] i32, ctx_offsets [B+1] i32, prefix_len [B] i32
      k_ctx, v_ctx [sum L, Hkv, Dh]; q [B, N, Hq, Dh]; k_tree, v_tree [B, N, Hkv, Dh]
      draft_logits [B, D+1, V] f32 (row d predicts depth d+1; rows 0..D-1 feed
        the draft top-K, row D only gives depth-D nodes a target row)
      root_tok [B] i32, uniforms [B, N, 2] u64
    The tree build's inputs (draft_tok, draft_lp) are the draft top-K of the
    first D rows: ddtree_draft_topk on the GPU, or the oracle's draft_topk.
    """
    B, N, D, V = cfg.B, cfg.N, cfg.D, cfg.V
    lens = ctx_lengths(cfg)
    offs = np.zeros(B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    if offs[-1] >= 2 ** 31:
        raise ValueError("total context exceeds int32 offsets")
    out = {"ctx_lens": lens, "ctx_offsets": offs.astype(np.int32), "prefix_len": lens.copy()}
    dt = cfg.dtype
    if with_kv:
        tot = int(offs[-1])
        out["k_ctx"] = _normal(_rng(cfg.seed, "k_ctx"), (tot, cfg.Hkv, cfg.Dh), 1.0, dt)
        out["v_ctx"] = _normal(_rng(cfg.seed, "v_ctx"), (tot, cfg.Hkv, cfg.Dh), 1.0, dt)
    out["q"] = _normal(_rng(cfg.seed, "q"), (B, N, cfg.Hq, cfg.Dh), 1.0, dt)
    out["k_tree"] = _normal(_rng(cfg.seed, "k_tree"), (B, N, cfg.Hkv, cfg.Dh), 1.0, dt)
    out["v_tree"] = _normal(_rng(cfg.seed, "v_tree"), (B, N, cfg.Hkv, cfg.Dh), 1.0, dt)
    dl = _normal(_rng(cfg.seed, "draft"), (B, D + 1, V), cfg.sigma_draft, "f32")
    out["draft_logits"] = dl
    out["root_tok"] = _rng(cfg.seed, "root").integers(0, V, size=B).astype(np.int32)
    out["uniforms"] = np.stack([uniforms_for(cfg.seed, b, N) for b in range(B)])
    return out


def make_target_logits(cfg: Config, inputs: dict, depth: np.ndarray, num_nodes: np.ndarray,
                       plant_margin: float = 8.0):
    """Target logits [B, N, V] for a built tree (depth [B, N], num_nodes [B]).

    Node n at depth d gets draft row d plus N(0, sigma_target) noise.  Padding
    nodes (n >= num_nodes[b]) get noise around draft row 0.  With cfg.plant,
    every valid node independently gets a planted argmax: with p=0.6 the
    draft's top-1 token for depth d+1, otherwise uniformly one of the draft's
    ranks 2..4 (1-based) or a token outside that depth's top-K; the planted
    logit is the row maximum plus `plant_margin`.

    Planting reads the draft's ranking from inputs["draft_tok_all"] [B, D+1, >= 4]
    (each draft row's top tokens in rank order, from a draft top-K pass).

    Returns (logits, planted) where logits is uint16 bf16 bits or float32 and
    planted [B, N] i32 holds the planted token (-1 when not planting)."""
    B, N, V = cfg.B, cfg.N, cfg.V
    dl = inputs["draft_logits"]
    gen = _rng(cfg.seed, "noise")
    pgen = _rng(cfg.seed, "plant")
    planted = np.full((B, N), -1, dtype=np.int32)
    out = np.empty((B, N, V), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    for b in range(B):
        for n in range(N):
            d = int(depth[b, n]) if n < num_nodes[b] else 0
            row = dl[b, d] + gen.standard_normal(V, dtype=np.float32) * np.float32(cfg.sigma_target)
            if cfg.plant and n < num_nodes[b]:
                tops = inputs["draft_tok_all"][b, d]
                if pgen.random() < 0.6:
                    tok = int(tops[0])
                else:
                    choice = int(pgen.integers(0, 4))
                    if choice < 3 and choice + 1 < tops.shape[0]:
                        tok = int(tops[choice + 1])
                    else:
                        while True:
                            tok = int(pgen.integers(0, V))
                            if tok not in set(int(t) for t in tops):
                                break
                row[tok] = row.max() + np.float32(plant_margin)
                planted[b, n] = tok
            out[b, n] = f32_to_bf16_bits(row) if cfg.dtype == "bf16" else row
    return out, planted
