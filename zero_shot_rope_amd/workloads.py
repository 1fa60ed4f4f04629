"""Seeded synthetic inputs for the bifocal attention workloads.

This module draws random inputs and rounds them to bfloat16. It holds none of the
attention method's arithmetic (no group size, no aliasing, no rotation, no softmax),
so both the GPU path and the CPU oracle can be fed from it.

The workloads are layer shapes of the Qwen3 dense family that the Jet-Long pages
evaluate (review page, "Validation": Qwen3 1.7B/4B/8B base models with a 32K native
window, extended to 128K). The pages publish no activations, so every tensor is
drawn i.i.d. N(0, 1) from a numpy Generator seeded per workload; no dataset is read.

Inputs are post-base-RoPE queries/keys (the cache holds keys rotated at their base
absolute positions). Since RoPE is orthogonal, i.i.d. Gaussian vectors keep their
distribution under it, so drawing them directly is equivalent to drawing raw vectors
and applying base RoPE.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the uint16 bit patterns.

    Inputs here are finite Gaussian draws, so NaN handling is not needed; a NaN input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        bits = flat_in[s:s + step]
        # Finite values stay below 0xFF800000, so the 32-bit sum cannot wrap.
        if np.any((bits & 0x7F800000) == 0x7F800000):
            raise ValueError("bf16 rounding expects finite inputs")
        flat_out[s:s + step] = ((bits + (0x7FFF + ((bits >> 16) & 1))) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Prefill:
    """A prefill workload: Q [B, L, Hq, D], K/V [B, L, Hkv, D] in BSHD order."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    L: int
    w0: int
    w_pretrained: int
    rope_theta: float
    seed: int
    k_scale: float = 1.0

    def flops(self) -> float:
        """Algorithmic flops: one D-long score and one D-long PV product per causal pair."""
        return 4.0 * self.batch * self.n_q_heads * self.head_dim * self.L * (self.L + 1) / 2.0


@dataclasses.dataclass(frozen=True)
class Decode:
    """Single-batch decode: one query per step against a cache [B, Lcap, Hkv, D]."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    L_first: int  # keys attended at step 0 (the new token included)
    steps: int
    w0: int
    w_pretrained: int
    rope_theta: float
    seed: int

    @property
    def capacity(self) -> int:
        return self.L_first + self.steps - 1

    def bytes_per_step(self, L: int) -> float:
        """Algorithmic HBM bytes of one step: every cached K and V row read once (bf16)."""
        return 2.0 * L * self.n_kv_heads * self.head_dim * 2 * self.batch


# Tiny prefill: one head, D=64, L=512, theta 1e4, pretrained window 128, local window 32.
TINY = Prefill("tiny_L512_D64", 1, 1, 1, 64, 512, 32, 128, 1.0e4, seed=1)
# Qwen3-1.7B layer shape at L=8192 <= 32768: the in-window case.
QWEN3_1_7B_8K = Prefill("qwen3_1.7b_L8192", 1, 16, 8, 128, 8192, 2048, 32768, 1.0e6, seed=2)
# Qwen3-4B layer shape at L=65536 with keys scaled by 0.5; w0 swept.
QWEN3_4B_64K = {
    w0: Prefill(f"qwen3_4b_L65536_w{w0}", 1, 32, 8, 128, 65536, w0, 32768, 1.0e6, seed=3, k_scale=0.5)
    for w0 in (1024, 2048, 4096)
}
# Qwen3-8B layer shape at L=131072.
QWEN3_8B_128K = Prefill("qwen3_8b_L131072", 1, 32, 8, 128, 131072, 2048, 32768, 1.0e6, seed=4)
# Single-batch decode, Qwen3-8B heads, 512 steps from 98001 keys (query position 98000).
QWEN3_8B_DECODE = Decode("qwen3_8b_decode_98k", 1, 32, 8, 128, 98001, 512, 2048, 32768, 1.0e6, seed=5)
# Single-batch decode at 128K: the same heads, 512 steps ending at 131072 keys (G = 4 throughout).
QWEN3_8B_DECODE_128K = Decode("qwen3_8b_decode_128k", 1, 32, 8, 128, 131072 - 511, 512, 2048, 32768, 1.0e6, seed=8)


def _draw(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return x


def prefill_inputs(cfg: Prefill, L: Optional[int] = None):
    """Draw Q, K, V for a prefill workload; return dict of bf16 bit arrays (uint16).

    Draw order is Q, K, V. `L` may shorten the sequence (a smaller case of the same shape
    and distribution); the draw then uses that L.
    """
    L = cfg.L if L is None else L
    rng = np.random.default_rng(cfg.seed)
    q = _draw(rng, (cfg.batch, L, cfg.n_q_heads, cfg.head_dim))
    k = _draw(rng, (cfg.batch, L, cfg.n_kv_heads, cfg.head_dim), cfg.k_scale)
    v = _draw(rng, (cfg.batch, L, cfg.n_kv_heads, cfg.head_dim))
    return {"q": round_to_bf16_bits(q), "k": round_to_bf16_bits(k), "v": round_to_bf16_bits(v)}


def decode_inputs(cfg: Decode, capacity: Optional[int] = None):
    """Draw the K/V cache and the per-step queries for a decode workload (bf16 bits).

    Draw order: K cache, V cache, then all step queries [steps, B, Hq, D].
    """
    cap = cfg.capacity if capacity is None else capacity
    rng = np.random.default_rng(cfg.seed)
    kc = _draw(rng, (cfg.batch, cap, cfg.n_kv_heads, cfg.head_dim))
    vc = _draw(rng, (cfg.batch, cap, cfg.n_kv_heads, cfg.head_dim))
    qs = _draw(rng, (cfg.steps, cfg.batch, cfg.n_q_heads, cfg.head_dim))
    return {"k_cache": round_to_bf16_bits(kc), "v_cache": round_to_bf16_bits(vc), "q_steps": round_to_bf16_bits(qs)}


def random_case(seed: int, batch: int, L: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                scale: float = 1.0):
    """Generic seeded Q/K/V draw (bf16 bits) for parity cases of arbitrary shape."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (batch, L, n_q_heads, head_dim), scale)
    k = _draw(rng, (batch, L, n_kv_heads, head_dim), scale)
    v = _draw(rng, (batch, L, n_kv_heads, head_dim))
    return {"q": round_to_bf16_bits(q), "k": round_to_bf16_bits(k), "v": round_to_bf16_bits(v)}
