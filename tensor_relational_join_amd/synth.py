"""Seeded synthetic inputs.

This module only produces input tensors; it holds none of the join-agg
arithmetic and imports neither the HIP binding nor the CPU checker, so both
sides can be fed the same bytes from it.

Generator (counter-based, so any element can be produced independently):
  * SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) applied to the counter
    value  key + (i + 1) * 0x9E3779B97F4A7C15, where
    key = mix(seed * 0x100000001B3 + stream)  and i is the element index;
  * a 24-bit uniform  u = (z >> 40) * 2^-24  in [0, 1);
  * normals by the Box-Muller transform in float64 on the pair of uniforms
    drawn from counters 2i and 2i + 1 (u1 is shifted into (0, 1]);
  * values are rounded to float32 (nearest-even), and to bfloat16
    (nearest-even) where a bf16 tensor is requested.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        v = np.array([(seed * 0x100000001B3 + stream) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        return _mix(v)[0]


def raw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """SplitMix64 outputs for counters start .. start+count-1."""
    key = _key(seed, stream)
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + i * _GAMMA)


def _uniform24(z: np.ndarray) -> np.ndarray:
    return (z >> np.uint64(40)).astype(np.float64) * (1.0 / 16777216.0)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _run_chunks(fn, starts):
    starts = list(starts)
    if len(starts) <= 1:
        for s in starts:
            fn(s)
        return
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fn, starts))


def uniform(seed: int, stream: int, shape: Sequence[int], lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """float32 values uniform on [lo, hi)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)

    def chunk(s):
        c = min(_CHUNK, n - s)
        u = _uniform24(raw_u64(seed, stream, s, c))
        out[s:s + c] = (lo + (hi - lo) * u).astype(np.float32)

    _run_chunks(chunk, range(0, n, _CHUNK))
    return out.reshape(tuple(shape))


def normal(seed: int, stream: int, shape: Sequence[int], mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """float32 values N(mean, std^2) by Box-Muller."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    npair = (n + 1) // 2

    def chunk(s):
        c = min(_CHUNK, npair - s)
        z = raw_u64(seed, stream, 2 * s, 2 * c)
        u1 = ((z[0::2] >> np.uint64(40)).astype(np.float64) + 1.0) * (1.0 / 16777216.0)
        u2 = _uniform24(z[1::2])
        r = np.sqrt(-2.0 * np.log(u1))
        th = 2.0 * np.pi * u2
        pair = np.empty(2 * c, dtype=np.float64)
        pair[0::2] = r * np.cos(th)
        pair[1::2] = r * np.sin(th)
        lo = 2 * s
        hi = min(n, lo + 2 * c)
        out[lo:hi] = (mean + std * pair[: hi - lo]).astype(np.float32)

    _run_chunks(chunk, range(0, npair, _CHUNK))
    return out.reshape(tuple(shape))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), nearest-even (inputs only)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def normal_bf16(seed: int, stream: int, shape: Sequence[int], mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of N(mean, std^2) draws."""
    return f32_to_bf16_bits(normal(seed, stream, shape, mean, std))


def normal_f16(seed: int, stream: int, shape: Sequence[int], mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """IEEE half bit patterns (uint16) of N(mean, std^2) draws, rounded once
    from float64 to nearest even (numpy's float16 conversion)."""
    return np.asarray(normal(seed, stream, shape, mean, std), dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for convenience in
    harness code; not used by either implementation's arithmetic)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


LLAMA_BLOCK_STREAMS = ["x", "g1", "w_qkv", "w_o", "g2", "w_gate", "w_up", "w_down"]


def llama_block_inputs(seed: int, batch: int, seq: int, dm: int, ffn: int, qkv_cols: Optional[int] = None,
                       dtype: str = "bf16") -> dict:
    """bf16 (dtype "f16": IEEE half) bit patterns of one block's inputs: x ~ N(0,1) [batch*seq, dm];
    gains ~ N(1, 0.1) [dm]; weights ~ N(0, 0.02): w_qkv [dm, qkv_cols] (= [W_q
    | W_k | W_v]; 3 dm columns unless given, fewer with grouped key-value
    heads), w_o [dm, dm], w_gate and w_up [dm, ffn], w_down [ffn, dm], and
    w_gu [dm, ffn, 2], the gate and up weights paired column by column.
    Stream i of `seed` feeds the i-th tensor of LLAMA_BLOCK_STREAMS."""
    T = batch * seq
    shapes = {"x": (T, dm), "g1": (dm,), "w_qkv": (dm, qkv_cols or 3 * dm), "w_o": (dm, dm), "g2": (dm,),
              "w_gate": (dm, ffn), "w_up": (dm, ffn), "w_down": (ffn, dm)}
    out = {}
    for i, name in enumerate(LLAMA_BLOCK_STREAMS):
        if name == "x":
            mean, std = 0.0, 1.0
        elif name in ("g1", "g2"):
            mean, std = 1.0, 0.1
        else:
            mean, std = 0.0, 0.02
        draw = normal_f16 if dtype == "f16" else normal_bf16
        out[name] = draw(seed, i, shapes[name], mean=mean, std=std)
    # the same weights laid out for a gate-and-up contraction: [dm, ffn, 2],
    # the gate weight then the up weight of each column side by side
    out["w_gu"] = np.ascontiguousarray(np.stack([out["w_gate"], out["w_up"]], axis=2))
    return out
