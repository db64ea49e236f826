"""Seeded synthetic inputs for the pooled Gated DeltaNet decode step.

This module is the only thing the HIP path and the CPU oracle share.  It draws
arrays and holds none of the step's arithmetic: values are drawn with numpy's
PCG64 and rounded to bf16 where the layout stores bf16.  The gates are drawn
already transformed (g = -softplus(n), beta = sigmoid(n)), as the step takes
them precomputed.

Workloads (synthetic stand-ins for the serving runs on the mstar pages, whose
prompts and weights are not available; the step's work depends only on the
shapes and the slot indices):

  tiny     B=4, H_k=H_v=4, d=64, 9-slot pool, 8 chained steps, twin slots
  0.8b     B=64, H_k=H_v=16, d=128, 257 slot pairs (N=513), twin slots
  sweep    the 0.8b shapes at B in {1, 4, 16, 64, 128}
  9b       B=64, H_k=16, H_v=32, d=128, 24 layers, one 129-slot pool each
  padded   the 0.8b shapes, 128 rows of which the last 82 sit on slot 0

Draw order (one Generator(PCG64(seed)) per case): for each layer the pool
state, the conv windows, the conv weights and the slot permutation; then for
each step and each layer x, the g normals and the beta normals.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Shape:
    """Sizes of one decode step: rows, tokens per row, heads, head dims, conv width, pool slots."""
    B: int
    T: int
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    W: int
    N: int

    @property
    def C(self) -> int:
        """Conv channels: q and k of every key head, v of every value head."""
        return 2 * self.H_k * self.d_k + self.H_v * self.d_v

    @property
    def G(self) -> int:
        return self.H_v // self.H_k


# ------------------------------------------------------------------ bf16 storage

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest even) and return the bit patterns (uint16)."""
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ draws

@dataclass
class Pool:
    """One layer's slot pool and its conv weights, plus the step's slot arrays."""
    state: np.ndarray        # [N][H_v][d_k][d_v] fp32, slot 0 all zero
    conv_state: np.ndarray   # [N][W-1][C] bf16 bits, slot 0 all zero
    conv_w: np.ndarray       # [C][W] bf16 bits
    read_slot: np.ndarray    # [B] int32
    write_slot: np.ndarray   # [B] int32 (twin slots; equal to read_slot in place)


@dataclass
class StepInputs:
    x: np.ndarray            # [B][T][C] bf16 bits
    g: np.ndarray            # [B][T][H_v] fp32, log decay (<= 0)
    beta: np.ndarray         # [B][T][H_v] fp32, in (0, 1)


@dataclass
class Case:
    name: str
    shape: Shape
    pools: list              # one Pool per layer
    steps: list              # steps[s][layer] -> StepInputs
    real_rows: int
    twin: bool
    meta: dict = field(default_factory=dict)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def draw_pool(rng: np.random.Generator, s: Shape, real_rows: int, state_std: float = 0.1,
              conv_w_bound: float = 0.5) -> Pool:
    """Pool state ~ N(0, state_std^2) and conv windows ~ N(0, 1) in every slot but 0;
    conv weights ~ U(-bound, bound); rows 0..real_rows-1 take a random permutation of the
    slot pairs (2p-1, 2p), the rest sit on slot 0."""
    if (s.N - 1) % 2 != 0:
        raise ValueError("pool must hold the null slot plus whole slot pairs")
    pairs = (s.N - 1) // 2
    if real_rows > pairs:
        raise ValueError("more real rows than slot pairs")
    state = np.zeros((s.N, s.H_v, s.d_k, s.d_v), np.float32)
    state[1:] = rng.standard_normal((s.N - 1, s.H_v, s.d_k, s.d_v), dtype=np.float32)
    state[1:] *= np.float32(state_std)
    conv_state = np.zeros((s.N, s.W - 1, s.C), np.uint16)
    conv_state[1:] = bf16_bits(rng.standard_normal((s.N - 1, s.W - 1, s.C), dtype=np.float32))
    conv_w = bf16_bits(rng.uniform(-conv_w_bound, conv_w_bound, (s.C, s.W)).astype(np.float32))
    perm = rng.permutation(pairs)[:real_rows].astype(np.int64) + 1
    read_slot = np.zeros(s.B, np.int32)
    write_slot = np.zeros(s.B, np.int32)
    read_slot[:real_rows] = 2 * perm - 1
    write_slot[:real_rows] = 2 * perm
    return Pool(state, conv_state, conv_w, read_slot, write_slot)


def draw_step(rng: np.random.Generator, s: Shape) -> StepInputs:
    """x ~ N(0, 1) as bf16; g = -softplus(N(0, 1)); beta = sigmoid(N(0, 1))."""
    x = bf16_bits(rng.standard_normal((s.B, s.T, s.C), dtype=np.float32))
    g = (-_softplus(rng.standard_normal((s.B, s.T, s.H_v)))).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((s.B, s.T, s.H_v))).astype(np.float32)
    return StepInputs(x, g, beta)


def make_case(name: str, shape: Shape, *, steps: int = 1, layers: int = 1, real_rows: int | None = None,
              twin: bool = True, seed: int = 0) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    rr = shape.B if real_rows is None else real_rows
    pools = [draw_pool(rng, shape, rr) for _ in range(layers)]
    if not twin:
        for p in pools:
            p.write_slot[:] = p.read_slot
    st = [[draw_step(rng, shape) for _ in range(layers)] for _ in range(steps)]
    return Case(name, shape, pools, st, rr, twin)


# ------------------------------------------------------------------ named workloads

SHAPE_TINY = Shape(B=4, T=1, H_k=4, H_v=4, d_k=64, d_v=64, W=4, N=9)
SHAPE_08B = Shape(B=64, T=1, H_k=16, H_v=16, d_k=128, d_v=128, W=4, N=513)
SHAPE_9B = Shape(B=64, T=1, H_k=16, H_v=32, d_k=128, d_v=128, W=4, N=129)
SWEEP_ROWS = (1, 4, 16, 64, 128)
PADDED_ROWS, PADDED_REAL = 128, 46


def tiny(seed: int = 0) -> Case:
    """4 rows, 4+4 heads of 64, 8 chained twin-slot steps with commit between."""
    return make_case("tiny", SHAPE_TINY, steps=8, seed=seed)


def qwen08b(seed: int = 0, B: int = 64, twin: bool = True, steps: int = 1, T: int = 1) -> Case:
    """One 0.8B-like GDN layer: 16+16 heads of 128, 6144 conv channels, 257 slot pairs."""
    s = Shape(B=B, T=T, H_k=16, H_v=16, d_k=128, d_v=128, W=4, N=513)
    return make_case("0.8b" if B == 64 else f"sweep-B{B}", s, steps=steps, twin=twin, seed=seed)


def qwen9b(seed: int = 0, layers: int = 24) -> Case:
    """9B-like: 16 key heads shared by 32 value heads, 24 layers on separate 129-slot pools."""
    return make_case("9b", SHAPE_9B, layers=layers, seed=seed)


def padded(seed: int = 0, T: int = 1, twin: bool = True) -> Case:
    """128-row bucket: 46 real rows first, 82 padding rows on slot 0 (decode-first order)."""
    s = Shape(B=PADDED_ROWS, T=T, H_k=16, H_v=16, d_k=128, d_v=128, W=4, N=513)
    return make_case(f"padded-T{T}", s, real_rows=PADDED_REAL, twin=twin, seed=seed)


def small(B: int, T: int, H_k: int, H_v: int, d: int, N: int | None = None, *, twin: bool = True,
          real_rows: int | None = None, steps: int = 1, seed: int = 0, d_v: int | None = None) -> Case:
    """A small case of any shape for parity tests (pool sized to the rows unless N is given)."""
    dv = d if d_v is None else d_v
    rr = B if real_rows is None else real_rows
    n = N if N is not None else 2 * max(rr, 1) + 1
    s = Shape(B=B, T=T, H_k=H_k, H_v=H_v, d_k=d, d_v=dv, W=4, N=n)
    return make_case(f"small-B{B}-T{T}-{H_k}x{H_v}-d{d}", s, steps=steps, real_rows=rr, twin=twin, seed=seed)


# ------------------------------------------------------------------ packed prompts (prefill)

@dataclass
class PrefillCase:
    shape: Shape             # B = sequences, T = total tokens
    pool: Pool               # read_slot holds each sequence's slot (0: padding)
    x: np.ndarray            # [T][C] bf16 bits
    g: np.ndarray            # [T][H_v] fp32
    beta: np.ndarray         # [T][H_v] fp32
    cu_seqlens: np.ndarray   # [B+1] int32


def prefill(lengths, *, H_k: int, H_v: int, d: int, d_v: int | None = None, pad: tuple = (), seed: int = 0,
            N: int | None = None) -> PrefillCase:
    """Packed prompts of the given lengths (one slot each, a random permutation of
    slot pairs' first slots); sequences whose index is in `pad` sit on slot 0.
    Values drawn as for a decode step, per token."""
    dv = d if d_v is None else d_v
    B = len(lengths)
    n = N if N is not None else 2 * B + 1
    total = int(sum(lengths))
    s = Shape(B=B, T=total, H_k=H_k, H_v=H_v, d_k=d, d_v=dv, W=4, N=n)
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = draw_pool(rng, s, B)
    for b in pad:
        pool.read_slot[b] = 0
        pool.write_slot[b] = 0
    x = bf16_bits(rng.standard_normal((total, s.C), dtype=np.float32))
    g = (-_softplus(rng.standard_normal((total, H_v)))).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((total, H_v))).astype(np.float32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return PrefillCase(s, pool, x, g, beta, cu)
