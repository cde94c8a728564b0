"""Seeded synthetic inputs for the affine-Q4 mixture-of-experts hot path.

Every tensor here is drawn from numpy ``SeedSequence`` substreams and returned
as raw bit patterns: uint32 words holding eight 4-bit codes each, and uint16
words holding bfloat16 values.  Both the HIP path and the CPU oracle read these
same arrays; this module holds none of the method's arithmetic (no unpacking,
no dequantization, no products), only the recipe that makes the inputs.

Recipe (the pages give the weight format, MLX affine 4-bit with group size 64
(lily README, introduction and "Requirements"), but no distributions):

* codes: uniform uint32 words, i.e. eight i.i.d. uniform nibbles per word;
* scales: |N(0, 0.02)|, rounded to bfloat16;
* biases: ``bf16(-8 * scale_bf16 + N(0, 0.002))``, so that dequantized weights
  are roughly centred on zero;
* router: N(0, 0.02) in bfloat16; hidden vectors and token rows: N(0, 1) in
  bfloat16.

Rounding to bfloat16 is round-to-nearest-even from float32 (float64 draws are
first rounded to float32).  Substreams: a Q4 matrix uses
``SeedSequence([seed, layer, expert, matrix])`` with matrix 0/1/2 for
gate/up/down and expert ``n_experts`` for the shared expert; the router uses
``[seed, layer, ROUTER_STREAM]``; a decode hidden vector uses
``[seed, X_STREAM + step, layer]``; a block of token rows uses
``[seed, X_STREAM + index, 0]``.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

GROUP = 64
X_STREAM = 10_000
ROUTER_STREAM = 20_000
GATE, UP, DOWN = 0, 1, 2

# Shapes of the 35B-total / 3B-active MoE layer used throughout.
HIDDEN = 2048
INTER = 512
N_EXPERTS = 256
TOP_K = 8
VOCAB = 151_936


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def to_bf16_bits(a) -> np.ndarray:
    """Round float values to bfloat16 (nearest-even, via float32); return uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def q4_matrix(seed: int, layer: int, expert: int, matrix: int, n: int, k: int):
    """One affine-Q4 matrix of n rows and k columns.

    Returns ``(codes uint32[n][k/8], scales uint16[n][k/64], biases uint16[n][k/64])``.
    """
    if k % GROUP:
        raise ValueError("k must be a multiple of 64")
    rng = _rng(seed, layer, expert, matrix)
    codes = rng.integers(0, 1 << 32, size=(n, k // 8), dtype=np.uint32)
    scales = to_bf16_bits(np.abs(rng.normal(0.0, 0.02, size=(n, k // GROUP))))
    noise = rng.normal(0.0, 0.002, size=(n, k // GROUP))
    biases = to_bf16_bits(-8.0 * _bf16_bits_to_f32(scales).astype(np.float64) + noise)
    return codes, scales, biases


def q8_matrix(seed: int, layer: int, expert: int, matrix: int, n: int, k: int, scale_std: float = 0.02 / 16):
    """One affine-Q8 matrix of n rows and k columns: 8-bit codes, 4 per uint32 word.

    Codes are uniform bytes; scales ``|N(0, scale_std)|`` and biases ``-128*scale +
    N(0, 0.002)`` (the default scale makes the weights span the range of the 4-bit ones).
    Returns ``(codes uint32[n][k/4], scales uint16[n][k/64], biases uint16[n][k/64])``.
    """
    if k % GROUP:
        raise ValueError("k must be a multiple of 64")
    rng = _rng(seed, layer, expert, matrix, 8)
    codes = rng.integers(0, 1 << 32, size=(n, k // 4), dtype=np.uint32)
    scales = to_bf16_bits(np.abs(rng.normal(0.0, scale_std, size=(n, k // GROUP))))
    noise = rng.normal(0.0, 0.002, size=(n, k // GROUP))
    biases = to_bf16_bits(-128.0 * _bf16_bits_to_f32(scales).astype(np.float64) + noise)
    return codes, scales, biases


def router(seed: int, layer: int, n_experts: int = N_EXPERTS, hidden: int = HIDDEN):
    """bfloat16 router matrix [n_experts][hidden], N(0, 0.02)."""
    return to_bf16_bits(_rng(seed, layer, ROUTER_STREAM).normal(0.0, 0.02, size=(n_experts, hidden)))


def hidden_vector(seed: int, step: int, layer: int, hidden: int = HIDDEN):
    """One decode-step input of a layer: bfloat16 [hidden], N(0, 1)."""
    return to_bf16_bits(_rng(seed, X_STREAM + step, layer).standard_normal(hidden))


def token_rows(seed: int, rows: int, hidden: int = HIDDEN, index: int = 0):
    """A block of token rows: bfloat16 [rows][hidden], N(0, 1)."""
    return to_bf16_bits(_rng(seed, X_STREAM + index, 0).standard_normal((rows, hidden)))


class Q4Stack:
    """``count`` stacked affine matrices of shape n x k (4-bit codes, or 8-bit with
    bits = 8), as three contiguous arrays."""

    def __init__(self, count: int, n: int, k: int, bits: int = 4):
        self.count, self.n, self.k = count, n, k
        self.codes = np.empty((count, n, k * bits // 32), dtype=np.uint32)
        self.scales = np.empty((count, n, k // GROUP), dtype=np.uint16)
        self.biases = np.empty((count, n, k // GROUP), dtype=np.uint16)

    def fill(self, i: int, mat) -> None:
        self.codes[i], self.scales[i], self.biases[i] = mat

    def matrix(self, i: int):
        return self.codes[i], self.scales[i], self.biases[i]

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes + self.biases.nbytes


class MoELayer:
    """Weights of one MoE feed-forward layer (routed experts plus an optional shared one).

    ``gate``/``up`` stack ``[n_experts][inter][hidden/8]`` words, ``down`` stacks
    ``[n_experts][hidden][inter/8]``; ``sh_gate``/``sh_up``/``sh_down`` hold the
    shared expert (count 1) or are None.
    """

    def __init__(self, hidden, inter, n_experts, top_k, router_bits, gate, up, down,
                 sh_gate=None, sh_up=None, sh_down=None, router_q8=None, sh_gate_w=None):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.router = router_bits
        self.router_q8 = router_q8  # (codes, scales, biases) of an 8-bit router, replacing `router`
        self.sh_gate_w = sh_gate_w  # bf16 [hidden]: the shared expert's weight is sigmoid(sh_gate_w . x)
        self.gate, self.up, self.down = gate, up, down
        self.sh_gate, self.sh_up, self.sh_down = sh_gate, sh_up, sh_down

    @property
    def has_shared(self) -> bool:
        return self.sh_gate is not None

    def expert(self, e: int):
        """(gate, up, down) matrices of routed expert e, or of the shared expert when e == n_experts."""
        if e == self.n_experts:
            return self.sh_gate.matrix(0), self.sh_up.matrix(0), self.sh_down.matrix(0)
        return self.gate.matrix(e), self.up.matrix(e), self.down.matrix(e)

    @property
    def nbytes(self) -> int:
        total = self.router.nbytes + self.gate.nbytes + self.up.nbytes + self.down.nbytes
        if self.has_shared:
            total += self.sh_gate.nbytes + self.sh_up.nbytes + self.sh_down.nbytes
        return total


def moe_layer(seed: int, layer: int = 0, hidden: int = HIDDEN, inter: int = INTER,
              n_experts: int = N_EXPERTS, top_k: int = TOP_K, shared: bool = True,
              threads: int | None = None, router_bits: int = 16, shared_gate: bool = False,
              shared_bits: int = 4) -> MoELayer:
    """Generate one MoE layer; experts are drawn in parallel threads (numpy releases the GIL).
    router_bits = 8 adds an affine-Q8 router (weights of about the bf16 router's spread,
    0.02) that replaces the bf16 one.  shared_gate adds a bf16 shared-expert gate vector,
    N(0, 0.02), stream [seed, layer, 20001].  shared_bits = 8 draws the shared expert as
    affine-Q8 matrices (q8_matrix streams, weights of about the 4-bit experts' spread)."""
    gate = Q4Stack(n_experts, inter, hidden)
    up = Q4Stack(n_experts, inter, hidden)
    down = Q4Stack(n_experts, hidden, inter)
    sh_shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    sh = [Q4Stack(1, n, k, bits=shared_bits) for n, k in sh_shapes] if shared else [None] * 3

    def one(e: int) -> None:
        if e == n_experts and shared_bits == 8:
            for m, (n, k), which in zip(sh, sh_shapes, (GATE, UP, DOWN)):
                m.fill(0, q8_matrix(seed, layer, e, which, n, k))
            return
        g = q4_matrix(seed, layer, e, GATE, inter, hidden)
        u = q4_matrix(seed, layer, e, UP, inter, hidden)
        d = q4_matrix(seed, layer, e, DOWN, hidden, inter)
        if e == n_experts:
            sh[0].fill(0, g), sh[1].fill(0, u), sh[2].fill(0, d)
        else:
            gate.fill(e, g), up.fill(e, u), down.fill(e, d)

    ids = list(range(n_experts + (1 if shared else 0)))
    workers = threads or min(16, os.cpu_count() or 1)
    if workers > 1 and len(ids) > 4:
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(one, ids))
    else:
        for e in ids:
            one(e)
    rq8 = q8_matrix(seed, layer, ROUTER_STREAM, 0, n_experts, hidden, scale_std=0.02 / 74) if router_bits == 8 else None
    gw = to_bf16_bits(_rng(seed, layer, ROUTER_STREAM + 1).normal(0.0, 0.02, size=hidden)) if shared_gate else None
    return MoELayer(hidden, inter, n_experts, top_k, router(seed, layer, n_experts, hidden),
                    gate, up, down, *sh, router_q8=rq8, sh_gate_w=gw)


def lm_head(seed: int = 4, rows: int = VOCAB, hidden: int = HIDDEN, bits: int = 4):
    """LM-head-shaped affine matrix (rows x hidden), 4-bit or 8-bit codes."""
    return (q8_matrix if bits == 8 else q4_matrix)(seed, 0, 0, 0, rows, hidden)


def fnv1a64(values) -> int:
    """64-bit FNV-1a over the little-endian bytes of an int32 array (a determinism digest)."""
    h = 0xCBF29CE484222325
    for byte in np.ascontiguousarray(np.asarray(values, dtype=np.int32).ravel()).view(np.uint8).tolist():
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h
