"""CPU oracle for the affine-Q4 MoE feed-forward hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports or calls this
module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

What it computes: the exact mathematical result on the given bfloat16 inputs
and the exactly dequantized weights, in float64, with no intermediate rounding.
Floating-point parity is judged against these values.

Sources (web pages; no code is taken from them):

* "lily" README (pplx-garden), introduction and "Requirements": the weights
  are MLX affine 4-bit with group size 64, and decoding is always greedy.
* "lily-qwen3.8-flash-next" README, "How the speed was achieved": decode is a
  bandwidth-bound stream of 4-bit weights; prefill runs the expert GEMM on
  token-to-expert groups.
* "2026-09-02: Lily vs MLX 0.32.2", "Measurement contract": batch 1, greedy
  argmax, prompts processed in 2,048-token chunks; "Hardware and software": the
  checkpoint is affine Q4 with group 64, with affine Q8 exceptions.
* "lily-qwen3.8-flash-next" README, "The model": the q4-xl checkpoint keeps the
  shared expert, the LM head and the embedding at 8 bits.

The pages never spell out the arithmetic, so it follows these plain readings
(each is listed with its reason in the design notes):

* A 4-bit code for column j of a row sits in 32-bit word j//8 at bits
  [4*(j%8), 4*(j%8)+4) (least significant nibble first, as MLX packs).
* One (scale, bias) pair per 64 consecutive columns of a row; the weight is
  ``w = scale * q + bias``.  8-bit matrices (the checkpoint's 8-bit exceptions)
  hold byte j%4 of word j//4, least significant byte first, with the same
  groups and formula.
* Routing: logits = router . x, softmax over all experts, keep the top_k
  largest (descending, equal logits ordered by lower expert id), renormalise
  the kept probabilities to sum to one.
* Expert: ``down . (silu(gate . x) * (up . x))`` with silu(z) = z / (1 + e^-z);
  the shared expert is added with weight 1, or with weight sigmoid(g . x) when the
  layer carries a shared-expert gate vector g.
* Permutation: stable counting sort of the (token, slot) rows by expert id.
* LM head: logits = W . x, greedy id = argmax with the lowest index on ties.
* Residual stream (layers chained in a decode step): the next input is
  bfloat16(x + y), round to nearest, ties to even.

Every function is pinned by CPU tests against hand-computed examples, closed
forms, library routines or brute force; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

GROUP = 64


# ----------------------------------------------------------------- formats --

def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: bfloat16 is the top half of a float32)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def unpack_codes(codes, k: int) -> np.ndarray:
    """Nibble codes q[n][j] in 0..15 for j < k, least significant nibble first."""
    codes = np.asarray(codes, dtype=np.uint32)
    j = np.arange(k)
    words = codes[..., j // 8]
    shifts = (4 * (j % 8)).astype(np.uint32)
    return ((words >> shifts) & np.uint32(0xF)).astype(np.int64)


def unpack_codes8(codes, k: int) -> np.ndarray:
    """8-bit codes q[n][j] in 0..255 for j < k: byte j%4 of word j//4, least significant first."""
    codes = np.asarray(codes, dtype=np.uint32)
    j = np.arange(k)
    words = codes[..., j // 4]
    shifts = (8 * (j % 4)).astype(np.uint32)
    return ((words >> shifts) & np.uint32(0xFF)).astype(np.int64)


def code_bits(codes, k: int) -> int:
    """4 or 8: the code width of a matrix whose rows hold k columns in codes.shape[-1] words."""
    words = np.asarray(codes).shape[-1]
    if words * 8 == k:
        return 4
    if words * 4 == k:
        return 8
    raise ValueError(f"{words} code words per row do not hold {k} columns at 4 or 8 bits")


def dequantize(codes, scales, biases, k: int) -> np.ndarray:
    """Affine dequantization w = scale*q + bias, one (scale, bias) per 64 columns (exact in fp64);
    q is the 4-bit or 8-bit code, by the width of ``codes``."""
    q = (unpack_codes(codes, k) if code_bits(codes, k) == 4 else unpack_codes8(codes, k)).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases), GROUP, axis=-1)
    return s * q + b


# ---------------------------------------------------------- GEMV and GEMM --

def q4_gemv(codes, scales, biases, x_bits) -> np.ndarray:
    """y = W x for one bfloat16 vector x (decode-form product)."""
    x = bf16_to_f64(x_bits)
    return dequantize(codes, scales, biases, x.shape[-1]) @ x


def q4_gemm(codes, scales, biases, X_bits) -> np.ndarray:
    """Y[m][n] = sum_j X[m][j] W[n][j] for bfloat16 rows X (prefill-form product)."""
    X = bf16_to_f64(X_bits)
    return X @ dequantize(codes, scales, biases, X.shape[-1]).T


# ---------------------------------------------------------------- routing --

def router_logits(router_bits, X_bits) -> np.ndarray:
    """logits[t][e] = sum_h router[e][h] X[t][h]."""
    X = np.atleast_2d(bf16_to_f64(X_bits))
    return X @ bf16_to_f64(router_bits).T


def topk_from_logits(logits, top_k: int):
    """Top-k selection and renormalised softmax weights from a row (or rows) of logits.

    Order: descending logit, equal logits by lower expert id.  Weights: the
    softmax probabilities of the kept experts divided by their sum.
    """
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T, E = L.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-L[t, e], e))[:top_k]
        p = np.exp(L[t] - L[t].max())
        p = p / p.sum()
        kept = p[order]
        ids[t] = order
        w[t] = kept / kept.sum()
    return ids, w


def route_topk(router_bits, X_bits, top_k: int):
    """(ids int32[T][k], weights f64[T][k], logits f64[T][E]) for bfloat16 token rows."""
    logits = router_logits(router_bits, X_bits)
    ids, w = topk_from_logits(logits, top_k)
    return ids, w, logits


def weights_for_ids(logits_row, ids_row) -> np.ndarray:
    """Renormalised softmax weights of a given expert set (used when a near-tie picks another set)."""
    L = np.asarray(logits_row, dtype=np.float64)
    p = np.exp(L - L.max())
    p = p / p.sum()
    kept = p[np.asarray(ids_row)]
    return kept / kept.sum()


def boundary_gap(logits_row, top_k: int) -> float:
    """Logit gap between the k-th and (k+1)-th ranked experts (inf when k equals the expert count)."""
    v = np.sort(np.asarray(logits_row, dtype=np.float64))[::-1]
    return float(v[top_k - 1] - v[top_k]) if top_k < v.size else float("inf")


# ------------------------------------------------------------ permutation --

def permute(ids, n_experts: int):
    """Stable counting sort of the rows r = t*k + slot by expert id.

    Returns (offsets int32[E+1], sorted_rows int32[T*k], inv_rows int32[T*k])
    with sorted_rows listing, expert by expert, the rows in increasing r, and
    inv_rows[sorted_rows[p]] = p.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:                       # histogram
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):           # exclusive scan
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_rows = np.empty(flat.size, dtype=np.int64)
    for r, e in enumerate(flat):         # stable scatter, rows in increasing order
        sorted_rows[cursor[e]] = r
        cursor[e] += 1
    inv = np.empty(flat.size, dtype=np.int64)
    inv[sorted_rows] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_rows.astype(np.int32), inv.astype(np.int32)


# ------------------------------------------------------------- expert FFN --

def silu(z):
    """silu(z) = z / (1 + e^-z), the SwiGLU gate activation; for z < 0 evaluated as the
    equal z e^z / (1 + e^z), which never forms e^-z (that overflows below -709)."""
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(-np.abs(z))                    # e^-|z| in (0, 1]
    return np.where(z >= 0, z / (1.0 + ez), z * ez / (1.0 + ez))


def swiglu(g, u):
    """a = silu(g) * u."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def expert_ffn(expert, X) -> np.ndarray:
    """down . (silu(gate . x) * (up . x)) for float64 rows X[m][hidden] (or one vector)."""
    (gc, gs, gb), (uc, us, ub), (dc, ds, db) = expert
    X = np.asarray(X, dtype=np.float64)
    hidden = X.shape[-1]
    Wg = dequantize(gc, gs, gb, hidden)
    Wu = dequantize(uc, us, ub, hidden)
    a = swiglu(X @ Wg.T, X @ Wu.T)
    Wd = dequantize(dc, ds, db, a.shape[-1])
    return a @ Wd.T


def layer_router_logits(layer, X_bits) -> np.ndarray:
    """The layer's router logits [T][E]: the 8-bit router ``layer.router_q8`` when the layer
    has one (the checkpoint's affine Q8 router-gate exception), else the bf16 router."""
    rq8 = getattr(layer, "router_q8", None)
    if rq8 is None:
        return router_logits(layer.router, X_bits)
    X = np.atleast_2d(bf16_to_f64(X_bits))
    return X @ dequantize(*rq8, X.shape[-1]).T


def sigmoid(z):
    """1 / (1 + e^-z), evaluated without forming e^-z for z < 0 (e^z / (1 + e^z) there)."""
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))


def shared_gate(layer, X_bits) -> np.ndarray:
    """Weight of the shared expert per token: sigmoid(sh_gate_w . x) when the layer carries a
    shared-expert gate vector, else 1."""
    X = np.atleast_2d(bf16_to_f64(X_bits))
    w = getattr(layer, "sh_gate_w", None)
    if w is None:
        return np.ones(X.shape[0])
    return sigmoid(X @ bf16_to_f64(w))


def moe_ffn_token(layer, x_bits, ids=None):
    """One token through the MoE layer (the decode form).

    ``layer`` exposes ``router``, ``top_k``, ``n_experts``, ``has_shared`` and
    ``expert(e)`` -> ((codes, scales, biases) x 3 for gate/up/down), with
    e == n_experts naming the shared expert.  When ``ids`` is given, those
    experts are used instead of the top-k choice (weights are recomputed for
    them from the logits).  Returns (y f64[hidden], ids, weights, logits).
    """
    x = bf16_to_f64(x_bits)
    logits = layer_router_logits(layer, x_bits)[0]
    if ids is None:
        sel, w = topk_from_logits(logits, layer.top_k)
        sel, w = sel[0], w[0]
    else:
        sel = np.asarray(ids, dtype=np.int32)
        w = weights_for_ids(logits, sel)
    y = np.zeros(x.shape[-1], dtype=np.float64)
    for e, we in zip(sel, w):
        y += we * expert_ffn(layer.expert(int(e)), x)
    if layer.has_shared:
        y += shared_gate(layer, x_bits)[0] * expert_ffn(layer.expert(layer.n_experts), x)
    return y, sel, w, logits


def moe_ffn_prefill(layer, X_bits, ids=None):
    """Every token of a chunk through the MoE layer.

    The result is, row by row, ``moe_ffn_token``; it is evaluated one expert
    at a time over the tokens that chose it (the permutation only changes the
    order of evaluation).  When ``ids`` is given it replaces the top-k choice.
    Returns (Y f64[T][hidden], ids, weights, logits).
    """
    X = np.atleast_2d(bf16_to_f64(X_bits))
    T = X.shape[0]
    logits = layer_router_logits(layer, X_bits)
    if ids is None:
        sel, w = topk_from_logits(logits, layer.top_k)
    else:
        sel = np.asarray(ids, dtype=np.int32).reshape(T, -1)
        w = np.stack([weights_for_ids(logits[t], sel[t]) for t in range(T)])
    Y = np.zeros_like(X)
    for e in range(layer.n_experts):
        tok, slot = np.nonzero(sel == e)
        if tok.size:
            Y[tok] += w[tok, slot][:, None] * expert_ffn(layer.expert(e), X[tok])
    if layer.has_shared:
        Y += shared_gate(layer, X_bits)[:, None] * expert_ffn(layer.expert(layer.n_experts), X)
    return Y, sel, w, logits


# ------------------------------------------------------- residual stream --

def f64_to_bf16_rne(v) -> np.ndarray:
    """Nearest bfloat16 to each float64 value, ties to an even significand, as bit patterns.

    From the definition: bfloat16 keeps 8 significant bits, so v = m * 2**e with
    m in [0.5, 1) rounds to rint(m * 256) * 2**(e - 8), where rint rounds halves
    to even.  Finite values in the normal range of bfloat16 only."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(m * 256.0), e - 8)     # exact in float64 and in float32
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def residual_next(x_bits, y) -> np.ndarray:
    """The next layer's input on a residual stream: bfloat16(x + y), rounded once from
    the exact sum (x bfloat16 bits, y the layer's float64 output)."""
    return f64_to_bf16_rne(bf16_to_f64(x_bits) + np.asarray(y, dtype=np.float64))


# ---------------------------------------------------------------- LM head --

def lmhead_logits(codes, scales, biases, X_bits, rows_per_chunk: int = 8192) -> np.ndarray:
    """logits[b][n] = W[n] . X[b], dequantizing the rows chunk by chunk to bound memory."""
    X = np.atleast_2d(bf16_to_f64(X_bits))
    n = codes.shape[0]
    out = np.empty((X.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        W = dequantize(codes[r0:r1], scales[r0:r1], biases[r0:r1], X.shape[1])
        out[:, r0:r1] = X @ W.T
    return out


def greedy_argmax(logits):
    """(ids, max, gap) per row: first index of the maximum, its value, and top1 - top2."""
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    ids = np.argmax(L, axis=1).astype(np.int32)         # first occurrence on ties
    top = L[np.arange(L.shape[0]), ids]
    if L.shape[1] > 1:
        second = np.partition(L, -2, axis=1)[:, -2]
    else:
        second = np.full(L.shape[0], -np.inf)
    return ids, top, top - second


def lmhead_argmax(codes, scales, biases, X_bits):
    return greedy_argmax(lmhead_logits(codes, scales, biases, X_bits))
