"""Pins for the CPU oracle: hand-computed examples, closed forms, exact rational
brute force, library routines and invariants.  Each would fail on a plausible
slip in the oracle (nibble order, group index, sign, transposed operand,
softmax scope, tie order, instability of the sort)."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits_of(value: float) -> int:
    """bfloat16 bits of a value that bfloat16 holds exactly (checked)."""
    bits = struct.unpack(">I", struct.pack(">f", value))[0]
    assert bits & 0xFFFF == 0, value
    return bits >> 16


def _pack_nibbles(q_rows):
    """Independent packer: element j of a row goes to word j//8, nibble j%8 (LSB first)."""
    out = []
    for row in q_rows:
        words = []
        for w in range(len(row) // 8):
            acc = 0
            for i in range(8):
                acc += int(row[8 * w + i]) * (16 ** i)
            words.append(acc)
        out.append(words)
    return np.array(out, dtype=np.uint32)


# ------------------------------------------------------------------ a0 ------

def test_dequant_hand_example():
    g = _golden("dequant_hand_example.json")
    codes = np.array([[int(h, 16) for h in g["codes_hex"]]], dtype=np.uint32)
    scales = np.array([[int(h, 16) for h in g["scales_hex"]]], dtype=np.uint16)
    biases = np.array([[int(h, 16) for h in g["biases_hex"]]], dtype=np.uint16)
    assert list(orc.bf16_to_f64(scales[0])) == g["scale_values"]
    assert list(orc.bf16_to_f64(biases[0])) == g["bias_values"]
    exp = g["expected"]
    q = orc.unpack_codes(codes, g["k"])[0]
    assert list(q[:16]) == exp["q_first_16"]
    assert np.all(q[16:64] == exp["q_16_to_63"]) and np.all(q[64:] == exp["q_64_to_127"])
    W = orc.dequantize(codes, scales, biases, g["k"])[0]
    assert W[13] == exp["w_13"] and W[63] == exp["w_63"] and W[64] == exp["w_64"]
    assert W[:64].sum() == exp["group0_sum"] and W[64:].sum() == exp["group1_sum"]
    x = np.full(g["k"], 0x3F80, dtype=np.uint16)
    assert orc.q4_gemv(codes, scales, biases, x)[0] == exp["y"]


def test_one_hot_x_returns_a_column():
    codes, scales, biases = synth.q4_matrix(7, 0, 0, 0, 5, 192)
    q = orc.unpack_codes(codes, 192)
    for j in (0, 7, 8, 63, 64, 100, 191):
        x = np.zeros(192, dtype=np.uint16)
        x[j] = 0x3F80
        y = orc.q4_gemv(codes, scales, biases, x)
        s = orc.bf16_to_f64(scales[:, j // 64])
        b = orc.bf16_to_f64(biases[:, j // 64])
        np.testing.assert_array_equal(y, s * q[:, j] + b)


@pytest.mark.parametrize("n,k,seed", [(1, 64, 0), (3, 64, 1), (2, 128, 2), (3, 192, 3)])
def test_gemv_exact_rational_brute_force(n, k, seed):
    """y from Fractions on an independently packed matrix equals the fp64 oracle exactly."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(n, k))
    dy = [0.5, 0.25, 0.125, 0.75, 1.5, 0.0625, 2.0, -0.375]     # exact in bfloat16
    s = rng.choice(dy[:7], size=(n, k // 64))
    b = rng.choice(dy, size=(n, k // 64)) * -1.0
    x = rng.choice([-2.0, -1.0, -0.5, 0.0, 0.25, 1.0, 3.0], size=k)
    codes = _pack_nibbles(q)
    scales = np.array([[_bf16_bits_of(v) for v in r] for r in s], dtype=np.uint16)
    biases = np.array([[_bf16_bits_of(v) for v in r] for r in b], dtype=np.uint16)
    xb = np.array([_bf16_bits_of(v) for v in x], dtype=np.uint16)
    expect = []
    for r in range(n):
        acc = Fraction(0)
        for j in range(k):
            w = Fraction(s[r, j // 64]) * int(q[r, j]) + Fraction(b[r, j // 64])
            acc += w * Fraction(x[j])
        expect.append(float(acc))
    got = orc.q4_gemv(codes, scales, biases, xb)
    assert list(got) == expect
    # the GEMM form is the same contraction with rows of X
    X = np.stack([xb, xb[::-1].copy()])
    Y = orc.q4_gemm(codes, scales, biases, X)
    assert list(Y[0]) == expect
    np.testing.assert_array_equal(Y[1], orc.q4_gemv(codes, scales, biases, X[1]))


def test_unpack_roundtrips_independent_packer():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(4, 256))
    np.testing.assert_array_equal(orc.unpack_codes(_pack_nibbles(q), 256), q)


# ------------------------------------------------------------- a1 / a2 ------

def _router_eye(logits):
    """Router = identity and x = logits, so that the router logits are exactly the given values."""
    E = len(logits)
    router = np.zeros((E, E), dtype=np.uint16)
    for e in range(E):
        router[e, e] = 0x3F80
    x = np.array([_bf16_bits_of(v) for v in logits], dtype=np.uint16)
    return router, x


def test_route_worked_example():
    g = _golden("route_worked_example.json")
    router, x = _router_eye(g["logits"])
    ids, w, logits = orc.route_topk(router, x, g["top_k"])
    assert list(logits[0]) == g["logits"]
    assert list(ids[0]) == g["expected_ids"]
    np.testing.assert_allclose(w[0], g["expected_weights"], rtol=0, atol=1e-15)
    assert w[0][0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), abs=1e-15)


def test_route_tie_order_and_descending():
    router, x = _router_eye([1.0, 3.0, 3.0, 0.0, 3.0])
    ids, w, _ = orc.route_topk(router, x, 3)
    assert list(ids[0]) == [1, 2, 4]          # equal logits: lower expert id first
    np.testing.assert_allclose(w[0], [1 / 3] * 3, atol=1e-15)
    ids1, _, _ = orc.route_topk(router, x, 1)
    assert list(ids1[0]) == [1]


def test_route_matches_scipy_softmax_and_invariants():
    E, H, T, k = 32, 128, 6, 5
    router = synth.router(11, 0, E, H)
    X = synth.token_rows(11, T, H)
    ids, w, logits = orc.route_topk(router, X, k)
    p = scipy.special.softmax(logits, axis=1)
    for t in range(T):
        assert len(set(ids[t])) == k and ids[t].min() >= 0 and ids[t].max() < E
        assert np.all(np.diff(logits[t, ids[t]]) <= 0)
        # the kept set is exactly the k largest
        assert logits[t, ids[t]].min() >= np.sort(logits[t])[::-1][k - 1]
        np.testing.assert_allclose(w[t], p[t, ids[t]] / p[t, ids[t]].sum(), rtol=1e-13)
        assert abs(w[t].sum() - 1.0) < 1e-12 and np.all(w[t] > 0)
    # scope: softmax over all experts then renormalised == softmax over the kept logits
    np.testing.assert_allclose(w, scipy.special.softmax(np.take_along_axis(logits, ids.astype(np.int64), 1), axis=1), rtol=1e-13)


def test_router_logits_orientation():
    """logits[e] = router[e] . x (a transposed router would fail)."""
    router = np.zeros((3, 64), dtype=np.uint16)
    router[2, 5] = _bf16_bits_of(2.0)
    router[0, 1] = _bf16_bits_of(-1.0)
    x = np.zeros(64, dtype=np.uint16)
    x[5] = _bf16_bits_of(3.0)
    x[1] = _bf16_bits_of(0.5)
    assert list(orc.router_logits(router, x)[0]) == [-0.5, 0.0, 6.0]


# ------------------------------------------------------------------ a3 ------

def test_permute_worked_example():
    g = _golden("permute_worked_example.json")
    off, rows, inv = orc.permute(np.array(g["ids"]), g["n_experts"])
    assert list(off) == g["expected_offsets"]
    assert list(rows) == g["expected_sorted_rows"]
    assert list(inv) == g["expected_inv_rows"]


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 5, 1), (50, 4, 16, 2), (300, 8, 64, 3)])
def test_permute_invariants_and_brute_force(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    off, rows, inv = orc.permute(ids, E)
    flat = ids.reshape(-1)
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
    assert sorted(rows.tolist()) == list(range(T * k))                  # conservation
    assert list(rows) == sorted(range(T * k), key=lambda r: (flat[r], r))
    np.testing.assert_array_equal(rows, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(inv[rows], np.arange(T * k))
    np.testing.assert_array_equal(np.bincount(flat, minlength=E), np.diff(off))
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)      # stable in segments


# ------------------------------------------------------------------ a5 ------

def test_swiglu_closed_form_and_torch():
    for c in _golden("swiglu_closed_form.json")["cases"]:
        assert orc.swiglu(c["g"], c["u"]) == pytest.approx(c["a"], abs=1e-15)
    z = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(orc.silu(z), ref, rtol=1e-14, atol=1e-300)


# --------------------------------------------------------------- a4-a7 ------

def _tiny_layer(seed, hidden=128, inter=64, E=4, top_k=2, shared=True, zero_shared=False):
    layer = synth.moe_layer(seed, 0, hidden, inter, E, top_k, shared=shared, threads=1)
    if zero_shared:
        for st in (layer.sh_gate, layer.sh_up, layer.sh_down):
            st.codes[:] = 0
            st.scales[:] = 0
            st.biases[:] = 0
    return layer


def test_ffn_one_hot_route_is_dense_swiglu_mlp():
    """k=1, shared expert zero: the layer is one dense SwiGLU MLP (checked with torch in fp64)."""
    hidden, inter, E = 128, 64, 4
    layer = _tiny_layer(3, hidden, inter, E, top_k=1, zero_shared=True)
    x = synth.hidden_vector(3, 0, 0, hidden)
    layer.router[:] = 0
    layer.router[2] = x                     # logit of expert 2 = |x|^2 > 0, others 0
    y, ids, w, _ = orc.moe_ffn_token(layer, x)
    assert list(ids) == [2] and w[0] == 1.0
    (gc, gs, gb), (uc, us, ub), (dc, ds, db) = layer.expert(2)
    Wg = torch.from_numpy(orc.dequantize(gc, gs, gb, hidden))
    Wu = torch.from_numpy(orc.dequantize(uc, us, ub, hidden))
    Wd = torch.from_numpy(orc.dequantize(dc, ds, db, inter))
    xt = torch.from_numpy(orc.bf16_to_f64(x))
    mlp = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, Wg)) * torch.nn.functional.linear(xt, Wu), Wd)
    np.testing.assert_allclose(y, mlp.numpy(), rtol=1e-12, atol=1e-12)


def test_ffn_weighted_sum_and_shared_expert():
    """y = sum_i w_i FFN_{e_i}(x) + FFN_shared(x), checked term by term with torch fp64."""
    hidden, inter, E, k = 128, 64, 6, 3
    layer = _tiny_layer(4, hidden, inter, E, top_k=k)
    x = synth.hidden_vector(4, 0, 0, hidden)
    y, ids, w, logits = orc.moe_ffn_token(layer, x)
    xt = torch.from_numpy(orc.bf16_to_f64(x))

    def mlp(e):
        (gc, gs, gb), (uc, us, ub), (dc, ds, db) = layer.expert(e)
        Wg = torch.from_numpy(orc.dequantize(gc, gs, gb, hidden))
        Wu = torch.from_numpy(orc.dequantize(uc, us, ub, hidden))
        Wd = torch.from_numpy(orc.dequantize(dc, ds, db, inter))
        return (Wd @ (torch.nn.functional.silu(Wg @ xt) * (Wu @ xt))).numpy()

    p = scipy.special.softmax(logits)
    expect = sum(p[e] / p[ids].sum() * mlp(e) for e in ids) + mlp(E)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_prefill_rows_equal_decode_and_permutation_equivariance():
    hidden, inter, E, k, T = 128, 64, 8, 3, 9
    layer = _tiny_layer(5, hidden, inter, E, top_k=k)
    X = synth.token_rows(5, T, hidden)
    Y, ids, w, _ = orc.moe_ffn_prefill(layer, X)
    for t in range(T):
        y, i1, w1, _ = orc.moe_ffn_token(layer, X[t])
        np.testing.assert_array_equal(i1, ids[t])
        np.testing.assert_allclose(Y[t], y, rtol=1e-12, atol=1e-12)
    perm = np.random.default_rng(0).permutation(T)
    Yp, _, _, _ = orc.moe_ffn_prefill(layer, X[perm])
    np.testing.assert_allclose(Yp, Y[perm], rtol=1e-12, atol=1e-12)


def test_given_ids_reproduce_topk_result():
    layer = _tiny_layer(6, 128, 64, 8, top_k=2)
    x = synth.hidden_vector(6, 1, 0, 128)
    y, ids, w, _ = orc.moe_ffn_token(layer, x)
    y2, ids2, w2, _ = orc.moe_ffn_token(layer, x, ids=ids)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(w, w2)


def test_boundary_gap_hand_values():
    # ranked logits 2 > 1 > 0 > -1 in scrambled positions: the k-th minus the (k+1)-th
    row = [0.0, 2.0, -1.0, 1.0]
    assert orc.boundary_gap(row, 1) == 1.0          # 2 - 1
    assert orc.boundary_gap(row, 2) == 1.0          # 1 - 0
    assert orc.boundary_gap(row, 3) == 1.0          # 0 - (-1)
    assert orc.boundary_gap([5.0, 0.25, 3.0, 3.0, -7.0], 2) == 0.0  # exact tie across the k / k+1 boundary
    assert orc.boundary_gap([5.0, 0.25, 3.0, 3.5, -7.0], 2) == 0.5  # 3.5 - 3.0, not 5 - 3.5
    assert orc.boundary_gap([5.0, 0.25, 3.0, 3.5, -7.0], 4) == 7.25  # 0.25 - (-7)
    assert orc.boundary_gap(row, 4) == math.inf     # k equal to the expert count: no (k+1)-th expert
    assert orc.boundary_gap([-3.0], 1) == math.inf


@pytest.mark.parametrize("seed", range(6))
def test_boundary_gap_brute_force_distinct(seed):
    # brute force on distinct values: the gap is min(selected) - max(unselected) of the top-k set
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 40))
    row = rng.permutation(np.arange(E, dtype=np.float64) * 0.37 - 5.0) + rng.normal(0, 1e-3, E)
    for k in range(1, E):
        chosen = set()
        for _ in range(k):  # repeated selection of the largest remaining value, no sorting
            best = None
            for e in range(E):
                if e not in chosen and (best is None or row[e] > row[best]):
                    best = e
            chosen.add(best)
        lo_in = min(row[e] for e in chosen)
        hi_out = max(row[e] for e in range(E) if e not in chosen)
        assert orc.boundary_gap(row, k) == lo_in - hi_out
        assert orc.boundary_gap(row, k) > 0


def test_weights_for_ids_off_the_topk_set():
    # logits (2, 1, 0, -1): the set {3, 1} is not the top-2; its weights are
    # e^1 / (e^1 + e^-1) and e^-1 / (e^1 + e^-1) in the given order, i.e. sigma(2), sigma(-2)
    w = orc.weights_for_ids([2.0, 1.0, 0.0, -1.0], [1, 3])
    np.testing.assert_allclose(w, [1 / (1 + math.exp(-2)), 1 / (1 + math.exp(2))], rtol=1e-15)
    w = orc.weights_for_ids([2.0, 1.0, 0.0, -1.0], [3, 1])     # order follows the given ids
    np.testing.assert_allclose(w, [1 / (1 + math.exp(2)), 1 / (1 + math.exp(-2))], rtol=1e-15)
    w = orc.weights_for_ids([2.0, 1.0, 0.0, -1.0], [2, 3, 0])  # three experts: e^0, e^-1, e^2 over their sum
    den = 1 + math.exp(-1) + math.exp(2)
    np.testing.assert_allclose(w, [1 / den, math.exp(-1) / den, math.exp(2) / den], rtol=1e-14)
    # invariance under a constant shift of all logits, and large logits do not overflow
    w2 = orc.weights_for_ids([802.0, 801.0, 800.0, 799.0], [2, 3, 0])
    np.testing.assert_allclose(w2, w, rtol=1e-12)
    # scipy's softmax of the kept logits gives the same (softmax over all, then renormalise)
    rng = np.random.default_rng(3)
    L = rng.normal(0, 1, 64)
    ids = rng.choice(64, 8, replace=False)
    np.testing.assert_allclose(orc.weights_for_ids(L, ids), scipy.special.softmax(L[ids]), rtol=1e-13)


# ------------------------------------------------------------------ a8 ------

def test_lmhead_planted_maximum_and_ties():
    n, k = 300, 128
    codes, scales, biases = synth.q4_matrix(8, 0, 0, 0, n, k)
    x = np.full(k, 0x3F80, dtype=np.uint16)                  # x = ones
    # plant row 123: all codes 15, scale 1, bias 0 -> logit 15*k, far above the rest
    codes[123] = 0xFFFFFFFF
    scales[123] = _bf16_bits_of(1.0)
    biases[123] = 0
    ids, top, gap = orc.lmhead_argmax(codes, scales, biases, x)
    assert ids[0] == 123 and top[0] == 15.0 * k and gap[0] > 1.0
    # an identical row later does not win; an identical row earlier does
    codes[200], scales[200], biases[200] = codes[123], scales[123], biases[123]
    ids, _, gap = orc.lmhead_argmax(codes, scales, biases, x)
    assert ids[0] == 123 and gap[0] == 0.0
    codes[5], scales[5], biases[5] = codes[123], scales[123], biases[123]
    assert orc.lmhead_argmax(codes, scales, biases, x)[0][0] == 5


def test_lmhead_brute_force_batch():
    n, k = 257, 192
    codes, scales, biases = synth.q4_matrix(9, 0, 0, 0, n, k)
    X = synth.token_rows(9, 3, k)
    ids, top, _ = orc.lmhead_argmax(codes, scales, biases, X)
    W = orc.dequantize(codes, scales, biases, k)
    for b in range(3):
        x = orc.bf16_to_f64(X[b])
        vals = [float(np.dot(W[r], x)) for r in range(n)]
        best = max(range(n), key=lambda r: (vals[r], -r))
        assert ids[b] == best and top[b] == pytest.approx(vals[best], rel=1e-12)
    # chunked evaluation equals one-shot
    np.testing.assert_allclose(orc.lmhead_logits(codes, scales, biases, X, rows_per_chunk=50),
                               orc.bf16_to_f64(X) @ W.T, rtol=1e-13)


# ------------------------------------------------------------ residual stream --

def test_bf16_rne_hand_ties():
    """Worked by hand: bfloat16 spacing at 1 is 2^-7, so 1 + 2^-8 is a tie (rounds down to
    the even 1.0), 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even), and
    anything past a tie rounds away from it."""
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,
        -(1.0 + 2.0 ** -8): 0xBF80,
        -(1.0 + 3 * 2.0 ** -8): 0xBF82,
        3.0: 0x4040,
        0.0: 0x0000,
        2.0 - 2.0 ** -9: 0x4000,  # rounds up across the binade boundary
    }
    for v, bits in cases.items():
        assert int(orc.f64_to_bf16_rne(v)) == bits, (v, hex(int(orc.f64_to_bf16_rne(v))), hex(bits))


def test_bf16_rne_brute_force():
    """Against a search over neighbouring bfloat16 patterns: the nearest one, and on an exact
    tie the one with an even last significand bit."""
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.normal(0, 1, 2000), rng.normal(0, 1e3, 500), rng.normal(0, 1e-3, 500),
                        (1 + rng.integers(0, 256, 200) / 128 + 2.0 ** -8) * rng.choice([-1, 1], 200)])
    got = orc.f64_to_bf16_rne(v)
    for val, g in zip(v, got):
        base = int(np.float32(val).view(np.uint32)) >> 16
        best = None
        for cand in range(base - 2, base + 3):
            cv = float(np.uint32((cand & 0xFFFF) << 16).view(np.float32))
            d = abs(cv - val)
            key = (d, cand & 1)  # nearest, then even
            if best is None or key < best[0]:
                best = (key, cand & 0xFFFF)
        assert int(g) == best[1], (val, hex(int(g)), hex(best[1]))


def test_residual_next_exact_cases():
    """x + 0 returns x; sums that are bfloat16 values come back exactly."""
    x = synth.token_rows(8, 1, 256)[0]
    assert np.array_equal(orc.residual_next(x, np.zeros(256)), x)
    xf = orc.bf16_to_f64(x)
    z = orc.residual_next(x, xf)  # x + x = 2x: exact, one binade up
    assert np.array_equal(orc.bf16_to_f64(z), 2 * xf)


# ------------------------------------------------------- 8-bit affine codes --

def _pack_bytes(q_rows):
    """Independent packer: element j of a row goes to byte j%4 of word j//4 (LSB first)."""
    return np.array([[struct.unpack("<I", bytes(int(v) for v in row[4 * w:4 * w + 4]))[0]
                      for w in range(len(row) // 4)] for row in q_rows], dtype=np.uint32)


def test_q8_dequant_hand_example():
    """Worked by hand: one row, K = 128, x = ones.  Group 0 holds q = 0..63 with scale 0.5 and
    bias -4, so w_j = j/2 - 4 (w_13 = 2.5) and the group sums to 1008 - 256 = 752; group 1
    holds q = 255 with scale 0.25 and bias 1, so w = 64.75 and the group sums to 4144."""
    words = [0x03020100 + 0x04040404 * i for i in range(16)] + [0xFFFFFFFF] * 16
    codes = np.array([words], dtype=np.uint32)
    scales = np.array([[0x3F00, 0x3E80]], dtype=np.uint16)
    biases = np.array([[0xC080, 0x3F80]], dtype=np.uint16)
    W = orc.dequantize(codes, scales, biases, 128)
    assert W[0, 13] == 2.5 and W[0, 63] == 27.5 and W[0, 64] == 64.75
    ones = np.full(128, 0x3F80, dtype=np.uint16)
    assert orc.q4_gemv(codes, scales, biases, ones)[0] == 752.0 + 4144.0


def test_q8_unpack_roundtrips_independent_packer_and_width():
    rng = np.random.default_rng(6)
    q = rng.integers(0, 256, size=(3, 192))
    codes = _pack_bytes(q)
    np.testing.assert_array_equal(orc.unpack_codes8(codes, 192), q)
    assert orc.code_bits(codes, 192) == 8 and orc.code_bits(_pack_nibbles(q % 16), 192) == 4
    with pytest.raises(ValueError):
        orc.code_bits(codes, 100)


@pytest.mark.parametrize("n,k,seed", [(3, 64, 0), (2, 128, 1)])
def test_q8_gemv_exact_rational_brute_force(n, k, seed):
    """y from Fractions on an independently packed 8-bit matrix equals the fp64 oracle exactly."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(n, k))
    dy = [0.5, 0.25, 0.125, 0.75, 1.5, 0.0625, 2.0, -0.375]
    s = rng.choice(dy[:7], size=(n, k // 64)) / 64
    b = rng.choice(dy, size=(n, k // 64)) * -1.0
    x = rng.choice([-2.0, -1.0, -0.5, 0.0, 0.25, 1.0, 3.0], size=k)
    codes = _pack_bytes(q)
    scales = np.array([[_bf16_bits_of(v) for v in r] for r in s], dtype=np.uint16)
    biases = np.array([[_bf16_bits_of(v) for v in r] for r in b], dtype=np.uint16)
    xb = np.array([_bf16_bits_of(v) for v in x], dtype=np.uint16)
    expect = []
    for r in range(n):
        acc = Fraction(0)
        for j in range(k):
            acc += (Fraction(s[r, j // 64]) * int(q[r, j]) + Fraction(b[r, j // 64])) * Fraction(x[j])
        expect.append(float(acc))
    assert list(orc.q4_gemv(codes, scales, biases, xb)) == expect
    ids, top, _ = orc.lmhead_argmax(codes, scales, biases, xb)
    assert int(ids[0]) == int(np.argmax(expect)) and top[0] == max(expect)


def test_q8_router_equals_bf16_router_on_shared_values():
    """An 8-bit router whose weights (q - 128) / 128 are also bfloat16 values gives the same
    logits, ids and layer output as the bfloat16 router holding those values."""
    H, I, E, k = 128, 64, 8, 2
    layer = synth.moe_layer(9, 0, H, I, E, k)
    rng = np.random.default_rng(9)
    q = rng.integers(0, 256, size=(E, H))
    layer.router = np.array([[_bf16_bits_of((v - 128) / 128) for v in r] for r in q], dtype=np.uint16)
    x = synth.hidden_vector(9, 0, 0, H)
    y16, ids16, w16, l16 = orc.moe_ffn_token(layer, x)
    scales = np.full((E, H // 64), _bf16_bits_of(1 / 128), dtype=np.uint16)
    biases = np.full((E, H // 64), _bf16_bits_of(-1.0), dtype=np.uint16)
    layer.router_q8 = (_pack_bytes(q), scales, biases)
    y8, ids8, w8, l8 = orc.moe_ffn_token(layer, x)
    np.testing.assert_array_equal(l8, l16)
    np.testing.assert_array_equal(ids8, ids16)
    np.testing.assert_array_equal(y8, y16)
    Y8, _, _, _ = orc.moe_ffn_prefill(layer, np.stack([x, x]))
    np.testing.assert_allclose(Y8[1], y16, rtol=1e-12, atol=1e-12)  # another fp64 summation order


def test_shared_gate_closed_forms():
    """A zero gate vector weighs the shared expert by sigmoid(0) = 1/2 exactly; a gate vector
    along x with a large product weighs it by ~1; the routed part never changes."""
    H, I, E, k = 128, 64, 8, 2
    layer = synth.moe_layer(12, 0, H, I, E, k)
    x = synth.hidden_vector(12, 0, 0, H)
    y1, ids, _, _ = orc.moe_ffn_token(layer, x)
    sh = orc.expert_ffn(layer.expert(E), orc.bf16_to_f64(x))
    layer.sh_gate_w = np.zeros(H, dtype=np.uint16)
    yh, ids_h, _, _ = orc.moe_ffn_token(layer, x)
    np.testing.assert_array_equal(ids_h, ids)
    np.testing.assert_allclose(yh, y1 - 0.5 * sh, rtol=1e-12, atol=1e-12)
    layer.sh_gate_w = x.copy()  # w . x = |x|^2 > 100: sigmoid within 1e-40 of 1
    yf, _, _, _ = orc.moe_ffn_token(layer, x)
    np.testing.assert_allclose(yf, y1, rtol=1e-12, atol=1e-12)
    assert orc.sigmoid(0.0) == 0.5 and orc.sigmoid(-800.0) == 0.0 and orc.sigmoid(800.0) == 1.0
    np.testing.assert_allclose(orc.sigmoid(np.array([-3.0, 1.0])), scipy.special.expit([-3.0, 1.0]), rtol=1e-15)
    Y, _, _, _ = orc.moe_ffn_prefill(layer, np.stack([x, x]))
    np.testing.assert_allclose(Y[1], yf, rtol=1e-12, atol=1e-12)


def _nibbles(words):
    """Independent unpacker of 4-bit rows: nibble j of a row from bits [4(j%8), 4(j%8)+4) of word j//8."""
    return np.array([[(int(wd) >> (4 * j)) & 15 for wd in row for j in range(8)] for row in words])


def test_q8_shared_expert_equals_q4_on_same_codes():
    """A shared expert stored as 8-bit codes that hold the 4-bit expert's codes (same scales and
    biases) gives the layer output of the 4-bit one exactly; an 8-bit shared expert drawn by
    the generator uses codes above 15 and changes only the shared part."""
    H, I, E, k = 128, 64, 8, 2
    layer = synth.moe_layer(13, 0, H, I, E, k)
    x = synth.hidden_vector(13, 0, 0, H)
    y4, ids4, _, _ = orc.moe_ffn_token(layer, x)
    routed = y4 - orc.expert_ffn(layer.expert(E), orc.bf16_to_f64(x))
    for name in ("sh_gate", "sh_up", "sh_down"):
        st = getattr(layer, name)
        c, s, b = st.matrix(0)
        q8 = synth.Q4Stack(1, st.n, st.k, bits=8)
        q8.fill(0, (_pack_bytes(_nibbles(c)), s, b))
        setattr(layer, name, q8)
    y8, ids8, _, _ = orc.moe_ffn_token(layer, x)
    np.testing.assert_array_equal(ids8, ids4)
    np.testing.assert_array_equal(y8, y4)
    wide = synth.moe_layer(13, 0, H, I, E, k, shared_bits=8)
    assert wide.sh_down.codes.shape == (1, H, I // 4) and (wide.sh_gate.codes >> 4 & 15).any()
    yw, idsw, _, _ = orc.moe_ffn_token(wide, x)
    np.testing.assert_array_equal(idsw, ids4)  # same router and routed experts
    np.testing.assert_allclose(yw - orc.expert_ffn(wide.expert(E), orc.bf16_to_f64(x)), routed,
                               rtol=1e-12, atol=1e-12)
