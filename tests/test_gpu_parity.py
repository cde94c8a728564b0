"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Floats: relative L2 <= 2e-3 (the stated bar) plus a tighter check where the
arithmetic guarantees more (fp32 accumulation of exact products).  Integer
stages (top-k ids, permutation, argmax) must match exactly, except where the
deciding logit gap is within 1e-3; there the GPU's own choice is checked for
validity and the float result is compared with the oracle evaluated on it.
"""
import numpy as np
import pytest
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth
from tests.parity_util import REL_L2_TOL, TIE_BAND, check_bf16_output, rel_l2, routing_ok, say, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_decode_affine_amd import binding
    binding.load_library()
    return binding


def _q4(B, mat):
    return B.DeviceQ4(*mat, device=DEV)


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------- q4_gemv --

def test_gemv_hand_example_exact(B):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dequant_hand_example.json")))
    codes = np.array([[int(h, 16) for h in g["codes_hex"]]], dtype=np.uint32)
    scales = np.array([[int(h, 16) for h in g["scales_hex"]]], dtype=np.uint16)
    biases = np.array([[int(h, 16) for h in g["biases_hex"]]], dtype=np.uint16)
    say("gemv hand example")
    W = _q4(B, (codes, scales, biases))
    x = B.bf16_tensor(np.full(g["k"], 0x3F80, dtype=np.uint16))
    y = B.q4_gemv(W, x)
    _sync()
    assert float(y[0]) == g["expected"]["y"]


def test_gemv_one_hot_columns_exact(B):
    n, k = 70, 192
    mat = synth.q4_matrix(21, 0, 0, 0, n, k)
    W = _q4(B, mat)
    Wref = orc.dequantize(*mat, k)
    for j in (0, 5, 63, 64, 127, 128, 191):
        say(f"gemv one-hot column {j}")
        x = np.zeros(k, dtype=np.uint16)
        x[j] = 0x3F80
        y = B.q4_gemv(W, B.bf16_tensor(x))
        _sync()
        np.testing.assert_array_equal(to_f64(y), Wref[:, j])


@pytest.mark.parametrize("n,k,seed", [(512, 2048, 0), (1, 64, 1), (3, 128, 2), (777, 192, 3), (1000, 4096, 4),
                                      (64, 16384, 5), (257, 512, 6)])
def test_gemv_parity(B, n, k, seed):
    say(f"gemv n={n} k={k}")
    mat = synth.q4_matrix(seed, 0, 0, 0, n, k)
    xb = synth.hidden_vector(seed, 0, 0, k)
    W, x = _q4(B, mat), B.bf16_tensor(xb)
    y = B.q4_gemv(W, x, 0)
    yb = B.q4_gemv(W, x, 1)
    _sync()
    ref = orc.q4_gemv(*mat, xb)
    err = rel_l2(to_f64(y), ref)
    assert err <= REL_L2_TOL and err <= 1e-5
    check_bf16_output(yb, y, ref)


# ---------------------------------------------------------------- LM head --

def _check_argmax(ids, mx, logits):
    rid, rmax, gap = orc.greedy_argmax(logits)
    for b in range(len(rid)):
        if gap[b] > TIE_BAND:
            assert int(ids[b]) == int(rid[b]), (b, gap[b])
        else:   # near-tie: the GPU's pick must be within the band of the maximum
            assert logits[b, int(ids[b])] >= rmax[b] - TIE_BAND
        if mx is not None:
            assert abs(float(mx[b]) - logits[b, int(ids[b])]) <= 1e-4 * max(1.0, abs(rmax[b]))


@pytest.mark.parametrize("rows,k,batch", [(5000, 2048, 1), (5000, 2048, 4), (4097, 512, 8), (300, 128, 2),
                                          (1, 64, 1), (9000, 1024, 3), (77, 64, 5), (130, 192, 7),
                                          (1, 128, 6), (2111, 2048, 2)])
def test_lmhead_parity(B, rows, k, batch):
    say(f"lmhead rows={rows} k={k} B={batch}")
    mat = synth.q4_matrix(40 + batch, 0, 0, 0, rows, k)
    X = synth.token_rows(40 + batch, batch, k)
    ids, mx = B.lmhead_argmax(_q4(B, mat), B.bf16_tensor(X))
    _sync()
    _check_argmax(ids.cpu().numpy(), mx.cpu().numpy(), orc.lmhead_logits(*mat, X))


def test_lmhead_planted_and_ties(B):
    rows, k = 3000, 256
    codes, scales, biases = synth.q4_matrix(50, 0, 0, 0, rows, k)
    x = np.full((1, k), 0x3F80, dtype=np.uint16)
    for planted in ((2999,), (1234, 2000), (7, 2500, 2999)):
        say(f"lmhead planted {planted}")
        c, s, b = codes.copy(), scales.copy(), biases.copy()
        for r in planted:                 # identical maximal rows: the lowest index must win
            c[r] = 0xFFFFFFFF
            s[r] = 0x3F80
            b[r] = 0
        ids, mx = B.lmhead_argmax(_q4(B, (c, s, b)), B.bf16_tensor(x))
        _sync()
        assert int(ids[0]) == min(planted) and float(mx[0]) == 15.0 * k


@pytest.mark.parametrize("batch", [2, 4, 7])
def test_lmhead_planted_batches(B, batch):
    """Batched LM head: identical maximal rows in every batch row resolve to the
    lowest index, with the exact maximum."""
    rows, k = 3000, 256
    codes, scales, biases = synth.q4_matrix(51, 0, 0, 0, rows, k)
    x = np.full((batch, k), 0x3F80, dtype=np.uint16)
    for planted in ((2999,), (64, 65, 2000), (7, 2500)):
        say(f"lmhead planted B={batch} {planted}")
        c, s, b = codes.copy(), scales.copy(), biases.copy()
        for r in planted:
            c[r] = 0xFFFFFFFF
            s[r] = 0x3F80
            b[r] = 0
        ids, mx = B.lmhead_argmax(_q4(B, (c, s, b)), B.bf16_tensor(x))
        _sync()
        assert [int(v) for v in ids.cpu()] == [min(planted)] * batch
        assert [float(v) for v in mx.cpu()] == [15.0 * k] * batch


def test_lmhead_workspace_reuse(B):
    """Consecutive calls on one workspace: each result is right and the arrival
    counter (first word of the workspace) is back at zero after every call."""
    rows, k = 20000, 2048
    mat = synth.q4_matrix(60, 0, 0, 0, rows, k)
    W = _q4(B, mat)
    for batch in (1, 4):
        ws = B.workspace(B.workspace_bytes(B.OP_LMHEAD, W=W, rows=batch), "cuda")
        for call in range(3):
            say(f"lmhead reuse B={batch} call={call}")
            X = synth.token_rows(61 + call, batch, k)
            ids, mx = B.lmhead_argmax(W, B.bf16_tensor(X), ws=ws)
            _sync()
            assert int(ws[:4].view(torch.int32).item()) == 0
            _check_argmax(ids.cpu().numpy(), mx.cpu().numpy(), orc.lmhead_logits(*mat, X))


def test_lmhead_full_vocab(B):
    """LM-head shape 151,936 x 2048, batch 1, 4 and 8 (8 x 2048: the largest activation block)."""
    mat = synth.lm_head()
    W = _q4(B, mat)
    for batch in (1, 4, 8):
        say(f"lmhead full vocab B={batch}")
        X = synth.token_rows(4, batch, synth.HIDDEN, index=batch)
        ids, mx = B.lmhead_argmax(W, B.bf16_tensor(X))
        _sync()
        _check_argmax(ids.cpu().numpy(), mx.cpu().numpy(), orc.lmhead_logits(*mat, X))


# ---------------------------------------------------------------- routing --

@pytest.mark.parametrize("T,E,H,k", [(1, 8, 128, 1), (37, 64, 256, 6), (300, 256, 2048, 8), (5, 1024, 64, 32),
                                     (70, 100, 192, 3)])
def test_route_topk(B, T, E, H, k):
    say(f"route T={T} E={E} H={H} k={k}")
    router = synth.router(60, 0, E, H)
    X = synth.token_rows(60, T, H)
    ids, w = B.moe_route_topk(B.bf16_tensor(router), B.bf16_tensor(X), k)
    _sync()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    logits = orc.router_logits(router, X)
    n_exact = 0
    for t in range(T):
        ok, exact = routing_ok(ids[t], logits[t], k)
        assert ok, (t, ids[t])
        n_exact += exact
        ref_w = orc.weights_for_ids(logits[t], ids[t])
        np.testing.assert_allclose(w[t], ref_w, rtol=1e-4, atol=1e-6)
        assert abs(w[t].sum() - 1.0) < 1e-5
    assert n_exact >= 0.9 * T


def test_route_ties_resolve_to_lower_id(B):
    E, H = 16, 64
    router = np.zeros((E, H), dtype=np.uint16)
    for e in range(E):
        router[e, e % 4] = 0x3F80          # experts e and e+4, e+8, e+12 have equal logits
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, :4] = [0x4040, 0x3F80, 0x4000, 0x0000]   # 3, 1, 2, 0
    say("route exact ties")
    ids, w = B.moe_route_topk(B.bf16_tensor(router), B.bf16_tensor(x), 6)
    _sync()
    assert list(ids.cpu().numpy()[0]) == [0, 4, 8, 12, 2, 6]


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 5, 1), (300, 4, 16, 2), (2048, 8, 256, 3),
                                        (1000, 3, 1000, 4), (33, 8, 40, 5)])
def test_permute_exact(B, T, k, E, seed):
    say(f"permute T={T} k={k} E={E}")
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    off, rows, inv = B.moe_permute(torch.from_numpy(ids).to(DEV), E)
    _sync()
    r_off, r_rows, r_inv = orc.permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    np.testing.assert_array_equal(rows.cpu().numpy(), r_rows)
    np.testing.assert_array_equal(inv.cpu().numpy(), r_inv)


def test_permute_chunk_edges(B):
    """Rows crossing several 1,024-row ranking chunks, a ragged last chunk, one
    expert taking every row of a chunk and experts absent from whole chunks."""
    rng = np.random.default_rng(7)
    T, k, E = 1500, 3, 40
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[200:560, 0] = 17          # expert 17 dense across the first chunk boundary (row 1024 = token 341)
    ids[700:, 1] = np.where(ids[700:, 0] != 39, 39, 38)
    ids[ids == 5] = 6             # expert 5 never used
    for t in range(T):            # keep the k ids of a token distinct
        if len(set(ids[t])) < k:
            ids[t] = rng.choice([e for e in range(E) if e != 5], size=k, replace=False)
    say("permute chunk edges")
    off, rows, inv = B.moe_permute(torch.from_numpy(ids).to(DEV), E)
    _sync()
    r_off, r_rows, r_inv = orc.permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    np.testing.assert_array_equal(rows.cpu().numpy(), r_rows)
    np.testing.assert_array_equal(inv.cpu().numpy(), r_inv)


def test_permute_skewed(B):
    """Most tokens pick expert 3: one segment spans many rows, several are empty."""
    T, k, E = 700, 2, 12
    ids = np.stack([[3, (t % 5) + 5] if t % 7 else [(t % 11) + 1 if (t % 11) + 1 != 3 else 0, 3]
                    for t in range(T)]).astype(np.int32)
    say("permute skewed")
    off, rows, inv = B.moe_permute(torch.from_numpy(ids).to(DEV), E)
    _sync()
    r_off, r_rows, r_inv = orc.permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    np.testing.assert_array_equal(rows.cpu().numpy(), r_rows)
    np.testing.assert_array_equal(inv.cpu().numpy(), r_inv)


# ----------------------------------------------------------------- q4_gemm --

@pytest.mark.parametrize("m,n,k,seed", [(1, 32, 64, 0), (300, 777, 640, 1), (128, 256, 2048, 2),
                                        (2048, 512, 2048, 3), (129, 2048, 512, 4), (40, 100, 192, 5)])
def test_gemm_parity(B, m, n, k, seed):
    say(f"gemm m={m} n={n} k={k}")
    mat = synth.q4_matrix(70 + seed, 0, 0, 0, n, k)
    X = synth.token_rows(70 + seed, m, k)
    W, Xd = _q4(B, mat), B.bf16_tensor(X)
    Y = B.q4_gemm(W, Xd, 0)
    Yb = B.q4_gemm(W, Xd, 1)
    _sync()
    ref = orc.q4_gemm(*mat, X)
    got = to_f64(Y)
    err = rel_l2(got, ref)
    # fp16 operands: each s*q is rounded once (at most 2^-12 of itself, and |s*q| is
    # typically about twice |w|), the rows convert exactly; the whole product stays
    # far inside the 2e-3 bar
    assert err <= REL_L2_TOL and err <= 5e-4
    # row by row as well: no row may be off (a wrong tile would hide in the global norm)
    for r in range(0, m, max(1, m // 17)):
        assert rel_l2(got[r], ref[r]) <= 1e-3
    check_bf16_output(Yb, Y, ref)


# ------------------------------------------------------------ MoE decode --

def _decode_check(B, layer, dl, x_bits, with_bf16=False, ws=None):
    ids = torch.empty(layer.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(layer.top_k, dtype=torch.float32, device=DEV)
    xd = B.bf16_tensor(x_bits)
    y = B.moe_ffn_decode(dl, xd, 0, ids_out=ids, w_out=w, ws=ws)
    yb = B.moe_ffn_decode(dl, xd, 1, ws=ws) if with_bf16 else None
    _sync()
    gids = ids.cpu().numpy()
    ref, rids, rw, logits = orc.moe_ffn_token(layer, x_bits)
    ok, exact = routing_ok(gids, logits, layer.top_k)
    assert ok, (gids, rids)
    if not exact:
        ref, _, rw, _ = orc.moe_ffn_token(layer, x_bits, ids=gids)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-4, atol=1e-6)
    err = rel_l2(to_f64(y), ref)
    assert err <= REL_L2_TOL, err
    if with_bf16:
        check_bf16_output(yb, y, ref)
    return err, exact


@pytest.mark.parametrize("H,I,E,k,shared", [(128, 64, 8, 2, True), (384, 192, 16, 4, True),
                                            (256, 128, 32, 8, False), (2048, 512, 64, 8, True),
                                            (64, 64, 1, 1, True), (4096, 2048, 16, 4, True)])
def test_decode_small(B, H, I, E, k, shared):
    say(f"decode H={H} I={I} E={E} k={k} shared={shared}")
    layer = synth.moe_layer(80, 0, H, I, E, k, shared=shared)
    dl = B.DeviceLayer(layer)
    for step in range(3):
        x = synth.hidden_vector(80, step, 0, H)
        err, _ = _decode_check(B, layer, dl, x, with_bf16=True)
        assert err <= 1e-5


def test_decode_config1(B):
    """One MoE layer at decode: hidden 2048, 256 experts + 1 shared, top-8, one reused workspace."""
    say("decode full layer: generating")
    layer = synth.moe_layer(1)
    dl = B.DeviceLayer(layer)
    ws = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE, dl))
    n_exact = 0
    for step in range(8):
        say(f"decode full layer step {step}")
        err, exact = _decode_check(B, layer, dl, synth.hidden_vector(1, step, 0), ws=ws)
        assert err <= 1e-5
        n_exact += exact
    assert n_exact >= 6
    # no abandoned waits inside the kernel (the counter at byte offset 2048 of the workspace)
    assert int(ws[2048:2052].cpu().view(torch.int32)[0]) == 0


def test_decode_512_experts_top10(B):
    """Wider router at decode: hidden 2048, 512 routed experts + 1 shared, top-10."""
    say("decode 512 experts top-10: generating")
    layer = synth.moe_layer(92, 0, synth.HIDDEN, synth.INTER, 512, 10)
    dl = B.DeviceLayer(layer)
    ws = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE, dl))
    n_exact = 0
    for step in range(6):
        say(f"decode 512 experts top-10 step {step}")
        err, exact = _decode_check(B, layer, dl, synth.hidden_vector(92, step, 0), ws=ws)
        assert err <= 1e-5
        n_exact += exact
    assert n_exact >= 4
    assert int(ws[2048:2052].cpu().view(torch.int32)[0]) == 0


# ----------------------------------------------------------- MoE prefill --

def _prefill_check(B, layer, dl, X, with_bf16=True):
    """Whole-chunk comparison; tokens whose routing differs within the tie band are
    evaluated by the oracle on the GPU's expert choice."""
    Xd = B.bf16_tensor(X)
    Y = B.moe_ffn_prefill(dl, Xd, 0)
    Yb = B.moe_ffn_prefill(dl, Xd, 1) if with_bf16 else None
    ids, _ = B.gpu_routing(dl, B.bf16_tensor(X))
    _sync()
    got = to_f64(Y)
    gids = ids.cpu().numpy()
    logits = orc.layer_router_logits(layer, X)
    r_ids, _ = orc.topk_from_logits(logits, layer.top_k)
    use = r_ids.copy()
    for t in range(X.shape[0]):
        ok, exact = routing_ok(gids[t], logits[t], layer.top_k)
        assert ok, (t, gids[t])
        if not exact:
            use[t] = gids[t]
    ref, _, _, _ = orc.moe_ffn_prefill(layer, X, ids=use)
    worst = max(rel_l2(got[t], ref[t]) for t in range(X.shape[0]))
    if with_bf16:
        check_bf16_output(Yb, Y, ref)
    return rel_l2(got, ref), worst


@pytest.mark.parametrize("T,H,I,E,k,shared", [(1, 128, 64, 4, 2, True), (100, 256, 128, 16, 4, True),
                                              (300, 512, 192, 16, 4, True), (257, 384, 128, 8, 3, False),
                                              (520, 2048, 512, 32, 8, True),
                                              # 3 and 1 K groups: the shared expert's gate/up split into
                                              # uneven halves, or not at all; router quarters of unequal length
                                              (97, 192, 64, 8, 2, True), (33, 64, 128, 4, 2, True)])
def test_prefill_small(B, T, H, I, E, k, shared):
    say(f"prefill T={T} H={H} I={I} E={E} k={k} shared={shared}")
    layer = synth.moe_layer(90, 0, H, I, E, k, shared=shared)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(90, T, H)
    err, worst = _prefill_check(B, layer, dl, X)
    assert err <= REL_L2_TOL, err
    assert worst <= 2 * REL_L2_TOL


def test_prefill_skewed_routing(B):
    """Every token picks experts 1 and 5: two segments far above one 128-row tile, the rest empty."""
    T, H, I, E, k = 600, 256, 128, 8, 2
    layer = synth.moe_layer(91, 0, H, I, E, k)
    sign = np.where(np.arange(H) % 3 == 0, -1.0, 1.0)
    X = synth.to_bf16_bits(orc.bf16_to_f64(synth.token_rows(91, T, H)) + sign)
    layer.router[1] = synth.to_bf16_bits(0.1 * sign)
    layer.router[5] = synth.to_bf16_bits(0.09 * sign)
    dl = B.DeviceLayer(layer)
    say("prefill skewed routing")
    ids, _ = B.moe_route_topk(dl.router, B.bf16_tensor(X), k)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
    assert counts[1] == T and counts[5] == T
    err, worst = _prefill_check(B, layer, dl, X)
    assert err <= REL_L2_TOL and worst <= 2 * REL_L2_TOL


def test_prefill_config3(B):
    """2,048-token chunk through the full layer (hidden 2048, 256 + 1 experts, top-8)."""
    say("prefill full chunk: generating")
    layer = synth.moe_layer(1)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(3, 2048, synth.HIDDEN)
    say("prefill full chunk: running")
    err, worst = _prefill_check(B, layer, dl, X)
    say(f"prefill full chunk rel_l2={err:.3e} worst={worst:.3e}")
    assert err <= REL_L2_TOL and worst <= 2 * REL_L2_TOL


def test_prefill_4096_tokens_512_experts_top10(B):
    """A 4,096-token chunk through a layer with 512 routed experts + 1 shared, top-10."""
    say("prefill 4096 tokens, 512 experts top-10: generating")
    layer = synth.moe_layer(93, 0, synth.HIDDEN, synth.INTER, 512, 10)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(93, 4096, synth.HIDDEN)
    say("prefill 4096 tokens, 512 experts top-10: running")
    err, worst = _prefill_check(B, layer, dl, X, with_bf16=False)
    say(f"prefill 4096 tokens rel_l2={err:.3e} worst={worst:.3e}")
    assert err <= REL_L2_TOL and worst <= 2 * REL_L2_TOL


# ------------------------------------------- rows far outside the fp16 range --

def _scaled_rows(seed, T, H):
    """Rows of N(0,1) values, some scaled far past fp16's range (2^20: up to ~4e6), some far
    below it (2^-20), one all zero, one mixing magnitudes 2^-24..2^12 inside the row."""
    X = orc.bf16_to_f64(synth.token_rows(seed, T, H))
    X[0] *= 2.0 ** 20
    X[1] *= 2.0 ** -20
    X[2] = 0.0
    X[3] *= np.ldexp(1.0, (np.arange(H) % 37) - 24)
    if T > 5:
        X[5] *= 2.0 ** 14
    return synth.to_bf16_bits(X)


def test_gemm_row_magnitudes(B):
    """q4_gemm scales each row by a power of two into fp16: rows of any magnitude keep the
    accuracy of ordinary rows, and a zero row gives exactly zero."""
    m, n, k = 40, 300, 512
    say(f"gemm row magnitudes m={m} n={n} k={k}")
    mat = synth.q4_matrix(77, 0, 0, 0, n, k)
    X = _scaled_rows(77, m, k)
    Y = B.q4_gemm(_q4(B, mat), B.bf16_tensor(X), 0)
    _sync()
    got, ref = to_f64(Y), orc.q4_gemm(*mat, X)
    assert np.all(got[2] == 0.0)
    for r in range(m):
        if r != 2:
            assert rel_l2(got[r], ref[r]) <= 1e-3, (r, rel_l2(got[r], ref[r]))


def test_prefill_row_magnitudes(B):
    """The prefill layer on rows far outside fp16's range (and their SwiGLU activations,
    which scale with the square of the row) against the oracle, row by row."""
    T, H, I, E, k = 64, 256, 128, 16, 4
    say("prefill row magnitudes")
    layer = synth.moe_layer(94, 0, H, I, E, k)
    dl = B.DeviceLayer(layer)
    X = _scaled_rows(94, T, H)
    err, worst = _prefill_check(B, layer, dl, X, with_bf16=False)
    assert err <= REL_L2_TOL and worst <= 2 * REL_L2_TOL, (err, worst)


# ---------------------------------------------------- 8-bit affine matrices --

def test_q8_gemv_hand_example_exact(B):
    """The oracle's worked 8-bit example: x = ones gives exactly 752 + 4144."""
    words = [0x03020100 + 0x04040404 * i for i in range(16)] + [0xFFFFFFFF] * 16
    mat = (np.array([words], dtype=np.uint32), np.array([[0x3F00, 0x3E80]], dtype=np.uint16),
           np.array([[0xC080, 0x3F80]], dtype=np.uint16))
    y = B.q4_gemv(_q4(B, mat), B.bf16_tensor(np.full(128, 0x3F80, dtype=np.uint16)))
    _sync()
    assert float(y[0]) == 4896.0


@pytest.mark.parametrize("n,k,seed", [(512, 2048, 0), (777, 640, 1), (33, 64, 2), (1000, 192, 3)])
def test_q8_gemv_parity(B, n, k, seed):
    say(f"q8 gemv n={n} k={k}")
    mat = synth.q8_matrix(60 + seed, 0, 0, 0, n, k)
    x = synth.token_rows(60 + seed, 1, k)[0]
    W = _q4(B, mat)
    assert W.bits == 8
    y = B.q4_gemv(W, B.bf16_tensor(x))
    yb = B.q4_gemv(W, B.bf16_tensor(x), 1)
    _sync()
    ref = orc.q4_gemv(*mat, x)
    err = rel_l2(to_f64(y), ref)
    assert err <= 1e-5, err  # exact 8-bit x 8-bit products, fp32 sums
    check_bf16_output(yb, y, ref)


@pytest.mark.parametrize("batch", [1, 2, 4, 7, 8])
def test_q8_lmhead_parity(B, batch):
    rows, k = 20000, 1024
    say(f"q8 lmhead rows={rows} k={k} B={batch}")
    mat = synth.q8_matrix(61, 0, 0, 0, rows, k)
    X = synth.token_rows(61, batch, k, index=batch)
    ids, mx = B.lmhead_argmax(_q4(B, mat), B.bf16_tensor(X))
    _sync()
    _check_argmax(ids.cpu().numpy(), mx.cpu().numpy(), orc.lmhead_logits(*mat, X))


def test_q8_lmhead_planted_ties(B):
    """Identical maximal 8-bit rows: the lowest index wins, with the exact maximum."""
    rows, k = 3000, 256
    codes, scales, biases = synth.q8_matrix(62, 0, 0, 0, rows, k)
    x = np.full((1, k), 0x3F80, dtype=np.uint16)
    for planted in ((2999,), (1234, 2000)):
        c, s, b = codes.copy(), scales.copy(), biases.copy()
        for r in planted:
            c[r] = 0xFFFFFFFF
            s[r] = 0x3F80
            b[r] = 0
        ids, mx = B.lmhead_argmax(_q4(B, (c, s, b)), B.bf16_tensor(x))
        _sync()
        assert int(ids[0]) == min(planted) and float(mx[0]) == 255.0 * k


def test_q8_lmhead_full_vocab(B):
    """8-bit LM head of the q4-xl kind, 151,936 x 2048, batch 1, 4 and 8."""
    mat = synth.lm_head(bits=8)
    W = _q4(B, mat)
    for batch in (1, 4, 8):
        say(f"q8 lmhead full vocab B={batch}")
        X = synth.token_rows(4, batch, synth.HIDDEN, index=batch)
        ids, mx = B.lmhead_argmax(W, B.bf16_tensor(X))
        _sync()
        _check_argmax(ids.cpu().numpy(), mx.cpu().numpy(), orc.lmhead_logits(*mat, X))


@pytest.mark.parametrize("H,I,E,k", [(256, 128, 16, 4), (2048, 512, 256, 8)])
def test_decode_q8_router(B, H, I, E, k):
    """Batch-1 decode with the checkpoint's affine Q8 router gate in place of the bf16 router."""
    say(f"decode q8 router H={H} I={I} E={E} k={k}")
    layer = synth.moe_layer(97, 0, H, I, E, k, router_bits=8)
    dl = B.DeviceLayer(layer)
    assert dl.router_q8 is not None and dl.router_q8.bits == 8
    n_exact = 0
    for step in range(4):
        err, exact = _decode_check(B, layer, dl, synth.hidden_vector(97, step, 0, H))
        n_exact += exact
    assert n_exact >= 3


@pytest.mark.parametrize("T,H,I,E,k", [(300, 256, 128, 16, 4), (2048, 2048, 512, 256, 8)])
def test_prefill_q8_router(B, T, H, I, E, k):
    """Prefill with the checkpoint's affine-Q8 router gate: every token against the oracle,
    on the GPU's own routing (moe_route_topk_q8) wherever it differs within the tie band."""
    say(f"prefill q8 router T={T} H={H} E={E} k={k}")
    layer = synth.moe_layer(99, 0, H, I, E, k, router_bits=8)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(99, T, H)
    err, worst = _prefill_check(B, layer, dl, X)
    assert err <= REL_L2_TOL, err
    assert worst <= 2 * REL_L2_TOL


@pytest.mark.parametrize("T,H,E,k", [(300, 256, 16, 4), (2048, 2048, 256, 8), (777, 2048, 512, 10),
                                     (61, 192, 70, 5), (9, 64, 8, 2)])  # 3 and 1 groups: unequal K quarters
def test_route_topk_q8(B, T, H, E, k):
    """The standalone 8-bit router: ids bit-exact against the oracle outside the tie band,
    weights to 1e-4 (on the GPU's set where it differs within the band)."""
    say(f"route q8 T={T} H={H} E={E} k={k}")
    codes, scales, biases = synth.q8_matrix(113, 0, synth.ROUTER_STREAM, 0, E, H, scale_std=0.02 / 74)
    Rq = B.DeviceQ4(codes, scales, biases)
    X = synth.token_rows(113, T, H)
    ids, w = B.moe_route_topk_q8(Rq, B.bf16_tensor(X), k)
    _sync()
    gids, gw = ids.cpu().numpy(), w.cpu().numpy()
    logits = orc.q4_gemm(codes, scales, biases, X)        # the 8-bit router's logits, exact
    n_exact = 0
    for t in range(T):
        ok, exact = routing_ok(gids[t], logits[t], k)
        assert ok, (t, gids[t])
        n_exact += exact
        np.testing.assert_allclose(gw[t], orc.weights_for_ids(logits[t], gids[t]), rtol=1e-4, atol=1e-6)
    assert n_exact >= 0.9 * T


@pytest.mark.parametrize("H,I,E,k,rbits", [(256, 128, 16, 4, 16), (256, 128, 16, 4, 8),
                                           (2048, 512, 256, 8, 16), (2048, 512, 256, 8, 8)])
def test_decode_shared_gate(B, H, I, E, k, rbits):
    """Batch-1 decode with the shared expert weighted by sigmoid(g . x), with either router."""
    say(f"decode shared gate H={H} I={I} E={E} k={k} router bits={rbits}")
    layer = synth.moe_layer(98, 0, H, I, E, k, router_bits=rbits, shared_gate=True)
    dl = B.DeviceLayer(layer)
    n_exact = 0
    for step in range(4):
        err, exact = _decode_check(B, layer, dl, synth.hidden_vector(98, step, 0, H), with_bf16=True)
        assert err <= 1e-5
        n_exact += exact
    assert n_exact >= 3


@pytest.mark.parametrize("T,H,I,E,k", [(300, 256, 128, 16, 4), (2048, 2048, 512, 256, 8)])
def test_prefill_shared_gate(B, T, H, I, E, k):
    """Prefill with the shared expert weighted per token by sigmoid(g . x)."""
    say(f"prefill shared gate T={T} H={H} E={E} k={k}")
    layer = synth.moe_layer(100, 0, H, I, E, k, shared_gate=True)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(100, T, H)
    err, worst = _prefill_check(B, layer, dl, X)
    assert err <= REL_L2_TOL, err
    assert worst <= 2 * REL_L2_TOL


@pytest.mark.parametrize("H,I,E,k,rbits,gated", [(256, 128, 16, 4, 16, False), (384, 192, 16, 4, 8, True),
                                                 (64, 64, 4, 2, 16, False), (2048, 512, 256, 8, 8, False),
                                                 (2048, 512, 256, 8, 8, True), (4096, 1024, 16, 4, 16, False)])
def test_decode_q8_shared_expert(B, H, I, E, k, rbits, gated):
    """Batch-1 decode with the shared expert in affine-Q8 codes (the q4-xl checkpoint's form),
    alone or with the 8-bit router and the shared-expert gate."""
    say(f"decode q8 shared H={H} I={I} E={E} k={k} router bits={rbits} gated={gated}")
    layer = synth.moe_layer(101, 0, H, I, E, k, router_bits=rbits, shared_gate=gated, shared_bits=8)
    dl = B.DeviceLayer(layer)
    assert all(m.bits == 8 for m in dl.sh)
    n_exact = 0
    for step in range(4):
        err, exact = _decode_check(B, layer, dl, synth.hidden_vector(101, step, 0, H), with_bf16=True)
        assert err <= 1e-5
        n_exact += exact
    assert n_exact >= 3


def test_decode_q8_shared_residual(B):
    """The residual form with an 8-bit shared expert: bf16(x + y) of the layer's own fp32 output."""
    H, I, E, k = 2048, 512, 256, 8
    layer = synth.moe_layer(102, 0, H, I, E, k, router_bits=8, shared_bits=8)
    dl = B.DeviceLayer(layer)
    for step in range(3):
        x_bits = synth.hidden_vector(102, step, 0, H)
        x = B.bf16_tensor(x_bits)
        ids = torch.empty(k, dtype=torch.int32, device=DEV)
        xn = B.moe_ffn_decode(dl, x, B.OUT_BF16_RESIDUAL, ids_out=ids)
        y = B.moe_ffn_decode(dl, x, B.OUT_F32)
        _sync()
        # the same call's own rounding of x + y ...
        assert torch.equal(xn.cpu(), (x.cpu().float() + y.cpu()).to(torch.bfloat16))
        # ... and the oracle's: y to the float bar, bf16(x + y) within y's error plus half a step
        gids = ids.cpu().numpy()
        ref, _, _, logits = orc.moe_ffn_token(layer, x_bits)
        ok, exact = routing_ok(gids, logits, k)
        assert ok
        if not exact:
            ref, _, _, _ = orc.moe_ffn_token(layer, x_bits, ids=gids)
        yg = to_f64(y)
        assert rel_l2(yg, ref) <= 1e-5
        got = orc.bf16_to_f64(xn.cpu().view(torch.int16).numpy().view(np.uint16))
        want = orc.bf16_to_f64(orc.residual_next(x_bits, ref))
        _, e1 = np.frexp(got)
        _, e2 = np.frexp(want)
        half = np.where(got == 0, 0, np.ldexp(0.5, e1 - 8)) + np.where(want == 0, 0, np.ldexp(0.5, e2 - 8))
        assert np.all(np.abs(got - want) <= (np.abs(yg - ref) + half) * (1 + 1e-12))
        assert np.mean(got == want) >= 0.95


@pytest.mark.parametrize("T,H,I,E,k,rbits,gated", [(300, 256, 128, 16, 4, 16, False), (257, 384, 192, 8, 3, 8, True),
                                                   (2048, 2048, 512, 256, 8, 8, True)])
def test_prefill_q8_shared_expert(B, T, H, I, E, k, rbits, gated):
    """Prefill with the shared expert in affine-Q8 codes (its GEMM tiles on the 8-bit B
    operand), alone or in the checkpoint's full form (8-bit router, shared-expert gate)."""
    say(f"prefill q8 shared T={T} H={H} E={E} k={k} router bits={rbits} gated={gated}")
    layer = synth.moe_layer(115, 0, H, I, E, k, router_bits=rbits, shared_gate=gated, shared_bits=8)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(115, T, H)
    err, worst = _prefill_check(B, layer, dl, X)
    assert err <= REL_L2_TOL, err
    assert worst <= 2 * REL_L2_TOL
