"""Parity of the batched decode (moe_ffn_decode_batch, B = 1..8 tokens in one
step) against the fp64 CPU oracle, token by token, and against the batch-1
decode call on the same inputs.

Each row of the batch is one token through the layer (the oracle's
moe_ffn_token); the batch only changes how often each expert is read.  Expert
ids must match the oracle exactly outside the logit tie band; inside it the
GPU's choice is checked for validity and the oracle is evaluated on it.
"""
import numpy as np
import pytest
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth
from tests.parity_util import check_bf16_output, rel_l2, routing_ok, say, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-5  # every intermediate stays fp32: the error is fp32 accumulation of exact products


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_decode_affine_amd import binding
    binding.load_library()
    return binding


def _check_batch(B, layer, dl, X, ws=None, with_bf16=True):
    """Runs one batched step on the rows of X; returns (worst rel-L2, number of tokens routed exactly)."""
    nb, k = X.shape[0], layer.top_k
    Xd = B.bf16_tensor(X)
    ids = torch.empty((nb, k), dtype=torch.int32, device=DEV)
    w = torch.empty((nb, k), dtype=torch.float32, device=DEV)
    Y = B.moe_ffn_decode_batch(dl, Xd, 0, ids_out=ids, w_out=w, ws=ws)
    Yb = B.moe_ffn_decode_batch(dl, Xd, 1, ws=ws) if with_bf16 else None
    torch.cuda.synchronize()
    got, gids, gw = to_f64(Y), ids.cpu().numpy(), w.cpu().numpy()
    worst, n_exact = 0.0, 0
    for t in range(nb):
        ref, rids, rw, logits = orc.moe_ffn_token(layer, X[t])
        ok, exact = routing_ok(gids[t], logits, k)
        assert ok, (t, gids[t], rids)
        if not exact:
            ref, _, rw, _ = orc.moe_ffn_token(layer, X[t], ids=gids[t])
        n_exact += exact
        np.testing.assert_allclose(gw[t], rw, rtol=1e-4, atol=1e-6)
        worst = max(worst, rel_l2(got[t], ref))
        if with_bf16:
            check_bf16_output(Yb[t], Y[t], ref)
    return worst, n_exact


@pytest.mark.parametrize("H,I,E,k,shared,nb", [(128, 64, 8, 2, True, 1), (128, 64, 8, 2, True, 8),
                                               (384, 192, 16, 4, True, 5), (256, 128, 32, 8, False, 3),
                                               (64, 64, 1, 1, True, 4), (256, 640, 4, 4, True, 8),
                                               (2048, 512, 64, 8, True, 7), (4096, 1024, 16, 4, True, 2)])
def test_decode_batch_small(B, H, I, E, k, shared, nb):
    say(f"decode batch H={H} I={I} E={E} k={k} shared={shared} B={nb}")
    layer = synth.moe_layer(95, 0, H, I, E, k, shared=shared)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(95, nb, H, index=nb)
    worst, _ = _check_batch(B, layer, dl, X)
    assert worst <= TOL, worst


def test_decode_batch_matches_single_token_calls(B):
    """Full layer (hidden 2048, 256 + 1 experts, top-8), B = 4: each row equals the batch-1 call on that row."""
    say("decode batch vs batch-1 calls: generating")
    layer = synth.moe_layer(1)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(96, 4, synth.HIDDEN)
    Y = B.moe_ffn_decode_batch(dl, B.bf16_tensor(X), 0)
    ws1 = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE, dl))
    Y1 = torch.stack([B.moe_ffn_decode(dl, B.bf16_tensor(X[t]), 0, ws=ws1) for t in range(4)])
    torch.cuda.synchronize()
    for t in range(4):
        assert rel_l2(to_f64(Y[t]), to_f64(Y1[t])) <= TOL  # two fp32 summation orders of the same exact products
    worst, n_exact = _check_batch(B, layer, dl, X)
    assert worst <= TOL and n_exact >= 3


@pytest.mark.parametrize("nb", [1, 4, 8])
def test_decode_batch_full_layer(B, nb):
    """Full layer, B = 1, 4 and 8 with one reused workspace over several steps."""
    say(f"decode batch full layer B={nb}: generating")
    layer = synth.moe_layer(1)
    dl = B.DeviceLayer(layer)
    ws = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE_BATCH, dl, rows=nb))
    n_exact = 0
    for step in range(3):
        X = synth.token_rows(97, nb, synth.HIDDEN, index=step)
        worst, ne = _check_batch(B, layer, dl, X, ws=ws, with_bf16=step == 0)
        assert worst <= TOL, (step, worst)
        n_exact += ne
    assert n_exact >= 3 * nb - 2


def test_decode_batch_shared_choices(B):
    """Eight copies of one token and a second token repeated: experts chosen by several rows are read once
    and every copy gets the same output, bit for bit."""
    layer = synth.moe_layer(1)
    dl = B.DeviceLayer(layer)
    a = synth.hidden_vector(98, 0, 0)
    b = synth.hidden_vector(98, 1, 0)
    X = np.stack([a, a, b, a, b, a, a, b])
    say("decode batch with repeated tokens")
    Y = B.moe_ffn_decode_batch(dl, B.bf16_tensor(X), 0)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    for t in range(8):
        src = 0 if (X[t] == a).all() else 2
        assert np.array_equal(Yh[t], Yh[src])
    worst, _ = _check_batch(B, layer, dl, X, with_bf16=False)
    assert worst <= TOL


def test_decode_batch_512_experts_top10(B):
    """512 routed experts + 1 shared, top-10 (lily-qwen3.8-flash-next, "The model"), B = 4 and 8."""
    say("decode batch 512 experts top-10: generating")
    layer = synth.moe_layer(92, 0, synth.HIDDEN, synth.INTER, 512, 10)
    dl = B.DeviceLayer(layer)
    for nb in (4, 8):
        X = synth.token_rows(99, nb, synth.HIDDEN, index=nb)
        worst, _ = _check_batch(B, layer, dl, X, with_bf16=False)
        assert worst <= TOL, (nb, worst)


@pytest.mark.parametrize("H,I,E,k,nb", [(256, 128, 16, 4, 4), (2048, 512, 256, 8, 8)])
def test_decode_batch_q8_router(B, H, I, E, k, nb):
    """Batched decode with the checkpoint's affine-Q8 router gate."""
    say(f"decode batch q8 router H={H} E={E} k={k} B={nb}")
    layer = synth.moe_layer(98, 0, H, I, E, k, router_bits=8)
    dl = B.DeviceLayer(layer)
    X = np.stack([synth.hidden_vector(98, s, 0, H) for s in range(nb)])
    worst, n_exact = _check_batch(B, layer, dl, X)
    assert worst <= 2e-3 and n_exact >= nb - 1, (worst, n_exact)


@pytest.mark.parametrize("H,I,E,k,nb,rbits,gated,sbits", [
    (256, 128, 16, 4, 3, 16, True, 4), (256, 128, 16, 4, 8, 8, True, 8), (384, 192, 16, 4, 5, 16, False, 8),
    (2048, 512, 256, 8, 4, 8, True, 8), (2048, 512, 256, 8, 8, 8, True, 8), (2048, 512, 256, 8, 8, 16, True, 4)])
def test_decode_batch_checkpoint_form(B, H, I, E, k, nb, rbits, gated, sbits):
    """Batched decode in the checkpoint's forms: the shared expert weighted by sigmoid(g . x)
    and/or held in affine-Q8 codes, with either router; every row against the oracle."""
    say(f"decode batch checkpoint form H={H} E={E} k={k} B={nb} router bits={rbits} gated={gated} shared bits={sbits}")
    layer = synth.moe_layer(114, 0, H, I, E, k, router_bits=rbits, shared_gate=gated, shared_bits=sbits)
    dl = B.DeviceLayer(layer)
    X = synth.token_rows(114, nb, H, index=nb)
    worst, n_exact = _check_batch(B, layer, dl, X)
    assert worst <= TOL, worst
    assert n_exact >= nb - 1
