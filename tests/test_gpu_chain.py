"""The decode step with the host off its critical path: layers chained through a residual
stream (moe_ffn_decode in its residual form writes bf16(x + y), the next layer's input),
then the LM-head argmax, enqueued launch by launch or replayed from a captured HIP graph.

Each layer is checked against the oracle on the GPU's own input to that layer (a chain
of random layers amplifies rounding differences, so later layers are not compared with
an oracle chain): the expert ids must match outside the 1e-3 logit tie band, the
layer's fp32 output y must meet the 2e-3 relative-L2 bar, the next input must be the
bfloat16 rounding of x + (that fp32 y), and each element may differ from the oracle's
rounding of the exact x + y by no more than the error of y at that element plus half a
bfloat16 step of each of the two values (rounding to nearest moves a value by at most
half a step and never reorders values; where x + y nearly cancels, a small error of y
spans several bfloat16 steps).  The graph replays must reproduce the eager step bit for
bit.
"""
import numpy as np
import pytest
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth, workloads
from tests.parity_util import REL_L2_TOL, TIE_BAND, rel_l2, routing_ok, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_decode_affine_amd import binding
    binding.load_library()
    return binding


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _half_step(v):
    """Half the bfloat16 spacing at each value (8 significant bits: v in [2^e, 2^(e+1)) has
    spacing 2^(e-7)); 0 for zeros."""
    _, e = np.frexp(v)
    return np.where(v == 0, 0.0, np.ldexp(0.5, e - 8))


def _check_residual(x_bits, got_next_bits, y_gpu, layer, gpu_ids):
    """The next input against the oracle on this input; returns the fraction exactly equal."""
    ref_y, _, _, logits = orc.moe_ffn_token(layer, x_bits)
    ok, exact = routing_ok(gpu_ids, logits, layer.top_k)
    assert ok, (gpu_ids, np.argsort(-logits)[:layer.top_k])
    if not exact:
        ref_y, _, _, _ = orc.moe_ffn_token(layer, x_bits, ids=gpu_ids)
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert rel_l2(y_gpu, ref_y) <= REL_L2_TOL
    ref_next = orc.residual_next(x_bits, ref_y)
    got, ref = orc.bf16_to_f64(got_next_bits), orc.bf16_to_f64(ref_next)
    bound = np.abs(y_gpu - ref_y) + _half_step(got) + _half_step(ref)
    bad = np.nonzero(np.abs(got - ref) > bound * (1 + 1e-12))[0]
    assert bad.size == 0, (bad[:8], got[bad[:8]], ref[bad[:8]])
    return float(np.mean(got_next_bits == ref_next))


@pytest.mark.parametrize("H,I,E,k", [(256, 128, 16, 4), (2048, 512, 256, 8)])
def test_residual_output_one_layer(B, H, I, E, k):
    say(f"residual form H={H} I={I} E={E} k={k}")
    layer = synth.moe_layer(95, 0, H, I, E, k)
    dl = B.DeviceLayer(layer)
    x = synth.hidden_vector(95, 0, 0, H)
    ids = torch.empty(k, dtype=torch.int32, device=DEV)
    xn = B.moe_ffn_decode(dl, B.bf16_tensor(x), B.OUT_BF16_RESIDUAL, ids_out=ids)
    yf = B.moe_ffn_decode(dl, B.bf16_tensor(x), B.OUT_F32)
    torch.cuda.synchronize()
    assert xn.dtype == torch.bfloat16
    # the residual form is the bf16 rounding of x + (the fp32 output) computed in fp32
    want = (torch.from_numpy(orc.bf16_to_f64(x)).float() + yf.cpu()).to(torch.bfloat16)
    assert np.array_equal(_bits(xn), _bits(want))
    frac = _check_residual(x, _bits(xn), yf.cpu().double().numpy(), layer, ids.cpu().numpy())
    assert frac >= 0.95, frac


def _small_chain(B, n_layers=6, H=256, I=128, E=16, k=4, vocab=3000):
    layers = [synth.moe_layer(96, l, H, I, E, k) for l in range(n_layers)]
    lm = synth.lm_head(seed=96, rows=vocab, hidden=H)
    chain = workloads.DecodeChain([B.DeviceLayer(L) for L in layers], B.DeviceQ4(*lm, device=DEV), DEV)
    return chain, layers, lm


def test_chain_teacher_forced(B):
    """Each layer of an eager step against the oracle on that layer's GPU input; the token
    against the oracle's argmax of the last input (bit-exact outside the tie band)."""
    say("chain: eager step, 6 layers + LM head")
    chain, layers, lm = _small_chain(B)
    x0 = synth.hidden_vector(96, 7, 0, chain.xs.shape[1])
    chain.xs[0].copy_(B.bf16_tensor(x0))
    chain.enqueue()
    torch.cuda.synchronize()
    xs, ids = _bits(chain.xs), chain.ids.cpu().numpy()
    assert np.array_equal(xs[0], x0)
    for l, layer in enumerate(layers):
        # the layer's fp32 output on the same input (the decode call is deterministic)
        y = B.moe_ffn_decode(chain.layers[l], chain.xs[l].clone(), B.OUT_F32)
        torch.cuda.synchronize()
        frac = _check_residual(xs[l], xs[l + 1], y.cpu().double().numpy(), layer, ids[l])
        assert frac >= 0.95, (l, frac)
    ref_ids, ref_max, gap = orc.greedy_argmax(orc.lmhead_logits(*lm, xs[-1]))
    if gap[0] > TIE_BAND:
        assert int(chain.token.item()) == int(ref_ids[0])
    assert abs(float(chain.max_logit.item()) - ref_max[0]) <= 1e-4 * max(1.0, abs(ref_max[0]))


def test_chain_graph_replay_matches_eager(B):
    """A captured step replayed three times, with eager steps on another input in between,
    reproduces the eager results of its input bit for bit every time."""
    say("chain: graph capture and replays")
    chain, _, _ = _small_chain(B)
    H = chain.xs.shape[1]
    xa = B.bf16_tensor(synth.hidden_vector(96, 11, 0, H))
    xb = B.bf16_tensor(synth.hidden_vector(96, 12, 0, H))

    def eager(x):
        chain.xs[0].copy_(x)
        chain.enqueue()
        torch.cuda.synchronize()
        return chain.xs.clone(), chain.ids.clone(), chain.token.clone()

    ref_a, ref_b = eager(xa), eager(xb)
    chain.xs[0].copy_(xa)
    chain.capture()
    for rep, (x, ref) in enumerate([(xa, ref_a), (xb, ref_b), (xa, ref_a)]):
        chain.xs[0].copy_(x)
        chain.replay()
        torch.cuda.synchronize()
        got = (chain.xs.clone(), chain.ids.clone(), chain.token.clone())
        for g, r in zip(got, ref):
            assert torch.equal(g, r), rep
        other = eager(xb if x is xa else xa)  # eager work between the replays
        assert other[2].numel() == 1
    chain.check()  # no layer launch of the eager steps or the replays abandoned a wait
    assert B.decode_timeouts(chain.ws) == 0


def test_decode_stack_timeout_word_stays_zero(B):
    """A 6-layer stack, 4 steps enqueued back to back on one workspace: the abandoned-wait
    counter stays 0 (every workgroup of every launch was resident and saw every word)."""
    say("decode stack: timeout word after back-to-back steps")
    stack = workloads.DecodeStack(seed=97, n_layers=6, n_steps=4, device=DEV)
    for s in range(4):
        stack.step(s)
    stack.check()
    assert B.decode_timeouts(stack.ws) == 0
