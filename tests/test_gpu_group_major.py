"""The group-major copy of the 4-bit codes that the prefill GEMMs can read.

The copy is a layout change only: the pack call must reproduce the codes
exactly in the documented order, and q4_gemm / moe_ffn_prefill must give the
same bits with and without it (the same products in the same order).  One
small case is also compared with the fp64 oracle directly.
"""
import numpy as np
import pytest
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth
from tests.parity_util import REL_L2_TOL, rel_l2, say, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_decode_affine_amd import binding
    binding.load_library()
    return binding


def _stack(seed, count, n, k):
    mats = [synth.q4_matrix(seed, i, 0, 0, n, k) for i in range(count)]
    return tuple(np.stack([m[j] for m in mats]) for j in range(3))


@pytest.mark.parametrize("count,n,k", [(1, 1, 64), (3, 100, 192), (2, 512, 2048), (1, 2048, 512)])
def test_pack_layout_exact(B, count, n, k):
    say(f"pack group-major count={count} n={n} k={k}")
    codes, scales, biases = _stack(130, count, n, k)
    W = B.DeviceQ4(codes, scales, biases, device=DEV)
    W.pack_group_major()
    torch.cuda.synchronize()
    got = W.codes_gm.cpu().numpy().view(np.uint32).reshape(count, k // 64, n, 8)
    want = codes.reshape(count, n, k // 64, 8).transpose(0, 2, 1, 3)
    assert np.array_equal(got, want)
    assert np.array_equal(W.codes.cpu().numpy().view(np.uint32), codes)  # the source is left alone


@pytest.mark.parametrize("m,n,k,seed", [(1, 32, 64, 0), (300, 777, 640, 1), (2048, 512, 2048, 2),
                                        (129, 2048, 512, 3), (97, 100, 192, 4)])
def test_gemm_group_major_bit_identical(B, m, n, k, seed):
    say(f"gemm group-major m={m} n={n} k={k}")
    mat = synth.q4_matrix(131 + seed, 0, 0, 0, n, k)
    X = B.bf16_tensor(synth.token_rows(131 + seed, m, k))
    W = B.DeviceQ4(*mat, device=DEV)
    Y0 = B.q4_gemm(W, X, 0)
    Yb0 = B.q4_gemm(W, X, 1)
    W.pack_group_major()
    Y1 = B.q4_gemm(W, X, 0)
    Yb1 = B.q4_gemm(W, X, 1)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int32), Y1.view(torch.int32))
    assert torch.equal(Yb0.view(torch.int16), Yb1.view(torch.int16))
    if m * n * k <= 300 * 777 * 640:
        assert rel_l2(to_f64(Y1), orc.q4_gemm(*mat, synth.token_rows(131 + seed, m, k))) <= 5e-4


def test_gemm_stack_ignores_group_major(B):
    """q4_gemm over a stack of matrices reads the row-major codes (the group-major
    copy is per matrix), so a stack with a copy gives the same result."""
    codes, scales, biases = _stack(136, 3, 96, 256)
    X = B.bf16_tensor(synth.token_rows(136, 50, 256))
    W = B.DeviceQ4(codes, scales, biases, device=DEV)
    Y0 = B.q4_gemm(W, X, 0)
    W.pack_group_major()
    Y1 = B.q4_gemm(W, X, 0)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int32), Y1.view(torch.int32))


def _layer_pair(B, layer):
    plain = B.DeviceLayer(layer, device=DEV)
    packed = B.DeviceLayer(layer, device=DEV)
    packed.pack_group_major()
    return plain, packed


@pytest.mark.parametrize("T,H,I,E,k,kw", [
    (1, 128, 64, 4, 2, {}),
    (300, 512, 192, 16, 4, {}),
    (257, 384, 128, 8, 3, {"shared": False}),
    (300, 256, 128, 16, 4, {"shared_bits": 8, "router_bits": 8, "shared_gate": True}),
    (2048, 2048, 512, 256, 8, {}),
    (777, 2048, 512, 512, 10, {"router_bits": 8, "shared_gate": True}),
])
def test_prefill_group_major_bit_identical(B, T, H, I, E, k, kw):
    say(f"prefill group-major T={T} H={H} I={I} E={E} k={k} {kw}")
    layer = synth.moe_layer(132, 0, H, I, E, k, **kw)
    plain, packed = _layer_pair(B, layer)
    X = B.bf16_tensor(synth.token_rows(132, T, H))
    Y0 = B.moe_ffn_prefill(plain, X, 0)
    Y1 = B.moe_ffn_prefill(packed, X, 0)
    Yb0 = B.moe_ffn_prefill(plain, X, 1)
    Yb1 = B.moe_ffn_prefill(packed, X, 1)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int32), Y1.view(torch.int32))
    assert torch.equal(Yb0.view(torch.int16), Yb1.view(torch.int16))


def test_prefill_group_major_oracle(B):
    """A packed layer against the oracle directly (tokens routed within the tie band
    are left out: their expert choice is checked by the other prefill tests)."""
    T, H, I, E, k = 200, 256, 128, 16, 4
    layer = synth.moe_layer(133, 0, H, I, E, k)
    _, packed = _layer_pair(B, layer)
    Xb = synth.token_rows(133, T, H)
    Y = B.moe_ffn_prefill(packed, B.bf16_tensor(Xb), 0)
    torch.cuda.synchronize()
    ref, _, _, logits = orc.moe_ffn_prefill(layer, Xb)
    srt = np.sort(logits, axis=1)[:, ::-1]
    clear = srt[:, k - 1] - srt[:, k] > 1e-3
    got = to_f64(Y)
    assert clear.sum() > T // 2
    assert rel_l2(got[clear], ref[clear]) <= REL_L2_TOL


def test_decode_ignores_group_major(B):
    """Decode reads the row-major codes: a packed layer gives the same bits."""
    layer = synth.moe_layer(134, 0, 256, 128, 16, 4)
    plain, packed = _layer_pair(B, layer)
    x = B.bf16_tensor(synth.token_rows(134, 1, 256)[0])
    y0 = B.moe_ffn_decode(plain, x, 0)
    y1 = B.moe_ffn_decode(packed, x, 0)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
