"""moe_ffn_decode_noalloc (the decode call on the library's fixed scratch array) against
moe_ffn_decode with a workspace: the same kernels, so ids, weights and outputs must be
identical bit for bit.  Two calls in a row, the second with a smaller layer, then the
first layer again (the scratch keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

from oracle import q4moe_oracle as orc
from quantized_moe_decode_affine_amd import synth
from tests.parity_util import REL_L2_TOL, rel_l2, routing_ok, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_decode_affine_amd import binding
    binding.load_library()
    return binding


def _both(B, dl, x_bits, out_dtype):
    H, k = dl.hidden, dl.top_k
    x = B.bf16_tensor(x_bits)
    dt = torch.float32 if out_dtype == B.OUT_F32 else torch.bfloat16
    y_ws, y_na = torch.empty(H, dtype=dt, device=DEV), torch.empty(H, dtype=dt, device=DEV)
    ids_ws, ids_na = (torch.empty(k, dtype=torch.int32, device=DEV) for _ in range(2))
    w_ws, w_na = (torch.empty(k, dtype=torch.float32, device=DEV) for _ in range(2))
    B.moe_ffn_decode(dl, x, out_dtype, out=y_ws, ids_out=ids_ws, w_out=w_ws)
    B.moe_ffn_decode_noalloc(dl, x, out_dtype, out=y_na, ids_out=ids_na, w_out=w_na)
    torch.cuda.synchronize()
    assert torch.equal(ids_ws, ids_na)
    assert torch.equal(w_ws, w_na)
    assert torch.equal(y_ws.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       y_na.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    return y_na, ids_na


def test_noalloc_matches_workspace_form(B):
    big = synth.moe_layer(110, 0)                                   # hidden 2048, inter 512, 256 + 1 experts, top-8
    small = synth.moe_layer(111, 0, 256, 128, 16, 4)               # a smaller layer second
    dbig, dsmall = B.DeviceLayer(big), B.DeviceLayer(small)
    for step, (layer, dl, H) in enumerate([(big, dbig, 2048), (small, dsmall, 256), (big, dbig, 2048)]):
        x_bits = synth.hidden_vector(110, step, 0, H)
        say(f"noalloc call {step}: hidden {H}")
        y, ids = _both(B, dl, x_bits, B.OUT_F32)
        _both(B, dl, x_bits, B.OUT_BF16)
        # and to the oracle's bar, on its own routing within the tie band
        ref, _, _, logits = orc.moe_ffn_token(layer, x_bits)
        gids = ids.cpu().numpy()
        ok, exact = routing_ok(gids, logits, layer.top_k)
        assert ok
        if not exact:
            ref, _, _, _ = orc.moe_ffn_token(layer, x_bits, ids=gids)
        assert rel_l2(y.cpu().double().numpy(), ref) <= REL_L2_TOL


def test_noalloc_rejects_layers_beyond_the_scratch(B):
    """top-k 32 of 64 experts with intermediate 2048: beyond what the decode kernel takes
    (its workspace would exceed the 1 MiB scratch as well)."""
    layer = synth.moe_layer(112, 0, 256, 2048, 64, 32, shared=True)
    dl = B.DeviceLayer(layer)
    x = B.bf16_tensor(synth.hidden_vector(112, 0, 0, 256))
    y = torch.empty(256, dtype=torch.float32, device=DEV)
    with pytest.raises(B.Q4Error) as err:
        B.moe_ffn_decode_noalloc(dl, x, B.OUT_F32, out=y)
    assert err.value.status == B.EUNSUPPORTED
