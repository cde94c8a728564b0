"""Shared helpers of the GPU parity tests (tolerances, routing tie band)."""
import sys

import numpy as np

# Float outputs: relative L2 error against the fp64 oracle (the target's bar).
REL_L2_TOL = 2e-3
# Integer decisions taken from floats (top-k ids, argmax) must match exactly
# unless the deciding logit gap is within this band (logit space).
TIE_BAND = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


# bfloat16 keeps 8 significant bits: rounding alone moves a value by up to 2^-8 of itself.
BF16_HALF_ULP_REL = 2.0 ** -8


def bf16_bits_of_f32(t) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bfloat16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(t.detach().cpu().numpy().astype(np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_bf16_output(got_bf16, got_f32, ref) -> None:
    """A bf16 output must be exactly the rounding of the same call's fp32 output, and lie
    within bfloat16's own rounding bound of the oracle."""
    np.testing.assert_array_equal(bf16_bits(got_bf16), bf16_bits_of_f32(got_f32))
    assert rel_l2(to_f64(got_bf16), ref) <= BF16_HALF_ULP_REL


def to_f64(t) -> np.ndarray:
    """A torch tensor (float32 or bfloat16, any device) -> float64 numpy (exact)."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def routing_ok(gpu_ids, logits_row, k: int, band: float = TIE_BAND):
    """(ok, exact): the GPU's top-k set is the oracle's, or differs only in experts
    whose logits lie within `band` of the k/k+1 boundary; `exact` also requires the
    same order wherever adjacent selected logits differ by more than `band`."""
    L = np.asarray(logits_row, dtype=np.float64)
    g = [int(v) for v in gpu_ids]
    order = sorted(range(L.size), key=lambda e: (-L[e], e))
    ref = order[:k]
    if len(set(g)) != k or min(g) < 0 or max(g) >= L.size:
        return False, False
    if set(g) != set(ref):
        vk = L[ref[-1]]
        vk1 = L[order[k]] if k < L.size else -np.inf
        for e in set(g) ^ set(ref):
            if not (vk1 - band <= L[e] <= vk + band):
                return False, False
    # order: the GPU list must be descending in logit up to the band
    for a, b in zip(g, g[1:]):
        if L[a] < L[b] - band:
            return False, False
    return True, g == ref
