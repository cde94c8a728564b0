"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and rejects invalid arguments with the
documented status before any HIP call is made."""
import ctypes
import os
import re

import pytest

from quantized_moe_decode_affine_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4moe.h")

A = 0x10000          # fake, well-aligned device addresses: never dereferenced on these paths
A2 = 0x20000


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B._LIB_PATH):
        from quantized_moe_decode_affine_amd import build
        build.build()
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in range(5):
        assert lib.q4moe_strerror(code)
    assert b"unknown" in lib.q4moe_strerror(99)


def _mat(count=1, n=64, k=128, codes=A, scales=A2, biases=A2 + 0x1000):
    return B.q4moe_matrix(codes, scales, biases, count, n, k)


def _layer(H=128, I=64, E=4, k=2, shared=True, **over):
    L = B.q4moe_layer(H, I, E, k, A, _mat(E, I, H), _mat(E, I, H), _mat(E, H, I),
                      *( [_mat(1, I, H), _mat(1, I, H), _mat(1, H, I)] if shared else [B.q4moe_matrix()] * 3))
    for key, v in over.items():
        setattr(L, key, v)
    return L


def test_gemv_rejects(lib):
    s = None
    assert lib.q4_gemv(None, A, A, 0, s) == B.EINVAL
    assert lib.q4_gemv(ctypes.byref(_mat(k=100)), A, A, 0, s) == B.EINVAL        # k % 64
    assert lib.q4_gemv(ctypes.byref(_mat(codes=A + 4)), A, A, 0, s) == B.EINVAL  # codes misaligned
    assert lib.q4_gemv(ctypes.byref(_mat(n=0)), A, A, 0, s) == B.EINVAL
    assert lib.q4_gemv(ctypes.byref(_mat()), None, A, 0, s) == B.EINVAL
    assert lib.q4_gemv(ctypes.byref(_mat()), A + 2, A, 0, s) == B.EINVAL         # x misaligned
    assert lib.q4_gemv(ctypes.byref(_mat()), A, A, 7, s) == B.EINVAL             # out dtype
    assert lib.q4_gemv(ctypes.byref(_mat(k=32768)), A, A, 0, s) == B.EUNSUPPORTED


def test_gemm_rejects(lib):
    W = ctypes.byref(_mat())
    need = lib.q4moe_workspace_bytes(B.OP_GEMM, None, W, 100)
    assert need > 0
    assert lib.q4_gemm(W, A, -1, A, 0, A, need, None) == B.EINVAL
    assert lib.q4_gemm(W, A, 100, A, 0, None, need, None) == B.EWORKSPACE
    assert lib.q4_gemm(W, A, 100, A, 0, A, need - 1, None) == B.EWORKSPACE
    assert lib.q4_gemm(W, A, 100, A, 0, A + 16, need, None) == B.EWORKSPACE      # workspace alignment
    assert lib.q4_gemm(W, A, 0, A, 0, None, 0, None) == B.OK                     # empty: nothing enqueued


def test_route_and_permute_reject(lib):
    need = lib.q4moe_workspace_bytes(B.OP_ROUTE, ctypes.byref(_layer(E=256, k=8)), None, 10)
    assert need >= 10 * 256 * 4
    f = lib.moe_route_topk
    assert f(A, 256, 2048, A, 10, 0, A, A, A, need, None) == B.EINVAL            # top_k 0
    assert f(A, 4, 2048, A, 10, 5, A, A, A, need, None) == B.EINVAL              # top_k > E
    assert f(A, 2048, 2048, A, 10, 8, A, A, A, need, None) == B.EUNSUPPORTED     # E > 1024
    assert f(A, 256, 2048, A, 10, 33, A, A, A, need, None) == B.EUNSUPPORTED     # top_k > 32
    assert f(A, 256, 100, A, 10, 8, A, A, A, need, None) == B.EINVAL             # hidden % 64
    assert f(A, 256, 2048, A, 10, 8, None, A, A, need, None) == B.EINVAL
    assert f(A, 256, 2048, A, 10, 8, A, A, A, 16, None) == B.EWORKSPACE
    assert f(A, 256, 2048, A, 0, 8, A, A, None, 0, None) == B.OK                 # T = 0
    pneed = lib.q4moe_workspace_bytes(B.OP_PERMUTE, ctypes.byref(_layer(E=256, k=8)), None, 2048)
    assert pneed > 0
    g = lib.moe_permute
    assert g(None, 10, 8, 256, A, A, A, A, pneed, None) == B.EINVAL
    assert g(A, 10, 0, 256, A, A, A, A, pneed, None) == B.EINVAL
    assert g(A, 10, 8, 4096, A, A, A, A, pneed, None) == B.EUNSUPPORTED
    assert g(A, 2048, 8, 256, A, A, A, A, 64, None) == B.EWORKSPACE


def test_ffn_rejects(lib):
    good = _layer()
    need_d = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(good), None, 1)
    need_p = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(good), None, 50)
    assert need_d > 0 and need_p > 0
    d, p = lib.moe_ffn_decode, lib.moe_ffn_prefill
    bad_shapes = [
        _layer(hidden=100), _layer(inter=96), _layer(top_k=0), _layer(top_k=5),
        _layer(router=None), _layer(router=A + 8),
    ]
    for L in bad_shapes:
        assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
        assert p(ctypes.byref(L), A, 50, A, 0, A, need_p, None) == B.EINVAL
    L = _layer()
    L.down = _mat(4, 64, 128)            # down must be hidden x inter
    assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
    L = _layer()
    L.sh_up = _mat(2, 64, 128)           # shared expert must have count 1
    assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
    assert d(ctypes.byref(_layer(n_experts=2048, gate=_mat(2048, 64, 128), up=_mat(2048, 64, 128),
                                 down=_mat(2048, 128, 64))), A, A2, 0, None, None, A, need_d, None) == B.EUNSUPPORTED
    assert d(ctypes.byref(good), A, A2, 0, None, None, A, need_d - 1, None) == B.EWORKSPACE
    assert d(ctypes.byref(good), A + 8, A2, 0, None, None, A, need_d, None) == B.EINVAL
    # the residual form writes bf16(x + y): y may not overlap x (hidden 128: x spans 256 bytes)
    for mode in (B.OUT_F32, B.OUT_BF16, B.OUT_BF16_RESIDUAL):
        assert d(ctypes.byref(good), A, A, mode, None, None, A, need_d, None) == B.EINVAL
        assert d(ctypes.byref(good), A, A + 128, mode, None, None, A, need_d, None) == B.EINVAL
        # y just below x: an fp32 y (512 bytes) reaches into x, a bf16 one (256 bytes) does not
        want = B.EINVAL if mode == B.OUT_F32 else B.EWORKSPACE
        assert d(ctypes.byref(good), A + 256, A, mode, None, None, A, need_d - 1, None) == want
        assert d(ctypes.byref(good), A, A + 256, mode, None, None, A, need_d - 1, None) == B.EWORKSPACE
    assert d(ctypes.byref(good), A, A2, 3, None, None, A, need_d, None) == B.EINVAL
    # the residual form is decode-only
    assert p(ctypes.byref(good), A, 50, A2, B.OUT_BF16_RESIDUAL, A, need_p, None) == B.EINVAL
    assert p(ctypes.byref(good), A, -3, A, 0, A, need_p, None) == B.EINVAL
    assert p(ctypes.byref(good), A, 50, A, 0, A, need_p - 256, None) == B.EWORKSPACE
    assert p(ctypes.byref(good), A, 0, A, 0, None, 0, None) == B.OK
    # a layer without a shared expert is valid and needs no more workspace
    noshared = _layer(shared=False)
    assert lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(noshared), None, 50) < need_p


def test_route_topk_q8_rejects(lib):
    r8 = _mat(1, 256, 2048)
    r8.bits = 8
    need = lib.q4moe_workspace_bytes(B.OP_ROUTE, ctypes.byref(_layer(E=256, k=8)), None, 10)
    f = lib.moe_route_topk_q8
    assert f(ctypes.byref(_mat(1, 256, 2048)), A, 10, 8, A, A, A, need, None) == B.EINVAL   # 4-bit codes
    r2 = _mat(2, 256, 2048)
    r2.bits = 8
    assert f(ctypes.byref(r2), A, 10, 8, A, A, A, need, None) == B.EINVAL                  # count 2
    assert f(ctypes.byref(r8), A, 10, 0, A, A, A, need, None) == B.EINVAL                  # top_k 0
    assert f(ctypes.byref(r8), A, 10, 257, A, A, A, need, None) == B.EINVAL                # top_k > E
    assert f(ctypes.byref(r8), A, 10, 33, A, A, A, need, None) == B.EUNSUPPORTED           # top_k > 32
    big = _mat(1, 2048, 2048)
    big.bits = 8
    assert f(ctypes.byref(big), A, 10, 8, A, A, A, need, None) == B.EUNSUPPORTED           # E > 1024
    assert f(ctypes.byref(r8), A + 8, 10, 8, A, A, A, need, None) == B.EINVAL              # X misaligned
    assert f(ctypes.byref(r8), A, 10, 8, None, A, A, need, None) == B.EINVAL               # ids null
    assert f(ctypes.byref(r8), A, 10, 8, A, A, A, 16, None) == B.EWORKSPACE
    assert f(ctypes.byref(r8), A, 0, 8, A, A, None, 0, None) == B.OK                       # T = 0


def test_decode_needs_coresident_workgroups(lib):
    """Every argument valid, but the call cannot confirm that one workgroup per CU fits on
    the device (here: no device at all): it refuses with EUNSUPPORTED and launches nothing,
    since its workgroups wait on each other's words."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the occupancy query can pass")
    good = _layer()
    need = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(good), None, 1)
    for mode in (B.OUT_F32, B.OUT_BF16, B.OUT_BF16_RESIDUAL):
        assert lib.moe_ffn_decode(ctypes.byref(good), A, A2, mode, None, None, A, need, None) == B.EUNSUPPORTED


def test_decode_batch_rejects(lib):
    good = _layer()
    need = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(good), None, 4)
    assert need > 0
    assert lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(good), None, 1) < need
    assert lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(good), None, 0) == 0
    assert lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(good), None, 9) == 0
    f = lib.moe_ffn_decode_batch
    assert f(ctypes.byref(_layer(hidden=100)), A, 4, A, 0, None, None, A, need, None) == B.EINVAL
    assert f(ctypes.byref(good), A, 0, A, 0, None, None, A, need, None) == B.EINVAL
    assert f(ctypes.byref(good), A, 9, A, 0, None, None, A, need, None) == B.EUNSUPPORTED
    assert f(ctypes.byref(good), None, 4, A, 0, None, None, A, need, None) == B.EINVAL
    assert f(ctypes.byref(good), A + 8, 4, A, 0, None, None, A, need, None) == B.EINVAL
    assert f(ctypes.byref(good), A, 4, A, 2, None, None, A, need, None) == B.EINVAL
    assert f(ctypes.byref(good), A, 4, A, 0, None, None, A, need - 256, None) == B.EWORKSPACE
    assert f(ctypes.byref(good), A, 4, A, 0, None, None, A + 16, need, None) == B.EWORKSPACE
    # staged SwiGLU outputs of one token beyond 64 KB of LDS: 33 slots x 4096 inter
    wide = _layer(H=128, I=4096, E=64, k=32, gate=_mat(64, 4096, 128), up=_mat(64, 4096, 128),
                  down=_mat(64, 128, 4096), sh_gate=_mat(1, 4096, 128), sh_up=_mat(1, 4096, 128),
                  sh_down=_mat(1, 128, 4096))
    wneed = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(wide), None, 2)
    assert f(ctypes.byref(wide), A, 2, A, 0, None, None, A, wneed, None) == B.EUNSUPPORTED


def test_lmhead_rejects(lib):
    W = ctypes.byref(_mat(1, 1000, 2048))
    need = lib.q4moe_workspace_bytes(B.OP_LMHEAD, None, W, 4)
    assert need > 0
    f = lib.lmhead_argmax
    assert f(W, A, 0, A, None, A, need, None) == B.EINVAL
    assert f(W, A, 9, A, None, A, need, None) == B.EUNSUPPORTED
    assert f(W, A, 4, None, None, A, need, None) == B.EINVAL
    assert f(W, A, 4, A, None, A, need - 8, None) == B.EWORKSPACE
    assert f(ctypes.byref(_mat(1, 1000, 8192)), A, 4, A, None, A, need, None) == B.EUNSUPPORTED


def test_group_major_rejects(lib):
    f = lib.q4moe_pack_group_major
    W = _mat(2, 64, 128)                                   # codes span 2*64*128/2 = 8 KiB from A
    assert f(None, A2 + 0x10000, None) == B.EINVAL
    assert f(ctypes.byref(W), None, None) == B.EINVAL
    assert f(ctypes.byref(W), A2 + 0x10004, None) == B.EINVAL    # dst misaligned
    assert f(ctypes.byref(W), A + 0x1000, None) == B.EINVAL      # dst overlaps the codes
    assert f(ctypes.byref(_mat(k=100)), A2 + 0x10000, None) == B.EINVAL
    q8 = B.q4moe_matrix(A, A2, A2 + 0x1000, 1, 64, 128, 8)
    assert f(ctypes.byref(q8), A2 + 0x10000, None) == B.EUNSUPPORTED
    # a group-major copy must be 16-byte aligned and belongs to 4-bit matrices only
    bad = _mat()
    bad.codes_gm = A2 + 0x10008
    assert lib.q4_gemv(ctypes.byref(bad), A, A, 0, None) == B.EINVAL
    q8.codes_gm = A2 + 0x10000
    assert lib.q4_gemv(ctypes.byref(q8), A, A, 0, None) == B.EINVAL
    L = _layer()
    L.down.codes_gm = A2 + 0x10008
    need_p = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(L), None, 50)
    assert lib.moe_ffn_prefill(ctypes.byref(L), A, 50, A, 0, A, need_p, None) == B.EINVAL


def test_workspace_queries(lib):
    assert lib.q4moe_workspace_bytes(B.OP_GEMV, None, None, 1) == 0
    assert lib.q4moe_workspace_bytes(99, None, None, 1) == 0
    assert lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(_layer(hidden=100)), None, 1) == 0
    assert lib.q4moe_workspace_bytes(B.OP_GEMM, None, None, 5) == 0
    small = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(_layer()), None, 10)
    big = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(_layer()), None, 1000)
    assert 0 < small < big


def test_q8_matrices_rejected_where_unsupported(lib):
    """8-bit matrices: accepted by the GEMV and the LM head only; an unknown width is invalid."""
    def m8(count=1, n=64, k=128, **kw):
        w = _mat(count, n, k, **kw)
        w.bits = 8
        return w
    bad = _mat(1, 64, 128)
    bad.bits = 7
    assert lib.q4_gemv(ctypes.byref(bad), A, A2, 0, None) == B.EINVAL
    need_g = lib.q4moe_workspace_bytes(B.OP_GEMM, None, ctypes.byref(m8()), 10)
    assert lib.q4_gemm(ctypes.byref(m8()), A, 10, A2, 0, A, need_g, None) == B.EUNSUPPORTED
    # a layer whose matrices are 8-bit
    L = _layer()
    L.up = m8(4, 64, 128)
    need_d = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(_layer()), None, 1)
    assert lib.moe_ffn_decode(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EUNSUPPORTED
    L = _layer()
    L.sh_down = m8(1, 128, 64)
    assert lib.moe_ffn_decode(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EUNSUPPORTED
    # LM head: up to 8 batch rows at 8 bits; short workspace before any launch
    W = ctypes.byref(m8(1, 1000, 2048))
    need8 = lib.q4moe_workspace_bytes(B.OP_LMHEAD, None, W, 8)
    f = lib.lmhead_argmax
    assert f(W, A, 9, A2, None, A, need8 * 2, None) == B.EUNSUPPORTED
    assert f(W, A, 8, A2, None, A, need8 - 1, None) == B.EWORKSPACE
    assert f(ctypes.byref(m8(1, 10, 16384)), A, 1, A2, None, A, need8, None) == B.EUNSUPPORTED


def test_q8_router_layers(lib):
    """An 8-bit router replaces the bf16 one in the layer calls; it must be one 8-bit
    n_experts x hidden matrix."""
    def rq8(E=4, H=128, bits=8):
        m = _mat(1, E, H)
        m.bits = bits
        return m
    L = _layer(router=None)
    L.router_q8 = rq8()
    need_d = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(L), None, 1)
    assert need_d > 0
    d = lib.moe_ffn_decode
    assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d - 1, None) == B.EWORKSPACE  # valid up to the workspace
    for bad in (rq8(bits=4), rq8(E=5), rq8(H=64)):
        L.router_q8 = bad
        assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
    L.router_q8 = rq8()
    need_p = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(L), None, 50)
    assert lib.moe_ffn_prefill(ctypes.byref(L), A, 50, A2, 0, A, need_p - 256, None) == B.EWORKSPACE
    need_b = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(L), None, 2)
    assert lib.moe_ffn_decode_batch(ctypes.byref(L), A, 2, A2, 0, None, None, A, need_b - 256, None) == B.EWORKSPACE


def test_shared_gate_layers(lib):
    """A shared-expert gate needs a shared expert and 16-byte alignment; every layer call takes one."""
    need_d = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(_layer()), None, 1)
    d = lib.moe_ffn_decode
    L = _layer(sh_gate_w=A)
    assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d - 1, None) == B.EWORKSPACE  # valid up to the workspace
    assert d(ctypes.byref(_layer(sh_gate_w=A + 2)), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
    assert d(ctypes.byref(_layer(shared=False, sh_gate_w=A)), A, A2, 0, None, None, A, need_d, None) == B.EINVAL
    need_p = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(L), None, 50)
    assert lib.moe_ffn_prefill(ctypes.byref(L), A, 50, A2, 0, A, need_p - 1, None) == B.EWORKSPACE
    need_b = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(L), None, 2)
    assert lib.moe_ffn_decode_batch(ctypes.byref(L), A, 2, A2, 0, None, None, A, need_b - 1, None) == B.EWORKSPACE


def test_q8_shared_expert_layers(lib):
    """An 8-bit shared expert (all three matrices) is taken by the decode calls; a mix of
    4- and 8-bit shared matrices is rejected everywhere."""
    def q8(n, k):
        m = _mat(1, n, k)
        m.bits = 8
        return m
    H, I = 128, 64
    L = _layer(sh_gate=q8(I, H), sh_up=q8(I, H), sh_down=q8(H, I))
    need_d = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE, ctypes.byref(L), None, 1)
    assert need_d > 0
    d = lib.moe_ffn_decode
    assert d(ctypes.byref(L), A, A2, 0, None, None, A, need_d - 1, None) == B.EWORKSPACE  # valid up to the workspace
    need_p = lib.q4moe_workspace_bytes(B.OP_FFN_PREFILL, ctypes.byref(L), None, 50)
    assert lib.moe_ffn_prefill(ctypes.byref(L), A, 50, A2, 0, A, need_p - 1, None) == B.EWORKSPACE
    need_b = lib.q4moe_workspace_bytes(B.OP_FFN_DECODE_BATCH, ctypes.byref(L), None, 2)
    assert lib.moe_ffn_decode_batch(ctypes.byref(L), A, 2, A2, 0, None, None, A, need_b - 1, None) == B.EWORKSPACE
    mixed = _layer(sh_gate=q8(I, H), sh_up=q8(I, H))
    assert d(ctypes.byref(mixed), A, A2, 0, None, None, A, need_d, None) == B.EUNSUPPORTED


def test_binding_structs_match_header(tmp_path):
    """The ctypes structures have the header's sizes and field offsets (gcc reads the header)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    checks = []
    for cname, cls in (("q4moe_matrix", B.q4moe_matrix), ("q4moe_layer", B.q4moe_layer)):
        checks.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            checks.append(f'printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "q4moe.h"\nint main(void) {\n'
                   + "\n".join(checks) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(line.split()[:2]): int(line.split()[2]) for line in out if line}
    for cname, cls in (("q4moe_matrix", B.q4moe_matrix), ("q4moe_layer", B.q4moe_layer)):
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert got[(cname, field)] == getattr(cls, field).offset, (cname, field)
