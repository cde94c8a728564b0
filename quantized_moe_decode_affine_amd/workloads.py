"""Device-resident workloads driven through the C ABI (used by bench.py and the
full-size tests).

* :class:`DecodeStack`: ``n_layers`` independent MoE layers (hidden 2048, 256
  routed + 1 shared expert, top-8, Q4 g64; about 455 MB each) and a batch-1
  decode loop.  Step s feeds layer l a seeded hidden vector x[s][l]; layers
  run in order on one stream, each a full router -> top-k -> experts chain.
* Byte and FLOP counts of the algorithmic work of each workload.
"""
from __future__ import annotations

import ctypes

import torch

from . import binding as B
from . import synth

GROUP = 64


def q4_matrix_bytes(n: int, k: int) -> int:
    """Bytes of one Q4 matrix: 4 bits per weight plus a bf16 scale and bias per 64 weights."""
    return n * k // 2 + 2 * 2 * n * (k // GROUP)


def q8_matrix_bytes(n: int, k: int) -> int:
    """Bytes of one affine-Q8 matrix: 8 bits per weight plus a bf16 scale and bias per 64 weights."""
    return n * k + 2 * 2 * n * (k // GROUP)


def decode_layer_bytes(hidden=synth.HIDDEN, inter=synth.INTER, n_experts=synth.N_EXPERTS, top_k=synth.TOP_K,
                       shared=True, out_bytes=4) -> int:
    """Algorithmic bytes of one decode MoE layer: the selected experts' weights (and the shared
    expert's), the bf16 router, the bf16 input and the output vector."""
    expert = 2 * q4_matrix_bytes(inter, hidden) + q4_matrix_bytes(hidden, inter)
    return (top_k + (1 if shared else 0)) * expert + n_experts * hidden * 2 + hidden * 2 + hidden * out_bytes


def prefill_expert_flops(T=2048, hidden=synth.HIDDEN, inter=synth.INTER, top_k=synth.TOP_K, shared=True) -> int:
    """FLOPs of the expert GEMMs of one prefill chunk (gate, up and down; 2 per multiply-add)."""
    return 2 * T * (top_k + (1 if shared else 0)) * 3 * hidden * inter


class DecodeStack:
    """n_layers MoE layers on the device plus the per-(step, layer) decode inputs."""

    def __init__(self, seed: int = 2, n_layers: int = 40, n_steps: int = 64, device="cuda", keep_host=(),
                 progress=None, **shape):
        self.seed, self.n_layers, self.n_steps = seed, n_layers, n_steps
        self.layers, self.host = [], {}
        for l in range(n_layers):
            lay = synth.moe_layer(seed, l, **shape)
            self.layers.append(B.DeviceLayer(lay, device))
            if l in keep_host:
                self.host[l] = lay
            del lay
            if progress:
                progress(l)
        H = self.layers[0].hidden
        xs = [[synth.hidden_vector(seed, s, l, H) for l in range(n_layers)] for s in range(n_steps)]
        import numpy as np
        self.x = B.bf16_tensor(np.asarray(xs, dtype=np.uint16), device)          # [steps][layers][H]
        self.y = torch.empty((n_layers, H), dtype=torch.float32, device=device)
        self.ids = torch.empty((n_layers, self.layers[0].top_k), dtype=torch.int32, device=device)
        self.ws = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE, self.layers[0]), device)
        lib = B.load_library()
        self._fn = lib.moe_ffn_decode
        self._refs = [ctypes.byref(d.struct) for d in self.layers]

    @property
    def weight_bytes(self) -> int:
        return sum(d.nbytes for d in self.layers)

    def step(self, s: int, record_ids: bool = False, events=None, ids_buf=None) -> None:
        """Enqueue one decode step (all layers, in order) on the current stream.

        The step's expert ids go to ``self.ids`` when `record_ids`, or to `ids_buf`
        (int32 [n_layers][top_k]) when given.  `events`, when given, is a list of
        (start, end) torch.cuda.Event pairs, one per layer, recorded around each
        layer's launch on the same stream."""
        stream = torch.cuda.current_stream().cuda_stream
        xs = self.x[s % self.n_steps]
        H = self.y.shape[1]
        x0, y0 = xs.data_ptr(), self.y.data_ptr()
        if ids_buf is not None:
            record_ids = True
        ids0, kk = (ids_buf if ids_buf is not None else self.ids).data_ptr(), self.ids.shape[1]
        ws, wsn = self.ws.data_ptr(), self.ws.numel()
        for l in range(self.n_layers):
            if events is not None:
                events[l][0].record()
            st = self._fn(self._refs[l], x0 + 2 * H * l, y0 + 4 * H * l, B.OUT_F32,
                          (ids0 + 4 * kk * l) if record_ids else None, None, ws, wsn, stream)
            if events is not None:
                events[l][1].record()
            if st != B.OK:
                B._check("moe_ffn_decode", st)

    def check(self) -> None:
        """Synchronise and raise binding.DecodeTimeout if any layer launch abandoned a wait."""
        B.check_decode_workspace(self.ws)

    def enable_q8_router(self, device="cuda") -> None:
        """Give every layer an affine-Q8 router (drawn as synth.moe_layer draws one) in place
        of its bf16 router; :meth:`step` then runs the layers with it.  Only the router
        changes: the experts are the same device tensors."""
        H, E = self.layers[0].hidden, self.layers[0].n_experts
        self.q8_routers, self._refs_q8 = [], []
        for l, d in enumerate(self.layers):
            m = B.DeviceQ4(*synth.q8_matrix(self.seed, l, synth.ROUTER_STREAM, 0, E, H, scale_std=0.02 / 74),
                           device=device)
            st = B.q4moe_layer()
            ctypes.pointer(st)[0] = d.struct  # a copy of the layer's descriptor
            st.router_q8 = m.struct
            self.q8_routers.append((m, st))
            self._refs_q8.append(ctypes.byref(st))
        self._refs_bf16 = self._refs

    def enable_q8_shared(self, device="cuda") -> None:
        """Also give every layer's 8-bit-router descriptor an affine-Q8 shared expert (drawn as
        synth.moe_layer draws one with shared_bits=8): the checkpoint's form, an 8-bit router and
        an 8-bit shared expert.  :meth:`use_q8_router` then runs the layers in that form."""
        H, I, E = self.layers[0].hidden, self.layers[0].inter, self.layers[0].n_experts
        self.q8_shared = []
        for l, (_, st) in enumerate(self.q8_routers):
            mats = [B.DeviceQ4(*synth.q8_matrix(self.seed, l, E, which, n, k), device=device)
                    for which, n, k in ((synth.GATE, I, H), (synth.UP, I, H), (synth.DOWN, H, I))]
            st.sh_gate, st.sh_up, st.sh_down = (m.struct for m in mats)
            self.q8_shared.append(mats)

    def use_q8_router(self, on: bool) -> None:
        self._refs = self._refs_q8 if on else self._refs_bf16

    def enable_batch(self, max_batch: int = 8, device="cuda") -> None:
        """Inputs for batched steps: x[s][l][b] drawn like the batch-1 inputs (seeded per
        step, layer and row), outputs, ids and one workspace sized for max_batch rows."""
        import numpy as np
        H, k = self.layers[0].hidden, self.layers[0].top_k
        xb = [[[synth.hidden_vector(self.seed, 1000 + s * max_batch + b, l, H) for b in range(max_batch)]
               for l in range(self.n_layers)] for s in range(self.n_steps)]
        self.xb = B.bf16_tensor(np.asarray(xb, dtype=np.uint16), device)       # [steps][layers][max_batch][H]
        self.yb = torch.empty((self.n_layers, max_batch, H), dtype=torch.float32, device=device)
        self.idsb = torch.empty((self.n_layers, max_batch, k), dtype=torch.int32, device=device)
        self.wsb = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE_BATCH, self.layers[0], rows=max_batch), device)
        self.max_batch = max_batch
        self._fnb = B.load_library().moe_ffn_decode_batch

    def step_batch(self, s: int, nb: int, record_ids: bool = False) -> None:
        """Enqueue one batched decode step of nb rows (all layers, in order) on the current stream."""
        stream = torch.cuda.current_stream().cuda_stream
        xs = self.xb[s % self.n_steps]
        mb, H = self.max_batch, self.yb.shape[2]
        k = self.idsb.shape[2]
        x0, y0, ids0 = xs.data_ptr(), self.yb.data_ptr(), self.idsb.data_ptr()
        ws, wsn = self.wsb.data_ptr(), self.wsb.numel()
        for l in range(self.n_layers):
            st = self._fnb(self._refs[l], x0 + 2 * H * mb * l, nb, y0 + 4 * H * mb * l, B.OUT_F32,
                           (ids0 + 4 * k * mb * l) if record_ids else None, None, ws, wsn, stream)
            if st != B.OK:
                B._check("moe_ffn_decode_batch", st)


class DecodeChain:
    """A decode step with every layer on the GPU: x_{l+1} = bf16(x_l + layer_l(x_l)) through
    the layers (``moe_ffn_decode`` in its residual form, each writing the next layer's
    input), then the LM-head argmax of the last x.  The step can be enqueued launch by
    launch or captured once into a HIP graph and replayed, which takes the host off the
    step's critical path: one replay call instead of one call per layer.

    ``xs[0]`` is the step's input; the caller writes it (outside any graph) before a step."""

    def __init__(self, layers, lm_head, device="cuda"):
        self.layers, self.lm = list(layers), lm_head
        H, k, L = self.layers[0].hidden, self.layers[0].top_k, len(self.layers)
        self.xs = torch.zeros((L + 1, H), dtype=torch.bfloat16, device=device)   # x_0 .. x_L
        self.ids = torch.zeros((L, k), dtype=torch.int32, device=device)
        self.token = torch.zeros(1, dtype=torch.int32, device=device)
        self.max_logit = torch.zeros(1, dtype=torch.float32, device=device)
        self.ws = B.workspace(B.workspace_bytes(B.OP_FFN_DECODE, self.layers[0]), device)
        self.ws_lm = B.workspace(B.workspace_bytes(B.OP_LMHEAD, W=lm_head, rows=1), device)
        lib = B.load_library()
        self._fn, self._lm = lib.moe_ffn_decode, lib.lmhead_argmax
        self._refs = [ctypes.byref(d.struct) for d in self.layers]
        self._lm_ref = ctypes.byref(lm_head.struct)
        self.graph = None

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    def enqueue(self) -> None:
        """Enqueue one step (every layer, then the LM head) on the current stream."""
        stream = torch.cuda.current_stream().cuda_stream
        H, k = self.xs.shape[1], self.ids.shape[1]
        x0, ids0 = self.xs.data_ptr(), self.ids.data_ptr()
        ws, wsn = self.ws.data_ptr(), self.ws.numel()
        for l in range(self.n_layers):
            st = self._fn(self._refs[l], x0 + 2 * H * l, x0 + 2 * H * (l + 1), B.OUT_BF16_RESIDUAL,
                          ids0 + 4 * k * l, None, ws, wsn, stream)
            if st != B.OK:
                B._check("moe_ffn_decode", st)
        st = self._lm(self._lm_ref, x0 + 2 * H * self.n_layers, 1, self.token.data_ptr(), self.max_logit.data_ptr(),
                      self.ws_lm.data_ptr(), self.ws_lm.numel(), stream)
        if st != B.OK:
            B._check("lmhead_argmax", st)

    def capture(self) -> None:
        """Run one step eagerly (so every host-side query the calls make is answered and
        cached), then capture a step into a graph."""
        self.enqueue()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.enqueue()
        torch.cuda.synchronize()
        self.graph = g

    def replay(self) -> None:
        self.graph.replay()

    def check(self) -> None:
        """Synchronise and raise binding.DecodeTimeout if any layer launch abandoned a wait."""
        B.check_decode_workspace(self.ws)
