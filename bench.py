#!/usr/bin/env python
"""Benchmark of the affine-Q4 MoE hot path on one MI355X.

Headline (`value`): HBM GB/s of the batch-1 decode MoE layer over a 40-layer
decode loop (hidden 2048, 256 routed + 1 shared expert, top-8, Q4 g64; about
18 GB of weights, far beyond the caches).  A step is one decode token through
all 40 layers, each a dependent router -> top-k -> experts chain; `--steps`
steps are timed after `--warmup` untimed ones.  Bytes per layer are the
algorithmic ones: the 9 touched experts at 4.5 bits per weight, the bf16
router, the bf16 input and the fp32 output.

Also reported: the same 40 layers chained through a residual stream and ended
by the LM-head argmax, as one decode step per token, enqueued launch by launch
and replayed from a captured HIP graph; the 2,048-token prefill chunk through one layer (grouped-GEMM
TFLOP/s against the bf16 MFMA peak), the LM-head GEMV + argmax
(151,936 x 2048, two weight copies alternated so the 175 MB matrix is not
cache-resident), and the CPU oracle timed on a bounded sample of the decode
workload.  All inputs are seeded and synthetic.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "decode MoE-layer GEMV HBM GB/s (% of peak) + prefill grouped-GEMM TFLOP/s"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_traffic():
    """HBM bytes per decode-layer launch from the committed rocprofv3 counter
    summary, or None when the decode kernel's sources changed since it was taken."""
    import re

    from quantized_moe_decode_affine_amd import profsum

    path = os.path.join(ROOT, "profiles", "decode_layer_kernel_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"decode sources sha256: ([0-9a-f]{64})", text)
    m_val = re.search(r"traffic bytes per launch: ([0-9]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != profsum.decode_sources_sha256():
        return None
    return int(m_val.group(1))


def profiled_gemm_us():
    """Per-layer time of the two grouped-GEMM launches of the prefill layer (gate/up
    with SwiGLU, down with the routing weight), from the committed rocprofv3 kernel
    trace; None when the kernel sources changed since the trace was taken."""
    import re

    from quantized_moe_decode_affine_amd import profsum

    path = os.path.join(ROOT, "profiles", "kernels_decode40_prefill2048_lmhead_trace.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel sources sha256: ([0-9a-f]{64})", text)
    m_row = re.search(r"\| `grouped_q4_gemm_kernel` \| (\d+) \| ([0-9.]+) \|", text)
    if not m_hash or not m_row or m_hash.group(1) != profsum.all_sources_sha256():
        return None
    return 2.0 * float(m_row.group(2))  # two launches per layer


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(stack_host, seed, budget_s=8.0):
    """The oracle (as it stands, numpy float64) timed on the host's cores: the decode
    workload's (step, layer) pairs until ~budget_s (the headline's unit, GB/s of the same
    byte count), and one call of each other configuration on a bounded sample, each at
    all BLAS threads and at one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import q4moe_oracle as orc
    from quantized_moe_decode_affine_amd import synth, workloads

    all_threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    layer0 = stack_host[min(stack_host)]
    x0 = synth.hidden_vector(seed, 0, 0)

    def timed(fn, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps

    # config 0: one GEMV 512 x 2048
    w0 = synth.q4_matrix(0, 0, 0, 0, 512, synth.HIDDEN)
    # config 3 sample: experts 0..15 of the 2,048-token chunk with all the tokens that chose them
    X3 = synth.token_rows(3, 2048, synth.HIDDEN)
    ids3, _, _ = orc.route_topk(layer0.router, X3, layer0.top_k)
    X3f = orc.bf16_to_f64(X3)
    sample_e = 16

    def prefill_sample():
        for e in range(sample_e):
            rows = np.nonzero((ids3 == e).any(axis=1))[0]
            if rows.size:
                orc.expert_ffn(layer0.expert(e), X3f[rows])
    # config 4 sample: 16,384 of the 151,936 LM-head rows, B = 1
    lm_rows = 16384
    w4 = synth.q4_matrix(4, 0, 0, 0, lm_rows, synth.HIDDEN)
    x4 = synth.token_rows(4, 1, synth.HIDDEN, index=1)
    per_config = {}
    for label, limit in (("all_threads", all_threads), ("one_thread", 1)):
        with threadpool_limits(limits=limit):
            c0 = timed(lambda: orc.q4_gemv(*w0, x0), reps=20)
            c1 = timed(lambda: orc.moe_ffn_token(layer0, x0), reps=3)
            c3 = timed(prefill_sample) * (synth.N_EXPERTS + 1) / sample_e
            c4 = timed(lambda: orc.lmhead_argmax(*w4, x4)) * synth.VOCAB / lm_rows
        per_config[label] = {"threads": limit, "config0_gemv_s": round(c0, 6), "config1_layer_s": round(c1, 4),
                             "config3_prefill_chunk_s": round(c3, 3), "config4_lmhead_B1_s": round(c4, 3)}
    # config 2 (the headline's unit): (step, layer) pairs until ~budget_s, all threads
    pairs = [(s, l) for s in range(64) for l in sorted(stack_host)]
    done, t0 = 0, time.perf_counter()
    for s, l in pairs:
        orc.moe_ffn_token(stack_host[l], synth.hidden_vector(seed, s, l))
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 2:
            break
    dt = time.perf_counter() - t0
    bytes_per = workloads.decode_layer_bytes()
    return {"value": round(bytes_per * done / dt / 1e9, 4), "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "sample": f"{done} (step, layer) decode MoE layers of the 40-layer workload, layers {sorted(stack_host)}, "
                      f"steps from 0; {dt:.1f} s wall at {all_threads} BLAS threads; numpy float64 oracle",
            "per_config_wall_s": per_config,
            "per_config_samples": "config 0: one 512x2048 GEMV; config 1: one decode layer (40-layer workload's layer, "
                                  "same shape); config 3: experts 0-15 of a 2,048-token chunk with their tokens, "
                                  "scaled by 257/16 experts; config 4: 16,384 of 151,936 LM-head rows, scaled by rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip every leg but the 40-layer decode loop")
    ap.add_argument("--legs", default="q8router,chain,batch,prefill,prefill_rm,wide,lmhead",
                    help="comma list of the legs run after the decode loop: q8router (the same loop with affine-Q8 "
                         "routers), chain (residual-chained step with the LM head, eager and as a replayed graph), "
                         "batch (several requests per step), prefill (2,048-token chunk), prefill_rm (the same chunk "
                         "reading the expert codes row-major), wide (512 experts, "
                         "top-10), lmhead")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (the known-size reference that scales the "
                         "byte counters of a rocprofv3 --pmc run)")
    args = ap.parse_args()
    legs = set() if args.no_extra else {x for x in args.legs.split(",") if x}
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path is single-GPU)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_moe_decode_affine_amd import binding as B
    from quantized_moe_decode_affine_amd import synth, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load_library()
    dev = "cuda"

    # ---------------------------------------------------------- decode loop
    log(f"building {args.layers} decode layers")
    t0 = time.perf_counter()
    stack = workloads.DecodeStack(seed=2, n_layers=args.layers, n_steps=64, device=dev,
                                  keep_host=(0, 1) if not args.no_cpu else (),
                                  progress=lambda l: log(f"layer {l} uploaded") if l % 10 == 9 else None)
    torch.cuda.synchronize()
    log(f"decode stack ready: {stack.weight_bytes / 1e9:.2f} GB in {time.perf_counter() - t0:.1f} s")

    for s in range(args.warmup):
        stack.step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # two rounds of exactly --steps steps (the measurement contract's repeated rounds): each
    # step's expert ids are recorded, their FNV-1a digest must repeat, the median round is reported
    ids_all = torch.empty((args.steps, args.layers, stack.ids.shape[1]), dtype=torch.int32, device=dev)
    rounds_ms, digests, host_s = [], [], 0.0
    for rnd in range(2):
        torch.cuda.synchronize()
        ev0.record()
        h0 = time.perf_counter()
        for s in range(args.steps):
            stack.step(s, ids_buf=ids_all[s])
        host_s = time.perf_counter() - h0
        ev1.record()
        torch.cuda.synchronize()
        rounds_ms.append(ev0.elapsed_time(ev1))
        digests.append(synth.fnv1a64(ids_all.cpu().numpy()))
        stack.check()  # no decode launch abandoned a wait (else its outputs are wrong)
    ms = float(np.median(rounds_ms))
    ms_step = ms / args.steps
    layer_bytes = workloads.decode_layer_bytes()
    step_bytes = layer_bytes * args.layers
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    layer_us = ms_step * 1e3 / args.layers
    log(f"decode: {ms_step * 1e3:.1f} us/step, {layer_us:.2f} us/layer, {gbs:.1f} GB/s; host enqueue "
        f"{host_s / args.steps * 1e6:.1f} us/step")

    digest_ok = digests[0] == digests[1]

    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.layers}-layer MoE decode loop, batch 1 (hidden 2048, 256 routed + 1 shared "
                               f"experts, top-8, SwiGLU, affine Q4 g64 weights, bf16 router); per-step seeded "
                               f"random layer inputs",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "weights_gb": round(stack.weight_bytes / 1e9, 2), "bytes_per_layer": layer_bytes,
                   "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "us_per_layer": round(layer_us, 3),
                   "host_enqueue_us_per_step": round(host_s / args.steps * 1e6, 1),
                   "rounds_ms": [round(r, 4) for r in rounds_ms], "statistic": "median of 2 rounds",
                   "ids_fnv1a64": [f"{d:016x}" for d in digests], "ids_repeat": digest_ok},
        # the timed loop is one decode_layer_kernel launch per layer, back to back on one
        # stream, so its event time / launches is the kernel's average launch duration
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                     "kernel": "decode_layer_kernel (moe_ffn_decode, one launch per layer)",
                     "unit_bytes": layer_bytes, "avg_launch_us": round(layer_us, 3)},
    }
    if "q8router" in legs:
        # ------------------------- the decode loop with the checkpoint's affine-Q8 router gates
        stack.enable_q8_router(dev)
        stack.use_q8_router(True)
        for s in range(args.warmup):
            stack.step(s)
        torch.cuda.synchronize()
        ev0.record()
        for s in range(args.steps):
            stack.step(s)
        ev1.record()
        torch.cuda.synchronize()
        q_us = ev0.elapsed_time(ev1) * 1e3 / (args.steps * args.layers)
        stack.check()
        stack.use_q8_router(False)
        q_bytes = layer_bytes - synth.N_EXPERTS * synth.HIDDEN * 2 + workloads.q8_matrix_bytes(synth.N_EXPERTS,
                                                                                               synth.HIDDEN)
        result["decode_q8_router"] = {
            "workload": f"{args.layers}-layer batch-1 decode loop with affine-Q8 router gates (decode_layer_q8router_kernel)",
            "us_per_layer": round(q_us, 3), "bytes_per_layer": q_bytes,
            "GB_s": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * q_bytes / (q_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        log(f"decode q8 router: {result['decode_q8_router']}")
        # the checkpoint's form: 8-bit router and 8-bit shared expert (decode_layer_q8router_q8shared_kernel)
        stack.enable_q8_shared(dev)
        stack.use_q8_router(True)
        for s in range(args.warmup):
            stack.step(s)
        torch.cuda.synchronize()
        ev0.record()
        for s in range(args.steps):
            stack.step(s)
        ev1.record()
        torch.cuda.synchronize()
        c_us = ev0.elapsed_time(ev1) * 1e3 / (args.steps * args.layers)
        stack.check()
        stack.use_q8_router(False)
        c_bytes = q_bytes - 2 * workloads.q4_matrix_bytes(synth.INTER, synth.HIDDEN) - \
            workloads.q4_matrix_bytes(synth.HIDDEN, synth.INTER) + \
            2 * workloads.q8_matrix_bytes(synth.INTER, synth.HIDDEN) + workloads.q8_matrix_bytes(synth.HIDDEN, synth.INTER)
        result["decode_q8_router"]["with_q8_shared_expert"] = {
            "workload": "the same loop with the shared expert in affine-Q8 codes as well "
                        "(decode_layer_q8router_q8shared_kernel)",
            "us_per_layer": round(c_us, 3), "bytes_per_layer": c_bytes,
            "GB_s": round(c_bytes / (c_us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * c_bytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        log(f"decode q8 router + q8 shared expert: {result['decode_q8_router']['with_q8_shared_expert']}")

    if "chain" in legs:
        # ------------------- residual-chained decode step + LM head: eager launches vs a replayed graph
        log("building the LM head for the chained step")
        mat = synth.lm_head()
        W = B.DeviceQ4(*mat, device=dev)
        del mat
        chain = workloads.DecodeChain(stack.layers, W, dev)
        csteps = 16

        def run_chain(fn):
            for s in range(2):
                chain.xs[0].copy_(stack.x[s % stack.n_steps][0])
                fn()
            torch.cuda.synchronize()
            ev0.record()
            h = time.perf_counter()
            for s in range(csteps):
                chain.xs[0].copy_(stack.x[s % stack.n_steps][0])
                fn()
            host = time.perf_counter() - h
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) * 1e3 / csteps, host * 1e6 / csteps

        e_us, e_host = run_chain(chain.enqueue)
        chain.capture()
        g_us, g_host = run_chain(chain.replay)
        chain.check()
        step_bytes = args.layers * workloads.decode_layer_bytes(out_bytes=2) + \
            workloads.q4_matrix_bytes(synth.VOCAB, synth.HIDDEN) + 2 * synth.HIDDEN
        result["chain"] = {
            "workload": f"decode step: {args.layers} layers chained through a residual stream (moe_ffn_decode "
                        f"writes bf16(x + y)), then the LM-head argmax (151,936 x 2048); one token per step",
            "eager_us_per_step": round(e_us, 1), "eager_host_enqueue_us_per_step": round(e_host, 1),
            "graph_us_per_step": round(g_us, 1), "graph_host_enqueue_us_per_step": round(g_host, 1),
            "graph_tokens_per_s": round(1e6 / g_us, 1), "bytes_per_step": step_bytes,
            "graph_GB_s": round(step_bytes / (g_us * 1e-6) / 1e9, 1)}
        log(f"chain: {result['chain']}")
        del chain, W
        torch.cuda.empty_cache()

    if "batch" in legs:
        # ------------------------------------------- batched decode (several requests per step)
        stack.enable_batch(8, dev)
        expert_bytes = workloads.decode_layer_bytes(top_k=1, shared=False, n_experts=0, out_bytes=0) - 2 * synth.HIDDEN
        batch = {}
        for nb in (1, 4, 8):
            for s in range(2):
                stack.step_batch(s, nb)
            torch.cuda.synchronize()
            bsteps = 16
            ev0.record()
            for s in range(bsteps):
                stack.step_batch(s, nb)
            ev1.record()
            torch.cuda.synchronize()
            b_us = ev0.elapsed_time(ev1) * 1e3 / (bsteps * args.layers)
            stack.step_batch(0, nb, record_ids=True)
            torch.cuda.synchronize()
            ids_nb = stack.idsb[:, :nb].cpu().numpy()
            distinct = float(np.mean([len(np.unique(ids_nb[l])) for l in range(args.layers)]))
            # algorithmic bytes: each distinct expert and the shared one once, the router, inputs and outputs
            b_bytes = (distinct + 1) * expert_bytes + synth.N_EXPERTS * synth.HIDDEN * 2 + nb * synth.HIDDEN * 6
            batch[f"B{nb}"] = {"us_per_layer": round(b_us, 3), "tokens_per_s": round(nb / (b_us * 1e-6 * args.layers), 1),
                               "distinct_experts_per_layer": round(distinct, 2),
                               "GB_s": round(b_bytes / (b_us * 1e-6) / 1e9, 1),
                               "pct_of_hbm_peak": round(100 * b_bytes / (b_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        result["decode_batch"] = dict(
            workload=f"{args.layers}-layer decode loop with B requests per step (moe_ffn_decode_batch: two "
                     f"launches per layer, one for B = 1); tokens_per_s counts all B rows; bytes = distinct + "
                     f"shared experts, router, inputs and outputs",
            batch1_kernel_tokens_per_s=round(1 / (layer_us * 1e-6 * args.layers), 1), **batch)
        log(f"decode batch: {batch}")

    host_layers = dict(stack.host)
    del stack
    torch.cuda.empty_cache()

    if "prefill" in legs:
        # ------------------------------------------------------- prefill chunk
        log("building the prefill layer")
        layer = synth.moe_layer(1)
        dl = B.DeviceLayer(layer, dev)
        dl.pack_group_major()  # the GEMMs read the expert codes group-major (a load-time layout step)
        del layer
        X = B.bf16_tensor(synth.token_rows(3, 2048, synth.HIDDEN), dev)
        ws = B.workspace(B.workspace_bytes(B.OP_FFN_PREFILL, dl, rows=2048), dev)
        Y = torch.empty((2048, synth.HIDDEN), dtype=torch.float32, device=dev)
        for _ in range(2):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        torch.cuda.synchronize()
        reps = 10
        ev0.record()
        for _ in range(reps):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        p_us = ev0.elapsed_time(ev1) * 1e3 / reps
        flops = workloads.prefill_expert_flops()
        tfl = flops / (p_us * 1e-6) / 1e12
        g_us = profiled_gemm_us()
        result["prefill"] = {"workload": "2,048-token chunk through one MoE layer (route, permute, grouped Q4 "
                                         "GEMMs with SwiGLU, combine; expert codes also held group-major)",
                             "us_per_layer": round(p_us, 2), "tokens_per_s": round(2048 / (p_us * 1e-6), 1),
                             "expert_gflop": round(flops / 1e9, 3),
                             "tflops_whole_layer": round(tfl, 2),
                             "pct_of_bf16_peak_whole_layer": round(100 * tfl / BF16_PEAK_TFLOPS, 2),
                             # expert GFLOP over the grouped-GEMM kernels' rocprofv3 time (both launches)
                             "grouped_gemm_us_rocprof": None if g_us is None else round(g_us, 2),
                             "tflops_grouped_gemm": None if g_us is None else round(flops / (g_us * 1e-6) / 1e12, 2),
                             "pct_of_bf16_peak_grouped_gemm":
                                 None if g_us is None else round(100 * flops / (g_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 2)}
        log(f"prefill: {p_us:.1f} us/layer, {tfl:.1f} TFLOP/s over the whole layer")
        # the same chunk with the checkpoint's affine-Q8 router gate (same experts)
        layer = synth.moe_layer(1)
        layer.router_q8 = synth.q8_matrix(1, 0, synth.ROUTER_STREAM, 0, synth.N_EXPERTS, synth.HIDDEN,
                                          scale_std=0.02 / 74)
        dl8 = B.DeviceLayer(layer, dev)
        dl8.pack_group_major()
        del layer
        for _ in range(2):
            B.moe_ffn_prefill(dl8, X, out=Y, ws=ws)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            B.moe_ffn_prefill(dl8, X, out=Y, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        result["prefill"]["q8_router_us_per_layer"] = round(ev0.elapsed_time(ev1) * 1e3 / reps, 2)
        log(f"prefill with q8 router: {result['prefill']['q8_router_us_per_layer']} us/layer")
        del dl, dl8, X, ws, Y
        torch.cuda.empty_cache()

    if "prefill_rm" in legs:
        # ---------------- the same chunk with the expert codes read in their row-major (MLX) layout only
        layer = synth.moe_layer(1)
        dl = B.DeviceLayer(layer, dev)
        del layer
        X = B.bf16_tensor(synth.token_rows(3, 2048, synth.HIDDEN), dev)
        ws = B.workspace(B.workspace_bytes(B.OP_FFN_PREFILL, dl, rows=2048), dev)
        Y = torch.empty((2048, synth.HIDDEN), dtype=torch.float32, device=dev)
        for _ in range(2):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        torch.cuda.synchronize()
        reps = 10
        ev0.record()
        for _ in range(reps):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        rm_us = round(ev0.elapsed_time(ev1) * 1e3 / reps, 2)
        result.setdefault("prefill", {})["row_major_codes_us_per_layer"] = rm_us
        log(f"prefill, row-major codes only: {rm_us} us/layer")
        del dl, X, ws, Y
        torch.cuda.empty_cache()

    if "wide" in legs:
        # ------------------------- wider layers: 512 routed experts, top-10, 4,096-token chunks
        log("building 8 wide layers (512 routed + 1 shared experts, top-10)")
        wide = dict(n_experts=512, top_k=10)
        wstack = workloads.DecodeStack(seed=5, n_layers=8, n_steps=8, device=dev, **wide)
        for s in range(2):
            wstack.step(s)
        torch.cuda.synchronize()
        wsteps = 16
        ev0.record()
        for s in range(wsteps):
            wstack.step(s)
        ev1.record()
        torch.cuda.synchronize()
        w_layer_us = ev0.elapsed_time(ev1) * 1e3 / (wsteps * wstack.n_layers)
        w_bytes = workloads.decode_layer_bytes(**wide)
        dl = wstack.layers[0]
        dl.pack_group_major()
        T4 = 4096
        X = B.bf16_tensor(synth.token_rows(5, T4, synth.HIDDEN), dev)
        ws = B.workspace(B.workspace_bytes(B.OP_FFN_PREFILL, dl, rows=T4), dev)
        Y = torch.empty((T4, synth.HIDDEN), dtype=torch.float32, device=dev)
        for _ in range(2):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        torch.cuda.synchronize()
        reps = 5
        ev0.record()
        for _ in range(reps):
            B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        w_p_us = ev0.elapsed_time(ev1) * 1e3 / reps
        w_flops = workloads.prefill_expert_flops(T=T4, top_k=10)
        result["wide"] = {
            "workload": "512 routed + 1 shared experts, top-10 (hidden 2048, inter 512, affine Q4 g64): "
                        "8-layer batch-1 decode loop and one 4,096-token prefill chunk",
            "decode_us_per_layer": round(w_layer_us, 3), "decode_bytes_per_layer": w_bytes,
            "decode_GB_s": round(w_bytes / (w_layer_us * 1e-6) / 1e9, 1),
            "decode_pct_of_hbm_peak": round(100 * w_bytes / (w_layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "prefill_us_per_layer": round(w_p_us, 2), "prefill_expert_gflop": round(w_flops / 1e9, 3),
            "prefill_tflops_whole_layer": round(w_flops / (w_p_us * 1e-6) / 1e12, 2)}
        log(f"wide: {result['wide']}")
        del wstack, dl, X, ws, Y
        torch.cuda.empty_cache()

    if "lmhead" in legs:
        # ------------------------------------------------------------ LM head
        log("building the LM head (two copies)")
        mat = synth.lm_head()
        Ws = [B.DeviceQ4(*mat, device=dev), B.DeviceQ4(*mat, device=dev)]
        del mat
        lm = {}
        for batch in (1, 4):
            Xh = B.bf16_tensor(synth.token_rows(4, batch, synth.HIDDEN, index=batch), dev)
            wsl = B.workspace(B.workspace_bytes(B.OP_LMHEAD, W=Ws[0], rows=batch), dev)
            for i in range(4):
                B.lmhead_argmax(Ws[i % 2], Xh, ws=wsl)
            torch.cuda.synchronize()
            reps = 20
            ev0.record()
            for i in range(reps):
                B.lmhead_argmax(Ws[i % 2], Xh, ws=wsl)
            ev1.record()
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / reps
            nbytes = workloads.q4_matrix_bytes(synth.VOCAB, synth.HIDDEN) + batch * synth.HIDDEN * 2
            lm[f"B{batch}"] = {"us": round(us, 2), "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                               "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        result["lmhead"] = dict(workload="LM-head Q4 GEMV + greedy argmax, 151,936 x 2048", **lm)
        log(f"lmhead: {lm}")
        del Ws
        torch.cuda.empty_cache()
        # the same head with 8-bit codes (the q4-xl checkpoint keeps its LM head at 8 bits)
        mat = synth.lm_head(bits=8)
        Ws = [B.DeviceQ4(*mat, device=dev), B.DeviceQ4(*mat, device=dev)]
        del mat
        lm8 = {}
        for batch in (1, 4):
            Xh = B.bf16_tensor(synth.token_rows(4, batch, synth.HIDDEN, index=batch), dev)
            wsl = B.workspace(B.workspace_bytes(B.OP_LMHEAD, W=Ws[0], rows=batch), dev)
            for i in range(4):
                B.lmhead_argmax(Ws[i % 2], Xh, ws=wsl)
            torch.cuda.synchronize()
            reps = 20
            ev0.record()
            for i in range(reps):
                B.lmhead_argmax(Ws[i % 2], Xh, ws=wsl)
            ev1.record()
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / reps
            nbytes = Ws[0].nbytes + batch * synth.HIDDEN * 2
            lm8[f"B{batch}"] = {"us": round(us, 2), "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        result["lmhead_q8"] = dict(workload="LM-head affine-Q8 GEMV + greedy argmax, 151,936 x 2048", **lm8)
        log(f"lmhead q8: {lm8}")
        del Ws
        torch.cuda.empty_cache()

    if args.calib_copy > 0:
        n = args.calib_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read and written per copy, 3 copies")
        del src, dst

    if not args.no_cpu:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(host_layers, seed=2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
