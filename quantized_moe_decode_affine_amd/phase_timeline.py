"""Per-phase timeline of the batch-1 decode layer kernel, from the diagnostic build.

    python -m quantized_moe_decode_affine_amd.build --stamps
    python -m quantized_moe_decode_affine_amd.phase_timeline [--out FILE.md]
    python -m quantized_moe_decode_affine_amd.phase_timeline --gemm [--out FILE.md]
    python -m quantized_moe_decode_affine_amd.phase_timeline --batch [--out FILE.md]

Runs the 40-layer decode loop (hidden 2048, 256 routed + 1 shared experts, top-8) on
``libq4moe_stamps.so``, where thread 0 of every workgroup records the 100 MHz
``s_memrealtime`` counter at the phase boundaries of the layer (decode.hip: launch
start, router logits published, top-k known, gate/up computed, activations staged,
end), and prints a Markdown table of the phase boundaries of the last launches
relative to each launch's first workgroup start: median and maximum over the
workgroups, and the gap from one launch's last workgroup end to the next launch's
first start.  The stamps cost a few stores per workgroup; the loop time printed
with them is the diagnostic library's, not the product's.

``--gemm`` instead runs the 2,048-token prefill layer and summarises the two
grouped-GEMM launches (gate/up with SwiGLU, down with the routing weight) from the
workgroup stamps of gemm.hip: how many workgroups carry a tile, the launch's span,
per-workgroup times by active row blocks (row indices known, main loop, bias term,
epilogue), how many workgroups run at once across the span, and where they ran
(XCC and CU ids).
"""
from __future__ import annotations

import argparse
import ctypes
import os

import numpy as np
import torch

from . import binding as B
from . import workloads

PKG = os.path.dirname(os.path.abspath(__file__))
STAMPS_LIB = os.path.join(PKG, "libq4moe_stamps.so")
NAMES = ["launch start", "router logits published", "top-k known", "gate/up computed", "activations staged", "end"]


def run(form: str, n_layers: int = 40, steps: int = 8):
    lib = B.load_library(STAMPS_LIB)
    stack = workloads.DecodeStack(seed=2, n_layers=n_layers, n_steps=steps, device="cuda")
    if form == "checkpoint":
        stack.enable_q8_router("cuda")
        stack.enable_q8_shared("cuda")
        stack.use_q8_router(True)
    for s in range(3):
        stack.step(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        stack.step(s)
    e1.record()
    torch.cuda.synchronize()
    stack.check()
    loop_us = e0.elapsed_time(e1) * 1e3 / (steps * n_layers)
    buf = np.zeros((4, 1024, 8), dtype=np.uint64)
    rc = lib.q4moe_decode_stamps(buf.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(buf.nbytes))
    if rc != 0:
        raise RuntimeError(f"q4moe_decode_stamps failed ({rc})")
    nb = torch.cuda.get_device_properties(0).multi_processor_count
    st = buf[:, :nb, :6].astype(np.int64)
    order = np.argsort(st[:, :, 0].min(axis=1))  # the four launches in time order
    rows = []
    for k in range(6):
        rel = np.concatenate([(st[i][:, k] - st[i][:, 0].min()) * 10 for i in order])  # ns
        rows.append((NAMES[k], int(np.median(rel)), int(rel.max())))
    gaps = [int((st[b][:, 0].min() - st[a][:, 5].max()) * 10) for a, b in zip(order[:-1], order[1:])]
    return loop_us, rows, gaps


FRONT_NAMES = ["launch start", "router logits published", "x staged", "top-k known", "plan ready",
               "end (every wave done, its stores out)"]
DOWN_NAMES = ["launch start", "plan in LDS", "task list built", "activations staged", "dots done",
              "end (every wave done, its stores out)"]


def batch_run(nb: int, n_layers: int = 40, steps: int = 4):
    """Phase stamps of the batched front launch (the last four launches of a 40-layer loop
    of nb-row steps)."""
    lib = B.load_library(STAMPS_LIB)
    stack = workloads.DecodeStack(seed=2, n_layers=n_layers, n_steps=steps, device="cuda")
    stack.enable_batch(8, "cuda")
    for s in range(2):
        stack.step_batch(s, nb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        stack.step_batch(s, nb)
    e1.record()
    torch.cuda.synchronize()
    loop_us = e0.elapsed_time(e1) * 1e3 / (steps * n_layers)
    def read(fn):
        buf = np.zeros((4, 1024, 8), dtype=np.uint64)
        rc = fn(buf.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(buf.nbytes))
        if rc != 0:
            raise RuntimeError(f"stamp read failed ({rc})")
        n = int(np.count_nonzero(buf[0, :, 0]))
        return buf[:, :n, :6].astype(np.int64), n

    fr, nbk = read(lib.q4moe_front_stamps)
    dn, ndn = read(lib.q4moe_down_stamps)
    order = np.argsort(fr[:, :, 0].min(axis=1))  # the four front launches in time order (same slots)

    def table(st, names):
        rows = []
        for k in range(6):
            rel = np.concatenate([(st[i][:, k] - st[i][:, 0].min()) * 10 for i in order])
            rows.append((names[k], int(np.median(rel)), int(rel.max())))
        return rows
    gaps = [(int((dn[i][:, 0].min() - fr[i][:, 5].max()) * 10), int((fr[j][:, 0].min() - dn[i][:, 5].max()) * 10))
            for i, j in zip(order[:-1], order[1:])]
    return loop_us, nbk, ndn, table(fr, FRONT_NAMES), table(dn, DOWN_NAMES), gaps


def batch_main(args):
    lines = ["# batch_front_kernel: phase timeline (40-layer batched decode loop)", "",
             "Phase boundaries of the front launch of batched decode (router for every token, per-token top-k, the "
             "step's expert plan, gate/up with SwiGLU for the planned experts; hidden 2048, 256 routed + 1 shared "
             "experts, top-8, affine Q4 g64), stamped by thread 0 of every workgroup with the 100 MHz s_memrealtime "
             "counter in the diagnostic build (decode_batch.hip with Q4MOE_DECODE_STAMPS, libq4moe_stamps.so), over "
             "the last four launches of each kind; times are relative to the launch's first workgroup start. "
             "The end stamps follow a wait for the stores and a workgroup barrier.", ""]
    if args.cmd:
        lines += [f"command: `{args.cmd}`", ""]
    for nb in (4, 8):
        loop_us, nbk, ndn, fr, dn, gaps = batch_run(nb)
        lines += [f"## B = {nb}", "", f"loop time with stamps (both launches): {loop_us:.2f} us per layer", ""]
        for title, n, rows in ((f"front launch, {nbk} workgroups", nbk, fr),
                               (f"down launch, {ndn} workgroups of the first token pass", ndn, dn)):
            lines += [title, "", "| phase boundary | median over workgroups (ns) | latest workgroup (ns) |",
                      "|---|---|---|"]
            lines += [f"| {a} | {m} | {x} |" for a, m, x in rows]
            lines += [""]
        lines += ["gaps from the front launch's last end to the down launch's first start, and from the down "
                  "launch's last end to the next front launch's first start (ns): "
                  + ", ".join(f"{a} / {b}" for a, b in gaps), ""]
    return lines


def gemm_run(reps: int = 3):
    """Stamps of the last prefill layer's two grouped-GEMM launches (bf16 router, 4-bit shared expert)."""
    from . import synth
    lib = B.load_library(STAMPS_LIB)
    dev = "cuda"
    dl = B.DeviceLayer(synth.moe_layer(1), dev)
    dl.pack_group_major()
    X = B.bf16_tensor(synth.token_rows(3, 2048, synth.HIDDEN), dev)
    ws = B.workspace(B.workspace_bytes(B.OP_FFN_PREFILL, dl, rows=2048), dev)
    Y = torch.empty((2048, synth.HIDDEN), dtype=torch.float32, device=dev)
    for _ in range(reps):
        B.moe_ffn_prefill(dl, X, out=Y, ws=ws)
    torch.cuda.synchronize()
    buf = np.zeros((4, 4096, 8), dtype=np.uint64)
    rc = lib.q4moe_gemm_stamps(buf.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(buf.nbytes))
    if rc != 0:
        raise RuntimeError(f"q4moe_gemm_stamps failed ({rc})")
    last = 2 * reps - 1  # launches are recorded in slots (launch index) % 4
    return {"gate/up": buf[(last - 1) % 4], "down": buf[last % 4]}


def gemm_summary(name, rec):
    used = np.nonzero(rec[:, 0])[0]
    r = rec[used].astype(np.int64)
    item = rec[used, 6]
    live = item != np.uint64(0xFFFFFFFFFFFFFFFF)
    t0 = r[:, 0].min()
    ns = lambda v: (v - t0) * 10  # noqa: E731
    start, known, main, bias, end = (ns(r[:, i]) for i in range(5))
    span = int(end.max())
    lines = [f"## {name}", "", f"workgroups launched: {len(used)}, with a tile: {int(live.sum())}; "
             f"span from the first start to the last end: {span} ns", ""]
    mb = (item[live] >> np.uint64(28)).astype(np.int64) & 0xF
    split = (item[live] >> np.uint64(32)).astype(np.int64) & 1  # a K-split workgroup (shared-expert tile)
    lines += ["| active row blocks | workgroups | entry -> rows known | main loop | bias term | epilogue | "
              "whole workgroup (p10 / median / p90) |", "|---|---|---|---|---|---|---|"]
    L = {k: v[live] for k, v in dict(start=start, known=known, main=main, bias=bias, end=end).items()}
    for sp, m in sorted(set(zip(split.tolist(), mb.tolist()))):
        sel = (mb == m) & (split == sp)
        d = L["end"][sel] - L["start"][sel]
        med = lambda a: int(np.median(a))  # noqa: E731
        lines.append(f"| {m}{' (K-split)' if sp else ''} | {int(sel.sum())} | {med(L['known'][sel] - L['start'][sel])} | "
                     f"{med(L['main'][sel] - L['known'][sel])} | {med(L['bias'][sel] - L['main'][sel])} | "
                     f"{med(L['end'][sel] - L['bias'][sel])} | {int(np.percentile(d, 10))} / {med(d)} / "
                     f"{int(np.percentile(d, 90))} |")
    # workgroups running at once, averaged over tenths of the span
    edges = np.linspace(0, span, 11)
    conc = []
    for a, b in zip(edges[:-1], edges[1:]):
        ov = np.clip(np.minimum(end, b) - np.maximum(start, a), 0, None)
        conc.append(ov.sum() / max(b - a, 1))
    lines += ["", "workgroups running at once, by tenth of the span: " + ", ".join(f"{c:.0f}" for c in conc)]
    starts = np.sort(L["start"])
    lines += [f"start times of workgroups with a tile (ns): first {int(starts[0])}, 25% {int(np.percentile(starts, 25))}, "
              f"median {int(np.median(starts))}, 75% {int(np.percentile(starts, 75))}, last {int(starts[-1])}"]
    hw = rec[used, 5]
    xcc = (hw >> np.uint64(32)).astype(np.int64) & 0xF
    lines += [f"workgroups on XCC blockIdx % 8: {int((xcc == used % 8).sum())} of {len(used)}"]
    tile = (item[live] & np.uint64(0xFFFFF)).astype(np.int64) + (split << 24)  # split tiles number on their own
    xl = xcc[live]
    same, spread = 0, []
    for t in np.unique(tile):
        sel = tile == t
        same += int(len(set(xl[sel].tolist())) == 1)
        spread.append(L["start"][sel].max() - L["start"][sel].min())
    lines += [f"tiles whose column slices all ran on one XCC: {same} of {len(np.unique(tile))}; spread of the "
              f"slices' start times per tile (ns): median {int(np.median(spread))}, 90% {int(np.percentile(spread, 90))}, "
              f"max {int(np.max(spread))}", ""]
    return lines


def gemm_main(args):
    recs = gemm_run()
    lines = ["# grouped_q4_gemm_kernel: workgroup timeline (2,048-token prefill layer)", "",
             "The two grouped-GEMM launches of one prefill layer (hidden 2048, inter 512, 256 routed + 1 shared "
             "experts, top-8, bf16 router, affine Q4 g64): thread 0 of every workgroup stamps the 100 MHz "
             "s_memrealtime counter at entry, once its tile's row indices are known, after the main loop, after the "
             "bias term and at the end, in the diagnostic build (gemm.hip with Q4MOE_GEMM_STAMPS, "
             "libq4moe_stamps.so). Times are in ns from the launch's first workgroup start; per-phase columns are "
             "medians.", ""]
    if args.cmd:
        lines += [f"command: `{args.cmd}`", ""]
    for name, rec in recs.items():
        lines += gemm_summary(name, rec)
    gu, dn = (r[np.nonzero(r[:, 0])[0]].astype(np.int64) for r in recs.values())
    lines += [f"from the gate/up launch's last workgroup end to the down launch's first workgroup start "
              f"(the activations' fp16 preparation runs between them): {int((dn[:, 0].min() - gu[:, 4].max()) * 10)} ns; "
              f"from the gate/up launch's first start to the down launch's last end: "
              f"{int((dn[:, 4].max() - gu[:, 0].min()) * 10)} ns", ""]
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the Markdown summary here as well")
    ap.add_argument("--cmd", default="", help="the command line to record in the summary")
    ap.add_argument("--gemm", action="store_true", help="the prefill layer's grouped GEMMs instead of decode")
    ap.add_argument("--batch", action="store_true", help="the batched decode's front launch instead")
    args = ap.parse_args()
    if args.gemm or args.batch:
        text = "\n".join(gemm_main(args) if args.gemm else batch_main(args))
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        return
    lines = ["# decode_layer_kernel: phase timeline (40-layer batch-1 decode loop)", "",
             "Phase boundaries of the batch-1 MoE decode layer (hidden 2048, 256 routed + 1 shared experts, top-8, "
             "affine Q4 g64), stamped by thread 0 of every workgroup with the 100 MHz s_memrealtime counter in the "
             "diagnostic build (decode.hip with Q4MOE_DECODE_STAMPS, libq4moe_stamps.so), over the last four "
             "launches of the loop; times are relative to the launch's first workgroup start.", ""]
    if args.cmd:
        lines += [f"command: `{args.cmd}`", ""]
    for form, label in (("bf16", "bf16 router, 4-bit shared expert"),
                        ("checkpoint", "8-bit router, 8-bit shared expert (the checkpoint's form)")):
        loop_us, rows, gaps = run(form)
        lines += [f"## {label}", "", f"loop time with stamps: {loop_us:.2f} us per layer", "",
                  "| phase boundary | median over workgroups (ns) | latest workgroup (ns) |", "|---|---|---|"]
        lines += [f"| {n} | {m} | {x} |" for n, m, x in rows]
        lines += ["", f"gap from a launch's last workgroup end to the next launch's first start: "
                      f"{', '.join(str(g) for g in gaps)} ns", ""]
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
