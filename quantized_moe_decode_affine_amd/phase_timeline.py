"""Per-phase timeline of the batch-1 decode layer kernel, from the diagnostic build.

    python -m quantized_moe_decode_affine_amd.build --stamps
    python -m quantized_moe_decode_affine_amd.phase_timeline [--out FILE.md]

Runs the 40-layer decode loop (hidden 2048, 256 routed + 1 shared experts, top-8) on
``libq4moe_stamps.so``, where thread 0 of every workgroup records the 100 MHz
``s_memrealtime`` counter at the phase boundaries of the layer (decode.hip: launch
start, router logits published, top-k known, gate/up computed, activations staged,
end), and prints a Markdown table of the phase boundaries of the last launches
relative to each launch's first workgroup start: median and maximum over the
workgroups, and the gap from one launch's last workgroup end to the next launch's
first start.  The stamps cost a few stores per workgroup; the loop time printed
with them is the diagnostic library's, not the product's.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the Markdown summary here as well")
    ap.add_argument("--cmd", default="", help="the command line to record in the summary")
    args = ap.parse_args()
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
