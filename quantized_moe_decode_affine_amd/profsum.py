"""Summaries of rocprofv3 output databases (the rocpd SQLite files that
`rocprofv3 --kernel-trace --stats -d DIR -o run` and `rocprofv3 --pmc ...`
write), as short Markdown for the profiles/ directory.

    python -m quantized_moe_decode_affine_amd.profsum stats DB --cmd "..."
    python -m quantized_moe_decode_affine_amd.profsum traffic --fetch DB1 --write DB2 \\
        --kernel decode_layer_kernel --copy-bytes N --unit-bytes B --cmd-fetch "..." --cmd-write "..."
    python -m quantized_moe_decode_affine_amd.profsum gemm-traffic --fetch DB1 --write DB2 \\
        --copy-bytes N --cmd-fetch "..." --cmd-write "..."

`traffic` scales the kernel's FETCH_SIZE / WRITE_SIZE readings (KiB per
dispatch) by what the same counters read for a plain device copy of known size
run in the same process (the largest `copyBuffer` dispatch), and records the
sha256 of the decode kernel's sources so a reader can tell whether the figure
still applies.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import re
import sqlite3
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ("decode.hip", "common.h", "vecstage.h", "topk.h", "kernels.h", "handoff.h")
ALL_SOURCES = ("abi.hip", "decode.hip", "decode_batch.hip", "gemm.hip", "gemv.hip", "route.hip", "common.h", "kernels.h", "topk.h",
               "vecstage.h", "handoff.h", "preprows.h")


def _sha256(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def decode_sources_sha256() -> str:
    return _sha256(DECODE_SOURCES)


def all_sources_sha256() -> str:
    """Hash of every kernel source: a kernel trace taken from other sources is stale."""
    return _sha256(ALL_SOURCES)


def _short(name: str) -> str:
    name = name.replace("q4moe::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def kernel_times(db: str):
    """{short kernel name: [duration_us, ...]} from a kernel-trace database."""
    con = sqlite3.connect(db)
    out = defaultdict(list)
    for name, start, end in con.execute("select name, start, end from kernels"):
        out[_short(name)].append((end - start) / 1000.0)
    return out


def stats_markdown(db: str, cmd: str) -> str:
    times = kernel_times(db)
    total = sum(sum(v) for v in times.values())
    lines = [f"command: `{cmd}`", "", "| kernel | calls | avg us | min us | max us | total ms | % |",
             "|---|---|---|---|---|---|---|"]
    for k, v in sorted(times.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k[:70]}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{sum(v) / 1000:.3f} | {100 * sum(v) / total:.1f} |")
    g = times.get("grouped_q4_gemm_kernel")
    if g:
        # the prefill layer launches it twice per layer: gate/up (SwiGLU), then down
        lines += ["", "| grouped_q4_gemm_kernel launch | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for name, v in (("gate/up (even dispatches)", g[0::2]), ("down (odd dispatches)", g[1::2])):
            if v:
                lines.append(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    lines += ["", f"kernel sources sha256: {all_sources_sha256()}"]
    return "\n".join(lines) + "\n"


def counter_per_dispatch(db: str, counter: str):
    """[(short kernel name, value)] per dispatch for one counter."""
    con = sqlite3.connect(db)
    acc = defaultdict(float)
    names = {}
    for did, kn, cn, v in con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if cn != counter:
            continue
        acc[did] += v
        names[did] = _short(kn)
    return [(names[d], acc[d]) for d in sorted(acc)]


def traffic_markdown(fetch_db: str, write_db: str, kernel: str, copy_bytes: int, unit_bytes: int,
                     cmd_fetch: str, cmd_write: str) -> str:
    rows = {}
    for db, counter in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        per = counter_per_dispatch(db, counter)
        kv = [v for n, v in per if n == kernel]
        cv = [v for n, v in per if "copyBuffer" in n]
        if not kv or not cv:
            raise SystemExit(f"{db}: no {counter} readings for {kernel} or for a copyBuffer dispatch")
        copy_kib = max(cv)  # the calibration copy is the largest copy in the run
        factor = copy_bytes / (copy_kib * 1024.0)
        rows[counter] = (sum(kv) / len(kv), len(kv), copy_kib, factor)
    fetch = rows["FETCH_SIZE"][0] * 1024.0 * rows["FETCH_SIZE"][3]
    write = rows["WRITE_SIZE"][0] * 1024.0 * rows["WRITE_SIZE"][3]
    traffic = int(round(fetch + write))
    lines = [
        f"kernel: `{kernel}`",
        f"fetch command: `{cmd_fetch}`",
        f"write command: `{cmd_write}`",
        "",
        "| counter | kernel avg KiB/dispatch | dispatches | copy reading KiB | copy bytes | scale |",
        "|---|---|---|---|---|---|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        avg, n, ck, f = rows[c]
        lines.append(f"| {c} | {avg:.1f} | {n} | {ck:.1f} | {copy_bytes} | {f:.4f} |")
    lines += [
        "",
        f"scaled fetch bytes per launch: {int(round(fetch))}",
        f"scaled write bytes per launch: {int(round(write))}",
        f"traffic bytes per launch: {traffic}",
        f"algorithmic bytes per launch: {unit_bytes}",
        f"traffic / algorithmic: {traffic / unit_bytes:.3f}",
        f"decode sources sha256: {decode_sources_sha256()}",
    ]
    return "\n".join(lines) + "\n"


def gemm_traffic_markdown(fetch_db: str, write_db: str, copy_bytes: int, cmd_fetch: str, cmd_write: str) -> str:
    """FETCH_SIZE / WRITE_SIZE of the grouped GEMM's gate/up (even) and down (odd)
    launches, scaled like traffic_markdown."""
    out = {}
    for db, counter in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        per = counter_per_dispatch(db, counter)
        kv = [v for n, v in per if n == "grouped_q4_gemm_kernel"]
        cv = [v for n, v in per if "copyBuffer" in n]
        if not kv or not cv:
            raise SystemExit(f"{db}: no {counter} readings for the grouped GEMM or for a copyBuffer dispatch")
        factor = copy_bytes / (max(cv) * 1024.0)
        for name, v in (("gate/up", kv[0::2]), ("down", kv[1::2])):
            out[(name, counter)] = (sum(v) / len(v), len(v), factor)
    lines = [f"fetch command: `{cmd_fetch}`", f"write command: `{cmd_write}`", "",
             "| launch | counter | avg KiB/dispatch | dispatches | scale | bytes per launch |", "|---|---|---|---|---|---|"]
    for (name, counter), (avg, n, f) in out.items():
        lines.append(f"| {name} | {counter} | {avg:.1f} | {n} | {f:.4f} | {int(round(avg * 1024 * f))} |")
    lines += ["", f"kernel sources sha256: {all_sources_sha256()}"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--unit-bytes", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    m = sub.add_parser("gemm-traffic")
    m.add_argument("--fetch", required=True)
    m.add_argument("--write", required=True)
    m.add_argument("--copy-bytes", type=int, required=True)
    m.add_argument("--cmd-fetch", required=True)
    m.add_argument("--cmd-write", required=True)
    args = ap.parse_args()
    if args.what == "gemm-traffic":
        print(gemm_traffic_markdown(args.fetch, args.write, args.copy_bytes, args.cmd_fetch, args.cmd_write), end="")
    elif args.what == "stats":
        print(stats_markdown(args.db, args.cmd), end="")
    else:
        print(traffic_markdown(args.fetch, args.write, args.kernel, args.copy_bytes, args.unit_bytes,
                               args.cmd_fetch, args.cmd_write), end="")


if __name__ == "__main__":
    main()
