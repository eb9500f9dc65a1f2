"""Summarise rocprofv3 result databases of bench.py runs into profiles/.

  python bench_profile.py trace  <results.db> <out.md> --cmd "<command>"
  python bench_profile.py traffic <fetch.db> <write.db> --workload NAME \
        --calib-mib MIB --cmd-fetch "<command>" --cmd-write "<command>"
  python bench_profile.py lds <results.db> <out.md> --cmd "<command>"
  python bench_profile.py valu <results.db> --workload NAME --cmd "<command>" \
        [--role assign|gate]

`trace` writes per-kernel duration statistics from a --kernel-trace run.
`lds` summarises a run with SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE and
SQ_INSTS_LDS: per kernel, the cycles LDS spent on bank conflicts against the
cycles it was busy with indexed accesses.
`valu` reads a run with SQ_INSTS_VALU and SQ_INSTS_SALU (`bench.py --path
assign`, or any run for the gate) and records the instructions one
moe_assign_tasks call (its two kernels) or one gate launch issues, in total
and per wave, in profiles/valu.json with the source hash.
`pack_orders` reads a --kernel-trace run and --pmc runs of
`bench.py --path pack_orders` and compares, per launch, the pack kernel with
the expert-major slots against the same kernel with slot k*T + t: duration
and the L2-to-memory write counters (requests, 64-byte requests, requests in
flight per cycle, cycles stalled for DRAM credits, ...).
`traffic` reads a FETCH_SIZE run and a WRITE_SIZE run of
`bench.py --fused-only ... --copy-calib-mib MIB`, scales each counter by what
it reads for the calibration copy (a device copy of MIB MiB, which reads and
writes exactly MIB MiB), and records HBM bytes per launch of the pack and
combine kernels in profiles/traffic.json together with the hash of each
kernel's source (bench.py reports the figure only while the hash matches).
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import re
import sqlite3

import bench

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def short(name: str) -> str:
    m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
    return m.group(1) if m else name[:48]


def trace(db: str, out: str, cmd: str) -> None:
    c = sqlite3.connect(db)
    by = collections.defaultdict(list)
    for n, d in c.execute("select name, duration from kernels"):
        by[short(n)].append(d / 1000.0)
    lines = [f"# Kernel trace summary\n", "Command:\n", f"    {cmd}\n",
             "Per-dispatch durations (microseconds):\n", "```",
             f"{'kernel':48s} {'n':>4s} {'avg':>10s} {'min':>10s} {'median':>10s} {'max':>10s}"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        lines.append(f"{k:48s} {len(v):4d} {sum(v) / len(v):10.3f} {v[0]:10.3f} "
                     f"{v[len(v) // 2]:10.3f} {v[-1]:10.3f}")
    lines.append("```\n")
    with open(out, "w") as f:
        f.write("\n".join(lines))


def _counter(db: str):
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select dispatch_id, kernel_name, grid_size, value from "
        "counters_collection order by dispatch_id"))
    return rows


def traffic(fetch_db: str, write_db: str, workload: str, calib_mib: int,
            cmd_fetch: str, cmd_write: str, kind: str = "flat",
            crossings: int = 0, part_bytes: int = 2, capacity: int = 0,
            dropped: int = 0) -> None:
    fr, wr = _counter(fetch_db), _counter(write_db)
    calib = calib_mib * 1024.0  # KiB read and written by the copy

    def calib_kib(rows):
        big = max((r for r in rows if "copyBuffer" in r[1]), key=lambda r: r[2])
        vals = [r[3] for r in rows if "copyBuffer" in r[1] and r[2] == big[2]]
        return sum(vals) / len(vals)

    f_scale = calib / calib_kib(fr)
    w_scale = calib / calib_kib(wr)

    def per_kernel(rows):
        by = collections.defaultdict(list)
        for _, n, _, v in rows:
            by[short(n)].append(v)
        return {k: sum(v) / len(v) for k, v in by.items()}

    fk, wk = per_kernel(fr), per_kernel(wr)
    w = bench.mi.WORKLOADS[workload]
    # role of a kernel: the first prefix its name starts with
    if kind == "fp8":
        alg = bench.fp8_kernel_bytes(w)
        prefixes = {"pack_fp8_": "pack_fp8", "combine_fp8_": "combine_fp8"}
    elif kind == "two_leg":
        if crossings <= 0:
            raise SystemExit("--crossings (dedup.crossing_rows) is required")
        alg = bench.two_leg_kernel_bytes(w, crossings, part_bytes)
        prefixes = {"pack_": "pack_nodes", "forward_": "forward",
                    "partial_": "partial", "sum_nodes_": "sum_nodes"}
    elif kind == "capacity":
        if capacity <= 0:
            raise SystemExit("--capacity (config.capacity) is required")
        alg = bench.capacity_kernel_bytes(w, capacity, dropped)
        # the padded pack is two kernels: used rows, then zeroed padding
        prefixes = {"pack_": "pack_capacity", "zero_rows_": "pack_capacity",
                    "combine_": "combine_capacity"}
    else:
        alg = bench.kernel_bytes(w)
        prefixes = {"pack_": "pack", "combine_": "combine"}
    path = os.path.join(PROFILES, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    name = workload if kind == "flat" else f"{workload}_{kind}"
    md = [f"# HBM traffic per launch: {name}\n",
          "Commands:\n", f"    {cmd_fetch}", f"    {cmd_write}\n",
          f"Calibration: a device copy of {calib_mib} MiB reads "
          f"{calib / f_scale / 1024:.1f} MiB as FETCH_SIZE and "
          f"{calib / w_scale / 1024:.1f} MiB as WRITE_SIZE; counters are "
          f"scaled by {f_scale:.3f} (fetch) and {w_scale:.3f} (write).\n",
          "```",
          f"{'kernel':42s} {'fetch MiB':>10s} {'write MiB':>10s} {'scaled MB':>10s} {'alg MB':>10s} {'ratio':>6s}"]
    def role_of(k):
        return next((r for pre, r in prefixes.items() if k.startswith(pre)),
                    None)

    kernels_of = {}
    for k in fk:
        if role_of(k):
            kernels_of.setdefault(role_of(k), []).append(k)
    for k in sorted(fk, key=lambda k: -(fk[k] + wk.get(k, 0))):
        fb = fk[k] * 1024 * f_scale
        wb = wk.get(k, 0.0) * 1024 * w_scale
        role = role_of(k)
        # a ratio per kernel only where the role is this one kernel
        a = alg.get(role) if role and len(kernels_of[role]) == 1 else None
        md.append(f"{k:42s} {fk[k] / 1024:10.1f} {wk.get(k, 0) / 1024:10.1f} "
                  f"{(fb + wb) / 1e6:10.1f} "
                  f"{(a / 1e6 if a else float('nan')):10.1f} "
                  f"{((fb + wb) / a if a else float('nan')):6.3f}")
    for role, ks in sorted(kernels_of.items()):
        fb = sum(fk[k] for k in ks) * 1024 * f_scale
        wb = sum(wk.get(k, 0.0) for k in ks) * 1024 * w_scale
        a = alg.get(role)
        if len(ks) > 1:
            md.append(f"{role + ' (all its kernels)':42s} "
                      f"{sum(fk[k] for k in ks) / 1024:10.1f} "
                      f"{sum(wk.get(k, 0) for k in ks) / 1024:10.1f} "
                      f"{(fb + wb) / 1e6:10.1f} {a / 1e6:10.1f} "
                      f"{(fb + wb) / a:6.3f}")
        data[f"{role}/{workload}"] = {
            "kernel": " + ".join(sorted(ks)), "bytes_per_launch": fb + wb,
            "fetch_bytes": fb, "write_bytes": wb, "alg_bytes": a,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "source_sha": bench.source_digest(bench.KERNEL_SOURCES[role]),
        }
    md.append("```\n")
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    with open(os.path.join(PROFILES, f"hbm_traffic_{name}.md"), "w") as f:
        f.write("\n".join(md))


def lds(db: str, out: str, cmd: str) -> None:
    c = sqlite3.connect(db)
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for n, counter, v in c.execute(
            "select kernel_name, counter_name, value from counters_collection"):
        per[short(n)][counter].append(v)
    lines = ["# LDS bank conflicts per dispatch\n", "Command:\n",
             f"    {cmd}\n",
             "Counters averaged over dispatches; conflict share = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles).\n", "```",
             f"{'kernel':44s} {'n':>4s} {'LDS instrs':>11s} {'active cyc':>11s} "
             f"{'conflict cyc':>12s} {'share':>6s}"]
    rows = []
    for k, d in per.items():
        ins = d.get("SQ_INSTS_LDS", [0])
        act = d.get("SQ_LDS_IDX_ACTIVE", [0])
        con = d.get("SQ_LDS_BANK_CONFLICT", [0])
        a, b = sum(act) / len(act), sum(con) / len(con)
        if sum(ins) == 0:
            continue
        rows.append((k, len(ins), sum(ins) / len(ins), a, b,
                     b / a if a else float("nan")))
    for k, n, i, a, b, r in sorted(rows, key=lambda r: -r[3]):
        lines.append(f"{k:44s} {n:4d} {i:11.0f} {a:11.0f} {b:12.0f} {r:6.3f}")
    lines.append("```\n")
    with open(out, "w") as f:
        f.write("\n".join(lines))


VALU_KERNELS = {"assign": ("assign_kernel", "expert_tables_kernel"),
                "gate": ("gate_kernel",)}


def valu(db: str, workload: str, cmd: str, role: str = "assign") -> None:
    c = sqlite3.connect(db)
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    waves = collections.defaultdict(list)
    for n, counter, v, grid in c.execute(
            "select kernel_name, counter_name, value, grid_size from "
            "counters_collection"):
        per[short(n)][counter].append(v)
        if counter == "SQ_INSTS_VALU":
            waves[short(n)].append(grid / 64.0)
    parts = {k: {ctr: sum(v) / len(v) for ctr, v in d.items()}
             for k, d in per.items() if k.startswith(VALU_KERNELS[role])}
    for k, d in parts.items():
        d["waves"] = sum(waves[k]) / len(waves[k])
    total = sum(d.get("SQ_INSTS_VALU", 0.0) for d in parts.values())
    path = os.path.join(PROFILES, "valu.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[f"{role}/{workload}"] = {
        "valu_insts_per_call": total, "kernels": parts,
        "source_sha": bench.source_digest(bench.KERNEL_SOURCES[role])}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    title = {"assign": "moe_assign_tasks", "gate": "moe_topk_gate"}[role]
    md = [f"# Vector instructions of {title}: {workload}\n",
          "Command:\n", f"    {cmd}\n",
          "Instruction counts per dispatch (averaged), and per wave "
          "(launched waves: grid size / 64):\n", "```",
          f"{'kernel':40s} {'SQ_INSTS_VALU':>14s} {'SQ_INSTS_SALU':>14s} "
          f"{'waves':>8s} {'VALU/wave':>10s} {'SALU/wave':>10s}"]
    for k, d in sorted(parts.items()):
        w = d.get("waves", 0.0) or 1.0
        md.append(f"{k:40s} {d.get('SQ_INSTS_VALU', 0):14.0f} "
                  f"{d.get('SQ_INSTS_SALU', 0):14.0f} {w:8.0f} "
                  f"{d.get('SQ_INSTS_VALU', 0) / w:10.1f} "
                  f"{d.get('SQ_INSTS_SALU', 0) / w:10.1f}")
    md.append("```\n")
    with open(os.path.join(PROFILES, f"valu_{role}_{workload}.md"), "w") as f:
        f.write("\n".join(md))


def _pack_dispatches(rows, steps: int, warmup: int):
    """Split the pack dispatches of a pack_orders run (dispatch order):
    2*warmup warm-up launches, then `steps` expert-major, then `steps`
    sequential.  rows: (dispatch_id, kernel_name, ...) tuples."""
    ids = sorted({r[0] for r in rows if short(r[1]).startswith("pack")})
    ids = ids[2 * warmup:2 * warmup + 2 * steps]
    return {"expert_major": set(ids[:steps]), "sequential": set(ids[steps:])}


def _per_instance(pmc_dbs: list, steps: int, warmup: int):
    """Per-instance TCC_EA0_WRREQ and TCC_EA0_WRREQ_LEVEL of the pack
    dispatches (rows of rocpd_pmc_event), when a run collected them."""
    import statistics
    for db in pmc_dbs:
        c = sqlite3.connect(db)
        names = dict(c.execute("select id, name from rocpd_info_pmc"))
        if not {"TCC_EA0_WRREQ", "TCC_EA0_WRREQ_LEVEL"} <= set(names.values()):
            continue
        ev = {}
        rows = list(c.execute("select dispatch_id, kernel_name, counter_name, "
                              "event_id from counters_collection"))
        for did, _, cname, eid in rows:
            ev[(did, cname)] = eid
        split = _pack_dispatches(rows, steps, warmup)
        vals = collections.defaultdict(list)
        for eid, pid, v in c.execute("select event_id, pmc_id, value from "
                                     "rocpd_pmc_event order by id"):
            vals[(eid, names.get(pid))].append(v)
        out = {}
        for order, ids in split.items():
            cvr, cvl, ml, n = [], [], [], 0
            for did in ids:
                r = vals[(ev[(did, "TCC_EA0_WRREQ")], "TCC_EA0_WRREQ")]
                lv = vals[(ev[(did, "TCC_EA0_WRREQ_LEVEL")],
                           "TCC_EA0_WRREQ_LEVEL")]
                pairs = [(a, b) for a, b in zip(r, lv) if a > 0]
                if len(pairs) < 2:
                    continue
                req = [a for a, _ in pairs]
                lat = [b / a for a, b in pairs]
                n = len(pairs)
                cvr.append(statistics.pstdev(req) / statistics.mean(req))
                cvl.append(statistics.pstdev(lat) / statistics.mean(lat))
                ml.append(statistics.mean(lat))
            if not cvr:
                return None
            out[order] = {"instances": n,
                          "requests cv": statistics.mean(cvr),
                          "in flight/request cv": statistics.mean(cvl),
                          "in flight/request mean": statistics.mean(ml)}
        return out
    return None


def pack_orders(trace_db: str, pmc_dbs: list, workload: str, steps: int,
                warmup: int, cmds: list) -> None:
    c = sqlite3.connect(trace_db)
    rows = list(c.execute("select dispatch_id, name, duration from kernels"))
    split = _pack_dispatches(rows, steps, warmup)
    dur = {o: [r[2] / 1000.0 for r in rows if r[0] in ids]
           for o, ids in split.items()}
    ctr = collections.defaultdict(lambda: collections.defaultdict(list))
    for db in pmc_dbs:
        c = sqlite3.connect(db)
        crow = list(c.execute(
            "select dispatch_id, kernel_name, counter_name, value from "
            "counters_collection"))
        sp = _pack_dispatches(crow, steps, warmup)
        for did, _, name, v in crow:
            for o, ids in sp.items():
                if did in ids:
                    ctr[o][name].append(v)
    w = bench.mi.WORKLOADS[workload]
    alg = bench.kernel_bytes(w)["pack"]
    names = sorted({n for d in ctr.values() for n in d})
    md = [f"# Pack destination order: {workload}\n", "Commands:\n"]
    md += [f"    {c}" for c in cmds]
    md += ["", "The pack kernel on the same buffers, once with the layout's "
           "expert-major slots, once with slot k*T + t (every destination "
           "row stream sequential).  Per launch, averaged over "
           f"{steps} launches of each; algorithmic bytes {alg}.\n", "```",
           f"{'':40s} {'expert_major':>16s} {'sequential':>16s}"]

    def avg(v):
        return sum(v) / len(v) if v else float("nan")
    md.append(f"{'duration (us)':40s} {avg(dur['expert_major']):16.2f} "
              f"{avg(dur['sequential']):16.2f}")
    md.append(f"{'algorithmic GB/s':40s} "
              f"{alg / avg(dur['expert_major']) / 1e3:16.1f} "
              f"{alg / avg(dur['sequential']) / 1e3:16.1f}")
    for n in names:
        md.append(f"{n:40s} {avg(ctr['expert_major'][n]):16.0f} "
                  f"{avg(ctr['sequential'][n]):16.0f}")
    lvl, req = "TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum"
    if lvl in names and req in names:
        md.append(f"{'write requests in flight / request':40s} "
                  f"{avg(ctr['expert_major'][lvl]) / avg(ctr['expert_major'][req]):16.1f} "
                  f"{avg(ctr['sequential'][lvl]) / avg(ctr['sequential'][req]):16.1f}")
    md.append("```\n")
    inst = _per_instance(pmc_dbs, steps, warmup)
    if inst:
        md += ["Per L2 channel (TCC instance; counters without _sum keep one "
               "value per instance): the spread of the write requests and of "
               "the requests in flight per request over the instances, as a "
               "coefficient of variation, averaged over the launches.\n",
               "```", f"{'':40s} {'expert_major':>16s} {'sequential':>16s}"]
        for k in ("instances", "requests cv", "in flight/request cv",
                  "in flight/request mean"):
            md.append(f"{k:40s} {inst['expert_major'][k]:16.3f} "
                      f"{inst['sequential'][k]:16.3f}")
        md.append("```\n")
    with open(os.path.join(PROFILES, f"pack_orders_{workload}.md"), "w") as f:
        f.write("\n".join(md))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    l = sub.add_parser("lds")
    l.add_argument("db")
    l.add_argument("out")
    l.add_argument("--cmd", required=True)
    v = sub.add_parser("valu")
    v.add_argument("db")
    v.add_argument("--workload", default="deepseek_v3")
    v.add_argument("--cmd", required=True)
    v.add_argument("--role", default="assign", choices=("assign", "gate"))
    o = sub.add_parser("pack_orders")
    o.add_argument("trace_db")
    o.add_argument("pmc_dbs", nargs="+")
    o.add_argument("--workload", default="deepseek_v3")
    o.add_argument("--steps", type=int, required=True)
    o.add_argument("--warmup", type=int, required=True)
    o.add_argument("--cmd", action="append", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("fetch_db")
    r.add_argument("write_db")
    r.add_argument("--workload", default="deepseek_v3")
    r.add_argument("--calib-mib", type=int, required=True)
    r.add_argument("--cmd-fetch", required=True)
    r.add_argument("--cmd-write", required=True)
    r.add_argument("--path", default="flat",
                   choices=("flat", "fp8", "two_leg", "capacity"))
    r.add_argument("--crossings", type=int, default=0,
                   help="two_leg: (token, node) crossings of the run")
    r.add_argument("--part-bytes", type=int, default=2,
                   help="two_leg: bytes per partial element (bf16 2, f32 4)")
    r.add_argument("--capacity", type=int, default=0,
                   help="capacity: rows per segment of the run")
    r.add_argument("--dropped", type=int, default=0,
                   help="capacity: dropped (token, slot) pairs of the run")
    a = ap.parse_args()
    if a.what == "trace":
        trace(a.db, a.out, a.cmd)
    elif a.what == "lds":
        lds(a.db, a.out, a.cmd)
    elif a.what == "valu":
        valu(a.db, a.workload, a.cmd, a.role)
    elif a.what == "pack_orders":
        pack_orders(a.trace_db, a.pmc_dbs, a.workload, a.steps, a.warmup,
                    a.cmd)
    else:
        traffic(a.fetch_db, a.write_db, a.workload, a.calib_mib, a.cmd_fetch,
                a.cmd_write, a.path, a.crossings, a.part_bytes, a.capacity,
                a.dropped)


if __name__ == "__main__":
    main()
