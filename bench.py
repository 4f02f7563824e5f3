#!/usr/bin/env python3
"""Throughput of the MLP training step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--extra-workloads A,B]

The figure is the wide MLP in strict float32 (1024 -> 4096 -> 4096 -> 1000,
batch 4096, the largest workload, priced against the f32 matrix-core peak);
the bf16 fast path of the same MLP and the skinny batch-8 MLP (priced against
HBM bandwidth) are measured the same way in the same run and reported under
"also".

A step is one pass of the whole hot path (forward GEMMs with fused ReLU/mask,
softmax cross-entropy, dX and dW+SGD GEMMs) over one batch of synthetic
input, through the C ABI.  Inputs are generated from fixed seeds, copied to
HBM before the timed region, and reused cyclically (the batch-1024 workload
draws a fresh batch for each of its 100 steps).  W untimed warm-up steps,
then K steps bracketed by device synchronisations (asynchronous launches:
the headline); when the W steps take less than --min-warmup-ms (100 ms),
untimed steps continue until that much time has passed, so that the timed
steps do not catch the GPU ramping up from idle.  Then up to 50 synchronous steps (the loss read back after
each one) give `sync_ms_per_step`.  For batches of at most 8 rows (float32,
SGD) the same K steps also run as one `mlp_train_steps` call, whose
first-layer update launch makes the next step's first forward too:
`run_ms_per_step`.  After that the same K steps run twice more
with per-launch HIP events on the library's stream (the first of the two
passes only fills the library's event pool, and two untimed steps precede
the second), to price the dominant kernel
against its roofline; then the float64
oracle is timed on the host cores over a bounded sample, and the GPU's ReLU
masks of the first step are counted against the oracle's rounding band.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense).
PEAK = {"f32_mfma_tflops": 157.3, "bf16_mfma_tflops": 2516.6, "hbm_gbps": 8000.0}
DEFAULT_WORKLOAD = "wide_f32"
# measured in the same run and reported under "also"
DEFAULT_EXTRA = "wide_bf16,skinny_b8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--extra-workloads", default=DEFAULT_EXTRA, metavar="A,B",
                    help="further workloads measured the same way and reported under \"also\" "
                         "(empty: none)")
    ap.add_argument("--mode", choices=["train", "forward", "probs", "checkpoint"], default="train",
                    help="train: the training step (the headline metric); forward: logits only "
                         "(inference of the same network); probs: class probabilities (inference); "
                         "checkpoint: save and restore of the state through host memory")
    ap.add_argument("--optimizer", choices=["sgd", "adam", "laprop"], default="sgd",
                    help="update rule of the step (Adam/LaProp: beta1 0.9, beta2 0.999, eps 1e-8)")
    ap.add_argument("--tune", type=int, default=0, metavar="R",
                    help="before timing, let the library choose tile shapes and K splits by timing "
                         "candidates over R steps each (mlp_tune); 0 = the planner's defaults")
    ap.add_argument("--min-warmup-ms", type=float, default=100.0,
                    help="after the W warm-up steps, keep running untimed steps until this much "
                         "wall time has passed since the first, so the GPU leaves its idle clocks "
                         "before the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--profile-steps", type=int, default=None,
                    help="steps of the per-launch event pass (default: --steps)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="no GPU work: turn the rocprofv3 runs collected under DIR "
                         "(bench_W.log, trace_W/, fetch_W/, write_W/) into profiles/W.md and "
                         "profiles/traffic.json for --workload")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a plain copy of "
                         "known size, for scaling hardware byte counters)")
    return ap.parse_args()


def _code_only(text):
    """C/C++ source without comments, trailing blanks and empty lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest():
    """sha256 over the HIP/C++ sources of the library (kernel identity):
    source files only, so that build artefacts or editor files beside them
    do not change it, and their code only, so that an edited comment does
    not either."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mlp_gemm_softmax_amd", "csrc")
    files = [f for ext in ("hip", "hpp", "cpp", "h") for f in glob.glob(os.path.join(csrc, f"*.{ext}"))]
    for f in sorted(files):
        with open(f, encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def recorded_counters(workload, kernel):
    """The committed counter record of launch slot `kernel` of `workload`
    (profiles/traffic.json keeps one per slot, since which of several
    near-equal slots dominates can change from run to run), or None when
    absent or when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_digest():
        return None
    if "slots" in rec:
        return rec["slots"].get(kernel)
    return rec if rec.get("kernel") == kernel else None


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs, or
    None (see recorded_counters)."""
    rec = recorded_counters(workload, kernel)
    return rec.get("bytes_per_launch") if rec else None


def roofline(rows, precision, steps):
    """Dominant kernel (largest total time) priced against its roofline."""
    rows = [r for r in rows if r["launches"] > 0]
    dom = max(rows, key=lambda r: r["total_ms"])
    avg_s = dom["total_ms"] / dom["launches"] / 1e3
    ridge = (PEAK["bf16_mfma_tflops"] if precision == "bf16" else PEAK["f32_mfma_tflops"]) * 1e12 \
        / (PEAK["hbm_gbps"] * 1e9)
    intensity = dom["flops"] / dom["bytes"] if dom["bytes"] else float("inf")
    if dom["flops"] > 0 and intensity >= ridge:
        peak = PEAK["bf16_mfma_tflops"] if precision == "bf16" else PEAK["f32_mfma_tflops"]
        achieved = dom["flops"] / avg_s / 1e12
        bound, unit = "mfma", "TFLOP/s"
    else:
        peak = PEAK["hbm_gbps"]
        achieved = dom["bytes"] / avg_s / 1e9
        bound, unit = "hbm", "GB/s"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None, "kernel": dom["name"],
            "avg_us": round(avg_s * 1e6, 3), "algorithmic_flops": dom["flops"],
            "algorithmic_bytes": dom["bytes"]}


def cpu_baseline(w, budget_s, rule="sgd"):
    """The float64 oracle as it stands, on this host's cores, over a bounded
    sample of the workload's steps (with the oracle's Adam/LaProp when the
    step uses one)."""
    import numpy as np
    from mlp_gemm_softmax_amd import synth
    from oracle import mlp_oracle
    blas = "BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
        blas = " + ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info})) or blas
    except Exception:
        cores = len(os.sched_getaffinity(0))
    Ws = synth.workload_weights(w)
    m = [np.zeros(a.shape) for a in Ws]
    v = [np.zeros(a.shape) for a in Ws]
    n, t0 = 0, time.perf_counter()
    while True:
        x, t, _ = synth.workload_batch(w, n)
        r = mlp_oracle.train_step(x, t, Ws, w.lr)
        if rule != "sgd":
            u = mlp_oracle.OPTIMIZERS[rule](Ws, r["dW"], m, v, n + 1, w.lr, 0.9, 0.999, 1e-8)
            r["W_new"], m, v = u["W_new"], u["m"], u["v"]
        Ws = [a.astype(np.float32) for a in r["W_new"]]
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20000:
            break
    # batch generation is inside the loop; it is small next to the f64 step
    return {"value": round(n / el, 4), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} consecutive training steps ({rule}) of {w.name} (float64 numpy on {blas}, "
                      f"BLAS threads {cores}), {el:.1f} s"}


# ---------------------------------------------------------------- profiles --

TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace_{w} -o {w} -- "
             "python3 bench.py --workload {w} --extra-workloads none --steps {s} --warmup {wu} --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d OUT/{d}_{w} -o {w} -- python3 bench.py "
           "--workload {w} --extra-workloads none --steps 2 --warmup 1 --profile-steps 1 --no-cpu-baseline "
           "--calib-copy-mb 256")
MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_{p} SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE"
N_SIMDS = 256 * 4     # MI355X: 256 CUs of 4 SIMDs
N_XCDS = 8            # GRBM_GUI_ACTIVE is summed over the 8 XCDs


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _bench_log(path):
    slots, line = [], None
    with open(path) as f:
        for ln in f:
            if ln.startswith("[bench] per-launch") and not slots:   # the headline workload
                body = ln.split(":", 1)[1]
                for item in body.split(","):
                    name, val = item.strip().rsplit("=", 1)
                    slots.append((name, float(val) * 1e3))
            elif ln.startswith("{"):
                line = json.loads(ln)
    return slots, line


def _short(name):
    import re
    name = name.replace("void mlp::(anonymous namespace)::", "").replace("mlp::(anonymous namespace)::", "")
    return re.sub(r"\((mlp::)?\w+Params\)$", "", name)


# The only slot with a second dispatch is a split-K product: its epilogue
# kernel follows the product's own launch in the same slot.
_FOLLOWER = "splitk_epilogue_kernel"


def _per_slot(dispatches, n_slots, steps):
    """Average a per-dispatch value by slot over the last `steps` whole steps.
    Dispatches are grouped per slot: a split-K epilogue joins the launch
    before it, and the group's value is the sum over its dispatches."""
    groups = []
    for name, val in dispatches:
        if "mlp::" not in name:
            continue
        if _FOLLOWER in name and groups:
            groups[-1][1] += val
            groups[-1][2].append(name)
        else:
            groups.append([name, val, [name]])
    if len(groups) < n_slots * steps:
        raise SystemExit(f"trace holds {len(groups)} slot dispatch groups, expected {n_slots * steps}")
    tail = groups[-n_slots * steps:]
    for k in range(steps):   # every step must repeat the same kernel sequence
        for i in range(n_slots):
            if tail[k * n_slots + i][2] != tail[i][2]:
                raise SystemExit(f"dispatch sequence differs between steps at slot {i}")
    names = [" + ".join(_short(n) for n in tail[i][2]) for i in range(n_slots)]
    avg = [sum(tail[k * n_slots + i][1] for k in range(steps)) / steps for i in range(n_slots)]
    return names, avg


def summarize(outdir, w, steps, warmup):
    slots, line = _bench_log(os.path.join(outdir, f"bench_{w}.log"))
    n = len(slots)
    trace = _csv(os.path.join(outdir, f"trace_{w}", f"{w}_kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    disp = [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace]
    full_steps = sum(1 for d in disp if "mlp::" in d[0] and _FOLLOWER not in d[0]) // n
    # the last `steps` steps: the bench's final pass of single steps (a run of
    # merged steps, with another launch sequence, may come before it)
    names, trace_us = _per_slot(disp, n, max(1, min(full_steps - 1, steps)))
    stats = _csv(os.path.join(outdir, f"trace_{w}", f"{w}_kernel_stats.csv"))

    counters, scale = {}, {}
    for cname, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = _csv(os.path.join(outdir, f"{d}_{w}", f"{w}_counter_collection.csv"))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == cname]
        copies = [v for k, v in vals if "copyBuffer" in k]
        scale[cname] = (256 * 1024) / max(copies)          # KiB the 256 MiB copy moved / counted
        _, per = _per_slot(vals, n, 2)
        counters[cname] = [v * scale[cname] * 1024 for v in per]   # bytes per launch

    # optional third pass: matrix-core busy cycles, MFMA ops and active cycles
    mfma = None
    mpath = os.path.join(outdir, f"mfma_{w}", f"{w}_counter_collection.csv")
    if os.path.exists(mpath):
        rows = _csv(mpath)
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        prec = "BF16" if line["config"]["precision"] == "bf16" else "F32"
        per = {}
        for cname in ("SQ_VALU_MFMA_BUSY_CYCLES", f"SQ_INSTS_VALU_MFMA_MOPS_{prec}", "GRBM_GUI_ACTIVE"):
            vals = [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == cname]
            per[cname] = _per_slot(vals, n, 2)[1]
        spans = {}
        for r in rows:   # duration of each dispatch, from the same run
            spans[r["Dispatch_Id"]] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        dur = _per_slot([spans[k] for k in sorted(spans, key=int)], n, 2)[1]
        mfma = []
        for i in range(n):
            cyc = per["GRBM_GUI_ACTIVE"][i] / N_XCDS
            mfma.append({"busy": per["SQ_VALU_MFMA_BUSY_CYCLES"][i] / (cyc * N_SIMDS) if cyc else 0.0,
                         "flops": per[f"SQ_INSTS_VALU_MFMA_MOPS_{prec}"][i] * 512,
                         "clock_ghz": cyc / (dur[i] * 1e3) if dur[i] else 0.0, "dur_us": dur[i]})

    roof = line["roofline"]
    dom = [i for i, (nm, _) in enumerate(slots) if nm == roof["kernel"]][0]
    lines = [f"# rocprofv3 summary: workload `{w}`", "",
             f"Kernel source digest (sha256 of the code, comments removed, of the .hip/.hpp/.cpp/.h files in mlp_gemm_softmax_amd/csrc): `{source_digest()}`", "",
             "Commands (repository root on one MI355X; OUT is the output folder):", "",
             "```", TRACE_CMD.format(w=w, s=steps, wu=warmup),
             PMC_CMD.format(c="FETCH_SIZE", d="fetch", w=w),
             PMC_CMD.format(c="WRITE_SIZE", d="write", w=w)]
    if mfma is not None:
        p = "BF16" if line["config"]["precision"] == "bf16" else "F32"
        lines.append(PMC_CMD.format(c=MFMA_COUNTERS.format(p=p), d="mfma", w=w).replace(" --calib-copy-mb 256", ""))
    lines += ["```", "",
             f"bench: {line['value']} steps/s, {line['ms_per_step']} ms/step, "
             f"{line['achieved_tflops']} TFLOP/s; dominant kernel `{roof['kernel']}` "
             f"{roof['achieved']} {roof['unit']} = {roof['frac']:.4f} of {roof['peak']} ({roof['bound']})", "",
             "## Per launch slot (one training step)", "",
             "HBM bytes are the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) scaled by what "
             f"they read for a 256 MiB device-to-device copy (x{scale['FETCH_SIZE']:.3f} fetch, "
             f"x{scale['WRITE_SIZE']:.3f} write).", "",
             "| slot | kernel | HIP-event avg us | trace avg us | fetch MB | write MB |",
             "|---|---|---|---|---|---|"]
    for i, (nm, ev) in enumerate(slots):
        kn = names[i]
        lines.append(f"| {nm} | `{kn}` | {ev:.2f} | {trace_us[i]:.2f} | "
                     f"{counters['FETCH_SIZE'][i] / 1e6:.2f} | {counters['WRITE_SIZE'][i] / 1e6:.2f} |")
    if mfma is not None:
        lines += ["", "## Matrix cores per launch slot", "",
                  "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); MFMA "
                  "GFLOP = SQ_INSTS_VALU_MFMA_MOPS x 512; clock = GRBM_GUI_ACTIVE / 8 over the dispatch's "
                  "duration in the same run, shown for launches of at least 100 us (the counter window "
                  "adds cycles outside the dispatch, which only long launches amortise).", "",
                  "| slot | MFMA busy | MFMA GFLOP (counter) | clock GHz |",
                  "|---|---|---|---|"]
        for i, (nm, _) in enumerate(slots):
            clk = f"{mfma[i]['clock_ghz']:.2f}" if mfma[i]["dur_us"] >= 100 else "-"
            lines.append(f"| {nm} | {mfma[i]['busy']:.3f} | {mfma[i]['flops'] / 1e9:.2f} | {clk} |")
        lines += ["", f"Dominant slot `{roof['kernel']}`: {mfma[dom]['flops'] / 1e9:.2f} GFLOP counted on the "
                      f"matrix cores against {roof['algorithmic_flops'] / 1e9:.2f} GFLOP of GEMM work (2MNK)."]
    lines += ["", "## kernel_stats (whole run)", "", "| kernel | calls | avg us | % |", "|---|---|---|---|"]
    for r in stats[:12]:
        kn = _short(r["Name"])[:90]
        lines.append(f"| `{kn}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{w}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(tpath) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    def slot_rec(i):
        return {"mfma_busy": round(mfma[i]["busy"], 4) if mfma else None,
                "clock_ghz": round(mfma[i]["clock_ghz"], 3) if mfma and mfma[i]["dur_us"] >= 100 else None,
                "bytes_per_launch": round(counters["FETCH_SIZE"][i] + counters["WRITE_SIZE"][i]),
                "fetch_bytes": round(counters["FETCH_SIZE"][i]),
                "write_bytes": round(counters["WRITE_SIZE"][i])}
    # every slot's counters, and the profiled run's dominant slot at the top
    allrec[w] = dict(slot_rec(dom), kernel=roof["kernel"], source_sha=source_digest(),
                     algorithmic_bytes=roof["algorithmic_bytes"],
                     fetch_scale=scale["FETCH_SIZE"], write_scale=scale["WRITE_SIZE"],
                     slots={nm: slot_rec(i) for i, (nm, _) in enumerate(slots)})
    with open(tpath, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    print(f"wrote profiles/{w}.md and profiles/traffic.json[{w}]")


def mask_counts(w, x, Ws, masks):
    """Per hidden layer of the first step (batch 0, initial weights): units,
    units inside the oracle's rounding band, GPU mask bits the oracle adopts
    there and bits that differ outside it (which the parity gate requires to
    be 0).  Runs the oracle's forward, untimed, after the CPU baseline."""
    from oracle import mlp_oracle
    ref = mlp_oracle.forward(x, Ws, kink_choice=masks, precision=w.precision)
    return [{"layer": l + 1, "units": int(w.batch * w.dims[l + 1]), "in_band": ib, "adopted": ad,
             "outside": out}
            for l, (ib, ad, out) in enumerate(zip(ref["in_band"], ref["adopted"], ref["outside"]))]


def measure(w, args, dev, want_cpu, want_masks):
    """Time one workload through the C ABI: warm-up, K asynchronous steps
    (the figure), up to 50 synchronous steps, then the same K steps with
    per-launch events for the roofline; then the oracle on the host."""
    import numpy as np
    import torch
    from mlp_gemm_softmax_amd import binding, synth

    print(f"[bench] workload {w.name} dims={w.dims} B={w.batch} {w.precision} "
          f"steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    Ws = synth.workload_weights(w)
    net = binding.Mlp(w.dims, w.batch, w.precision, device="cuda:0")
    net.set_params([torch.from_numpy(a).to(dev) for a in Ws])
    if args.optimizer != "sgd":
        net.set_optimizer(args.optimizer, 0.9, 0.999, 1e-8)
    n_batches = w.steps if w.fresh_batch else 1
    batches = []
    for s in range(n_batches):
        x, t, _ = synth.workload_batch(w, s)
        batches.append((torch.from_numpy(x).to(dev), torch.from_numpy(t).to(dev)))
    masks = None
    if want_masks and w.n_layers > 1 and args.mode == "train":
        # the GPU's ReLU masks of the first step, before any update
        net.grads(*batches[0])
        masks = [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, w.n_layers)]
    loss_dev = torch.zeros(1, dtype=torch.float32, device=dev)
    if args.calib_copy_mb > 0:
        src = torch.ones(args.calib_copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    if args.tune > 0:
        t0 = time.perf_counter()
        net.tune(*batches[0], args.tune)
        print(f"[bench] mlp_tune over {args.tune} steps per candidate: {time.perf_counter() - t0:.1f} s",
              file=sys.stderr, flush=True)

    logits = torch.empty((w.batch, w.dims[-1]), dtype=torch.float32, device=dev)

    def run(k, offset=0):
        for i in range(k):
            xb, tb = batches[(offset + i) % n_batches]
            if args.mode == "forward":
                net.forward_async(xb, logits)
            elif args.mode == "probs":
                net.forward_probs(xb, logits)
            else:
                net.train_step_async(xb, tb, w.lr, loss_dev)

    # W warm-up steps, then more untimed steps until at least
    # --min-warmup-ms of GPU work has run: after an idle GPU (the previous
    # workload's CPU baseline) a handful of short steps do not reach steady
    # clocks (bf16 wide step: 0.725-0.735 ms/step after 5 warm-up steps,
    # 0.677-0.678 after 50 or more)
    t0 = time.perf_counter()
    run(args.warmup)
    torch.cuda.synchronize()
    extra = 0
    while (time.perf_counter() - t0) * 1e3 < args.min_warmup_ms:
        run(1, args.warmup + extra)
        torch.cuda.synchronize()
        extra += 1
    t0 = time.perf_counter()
    run(args.steps, args.warmup)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    final_loss = float(loss_dev.item())

    # Synchronous steps (mlp_train_step: the loss read back to the host after
    # every step), a bounded number of them, reported beside the headline.
    sync_ms = None
    if args.mode == "train":
        ks = min(args.steps, 50)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(ks):
            xb, tb = batches[i % n_batches]
            net.train_step(xb, tb, w.lr)
        sync_ms = (time.perf_counter() - t0) / ks * 1e3

    # The same K steps as one mlp_train_steps run (batches stacked), where
    # the library hands the first layer's update to the next step's first
    # forward launch (batch <= 8, float32, SGD); reported beside the figure.
    # Not in counter runs (--profile-steps), whose dispatches must repeat
    # the single-step sequence.
    run_ms = None
    if (args.mode == "train" and w.precision == "f32" and w.batch <= 8 and args.optimizer == "sgd"
            and not args.profile_steps):
        order = [batches[(args.warmup + i) % n_batches] for i in range(args.steps)]
        xs = torch.stack([b[0] for b in order]).contiguous()
        ts = torch.stack([b[1] for b in order]).contiguous()
        run_loss = torch.zeros(args.steps, dtype=torch.float32, device=dev)
        net.train_steps(xs[:max(args.warmup, 1)], ts[:max(args.warmup, 1)], w.lr, run_loss[:max(args.warmup, 1)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        net.train_steps(xs, ts, w.lr, run_loss)
        torch.cuda.synchronize()
        run_ms = (time.perf_counter() - t0) / args.steps * 1e3
        del xs, ts, run_loss

    # Per-launch HIP events on the library's stream, same step sequence.  A
    # launch whose event pair the GPU reaches before the host has enqueued
    # the launch itself is timed with that wait.  So a first pass of the same
    # length fills the library's event pool (no event is created during the
    # measured pass) and is discarded, and two untimed steps go first, so the
    # host is ahead of the GPU when the measured steps start.
    pk = args.profile_steps or args.steps
    net.profile(True)
    net.profile_reset()
    run(pk)
    torch.cuda.synchronize()
    net.profile_reset()
    net.profile(False)
    run(2)
    net.profile(True)
    run(pk)
    torch.cuda.synchronize()
    rows = net.profile_read()
    net.profile(False)
    net.close()
    del net, batches
    torch.cuda.empty_cache()
    roof = roofline(rows, w.precision, pk)
    roof["traffic"] = recorded_traffic(w.name, roof["kernel"])
    rec = recorded_counters(w.name, roof["kernel"]) or {}
    for key in ("mfma_busy", "clock_ghz"):   # matrix-core busy share and clock from the counter runs
        if rec.get(key) is not None:
            roof[key] = rec[key]
    print(f"[bench] per-launch (ms avg) [{w.name}]: " + ", ".join(
        f"{r['name']}={r['total_ms'] / max(r['launches'], 1):.4f}" for r in rows),
        file=sys.stderr, flush=True)

    steps_per_s = args.steps / el
    fwd = args.mode in ("forward", "probs")
    flops = w.forward_flops() if fwd else w.gemm_flops()
    step_bytes = sum(r["bytes"] for r in rows if r["launches"] > 0)
    peak = PEAK["bf16_mfma_tflops"] if w.precision == "bf16" else PEAK["f32_mfma_tflops"]
    res = {
        "value": round(steps_per_s, 3),
        "ms_per_step": round(el / args.steps * 1e3, 5),
        "dtype": "bf16" if w.precision == "bf16" else "f32",
        "config": {"workload": w.name, "dims": list(w.dims), "batch": w.batch, "lr": w.lr,
                   "precision": w.precision, "fresh_batch_per_step": w.fresh_batch,
                   "optimizer": args.optimizer, "mode": args.mode, "tuned": args.tune > 0},
        "achieved_tflops": round(flops * steps_per_s / 1e12, 4),
        "step_flops": flops,
        # algorithmic HBM bytes of the launches one step makes (each operand
        # read once, each output written once), and their rate over the step
        "step_bytes": int(step_bytes),
        "step_gbps": round(step_bytes * steps_per_s / 1e9, 2),
        # untimed steps run after the W warm-up steps to reach --min-warmup-ms
        "extra_warmup_steps": extra,
        "sync_ms_per_step": round(sync_ms, 5) if sync_ms is not None else None,
        # K steps as one mlp_train_steps call (first-layer passes fused across steps)
        "run_ms_per_step": round(run_ms, 5) if run_ms is not None else None,
        "final_loss": final_loss,
        "roofline": roof,
    }
    # the whole step against the bound of its dominant kernel
    if roof["bound"] == "mfma":
        res["step_frac"] = round(res["achieved_tflops"] / peak, 4)
    else:
        res["step_frac"] = round(res["step_gbps"] / PEAK["hbm_gbps"], 4)
    if want_cpu and not fwd:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s, args.optimizer)
        if w.name in ("mnist_b32", "mnist_b1024", "skinny_b8"):
            # the same oracle restricted to one BLAS thread, over a shorter sample
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                res["cpu_baseline_1thread"] = cpu_baseline(w, min(args.cpu_budget_s, 8.0), args.optimizer)
    if masks is not None:
        x0, _, _ = synth.workload_batch(w, 0)
        res["mask_bits"] = mask_counts(w, x0, Ws, masks)
    return res


def measure_checkpoint(w, args, dev):
    """Save and restore the workload's state through the C ABI: the weights,
    and with --optimizer adam|laprop the moments too, into a pinned and into
    a pageable host buffer (min(K, 20) of each after the warm-up).  A save
    synchronises, copies to the host and checksums; a restore checks the
    whole checkpoint, then copies to the device."""
    import torch
    from mlp_gemm_softmax_amd import binding, synth

    Ws = synth.workload_weights(w)
    net = binding.Mlp(w.dims, w.batch, w.precision, device="cuda:0")
    net.set_params([torch.from_numpy(a).to(dev) for a in Ws])
    withopt = args.optimizer != "sgd"
    if withopt:
        net.set_optimizer(args.optimizer, 0.9, 0.999, 1e-8)
    nbytes = net.checkpoint_bytes(withopt)
    reps = max(1, min(args.steps, 20))
    res = {}
    for kind in ("pinned", "pageable"):
        buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=kind == "pinned")
        for _ in range(max(args.warmup, 1)):
            net.save_checkpoint(withopt, out=buf)
            net.load_checkpoint(buf)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            net.save_checkpoint(withopt, out=buf)
        t1 = time.perf_counter()
        for _ in range(reps):
            net.load_checkpoint(buf)
        t2 = time.perf_counter()
        save_s, load_s = (t1 - t0) / reps, (t2 - t1) / reps
        res[kind] = {"save_ms": round(save_s * 1e3, 4), "load_ms": round(load_s * 1e3, 4),
                     "save_gbps": round(nbytes / save_s / 1e9, 2), "load_gbps": round(nbytes / load_s / 1e9, 2)}
        del buf
    net.close()
    rt = res["pinned"]["save_ms"] + res["pinned"]["load_ms"]
    return {"value": round(1e3 / rt, 3), "ms_per_step": round(rt, 4), "dtype": "f32",
            "config": {"workload": w.name, "dims": list(w.dims), "batch": w.batch, "precision": w.precision,
                       "optimizer": args.optimizer, "mode": "checkpoint", "with_moments": withopt},
            "checkpoint_bytes": nbytes, "reps": reps, "pinned": res["pinned"], "pageable": res["pageable"]}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.workload, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch
    from mlp_gemm_softmax_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    if args.mode == "checkpoint":
        head = measure_checkpoint(w, args, dev)
        out = {"metric": "checkpoint save + restore round trips/sec (pinned host buffer), 1 GPU",
               "value": head.pop("value"), "unit": "round trips/s", "n_gpus": 1, "steps": head.pop("reps"),
               "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": head.pop("dtype"),
               "data": "synthetic (seeded initial weights)", "config": head.pop("config")}
        out.update(head)
        extra = [n for n in args.extra_workloads.split(",") if n and n not in ("none", w.name)]
        if extra:
            out["also"] = {n: measure_checkpoint(synth.WORKLOADS[n], args, dev) for n in extra}
        print(json.dumps(out), flush=True)
        return
    fwd = args.mode in ("forward", "probs")
    head = measure(w, args, dev, not args.no_cpu_baseline, not args.no_cpu_baseline)
    out = {
        "metric": (f"MLP forward passes/sec ({'probabilities' if args.mode == 'probs' else 'logits'}, "
                   "inference) + achieved TFLOP/s, 1 GPU" if fwd else
                   "MLP train steps/sec + achieved TFLOP/s (fraction of MFMA/HBM roofline), 1 GPU"),
        "value": head.pop("value"),
        "unit": "forward passes/s" if fwd else "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic (seeded; MNIST-shaped uniform [0,1) pixels or N(0,1) features, uniform class ids)",
        "config": head.pop("config"),
    }
    out.update(head)
    # the other targeted workloads, measured the same way in the same run
    extra = [n for n in args.extra_workloads.split(",") if n and n not in ("none", w.name)]
    if extra:
        out["also"] = {}
        for name in extra:
            out["also"][name] = measure(synth.WORKLOADS[name], args, dev, not args.no_cpu_baseline,
                                        not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
