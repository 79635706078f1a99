"""rocprofv3 output -> short text summaries (kernel times, HBM traffic).

The counter workload (``bench.py --pmc-workload``) runs, on one device:
  * a plain device-to-device copy of COPY_BYTES (the calibration: its
    FETCH_SIZE / WRITE_SIZE readings are compared with the bytes it moves),
  * the MoE block of one layer at the canvas shape, a few times.
``summarize_traffic`` turns the two counter passes into HBM bytes per launch
of the expert gate/up kernel, scaled by the copy's factor.  Each summary
records the command that produced it and a hash of the GEMM sources, so a
stale traffic figure is recognised once the kernel changes.
"""
import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_BYTES = 1 << 30
GATEUP_KERNEL = "gemm_wide_kernel<2, 1, 2, 4, 2, 3, 3>"                     # expert gate/up (SwiGLU)
GATEUP_KERNEL_FP8 = "gemm_wide_f8_kernel<2, 1, 4, 3>"                         # the same with e4m3 weights
DOWN_KERNEL = "gemm_down_ring_kernel<2, 4, 3, 4, false>"                    # expert down (routing-weight row scale)
DOWN_KERNEL_FP8 = "gemm_down_ring_kernel<2, 4, 2, 4, true>"                 # the same with e4m3 weights
COPY_KERNEL = "copyBuffer"
GEMM_SOURCES = ("csrc/k_gemm.hip", "csrc/dg_common.h")   # the GEMM kernels and their tile settings


def gemm_source_hash():
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_workload(n_reps=5, fp8=False):
    """Copy calibration + MoE layer launches (run under rocprofv3 --pmc);
    fp8 quantises the expert weights to e4m3 first."""
    import torch

    from . import binding as B
    from . import synth
    dev = "cuda"
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    mc = synth.moe_cfg(2816, 128, 8, 704, 704)
    g = synth.generator(53, dev)
    w = synth.moe_weights(mc, g, device=dev)
    if fp8:
        w = B.quantize_moe_weights(w)
        mc["expert_format"] = "fp8_e4m3"
    x = synth.hidden_states(256, 2816, g, "bf16", dev)
    for _ in range(n_reps):
        B.dg_moe_block(mc, w, x)
    torch.cuda.synchronize()
    print("pmc workload done", flush=True)


def attn_workload(n_reps=20):
    """The attention layers of the canvas step at its shape (256 canvas rows
    after 4,096 committed rows; the sliding layer's window of 1,024 and the
    global layer's 4,352 keys), n_reps calls of each; run under rocprofv3
    --kernel-trace --stats or --pmc."""
    import torch

    from . import binding as B
    from . import synth
    P, C = 4096, 256
    for cfg in (synth.sliding_cfg(), synth.global_cfg()):
        g = synth.generator(5)
        w = {k: (v.cuda() if v is not None else None) for k, v in synth.attn_weights(cfg, g).items()}
        cap = P + C
        ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], cap, cfg["head_dim"], g, "bf16")
        kd, vtd = ck.cuda(), cv.transpose(1, 2).contiguous().cuda()
        x = synth.hidden_states(C, cfg["hidden"], g, "bf16").cuda()
        for _ in range(n_reps):
            xd = x.clone()
            B.dg_attn_layer(cfg, w, kd, vtd, P, xd, 0)
        torch.cuda.synchronize()
        print(f"attention workload: layer type {cfg['layer_type']} done", flush=True)


def summarize_counters(counter_csvs, name_part="attn_"):
    """Per kernel (name containing name_part): the mean over dispatches of
    each counter, summed over its instances, from rocprofv3 --pmc runs."""
    per = {}   # (kernel, counter) -> per-run means (dispatch ids restart in every run)
    for path in counter_csvs:
        run = {}
        for r in _rows(path):
            n = r["Kernel_Name"]
            if name_part not in n:
                continue
            short = n.split("(anonymous namespace)::")[-1].split("(")[0]
            d = run.setdefault((short, r["Counter_Name"]), {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        for key, d in run.items():
            per.setdefault(key, []).append(sum(d.values()) / len(d))
    kernels = sorted({k for k, _ in per})
    out = []
    for k in kernels:
        vals = {c: sum(m) / len(m) for (kk, c), m in per.items() if kk == k}
        out.append(k)
        for c in sorted(vals):
            out.append(f"  {c:28s} {vals[c]:16.0f}")
        waves = vals.get("SQ_WAVES")
        if waves:
            for c, label in (("SQ_INSTS_VALU", "VALU instructions per wave"), ("SQ_INSTS_MFMA", "MFMA instructions per wave"),
                             ("SQ_INSTS_LDS", "LDS instructions per wave")):
                if c in vals:
                    out.append(f"  {label:28s} {vals[c] / waves:16.1f}")
    return "\n".join(out) + "\n"


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, name_part, counter):
    """Mean over dispatches of kernels whose name contains name_part of the
    counter summed over its instances."""
    per = {}
    for r in rows:
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of {name_part!r} with counter {counter}")
    v = sorted(per.values())
    return sum(v) / len(v), len(v)


def summarize_traffic(fetch_csv, write_csv, command, algorithmic_bytes, fp8=False, product="gate/up"):
    if product == "down":
        kern = DOWN_KERNEL_FP8 if fp8 else DOWN_KERNEL
    else:
        kern = GATEUP_KERNEL_FP8 if fp8 else GATEUP_KERNEL
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    cf, ncf = _per_dispatch(fr, COPY_KERNEL, "FETCH_SIZE")
    cw, ncw = _per_dispatch(wr, COPY_KERNEL, "WRITE_SIZE")
    gf, ngf = _per_dispatch(fr, kern, "FETCH_SIZE")
    gw, ngw = _per_dispatch(wr, kern, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    ff, fw = kib / cf, kib / cw          # bytes actually moved per counted KiB, in KiB
    fetch_b = gf * ff * 1024.0
    write_b = gw * fw * 1024.0
    lines = [
        f"# HBM traffic of the expert {product} launch (MoE layer, 256-token canvas, 128 experts top-8 + shared"
        + (", fp8 e4m3 weights)" if fp8 else ")"),
        f"kernel: {kern}",
        f"command: {command}",
        f"gemm_source_hash: {gemm_source_hash()}",
        f"copy calibration: {COPY_BYTES} B device copy; FETCH_SIZE {cf:.0f} KiB ({ncf} dispatches), "
        f"WRITE_SIZE {cw:.0f} KiB ({ncw}); factors fetch {ff:.4f}, write {fw:.4f}",
        f"{product} raw: FETCH_SIZE {gf:.0f} KiB ({ngf} dispatches), WRITE_SIZE {gw:.0f} KiB ({ngw})",
        f"{product} scaled: fetch_bytes {fetch_b:.0f}, write_bytes {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {algorithmic_bytes}",
        f"traffic / algorithmic: {(fetch_b + write_b) / algorithmic_bytes:.3f}",
    ]
    return "\n".join(lines) + "\n"


def summarize_stats(stats_csv, command, top=25, step_calls=None):
    rows = _rows(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"command: {command}", f"gemm_source_hash: {gemm_source_hash()}",
           f"{'total_ms':>9} {'calls':>6} {'avg_us':>9} {'pct':>6}  kernel"]
    for r in rows[:top]:
        name = r["Name"].replace("void dg::(anonymous namespace)::", "").replace("dg::(anonymous namespace)::", "")
        out.append(f"{float(r['TotalDurationNs']) / 1e6:9.2f} {int(r['Calls']):6d} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {100 * float(r['TotalDurationNs']) / tot:6.2f}  {name[:150]}")
    return "\n".join(out) + "\n"


def summarize_step(trace_csv, marker="sample_finalize_kernel"):
    """Per-kernel time inside one denoising step: the launches after one
    sampler finalisation up to the next.  Of the complete steps in the trace
    (same launch count as the last one) the one with the median span is
    shown, so a host stall under the profiler does not stand for the step."""
    rows = _rows(trace_csv)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    idx = [i for i, r in enumerate(rows) if marker in r["Kernel_Name"]]
    if len(idx) < 2:
        return "no complete step in the trace\n"
    steps = [rows[i + 1: j + 1] for i, j in zip(idx[:-1], idx[1:])]
    steps = [q for q in steps if len(q) == len(steps[-1])]
    steps.sort(key=lambda q: int(q[-1]["End_Timestamp"]) - int(q[0]["Start_Timestamp"]))
    seq = steps[len(steps) // 2]
    agg = {}
    for r in seq:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = r["Kernel_Name"].replace("void dg::(anonymous namespace)::", "").replace("dg::(anonymous namespace)::", "")
        name = name.split("(")[0]
        t, c = agg.get(name, (0.0, 0))
        agg[name] = (t + d, c + 1)
    span = (int(seq[-1]["End_Timestamp"]) - int(seq[0]["Start_Timestamp"])) / 1e3
    busy = sum(t for t, _ in agg.values())
    out = [f"one step: {len(seq)} launches, span {span:.1f} us, kernel time {busy:.1f} us",
           f"{'step_us':>9} {'calls':>6} {'avg_us':>9} {'pct':>6}  kernel"]
    for name, (t, c) in sorted(agg.items(), key=lambda x: -x[1][0]):
        out.append(f"{t:9.1f} {c:6d} {t / c:9.2f} {100 * t / busy:6.2f}  {name[:150]}")
    return "\n".join(out) + "\n"


def traffic_path(fp8=False):
    name = "moe_gateup_fp8_traffic_canvas256.txt" if fp8 else "moe_gateup_traffic_canvas256.txt"
    return os.path.join(ROOT, "profiles", name)


def read_traffic(path=None, fp8=False):
    """Stored traffic per launch, or None when absent or taken on other GEMM sources."""
    path = path or traffic_path(fp8)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("gemm_source_hash") != gemm_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "traffic":
        fetch_csv, write_csv, command, alg = sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5])
        fp8 = len(sys.argv) > 6 and sys.argv[6] == "fp8"
        product = sys.argv[7] if len(sys.argv) > 7 else "gate/up"
        sys.stdout.write(summarize_traffic(fetch_csv, write_csv, command, alg, fp8=fp8, product=product))
    elif what == "counters":
        sys.stdout.write(summarize_counters(sys.argv[2:]))
    elif what == "stats":
        sys.stdout.write(summarize_stats(sys.argv[2], sys.argv[3]))
        if len(sys.argv) > 4:
            sys.stdout.write("\n" + summarize_step(sys.argv[4]))
    else:
        raise SystemExit("usage: profiling.py traffic|stats|counters ...")
