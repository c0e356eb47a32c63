#!/usr/bin/env python3
"""One-GPU benchmark of the TwoTower denoiser hot path on MI355X.

Workload: the full denoise loop for one 16-token block -- B=32 sequences,
6 attention layers with independent paged bf16 context caches (H_q=32,
H_kv=2, D=128, 256-token pages, lengths uniform over multiples of 16 in
[2048, 8192]), T=4 denoise steps, each step = 6 x tt_block_attn + 1 x tt_unmask
on fp32 logits [512, 131072] committing ceil(masked / remaining) slots per
sequence, then 6 x tt_kv_append (block commit).

One bench step = one block = 4 denoise steps + the commit; the block's state
(ctx_lens, mask) is reset from a saved copy at the start of each block so
every block runs the same workload.  value = denoise steps per second for the
whole batch.  Inputs are resident in HBM before timing; the 1 GiB of per-step
logits and ~1.1 GB of caches exceed the 256 MB Infinity Cache, so the loop
streams from HBM.

The dominant kernel (block attention) is timed again on its own with HIP
events (rotating over the 24 (step, layer) inputs) for the roofline entry;
the CPU oracle is timed on a bounded sample for the cpu_baseline entry.

The same line carries block attention alone at the other measured shapes
(configs 2-4: B=8 x 4K, a ragged B=64 batch of 1K-16K contexts, B=4 x 64K),
each with inputs rotated over more than 768 MB so that the Infinity Cache
cannot serve them, against the HBM and MFMA peaks and a measured copy rate;
and the oracle timed over whole configs 1-4 on all host threads (configs 1
and 2 also on one).  `--config N` runs config N's attention alone.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("block-attn HBM GB/s & TFLOP/s (fraction of peak); denoise-steps/sec, 1 GPU")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# bytes the rotating input sets of a config total at least: three times the
# 256 MB Infinity Cache, so every launch streams its inputs from HBM
ROT_BYTES = 768 * 10 ** 6
ATTN_WORKLOADS = {
    2: "block attention, B=8, S=16, H_q=32, H_kv=2, D=128, L=4096 each, 256-token bf16 pages",
    3: ("block attention, ragged decode batch: B=64, S=16, H_q=32, H_kv=2, D=128, L uniform over "
        "multiples of 16 in [1024, 16384], 256-token bf16 pages"),
    4: "block attention, long context: B=4, S=16, H_q=32, H_kv=2, D=128, L=65536 each, 256-token bf16 pages",
    5: ("block attention of one denoise-loop layer: B=32, S=16, H_q=32, H_kv=2, D=128, L uniform over "
        "multiples of 16 in [2048, 8192], 256-token bf16 pages"),
}


def counters_file(cfg):
    return os.path.join(ROOT, "profiles", "attn_split_config%d_counters.md" % cfg)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def attn_source_hash():
    """Identifies the attention kernel source the counters were taken on."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "two_tower_attention_amd", "csrc", "attn_bf16.hip"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(cfg):
    """HBM bytes per launch of a config's attention from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None."""
    path = counters_file(cfg)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("COUNTERS_JSON "):
                rec = json.loads(line[len("COUNTERS_JSON "):])
    if not rec or rec.get("source_hash") != attn_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


CALIB_BYTES = 256 << 20
ATTN_KERNELS = ("attn_split_kernel", "attn_combine_kernel")


def _read_counters(path, counter):
    """Mean per-dispatch value of `counter` per kernel family from a rocprofv3
    counter_collection.csv."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if "attn_split_kernel" in name:
                key = "attn_split_kernel"
            elif "attn_combine_kernel" in name:
                key = "attn_combine_kernel"
            elif "direct_copy" in name or "copyBuffer" in name:
                key = "copy"
            else:
                continue
            per.setdefault(key, []).append(float(r["Counter_Value"]))
    return per


def summarize_pmc(fetch_csv, write_csv, out_md, command="", cfg=5):
    fetch = _read_counters(fetch_csv, "FETCH_SIZE")
    write = _read_counters(write_csv, "WRITE_SIZE")
    # the calibration copy is the largest copy dispatch
    cf, cw = max(fetch["copy"]), max(write["copy"])
    kib = CALIB_BYTES / 1024.0
    sf, sw = kib / cf, kib / cw
    rec = {"source_hash": attn_source_hash(), "fetch_scale": sf, "write_scale": sw}
    lines = ["# Attention HBM traffic counters (config %d)" % cfg, "",
             "Workload: %s." % ATTN_WORKLOADS[cfg], "",
             "Counters from two `rocprofv3 --pmc` passes (FETCH_SIZE, then WRITE_SIZE, KiB per",
             "dispatch) over `python3 bench.py --config %d --only-attn`, scaled by the same counter on a plain" % cfg,
             "256 MiB device copy (fetch scale %.4f, write scale %.4f)." % (sf, sw), "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |",
             "|---|---|---|---|---|"]
    total = 0.0
    for k in ATTN_KERNELS:
        f = sum(fetch.get(k, [0])) / max(len(fetch.get(k, [])), 1)
        w = sum(write.get(k, [0])) / max(len(write.get(k, [])), 1)
        b = (f * sf + w * sw) * 1024.0
        total += b
        lines.append("| %s | %d | %.0f | %.0f | %.3e |" % (k, len(fetch.get(k, [])), f, w, b))
        rec[k] = {"fetch_kib": f, "write_kib": w, "bytes": b}
    rec["hbm_bytes_per_launch"] = total
    lines += ["", "HBM bytes per tt_block_attn launch (split + combine): %.4e" % total, ""]
    if command:
        lines += ["Command (run from /tmp on the GPU host, REPO = the repository root):", "", "```",
                  command, "```", ""]
    lines += ["COUNTERS_JSON " + json.dumps(rec)]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _short_kernel(name):
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    cut = [i for i in (n.find("("), n.find("<")) if i > 0]
    return (n[:min(cut)] if cut else n)[:60]


def summarize_pmc_all(fetch_csv, write_csv, out_md, title, command=""):
    """Every kernel's mean FETCH_SIZE / WRITE_SIZE per dispatch, scaled by
    what the counters read for the run's 256 MiB calibration copy (its
    largest copy dispatch)."""
    import csv
    data = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = _short_kernel(r["Kernel_Name"])
                data.setdefault(k, {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    copies = [k for k in data if "copy" in k.lower() or "Copy" in k]
    cf = max(max(data[k].get("FETCH_SIZE", [0])) for k in copies)
    cw = max(max(data[k].get("WRITE_SIZE", [0])) for k in copies)
    kib = CALIB_BYTES / 1024.0
    sf, sw = kib / cf, kib / cw
    lines = ["# %s" % title, "",
             "Counters from two `rocprofv3 --pmc` passes (FETCH_SIZE, then WRITE_SIZE, KiB per",
             "dispatch, mean over dispatches), scaled by the same counter on the run's plain",
             "256 MiB device copy (fetch scale %.4f, write scale %.4f)." % (sf, sw), "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB (scaled) |",
             "|---|---|---|---|---|---|"]
    rows = []
    for k, v in data.items():
        f = v.get("FETCH_SIZE", [0.0])
        w = v.get("WRITE_SIZE", [0.0])
        fm, wm = sum(f) / len(f), sum(w) / len(w)
        rows.append((fm * sf + wm * sw, k, len(f), fm, wm))
    for _, k, n, fm, wm in sorted(rows, reverse=True)[:16]:
        lines.append("| %s | %d | %.0f | %.0f | %.1f | %.1f |" % (
            k, n, fm, wm, fm * sf * 1024 / 1e6, wm * sw * 1024 / 1e6))
    if command:
        lines += ["", "Commands (run from /tmp on the GPU host, REPO = the repository root):", "",
                  "```", command, "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq(csv_a, csv_b, out_md, cfg, command=""):
    """The attention split kernel's SQ counters (two passes of 8) and the
    ratios that locate its bound: wait and issue stalls per wave cycle, MFMA
    busy per SIMD cycle, LDS instructions per MFMA, bank conflicts."""
    import csv
    vals = {}
    for path in (csv_a, csv_b):
        with open(path) as f:
            for r in csv.DictReader(f):
                if "attn_split_kernel" in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    ndisp = len(vals.get("SQ_WAVES", []))
    lines = ["# Attention split kernel: SQ counters (config %d)" % cfg, "",
             "Workload: %s." % ATTN_WORKLOADS[cfg], "",
             "Two `rocprofv3 --pmc` passes of 8 SQ counters each over `python3 bench.py --config %d "
             "--only-attn` (%d dispatches of `attn_split_kernel`; mean per dispatch, totals over the "
             "chip)." % (cfg, ndisp), "", "| counter | mean per dispatch |", "|---|---|"]
    for k in sorted(m):
        lines.append("| %s | %.4g |" % (k, m[k]))
    g = lambda k: m.get(k, float("nan"))
    lines += ["", "Derived (ratios of counters in the same unit):", "", "| quantity | value |", "|---|---|",
              "| MFMA instructions per launch | %.3g M |" % (g("SQ_INSTS_MFMA") / 1e6),
              "| LDS instructions per MFMA instruction (SQ_INSTS_LDS / SQ_INSTS_MFMA) | %.2f |"
              % (g("SQ_INSTS_LDS") / g("SQ_INSTS_MFMA")),
              "| VALU instructions per MFMA instruction (SQ_INSTS_VALU / SQ_INSTS_MFMA) | %.2f |"
              % (g("SQ_INSTS_VALU") / g("SQ_INSTS_MFMA")),
              "| wave cycles waiting at s_waitcnt (SQ_WAIT_ANY / SQ_WAVE_CYCLES) | %.0f%% |"
              % (100 * g("SQ_WAIT_ANY") / g("SQ_WAVE_CYCLES")),
              "| wave cycles not issuing (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) | %.0f%% |"
              % (100 * g("SQ_WAIT_INST_ANY") / g("SQ_WAVE_CYCLES")),
              "| wave cycles waiting to issue an LDS instruction (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES) | %.1f%% |"
              % (100 * g("SQ_WAIT_INST_LDS") / g("SQ_WAVE_CYCLES")),
              "| LDS bank conflict cycles per LDS-active cycle (SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS) | %.1f%% |"
              % (100 * g("SQ_LDS_BANK_CONFLICT") / g("SQ_ACTIVE_INST_LDS")),
              "| MFMA busy per SIMD cycle (SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES)) | %.0f%% |"
              % (100 * g("SQ_VALU_MFMA_BUSY_CYCLES") / (4 * g("SQ_BUSY_CU_CYCLES")))]
    if command:
        lines += ["", "Commands (run from /tmp on the GPU host, REPO = the repository root):", "",
                  "```", command, "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def calibration_copy(torch, dev):
    """A plain 256 MiB device copy: the reference dispatch for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a run."""
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def summarize_stats(stats_csv, out_md, command=""):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows[:12]:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        short = name.split("(")[0]
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.2f |" % (
            short[:80], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if command:
        lines += ["", "Command (run from /tmp on the GPU host, REPO = the repository root):", "", "```",
                  command, "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def lmhead_bench(np, torch, tt, workloads, dev, B=32, S=16, H=4096, V=131072, iters=20, warm=20):
    """The LM head fused with the unmask (tt_lmhead_unmask) at the unmask
    workload's shape with a head of hidden size H_q * D = 4096, against the
    same head as a library GEMM to fp32 logits followed by tt_unmask."""
    rng = np.random.Generator(np.random.PCG64(57))
    c = workloads.make_lmhead_case(rng, B, S, H, V, seed=57)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    hid, w = bf(c.hidden), bf(c.weight)
    del c
    mask = torch.ones((B, S), dtype=torch.uint8, device=dev)
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    com = torch.empty((B, S), dtype=torch.uint8, device=dev)
    conf = torch.empty((B, S), dtype=torch.float32, device=dev)
    ws = torch.empty(tt.tt_lmhead_unmask_workspace_bytes(B, S, V, H), dtype=torch.uint8, device=dev)
    uws = torch.empty(max(16, tt.tt_unmask_workspace_bytes(B, S, V)), dtype=torch.uint8, device=dev)

    # both paths run warm-up calls first: the clock rises over the first tens
    # of milliseconds of sustained matrix-core load
    def timeit(f):
        for _ in range(warm):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / iters

    t_f = timeit(lambda: tt.tt_lmhead_unmask(hid, w, mask, None, 4, ids, com, conf, 0, ws))
    wt = w.t()
    try:
        gemm = lambda: torch.mm(hid, wt, out_dtype=torch.float32)
        gemm()
        kind = "torch.mm bf16 -> fp32 (hipBLASLt)"
    except Exception:
        gemm = lambda: torch.mm(hid, wt).float()
        kind = "torch.mm bf16 -> bf16, widened to fp32"
    t_g = timeit(gemm)
    logits = gemm().contiguous()
    t_u = timeit(lambda: tt.tt_unmask(logits, mask, None, 4, ids, com, conf, 0, uws))
    del logits
    flops = 2.0 * B * S * H * V
    log("lm head + unmask: fused %.1f us (%.0f TFLOP/s); unfused %.1f us (GEMM %.1f + unmask %.1f)"
        % (t_f * 1e6, flops / t_f / 1e12, (t_g + t_u) * 1e6, t_g * 1e6, t_u * 1e6))
    return {"us_per_call": t_f * 1e6, "TFLOP/s": flops / t_f / 1e12,
            "frac_mfma": flops / t_f / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "weight_GB/s": V * H * 2 / t_f / 1e9,
            "unfused_us": (t_g + t_u) * 1e6, "unfused_gemm_us": t_g * 1e6, "unfused_unmask_us": t_u * 1e6,
            "unfused_gemm": kind, "speedup_vs_unfused": (t_g + t_u) / t_f,
            "shape": "hidden [%d, %d] x head [%d, %d] bf16 -> ids/conf/commit (k = ceil(16/4))"
                     % (B * S, H, V, H),
            "weights": "synthetic: hidden ~ N(0,1), head ~ N(0, 9/H), so logits ~ N(0, 3^2)"}


def attn_bytes_flops(np, c):
    """Algorithmic bytes (context K/V once, Q and O, the block's K/V) and
    flops (Q.K^T and P.V over context plus block keys) of one launch."""
    lens = c.ctx_lens.astype(np.int64)
    kv = int(lens.sum()) * c.Hkv * c.D * 2 * 2
    qo = 2 * c.B * c.S * c.Hq * c.D * 2
    blk = 2 * c.B * c.S * c.Hkv * c.D * 2
    flops = 4 * c.D * c.S * c.Hq * int((lens + c.S).sum())
    return kv + qo + blk, flops


def copy_bandwidth(torch, dev, nbytes=1 << 30, iters=10):
    """Device-to-device copy of 1 GiB (read + write counted): the streaming
    rate a plain copy kernel reaches on this GPU."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / iters
    del src, dst
    return {"GB/s": 2.0 * nbytes / t / 1e9, "bytes_per_copy": 2 * nbytes,
            "kernel": "torch device-to-device copy_ of 1 GiB fp32 (read + write bytes)"}


def attn_config_bench(np, torch, tt, workloads, dev, cfg, copy_gbs, iters=48, graph=True):
    """One config's block attention timed alone: inputs rotated over enough
    device copies that they total more than ROT_BYTES, HIP events on the
    launch stream around `iters` launches (eager, then replayed from a HIP
    graph)."""
    c = {2: workloads.config2, 3: workloads.config3, 4: workloads.config4}[cfg]()
    nbytes, flops = attn_bytes_flops(np, c)
    copies = ROT_BYTES // nbytes + 1
    iters = -(-max(iters, copies) // copies) * copies

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = [bf(c.q), bf(c.k_blk), bf(c.v_blk), bf(c.k_pages), bf(c.v_pages),
            torch.from_numpy(c.page_table).to(dev), torch.from_numpy(c.ctx_lens).to(dev)]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    desc = tt.make_desc(c.B, c.S, c.Hq, c.Hkv, c.D, c.page_size, c.page_table.shape[1],
                        c.k_pages.shape[0], int(c.ctx_lens.max()))
    out = torch.empty((c.B, c.S, c.Hq, c.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(tt.tt_block_attn_workspace_bytes(desc), 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def loop():
        for it in range(iters):
            tt.tt_block_attn(desc, *sets[it % copies], out, ws)

    loop()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    loop()
    e1.record(stream)
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / 1e3 / iters
    t = t_eager
    if graph:
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(stream)
        with torch.cuda.stream(s_cap):
            with torch.cuda.graph(g, stream=s_cap):
                loop()
        stream.wait_stream(s_cap)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / iters
        del g
    gbs, tfs = nbytes / t / 1e9, flops / t / 1e12
    lens = c.ctx_lens.astype(np.int64)
    res = {"workload": ATTN_WORKLOADS[cfg], "us_per_launch": t * 1e6,
           "us_per_launch_eager": t_eager * 1e6, "launches_timed": iters,
           "alg_bytes_per_launch": nbytes, "alg_flops_per_launch": flops,
           "GB/s": gbs, "TFLOP/s": tfs, "frac_hbm": gbs / HBM_PEAK_GBS,
           "frac_mfma": tfs / MFMA_BF16_PEAK_TFLOPS,
           "frac_copy": gbs / copy_gbs if copy_gbs else None,
           "mean_ctx_len": float(lens.mean()), "seed": c.seed,
           "rotation": {"sets": copies, "bytes": copies * nbytes},
           "traffic": read_traffic(cfg), "timing": "graph replay" if graph else "eager"}
    log("config %d attention: %.1f us/launch (eager %.1f), %.0f GB/s (%.2f of HBM, %.2f of copy), "
        "%.0f TFLOP/s; %d rotating sets" % (cfg, t * 1e6, t_eager * 1e6, gbs, gbs / HBM_PEAK_GBS,
                                             res["frac_copy"] or 0.0, tfs, copies))
    del sets, base, out, ws
    return res


def oracle_timings(np, workloads, configs=(1, 2, 3, 4), single=(1, 2)):
    """The fp64 CPU oracle's block attention over whole configs (every query
    row), on all OpenMP threads and, for the small configs, on one."""
    import oracle
    makers = {1: lambda: workloads.config1()[0], 2: workloads.config2, 3: workloads.config3,
              4: workloads.config4}
    nthr = oracle.num_threads()
    res = {"threads": nthr, "kind": "oracle",
           "what": "oracle.block_attn over every query row of the config (fp64 C, OpenMP)"}

    def one(c, threads):
        with oracle.threads(threads):
            t0 = time.perf_counter()
            oracle.block_attn(c)
            dt = time.perf_counter() - t0
        rows = c.B * c.S * c.Hq
        return {"s": dt, "threads": threads, "rows": rows, "rows_per_s": rows / dt}

    for k in configs:
        c = makers[k]()
        res["config%d" % k] = one(c, nthr)
        if k in single:
            res["config%d_1thread" % k] = one(c, 1)
        log("oracle config %d: %.2f s on %d threads%s" % (
            k, res["config%d" % k]["s"], nthr,
            (", %.2f s on 1" % res["config%d_1thread" % k]["s"]) if k in single else ""))
        del c
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", type=int, default=5, choices=(2, 3, 4, 5),
                    help="5: the denoise loop (headline line, with configs 2-4 as attention "
                         "entries); 2, 3, 4: that config's block attention alone")
    ap.add_argument("--steps", type=int, default=20, help="timed blocks (4 denoise steps each)")
    # the matrix cores' clock ramps up over the first tens of milliseconds of
    # sustained load; 20 untimed blocks (about 36 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-iters", type=int, default=96, help="launches in the attention-only timing")
    ap.add_argument("--only-attn", action="store_true",
                    help="counter runs: attention launches plus one 256 MiB calibration copy")
    ap.add_argument("--core", action="store_true",
                    help="kernel-trace runs: the denoise loop and the attention timing only (no "
                         "chunk ingest, block sizes, threshold unmask or CPU baseline)")
    ap.add_argument("--only-lmhead", action="store_true",
                    help="kernel-trace runs: the fused LM head + unmask timing only (prints that "
                         "section's JSON)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files into a summary")
    ap.add_argument("--summarize-pmc-all", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD", "TITLE"),
                    help="every kernel's FETCH_SIZE / WRITE_SIZE from two counter runs")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("CSV_A", "CSV_B", "OUT_MD"),
                    help="the attention split kernel's SQ counters from two counter runs")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="turn a rocprofv3 --stats kernel_stats.csv into a summary")
    ap.add_argument("--profile-command", default="",
                    help="command line recorded in a --summarize-* summary")
    ap.add_argument("--only-block", type=int, default=0, choices=(0, 8, 32, 64),
                    help="counter runs: the denoise layer's attention at this block size alone")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the config 2-4 attention entries and the oracle timings")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, command=args.profile_command, cfg=args.config)
        return
    if args.summarize_pmc_all:
        summarize_pmc_all(*args.summarize_pmc_all, command=args.profile_command)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq, cfg=args.config, command=args.profile_command)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats, command=args.profile_command)
        return
    if args.core:
        args.no_cpu_baseline = True
    extras = not (args.only_attn or args.core)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import two_tower_attention_amd as tt
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not os.path.exists(tt.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    tt.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only_lmhead:
        print(json.dumps({"lmhead_unmask": lmhead_bench(np, torch, tt, workloads, dev)}), flush=True)
        calibration_copy(torch, dev)
        return
    if args.config != 5:
        config_main(args, np, torch, tt, workloads, dev)
        return

    t_gen = time.perf_counter()
    lp = workloads.config5(extra_blocks=1)
    B, S, T, NL, V = lp.B, lp.S, lp.steps, lp.layers, lp.vocab
    log("generated inputs in %.1fs" % (time.perf_counter() - t_gen))

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    p0 = lp.pools[0]
    desc = tt.make_desc(B, S, lp.Hq, lp.Hkv, lp.D, lp.page_size, p0.page_table.shape[1],
                        p0.k_pages.shape[0], int(p0.ctx_lens.max()))
    kp = [dev_bf16(p.k_pages) for p in lp.pools]
    vp = [dev_bf16(p.v_pages) for p in lp.pools]
    pt = [dev_t(p.page_table) for p in lp.pools]
    ctx0 = torch.stack([dev_t(p.ctx_lens) for p in lp.pools])       # [NL, B] saved lengths
    ctx = ctx0.clone()
    q = [[dev_bf16(lp.q[s][i]) for i in range(NL)] for s in range(T)]
    kb = [[dev_bf16(lp.k_blk[s][i]) for i in range(NL)] for s in range(T)]
    vb = [[dev_bf16(lp.v_blk[s][i]) for i in range(NL)] for s in range(T)]
    logits = [dev_t(l) for l in lp.logits]
    ones = torch.ones((B, S), dtype=torch.uint8, device=dev)
    mask = ones.clone()
    out = [torch.empty((B, S, lp.Hq, lp.D), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    com = torch.empty((B, S), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(tt.tt_block_attn_workspace_bytes(desc), 16), dtype=torch.uint8, device=dev)
    uws = torch.empty(max(tt.tt_unmask_workspace_bytes(B, S, V), 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def attn(s, i, stream=None):
        tt.tt_block_attn(desc, q[s][i], kb[s][i], vb[s][i], kp[i], vp[i], pt[i], ctx[i], out[i],
                         ws, stream)

    def block_size_bench(S2):
        """One attention launch per layer at block size S2 over the loop's
        context pools, timed over 4 rounds of the layers (HIP events)."""
        lens2 = p0.ctx_lens.astype(np.int64)
        kvb = int(lens2.sum()) * lp.Hkv * lp.D * 2 * 2
        stream2 = torch.cuda.current_stream()
        d2 = tt.make_desc(B, S2, lp.Hq, lp.Hkv, lp.D, lp.page_size, p0.page_table.shape[1],
                          p0.k_pages.shape[0], int(p0.ctx_lens.max()))
        rng2 = np.random.Generator(np.random.PCG64(lp.seed * 100 + S2))
        inp = [[dev_bf16(a) for a in workloads.block_inputs(rng2, B, S2, lp.Hq, lp.Hkv, lp.D)]
               for _ in range(NL)]
        o2 = torch.empty((B, S2, lp.Hq, lp.D), dtype=torch.bfloat16, device=dev)
        ws2 = torch.empty(max(tt.tt_block_attn_workspace_bytes(d2), 16), dtype=torch.uint8,
                          device=dev)
        ctx.copy_(ctx0)
        n2 = 4 * NL

        def launches():
            for it in range(n2):
                i = it % NL
                tt.tt_block_attn(d2, *inp[i], kp[i], vp[i], pt[i], ctx[i], o2, ws2)

        launches()                       # warm-up (also settles the clock)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream2)
        launches()
        b1.record(stream2)
        torch.cuda.synchronize()
        t2 = b0.elapsed_time(b1) / 1e3 / n2
        if not args.no_graph and not args.only_block:
            # replayed from a HIP graph like the other attention figures: kernel
            # time plus the inter-kernel gaps, without the host's launch cost
            g2 = torch.cuda.CUDAGraph()
            s_cap = torch.cuda.Stream()
            s_cap.wait_stream(stream2)
            with torch.cuda.stream(s_cap):
                with torch.cuda.graph(g2, stream=s_cap):
                    launches()
            stream2.wait_stream(s_cap)
            g2.replay()
            torch.cuda.synchronize()
            b0.record(stream2)
            g2.replay()
            b1.record(stream2)
            torch.cuda.synchronize()
            t2 = b0.elapsed_time(b1) / 1e3 / n2
            del g2
        by2 = kvb + 2 * B * S2 * lp.Hq * lp.D * 2 + 2 * B * S2 * lp.Hkv * lp.D * 2
        fl2 = 4 * lp.D * S2 * lp.Hq * int((lens2 + S2).sum())
        log("block size %d: %.1f us/launch, %.0f GB/s, %.0f TFLOP/s" % (
            S2, t2 * 1e6, by2 / t2 / 1e9, fl2 / t2 / 1e12))
        return {"us_per_launch": t2 * 1e6, "GB/s": by2 / t2 / 1e9, "TFLOP/s": fl2 / t2 / 1e12,
                "frac_hbm": by2 / t2 / 1e9 / HBM_PEAK_GBS,
                "frac_mfma": fl2 / t2 / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "query_chunks": -(-S2 * (lp.Hq // lp.Hkv) // 256),
                "timing": "graph replay" if not args.no_graph else "eager"}

    if args.only_block:
        # counter runs: this block size's attention alone, then the calibration copy
        block_size_bench(args.only_block)
        calibration_copy(torch, dev)
        return

    def one_block():
        ctx.copy_(ctx0)
        mask.copy_(ones)
        for s in range(T):
            for i in range(NL):
                attn(s, i)
            tt.tt_unmask(logits[s], mask, None, T - s, ids, com, None, tt.TT_UNMASK_UPDATE_MASK, uws)
        for i in range(NL):
            tt.tt_kv_append(desc, kb[T - 1][i], vb[T - 1][i], kp[i], vp[i], pt[i], ctx[i])

    use_graph = not args.no_graph and not args.only_attn
    graph = None
    if not args.only_attn:
        one_block()                      # eager run first (also warms the library)
        torch.cuda.synchronize()
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            s_cap = torch.cuda.Stream()
            s_cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_cap):
                with torch.cuda.graph(graph, stream=s_cap):
                    one_block()
            torch.cuda.current_stream().wait_stream(s_cap)
            torch.cuda.synchronize()
        run = graph.replay if graph is not None else one_block
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_s = e0.elapsed_time(e1) / 1e3
        log("timed %d blocks: wall %.3f ms, events %.3f ms" % (args.steps, wall * 1e3, ev_s * 1e3))
        block_s = max(wall, ev_s) / args.steps
        # the last block must have committed every slot
        assert int(mask.sum().item()) == 0, "denoise loop left masked slots"
    else:
        block_s = float("nan")

    # ---- attention alone, HIP events on the launch stream, rotating inputs.
    # The launches are replayed from a HIP graph (as in the timed loop), so the
    # figure is kernel time plus the inter-kernel gaps, not host launch cost;
    # the eagerly launched figure is reported beside it.
    stream = torch.cuda.current_stream()
    ctx.copy_(ctx0)
    copy_bw = None if (args.only_attn or args.core) else copy_bandwidth(torch, dev)
    if copy_bw:
        log("copy bandwidth: %.0f GB/s" % copy_bw["GB/s"])
    for it in range(6):
        attn(it % T, it % NL)
    torch.cuda.synchronize()

    def attn_loop():
        for it in range(args.attn_iters):
            attn((it // NL) % T, it % NL)

    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    attn_loop()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_eager_s = a0.elapsed_time(a1) / 1e3 / args.attn_iters
    attn_s = attn_eager_s
    if not args.no_graph and not args.only_attn:
        agraph = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(stream)
        with torch.cuda.stream(s_cap):
            with torch.cuda.graph(agraph, stream=s_cap):
                attn_loop()
        stream.wait_stream(s_cap)
        agraph.replay()
        torch.cuda.synchronize()
        a0.record(stream)
        agraph.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        attn_s = a0.elapsed_time(a1) / 1e3 / args.attn_iters
        del agraph
    log("attention: eager %.1f us/launch, graph replay %.1f us/launch" % (attn_eager_s * 1e6, attn_s * 1e6))
    # the context tower's causal chunk ingest on the same inputs
    chunk_s = None
    if extras:
        a0.record(stream)
        for it in range(args.attn_iters):
            s_, i_ = (it // NL) % T, it % NL
            tt.tt_chunk_attn(desc, q[s_][i_], kb[s_][i_], vb[s_][i_], kp[i_], vp[i_], pt[i_], ctx[i_],
                             out[i_], ws)
        a1.record(stream)
        torch.cuda.synchronize()
        chunk_s = a0.elapsed_time(a1) / 1e3 / args.attn_iters
    lens = p0.ctx_lens.astype(np.int64)
    kv_bytes = int(lens.sum()) * lp.Hkv * lp.D * 2 * 2
    qo_bytes = 2 * B * S * lp.Hq * lp.D * 2
    blk_bytes = 2 * B * S * lp.Hkv * lp.D * 2
    attn_bytes = kv_bytes + qo_bytes + blk_bytes
    attn_flops = 4 * lp.D * S * lp.Hq * int((lens + S).sum())
    attn_gbs = attn_bytes / attn_s / 1e9
    attn_tfs = attn_flops / attn_s / 1e12
    log("attention: %.1f us/launch, %.0f GB/s, %.0f TFLOP/s" % (attn_s * 1e6, attn_gbs, attn_tfs))
    chunk = None
    if chunk_s is not None:
        chunk = {"us_per_launch": chunk_s * 1e6, "GB/s": attn_bytes / chunk_s / 1e9,
                 "frac_hbm": attn_bytes / chunk_s / 1e9 / HBM_PEAK_GBS,
                 "workload": "causal chunk ingest of the 16-token block, same layer inputs"}
        log("chunk ingest: %.1f us/launch, %.0f GB/s" % (chunk_s * 1e6, chunk["GB/s"]))

    # ---- sampling block sizes: one attention launch per layer at S = 8, 32,
    # 64 over the same context pools (the pages' block-size knob)
    block_sizes = None
    if extras:
        block_sizes = {str(S2): block_size_bench(S2) for S2 in (8, 32, 64)}

    # ---- unmask alone (flags 0: the all-masked state is left untouched)
    mask.copy_(ones)
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_un = 16
    u0.record(stream)
    for it in range(n_un):
        tt.tt_unmask(logits[it % T], mask, None, 4, ids, com, None, 0, uws)
    u1.record(stream)
    torch.cuda.synchronize()
    un_s = u0.elapsed_time(u1) / 1e3 / n_un
    un_gbs = B * S * V * 4 / un_s / 1e9
    log("unmask: %.1f us/call, %.0f GB/s" % (un_s * 1e6, un_gbs))

    # ---- threshold form of the commit rule (gamma = 0.8) on peaked logits:
    # the adaptive-step sampler run to completion, then the call timed alone
    thr = None
    if extras:
        rng = np.random.Generator(np.random.PCG64(lp.seed + 100))
        blk = workloads.make_peaked_block(rng, B, S, V, seed=lp.seed + 100)
        pk = [dev_t(workloads.peaked_logits(rng, blk, s)) for s in range(4)]
        nst = torch.zeros(B, dtype=torch.int32, device=dev)
        mask.copy_(ones)
        sampler_steps = 0
        while sampler_steps < 16 and int(mask.sum().item()) > 0:
            tt.tt_unmask_threshold(pk[sampler_steps % len(pk)], mask, 0.8, ids, com, None, nst,
                                   tt.TT_UNMASK_UPDATE_MASK, uws)
            sampler_steps += 1
        steps_per_seq = nst.cpu().numpy()
        mask.copy_(ones)
        torch.cuda.synchronize()
        u0.record(stream)
        for it in range(n_un):
            tt.tt_unmask_threshold(pk[it % len(pk)], mask, 0.8, ids, com, None, None, 0, uws)
        u1.record(stream)
        torch.cuda.synchronize()
        th_s = u0.elapsed_time(u1) / 1e3 / n_un
        th_gbs = B * S * V * 4 / th_s / 1e9
        thr = {"us_per_call": th_s * 1e6, "GB/s": th_gbs, "frac_hbm": th_gbs / HBM_PEAK_GBS,
               "gamma": 0.8, "sampler_steps_to_resolve_batch": sampler_steps,
               "mean_steps_per_sequence": float(steps_per_seq.mean()),
               "max_steps_per_sequence": int(steps_per_seq.max()),
               "logits": "N(0, 3^2) fp32 [512, 131072] plus one seeded spike per row (peaked)"}
        log("threshold unmask: %.1f us/call, %.0f GB/s; sampler resolved the batch in %d steps "
            "(mean %.2f per sequence)" % (th_s * 1e6, th_gbs, sampler_steps, steps_per_seq.mean()))
    lm = lmhead_bench(np, torch, tt, workloads, dev) if extras else None
    if args.only_attn:
        calibration_copy(torch, dev)   # for scaling FETCH_SIZE / WRITE_SIZE
        log("attention algorithmic bytes per launch: %d" % attn_bytes)
        return

    # ---- CPU oracle on a bounded sample of the same workload: one denoise
    # step's attention (all 6 layers) for as many sequences as fit about 20 s
    # on this host, plus their unmask rows, scaled to the whole batch
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.num_threads()
        order = np.argsort(lens)
        probe = int(order[len(order) // 2])
        c0 = time.perf_counter()
        oracle.block_attn(lp.pools[0], rows=[(probe, t, h) for t in range(S) for h in range(lp.Hq)],
                          q=lp.q[0][0], k_blk=lp.k_blk[0][0], v_blk=lp.v_blk[0][0])
        per_seq_layer = time.perf_counter() - c0
        nseq = int(min(B, max(2, 20.0 / max(per_seq_layer * NL, 1e-3))))
        sample = sorted(int(order[(len(order) - nseq) // 2 + j]) for j in range(nseq))
        rows = [(b, t, h) for b in sample for t in range(S) for h in range(lp.Hq)]
        c0 = time.perf_counter()
        for i in range(NL):
            oracle.block_attn(lp.pools[i], rows=rows, q=lp.q[0][i], k_blk=lp.k_blk[0][i],
                              v_blk=lp.v_blk[0][i])
        c_attn = time.perf_counter() - c0
        c1 = time.perf_counter()
        sub = np.concatenate([lp.logits[0][b * S:(b + 1) * S] for b in sample])
        oracle.unmask(sub, np.ones((len(sample), S), np.uint8), None, 4)
        c_un = time.perf_counter() - c1
        tok_sample = int((lens[sample] + S).sum())
        tok_all = int((lens + S).sum())
        step_s = c_attn * tok_all / tok_sample + c_un * B / len(sample)
        cpu = {"value": 1.0 / step_s, "unit": "denoise-steps/s", "cores": threads, "kind": "oracle",
               "sample": ("fp64 C oracle (OpenMP, %d threads): step-0 attention of %d of %d "
                          "sequences (mean L=%.0f) over all 6 layers (%d query rows) plus their "
                          "unmask rows, %.1f s; scaled to the whole batch by context tokens "
                          "(attention) and rows (unmask)"
                          % (threads, len(sample), B, float(lens[sample].mean()), len(rows) * NL,
                             c_attn + c_un))}
        log("cpu oracle: %.2f s per denoise step (extrapolated from %.1f s)" % (step_s, c_attn + c_un))

    # ---- configs 2-4: block attention alone at the other measured shapes,
    # and the oracle over whole configs
    configs = None
    oracle_t = None
    if extras and not args.no_configs:
        configs = {}
        for k in (2, 3, 4):
            configs["config%d" % k] = attn_config_bench(np, torch, tt, workloads, dev, k,
                                                        copy_bw["GB/s"], graph=not args.no_graph)
        if not args.no_cpu_baseline:
            oracle_t = oracle_timings(np, workloads)

    steps_per_s = T / block_s
    traffic = read_traffic(5)
    res = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "denoise-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": block_s * 1e3,
        "blocks_timed": args.steps,
        "ms_per_denoise_step": block_s / T * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("denoise loop for one 16-token block: B=32, 6 attention layers, "
                                "H_q=32, H_kv=2, D=128, paged bf16 KV (256-token pages), ctx "
                                "U{2048..8192 step 16}, T=4 steps, unmask on fp32 [512, 131072]"),
                   "global_batch": B, "block": S, "layers": NL, "denoise_steps_per_step": T,
                   "vocab": V, "mean_ctx_len": float(lens.mean()), "graph": graph is not None,
                   "parallelism": "none (1 GPU)", "seed": lp.seed},
        "roofline": {"bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": attn_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "frac_copy": attn_gbs / copy_bw["GB/s"] if copy_bw else None,
                     "kernel": "tt_block_attn (split + combine launches)",
                     "us_per_launch": attn_s * 1e6, "us_per_launch_eager": attn_eager_s * 1e6,
                     "alg_bytes_per_launch": attn_bytes,
                     "tflops": attn_tfs, "mfma_frac": attn_tfs / MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "unmask": {"us_per_call": un_s * 1e6, "GB/s": un_gbs, "frac_hbm": un_gbs / HBM_PEAK_GBS},
        "unmask_threshold": thr,
        "chunk_attn": chunk,
        "block_sizes": block_sizes,
        "lmhead_unmask": lm,
        "copy_bandwidth": copy_bw,
        "attn_configs": configs,
        "oracle_timings": oracle_t,
    }
    print(json.dumps(res), flush=True)
    if args.core:
        calibration_copy(torch, dev)   # for scaling FETCH_SIZE / WRITE_SIZE


def config_main(args, np, torch, tt, workloads, dev):
    """--config 2, 3 or 4: that config's block attention alone, one JSON line
    (value = algorithmic GB/s).  With --only-attn (counter runs): the
    launches eagerly, then one 256 MiB calibration copy."""
    if args.only_attn:
        attn_config_bench(np, torch, tt, workloads, dev, args.config, None, graph=False)
        calibration_copy(torch, dev)
        return
    copy_bw = copy_bandwidth(torch, dev)
    log("copy bandwidth: %.0f GB/s" % copy_bw["GB/s"])
    r = attn_config_bench(np, torch, tt, workloads, dev, args.config, copy_bw["GB/s"],
                          graph=not args.no_graph)
    cpu = None
    if not args.no_cpu_baseline:
        ot = oracle_timings(np, workloads, configs=(args.config,),
                            single=(args.config,) if args.config == 2 else ())
        o = ot["config%d" % args.config]
        cpu = {"value": r["alg_bytes_per_launch"] / o["s"] / 1e9, "unit": "GB/s",
               "cores": o["threads"], "kind": "oracle",
               "sample": "the whole config (%d query rows) through oracle.block_attn in %.2f s, "
                         "scaled to the same algorithmic bytes" % (o["rows"], o["s"]),
               "timings": ot}
    res = {
        "metric": "block-attn HBM GB/s (fraction of peak), config %d, 1 GPU" % args.config,
        "value": r["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": r["launches_timed"],
        "warmup": r["launches_timed"], "ms_per_step": r["us_per_launch"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "mean_ctx_len": r["mean_ctx_len"], "seed": r["seed"],
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": r["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["frac_hbm"], "traffic": r["traffic"], "frac_copy": r["frac_copy"],
                     "kernel": "tt_block_attn (split + combine launches)",
                     "us_per_launch": r["us_per_launch"], "alg_bytes_per_launch": r["alg_bytes_per_launch"],
                     "tflops": r["TFLOP/s"], "mfma_frac": r["frac_mfma"]},
        "cpu_baseline": cpu,
        "attn": r,
        "copy_bandwidth": copy_bw,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
