"""Benchmark of the FGP step on one MI355X.

Prints one JSON line.  The metric is ms per FGP step over the whole volume;
the default workload is the 512^3 ellipsoid phantom, 20 outer x 10 inner
steps, lambda = 0.002, run by tv_fgp_run_pp with the three-steps-per-pass
kernel (variant tb3: three consecutive steps in one launch, bit for bit the
same as three one-step launches; 200 steps = 66 launches of three and one of
two).  tv_fgp_run_pp is tv_fgp_run leaving p where the last pass wrote it (the
caller's p or the workspace, reported like the r buffer) instead of copying
it back.
The timed region runs exactly --steps steps (in outer iterations of 10,
momentum restarted at each) on one stream, bracketed by device
synchronisation; inputs are resident in HBM before it starts.  It is run three
times (five up to 256^3 voxels) and `value` is the median (the page reports
medians of repeated solves);
`config.timed` lists the launches one timed region makes and whether p ends in
the workspace.

Besides the headline ms/step it reports:
  roofline      algorithmic bytes per launch (52 B per voxel: read b, r (3),
                p (3); write p (3), r (3); for tb3 that covers three steps)
                over
                the average launch duration, timed with events around every
                launch on the launch stream, against MI355X's 8 TB/s HBM peak;
                `traffic` is the HBM bytes per launch from the rocprofv3
                FETCH_SIZE / WRITE_SIZE record committed under profiles/
                (null when the kernel's sources have changed since those
                counters were taken); `bench.py --traffic` builds that record
                from the two counter runs
  one_step_kernel  the one-step fused kernel (tv_fgp_step's default) timed
                launch by launch on the same data, with its own traffic record
  gap_kernel    time of one duality-gap evaluation of the final p (reads b and
                p: 16 B per voxel) and the gap triple itself
  vs_one_step_roofline  the time a one-step pass needs at the 8 TB/s peak
                (52 B per voxel per step) and its ratio to the measured ms/step
  repeats       the timed region run again, 3 times in all above 256^3 voxels
                and 5 times up to it (ms/step of every run, their median, which
                is `value`, and spread) and T0, the same solve with zero dual
                steps per outer iteration, with (T - T0) / steps
  copy          bandwidth of a plain device copy of 2 x 1 GiB on the same box
  ceiling       tv_fgp_stream_probe: the 7-read / 6-write traffic of one step
                over the same volume size as a linear stream with
                non-temporal stores, the bandwidth a step kernel's bytes can
                reach here; one_step_kernel.pct_of_ceiling and
                roofline.pct_of_ceiling set the kernels against it.  It is
                measured before the warm-up steps, after an untimed lead-in
                of about 0.25 s (lead_in_launches) that also brings the GPU
                from idle to its loaded clocks.  `shapes` holds the part's
                rates for reading 7 volumes, writing 6 and copying one
                (tv_fgp_stream_probe_ex)
  cpu_baseline  the CPU oracle (fp32, OpenMP over z planes) timed on the host
                cores on a bounded sample: the first 10 outer iterations (100
                steps) of the same workload at full size (with --storage half:
                the first outer iteration, 10 steps, of the oracle's half
                mode) on up to 16 threads, plus 5 steps (half: 2) on one
                thread; with the thread count, nproc and the CPU model

--storage half runs the step with p and r stored as binary16 (fp32
arithmetic; 28 B per voxel: read b, r (3), p (3) at 4 + 6 + 6 B, write p (3),
r (3) at 6 + 6 B), by default two steps per pass (tv_fgp_run2_h; --variant
fused for one step per pass); its CPU baseline is the oracle's half mode.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
# algorithmic bytes per voxel per launch, and FGP steps per launch
BYTES_PER_VOXEL = {"fused": 52, "lds_march": 52, "point": 52, "reg_march": 52, "pair": 52,
                   "two_kernel": 72, "tb2": 52, "tb3": 52, "cube": 52, "cube_32x8x2": 52,
                   "cube_64x8x1": 52, "cube_8x8x8": 52, "cube_32x4x4": 52}
STEPS_PER_LAUNCH = {"tb2": 2, "tb3": 3}
BYTES_PER_VOXEL_HALF = 28
METRIC = "ms per FGP step at 512³ fp32; achieved HBM GB/s and % of MI355X peak"

# Kernel measured for each variant's roofline, and the sources it is compiled
# from: a committed traffic record (profiles/traffic_<variant>_512.json) is
# reported only while these sources are unchanged.
KERNELS = {
    "tb3": ("tb3_kernel", ("tv_fgp_device.hpp", "tv_fgp_hwmath.hpp", "tv_fgp_fused_kernel.hpp",
                           "tv_fgp_tb2_kernel.hpp", "tv_fgp_tb3_kernel.hpp", "tv_fgp_tb3.hip")),
    "tb2": ("tb2_kernel", ("tv_fgp_device.hpp", "tv_fgp_hwmath.hpp", "tv_fgp_fused_kernel.hpp",
                           "tv_fgp_tb2_kernel.hpp", "tv_fgp_tb2.hip")),
    "fused": ("fused_zx_kernel", ("tv_fgp_device.hpp", "tv_fgp_hwmath.hpp",
                                  "tv_fgp_fused_kernel.hpp", "tv_fgp_fused.hip")),
}


def traffic_file(variant):
    return os.path.join(ROOT, "profiles", "traffic_%s_512.json" % variant)


def strip_comments(text):
    """C/C++ source without its comments and with whitespace runs collapsed,
    so that an edit of comments or layout leaves the digest unchanged.
    String and character literals are kept as they are."""
    out = []
    i, n = 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest(variant):
    """Digest of the device code a variant's kernel is built from (comments
    and layout excluded)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "stencil_dual_update_amd", "csrc")
    for name in KERNELS[variant][1]:
        with open(os.path.join(csrc, name)) as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()


def measured_traffic(variant, workload):
    """HBM bytes per launch from the committed counter summary, if current."""
    path = traffic_file(variant)
    if variant not in KERNELS or workload != 3 or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(path):
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = rows.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                        "grid": r["Grid_Size"], "value": 0.0})
            d["value"] += float(r["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def probe_copies(rows, value, count):
    """Counter readings of the 1 GiB copy the counters are scaled by: the last
    `count` copies (copyBuffer dispatches, in dispatch order) of the run, which
    are the probe's; torch's copies of p and r come earlier."""
    copies = [r for r in rows if "copyBuffer" in r["name"]]
    return [value(r) for r in copies[-count:]]


def write_traffic(fetch_csv, write_csv, variant):
    """Turn two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then WRITE_SIZE,
    KiB per dispatch) into the per-launch HBM traffic of the variant's kernel.

    Each counter is scaled by what it reads for the bench's copy probe, a
    device copy of exactly 1 GiB read + 1 GiB written.
    """
    import statistics
    kname = KERNELS[variant][0]
    res = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _counter_rows(path)
        # the copy probe makes the run's last 23 copies (3 untimed, 20 timed)
        copy = probe_copies(rows, lambda r: r["value"], 23)
        kern = [r["value"] for r in rows if kname in r["name"]]
        if not copy or not kern:
            raise SystemExit("%s: no copy or %s dispatches found" % (path, kname))
        copy_kib = statistics.median(copy)
        scale = (1 << 20) / copy_kib          # KiB of 1 GiB / counter reading
        res[key] = {"kernel_kib_median": statistics.median(kern),
                    "copy_kib_median": copy_kib, "scale": scale,
                    "dispatches": len(kern)}
    fetch_b = res["fetch"]["kernel_kib_median"] * res["fetch"]["scale"] * 1024
    write_b = res["write"]["kernel_kib_median"] * res["write"]["scale"] * 1024
    vol = 512 ** 3 * 4
    rec = {"kernel": kname, "variant": variant, "workload": "ellipsoids 512^3",
           "steps_per_launch": STEPS_PER_LAUNCH.get(variant, 1),
           "kernel_source_sha256": kernel_source_digest(variant),
           "fetch": res["fetch"], "write": res["write"],
           "hbm_read_bytes_per_launch": round(fetch_b),
           "hbm_write_bytes_per_launch": round(write_b),
           "hbm_bytes_per_launch": round(fetch_b + write_b),
           "volumes_read": round(fetch_b / vol, 3), "volumes_written": round(write_b / vol, 3),
           "algorithmic_bytes_per_launch": BYTES_PER_VOXEL[variant] * 512 ** 3}
    with open(traffic_file(variant), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# The marching tile shapes (x, y, planes) the page sweeps ("TV solver: the FGP
# step on the GPU", section "What made the difference").
MARCH_SWEEP = [(32, 8, 32), (32, 8, 16), (32, 8, 8), (32, 8, 4), (32, 8, 2), (32, 16, 16),
               (32, 16, 8), (32, 4, 32), (64, 4, 16), (64, 8, 8), (64, 4, 8)]


def march_sweep(args, tvf, torch, np, phantoms, dev, dims, lam, n_inner):
    """ms per step of the LDS z-march kernel at each shape of MARCH_SWEEP: the
    same state (after --warmup steps of the one-step kernel) for every shape,
    5 untimed and 20 timed launches each, the median of the launch times."""
    nx, ny, nz = dims
    nvox = nx * ny * nz
    b_host, p0_host, _ = phantoms.make_inputs(args.workload, dims)
    b = torch.from_numpy(b_host).to(dev)
    p = torch.from_numpy(p0_host).to(dev)
    r = p.clone()
    rn = torch.empty_like(r)
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for k in range(args.warmup):
            tvf.tv_fgp_step(b, p, r, rn, lam, tvf.momentum(k % n_inner + 1), stream=stream)
            r, rn = rn, r
        torch.cuda.synchronize()
        p_keep, r_keep = p.clone(), r.clone()
        rows = []
        for tx, ty, planes in MARCH_SWEEP:
            p.copy_(p_keep)
            r.copy_(r_keep)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(25)]
            for q, (e0, e1) in enumerate(evs):
                e0.record(stream)
                tvf.tv_fgp_step_march(b, p, r, rn, lam, tvf.momentum(q % n_inner + 1), tx, ty,
                                      planes, stream=stream)
                e1.record(stream)
                r, rn = rn, r
            torch.cuda.synchronize()
            ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs[5:])
            ms = ts[len(ts) // 2]
            gbs = 52 * nvox / (ms * 1e-3) / 1e9
            rows.append({"shape": "%dx%dx%d" % (tx, ty, planes), "ms_per_step": round(ms, 5),
                         "min_ms": round(ts[0], 5), "max_ms": round(ts[-1], 5),
                         "gbps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            print(json.dumps(rows[-1]), flush=True)
    print(json.dumps({"march_sweep": rows, "dims": [nx, ny, nz], "launches_timed": 20,
                      "device": torch.cuda.get_device_name(dev)}), flush=True)
    return 0


# Cube edge lengths of the size sweep (the ellipsoid recipe at each size).
SIZE_SWEEP = (64, 96, 128, 192, 256, 320, 384, 448, 512, 640, 768)


def size_sweep(args, tvf, torch, phantoms, dev, lam, n_inner):
    """ms per step against volume size.  At each size, after the inputs are
    made on the host: the 7-read / 6-write stream (tv_fgp_stream_probe) for
    an untimed quarter of a second (which also brings the GPU back to its
    loaded clocks), then timed (the median of 20 launches); the three-step
    run (tv_fgp_run_pp, 30 steps after 6 warm-up steps, the median of 3
    runs); the one-step kernel (tv_fgp_step, the median of 20 launches after
    5)."""
    rows = []
    stream = torch.cuda.Stream(device=dev)

    def med(ts):
        ts = sorted(ts)
        return ts[len(ts) // 2]

    def launch_times(fn, count, skip):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(count + skip)]
        for q, (a, z) in enumerate(evs):
            a.record(stream)
            fn(q)
            z.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(z) for a, z in evs[skip:]]

    for n in SIZE_SWEEP:
        dims = (n, n, n)
        nvox = n ** 3
        b_host, p0_host, _ = phantoms.make_inputs(3, dims)
        vols = [torch.empty(nvox, dtype=torch.float32, device=dev).fill_(0.5) for _ in range(13)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            t_lead = time.perf_counter()
            while time.perf_counter() - t_lead < 0.25:
                for _ in range(3):
                    tvf.tv_fgp_stream_probe(vols[:7], vols[7:], stream=stream)
                torch.cuda.synchronize()
            tc = launch_times(lambda q: tvf.tv_fgp_stream_probe(vols[:7], vols[7:], stream=stream),
                              20, 0)
        del vols
        b = torch.from_numpy(b_host).to(dev)
        p = torch.from_numpy(p0_host).to(dev)
        ws = torch.empty_like(p)
        rr = [p.clone(), torch.empty_like(p)]
        pw = [p, ws]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            def run(n_outer, ni):
                r_where, p_where = tvf.tv_fgp_run_pp(b, pw[0], rr[0], rr[1], lam, n_outer, ni,
                                                     variant=tvf.TB3, z_ws=pw[1], stream=stream)
                if p_where:
                    pw.reverse()
                if r_where:
                    rr.reverse()
            run(1, 6)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t3 = []
            for _ in range(3):
                e0.record(stream)
                run(3, n_inner)
                e1.record(stream)
                torch.cuda.synchronize()
                t3.append(e0.elapsed_time(e1) / (3 * n_inner))

            def one(q):
                tvf.tv_fgp_step(b, pw[0], rr[0], rr[1], lam, tvf.momentum(q % n_inner + 1),
                                stream=stream)
                rr.reverse()
            t1 = launch_times(one, 20, 5)
        del b, p, ws, rr, pw
        m3, m1, mc = med(t3), med(t1), med(tc)
        row = {"n": n, "voxels": nvox, "working_set_mb": round(13 * 4 * nvox / 2 ** 20, 1),
               "three_step_ms_per_step": round(m3, 5), "one_step_ms": round(m1, 5),
               "stream_ms": round(mc, 5),
               "three_step_step_gbps": round(52 * nvox / (m3 * 1e-3) / 1e9, 1),
               "one_step_gbps": round(52 * nvox / (m1 * 1e-3) / 1e9, 1),
               "stream_gbps": round(52 * nvox / (mc * 1e-3) / 1e9, 1),
               "one_step_pct_of_stream": round(100 * mc / m1, 1),
               "three_step_speedup": round(m1 / m3, 2)}
        rows.append(row)
        print(json.dumps(row), flush=True)
    print(json.dumps({"size_sweep": rows, "device": torch.cuda.get_device_name(dev)}), flush=True)
    return 0


# Variants of the counter table and the kernels each launches (name prefixes
# as the kernel trace prints them).
TABLE_VARIANTS = [("fused", ["fused_zx_kernel"]), ("pair", ["fused_pair_kernel"]),
                  ("point", ["fused_point_kernel"]), ("reg_march", ["fused_march_kernel"]),
                  ("lds_march", ["lds_march_kernel"]),
                  ("two_kernel", ["primal_kernel", "dual_kernel"]),
                  ("cube", ["cube_kernel"]), ("tb2", ["tb2_kernel"]), ("tb3", ["tb3_kernel"])]


def variant_table_run(args, tvf, torch, phantoms, dev, dims, lam, n_inner):
    """Each variant of TABLE_VARIANTS launched 2 + 5 times on the state after
    --warmup one-step steps (tb2 and tb3 through tv_fgp_step2 / step3), and
    the 1 GiB copy the counters are scaled by.  For rocprofv3 passes."""
    b_host, p0_host, _ = phantoms.make_inputs(args.workload, dims)
    b = torch.from_numpy(b_host).to(dev)
    p = torch.from_numpy(p0_host).to(dev)
    r = p.clone()
    rn = torch.empty_like(r)
    for k in range(args.warmup):
        tvf.tv_fgp_step(b, p, r, rn, lam, tvf.momentum(k % n_inner + 1))
        r, rn = rn, r
    p_keep, r_keep = p.clone(), r.clone()
    p_out = torch.empty_like(p)
    z_ws = torch.empty_like(b)
    m = [tvf.momentum(k) for k in (2, 3, 4)]
    for name, _ in TABLE_VARIANTS:
        p.copy_(p_keep)
        r.copy_(r_keep)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(7):
            if name == "tb2":
                tvf.tv_fgp_step2(b, p, p_out, r, rn, lam, m[0], m[1])
            elif name == "tb3":
                tvf.tv_fgp_step3(b, p, p_out, r, rn, lam, *m)
            else:
                v = tvf.VARIANTS[name]
                tvf.tv_fgp_step(b, p, r, rn, lam, m[0], variant=v,
                                z_ws=z_ws if v == tvf.TWO_KERNEL else None)
        torch.cuda.synchronize()
        print("%s: 7 launches, %.1f ms" % (name, (time.perf_counter() - t0) * 1e3), flush=True)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("variant table run done", flush=True)
    return 0


def _per_dispatch(path):
    """{dispatch id: {"name":..., "grid":..., counter: value}} from a rocprofv3 counter CSV."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = rows.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                        "grid": r["Grid_Size"]})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return rows


def variant_table(root):
    """The per-variant counter table (the page's section "Profiler counters",
    at 512^3) from the rocprofv3 passes over --variant-table-run."""
    import csv
    import statistics

    def find(sub, suffix):
        d = os.path.join(root, sub)
        for f in sorted(os.listdir(d)):
            if f.endswith(suffix):
                return os.path.join(d, f)
        raise SystemExit("no *%s under %s" % (suffix, d))

    trace = list(csv.DictReader(open(find("trace", "kernel_trace.csv"))))
    fetch = _per_dispatch(find("fetch", "counter_collection.csv"))
    write = _per_dispatch(find("write", "counter_collection.csv"))
    tcc = _per_dispatch(find("tcc", "counter_collection.csv"))
    occ = _per_dispatch(find("occ", "counter_collection.csv"))

    def kernel_rows(rows, prefix):
        return [v for k, v in sorted(rows.items()) if _bare(v["name"]) == prefix]

    def scale(rows, counter):
        # the run ends with the three probe copies
        copy = probe_copies([rows[k] for k in sorted(rows)], lambda r: r[counter], 3)
        return (1 << 20) / statistics.median(copy)   # KiB of 1 GiB / reading

    fs, ws = scale(fetch, "FETCH_SIZE"), scale(write, "WRITE_SIZE")
    nvox = 512 ** 3
    vol = nvox * 4
    lines = ["%-11s %-18s %8s %8s %6s %8s %7s %6s %8s %7s %9s %5s %6s %5s" % (
        "variant", "kernel", "us", "alg GB/s", "% 8TB", "HBM MiB", "volumes", "x alg", "HBM GB/s",
        "L2 hit", "occupancy", "VGPR", "LDS KB", "waves")]
    for name, kernels in TABLE_VARIANTS:
        for kn in kernels:
            tr = [t for t in trace if _bare(t["Kernel_Name"]) == kn]
            if not tr:
                continue
            dur = [int(t["End_Timestamp"]) - int(t["Start_Timestamp"]) for t in tr][2:]
            us = statistics.median(dur) / 1e3
            f_kib = statistics.median([v["FETCH_SIZE"] for v in kernel_rows(fetch, kn)][2:])
            w_kib = statistics.median([v["WRITE_SIZE"] for v in kernel_rows(write, kn)][2:])
            hbm = (f_kib * fs + w_kib * ws) * 1024
            t_rows = kernel_rows(tcc, kn)[2:]
            hit = statistics.median([v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"])
                                     for v in t_rows])
            o = statistics.median([v["MeanOccupancyPerActiveCU"] for v in kernel_rows(occ, kn)][2:])
            alg = (20 if kn == "primal_kernel" else 52) * nvox
            t0 = tr[0]
            # the trace's VGPR_Count is half the count the code object declares
            # on this part (e.g. 64 for the three-step kernel's 128)
            vgpr, agpr = 2 * int(t0["VGPR_Count"]), int(t0["Accum_VGPR_Count"])
            lds = int(t0["LDS_Block_Size"])
            wg_waves = (int(t0["Workgroup_Size_X"]) + 63) // 64
            # waves per SIMD the registers and the LDS allow (512 VGPRs of 64
            # lanes per SIMD in granules of 8, 160 KiB of LDS per CU of four
            # SIMDs, at most 8 waves per SIMD)
            regs = ((vgpr + 3) // 4 * 4 + agpr) if agpr else vgpr
            by_vgpr = 512 // ((regs + 7) // 8 * 8)
            by_lds = (160 * 1024 // lds) * wg_waves / 4.0 if lds else 8.0
            theo = min(8.0, by_vgpr, by_lds)
            lines.append("%-11s %-18s %8.1f %8.1f %6.1f %8.0f %7.2f %6.2f %8.1f %6.1f%% %4.2f/%-4.1f %5d %6.1f %5d" % (
                name, kn, us, alg / (us * 1e3), 100 * alg / (us * 1e3) / HBM_PEAK_GBS, hbm / 2 ** 20,
                hbm / vol, hbm / alg, hbm / (us * 1e3), 100 * hit, o, theo, regs, lds / 1024, wg_waves))
    print("\n".join(lines))
    return 0


def _bare(name):
    """Kernel name without 'void ', namespaces and arguments."""
    n = name.replace("void ", "").replace("tvfgp::(anonymous namespace)::", "")
    n = n.replace("tvfgp::", "")
    return n.split("(")[0].split("<")[0] if not n.startswith("at::") else n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--dims", type=int, nargs=3, metavar=("NX", "NY", "NZ"),
                    help="run the workload's recipe at other dimensions")
    ap.add_argument("--variant", default=None, choices=sorted(BYTES_PER_VOXEL),
                    help="kernel variant (default: tb3, three steps per pass; with "
                         "--storage half: tb2, two steps per pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg")
    ap.add_argument("--storage", default="f32", choices=["f32", "half"],
                    help="storage of the dual p and r (half: binary16, fused kernel only)")
    ap.add_argument("--no-copy", action="store_true", help="skip the copy probe")
    ap.add_argument("--size-sweep", action="store_true",
                    help="ms per step of the three-step run, the one-step kernel and the "
                         "13-volume stream at cube sizes 64^3 .. 768^3 (ellipsoid recipe)")
    ap.add_argument("--march-sweep", action="store_true",
                    help="time the LDS z-march kernel at every tile shape of the page's sweep "
                         "(one step per launch) instead of the headline run")
    ap.add_argument("--variant-table-run", action="store_true",
                    help="launch every step kernel a few times on one state (the run the "
                         "counter table is profiled on) instead of the headline run")
    ap.add_argument("--variant-table", metavar="DIR",
                    help="no GPU run: print the per-variant counter table from the rocprofv3 "
                         "passes under DIR (trace/, fetch/, write/, tcc/, occ/) over "
                         "--variant-table-run")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: build the traffic record under profiles/ from "
                         "two rocprofv3 --pmc counter_collection.csv files of this bench")
    return ap.parse_args()


def main():
    args = parse()
    if args.variant is None:
        # fp32: three steps per pass; binary16: two (its pass is bound by
        # arithmetic, which a third level of halo would add to)
        args.variant = "tb2" if args.storage == "half" else "tb3"
    if args.traffic:
        write_traffic(*args.traffic, args.variant)
        return 0
    if args.variant_table:
        return variant_table(args.variant_table)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the step would shard by z-slabs with a one-plane halo; not built). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import phantoms
    import stencil_dual_update_amd as tvf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = phantoms.workload(args.workload)
    nx, ny, nz = args.dims or w["dims"]
    lam = w["lam"]
    n_inner = w["n_inner"]
    variant = tvf.VARIANTS[args.variant]
    half = args.storage == "half"
    if half and args.variant not in ("fused", "tb2"):
        print("--storage half runs the one-step (fused) or two-steps-per-pass (tb2) kernels",
              file=sys.stderr)
        return 2
    nvox = nx * ny * nz

    if args.march_sweep:
        return march_sweep(args, tvf, torch, np, phantoms, dev, (nx, ny, nz), lam, n_inner)
    if args.size_sweep:
        return size_sweep(args, tvf, torch, phantoms, dev, lam, n_inner)
    if args.variant_table_run:
        return variant_table_run(args, tvf, torch, phantoms, dev, (nx, ny, nz), lam, n_inner)

    t0 = time.time()
    b_host, p0_host, _ = phantoms.make_inputs(args.workload, (nx, ny, nz))
    gen_s = time.time() - t0
    b = torch.from_numpy(b_host).to(dev)
    p = torch.from_numpy(p0_host).to(dev)
    if half:
        p = p.to(torch.float16)  # round to nearest even, as the oracle's half mode
    ra = p.clone()
    rb = torch.empty_like(ra)
    ws = (torch.empty_like(b) if variant == tvf.TWO_KERNEL else
          torch.empty_like(p) if variant in (tvf.TB2, tvf.TB3) else None)
    spl = STEPS_PER_LAUNCH.get(args.variant, 1)
    # timed regions: the median of 5 up to 256^3 voxels, of 3 above (the
    # page's protocol: medians of repeated solves)
    n_runs = 5 if nvox <= 256 ** 3 else 3
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    # the dual p and, for the multi-step variants, the workspace it alternates
    # with: tv_fgp_run_pp leaves p where its last pass put it and says where
    # (as it does for r), so pw[0] is always the current p
    pw = [p, ws]

    def run(r_cur, r_nxt, n_outer, ni):
        if half and spl == 2:
            return tvf.tv_fgp_run2_h(b, p, ws, r_cur, r_nxt, lam, n_outer, ni, stream=stream)
        if half:
            return tvf.tv_fgp_run_h(b, p, r_cur, r_nxt, lam, n_outer, ni, stream=stream)
        r_where, p_where = tvf.tv_fgp_run_pp(b, pw[0], r_cur, r_nxt, lam, n_outer, ni,
                                             variant=variant, z_ws=pw[1], stream=stream)
        if p_where:
            pw.reverse()
        return r_where

    def step(r_cur, r_nxt, m):
        if half:
            tvf.tv_fgp_step_h(b, p, r_cur, r_nxt, lam, m, stream=stream)
        else:
            tvf.tv_fgp_step(b, p, r_cur, r_nxt, lam, m, variant=variant, z_ws=ws,
                            stream=stream)

    def passes_of(k):
        """Launches tv_fgp_run makes for k steps in outer iterations of n_inner
        (passes of three and two steps, single steps) and whether p ends in
        the workspace (tv_fgp_run would copy it back; tv_fgp_run_pp, which the
        fp32 runs use, leaves it there)."""
        full, rest = divmod(k, n_inner)
        counts = {3: 0, 2: 0, 1: 0}
        copies = 0
        for n_outer, ni in ((full, n_inner), (1 if rest else 0, rest)):
            left = n_outer * ni
            flips = 0
            while left > 0:
                if spl >= 3 and (left >= 5 or left == 3):
                    todo = 3
                elif spl >= 2:
                    todo = 2 if left >= 2 else 1
                else:
                    todo = 1
                counts[todo] += 1
                flips += todo > 1
                left -= todo
            copies += flips % 2
        return counts, copies

    def run_steps(k, r_cur, r_nxt):
        """k steps in outer iterations of n_inner; returns (r_cur, r_nxt) after."""
        full, rest = divmod(k, n_inner)
        for n_outer, ni in ((full, n_inner), (1 if rest else 0, rest)):
            if n_outer * ni == 0:
                continue
            if run(r_cur, r_nxt, n_outer, ni):
                r_cur, r_nxt = r_nxt, r_cur
        return r_cur, r_nxt

    # The stream ceiling (tv_fgp_stream_probe: the 7-read / 6-write bytes of
    # one step as a linear stream over 13 scratch volumes) is measured first.
    # Its untimed lead-in streams for about a quarter of a second, which also
    # brings the GPU from idle to its loaded clocks before the warm-up steps;
    # without it the first timed region of a short run starts on a GPU that
    # is still ramping up.
    ceil_ms, ceil_lead, ceil_shapes = None, 0, {}
    if not args.no_copy and not half:
        vols = [torch.empty(nvox, dtype=torch.float32, device=dev).fill_(0.5)
                for _ in range(13)]
        torch.cuda.synchronize()  # the fills ran on the default stream
        with torch.cuda.stream(stream):
            t_lead = time.perf_counter()
            while ceil_lead < 3 or (time.perf_counter() - t_lead < 0.25 and ceil_lead < 2000):
                for _ in range(3):
                    tvf.tv_fgp_stream_probe(vols[:7], vols[7:], stream=stream)
                ceil_lead += 3
                torch.cuda.synchronize()
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            reps = 20
            for _ in range(reps):
                tvf.tv_fgp_stream_probe(vols[:7], vols[7:], stream=stream)
            c1.record(stream)
            torch.cuda.synchronize()
            ceil_ms = c0.elapsed_time(c1) / reps
            # the part's rates for the read half, the write half and a copy
            for name, ns, nd in (("read7", 7, 0), ("write6", 0, 6), ("copy1", 1, 1)):
                srcs, dsts = vols[:ns], vols[7:7 + nd]
                for _ in range(3):
                    tvf.tv_fgp_stream_probe_ex(srcs, dsts, stream=stream)
                c0.record(stream)
                for _ in range(reps):
                    tvf.tv_fgp_stream_probe_ex(srcs, dsts, stream=stream)
                c1.record(stream)
                torch.cuda.synchronize()
                ms = c0.elapsed_time(c1) / reps
                gbs = 4 * (ns + nd) * nvox / (ms * 1e-3) / 1e9
                ceil_shapes[name] = {"ms": round(ms, 5), "gbps": round(gbs, 1),
                                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del vols

    with torch.cuda.stream(stream):
        r_cur, r_nxt = run_steps(args.warmup, ra, rb)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        start.record(stream)
        r_cur, r_nxt = run_steps(args.steps, r_cur, r_nxt)
        stop.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t_wall) * 1e3
        region_ms = start.elapsed_time(stop)

        # the same timed region twice more (spread across runs), and the solve
        # with zero dual steps per outer iteration (T0: per step = (T - T0) / steps)
        repeat_ms = []
        for _ in range(n_runs - 1):
            start.record(stream)
            r_cur, r_nxt = run_steps(args.steps, r_cur, r_nxt)
            stop.record(stream)
            torch.cuda.synchronize()
            repeat_ms.append(start.elapsed_time(stop))
        start.record(stream)
        run(r_cur, r_nxt, max(1, args.steps // n_inner), 0)
        stop.record(stream)
        torch.cuda.synchronize()
        t0_ms = start.elapsed_time(stop)

        # per-launch durations: an event pair around every launch (a launch of
        # the two- or three-steps-per-pass kernel runs steps k, k+1 (, k+2),
        # p_in -> p_out)
        n_launch = max(1, args.steps // spl)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_launch)]
        if not half:
            p, ws = pw
        p_cur, p_alt = p, ws
        for q in range(n_launch):
            k = q * spl
            evs[q][0].record(stream)
            if spl == 3:
                tvf.tv_fgp_step3(b, p_cur, p_alt, r_cur, r_nxt, lam,
                                 *(tvf.momentum((k + i) % n_inner + 1) for i in range(3)),
                                 stream=stream)
                p_cur, p_alt = p_alt, p_cur
            elif spl == 2:
                step2 = tvf.tv_fgp_step2_h if half else tvf.tv_fgp_step2
                step2(b, p_cur, p_alt, r_cur, r_nxt, lam, tvf.momentum(k % n_inner + 1),
                      tvf.momentum((k + 1) % n_inner + 1), stream=stream)
                p_cur, p_alt = p_alt, p_cur
            else:
                step(r_cur, r_nxt, tvf.momentum(k % n_inner + 1))
            evs[q][1].record(stream)
            r_cur, r_nxt = r_nxt, r_cur
        torch.cuda.synchronize()
        p = p_cur
        launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]

    # the reported figure is the median of the timed regions (the page
    # reports medians of repeated solves)
    runs = sorted([region_ms] + repeat_ms)
    mid = runs[len(runs) // 2]
    ms_per_step = mid / args.steps
    repeats = {"ms_per_step": [round(v / args.steps, 5) for v in [region_ms] + repeat_ms],
               "median_ms_per_step": round(ms_per_step, 5),
               "spread_pct": round(100.0 * (runs[-1] - runs[0]) / mid, 2),
               "t0_ms": round(t0_ms, 4),
               "t_minus_t0_ms_per_step": round((mid - t0_ms) / args.steps, 5)}
    step_bytes = (BYTES_PER_VOXEL_HALF if half else BYTES_PER_VOXEL[args.variant]) * nvox
    launch_avg_ms = float(np.mean(launch_ms))
    achieved = step_bytes / (launch_avg_ms * 1e-3) / 1e9
    region_gbs = step_bytes / spl / (ms_per_step * 1e-3) / 1e9

    # the one-step kernel (tv_fgp_step's default) timed alongside, launch by launch
    one_step = None
    if spl > 1:
        with torch.cuda.stream(stream):
            n1 = 50
            ev1 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n1 + 5)]
            for q in range(n1 + 5):
                ev1[q][0].record(stream)
                m = tvf.momentum(q % n_inner + 1)
                if half:
                    tvf.tv_fgp_step_h(b, p, r_cur, r_nxt, lam, m, stream=stream)
                else:
                    tvf.tv_fgp_step(b, p, r_cur, r_nxt, lam, m, stream=stream)
                ev1[q][1].record(stream)
                r_cur, r_nxt = r_nxt, r_cur
            torch.cuda.synchronize()
        ms1 = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev1[5:]]))
        bpv1 = BYTES_PER_VOXEL_HALF if half else 52
        gbs1 = bpv1 * nvox / (ms1 * 1e-3) / 1e9
        one_step = {"kernel": "fused_pair_kernel (binary16)" if half else "fused_zx_kernel",
                    "ms_per_step": round(ms1, 5), "achieved_gbps": round(gbs1, 1),
                    "frac": round(gbs1 / HBM_PEAK_GBS, 4),
                    "traffic": None if (args.dims or half) else
                    measured_traffic("fused", args.workload),
                    "launches": n1}

    # duality-gap reduction (reads b and p: 16 B per voxel), of the fp32 dual
    if half:
        p = p.float()
    gap_ws = torch.empty(tvf.gap_workspace_bytes(nx, ny, nz) // 8, dtype=torch.float64,
                         device=dev)
    gap_out = torch.empty(3, dtype=torch.float64, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            tvf.tv_fgp_duality_gap(b, p, lam, gap_out, gap_ws, stream=stream)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        gap_reps = 20
        for _ in range(gap_reps):
            tvf.tv_fgp_duality_gap(b, p, lam, gap_out, gap_ws, stream=stream)
        g1.record(stream)
        torch.cuda.synchronize()
    gap_ms = g0.elapsed_time(g1) / gap_reps
    gap_vals = gap_out.cpu().tolist()
    # the two-voxels-per-lane first pass takes even nx (torch allocations are
    # aligned); odd nx takes the one-voxel pass
    gap = {"first_pass": "gap_partial_pair_kernel" if nx % 2 == 0 else "gap_partial_kernel",
           "ms": round(gap_ms, 5), "algorithmic_bytes": 16 * nvox,
           "gbps": round(16 * nvox / (gap_ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(16 * nvox / (gap_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "gap": gap_vals[0], "tv": gap_vals[1], "fidelity": gap_vals[2]}
    del gap_ws, gap_out

    copy = None
    if not args.no_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            reps = 20
            for _ in range(reps):
                dst.copy_(src)
            c1.record(stream)
            torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1) / reps
        copy = {"bytes": 2 * src.numel() * 4, "ms": round(copy_ms, 4),
                "gbps": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1)}
        del src, dst

    # the same 7-read / 6-write traffic as one step, as a plain linear stream
    # with non-temporal stores: what the part achieves for a step's bytes
    ceiling = None
    pct_ceiling = None
    if ceil_ms is not None:
        ceil_gbs = 52 * nvox / (ceil_ms * 1e-3) / 1e9
        ceiling = {"kernel": "stream13_kernel", "bytes": 52 * nvox, "ms": round(ceil_ms, 5),
                   "gbps": round(ceil_gbs, 1), "frac_of_hbm_peak": round(ceil_gbs / HBM_PEAK_GBS, 4),
                   "lead_in_launches": ceil_lead, "shapes": ceil_shapes}
        if one_step is not None:
            one_step["pct_of_ceiling"] = round(100.0 * ceil_ms / one_step["ms_per_step"], 1)
        if args.variant in ("fused", "tb2", "tb3"):
            # compulsory bytes of a launch (52 B per voxel) at the ceiling's rate
            # against the launch's time
            pct_ceiling = round(100.0 * ceil_ms / launch_avg_ms, 1)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nproc = os.cpu_count() or 1
        try:
            usable = len(os.sched_getaffinity(0))
        except AttributeError:
            usable = nproc
        # the GPU machine's CPU share is 16 threads whatever the machine shows
        threads = min(16, usable)
        p0 = p0_host
        if half:
            p0 = oracle.f32_to_f16_bits(p0)

        def oracle_sample(n_outer, ni):
            t1 = time.perf_counter()
            if half:
                oracle.run_half(b_host, p0, p0, lam, n_outer, ni)
            else:
                oracle.run(b_host, p0, p0, lam, n_outer, ni)
            return time.perf_counter() - t1

        cpu_outer = 1 if half else 10  # the half mode converts p, r every step: slower
        oracle.set_threads(threads)
        cpu_s = oracle_sample(cpu_outer, n_inner)
        used = oracle.get_threads()
        cpu_steps = cpu_outer * n_inner
        one_steps = 2 if half else 5
        oracle.set_threads(1)
        one_s = oracle_sample(1, one_steps)
        oracle.set_threads(threads)
        cpu = {"value": round(cpu_s * 1e3 / cpu_steps, 3), "unit": "ms/step",
               "cores": used, "kind": "oracle",
               "sample": "first %d outer iterations (%d steps) of the same workload at "
                         "full size, fp32 exact-order oracle%s, OpenMP over z planes, "
                         "%d threads, %.1f s" % (
                             cpu_outer, cpu_steps, " (binary16 dual)" if half else "",
                             used, cpu_s),
               "threads": used, "nproc": nproc, "usable_cpus": usable,
               "cpu_model": cpu_model(),
               "one_thread": {"value": round(one_s * 1e3 / one_steps, 3), "unit": "ms/step",
                              "sample": "first %d steps of the same workload at full size, "
                                        "1 thread, %.1f s" % (one_steps, one_s)}}

    traffic = None if (args.dims or half) else measured_traffic(args.variant, args.workload)
    base = phantoms.BASE_NAMES[args.workload]
    if args.dims:
        base = "%s recipe at %dx%dx%d" % (base, nx, ny, nz)
    counts, copies = passes_of(args.steps)
    full, rest = divmod(args.steps, n_inner)
    workload_label = "%s, lambda %g: %d steps timed (%s), median of %d timed runs" % (
        base, lam, args.steps,
        " + ".join(x for x in ("%d outer x %d inner" % (full, n_inner) if full else "",
                               "1 outer x %d inner" % rest if rest else "") if x),
        n_runs)
    timed = {"steps": args.steps,
             "launches": {"three_step": counts[3], "two_step": counts[2],
                          "one_step": counts[1]},
             "p_ends_in_workspace": copies > 0,
             "p_copy_back": copies > 0 and half,
             "runs": n_runs}
    # the headline metric's wording, with the volume actually run
    metric = METRIC if not half else METRIC.replace("fp32", "fp32 with binary16 p, r")
    if (nx, ny, nz) != (512, 512, 512):
        metric = metric.replace("512³", "%d³" % nx if nx == ny == nz else "%d×%d×%d" % (nx, ny, nz))
    out = {
        "metric": metric,
        "value": round(ms_per_step, 5),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload_label, "timed": timed,
                   "dims": [nx, ny, nz], "lambda": lam, "steps_per_outer": n_inner,
                   "variant": args.variant, "dual_storage": "binary16" if half else "f32",
                   "parallelism": "single GPU"},
        "gbps": round(region_gbs, 1),
        "pct_hbm_peak": round(100.0 * region_gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": step_bytes,
                     "steps_per_launch": spl,
                     "launch_ms_avg": round(launch_avg_ms, 5),
                     "launch_ms_min": round(float(np.min(launch_ms)), 5),
                     "launch_ms_max": round(float(np.max(launch_ms)), 5),
                     "pct_of_ceiling": pct_ceiling},
        "one_step_kernel": one_step,
        "repeats": repeats,
        # a pass that does one step moves 52 B per voxel per step: its time at
        # the 8 TB/s peak is the one-step roofline, which several steps per
        # pass can beat
        "vs_one_step_roofline": ({
            "one_step_ms_at_peak": round(52 * nvox / (HBM_PEAK_GBS * 1e9) * 1e3, 5),
            "ratio": round(52 * nvox / (HBM_PEAK_GBS * 1e9) * 1e3 / ms_per_step, 3)}
            if not half else None),
        "gap_kernel": gap,
        "copy": copy,
        "pct_of_copy": (round(100.0 * region_gbs / copy["gbps"], 1) if copy else None),
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "wall_ms_timed_region": round(wall_ms, 2),
        "input_gen_s": round(gen_s, 2),
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
