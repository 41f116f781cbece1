#!/usr/bin/env python3
"""Decode-step throughput of the PackKV packed cache on one MI355X.

One step is one decode-attention pass over the packed cache of every stream:
append one new token per stream (open-tail re-encode: quantise, reorder,
pack), then the K decompress-GEMV, softmax and the V decompress-GEMV, run as
one fused launch.  The same steps are timed again with the three kernels
launched separately (scores and weights through HBM), and on paged copies
of the cache (one page pool behind per-stream block tables), once with every
stream at the workload's length and once with lengths spread from T to T/4.
The caches are prefilled (bulk compress) before the timed region, so every
input is resident in HBM when timing starts.

value = compressed bytes the step reads (K and V records plus their offset
tables) / time per step, in GB/s (1e9 B/s).  Each step is timed with HIP
events on the launch stream; before every step a 512 MiB write evicts the
device's 256 MB memory-side cache (MALL), outside the step's events, so no
step reads records a previous one left cached.  The per-kernel split (event
medians and means), each GEMV's effective bandwidth, the roofline of the
dominant kernel (bytes per launch over its mean HIP-event duration), the
compression ratios (ideal, physical, full, and plain b-bit quantisation) and
the oracle's CPU throughput are reported beside.

The default workload is append-64k, the largest: 256 streams of 65536
tokens at 3 bits, one appended token per stream and step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kvsynth  # noqa: E402

METRIC = "fused decompress-GEMV effective GB/s & % of HBM peak; K/V compression ratio"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_gemv_amd", "csrc", f)
                  for f in ("gemv.hip", "common.hpp", "kernels.hpp", "api.hip")]   # kernels and their launch shapes


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def generate(w: kvsynth.Workload, torch, dev):
    """Upload seeded K, V [S][T][D] fp16 stream by stream."""
    S, T, D = w.streams, w.tokens, w.head_dim
    K = torch.empty((S, T, D), dtype=torch.float16, device=dev)
    V = torch.empty_like(K)
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        for s, (k, v) in enumerate(ex.map(lambda i: kvsynth.stream_kv(w, i), range(S))):
            K[s].copy_(torch.from_numpy(k))
            V[s].copy_(torch.from_numpy(v))
    return K, V


def cpu_baseline(w: kvsynth.Workload, n_streams: int, budget_s: float, permute: int = 1,
                 payload_order: int = 0) -> dict:
    """The fp64 oracle's decode steps on a sample of streams, single-threaded,
    for about budget_s seconds (whole steps over the sample, at least one)."""
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import stream as ostream, attention
    cfg = oracle.Config(bits=w.bits, block=w.block, permute=permute, payload_order=payload_order)
    with threadpool_limits(limits=1):
        caches = []
        for s in range(n_streams):
            k, v = kvsynth.stream_kv(w, s)
            caches.append(ostream.compress(k, v, cfg))          # prefill: not timed
        nbytes = 0
        n_steps = 0
        dt = 0.0
        while n_steps == 0 or dt < budget_s:
            inputs = [(kvsynth.stream_q(w, s, step=n_steps), kvsynth.append_kv(w, s, n_steps))
                      for s in range(n_streams)]
            t0 = time.perf_counter()
            for s in range(n_streams):
                q, kv_new = inputs[s]
                caches[s] = c = ostream.append(caches[s], *kv_new)   # tail re-encode
                kh, vh, _, _ = ostream.decode_stream(c)                # unpack + fp64 dequant
                p = attention.softmax(attention.qk(q, kh), w.head_dim)
                attention.pv(p, vh)
                nbytes += len(c.arena("K")) + len(c.arena("V")) + 2 * 4 * (len(c.blocks) + 1)
            dt += time.perf_counter() - t0
            n_steps += 1
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle", "host": host_cpu(),
            "sample": f"{n_streams} of {w.streams} streams at {w.tokens}+ tokens, {n_steps} decode steps each "
                      f"(tail re-encode, unpack, fp64 dequantise, K GEMV, softmax, V GEMV), {dt:.1f} s of "
                      f"single-threaded CPU time; value = compressed bytes (records + offsets) decoded per second"}


def compression_ratios(st: dict, S: int, T: int, D: int, bits: int, nb: int) -> dict:
    """Compression ratios of the cache after prefill, from the library's
    width statistics: fp16 bytes over compressed bytes, counted three ways
    (ideal: payload bits + header bits + fp16 parameters; physical: the stored
    records, padding included; full: physical plus the one-byte-per-token
    permutation), next to plain b-bit quantisation with the same parameters
    (T*D*b bits + parameters), and PackKV's gain over it (CR / CR_plain - 1)."""
    raw = 16 * S * T * D
    hb = 1 if bits <= 4 else 2
    res = {}
    for side, params in (("k", 32 * D * nb * S), ("v", 32 * T * S)):
        ideal = 32 * st[f"{side}_words"] + 8 * hb * st[f"{side}_runs"] + params
        phys = 8 * st[f"{side}_bytes"]
        full = phys + 8 * S * T
        plain = S * T * D * bits + params
        res[side] = {"ideal": round(raw / ideal, 4), "physical": round(raw / phys, 4), "full": round(raw / full, 4),
                     "plain_quant": round(raw / plain, 4),
                     "pct_vs_plain_quant": {k: round(100 * (raw / b_ / (raw / plain) - 1), 2)
                                            for k, b_ in (("ideal", ideal), ("physical", phys), ("full", full))}}
    res["note"] = ("fp16 bytes / compressed bytes at the prefill length; pct_vs_plain_quant = CR / CR of plain "
                   "b-bit quantisation - 1 (the pages' 'higher memory reduction' is stated against "
                   "quantisation baselines); negative on data without token structure, where the run "
                   "headers cost more than the narrower runs save")
    return res


def host_cpu() -> dict:
    """The host the oracle runs on: CPU model, logical CPUs, CPUs this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = None
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "cpus_usable": usable}


def gpu_info(torch) -> dict:
    """The device and software measured on: name, architecture, compute
    units, HIP version, and the engine and memory clocks rocm-smi reports at
    the call (None where a field cannot be read)."""
    import re
    import subprocess
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "hip": torch.version.hip, "sclk_mhz": None, "mclk_mhz": None}
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                             timeout=20).stdout
        for card in json.loads(out).values():
            for k, v in card.items():
                m = re.search(r"(\d+)\s*Mhz", str(v), re.I)
                if m and "sclk" in k.lower() and info["sclk_mhz"] is None:
                    info["sclk_mhz"] = int(m.group(1))
                if m and "mclk" in k.lower() and info["mclk_mhz"] is None:
                    info["mclk_mhz"] = int(m.group(1))
            break
    except Exception:
        pass
    return info


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    e = t.get(workload)
    if not e or e.get("kernel_source") != kernel_source_hash():
        return None
    return e


def summarize_profile(pdir: str, workload: str) -> None:
    """Write profiles/<kernels>_<workload>.md and the workload's entry of
    profiles/traffic.json from a profile directory holding a kernel-trace run
    (kt/, whose stdout kt.log ends with this script's JSON line) and counter
    passes p*/ (rocprofv3 --pmc, CSV output), among them one FETCH_SIZE and
    one WRITE_SIZE pass over a run that ends with the 1 GiB device copy.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read
    for that copy of known size (bytes moved / counter bytes), so `traffic`
    is in the same bytes as the algorithmic figure."""
    import csv
    import glob
    import re

    def short(name):
        name = name.replace("void ", "").replace("packkv::", "")
        return re.sub(r"\(.*", "", name)

    stats = {}
    with open(os.path.join(pdir, "kt", "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            stats[short(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                                       float(r["MaxNs"]) / 1e3)
    # median duration per kernel from the per-dispatch trace: unlike the mean
    # it is not pulled up by the launches made while the clock still ramps
    durs = {}
    trace = os.path.join(pdir, "kt", "run_kernel_trace.csv")
    if os.path.exists(trace):
        for r in csv.DictReader(open(trace)):
            durs.setdefault(short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    med = {k: float(np.median(v)) for k, v in durs.items()}
    # the launches in the order they ran, for the timed-loop figures below
    seq = []
    if os.path.exists(trace):
        rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"]))
        seq = [(short(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
               for r in rows]
    bench_line = None
    for line in open(os.path.join(pdir, "kt.log")):
        if line.startswith("{") and '"metric"' in line:
            bench_line = json.loads(line)
    counters, copy = {}, {}
    for f in sorted(glob.glob(os.path.join(pdir, "p*", "run_counter_collection.csv"))):
        per = {}
        for r in csv.DictReader(open(f)):
            key = (int(r["Dispatch_Id"]), short(r["Kernel_Name"]), r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        acc = {}
        for (d, k, c), v in per.items():
            if "copyBuffer" in k:                       # the largest copy is the 1 GiB probe
                copy[c] = max(copy.get(c, 0.0), v)
                continue
            acc.setdefault((k, c), []).append(v)
        for (k, c), vs in acc.items():
            counters.setdefault(k, {})[c] = sum(vs) / len(vs)
    probe = 1 << 30
    f_fetch = probe / (copy["FETCH_SIZE"] * 1024) if copy.get("FETCH_SIZE") else None
    f_write = probe / (copy["WRITE_SIZE"] * 1024) if copy.get("WRITE_SIZE") else None

    def traffic(k):
        c = counters.get(k, {})
        if f_fetch is None or f_write is None or "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            return None
        return int(c["FETCH_SIZE"] * 1024 * f_fetch + c["WRITE_SIZE"] * 1024 * f_write)

    gemvs = {"attn": next((k for k in stats if k.startswith("k_attn_decode") and "true" not in k), None),
             "qk": next((k for k in stats if k.startswith("k_qk_gemv")), None),
             "pv": next((k for k in stats if k.startswith("k_pv_gemv")), None)}
    if not bench_line:
        raise SystemExit(f"{pdir}/kt.log holds no bench line")
    # the hash of the sources the profiled run was built from, not of today's
    entry = {"kernel_source": bench_line["kernel_source"], "fetch_factor": f_fetch, "write_factor": f_write}
    for tag, k in gemvs.items():
        if k and traffic(k) is not None:
            entry[tag] = traffic(k)
    tf = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    tf[workload] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(tf, f, indent=1, sort_keys=True)

    alg = {gemvs[t]: b for t, b in bench_line["alg_bytes_per_launch"].items() if gemvs.get(t)}
    lines = [f"# Kernel trace and counters: {workload}", "",
             "Commands (repository root, one rocprofv3 process each):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt -o run -- "
             f"python bench.py --workload {workload} --steps 20 --warmup 5 --no-cpu-baseline > <dir>/kt.log",
             f"rocprofv3 --pmc <counters> --output-format csv -d <dir>/p<i> -o run -- "
             f"python bench.py --workload {workload} --steps 3 --warmup 1 --no-cpu-baseline --no-paged",
             f"python bench.py --summarize <dir> --workload {workload}", "```", "",
             "Counter passes: (1) SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM_RD "
             "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_LDS; (2) SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
             "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_SCA SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT "
             "SQ_ACTIVE_INST_ANY; (3) FETCH_SIZE; (4) WRITE_SIZE; (5) GRBM_GUI_ACTIVE SQ_INSTS_VALU_CVT "
             "SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_INT32.", "",
             f"Kernel source hash: `{entry['kernel_source']}`", "",
             "## Kernel durations (rocprofv3 --stats)", "",
             "| kernel | calls | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for k, (n, avg, mn, mx) in sorted(stats.items(), key=lambda x: -x[1][0] * x[1][1]):
        m = f"{med[k]:.1f}" if k in med else "-"
        lines.append(f"| {k} | {n} | {avg:.1f} | {m} | {mn:.1f} | {mx:.1f} |")
    # The launches the bench line's HIP events time: in the fused loop each
    # attention launch follows a cache flush and the append; the GEMVs run
    # in the separate loop only.  Warm-up steps first, then the timed ones.
    warm, steps = int(bench_line.get("warmup", 0)), int(bench_line.get("steps", 0))
    timed = {}
    if seq and gemvs["attn"]:
        timed["attn"] = [d for i, (n, d) in enumerate(seq) if n == gemvs["attn"] and i >= 2
                         and seq[i - 1][0].startswith("k_encode")
                         and "FillFunctor<unsigned char>" in seq[i - 2][0]][warm:warm + steps]
    for tag in ("qk", "pv"):
        if seq and gemvs[tag]:
            timed[tag] = [d for n, d in seq if n == gemvs[tag]][warm:warm + steps]
    if any(timed.values()):
        ev = bench_line.get("kernels_ms_mean", {})
        evk = {"attn": "attention", "qk": "qk_gemv", "pv": "pv_gemv"}
        lines += ["", "## Launches of the timed loops", "",
                  "The same launches as the bench line's HIP events (its `kernels_ms_mean`); the table "
                  "above also counts the clock warm-up and the paged loops.", "",
                  "| kernel | launches | mean us | median us | HIP events, mean us |", "|---|---|---|---|---|"]
        for tag, v in timed.items():
            if v:
                e = ev.get(evk[tag])
                lines.append(f"| {gemvs[tag]} | {len(v)} | {np.mean(v):.1f} | {np.median(v):.1f} | "
                             f"{e * 1e3:.1f} |" if e is not None else
                             f"| {gemvs[tag]} | {len(v)} | {np.mean(v):.1f} | {np.median(v):.1f} | - |")
    lines += ["", "## HBM traffic per launch", "",
              f"1 GiB device copy: FETCH_SIZE {copy.get('FETCH_SIZE', 0):.0f} KiB, WRITE_SIZE "
              f"{copy.get('WRITE_SIZE', 0):.0f} KiB, so fetch factor {f_fetch and round(f_fetch, 4)}, "
              f"write factor {f_write and round(f_write, 4)}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic bytes | algorithmic bytes | traffic / alg |",
              "|---|---|---|---|---|---|"]
    for tag, k in gemvs.items():
        if not k or k not in counters:
            continue
        c = counters[k]
        t = traffic(k)
        a = alg.get(k)
        ratio = f"{t / a:.3f}" if (t and a) else "-"
        lines.append(f"| {k} | {c.get('FETCH_SIZE', 0):.0f} | {c.get('WRITE_SIZE', 0):.0f} | {t} | {a or '-'} | {ratio} |")
    lines += ["", "## Other counters (average per dispatch)", ""]
    for k in [gemvs["attn"], gemvs["qk"], gemvs["pv"]] + [x for x in counters if x.startswith(("k_softmax", "k_encode"))]:
        if k and k in counters:
            c = counters[k]
            lines.append(f"- **{k}**: " + ", ".join(f"{n} {v:.4g}" for n, v in sorted(c.items())))
    if bench_line:
        lines += ["", "## Bench line of the traced run", "", "```", json.dumps(bench_line), "```"]
    name = f"decode_step_{workload}.md"
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote profiles/{name} and the {workload} entry of profiles/traffic.json")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="append-64k", choices=sorted(kvsynth.WORKLOADS))
    ap.add_argument("--cpu-streams", type=int, default=4, help="streams in the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="timed oracle work (whole decode steps over the sampled streams)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="bytes written before every timed step to evict the memory-side cache (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache measurement")
    ap.add_argument("--page-kib", type=int, default=64, help="page size of the paged cache")
    ap.add_argument("--layers", type=int, default=1,
                    help="also time decode attention over this many caches of the workload's shape "
                         "(a model's layers): one multi-cache launch against one launch per cache")
    ap.add_argument("--permute", type=int, default=1, choices=(0, 1, 2),
                    help="token order inside blocks: 0 identity, 1 greedy grouping, 2 sort key")
    ap.add_argument("--payload-order", type=int, default=0, choices=(0, 1),
                    help="K payload order: 0 by channel, 1 each run row by decreasing width (b <= 4)")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of a plain device copy run after timing (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write the profiles/ summary and traffic entry from a rocprofv3 profile directory")
    args = ap.parse_args()
    if args.summarize:
        summarize_profile(args.summarize, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the packed cache is per stream and this build runs on a "
              "single MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_gemv_amd import PackedKVCache, attention_multi, attention_multi_workspace, softmax_rows

    w = kvsynth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    S, G, T0, D = w.streams, w.group, w.tokens, w.head_dim
    n_steps = args.warmup + args.steps
    T_max = T0 + 2 * n_steps                 # room for the fused pass's appends too
    log(w.describe())

    t = time.perf_counter()
    K, V = generate(w, torch, dev)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")
    cache = PackedKVCache(S, T_max, bits=w.bits, block=w.block, permute=args.permute, device="cuda:0",
                         payload_order=args.payload_order)
    torch.cuda.synchronize()
    t = time.perf_counter()
    cache.compress(K, V)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    assert cache.check() == 0
    layer_caches = [cache]
    for _ in range(args.layers - 1):            # the other layers hold the same tokens
        c2 = PackedKVCache(S, T_max, bits=w.bits, block=w.block, permute=args.permute, device="cuda:0",
                         payload_order=args.payload_order)
        c2.compress(K, V)
        layer_caches.append(c2)
    # the same tokens in paged caches: every stream at T0, and streams spread
    # linearly from T0 down to T0/4 (ragged lengths)
    paged = {}
    if not args.no_paged:
        from decode_gemv_amd import PagedKVCache
        ko = cache.offsets("K").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        vo = cache.offsets("V").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        nb0 = -(-T0 // w.block)
        per_token = (ko[:, nb0].sum() + vo[:, nb0].sum()) / (S * T0)
        page = args.page_kib << 10
        for kind in ("uniform", "ragged"):
            lens = [T0] * S if kind == "uniform" else [T0 - (3 * T0 // 4) * s // S for s in range(S)]
            n_pages = sum(int(np.ceil(1.1 * (L + n_steps) * per_token / page)) + 2 for L in lens) + 16
            pc = PagedKVCache(S, T0 + n_steps + 8, n_pages, page_bytes=page, bits=w.bits, block=w.block,
                              permute=args.permute, device="cuda:0",
                         payload_order=args.payload_order)
            if kind == "uniform":
                pc.prefill(0, K, V)
            else:
                for s_, L in enumerate(lens):
                    pc.prefill(s_, K[s_:s_ + 1, :L].contiguous(), V[s_:s_ + 1, :L].contiguous())
            if pc.check() != 0:
                raise RuntimeError(f"paged prefill ({kind}) failed")
            paged[kind] = pc
    del K, V
    torch.cuda.empty_cache()

    def used_bytes():
        ko = cache.offsets("K").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        vo = cache.offsets("V").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        nb = -(-cache.n_tokens // w.block)
        return int(ko[:, nb].sum()), int(vo[:, nb].sum()), nb

    kb0, vb0, nb0 = used_bytes()
    st = cache.stats()
    cr = compression_ratios(st, S, T0, D, w.bits, nb0)
    log(f"prefill {prefill_s * 1e3:.1f} ms; CR (physical) K {cr['k']['physical']:.3f} V {cr['v']['physical']:.3f}")

    # per-step inputs, generated before timing
    kn = torch.empty((n_steps, S, 1, D), dtype=torch.float16)
    vn = torch.empty_like(kn)
    qn = torch.empty((n_steps, S, G, D), dtype=torch.float16)
    for i in range(n_steps):
        for s in range(S):
            k1, v1 = kvsynth.append_kv(w, s, i)
            kn[i, s], vn[i, s] = torch.from_numpy(k1), torch.from_numpy(v1)
            qn[i, s] = torch.from_numpy(kvsynth.stream_q(w, s, step=i))
    kn, vn, qn = kn.to(dev), vn.to(dev), qn.to(dev)
    scores = torch.empty((S, G, T_max), dtype=torch.float32, device=dev)
    p = torch.empty_like(scores)
    out = torch.empty((S, G, D), dtype=torch.float32, device=dev)
    ws = cache.workspace(G)
    scale = 1.0 / float(np.sqrt(D))

    def status_ok(where):
        code = cache.check()
        if code:
            raise RuntimeError(f"cache status {code} after {where}")

    # a write of twice the 256 MB memory-side cache before every step (outside
    # the step's events), so no step finds records a previous one left there
    flush_buf = torch.empty(max(args.flush_mib, 1) << 20, dtype=torch.uint8, device=dev)

    def flush(i):
        if args.flush_mib > 0:
            flush_buf.fill_(i & 0xFF)

    def timed_loop(launch, n_ev):
        """W untimed + K timed steps, each after a cache flush.  Returns (mean
        and median ms per step from the HIP events around each step, wall ms
        per step over the K steps with their flushes, per-step events)."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n_steps)]
        torch.cuda.synchronize()
        t0 = None
        for i in range(n_steps):
            if i == args.warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            flush(i)
            launch(i, ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        status_ok(launch.__name__)
        evs = ev[args.warmup:]
        per = [x[0].elapsed_time(x[-1]) for x in evs]
        return float(np.mean(per)), float(np.median(per)), wall / args.steps * 1e3, evs

    def avg_ms(evs, a, b):
        return float(np.mean([x[a].elapsed_time(x[b]) for x in evs]))

    def med_ms(evs, a, b):
        return float(np.median([x[a].elapsed_time(x[b]) for x in evs]))

    # the step: append one token per stream, then decode attention in one
    # launch (K GEMV, softmax and V GEMV fused)
    aws = cache.attention_workspace(G)
    fout = torch.empty((S, G, D), dtype=torch.float32, device=dev)

    def fused_step(i, e):
        e[0].record()
        cache.append(kn[i], vn[i])
        e[1].record()
        cache.attention(qn[i], scale, out=fout, workspace=aws)
        e[2].record()

    # bring the GPU to its steady clock first: ~0.3 s of attention launches
    # on the prefilled cache (they change no state)
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:
        for _ in range(20):
            cache.attention(qn[0], scale, out=fout, workspace=aws)
        torch.cuda.synchronize()
    status_ok("the clock warm-up")

    multi = None
    if args.layers > 1:
        # decode attention over every layer at one step: one launch per
        # layer, then the multi-cache launch (up to 32 caches per launch)
        L = args.layers
        qm = qn[0].unsqueeze(0).expand(L, S, G, D).contiguous()
        outm = torch.empty((L, S, G, D), dtype=torch.float32, device=dev)
        wsm = attention_multi_workspace(layer_caches, G)
        ws1 = [c.attention_workspace(G) for c in layer_caches]
        reps = 20

        def per_layer():
            for i, c in enumerate(layer_caches):
                c.attention(qm[i], scale, out=outm[i], workspace=ws1[i])

        def one_launch():
            attention_multi(layer_caches, qm, scale, out=outm, workspace=wsm)

        res_ms = {}
        for name, fn in (("per_layer", per_layer), ("multi", one_launch)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res_ms[name] = e0.elapsed_time(e1) / reps
        for c in layer_caches:
            assert c.check() == 0
        kbl, vbl, nbl = used_bytes()
        layer_bytes = kbl + vbl + 2 * 4 * S * (nbl + 1)
        multi = {"layers": L, "per_layer_launches_ms": round(res_ms["per_layer"], 4),
                 "multi_launch_ms": round(res_ms["multi"], 4),
                 "multi_GBps": round(L * layer_bytes / (res_ms["multi"] * 1e-3) / 1e9, 1),
                 "note": "decode attention over L caches of this shape at the prefill length"}
        log(f"{L} layers: {res_ms['per_layer']:.3f} ms as {L} launches, {res_ms['multi']:.3f} ms as one")
        del layer_caches[1:], wsm, ws1, outm, qm
        torch.cuda.empty_cache()

    ms_step, ms_step_med, wall_step, fev = timed_loop(fused_step, 3)
    kb1, vb1, nb1 = used_bytes()
    t_app, t_attn = avg_ms(fev, 0, 1), avg_ms(fev, 1, 2)
    m_app, m_attn = med_ms(fev, 0, 1), med_ms(fev, 1, 2)

    # the same steps with the three kernels of the path launched separately
    # (scores and weights go through HBM); the appends continue the cache
    def separate_step(i, e):
        e[0].record()
        cache.append(kn[i], vn[i])
        e[1].record()
        cache.qk(qn[i], scores)
        e[2].record()
        softmax_rows(scores, cache.n_tokens, scale, out=p)
        e[3].record()
        cache.pv(p, out, workspace=ws)
        e[4].record()

    sep_ms_step, _, _, sev = timed_loop(separate_step, 5)
    gpu = gpu_info(torch)                    # clocks read right after the timed loops
    kb2, vb2, nb2 = used_bytes()
    t_qk, t_sm, t_pv = avg_ms(sev, 1, 2), avg_ms(sev, 2, 3), avg_ms(sev, 3, 4)
    m_qk, m_sm, m_pv = med_ms(sev, 1, 2), med_ms(sev, 2, 3), med_ms(sev, 3, 4)

    # compressed bytes read per step (records + offset tables), mean over each loop
    k_bytes = (kb0 + kb1) / 2 + 4 * S * (nb1 + 1)
    v_bytes = (vb0 + vb1) / 2 + 4 * S * (nb1 + 1)
    value = (k_bytes + v_bytes) / (ms_step * 1e-3) / 1e9
    k_bytes2 = (kb1 + kb2) / 2 + 4 * S * (nb2 + 1)
    v_bytes2 = (vb1 + vb2) / 2 + 4 * S * (nb2 + 1)
    sep_value = (k_bytes2 + v_bytes2) / (sep_ms_step * 1e-3) / 1e9
    T1 = T0 + args.warmup + args.steps / 2                      # mean length, fused loop
    T2 = T0 + n_steps + args.warmup + args.steps / 2            # mean length, separate loop

    # algorithmic bytes per launch: records and offset tables, q, and the
    # outputs (scores / weights / out); the V GEMV's and the fused kernel's
    # split partials (< 0.5 %) are not counted
    attn_alg = k_bytes + v_bytes + S * G * D * 2 + S * G * D * 4
    qk_alg = k_bytes2 + S * G * D * 2 + S * G * T2 * 4
    pv_alg = v_bytes2 + S * G * T2 * 4 + S * G * D * 4
    attn_gbps = attn_alg / (t_attn * 1e-3) / 1e9
    qk_gbps = qk_alg / (t_qk * 1e-3) / 1e9
    pv_gbps = pv_alg / (t_pv * 1e-3) / 1e9
    tr = load_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                "traffic": tr.get("attn") if tr else None,
                "kernel": "k_attn_decode", "bytes_per_launch": int(attn_alg), "launch_ms": round(t_attn, 4),
                "launch_ms_median": round(m_attn, 4),
                "frac_at_median": round(attn_alg / (m_attn * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    # the step on the paged caches: append, then fused attention through the
    # block tables
    paged_res = None
    if paged:
        paged_res = {"page_bytes": args.page_kib << 10,
                     "contiguous_arenas_MiB": round(2 * cache.sizes.arena_bytes / 2**20, 1)}
        pout = torch.empty((S, G, D), dtype=torch.float32, device=dev)
        for kind, pc in paged.items():
            pws = pc.attention_workspace(G)

            def alg_bytes():
                (ks_, kz_), (vs_, vz_) = pc.tables()
                tot = 0
                for s_, L in enumerate(pc.lengths):
                    nb_ = -(-L // w.block)
                    tot += int(kz_[s_, :nb_].sum() + vz_[s_, :nb_].sum()) + 16 * nb_
                return tot + S * G * D * 2 + S * G * D * 4

            a0 = alg_bytes()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_steps)]
            torch.cuda.synchronize()
            for i in range(n_steps):
                if i == args.warmup:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                flush(i)
                ev[i][0].record()
                pc.append(kn[i], vn[i])
                ev[i][1].record()
                if kind == "uniform" and i % 2:
                    # paired control: the contiguous cache's launch in the same
                    # loop, before the paged one on odd steps and after on even
                    cache.attention(qn[i], scale, out=fout, workspace=aws)
                    ev[i][2].record()
                pc.attention(qn[i], scale, out=pout, workspace=pws)
                ev[i][3 if kind == "uniform" and i % 2 else 2].record()
                if kind == "uniform" and i % 2 == 0:
                    cache.attention(qn[i], scale, out=fout, workspace=aws)
                    ev[i][3].record()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / args.steps * 1e3
            code = pc.check()
            if code:
                raise RuntimeError(f"paged cache status {code} after the {kind} loop")
            a1 = alg_bytes()
            evs = ev[args.warmup:]
            if kind == "uniform":
                steps_i = range(args.warmup, n_steps)
                t_pa = float(np.mean([ev[i][2].elapsed_time(ev[i][3]) if i % 2 else ev[i][1].elapsed_time(ev[i][2])
                                      for i in steps_i]))
                t_ctl = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) if i % 2 else ev[i][2].elapsed_time(ev[i][3])
                                       for i in steps_i]))
            else:
                t_pa = avg_ms(evs, 1, 2)
            used_pages = pc.n_pages - pc.free_pages()
            lens = pc.lengths
            paged_res[kind] = {
                "attention_ms": round(t_pa, 4), "GBps": round((a0 + a1) / 2 / (t_pa * 1e-3) / 1e9, 1),
                "append_ms": round(avg_ms(evs, 0, 1), 4), "ms_per_step": round(wall, 4),
                "tokens_min": min(lens), "tokens_max": max(lens), "tokens_mean": round(float(np.mean(lens)), 1),
                "pages_used": used_pages,
                "pool_used_MiB": round((used_pages * pc.page_bytes + 2 * S * pc.sizes.slot_bytes) / 2**20, 1),
                "record_MiB": round(((a0 + a1) / 2 - S * G * D * 6) / 2**20, 1)}
            if kind == "uniform":
                paged_res[kind]["contiguous_attention_ms"] = round(t_ctl, 4)
                paged_res[kind]["ms_per_step"] = None          # the loop also ran the control
            log(f"paged {kind}: attention {t_pa:.4f} ms, {paged_res[kind]['GBps']} GB/s, "
                f"{used_pages} pages")
        paged_res["note"] = ("append then fused attention per step through the block tables; ragged: "
                             "stream lengths spread linearly from T to T/4")
        del paged

    # the device's streaming-read ceiling, measured like the fused launch: the
    # library's read probe over as many bytes as one launch reads, averaged
    # over back-to-back launches
    from decode_gemv_amd import stream_read
    rbytes = (int(attn_alg) + 255) // 256 * 256
    rbuf = torch.ones(rbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    for _ in range(5):
        stream_read(rbuf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        stream_read(rbuf, sink)
    e1.record()
    torch.cuda.synchronize()
    read_ceiling = rbytes / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    del rbuf
    roofline["read_ceiling_GBps"] = round(read_ceiling, 1)
    roofline["frac_of_read_ceiling"] = round(attn_gbps / read_ceiling, 4)
    log(f"streaming-read ceiling {read_ceiling:.0f} GB/s")

    # a plain device copy of known size, for counter calibration runs
    if args.copy_probe_mib > 0:
        a = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        cpu = cpu_baseline(w, args.cpu_streams, args.cpu_seconds, args.permute, args.payload_order)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 acc; V weights 20-bit fixed point x u4/u8 ints",
        "arithmetic": ("K GEMV: fp32 FMA of q*scale with the exact 4-bit containers (one query per "
                       "stream) or int8 matrix cores on q*scale in 24-bit fixed point (four queries); "
                       "V GEMV: weights*scale in 20-bit fixed point per block times the ints by integer "
                       "dot products (v_dot8 / v_dot4 / int8 matrix cores), exact integer sums, fp32 "
                       "accumulation; softmax fp32; encoder fp64 (bit-exact with the oracle)"),
        "data": "synthetic (seeded kvsynth generator; stands in for the pages' models and benchmarks)",
        "config": {"workload": w.key, "batch": w.batch, "kv_heads": w.kv_heads, "group": G,
                   "tokens": T0, "head_dim": D, "bits": w.bits, "block": w.block, "run": 32,
                   "append_per_step": 1, "permute": args.permute, "payload_order": args.payload_order,
                   "parallelism": "single-gpu"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "ms_per_step_median": round(ms_step_med, 4),
        "wall_ms_per_step": round(wall_step, 4),
        "kernels_ms": {"append": round(m_app, 4), "attention": round(m_attn, 4), "qk_gemv": round(m_qk, 4),
                       "softmax": round(m_sm, 4), "pv_gemv": round(m_pv, 4), "stat": "median"},
        "kernels_ms_mean": {"append": round(t_app, 4), "attention": round(t_attn, 4), "qk_gemv": round(t_qk, 4),
                            "softmax": round(t_sm, 4), "pv_gemv": round(t_pv, 4)},
        "timing": (f"HIP events on the launch stream around each step and kernel; a {args.flush_mib} MiB "
                   "write before every step evicts the memory-side cache (not timed); ms_per_step and "
                   "value from the mean step time, wall_ms_per_step includes the flushes"),
        "kernel_GBps": {"attention": round(attn_gbps, 1), "qk_gemv": round(qk_gbps, 1),
                        "pv_gemv": round(pv_gbps, 1)},
        "gemv_effective_GBps": {"qk": round(k_bytes2 / (t_qk * 1e-3) / 1e9, 1),
                                "pv": round(v_bytes2 / (t_pv * 1e-3) / 1e9, 1)},
        "separate_path": {"ms_per_step": round(sep_ms_step, 4), "value": round(sep_value, 1),
                          "note": "append, K GEMV, softmax, V GEMV as four launches"},
        "cr": cr,
        "width_hist": {"k": st["k_width_hist"], "v": st["v_width_hist"]},
        "prefill_ms": round(prefill_s * 1e3, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "multi_layer": multi,
        "paged": paged_res,
        "alg_bytes_per_launch": {"attn": int(attn_alg), "qk": int(qk_alg), "pv": int(pv_alg)},
        "gpu": gpu,
        "kernel_source": kernel_source_hash(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
