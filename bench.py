#!/usr/bin/env python3
"""Decode-step throughput of the PackKV packed cache on one MI355X.

One step is one decode-attention pass over the packed cache of every stream:
append one new token per stream (open-tail re-encode: quantise, reorder,
pack), the fused K decompress-GEMV, softmax, and the fused V decompress-GEMV.
The cache is prefilled (bulk compress) before the timed region, so every
input is resident in HBM when timing starts.

value = compressed bytes the two fused GEMVs read per step (K and V records
plus their offset tables) / wall time per step, in GB/s (1e9 B/s).  The
per-kernel split, the roofline of the dominant kernel (bytes per launch over
its HIP-event duration) and the oracle's CPU throughput are reported beside.

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
                  for f in ("gemv.hip", "common.hpp", "kernels.hpp")]


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


def cpu_baseline(w: kvsynth.Workload, n_streams: int) -> dict:
    """The fp64 oracle's decode step on a sample of streams, single-threaded."""
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import stream as ostream, attention
    cfg = oracle.Config(bits=w.bits, block=w.block)
    with threadpool_limits(limits=1):
        caches, qs, kv_new = [], [], []
        for s in range(n_streams):
            k, v = kvsynth.stream_kv(w, s)
            caches.append(ostream.compress(k, v, cfg))          # prefill: not timed
            qs.append(kvsynth.stream_q(w, s, step=0))
            kv_new.append(kvsynth.append_kv(w, s, 0))
        nbytes = 0
        t0 = time.perf_counter()
        for s in range(n_streams):
            c = ostream.append(caches[s], *kv_new[s])           # tail re-encode
            kh, vh, _, _ = ostream.decode_stream(c)               # unpack + fp64 dequant
            p = attention.softmax(attention.qk(qs[s], kh), w.head_dim)
            attention.pv(p, vh)
            nbytes += len(c.arena("K")) + len(c.arena("V")) + 8 * (len(c.blocks) + 1)
        dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_streams} of {w.streams} streams at the full {w.tokens} tokens, one decode "
                      f"step each (tail re-encode, unpack, fp64 dequantise, K GEMV, softmax, V GEMV), "
                      f"{dt:.2f} s; value = compressed bytes decoded per second"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b-32k", choices=sorted(kvsynth.WORKLOADS))
    ap.add_argument("--cpu-streams", type=int, default=2, help="streams in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of a plain device copy run after timing (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the packed cache is per stream and this build runs on a "
              "single MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_gemv_amd import PackedKVCache, softmax_rows

    w = kvsynth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    S, G, T0, D = w.streams, w.group, w.tokens, w.head_dim
    n_steps = args.warmup + args.steps
    T_max = T0 + n_steps
    log(w.describe())

    t = time.perf_counter()
    K, V = generate(w, torch, dev)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")
    cache = PackedKVCache(S, T_max, bits=w.bits, block=w.block, device="cuda:0")
    torch.cuda.synchronize()
    t = time.perf_counter()
    cache.compress(K, V)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    assert cache.check() == 0
    del K, V
    torch.cuda.empty_cache()

    def used_bytes():
        ko = cache.offsets("K").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        vo = cache.offsets("V").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        nb = -(-cache.n_tokens // w.block)
        return int(ko[:, nb].sum()), int(vo[:, nb].sum()), nb

    kb0, vb0, _ = used_bytes()
    st = cache.stats()
    raw = 2 * S * T0 * D
    log(f"prefill {prefill_s * 1e3:.1f} ms; CR K {raw / kb0:.3f} V {raw / vb0:.3f}")

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

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    t0 = None
    for i in range(n_steps):
        if i == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        e = ev[i]
        e[0].record()
        cache.append(kn[i], vn[i])
        e[1].record()
        cache.qk(qn[i], scores)
        e[2].record()
        softmax_rows(scores, cache.n_tokens, scale, out=p)
        e[3].record()
        cache.pv(p, out, workspace=ws)
        e[4].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert cache.check() == 0
    kb1, vb1, nb1 = used_bytes()

    timed = ev[args.warmup:]
    def avg_ms(a, b):
        return float(np.mean([x[a].elapsed_time(x[b]) for x in timed]))
    t_app, t_qk, t_sm, t_pv = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3), avg_ms(3, 4)
    ms_step = wall / args.steps * 1e3

    # compressed bytes the GEMVs read per step (records + offset tables), mean over the run
    k_bytes = (kb0 + kb1) / 2 + 4 * S * (nb1 + 1)
    v_bytes = (vb0 + vb1) / 2 + 4 * S * (nb1 + 1)
    T_mid = T0 + args.warmup + args.steps / 2
    value = (k_bytes + v_bytes) / (ms_step * 1e-3) / 1e9

    # roofline of the dominant GEMV: algorithmic bytes of one launch / its event time
    qk_alg = k_bytes + S * G * D * 2 + S * G * T_mid * 4
    pv_alg = v_bytes + S * G * T_mid * 4 + S * G * D * 4
    qk_gbps = qk_alg / (t_qk * 1e-3) / 1e9
    pv_gbps = pv_alg / (t_pv * 1e-3) / 1e9
    dom = "qk" if t_qk >= t_pv else "pv"
    ach = qk_gbps if dom == "qk" else pv_gbps
    tr = load_traffic(args.workload)
    traffic = None
    if tr and dom in tr:
        traffic = tr[dom]
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "k_qk_gemv" if dom == "qk" else "k_pv_gemv (+k_pv_reduce)",
                "bytes_per_launch": int(qk_alg if dom == "qk" else pv_alg),
                "launch_ms": round(t_qk if dom == "qk" else t_pv, 4)}

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
        cpu = cpu_baseline(w, args.cpu_streams)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded kvsynth generator; stands in for the pages' models and benchmarks)",
        "config": {"workload": w.key, "batch": w.batch, "kv_heads": w.kv_heads, "group": G,
                   "tokens": T0, "head_dim": D, "bits": w.bits, "block": w.block, "run": 32,
                   "append_per_step": 1, "parallelism": "single-gpu"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "kernels_ms": {"append": round(t_app, 4), "qk_gemv": round(t_qk, 4), "softmax": round(t_sm, 4),
                       "pv_gemv": round(t_pv, 4)},
        "gemv_GBps": {"qk": round(qk_gbps, 1), "pv": round(pv_gbps, 1)},
        "cr": {"k": round(2 * S * T0 * D / kb0, 4), "v": round(2 * S * T0 * D / vb0, 4)},
        "width_hist": {"k": st["k_width_hist"], "v": st["v_width_hist"]},
        "prefill_ms": round(prefill_s * 1e3, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
