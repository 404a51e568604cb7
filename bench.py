"""Benchmark of the KVarN hot path on one MI355X.

One step = kvarn_quantize over every full page of the cache that leaves the
fp16 sink and tail (keys and values), then one kvarn_decode_attn step over the
whole batch reading those records plus the fp16 sink and tail.

Default workload: a dense 8B-like layer -- 32 query / 8 KV heads, head_dim
128, batch 16, 32768-token context, k4v2 with 128-token tiles, fp16 first 128
and last 1024 tokens, page size 128, K/V ~ N(0,1) with 1% outlier channels
x20 (synthetic, seeded).

Reported (one JSON line):
  value     (fp16 bytes consumed by quantize + decode effective bytes) /
            (quantize time + decode time), GB/s; times from HIP events around
            each call on the stream the kernels run on, averaged over the
            timed steps.  L2 and the 256 MB last-level cache are flushed
            before each call, outside the event pairs, by reading a 1 GiB
            buffer: the caches then hold clean lines of an unrelated buffer
            (a fill would leave dirty lines whose write-back lands inside the
            next timed call).
  roofline  the quantize kernel (the step's dominant kernel): algorithmic
            bytes per launch (fp16 read + records written) / launch time,
            against 8 TB/s HBM.  traffic: HBM bytes per launch from the
            FETCH_SIZE / WRITE_SIZE counter passes recorded under profiles/
            for this workload, scaled by a 1 GiB copy's readings; null when
            the quantize sources differ from the ones profiled.
  components quantize and decode separately, each as GB/s and % of peak.
  cpu_baseline the oracle (plain C, fp64, OpenMP) on a bounded sample of the
            same workload, same byte formulas.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# sources whose compiled code the recorded counter passes measured
QUANTIZE_SOURCES = ["kv_cache_quantization_kvarn_amd/build.py"] + [
    "kv_cache_quantization_kvarn_amd/csrc/" + f for f in
    ("kvarn_device.hpp", "kvarn_internal.hpp", "quantize_impl.hpp", "quantize.hip", "quantize_d128.hip",
     "quantize_d256.hip", "quantize_d512.hip")]


def quantize_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in QUANTIZE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per quantize launch recorded for this workload, if the
    quantize sources are the ones that were profiled."""
    path = os.path.join(ROOT, "profiles", f"quantize_kernel_{workload}_hbm.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != quantize_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
METRIC = "quantize fp16 GB/s + decode-attn effective HBM GB/s, % of MI355X peak"


def byte_counts(case):
    """Algorithmic bytes of one step (the formulas of the design notes)."""
    lay = case["layout"]
    T, D, H, kb, vb, mla = lay["T"], lay["D"], lay["H"], lay["k_bits"], lay["v_bits"], lay["mla"]
    rec = lambda b: T * D * b // 8 + 4 * T + 2 * D
    nq = case["n_qpages"]
    kinds = [kb] if mla else [kb, vb]
    q_fp16 = nq * H * T * D * 2 * len(kinds)
    q_out = nq * H * sum(rec(b) for b in kinds)
    # decode: every record of every sequence + fp16 sink/tail tokens + q + out
    seq = case["seq_lens"].cpu().tolist()
    dec = 0
    for L in seq:
        nqs = max(0, (L - lay["sink"] - lay["tail"]) // T)
        nf_tok = L - nqs * T
        dec += nqs * H * sum(rec(b) for b in kinds)
        dec += nf_tok * H * D * 2 * len(kinds)
    qbytes = case["q"].numel() * case["q"].element_size()
    dec += qbytes + case["B"] * case["Hq"] * D * 4
    return q_fp16, q_out, dec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense8b_b16_32k_k4v2_g128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-records", type=int, default=0,
                    help="records in the oracle's quantize sample (0: every record of the workload)")
    ap.add_argument("--cpu-rows", type=int, default=64, help="(sequence, head) rows in the oracle's decode sample")
    ap.add_argument("--print-source-hash", action="store_true", help="print the quantize source hash and exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.print_source_hash:
        print(quantize_source_hash())
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_quantization_kvarn_amd as kv
    from synth.cases import WORKLOADS, make_case

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.steps)
        return
    w = WORKLOADS[args.workload]
    print(f"[bench] building {args.workload} on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    case = make_case(w, device=dev)
    lay = case["layout"]
    L = kv.layout_from_dict(lay)
    H = lay["H"]
    krec = torch.empty((case["n_qpages"], H, kv.record_bytes(L, 0)), dtype=torch.uint8, device=dev)
    vrec = None if lay["mla"] else torch.empty((case["n_qpages"], H, kv.record_bytes(L, 1)), dtype=torch.uint8,
                                               device=dev)
    out = torch.empty((case["B"], case["Hq"], lay["D"]), dtype=torch.float32, device=dev)
    ws = kv.alloc_workspace(L, case["B"], case["Hq"], case["max_pages"], dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    flush_sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def flush():
        flush_sink.add_(flush_buf.sum())

    q_fp16, q_out, dec_bytes = byte_counts(case)

    def quantize():
        kv.quantize(L, case["k16"], case["v16"], krec, vrec, case["src"], case["dst"])

    def decode():
        kv.decode_attn(L, krec, vrec, case["k16"], case["v16"], case["block_table"], case["seq_lens"], case["q"],
                       case["sm_scale"], out=out, workspace=ws)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(timed):
        flush()
        ev[0].record()
        quantize()
        ev[1].record()
        flush()
        ev[2].record()
        decode()
        ev[3].record()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    tq, td = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        tq.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        td.append(ev[2].elapsed_time(ev[3]) * 1e-3)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps", file=sys.stderr, flush=True)

    tq_m, td_m = float(np.mean(tq)), float(np.mean(td))
    value = (q_fp16 + dec_bytes) / (tq_m + td_m) / 1e9
    q_gbs_i = q_fp16 / tq_m / 1e9
    q_gbs_ii = (q_fp16 + q_out) / tq_m / 1e9
    d_gbs = dec_bytes / td_m / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "kernel_ms_per_step": round((tq_m + td_m) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": case["B"], "context": int(w["L"]), "q_heads": case["Hq"],
                   "kv_heads": H, "head_dim": lay["D"], "tile_tokens": lay["T"], "k_bits": lay["k_bits"],
                   "v_bits": None if lay["mla"] else lay["v_bits"], "iters": lay["n_iters"],
                   "sink": lay["sink"], "tail": lay["tail"], "mla": bool(lay["mla"])},
        "roofline": {"bound": "hbm", "kernel": "quantize_kernel", "achieved": round(q_gbs_ii, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(q_gbs_ii / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": q_fp16 + q_out, "launch_us": round(tq_m * 1e6, 2),
                     "traffic": recorded_traffic(args.workload)},
        "components": {
            "quantize": {"us": round(tq_m * 1e6, 2), "fp16_GBs": round(q_gbs_i, 1),
                         "fp16_frac": round(q_gbs_i / HBM_PEAK_GBS, 4), "traffic_GBs": round(q_gbs_ii, 1),
                         "traffic_frac": round(q_gbs_ii / HBM_PEAK_GBS, 4), "fp16_bytes": q_fp16,
                         "out_bytes": q_out},
            "decode": {"us": round(td_m * 1e6, 2), "GBs": round(d_gbs, 1), "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                       "bytes": dec_bytes},
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, krec, vrec, args.cpu_records, args.cpu_rows)
    print(json.dumps(res), flush=True)


def copy_probe(steps):
    """1 GiB read + 1 GiB write per launch: the reference for byte counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(steps):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[len(ts) // 2]
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "median_us": round(t * 1e6, 2),
                      "GBs": round(2 * n / t / 1e9, 1)}), flush=True)


def cpu_baseline(case, krec, vrec, n_records, n_rows):
    """The oracle on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle

    lay = case["layout"]
    T, D, H, mla = lay["T"], lay["D"], lay["H"], lay["mla"]
    threads = len(os.sched_getaffinity(0))
    threads = min(threads, int(os.environ.get("OMP_NUM_THREADS", threads)))
    kinds = 1 if mla else 2
    # quantize: n_records records (pages x heads x K/V) of the workload
    if n_records <= 0:
        n_records = case["n_qpages"] * H * kinds
    n_pages = max(1, min(case["n_qpages"], math.ceil(n_records / (H * kinds))))
    src = case["src"][:n_pages].cpu().numpy()
    pages = np.unique(src)
    remap = {int(p): i for i, p in enumerate(pages)}
    k16 = case["k16"][torch.as_tensor(pages, device=case["k16"].device).long()].cpu().contiguous()
    k16 = k16.view(torch.int16).numpy().view(np.uint16)
    v16 = None
    if not mla:
        v16 = case["v16"][torch.as_tensor(pages, device=case["v16"].device).long()].cpu().contiguous()
        v16 = v16.view(torch.int16).numpy().view(np.uint16)
    s_loc = np.array([remap[int(p)] for p in src], np.int32)
    d_loc = np.arange(n_pages, dtype=np.int32)
    rb = lambda b: T * D * b // 8 + 4 * T + 2 * D
    kr = np.zeros((n_pages, H, rb(lay["k_bits"])), np.uint8)
    vr = None if mla else np.zeros((n_pages, H, rb(lay["v_bits"])), np.uint8)
    t0 = time.perf_counter()
    oracle.quantize_pages(lay, k16, v16, s_loc, d_loc, kr, vr, n_threads=threads)
    tq = time.perf_counter() - t0
    qbytes = n_pages * H * T * D * 2 * kinds
    # decode: n_rows (sequence, query head) rows, on the HIP path's records
    rng = np.random.default_rng(5)
    pairs = np.array([(int(rng.integers(case["B"])), int(rng.integers(case["Hq"]))) for _ in range(n_rows)],
                     np.int32)
    bt = case["block_table"].cpu().numpy()
    sl = case["seq_lens"].cpu().numpy()
    k16a = case["k16"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    v16a = None if mla else case["v16"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    q = case["q"]
    qh = q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16) if q.dtype == torch.bfloat16 \
        else q.cpu().numpy()
    krh = krec.cpu().numpy()
    vrh = None if vrec is None else vrec.cpu().numpy()
    t0 = time.perf_counter()
    oracle.decode(lay, krh, vrh, k16a, v16a, bt, sl, qh, case["Hq"], case["sm_scale"], pairs=pairs,
                  n_threads=threads)
    td = time.perf_counter() - t0
    # decode bytes of those rows: each row reads its KV head's cache once (a
    # query head's share of the group's read: 1/G of the KV head's bytes)
    G = case["Hq"] // H
    dbytes = 0
    for b, _ in pairs:
        Lb = int(sl[b])
        nqs = max(0, (Lb - lay["sink"] - lay["tail"]) // T)
        per_head = nqs * (rb(lay["k_bits"]) + (0 if mla else rb(lay["v_bits"]))) + (Lb - nqs * T) * D * 2 * kinds
        dbytes += per_head / G
    return {"value": round((qbytes + dbytes) / (tq + td) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "quantize_GBs": round(qbytes / tq / 1e9, 4), "decode_GBs": round(dbytes / td / 1e9, 4),
            "seconds": round(tq + td, 2),
            "sample": f"quantize {n_pages * H * kinds} of {case['n_qpages'] * H * kinds} records; decode "
                      f"{n_rows} of {case['B'] * case['Hq']} (sequence, query head) rows on the GPU's records"}


if __name__ == "__main__":
    main()
