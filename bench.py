"""Benchmark of the KVarN hot path on one MI355X.

One step = kvarn_quantize over every full page of the cache that leaves the
fp16 sink and tail (keys and values), then one kvarn_decode_attn step over the
whole batch reading those records plus the fp16 sink and tail.

Headline workload (the largest single-GPU configuration): a dense 8B-like
layer with 64-token tiles -- 32 query / 8 KV heads, head_dim 128, batch 64,
16384-token context, k4v2 (4-bit keys, 2-bit values), 6 normalization
iterations, fp16 first 128 and last 1024 tokens, page size 64, K/V ~ N(0,1)
with 4 outlier channels per head x20 (synthetic, seeded).  Exactly --steps
steps are timed after --warmup untimed ones.

Reported (one JSON line):
  value      (fp16 bytes consumed by quantize + decode effective bytes) /
             (median quantize time + median decode time), GB/s; times from
             HIP events around each call on the stream the kernels run on.
             L2 and the 256 MB last-level cache are flushed before each call,
             outside the event pairs, by reading a 1 GiB buffer (a fill would
             leave dirty lines whose write-back lands inside the next call).
  roofline   the quantize kernel (the step's dominant kernel): algorithmic
             bytes per launch (fp16 read + records written) / mean launch
             time, against 8 TB/s HBM.  traffic: HBM bytes per launch from
             the FETCH_SIZE / WRITE_SIZE counter passes recorded under
             profiles/ for this workload, scaled by a 1 GiB copy's readings;
             null when the quantize sources differ from the ones profiled.
  components every workload of the suite (the headline one included):
             quantize under both byte readings (fp16 consumed; fp16 read +
             records written) and decode, each as GB/s and fraction of HBM
             peak, median with p10 / p90 of the per-call times; the MLA decode
             also as a fraction of the fp16 MFMA peak (its roofline), and
             once more with a 64-wide fp16 rope key beside every latent
             (decode_rope64: the same cache plus its rope pools and 576-wide
             queries; bytes and flops include the rope part).
             The headline workload also times a verify step (decode of 4
             uncommitted query tokens per sequence, causal among themselves);
             the 16 x 32K workload also runs with the key/value code widths
             3/5, 5/3 and 8/8 (widths: quantize and decode times and
             fractions, records of those widths).
  cpu_baseline the oracle (plain C, fp64, OpenMP) on a bounded sample of the
             headline workload, same byte formulas; per_core: the oracle on
             one thread over the one-layer 1024-token case.
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
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 matrix peak of the MI355X
HEADLINE = "dense8b_b64_16k_k4v2_g64"
# the 16 x 32K layer also runs with these key/value code widths
WIDTHS_WORKLOAD, WIDTH_PAIRS = "dense8b_b16_32k_k4v2_g128", [(3, 5), (5, 3), (8, 8)]
SUITE = ["tiny_d128_k4v2", "dense8b_b16_32k_k4v2_g128", "dense8b_b64_16k_k4v2_g64", "wide_d256_b8_64k_k6v6",
         "wide_d512_b8_64k_k6v6", "mla_d512_b32_32k_int4"]
# sources whose compiled code the recorded counter passes measured
QUANTIZE_SOURCES = ["kv_cache_quantization_kvarn_amd/build.py"] + [
    "kv_cache_quantization_kvarn_amd/csrc/" + f for f in
    ("kvarn_device.hpp", "kvarn_internal.hpp", "quantize_impl.hpp", "quantize.hip", "quantize_d128.hip",
     "quantize_d256.hip", "quantize_d512.hip")]
METRIC = "quantize fp16 GB/s + decode-attn effective HBM GB/s, % of MI355X peak"


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


def byte_counts(case):
    """Algorithmic bytes of one step: fp16 consumed by quantize, records
    written by quantize, decode effective bytes (records + fp16 sink/tail +
    q + out); and the decode's matrix flops (4 per query head, channel and
    token: one multiply-add each for the score and the value sum)."""
    lay = case["layout"]
    T, D, H, kb, vb, mla = lay["T"], lay["D"], lay["H"], lay["k_bits"], lay["v_bits"], lay["mla"]
    rec = lambda b: T * D * b // 8 + 4 * T + 2 * D
    nq = case["n_qpages"]
    kinds = [kb] if mla else [kb, vb]
    q_fp16 = nq * H * T * D * 2 * len(kinds)
    q_out = nq * H * sum(rec(b) for b in kinds)
    seq = case["seq_lens"].cpu().tolist()
    dec = 0
    flops = 0
    for L in seq:
        nqs = max(0, (L - lay["sink"] - lay["tail"]) // T)
        nf_tok = L - nqs * T
        dec += nqs * H * sum(rec(b) for b in kinds)
        dec += nf_tok * H * D * 2 * len(kinds)
        flops += 4 * case["Hq"] * D * L
    qbytes = case["q"].numel() * case["q"].element_size()
    dec += qbytes + case["B"] * case["Hq"] * D * 4
    return q_fp16, q_out, dec, flops


def stats(ts):
    """median, p10, p90, mean of a list of seconds, in microseconds."""
    import numpy as np

    a = np.asarray(ts, np.float64) * 1e6
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean())}


class Runner:
    """One workload on the device: pools, records, workspace, and the timed
    quantize + decode calls."""

    def __init__(self, name, dev):
        import torch

        import kv_cache_quantization_kvarn_amd as kv
        from synth.cases import WORKLOADS, make_case

        self.kv, self.torch = kv, torch
        self.name = name
        self.w = WORKLOADS[name]
        self.case = case = make_case(self.w, device=dev)
        lay = case["layout"]
        self.L = kv.layout_from_dict(lay)
        H = lay["H"]
        nq = max(case["n_qpages"], 1)
        self.krec = torch.empty((nq, H, kv.record_bytes(self.L, 0)), dtype=torch.uint8, device=dev)
        self.vrec = None if lay["mla"] else torch.empty((nq, H, kv.record_bytes(self.L, 1)), dtype=torch.uint8,
                                                        device=dev)
        self.out = torch.empty((case["B"], case["Hq"], lay["D"]), dtype=torch.float32, device=dev)
        self.ws = kv.alloc_workspace(self.L, case["B"], case["Hq"], case["max_pages"], dev)
        self.bytes = byte_counts(case)

    def quantize(self):
        c = self.case
        self.kv.quantize(self.L, c["k16"], c["v16"], self.krec, self.vrec, c["src"], c["dst"])

    def decode(self):
        c = self.case
        self.kv.decode_attn(self.L, self.krec, self.vrec, c["k16"], c["v16"], c["block_table"], c["seq_lens"],
                            c["q"], c["sm_scale"], out=self.out, workspace=self.ws)

    def time_steps(self, steps, warmup, flush):
        """HIP events (on the current stream, where the calls are enqueued)
        around each call; returns per-step quantize and decode seconds."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

        def step():
            flush()
            ev[0].record()
            self.quantize()
            ev[1].record()
            flush()
            ev[2].record()
            self.decode()
            ev[3].record()

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        tq, td = [], []
        for _ in range(steps):
            step()
            torch.cuda.synchronize()
            tq.append(ev[0].elapsed_time(ev[1]) * 1e-3)
            td.append(ev[2].elapsed_time(ev[3]) * 1e-3)
        return tq, td

    def component(self, tq, td):
        q_fp16, q_out, dec, flops = self.bytes
        sq, sd = stats(tq), stats(td)
        lay = self.case["layout"]
        r = lambda x, n=2: round(x, n)
        comp = {
            "quantize": {"us": r(sq["median"]), "us_p10": r(sq["p10"]), "us_p90": r(sq["p90"]),
                         "us_mean": r(sq["mean"]),
                         "fp16_GBs": r(q_fp16 / sq["median"] / 1e3, 1),
                         "fp16_frac": r(q_fp16 / sq["median"] / 1e3 / HBM_PEAK_GBS, 4),
                         "traffic_GBs": r((q_fp16 + q_out) / sq["median"] / 1e3, 1),
                         "traffic_frac": r((q_fp16 + q_out) / sq["median"] / 1e3 / HBM_PEAK_GBS, 4),
                         "fp16_bytes": q_fp16, "out_bytes": q_out},
            "decode": {"us": r(sd["median"]), "us_p10": r(sd["p10"]), "us_p90": r(sd["p90"]), "us_mean": r(sd["mean"]),
                       "GBs": r(dec / sd["median"] / 1e3, 1), "frac": r(dec / sd["median"] / 1e3 / HBM_PEAK_GBS, 4),
                       "bytes": dec, "flops": flops},
        }
        if lay["mla"]:
            tf = flops / sd["median"] / 1e6
            comp["decode"]["bound"] = "mfma"
            comp["decode"]["TFLOPs"] = r(tf, 1)
            comp["decode"]["mfma_frac"] = r(tf / MFMA_F16_PEAK_TFLOPS, 4)
        else:
            comp["decode"]["bound"] = "hbm"
        if self.name == "tiny_d128_k4v2":
            comp["note"] = "cache-resident (fits L2 and the last-level cache): parity case, not a bandwidth figure"
        return comp

    def verify_setup(self, M):
        """A verify step over the same pools: the last M tokens of every
        sequence become uncommitted query tokens (committed length L - M; pages
        that only L would have quantized point back to their fp16 pages)."""
        torch, kv, c = self.torch, self.kv, self.case
        lay = c["layout"]
        T, sp = lay["T"], lay["sink"] // lay["T"]
        nq = lambda L: max(0, (L - lay["sink"] - lay["tail"]) // T)
        bt = c["block_table"].cpu().numpy().copy()
        src = c["src"].cpu().numpy()
        lens = c["seq_lens"].cpu().tolist()
        base = 0
        for b, L in enumerate(lens):
            for i in range(nq(L - M), nq(L)):
                bt[b, sp + i] = src[base + i]
            base += nq(L)
        dev = c["q"].device
        self.v_M = M
        self.v_bt = torch.tensor(bt, device=dev)
        self.v_lens = torch.tensor([L - M for L in lens], dtype=torch.int32, device=dev)
        from synth import normal

        B, Hq, D = c["B"], c["Hq"], lay["D"]
        self.v_q = normal(self.w["seed"], 60, B * M * Hq * D, device=dev).view(B, M, Hq, D).to(c["q"].dtype)
        self.v_out = torch.empty((B, M, Hq, D), dtype=torch.float32, device=dev)
        n = kv.decode_workspace_bytes_mq(self.L, B, M, Hq, c["max_pages"])
        self.v_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        rec = lambda bits: T * D * bits // 8 + 4 * T + 2 * D
        kinds = [lay["k_bits"]] if lay["mla"] else [lay["k_bits"], lay["v_bits"]]
        byts = 0
        for L in lens:
            n_q = nq(L - M)
            byts += n_q * lay["H"] * sum(rec(bb) for bb in kinds) + (L - n_q * T) * lay["H"] * D * 2 * len(kinds)
        byts += self.v_q.numel() * self.v_q.element_size() + self.v_out.numel() * 4
        self.v_bytes = byts

    def verify(self):
        c = self.case
        self.kv.decode_attn_mq(self.L, self.krec, self.vrec, c["k16"], c["v16"], self.v_bt, self.v_lens, self.v_q,
                               c["sm_scale"], out=self.v_out, workspace=self.v_ws)

    def time_verify(self, steps, warmup, flush):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(warmup + steps):
            flush()
            e0.record()
            self.verify()
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        st = stats(ts)
        return {"query_tokens": self.v_M, "us": round(st["median"], 2), "us_p10": round(st["p10"], 2),
                "us_p90": round(st["p90"], 2), "bytes": self.v_bytes,
                "GBs": round(self.v_bytes / st["median"] / 1e3, 1),
                "frac": round(self.v_bytes / st["median"] / 1e3 / HBM_PEAK_GBS, 4),
                "note": "verify step: M uncommitted query tokens per sequence, causal among themselves, one read of "
                        "the cache; bytes = cache + q + out"}

    def time_widths(self, pairs, steps, warmup, flush):
        """Quantize and decode of the same fp16 pages with other key/value code
        widths (3, 5 and 8 bits straddle or fill bytes; their quantize runs
        keys and values as two launches): per pair the same figures as the
        workload's own component."""
        torch, kv, c = self.torch, self.kv, self.case
        lay0, L0, k0, v0, b0 = c["layout"], self.L, self.krec, self.vrec, self.bytes
        H, nq = lay0["H"], max(c["n_qpages"], 1)
        dev = c["q"].device
        out = {}
        try:
            for kb, vb in pairs:
                lay = dict(lay0, k_bits=kb, v_bits=vb)
                c["layout"] = lay
                self.L = kv.layout_from_dict(lay)
                self.krec = torch.empty((nq, H, kv.record_bytes(self.L, 0)), dtype=torch.uint8, device=dev)
                self.vrec = torch.empty((nq, H, kv.record_bytes(self.L, 1)), dtype=torch.uint8, device=dev)
                self.bytes = byte_counts(c)
                tq, td = self.time_steps(steps, warmup, flush)
                comp = self.component(tq, td)
                out[f"k{kb}v{vb}"] = {"quantize": {k: comp["quantize"][k] for k in ("us", "us_p10", "us_p90",
                                                                                      "traffic_frac", "fp16_frac")},
                                      "decode": {k: comp["decode"][k] for k in ("us", "us_p10", "us_p90", "frac")}}
                del self.krec, self.vrec
        finally:
            c["layout"], self.L, self.krec, self.vrec, self.bytes = lay0, L0, k0, v0, b0
        return out

    def time_rope(self, steps, warmup, flush, R=64):
        """MLA decode of the same cache with an R-wide fp16 rope key beside
        every latent: seeded rope pools (the quantize call copies each
        quantized page's rope keys to its record page) and queries of
        D + R channels."""
        torch, kv, c = self.torch, self.kv, self.case
        from synth import QROPE_STREAM, ROPE_STREAM, normal, to_f16

        lay = c["layout"]
        T, D, B, Hq = lay["T"], lay["D"], c["B"], c["Hq"]
        dev = c["q"].device
        Lr = kv.layout_from_dict(dict(lay, rope=R))
        rope16 = to_f16(normal(self.w["seed"], ROPE_STREAM, c["n_fpages"] * T * R, device=dev)).view(-1, T, R)
        rrec = torch.empty((max(c["n_qpages"], 1), T, R), dtype=torch.float16, device=dev)
        kv.quantize(Lr, c["k16"], None, self.krec, None, c["src"], c["dst"], rope_fp16=rope16, rope_records=rrec)
        qr = normal(self.w["seed"], QROPE_STREAM, B * Hq * R, device=dev).view(B, Hq, R).to(c["q"].dtype)
        q = torch.cat([c["q"], qr], dim=2).contiguous()
        sm = 1.0 / math.sqrt(D + R)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(warmup + steps):
            flush()
            e0.record()
            kv.decode_attn(Lr, self.krec, None, c["k16"], None, c["block_table"], c["seq_lens"], q, sm, out=self.out,
                           workspace=self.ws, rope_records=rrec, rope_fp16=rope16)
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        st = stats(ts)
        _, _, dec, flops = self.bytes
        ntok = sum(c["seq_lens"].cpu().tolist())
        byts = dec + ntok * R * 2 + B * Hq * R * q.element_size()
        fl = flops + 2 * Hq * R * ntok   # one multiply-add per query head, rope channel and token (scores)
        tf = fl / st["median"] / 1e6
        return {"rope_dim": R, "us": round(st["median"], 2), "us_p10": round(st["p10"], 2),
                "us_p90": round(st["p90"], 2), "bytes": byts, "flops": fl, "bound": "mfma",
                "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                "GBs": round(byts / st["median"] / 1e3, 1), "frac": round(byts / st["median"] / 1e3 / HBM_PEAK_GBS, 4)}

    def free(self):
        del self.case, self.krec, self.vrec, self.out, self.ws
        for k in ("v_bt", "v_lens", "v_q", "v_out", "v_ws"):
            if hasattr(self, k):
                delattr(self, k)
        self.torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--component-steps", type=int, default=20,
                    help="timed calls per other workload of the suite (0: headline only)")
    ap.add_argument("--component-warmup", type=int, default=3)
    ap.add_argument("--verify-tokens", type=int, default=4,
                    help="query tokens per sequence of the headline workload's verify-step component (0: none)")
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
        print("bench.py measures one GPU: the path has no multi-GPU mode (each shard of a multi-GPU "
              "deployment runs this same single-GPU kernel); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.steps)
        return
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    flush_sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def flush():
        flush_sink.add_(flush_buf.sum())

    print(f"[bench] building {args.workload} on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    run = Runner(args.workload, dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tq, td = run.time_steps(args.steps, args.warmup, flush)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps of {args.workload}", file=sys.stderr, flush=True)

    q_fp16, q_out, dec_bytes, _ = run.bytes
    head = run.component(tq, td)
    sq, sd = stats(tq), stats(td)
    tq_med, td_med = sq["median"] * 1e-6, sd["median"] * 1e-6
    value = (q_fp16 + dec_bytes) / (tq_med + td_med) / 1e9
    ach = (q_fp16 + q_out) / (sq["mean"] * 1e-6) / 1e9
    case, lay, w = run.case, run.case["layout"], run.w
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / max(args.steps, 1) * 1e3, 4),
        "kernel_ms_per_step": round((tq_med + td_med) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if lay["mla"] else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": case["B"], "context": int(w["L"]), "q_heads": case["Hq"],
                   "kv_heads": lay["H"], "head_dim": lay["D"], "tile_tokens": lay["T"], "k_bits": lay["k_bits"],
                   "v_bits": None if lay["mla"] else lay["v_bits"], "iters": lay["n_iters"],
                   "sink": lay["sink"], "tail": lay["tail"], "mla": bool(lay["mla"])},
        "roofline": {"bound": "hbm", "kernel": "quantize_kernel", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": q_fp16 + q_out, "launch_us": round(sq["mean"], 2),
                     "launch_us_median": round(sq["median"], 2),
                     "traffic": recorded_traffic(args.workload)},
        "components": {args.workload: head},
    }
    if args.verify_tokens > 0:
        run.verify_setup(args.verify_tokens)
        res["components"][args.workload]["verify"] = run.time_verify(args.component_steps or 10, 3, flush)
        print(f"[bench] verify step with {args.verify_tokens} query tokens timed", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(run.case, run.krec, run.vrec, args.cpu_records, args.cpu_rows)
        print(f"[bench] oracle timed on the host", file=sys.stderr, flush=True)
    run.free()
    del run
    if args.component_steps > 0:
        for name in SUITE:
            if name == args.workload:
                continue
            r = Runner(name, dev)
            tq, td = r.time_steps(args.component_steps, args.component_warmup, flush)
            res["components"][name] = r.component(tq, td)
            if r.case["layout"]["mla"]:
                res["components"][name]["decode_rope64"] = r.time_rope(args.component_steps, args.component_warmup,
                                                                       flush)
            if name == WIDTHS_WORKLOAD:
                res["components"][name]["widths"] = r.time_widths(WIDTH_PAIRS, args.component_steps,
                                                                  args.component_warmup, flush)
            r.free()
            print(f"[bench] component {name} done", file=sys.stderr, flush=True)
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


def _threads():
    threads = len(os.sched_getaffinity(0))
    return min(threads, int(os.environ.get("OMP_NUM_THREADS", threads)))


def _oracle_quantize_sample(case, n_records, threads):
    """The oracle's quantize on the first records of the workload; returns
    (seconds, fp16 bytes consumed, records)."""
    import numpy as np
    import torch

    import oracle

    lay = case["layout"]
    T, D, H, mla = lay["T"], lay["D"], lay["H"], lay["mla"]
    kinds = 1 if mla else 2
    if n_records <= 0:
        n_records = case["n_qpages"] * H * kinds
    n_pages = max(1, min(case["n_qpages"], math.ceil(n_records / (H * kinds))))
    src = case["src"][:n_pages].cpu().numpy()
    pages = np.unique(src)
    remap = {int(p): i for i, p in enumerate(pages)}
    idx = torch.as_tensor(pages, device=case["k16"].device).long()
    k16 = case["k16"][idx].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    v16 = None if mla else case["v16"][idx].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    s_loc = np.array([remap[int(p)] for p in src], np.int32)
    d_loc = np.arange(n_pages, dtype=np.int32)
    rb = lambda b: T * D * b // 8 + 4 * T + 2 * D
    kr = np.zeros((n_pages, H, rb(lay["k_bits"])), np.uint8)
    vr = None if mla else np.zeros((n_pages, H, rb(lay["v_bits"])), np.uint8)
    t0 = time.perf_counter()
    oracle.quantize_pages(lay, k16, v16, s_loc, d_loc, kr, vr, n_threads=threads)
    return time.perf_counter() - t0, n_pages * H * T * D * 2 * kinds, n_pages * H * kinds


def cpu_baseline(case, krec, vrec, n_records, n_rows):
    """The oracle on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle

    lay = case["layout"]
    T, D, H, mla = lay["T"], lay["D"], lay["H"], lay["mla"]
    threads = _threads()
    kinds = 1 if mla else 2
    rb = lambda b: T * D * b // 8 + 4 * T + 2 * D
    tq, qbytes, nrec = _oracle_quantize_sample(case, n_records, threads)
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
    # one core: the oracle's quantize of the one-layer 1024-token case
    from synth.cases import WORKLOADS, make_case

    tiny = make_case(WORKLOADS["tiny_d128_k4v2"], device="cpu")
    t1, b1, n1 = _oracle_quantize_sample(tiny, 0, 1)
    return {"value": round((qbytes + dbytes) / (tq + td) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "quantize_GBs": round(qbytes / tq / 1e9, 4), "decode_GBs": round(dbytes / td / 1e9, 4),
            "seconds": round(tq + td, 2),
            "per_core": {"quantize_GBs": round(b1 / t1 / 1e9, 5), "cores": 1,
                         "sample": f"quantize all {n1} records of the one-layer 1024-token k4v2 case"},
            "sample": f"quantize {nrec} of {case['n_qpages'] * H * kinds} records; decode "
                      f"{n_rows} of {case['B'] * case['Hq']} (sequence, query head) rows on the GPU's records"}


if __name__ == "__main__":
    main()
