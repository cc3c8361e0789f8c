"""Benchmark: decode of a LLaMA-2-70B-shaped model, layer by layer, on one
MI355X.

Workload: 80 layers, each with q,o 8192x8192, k,v 1024x8192, gate,up
28672x8192, down 8192x28672 as Int8 codes (round(N(0, sigma)) clipped, sigma
~ U[0.8, 3.0] per layer and tensor) plus per-row fp32 scales. Every layer is
compressed (64-lane interleaved rANS, 65,536-symbol chunks) and all 80 stay
resident in HBM; one step decodes all 80 layers, one launch per layer, into
one reused bf16 layer buffer (decode happens before each block runs:
EntQuant, "Float8@2bits ...", technical summary §2 "Decodificación en Tiempo
de Inferencia"; per-block batching: DFloat11 write-up, "Descompresión por
bloque transformer").

Prints one JSON line (rank 0): decoded params/s over the timed steps, the
roofline of the decode kernel (algorithmic bytes per launch / mean launch
time from HIP events on the launch stream, against MI355X's 8 TB/s), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Hardware byte counts of the decode kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, calibrated against a plain copy), valid only for the kernel source
# they were taken with (its SHA-256 is stored beside them).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stream_bf16_llama2_70b_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "entropy_coded_weight_amd", "csrc", f)
                  for f in ("entq_decode.hip", "entq_stream.h")]
METRIC = "decoded params/s and achieved HBM GB/s (% of peak) for 70B-shaped layer decode"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=80,
                    help="layers in the model (80 is the workload; fewer only for quick checks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the untimed pass that compares every layer's GPU output with the "
                         "oracle (all host threads)")
    ap.add_argument("--cpu-sample-tensors", type=int, default=7,
                    help="tensors of layer 0 the oracle decodes for the CPU baseline "
                         "(7: the whole layer, about 7 s on one core)")
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--path", choices=("decode", "encode", "overlap", "fused", "lmhead", "adaptive",
                             "workloads"),
                    default="decode",
                    help="decode: the layer-by-layer decode (the headline line); encode: the "
                         "on-device encoder over 70B-shaped layers; overlap: decode of layer "
                         "l+1 overlapped with layer l's projection GEMMs; fused: decode and "
                         "product with m activation rows in one kernel vs decode + GEMM; lmhead: "
                         "the 32,000 x 8,192 output projection decoded on its own; adaptive: "
                         "per-chunk tables against shared tables; workloads: the smaller "
                         "workloads (and one 70B-shaped layer) each decoded alone")
    ap.add_argument("--tokens", type=str, default="",
                    help="activation rows per GEMM, comma-separated; the first value is the "
                         "line's (overlap default 2048,256,16; fused default 16,4,1,32,64)")
    ap.add_argument("--encode-layers", type=int, default=4,
                    help="resident layers of source codes the encode steps cycle through")
    ap.add_argument("--split-chunk-rows", type=int, default=1,
                    help="fused: rows per chunk of the lone BF16 8192 x 8192 split case")
    ap.add_argument("--row-chunk-max", type=int, default=8192,
                    help="fused: a chunk holds as many whole rows as fit in this many symbols "
                         "(at least one; 8192: one row of every 70B-shaped tensor per chunk)")
    ap.add_argument("--tile-cols", type=int, default=8192,
                    help="fused: columns per tile-ordered chunk (the widest multiple of 16 "
                         "dividing a tensor's columns that is at most this)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain fp32 negate (read N MiB, write N MiB) before timing, as a "
                         "known-size reference for hardware byte counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the decode has no cross-GPU step: each GPU decodes the chunks of its own shard", file=sys.stderr)
        sys.exit(2)
    if args.path == "encode":
        return bench_encode(args)
    if args.path == "overlap":
        return bench_overlap(args)
    if args.path == "fused":
        return bench_fused(args)
    if args.path == "lmhead":
        return bench_lm_head(args)
    if args.path == "adaptive":
        return bench_adaptive(args)
    if args.path == "workloads":
        return bench_workloads(args)
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    nthreads = args.threads or synth.default_threads()

    # ---------------------------------------------------------------- setup
    t0 = time.time()
    plans, blobs, scales = [], [], []
    host_layers = []  # per layer: the compressed batch and the scales, for the parity pass
    params_per_layer = 0
    layer_blob_bytes = []
    cpu_sample = None
    for layer in range(args.layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        b = E.encode_batch(specs, n_threads=nthreads)
        blob = torch.from_numpy(b.blob).to(dev)
        sc = torch.from_numpy(np.concatenate([s["scales"] for s in specs])).to(dev)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
        plans.append(p)
        blobs.append(blob)
        scales.append(sc)
        layer_blob_bytes.append(int(b.blob.size))
        params_per_layer = b.out_elems
        if not args.no_parity:
            host_layers.append((b, [(s["kind"], s["rows"], s["cols"], s["scales"]) for s in specs]))
        if layer == 0 and not args.no_cpu_baseline:
            cpu_sample = (specs[:args.cpu_sample_tensors], b)
        if layer % 10 == 0 or layer == args.layers - 1:
            log(f"layer {layer} ready ({time.time() - t0:.1f}s, {b.blob.size / 1e6:.1f} MB "
                f"compressed, {8.0 * b.blob.size / b.out_elems:.3f} bits/param)")
    torch.cuda.synchronize()
    n_chunks_layer = int(plans[0].n_chunks)
    scale_bytes_layer = int(scales[0].numel()) * 4
    out = torch.empty(params_per_layer, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        for layer in range(args.layers):
            if events is not None:
                events[layer][0].record(stream)
            E.decode(plans[layer], blobs[layer], out, E.OUT_BF16, scales[layer], None, stream)
            if events is not None:
                events[layer][1].record(stream)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibration_copy_mib} MiB read + written")
        del src, dst

    # ---------------------------------------------------------------- timing
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in range(args.layers)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(ev[s])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    launch_ms = np.array([[e[0].elapsed_time(e[1]) for e in ev[s]] for s in range(args.steps)])
    ms_per_step = total_ms / args.steps
    step_ms = launch_ms.sum(axis=1)  # per step: sum of its launches (HIP events)
    params_total = params_per_layer * args.layers
    value = params_total / (ms_per_step / 1e3)

    # algorithmic bytes of one launch (one layer): compressed payload (states,
    # words, padding) + scales read + bf16 written
    blob_mean = float(np.mean(layer_blob_bytes))
    alg_bytes_layer = blob_mean + scale_bytes_layer + 2.0 * params_per_layer
    mean_launch_s = float(launch_ms.mean()) / 1e3
    achieved_gbs = alg_bytes_layer / mean_launch_s / 1e9
    log(f"{args.steps} steps x {args.layers} layers: {ms_per_step:.3f} ms/step "
        f"(wall {1e3 * t_wall / args.steps:.3f}), launch mean {1e6 * mean_launch_s:.1f} us "
        f"p10 {1e3 * np.percentile(launch_ms, 10):.1f} p90 "
        f"{1e3 * np.percentile(launch_ms, 90):.1f} us, {achieved_gbs:.0f} GB/s")

    # ------------------------------------------- context: device-to-device copy
    copy_gbs = d2d_copy_gbs(out)

    # ---------------------------------------------------------- CPU baseline
    cpu = None
    if cpu_sample is not None:
        cpu = cpu_baseline(cpu_sample, plans[0], blobs[0], scales[0], out, stream)

    # ------------------------------------------- parity of every layer (untimed)
    parity = None
    if not args.no_parity:
        parity = parity_pass(plans, blobs, scales, host_layers, out, stream)
        if cpu is not None:
            cpu["all_threads"] = {
                "value": parity["oracle_params_per_s"], "unit": "params/s",
                "gbs": alg_bytes_layer * args.layers / parity["oracle_s"] / 1e9,
                "threads": parity["oracle_threads"],
                "sample": f"all {args.layers} layers ({parity['elements_compared']} params): the "
                          "same single-threaded oracle functions over disjoint row-aligned chunk "
                          "ranges, one range per thread at a time; time of the parity pass's "
                          "oracle phases"}

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32->bf16",
        "data": "synthetic (seeded int8 codes of the stated distribution; no trained weights)",
        "config": {
            "workload": "llama2-70b-shaped layer-by-layer decode, int8 rANS codes -> bf16 with per-row fp32 scale",
            "layers": args.layers,
            "params_per_layer": params_per_layer,
            "chunk_symbols": 65536,
            "chunks_per_layer": n_chunks_layer,
            "compressed_bytes_per_layer": blob_mean,
            "bits_per_param": 8.0 * blob_mean / params_per_layer,
            "algorithmic_bytes_per_layer": alg_bytes_layer,
            "hbm_gbs_whole_step": alg_bytes_layer * args.layers / (ms_per_step / 1e3) / 1e9,
            "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
            "launch_us_p10_p50_p90": [float(1e3 * np.percentile(launch_ms, q)) for q in (10, 50, 90)],
            "d2d_copy_gbs_context": copy_gbs,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)
    if parity is not None and parity["layers_bit_exact"] != parity["layers"]:
        raise SystemExit("GPU output differs from the oracle on "
                         f"{parity['layers'] - parity['layers_bit_exact']} layers")


def host_cpu():
    """(os.cpu_count(), CPU model string from /proc/cpuinfo)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count(), model


def parity_pass(plans, blobs, scales, host_layers, out, stream):
    """Decodes every layer again, in the timed launch configuration plus a
    per-chunk status buffer, copies the bf16 output to the host and has the
    oracle (decode + dequant of the same compressed bytes, fanned out over
    the host's threads) compare every element. Returns the record."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    import entropy_coded_weight_amd as E
    from oracle import fanout

    threads = fanout.default_threads()
    pinned = torch.empty(out.numel(), dtype=torch.int16, pin_memory=True)
    host_out = pinned.numpy().view(np.uint16)
    n_layers = len(host_layers)
    exact = mismatches = bad = status_bad = elems = 0
    first_bad = None
    oracle_s = 0.0
    t_all = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool, ThreadPoolExecutor(8) as drivers:
        for layer, (b, tens) in enumerate(host_layers):
            status = torch.full((b.chunks.size,), -7, dtype=torch.int32, device=out.device)
            E.decode(plans[layer], blobs[layer], out, E.OUT_BF16, scales[layer], status, stream)
            pinned.copy_(out, non_blocking=True)
            st = status.cpu().numpy()  # waits for the decode and the copy
            t0 = time.perf_counter()
            jobs = []
            for t, (kind, rows, cols, sc) in enumerate(tens):
                ch = b.chunks[b.chunks["tensor"] == t]
                ch = ch[np.argsort(ch["elem_offset"])]
                desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"],
                                 ch["elem_offset"]], axis=1).astype(np.uint64)
                o = int(b.tensors[t]["out_elem_offset"])
                jobs.append(drivers.submit(fanout.tensor_bf16, b.blob, desc, b.freq[t], kind,
                                           rows, cols, sc, threads,
                                           host_out[o:o + rows * cols], None, False, pool))
            res = [j.result() for j in jobs]
            oracle_s += time.perf_counter() - t0
            lm = sum(r.mismatches for _, r in res)
            lb = sum(r.bad_chunks for _, r in res)
            ls = int(np.count_nonzero(st != 0))
            mismatches += lm
            bad += lb
            status_bad += ls
            elems += int(b.out_elems)
            if lm == 0 and lb == 0 and ls == 0:
                exact += 1
            elif first_bad is None:
                first_bad = layer
            if layer % 10 == 0 or layer == n_layers - 1:
                log(f"parity: layer {layer} {'bit-exact' if lm == lb == ls == 0 else 'DIFFERS'} "
                    f"({exact}/{layer + 1} so far, {time.perf_counter() - t_all:.1f}s)")
    wall = time.perf_counter() - t_all
    cores, model = host_cpu()
    log(f"parity: {exact}/{n_layers} layers bit-exact, {elems} elements, oracle {oracle_s:.1f}s "
        f"on {threads} threads ({elems / oracle_s / 1e6:.0f} M params/s)")
    return {"layers": n_layers, "layers_bit_exact": exact, "elements_compared": elems,
            "mismatches": mismatches, "bad_chunks": bad, "status_nonzero": status_bad,
            "first_differing_layer": first_bad, "oracle_threads": threads,
            "oracle_s": oracle_s, "wall_s": wall, "oracle_params_per_s": elems / oracle_s,
            "host_cores": cores, "cpu_model": model,
            "what": "every bf16 output of every layer, decoded on the GPU in the timed launch "
                    "configuration with a status buffer, equals the oracle's decode + dequant of "
                    "the same compressed bytes; every chunk status is 0"}


def d2d_copy_gbs(buf):
    """Bandwidth of a plain device-to-device copy of the layer buffer (read +
    write bytes / time, median of 5), as context for the decode's GB/s."""
    import torch
    other = torch.empty_like(buf)
    times = []
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        other.copy_(buf)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    del other
    return 2.0 * buf.numel() * buf.element_size() / float(np.median(times[1:])) / 1e9


def kernel_sources_sha256():
    """SHA-256 over the decode kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter record, or None when
    the kernel source has changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        digest = kernel_sources_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256") != digest:
        return None
    return float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])


def cpu_baseline(sample, plan0, blob0, scales0, out_gpu, stream):
    """The oracle (single-threaded C) decoding + dequantising the first
    tensors of layer 0 from the same compressed bytes, timed on this host.
    Its output is also compared with the GPU's for those tensors."""
    import torch

    import entropy_coded_weight_amd as E
    import oracle

    specs, b = sample
    E.decode(plan0, blob0, out_gpu, E.OUT_BF16, scales0, None, stream)
    torch.cuda.synchronize()
    n_sample = sum(s["rows"] * s["cols"] for s in specs)
    gpu = out_gpu[:n_sample].cpu().numpy().view(np.uint16)
    t = time.perf_counter()
    outs = []
    for ti, sp in enumerate(specs):
        sel = b.chunks["tensor"] == ti
        ch = b.chunks[sel]
        desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                        axis=1).astype(np.uint64)
        sym, st = oracle.decode_tensor(b.blob, desc, b.freq[ti], sp["rows"] * sp["cols"])
        assert np.all(st == 0)
        outs.append(oracle.dequant_tensor(sym, sp["rows"], sp["cols"], sp["kind"], sp["scales"]))
    dt = time.perf_counter() - t
    # the same byte accounting as the GPU line: compressed regions, scales, bf16 written
    comp = 0
    for ti in range(len(specs)):
        nw = b.chunks[b.chunks["tensor"] == ti]["n_words"].astype(np.int64)
        comp += int(np.sum((256 + 2 * nw + 15) // 16 * 16))
    alg = comp + 4 * sum(int(s["rows"]) for s in specs) + 2 * n_sample
    ok = bool(np.array_equal(np.concatenate(outs), gpu))
    log(f"cpu oracle: {n_sample} params in {dt:.2f}s ({n_sample / dt / 1e6:.1f} M params/s); "
        f"matches GPU: {ok}")
    if not ok:
        raise SystemExit("GPU output differs from the oracle on the CPU-baseline sample")
    cores, model = host_cpu()
    return {"value": n_sample / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, first {len(specs)} tensors ({n_sample} params): single-threaded "
                      "C oracle rANS decode + fp32 dequant + RNE bf16 from the same compressed bytes",
            "gbs": alg / dt / 1e9, "sample_seconds": dt,
            "x80_layers_seconds_extrapolated": dt * 80.0 * (plan0.out_elems / n_sample),
            "host_cores": cores, "cpu_model": model}


ENCODE_METRIC = "encoded symbols/s for 70B-shaped layer encode on the GPU (counts, rANS encode, layout, pack)"


def bench_encode(args):
    """One step = the on-device encoder over one 70B-shaped layer (855.6 M
    int8 codes, 7 tensors, 65,536-symbol chunks), resident in HBM: byte
    counts, frequency tables, 64-lane rANS encode, region layout and
    packing, ending with the chunk index on the host. The steps cycle over
    --encode-layers layers. The roofline entry is the encode kernel's:
    algorithmic bytes = symbols read + final states and words written."""
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    nthreads = args.threads or synth.default_threads()
    layers, host_layer0 = [], None
    t0 = time.time()
    for layer in range(args.encode_layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        if layer == 0:
            host_layer0 = specs
        layers.append([dict(sp, symbols=torch.from_numpy(
            np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()).to(dev)) for sp in specs])
        log(f"encode: layer {layer} resident ({time.time() - t0:.1f}s)")
    n_layer = sum(sp["symbols"].numel() for sp in layers[0])
    stream = torch.cuda.current_stream()
    for w in range(args.warmup):
        E.encode_batch_device(layers[w % len(layers)], stream)
    torch.cuda.synchronize()
    events, wall, comp = [], [], []
    for st in range(args.steps):
        ev = []
        t = time.perf_counter()
        b = E.encode_batch_device(layers[st % len(layers)], stream, events=ev)
        wall.append(time.perf_counter() - t)
        comp.append(int(b.blob.numel()))
        events.append(ev)
        del b
    torch.cuda.synchronize()
    ms_per_step = 1e3 * float(np.mean(wall))
    value = n_layer / (ms_per_step / 1e3)
    per_kind = {}
    for ev in events:
        for name, a, z in ev:
            per_kind.setdefault(name, []).append(a.elapsed_time(z) * 1e3)
    # per step, kernel microseconds by kind; encode launches per tensor
    kind_us = {k: float(np.sum(v)) / args.steps for k, v in per_kind.items()}
    enc_us = np.array(per_kind["encode"])
    n_t = len(layers[0])
    comp_mean = float(np.mean(comp))
    # encode kernel: reads every symbol once, writes 64 states + the words of
    # each chunk (the compressed bytes minus the regions' zero padding ~ the
    # blob); counted per step over its n_t launches.
    enc_bytes_step = n_layer + comp_mean
    enc_gbs = enc_bytes_step / (kind_us["encode"] / 1e6) / 1e9
    log(f"encode: {ms_per_step:.2f} ms/step wall, kernels per step (us): "
        + ", ".join(f"{k} {v:.0f}" for k, v in kind_us.items())
        + f"; encode {n_layer / kind_us['encode'] / 1e6:.3f} T sym/s, {enc_gbs:.0f} GB/s")
    # the same layers with per-chunk tables (counts per chunk, tables on the host)
    E.encode_batch_device_adaptive(layers[0], stream)
    torch.cuda.synchronize()
    ad_wall, ad_kinds, ad_comp = [], {}, []
    for st in range(args.steps):
        ev = []
        t = time.perf_counter()
        b = E.encode_batch_device_adaptive(layers[st % len(layers)], stream, events=ev)
        ad_wall.append(time.perf_counter() - t)
        ad_comp.append(int(b.blob.numel()))
        for name, a_, z_ in ev:
            ad_kinds.setdefault(name, []).append(a_.elapsed_time(z_) * 1e3)
        del b
    ad_kind_us = {k: float(np.sum(v)) / args.steps for k, v in ad_kinds.items()}
    per_chunk = {"ms_per_step_wall": 1e3 * float(np.mean(ad_wall)),
                 "kernel_us_per_step": ad_kind_us,
                 "compressed_bytes_per_layer": float(np.mean(ad_comp))}
    log(f"encode, per-chunk tables: {per_chunk['ms_per_step_wall']:.2f} ms/step wall, kernels "
        "per step (us): " + ", ".join(f"{k} {v:.0f}" for k, v in ad_kind_us.items()))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = encode_cpu_baseline(host_layer0[1:3], layers[0][1:3], stream)
    rec = {
        "metric": ENCODE_METRIC,
        "value": value,
        "unit": "symbols/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8->u16 words+u32 states",
        "data": "synthetic (seeded int8 codes of the stated distribution; no trained weights)",
        "config": {
            "workload": "llama2-70b-shaped layer encode, int8 codes -> rANS container, 65,536-symbol chunks",
            "layers_cycled": len(layers),
            "symbols_per_layer": n_layer,
            "compressed_bytes_per_layer": comp_mean,
            "kernel_us_per_step": kind_us,
            "encode_launch_us_p10_p50_p90": [float(np.percentile(enc_us, q)) for q in (10, 50, 90)],
            "step_ms_wall_p10_p50_p90": [1e3 * float(np.percentile(wall, q)) for q in (10, 50, 90)],
            "note": "value is wall time per layer including the final host read of the word "
                    "counts, offsets and tables; counts, tables, encode, offsets and packing all "
                    "run on the GPU",
            "per_chunk_tables": per_chunk,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": enc_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": enc_gbs / HBM_PEAK_GBS,
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def encode_cpu_baseline(specs, dspecs, stream):
    """The oracle encoder (single-threaded C: counts, table, 64-lane rANS,
    layout) over the given tensors, timed on this host; its blob must equal
    the device encoder's for the same tensors."""
    import entropy_coded_weight_amd as E
    import oracle

    t = time.perf_counter()
    c = oracle.encode_container(specs)
    dt = time.perf_counter() - t
    n = sum(int(np.asarray(sp["symbols"]).size) for sp in specs)
    d = E.encode_batch_device(dspecs, stream)
    ok = bool(d.blob.numel() == c.blob.size and np.array_equal(d.blob.cpu().numpy(), c.blob))
    log(f"cpu oracle encode: {n} symbols in {dt:.2f}s ({n / dt / 1e6:.1f} M sym/s); "
        f"matches GPU: {ok}")
    if not ok:
        raise SystemExit("device encoder differs from the oracle on the CPU-baseline sample")
    return {"value": n / dt, "unit": "symbols/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, tensors k and v ({n} symbols): single-threaded C oracle "
                      "counts + frequency table + 64-lane rANS encode + container layout"}


OVERLAP_METRIC = ("tokens/s through the 80-layer 70B-shaped projection stack with each layer's "
                  "decode overlapped with the previous layer's GEMMs")


def bench_overlap(args):
    """One step = one pass over the 80 layers: decode layer l (entq_decode,
    bf16, into one of two layer buffers) and run layer l's seven projection
    GEMMs (torch.mm on bf16: q,k,v,gate,up from X [T, 8192], o from an
    [T, 8192] and down from an [T, 28672] activation, all synthetic) on the
    decoded weights. Four schedules are timed: decode only, GEMMs only,
    serial (one stream: decode, GEMMs, next layer) and overlapped (decode of
    l+1 on its own stream during l's GEMMs). Compressed layers are built by
    the on-device encoder."""
    import torch

    import entropy_coded_weight_amd as E
    import synth
    from entropy_coded_weight_amd.layer_pipeline import LayerPipeline

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    nthreads = args.threads or synth.default_threads()
    t0 = time.time()
    layers, out_elems, tens = [], 0, None
    for layer in range(args.layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        ds = [dict(sp, symbols=torch.from_numpy(
            np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()).to(dev)) for sp in specs]
        b = E.encode_batch_device(ds)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.numel())
        sc = torch.from_numpy(np.concatenate([s_["scales"] for s_ in specs])).to(dev)
        layers.append((p, b.blob.clone(), sc))
        out_elems, tens = b.out_elems, b.tensors
        del ds, b
        if layer % 10 == 0 or layer == args.layers - 1:
            log(f"overlap: layer {layer} encoded on the device ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    pipe = LayerPipeline(layers, out_elems, dev)
    names = [n for n, _, _ in synth.LLAMA2_70B_LAYER]
    views = [(names[t], int(tens["rows"][t]), int(tens["cols"][t]), int(tens["out_elem_offset"][t]))
             for t in range(len(tens))]
    gen = torch.Generator().manual_seed(0)
    results = []
    for T in [int(v) for v in (args.tokens or "2048,256,16").split(",") if v]:
        X = (torch.randn(T, 8192, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        H = (torch.randn(T, 28672, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        Y = {n: torch.empty(T, r, dtype=torch.bfloat16, device=dev) for n, r, c, o in views}

        def consume(layer, W):
            for n, r, c, o in views:
                torch.mm(H if n == "down" else X, W[o:o + r * c].view(r, c).t(), out=Y[n])

        def decode_only():
            s = pipe.decode_stream
            for layer in range(len(layers)):
                p_, blob, sc_ = layers[layer]
                E.decode(p_, blob, pipe.buffers[layer % 2], E.OUT_BF16, sc_, None, s)
            return s

        def gemm_only():
            with torch.cuda.stream(pipe.compute_stream):
                for layer in range(len(layers)):
                    consume(layer, pipe.weights(layer % 2))
            return pipe.compute_stream

        def serial():
            pipe.run_serial(consume)
            return pipe.compute_stream

        def overlapped():
            pipe.run_overlapped(consume)
            return pipe.compute_stream

        row = {"tokens": T}
        for name, fn in (("decode_only", decode_only), ("gemm_only", gemm_only),
                         ("serial", serial), ("overlapped", overlapped)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            row[name + "_ms"] = 1e3 * (time.perf_counter() - t) / args.steps
        row["decode_hidden_frac"] = ((row["serial_ms"] - row["overlapped_ms"]) /
                                     row["decode_only_ms"])
        row["gemm_tflops"] = 2.0 * out_elems * T * len(layers) / (row["gemm_only_ms"] / 1e3) / 1e12
        log(f"overlap T={T}: " + ", ".join(f"{k} {v:.3f}" for k, v in row.items() if k != "tokens"))
        results.append(row)
        del X, H, Y
    r0 = results[0]
    ms = r0["overlapped_ms"]
    rec = {
        "metric": OVERLAP_METRIC,
        "value": r0["tokens"] / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded int8 codes of the stated distribution and random bf16 activations; no trained weights)",
        "config": {
            "workload": "llama2-70b-shaped 80-layer projection stack: per layer entq_decode to bf16 + 7 torch.mm GEMMs",
            "layers": args.layers,
            "params_per_layer": out_elems,
            "schedules": results,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": r0["gemm_tflops"],
            "peak": 2500.0,
            "unit": "TFLOP/s",
            "frac": r0["gemm_tflops"] / 2500.0,
            "traffic": None,
            "kernel": "the library bf16 GEMMs (torch.mm) of the GEMM-only schedule",
        },
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


FUSED_METRIC = ("tokens/s through the 80-layer 70B-shaped projection stack with each layer's "
                "weights decoded inside the GEMM (entq_decode_gemm_tiles, tile-ordered chunks)")


def oracle_tensor_sample(blob, chunks, freq, spec, n_chunks):
    """The oracle decoding + dequantising the first n_chunks chunks of one
    tensor (shared tables; chunks: that tensor's CHUNK_DESC rows, byte
    offsets into blob) to bf16 bits. Returns (bits, seconds, elements);
    the chunks hold whole rows or the rows they touch are completed with
    zeros before the dequantiser."""
    import oracle
    ch = np.sort(chunks, order="elem_offset")[:n_chunks]
    desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                    axis=1).astype(np.uint64)
    n = int(ch["elem_offset"][-1]) + int(ch["n_symbols"][-1])
    t = time.perf_counter()
    sym, st = oracle.decode_tensor(blob, desc, freq, n)
    assert (st == 0).all()
    cols = int(spec["cols"])
    rows = -(-n // cols)
    full = np.zeros(rows * cols, np.uint8)
    full[:n] = sym
    bits = oracle.dequant_tensor(full, rows, cols, spec["kind"], spec["scales"][:rows])[:n]
    return bits, time.perf_counter() - t, n


def compressed_layers_row_aligned(args, E, synth, dev, torch, row_chunk_max=None):
    """The 80 layers encoded on the device with chunks of whole rows, as many
    as fit in row_chunk_max symbols (at least one), as the fused kernel
    needs."""
    nthreads = args.threads or synth.default_threads()
    rcm = row_chunk_max or args.row_chunk_max
    t0 = time.time()
    layers, out_elems, tens, meta0 = [], 0, None, None
    for layer in range(args.layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        for sp in specs:
            sp["chunk_symbols"] = sp["cols"] * max(1, rcm // sp["cols"])
        ds = [dict(sp, symbols=torch.from_numpy(
            np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()).to(dev)) for sp in specs]
        b = E.encode_batch_device(ds)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.numel())
        sc = torch.from_numpy(np.concatenate([s_["scales"] for s_ in specs])).to(dev)
        layers.append((p, b.blob.clone(), sc))
        out_elems, tens = b.out_elems, b.tensors
        if layer == 0:
            meta0 = (b.chunks, b.freq, [dict(sp, symbols=None) for sp in specs])
        del ds, b
        if layer % 10 == 0 or layer == args.layers - 1:
            log(f"layer {layer} encoded on the device, row-aligned chunks of at most {rcm} "
                f"symbols ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return layers, out_elems, tens, meta0


def tile_cols(cols, target):
    """Columns per tile-ordered chunk: the widest multiple of 16 that divides
    cols and is at most target."""
    for k in range(1, cols + 1):
        if cols % k == 0 and (cols // k) % 16 == 0 and cols // k <= target:
            return cols // k
    raise ValueError(f"no tile width for {cols} columns")


def compressed_layers_tiled(args, E, synth, dev, torch, target):
    """The 80 layers in tile order (chunks of 16 rows x tile_cols(cols,
    target) columns), put in order and encoded on the device."""
    nthreads = args.threads or synth.default_threads()
    t0 = time.time()
    layers, meta0 = [], None
    for layer in range(args.layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        ds = []
        for sp in specs:
            C = tile_cols(sp["cols"], target)
            src = torch.from_numpy(np.ascontiguousarray(sp["symbols"]).view(np.uint8)).to(dev)
            st = E.tile_order_device(src, sp["rows"], sp["cols"], C)
            ds.append(dict(sp, symbols=st, chunk_symbols=16 * C, C=C,
                           kind=sp["kind"] | E.LAYOUT_TILES))
            del src
        b = E.encode_batch_device(ds)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.numel())
        sc = torch.from_numpy(np.concatenate([s_["scales"] for s_ in specs])).to(dev)
        layers.append((p, b.blob.clone(), sc))
        if layer == 0:
            meta0 = (b.chunks, b.freq, [dict(sp, symbols=None) for sp in ds])
        del ds, b
        if layer % 10 == 0 or layer == args.layers - 1:
            log(f"layer {layer} encoded on the device in tile order, chunks of 16 rows x at most "
                f"{target} columns ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return layers, meta0


def bench_fused(args):
    """One step = one pass over the 80 layers computing every projection
    Y = X . W^T (q,k,v,gate,up from X [m, 8192], o from an [m, 8192] and down
    from an [m, 28672] activation, synthetic bf16) for m activation rows.
    Fused: one entq_decode_gemm_tiles call per layer (fp32 Y, the bf16
    weights never written) on the layers in tile order, chunks of 16 rows x
    at most --tile-cols columns (8,192 columns; 7,168 for the down
    projection). Beside it the row-major fused call, entq_decode_gemm, on a
    container of one-row chunks (--row-chunk-max): matrix cores in 16-chunk
    lockstep for m > 4, the vector units inside the decode loop for m <= 4.
    Unfused: entq_decode into a bf16 layer buffer, then seven torch.mm (bf16
    Y), on the container the decode runs fastest on (whole rows in chunks of
    at most 65,536 symbols, as the layer-decode line's). HIP events around
    every launch on the one stream."""
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    rows_layers, out_elems, tens, _ = compressed_layers_row_aligned(args, E, synth, dev, torch)
    dec_layers = compressed_layers_row_aligned(args, E, synth, dev, torch, 65536)[0]
    layers, meta0 = compressed_layers_tiled(args, E, synth, dev, torch, args.tile_cols)
    names = [n for n, _, _ in synth.LLAMA2_70B_LAYER]
    views = [(names[t], int(tens["rows"][t]), int(tens["cols"][t]), int(tens["out_elem_offset"][t]))
             for t in range(len(tens))]
    blob_mean = float(np.mean([l[1].numel() for l in layers]))
    scale_bytes = 4.0 * int(layers[0][2].numel())
    buf = torch.empty(out_elems, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    gen = torch.Generator().manual_seed(0)
    results = []
    for m in [int(v) for v in (args.tokens or "16,4,2,1,32,64").split(",") if v]:
        X = (torch.randn(m, 8192, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        H = (torch.randn(m, 28672, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        xs = [H if n == "down" else X for n, r, c, o in views]
        ys = [torch.empty(m, r, dtype=torch.float32, device=dev) for n, r, c, o in views]
        yb = [torch.empty(m, r, dtype=torch.bfloat16, device=dev) for n, r, c, o in views]

        ws_n = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(layers[0][0].handle, m))
        ws_raw = torch.empty(ws_n + 256, dtype=torch.uint8, device=dev)
        ws_at = (-ws_raw.data_ptr()) % 256
        ws = ws_raw[ws_at:ws_at + ws_n] if ws_n else None

        def fused(ev=None):
            for li, (p_, blob, sc_) in enumerate(layers):
                if ev is not None:
                    ev[li][0].record(stream)
                E.decode_gemm_tiles(p_, blob, sc_, xs, ys, None, stream, ws)
                if ev is not None:
                    ev[li][1].record(stream)

        def fused_row_chunks(ev=None):
            for li, (p_, blob, sc_) in enumerate(rows_layers):
                if ev is not None:
                    ev[li][0].record(stream)
                E.decode_gemm(p_, blob, sc_, xs, ys, None, stream)
                if ev is not None:
                    ev[li][1].record(stream)

        def unfused(ev=None):
            W = buf.view(torch.bfloat16)
            for li, (p_, blob, sc_) in enumerate(dec_layers):
                if ev is not None:
                    ev[li][0].record(stream)
                E.decode(p_, blob, buf, E.OUT_BF16, sc_, None, stream)
                for (n, r, c, o), x, y in zip(views, xs, yb):
                    torch.mm(x, W[o:o + r * c].view(r, c).t(), out=y)
                if ev is not None:
                    ev[li][1].record(stream)

        def decode_only(ev=None):
            for li, (p_, blob, sc_) in enumerate(dec_layers):
                if ev is not None:
                    ev[li][0].record(stream)
                E.decode(p_, blob, buf, E.OUT_BF16, sc_, None, stream)
                if ev is not None:
                    ev[li][1].record(stream)

        row = {"m": m}
        for name, fn in (("fused", fused), ("fused_row_chunks", fused_row_chunks),
                         ("unfused", unfused), ("decode_only", decode_only)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                   for _ in layers] for _ in range(args.steps)]
            t = time.perf_counter()
            for st in range(args.steps):
                fn(ev[st])
            torch.cuda.synchronize()
            row[name + "_ms_per_step"] = 1e3 * (time.perf_counter() - t) / args.steps
            lay = np.array([[e[0].elapsed_time(e[1]) for e in ev[st]] for st in range(args.steps)])
            row[name + "_us_per_layer"] = float(1e3 * lay.mean())
        row["speedup"] = row["unfused_ms_per_step"] / row["fused_ms_per_step"]
        log(f"fused m={m}: " + ", ".join(f"{k} {v:.3f}" for k, v in row.items() if k != "m"))
        results.append(row)
        del X, H, xs, ys, yb, ws, ws_raw
    split = fused_bf16_split_case(E, synth, torch, dev, stream, args)
    split_m1 = fused_bf16_split_case(E, synth, torch, dev, stream, args, m=1)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = fused_cpu_baseline(E, layers[0], meta0, views, stream, torch, dev)
    r0 = results[0]
    # algorithmic bytes of one fused launch: compressed layer + scales + the
    # activations read + the fp32 results written
    m0 = r0["m"]
    act_bytes = 2.0 * m0 * (8192 * 6 + 28672)
    y_bytes = 4.0 * m0 * sum(r for n, r, c, o in views)
    alg = blob_mean + scale_bytes + act_bytes + y_bytes
    gbs = alg / (r0["fused_us_per_layer"] / 1e6) / 1e9
    rec = {
        "metric": FUSED_METRIC,
        "value": m0 / (r0["fused_ms_per_step"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r0["fused_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 codes -> bf16 weights x bf16 activations, fp32 accumulation",
        "data": "synthetic (seeded int8 codes of the stated distribution and random bf16 activations; no trained weights)",
        "config": {
            "workload": "llama2-70b-shaped 80-layer projection stack, m activation rows, fused decode+GEMM vs decode then torch.mm",
            "layers": args.layers,
            "params_per_layer": out_elems,
            "compressed_bytes_per_layer": blob_mean,
            "chunking": f"fused: tile order, chunks of 16 rows x at most {args.tile_cols} "
                        "columns (the widest multiple of 16 dividing the tensor's columns); "
                        f"fused_row_chunks: whole rows, at most {args.row_chunk_max} symbols "
                        "per chunk (at least one row); unfused and decode only: whole rows, at "
                        "most 65,536 symbols per chunk",
            "fused_row_chunks_compressed_bytes_per_layer": float(np.mean([l[1].numel()
                                                                          for l in rows_layers])),
            "unfused_compressed_bytes_per_layer": float(np.mean([l[1].numel()
                                                                 for l in dec_layers])),
            "results": results,
            "bf16_split_8192x8192": split,
            "bf16_split_8192x8192_m1": split_m1,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


LMHEAD_METRIC = "decoded params/s for the LLaMA-2-70B output projection (32,000 x 8,192) decoded alone"


def fused_bf16_split_case(E, synth, torch, dev, stream, args, m=16, chunk_rows=None):
    """BF16 weights 8192 x 8192 stored as a coded exponent stream + raw
    sign+mantissa bytes (chunk_rows-row chunks: a tensor on its own needs
    enough chunks to fill the GPU, 16 per fused workgroup), m activation
    rows: fused
    (entq_decode_gemm_bf16_split) against entq_decode_bf16_split + torch.mm,
    and the split decode alone; medians of per-launch HIP events."""
    rows = cols = 8192
    w = synth.bf16_weights(rows, cols)[0]["bf16"]
    e, sm = E.bf16_split(w)
    chunk_rows = chunk_rows or args.split_chunk_rows
    b = E.encode_batch([dict(kind=E.KIND_BF16EXP, rows=rows, cols=cols, symbols=e,
                             chunk_symbols=cols * chunk_rows)])
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).to(dev)
    smd = torch.from_numpy(sm).to(dev)
    out = torch.empty(rows * cols, dtype=torch.int16, device=dev)
    X = (torch.randn(m, cols, generator=torch.Generator().manual_seed(2)) * 0.5).to(
        torch.bfloat16).to(dev)
    Y = torch.empty(m, rows, dtype=torch.float32, device=dev)
    Yb = torch.empty(m, rows, dtype=torch.bfloat16, device=dev)
    W = out.view(torch.bfloat16).view(rows, cols)

    def med(fn, reps=max(args.steps, 20)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, z in ev:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(z) for a, z in ev])) * 1e3

    def unfused():
        E.decode_bf16_split(p, blob, smd, out, None, stream)
        torch.mm(X, W.t(), out=Yb)

    r = {"m": m, "chunk_rows": chunk_rows, "compressed_exponent_bytes": int(b.blob.size),
         "fused_us": med(lambda: E.decode_gemm_bf16_split(p, blob, smd, [X], [Y], None, stream)),
         "unfused_us": med(unfused),
         "split_decode_only_us": med(lambda: E.decode_bf16_split(p, blob, smd, out, None, stream))}
    r["speedup"] = r["unfused_us"] / r["fused_us"]
    # the same weights in tile order (exponents and sign+mantissa bytes), chunks
    # of 16 rows x Ct columns (a tensor alone must fill the GPU with its chunks)
    for Ct in (512, 1024, 2048):
        e_t, sm_t = E.tile_order(e, rows, cols, Ct), E.tile_order(sm, rows, cols, Ct)
        bt = E.encode_batch([dict(kind=E.KIND_BF16EXP | E.LAYOUT_TILES, rows=rows, cols=cols,
                                  symbols=e_t, chunk_symbols=16 * Ct)])
        pt = E.plan(bt.tensors, bt.freq, bt.chunks, bt.blob.size)
        blob_t = torch.from_numpy(bt.blob).to(dev)
        sm_td = torch.from_numpy(sm_t).to(dev)
        n_ws = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(pt.handle, m))
        raw = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
        ws = raw[(-raw.data_ptr()) % 256:][:n_ws]
        r[f"tiles_{Ct}_fused_us"] = med(lambda: E.decode_gemm_tiles_bf16_split(
            pt, blob_t, sm_td, [X], [Y], None, stream, ws))
        pt.close()
    log(f"bf16 split 8192x8192 m={m}: fused {r['fused_us']:.1f} us (tile order, 512 / 1024 / "
        f"2048 columns per chunk: {r['tiles_512_fused_us']:.1f} / {r['tiles_1024_fused_us']:.1f} "
        f"/ {r['tiles_2048_fused_us']:.1f} us), split decode + GEMM {r['unfused_us']:.1f} us, "
        f"split decode alone {r['split_decode_only_us']:.1f} us")
    p.close()
    return r


def fused_cpu_baseline(E, layer0, meta0, views, stream, torch, dev, m=16, n_tensors=4):
    """The oracle (single-threaded C decode of the tile-ordered chunks, the
    inverse of the tile order, C dequant, then a one-thread fp64 product) for
    the first n_tensors tensors of layer 0 and m = 16 activation rows, timed
    on this host; the GPU's fused results for the same tensors must lie
    within the fp32 accumulation bound of it."""
    import oracle
    from threadpoolctl import threadpool_limits
    p0, blob_d, sc_d = layer0
    chunks, freq, specs = meta0
    blob = blob_d.cpu().numpy()
    gen = torch.Generator().manual_seed(1)
    X = (torch.randn(m, 8192, generator=gen) * 0.5).to(torch.bfloat16)
    H = (torch.randn(m, 28672, generator=gen) * 0.5).to(torch.bfloat16)
    xs = [(H if n == "down" else X).to(dev) for n, r, c, o in views]
    ys = [torch.empty(m, r, dtype=torch.float32, device=dev) for n, r, c, o in views]
    E.decode_gemm_tiles(p0, blob_d, sc_d, xs, ys, None, stream)
    torch.cuda.synchronize()
    xf = X.float().numpy().astype(np.float64)
    spent, params, ok = 0.0, 0, True
    with threadpool_limits(1):
        for t in range(n_tensors):
            sp = specs[t]
            rows, cols = int(sp["rows"]), int(sp["cols"])
            ch = np.sort(chunks[chunks["tensor"] == t], order="elem_offset")
            desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"],
                             ch["elem_offset"]], axis=1).astype(np.uint64)
            t0 = time.perf_counter()
            sym, st = oracle.decode_tensor(blob, desc, freq[t], rows * cols)
            codes = oracle.untile(sym, rows, cols, int(sp["C"]))
            bits = oracle.dequant_tensor(codes.ravel(), rows, cols, sp["kind"] & 0xFF,
                                         sp["scales"])
            w = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            w = w.reshape(rows, cols)
            ref = xf @ w.T
            spent += time.perf_counter() - t0
            assert (st == 0).all()
            bound = cols * 2.0 ** -24 * (np.abs(xf) @ np.abs(w).T)
            ok &= bool((np.abs(ys[t].cpu().numpy() - ref) <= bound).all())
            params += rows * cols
    log(f"cpu oracle, fused sample: {params} weights x {m} rows in {spent:.2f}s "
        f"({params / spent / 1e6:.1f} M weights/s); GPU within bound: {ok}")
    if not ok:
        raise SystemExit("fused results differ from the oracle beyond the accumulation bound")
    return {"value": params / spent, "unit": "weights/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, first {n_tensors} tensors ({params} weights, tile order), "
                      f"m = {m}: single-threaded C oracle decode + inverse tile order + "
                      "dequant, fp64 product on one thread"}


def bench_lm_head(args):
    """A single large tensor decoded on its own (the pages compress the
    embedding and output projection separately from the blocks): the
    LLaMA-2-70B output projection, int8 codes encoded on the device. A
    tensor decoded alone has to fill the GPU with its own chunks, so it is
    encoded in 32,768-symbol chunks (8,000 chunks, whole rows): the line's
    value is that bf16 decode; 65,536 and 16,384 are timed beside it. Also
    logits for m activation rows, fused (entq_decode_gemm) against decode +
    torch.mm, on the one-row (8,192-symbol) and the 32,768 containers, and
    fused on the tensor in tile order (entq_decode_gemm_tiles, chunks of 16
    rows x 2,048 or 4,096 columns)."""
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    nthreads = args.threads or synth.default_threads()
    conts = {}
    for C in (32768, 65536, 16384, 8192):
        specs = synth.llama2_70b_lm_head(nthreads=nthreads, chunk_symbols=C)
        ds = [dict(sp, symbols=torch.from_numpy(
            np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()).to(dev)) for sp in specs]
        b = E.encode_batch_device(ds)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.numel())
        conts[C] = (p, b.blob.clone(), torch.from_numpy(specs[0]["scales"]).to(dev),
                    int(b.blob.numel()), int(p.n_chunks))
        if C == 32768:
            meta = (b.chunks, b.freq[0], dict(specs[0], symbols=None))
        rows, cols = specs[0]["rows"], specs[0]["cols"]
        del ds, b
    torch.cuda.synchronize()
    n = rows * cols
    out = torch.empty(n, dtype=torch.int16, device=dev)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, z in ev:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(z) for a, z in ev])) * 1e3  # us

    reps = max(args.steps, 20)
    dec = {}
    for C, (p, blob, sc, nbytes, nch) in conts.items():
        us = timed(lambda: E.decode(p, blob, out, E.OUT_BF16, sc, None, stream), reps)
        alg = nbytes + 4.0 * rows + 2.0 * n
        dec[C] = {"chunk_symbols": C, "chunks": nch, "compressed_bytes": nbytes,
                  "decode_us": us, "params_per_s": n / (us / 1e6),
                  "alg_gbs": alg / (us / 1e6) / 1e9}
        log(f"lm head decode, {C}-symbol chunks ({nch}): {us:.1f} us, "
            f"{dec[C]['alg_gbs']:.0f} GB/s")
    W = out.view(torch.bfloat16)
    # the same codes in tile order: 16-row bands of 2,048 or 4,096 columns
    tiled = {}
    head = synth.llama2_70b_lm_head(nthreads=nthreads, chunk_symbols=32768)[0]
    for Ct in (2048, 4096):
        st = E.tile_order(head["symbols"], rows, cols, Ct, nthreads)
        b = E.encode_batch_device([dict(head, symbols=torch.from_numpy(st).to(dev),
                                        chunk_symbols=16 * Ct,
                                        kind=head["kind"] | E.LAYOUT_TILES)])
        tiled[Ct] = (E.plan(b.tensors, b.freq, b.chunks, b.blob.numel()), b.blob.clone(),
                     torch.from_numpy(head["scales"]).to(dev), int(b.blob.numel()))
        del b, st
    del head
    logits = []
    gen = torch.Generator().manual_seed(0)
    for m in [int(v) for v in (args.tokens or "16,1").split(",") if v]:
        X = (torch.randn(m, cols, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        Y = torch.empty(m, rows, dtype=torch.float32, device=dev)
        Yb = torch.empty(m, rows, dtype=torch.bfloat16, device=dev)
        for C in (8192, 32768):
            p, blob, sc, nbytes, nch = conts[C]

            def unfused():
                E.decode(p, blob, out, E.OUT_BF16, sc, None, stream)
                torch.mm(X, W.view(rows, cols).t(), out=Yb)

            f_us = timed(lambda: E.decode_gemm(p, blob, sc, [X], [Y], None, stream), reps)
            u_us = timed(unfused, reps)
            logits.append({"m": m, "chunk_symbols": C, "fused_us": f_us, "unfused_us": u_us,
                           "speedup": u_us / f_us})
            log(f"lm head logits m={m}, {C}-symbol chunks: fused {f_us:.1f} us, "
                f"decode + GEMM {u_us:.1f} us")
        for Ct, (p, blob, sc, nbytes) in tiled.items():
            n_ws = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(p.handle, m))
            raw = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
            ws = raw[(-raw.data_ptr()) % 256:][:n_ws]
            f_us = timed(lambda: E.decode_gemm_tiles(p, blob, sc, [X], [Y], None, stream, ws),
                         reps)
            logits.append({"m": m, "tile_cols": Ct, "compressed_bytes": nbytes, "fused_us": f_us})
            log(f"lm head logits m={m}, tile order, 16 x {Ct} chunks: fused {f_us:.1f} us")
    cpu = None
    if not args.no_cpu_baseline:
        p, blob, sc, nbytes, nch = conts[32768]
        E.decode(p, blob, out, E.OUT_BF16, sc, None, stream)
        torch.cuda.synchronize()
        ch, freq, spec = meta
        bits, dt, n_s = oracle_tensor_sample(blob.cpu().numpy(), ch, freq, spec, 4000)
        ok = bool(np.array_equal(out[:n_s].cpu().numpy().view(np.uint16), bits))
        log(f"cpu oracle, lm head sample: {n_s} params in {dt:.2f}s ({n_s / dt / 1e6:.1f} M "
            f"params/s); matches GPU: {ok}")
        if not ok:
            raise SystemExit("LM-head decode differs from the oracle on the CPU-baseline sample")
        cpu = {"value": n_s / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
               "sample": f"first 4,000 chunks ({n_s} params) of the 32,768-symbol container: "
                         "single-threaded C oracle decode + dequant + RNE bf16"}
    d0 = dec[32768]
    rec = {
        "metric": LMHEAD_METRIC,
        "value": d0["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": args.warmup,
        "ms_per_step": d0["decode_us"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32->bf16",
        "data": "synthetic (seeded int8 codes of the stated distribution; no trained weights)",
        "config": {
            "workload": "llama2-70b output projection 32000x8192 int8 rANS codes -> bf16, decoded alone, 32,768-symbol chunks",
            "params": n,
            "decode": list(dec.values()),
            "logits": logits,
            "timing": "median of per-launch HIP events",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": d0["alg_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": d0["alg_gbs"] / HBM_PEAK_GBS,
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


ADAPTIVE_METRIC = ("decoded params/s and achieved HBM GB/s for 70B-shaped layer decode with "
                   "per-chunk tables")


def bench_adaptive(args):
    """The 80-layer decode of the headline workload with every chunk coded
    by its own table (entq_encode_tensor_adaptive / entq_plan_adaptive),
    timed against the shared-table decode of the same codes in the same
    process (one launch per layer, HIP events on the stream). Also one
    70B-shaped layer of banded codes (the spread changes every 8 rows, sigma
    ~ U[0.3, 4.0]), the case per-chunk tables are for: sizes and decode
    times under both."""
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    nthreads = args.threads or synth.default_threads()

    def build(specs, adaptive):
        b = E.encode_batch_adaptive(specs, nthreads) if adaptive else E.encode_batch(specs, nthreads)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
        sc = torch.from_numpy(np.concatenate([s_["scales"] for s_ in specs])).to(dev)
        return p, torch.from_numpy(b.blob).to(dev), sc, int(b.blob.size), b.out_elems

    t0 = time.time()
    lay = {True: [], False: []}
    sample = None
    for layer in range(args.layers):
        specs = synth.llama2_70b_layer(layer, nthreads=nthreads)
        for adaptive in (True, False):
            lay[adaptive].append(build(specs, adaptive))
        if layer == 0 and not args.no_cpu_baseline:
            sample = (E.encode_batch_adaptive(specs[:3], nthreads), specs[:3])
        if layer % 10 == 0 or layer == args.layers - 1:
            log(f"adaptive: layer {layer} encoded both ways ({time.time() - t0:.1f}s)")
    params = lay[True][0][4]
    out = torch.empty(params, dtype=torch.int16, device=dev)

    def time_pass(layers):
        def run(ev=None):
            for li, (p_, blob, sc_, _, _) in enumerate(layers):
                if ev is not None:
                    ev[li][0].record(stream)
                E.decode(p_, blob, out, E.OUT_BF16, sc_, None, stream)
                if ev is not None:
                    ev[li][1].record(stream)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in layers] for _ in range(args.steps)]
        t = time.perf_counter()
        for st in range(args.steps):
            run(ev[st])
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t) / args.steps
        us = float(1e3 * np.mean([[e[0].elapsed_time(e[1]) for e in ev[st]]
                                   for st in range(args.steps)]))
        return ms, us

    res = {}
    for adaptive in (True, False):
        ms, us = time_pass(lay[adaptive])
        nbytes = float(np.mean([l[3] for l in lay[adaptive]]))
        alg = nbytes + 4.0 * int(lay[adaptive][0][2].numel()) + 2.0 * params
        res["per_chunk" if adaptive else "shared"] = {
            "ms_per_step": ms, "us_per_layer": us, "compressed_bytes_per_layer": nbytes,
            "bits_per_param": 8.0 * nbytes / params, "alg_gbs": alg / (us / 1e6) / 1e9}
        log(f"adaptive={adaptive}: {ms:.3f} ms/step, {us:.1f} us/layer, "
            f"{8.0 * nbytes / params:.4f} bits/param")
    cpu = None
    if sample is not None:
        cpu = adaptive_cpu_baseline(E, sample, lay[True][0], out, stream, torch)
    for k in lay:
        lay[k].clear()
    torch.cuda.empty_cache()
    # banded codes: one layer's shapes, sigma changing every 8 rows
    specs = [synth.banded_int8_tensor(r, c, 8, 20 + t, 65536, nthreads=nthreads)
             for t, (_, r, c) in enumerate(synth.LLAMA2_70B_LAYER)]
    banded = {}
    for adaptive in (True, False):
        one = [build(specs, adaptive)]
        ms, us = time_pass(one)
        banded["per_chunk" if adaptive else "shared"] = {
            "us": us, "compressed_bytes": one[0][3], "bits_per_param": 8.0 * one[0][3] / params}
        log(f"banded adaptive={adaptive}: {us:.1f} us, {8.0 * one[0][3] / params:.4f} bits/param")
        del one
    # BF16 exponent stream (8192 x 8192 weights ~ N(0, 0.02)) under both tables
    w = synth.bf16_weights()[0]
    e, sm = E.bf16_split(w["bf16"], nthreads)
    espec = [dict(kind=E.KIND_BF16EXP, rows=w["rows"], cols=w["cols"], chunk_symbols=65536,
                  symbols=e)]
    sm_d = torch.from_numpy(sm).to(dev)
    nw = w["bf16"].size
    outw = torch.empty(nw, dtype=torch.int16, device=dev)
    want = torch.from_numpy(w["bf16"].view(np.int16)).to(dev)
    exp_split = {}
    for adaptive in (True, False):
        b_ = E.encode_batch_adaptive(espec, nthreads) if adaptive else E.encode_batch(espec, nthreads)
        p_ = E.plan(b_.tensors, b_.freq, b_.chunks, b_.blob.size)
        blob_ = torch.from_numpy(b_.blob).to(dev)
        for _ in range(args.warmup + 1):
            E.decode_bf16_split(p_, blob_, sm_d, outw, None, stream)
        torch.cuda.synchronize()
        assert torch.equal(outw, want), "exponent-stream decode differs from the source"
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(20)]
        for a_, z_ in ev:
            a_.record(stream)
            E.decode_bf16_split(p_, blob_, sm_d, outw, None, stream)
            z_.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a_.elapsed_time(z_) for a_, z_ in ev])) * 1e3
        exp_split["per_chunk" if adaptive else "shared"] = {
            "us": us, "exp_stream_bytes": int(b_.blob.size),
            "exp_bits_per_weight": 8.0 * b_.blob.size / nw}
        log(f"bf16 exponent stream 8192x8192 adaptive={adaptive}: {us:.1f} us, "
            f"{8.0 * b_.blob.size / nw:.4f} exponent bits/weight")
        del p_, blob_
    r0 = res["per_chunk"]
    rec = {
        "metric": ADAPTIVE_METRIC,
        "value": params * args.layers / (r0["ms_per_step"] / 1e3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r0["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32->bf16",
        "data": "synthetic (seeded int8 codes of the stated distributions; no trained weights)",
        "config": {
            "workload": "llama2-70b-shaped layer-by-layer decode, int8 rANS codes with per-chunk tables -> bf16",
            "layers": args.layers,
            "params_per_layer": params,
            "chunk_symbols": 65536,
            "per_chunk_vs_shared": res,
            "banded_layer": banded,
            "bf16_exponent_stream_8192x8192": exp_split,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": r0["alg_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": r0["alg_gbs"] / HBM_PEAK_GBS,
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def adaptive_cpu_baseline(E, sample, layer0, out, stream, torch):
    """The oracle's per-chunk-table decode + dequant of layer 0's first three
    tensors (from the library's container, which the tests prove equal to
    the oracle's), timed on this host and compared with the GPU's bf16."""
    import oracle
    b, specs = sample
    p0, blob_d, sc_d, _, _ = layer0
    E.decode(p0, blob_d, out, E.OUT_BF16, sc_d, None, stream)
    torch.cuda.synchronize()
    n = sum(s_["rows"] * s_["cols"] for s_ in specs)
    gpu = out[:n].cpu().numpy().view(np.uint16)
    t = time.perf_counter()
    parts = []
    for ti, sp in enumerate(specs):
        sym = np.zeros(sp["rows"] * sp["cols"], np.uint8)
        for ch in b.chunks[b.chunks["tensor"] == ti]:
            s_, st = oracle.decode_adaptive_chunk(b.blob, int(ch["byte_offset"]),
                                                  int(ch["n_symbols"]), int(ch["n_words"]))
            assert st == 0
            e0 = int(ch["elem_offset"])
            sym[e0:e0 + s_.size] = s_
        parts.append(oracle.dequant_tensor(sym, sp["rows"], sp["cols"], sp["kind"], sp["scales"]))
    dt = time.perf_counter() - t
    ok = bool(np.array_equal(np.concatenate(parts), gpu))
    log(f"cpu oracle, per-chunk tables: {n} params in {dt:.2f}s ({n / dt / 1e6:.1f} M params/s); "
        f"matches GPU: {ok}")
    if not ok:
        raise SystemExit("per-chunk-table decode differs from the oracle on the CPU-baseline sample")
    return {"value": n / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, first 3 tensors ({n} params): single-threaded C oracle "
                      "per-chunk-table decode + dequant + RNE bf16"}


WORKLOADS_METRIC = "decoded params/s per workload, each decoded alone with caches flushed"


def bench_workloads(args):
    """The smaller workloads, each decoded alone: 256 x 256 Laplace int8
    codes (4,096-symbol chunks; codes and bf16), the e4m3 4096 x 4096 matrix
    (codes and bf16), one LLaMA-2-13B block (7 int8 tensors, bf16), the
    8192 x 8192 BF16 matrix from its coded exponents + raw sign/mantissa
    bytes, and one 70B-shaped layer for comparison. Each timed launch follows
    a 512 MB read that evicts the last-level cache; median of the per-launch
    HIP events. Lossless outputs (codes, the BF16 matrix) are compared with
    their sources; every bf16 output but the 70B layer's with the oracle
    (the CPU-baseline leg)."""
    import torch

    import entropy_coded_weight_amd as E
    import synth

    E.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    nthreads = args.threads or synth.default_threads()
    # Before each timed launch, a read of 512 MB of clean data evicts the
    # last-level cache (256 MB) without leaving dirty lines whose write-back
    # would land inside the timed launch.
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    flush_sum = torch.empty((), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    reps = max(args.steps, 20)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        times = []
        for _ in range(reps):
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_sum)
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            z.record(stream)
            z.synchronize()
            times.append(a.elapsed_time(z) * 1e3)
        return float(np.median(times)), float(np.percentile(times, 10)), float(np.percentile(times, 90))

    rows_out, checks, kept = [], {}, {}

    def coded(name, specs, outs):
        b = E.encode_batch(specs, n_threads=nthreads)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
        blob = torch.from_numpy(b.blob).to(dev)
        sc = torch.from_numpy(np.concatenate([np.asarray(s["scales"], np.float32)
                                              for s in specs])).to(dev)
        n = b.out_elems
        for kind in outs:
            if kind == "codes":
                out = torch.empty(n, dtype=torch.uint8, device=dev)
                med, p10, p90 = timed(lambda: E.decode(p, blob, out, E.OUT_CODES, None, None, stream))
                src = np.concatenate([np.asarray(s["symbols"]).view(np.uint8).ravel() for s in specs])
                checks[f"{name} codes equal the source"] = bool(np.array_equal(out.cpu().numpy(), src))
                written = n
            else:
                out = torch.empty(n, dtype=torch.int16, device=dev)
                med, p10, p90 = timed(lambda: E.decode(p, blob, out, E.OUT_BF16, sc, None, stream))
                kept[name] = (specs, b, out.cpu().numpy().view(np.uint16))
                written = 2 * n
            alg = b.blob.size + (4 * sc.numel() if kind == "bf16" else 0) + written
            rows_out.append({"workload": name, "output": kind, "params": n,
                             "chunks": int(p.n_chunks), "bits_per_param": 8.0 * b.blob.size / n,
                             "us_median": med, "us_p10": p10, "us_p90": p90,
                             "params_per_s": n / (med / 1e6), "alg_gbs": alg / (med / 1e6) / 1e9})
            log(f"{name} -> {kind}: {med:.1f} us (p10 {p10:.1f}, p90 {p90:.1f}), "
                f"{rows_out[-1]['alg_gbs']:.0f} GB/s")

    coded("laplace int8 256x256", synth.tiny_int8_laplace(), ("codes", "bf16"))
    coded("e4m3 4096x4096", synth.e4m3_matrix(), ("codes", "bf16"))
    coded("llama2-13b block", synth.llama2_13b_block(), ("bf16",))

    # The BF16 matrix at several chunk sizes (the pages fix none): each chunk
    # carries 64 x 4-byte states, so smaller chunks cost more bits, and a
    # lone matrix fills the GPU with more chunks.
    w = synth.bf16_weights()[0]
    e, sm = E.bf16_split(w["bf16"], n_threads=nthreads)
    n = w["rows"] * w["cols"]
    smd = torch.from_numpy(sm).to(dev)
    out = torch.empty(n, dtype=torch.int16, device=dev)
    for C in (8192, 16384, 32768, 65536):
        b = E.encode_batch([dict(kind=E.KIND_BF16EXP, rows=w["rows"], cols=w["cols"],
                                 chunk_symbols=C, symbols=e)], n_threads=nthreads)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
        blob = torch.from_numpy(b.blob).to(dev)
        out.zero_()
        med, p10, p90 = timed(lambda: E.decode_bf16_split(p, blob, smd, out, None, stream))
        split_bits = out.cpu().numpy().view(np.uint16)
        checks[f"bf16 8192x8192 ({C}-symbol chunks) equals the source weights"] = bool(
            np.array_equal(split_bits, w["bf16"]))
        if C == w["chunk_symbols"]:
            kept["bf16 split"] = (b, sm, split_bits, n)
        rows_out.append({"workload": "bf16 8192x8192 exponent stream + sign/mantissa",
                         "output": "bf16", "chunk_symbols": C,
                         "params": n, "chunks": int(p.n_chunks),
                         "bits_per_param": 8.0 * (b.blob.size + n) / n,
                         "exponent_bits_per_param": 8.0 * b.blob.size / n,
                         "us_median": med, "us_p10": p10, "us_p90": p90,
                         "params_per_s": n / (med / 1e6),
                         "alg_gbs": (b.blob.size + n + 2 * n) / (med / 1e6) / 1e9})
        log(f"bf16 8192x8192 split, {C}-symbol chunks ({p.n_chunks}): {med:.1f} us, "
            f"{rows_out[-1]['alg_gbs']:.0f} GB/s, {rows_out[-1]['exponent_bits_per_param']:.3f} "
            "exponent bits per weight")
        del blob
        p.close()
    del smd, out

    coded("llama2-70b layer 0", synth.llama2_70b_layer(0, nthreads=nthreads), ("bf16",))
    del flush

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t = time.perf_counter()
        n_s = 0
        for name in ("laplace int8 256x256", "e4m3 4096x4096", "llama2-13b block"):
            specs, bb, gpu = kept[name]
            ok, at = True, 0
            for ti, sp in enumerate(specs):
                ch = bb.chunks[bb.chunks["tensor"] == ti]
                desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"],
                                 ch["elem_offset"]], axis=1).astype(np.uint64)
                nt = sp["rows"] * sp["cols"]
                sym, st = oracle.decode_tensor(bb.blob, desc, bb.freq[ti], nt)
                bits = oracle.dequant_tensor(sym, sp["rows"], sp["cols"], sp["kind"], sp["scales"])
                ok = ok and bool((st == 0).all() and np.array_equal(bits, gpu[at:at + nt]))
                at += nt
            checks[f"{name} bf16 equals the oracle"] = ok
            n_s += at
        bb, sm_h, gpu, nw_ = kept["bf16 split"]
        desc = np.stack([bb.chunks["n_symbols"], bb.chunks["n_words"], bb.chunks["byte_offset"],
                         bb.chunks["elem_offset"]], axis=1).astype(np.uint64)
        sym, st = oracle.decode_tensor(bb.blob, desc, bb.freq[0], nw_)
        checks["bf16 8192x8192 equals the oracle"] = bool(
            (st == 0).all() and np.array_equal(oracle.bf16_merge(sym, sm_h), gpu))
        n_s += nw_
        dt = time.perf_counter() - t
        cpu = {"value": n_s / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
               "sample": "the whole 256x256 Laplace, e4m3 4096x4096, LLaMA-2-13B block and BF16 "
                         "8192x8192 workloads: single-threaded C oracle decode + dequant + RNE "
                         "bf16 (+ sign/mantissa merge)"}
        log(f"cpu oracle: {n_s} params in {dt:.2f}s")
    for k, ok in checks.items():
        log(f"check: {k}: {ok}")
    if not all(checks.values()):
        raise SystemExit("a workload's output differs from its source or from the oracle")
    main_row = next(r for r in rows_out if r["workload"] == "llama2-13b block")
    rec = {
        "metric": WORKLOADS_METRIC,
        "value": main_row["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": args.warmup,
        "ms_per_step": main_row["us_median"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32->bf16",
        "data": "synthetic (seeded codes and weights of the stated distributions; no trained weights)",
        "config": {
            "workload": "llama2-13b block (7 int8 tensors, 317,194,240 params) -> bf16; the other "
                        "workloads in 'workloads'",
            "workloads": rows_out,
            "timing": "per launch, after a 512 MB read that evicts the last-level cache; median",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": main_row["alg_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": main_row["alg_gbs"] / HBM_PEAK_GBS,
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
