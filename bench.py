"""Benchmark: generation throughput of the 4-bit weight + 4-bit KV-cache path.

Metric (FlexGen README, "Benchmark Results", Metric bullet): generated tokens
/ (prompt time + generation time), prompt 512, output 32.  One step = one
full pass of the path over one batch: prefill of every prompt through every
layer, then 31 decode steps (quantise-on-append, dequant-fused GEMMs, packed
KV attention, LM head, greedy argmax).  Inputs are synthetic and already in
HBM (weights generated and quantised on the device, prompt ids from the
seeded generator) before the timed region starts.

Default workload: the OPT-175B shape (96 layers, hidden 12288, 96 heads x 128,
FFN 49152, vocab 50272) with 4-bit group-64 weights and 4-bit KV resident on
one MI355X, batch 144, prompt 512, gen 32 -- the configuration of the pages'
"FlexGen with Compression" OPT-175B figure (effective batch 144).

Prints one JSON line.  Also measures, live over the timed region, the
per-launch device time of every kernel class (HIP events on the launching
stream) and reports the dominant kernel against its roofline, and times the
CPU oracle on a bounded sample of the same workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CONFIGS = {
    # name: (hidden, heads, ffn, layers, vocab, batch, prompt, gen, compression switches, streaming knobs)
    "opt175b-4bit": dict(hidden=12288, heads=96, ffn=49152, layers=96, vocab=50272, batch=144, prompt=512, gen=32,
                         compress_weight=True, desc="OPT-175B shape, 4-bit g64 weights + 4-bit KV resident in HBM"),
    "opt30b-4bit": dict(hidden=7168, heads=56, ffn=28672, layers=48, vocab=50272, batch=256, prompt=512, gen=32,
                        compress_weight=True, desc="OPT-30B shape, 4-bit g64 weights + 4-bit KV resident in HBM"),
    "opt175b-fp16-streamed": dict(hidden=12288, heads=96, ffn=49152, layers=96, vocab=50272, batch=256, prompt=512,
                                  gen=32, compress_weight=False, resident_layers=0, host_layers=12,
                                  desc="OPT-175B shape, fp16 weights streamed layer by layer from pinned host memory "
                                       "(12 distinct host layer blobs, layer l reads blob l mod 12: the GPU host "
                                       "allows ~58 GB of pinned memory per process), 4-bit KV"),
    "opt175b-4bit-b256-offload": dict(hidden=12288, heads=96, ffn=49152, layers=96, vocab=50272, batch=256, prompt=512,
                                      gen=32, compress_weight=True, resident_layers=78,
                                      desc="OPT-175B shape, batch 256: the 4-bit KV cache (184 GB) leaves HBM for 78 "
                                           "layers of 4-bit weights; the other 18 stream from pinned host memory in "
                                           "packed form (0.5625 byte per weight) every pass"),
    "opt175b-4bit-b256-kvoffload": dict(hidden=12288, heads=96, ffn=49152, layers=96, vocab=50272, batch=256,
                                        prompt=512, gen=32, compress_weight=True, cache_resident_layers=84,
                                        desc="OPT-175B shape, batch 256: all 4-bit weights in HBM; the 4-bit KV cache "
                                             "of layers 84-95 (23 GB) in pinned host memory, its valid prefix staged "
                                             "in and new positions written back every pass"),
    "opt175b-4bit-weights-f16-cache": dict(hidden=12288, heads=96, ffn=49152, layers=96, vocab=50272, batch=48,
                                           prompt=512, gen=32, compress_weight=True, compress_cache=False,
                                           desc="OPT-175B shape, weight-only compression: 4-bit g64 weights, fp16 KV "
                                                "cache (2 bytes per element: 123 GB at batch 48), all in HBM"),
    "tiny-2layer": dict(hidden=256, heads=4, ffn=1024, layers=2, vocab=512, batch=8, prompt=64, gen=5,
                        compress_weight=True, desc="tiny OPT-style model for smoke benchmarking"),
}
METRIC = "generation tokens/s (prompt 512, gen 32) at batch 144-256; % HBM/MFMA roofline"
PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak (published)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak (published)
PAGES_T4_TOKS = {"opt175b-4bit": 1.12}  # FlexGen with Compression, OPT-175B, T4 (context, other hardware)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="opt175b-4bit", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--max-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true", help="time only the oracle sample (no GPU)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the run, copy a BYTES-sized device buffer three times (a plain copy kernel of known "
                         "size, for scaling hardware byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure this GPU's practical ceilings (HBM copy stream, pinned host<->device copies, "
                         "the vendor library's fp16 GEMM at the prefill shape) and print them as one JSON line")
    ap.add_argument("--kernel-only", choices=["gemm_prefill", "gemm_decode", "decode_attention"], default=None,
                    help="launch only this kernel class, as one layer of the workload launches it (a short program "
                         "for hardware-counter passes); prints the launch list instead of the JSON line")
    return ap.parse_args()


def measured_traffic(kernel):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3
    counter summary, or None when there is none or the kernel source changed
    since the counters were taken."""
    import hashlib
    import re
    csrc = "bit_weight_kv_amd/csrc/"
    gemm_src = [csrc + "gemm.hip", csrc + "quant_group.h", csrc + "common.h"]
    summary = {"gemm_prefill": ("profiles/gemm_prefill_opt175b_4bit_b144.md", gemm_src),
               "gemm_decode": ("profiles/gemm_decode_opt175b_4bit_b144.md", gemm_src),
               "decode_attention": ("profiles/decode_attention_opt175b_4bit_b144.md",
                                    [csrc + "attention.hip", csrc + "common.h"])}
    if kernel not in summary:
        return None
    md, srcs = summary[kernel]
    try:
        text = open(os.path.join(ROOT, md)).read()
        h = hashlib.sha256()
        for f in srcs:  # the sources the kernel is built from, in this order
            h.update(open(os.path.join(ROOT, f), "rb").read())
        digest = h.hexdigest()
    except OSError:
        return None
    t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    h = re.search(r"^source_sha256: ([0-9a-f]{64})$", text, re.M)
    if not t or not h or h.group(1) != digest:
        return None
    return int(t.group(1))


def roofline(kstats, config):
    """Dominant kernel class by device time, against its own roofline."""
    name, st = max(kstats.items(), key=lambda kv: kv[1]["seconds"])
    if st["seconds"] <= 0:
        return None, {}
    per_launch_s = st["seconds"] / st["launches"]
    if name.startswith("gemm") or name == "lm_head":
        achieved = st["flops"] / st["seconds"] / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4), "traffic": None}
    else:
        achieved = st["bytes"] / st["seconds"] / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    if config == "opt175b-4bit":  # the counters were taken at this workload's shapes
        r["traffic"] = measured_traffic(name)
    r["kernel"] = name
    r["launches"] = st["launches"]
    r["avg_launch_ms"] = round(per_launch_s * 1e3, 4)
    r["work_per_launch"] = (st["flops"] if r["bound"] == "mfma" else st["bytes"]) / st["launches"]
    return name, r


def kernel_table(kstats, config):
    out = {}
    for name, st in kstats.items():
        if st["launches"] == 0:
            continue
        e = {"launches": st["launches"], "seconds": round(st["seconds"], 4),
             "avg_launch_ms": round(st["seconds"] / st["launches"] * 1e3, 4)}
        if st["flops"] > 0:
            e["tflops"] = round(st["flops"] / st["seconds"] / 1e12, 2)
            e["mfma_frac"] = round(st["flops"] / st["seconds"] / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)
        if st["bytes"] > 0:
            e["gbs"] = round(st["bytes"] / st["seconds"] / 1e9, 1)
            e["hbm_frac"] = round(st["bytes"] / st["seconds"] / 1e9 / PEAK_HBM_GBS, 4)
        if config == "opt175b-4bit":
            t = measured_traffic(name)
            if t is not None:
                e["traffic_per_launch"] = t
        out[name] = e
    return out


def cpu_baseline(cfg, seed):
    """The CPU oracle on a bounded sample of the same workload: three sequences
    through one layer of this shape -- prefill of the 512-token prompt, then the
    31 decode steps -- timed on the host cores, scaled to the full workload
    (every layer costs the same; cost is linear in the batch):
    tokens/s = 3 * gen / (t * layers)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth
    from synth.gen import layer_stream

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = min(16, os.cpu_count() or 1)
    h, H, F = cfg["hidden"], cfg["heads"], cfg["ffn"]
    lcfg = oracle.LayerConfig(h, H, F, compress_weight=cfg["compress_weight"],
                              compress_cache=cfg.get("compress_cache", True))
    workers = min(16, os.cpu_count() or 1)  # the host share of one GPU
    t0 = time.time()

    def gen(name, shape, sigma):
        n = int(np.prod(shape))
        out = np.empty(n, np.float16)
        step = max(1 << 22, n // (4 * workers) + 1)

        def part(s):
            e = min(n, s + step)
            out[s:e] = synth.normal_f16(seed, layer_stream(0, name), sigma=sigma,
                                        index=np.arange(s, e, dtype=np.uint64))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(part, range(0, n, step)))
        return out.reshape(shape)

    params = {"w_qkv": gen("w_qkv", (3 * h, h), 0.02), "w_out": gen("w_out", (h, h), 0.02),
              "w_fc1": gen("w_fc1", (F, h), 0.02), "w_fc2": gen("w_fc2", (h, F), 0.02)}
    for name, n in (("b_qkv", 3 * h), ("b_out", h), ("b_fc1", F), ("b_fc2", h)):
        params[name] = np.zeros(n, np.float16)
    for name in ("ln1_g", "ln2_g"):
        params[name] = np.ones(h, np.float16)
    for name in ("ln1_b", "ln2_b"):
        params[name] = np.zeros(h, np.float16)
    # load-time weight packing (not part of the metric), row blocks in parallel
    packed = {}
    for name in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        w = params[name]
        if not lcfg.compress_weight:
            packed[name] = w.astype(np.float64)
            continue
        out = np.empty(w.shape, np.float64)
        rows = max(64, w.shape[0] // (4 * workers))

        def part(r0, w=w, out=out):
            c, m = oracle.quantize(w[r0:r0 + rows])
            out[r0:r0 + rows] = oracle.dequant_f16(c, m)
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(part, range(0, w.shape[0], rows)))
        packed[name] = out
    setup_s = time.time() - t0
    P, G = cfg["prompt"], cfg["gen"]
    S = 3  # sequences in the sample (about 10-15 s of host time at the OPT-175B shape)
    x = synth.normal_f16(seed, synth.STREAM["hidden"], (S, P + G - 1, h), 1.0)
    cache = oracle.new_cache(lcfg, S, P + G)
    t1 = time.time()
    oracle.layer_step(x[:, :P], params, packed, cache, lcfg, 0)
    for t in range(G - 1):
        oracle.layer_step(x[:, P + t:P + t + 1], params, packed, cache, lcfg, P + t)
    t_sample = time.time() - t1
    value = S * G / (t_sample * cfg["layers"])
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{S} sequences x 1 layer of the {cfg['desc']} shape: prefill of {P} tokens + {G - 1} decode "
                      f"steps, {t_sample:.1f} s on the host; scaled to the {cfg['layers']}-layer model (every layer "
                      f"costs the same, and the oracle's cost is linear in the batch): tokens/s = "
                      f"{S}*gen/(t*layers); weight generation and packing ({setup_s:.0f} s, load-time) not timed",
            "sample_seconds": round(t_sample, 2)}


def ceilings(torch):
    """Practical ceilings of this GPU, measured with plain torch operations
    (reference points for the roofline fractions; not part of the path)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    out = {}
    n = 1 << 30  # 4 GiB of int32, far above the 256 MB MALL
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: torch.neg(src, out=dst), 5)
    out["hbm_copy_GBs"] = round(2 * 4 * n / t / 1e9, 1)  # read + write
    del src, dst
    torch.cuda.empty_cache()
    host = torch.empty(1 << 28, dtype=torch.int32, pin_memory=True)  # 1 GiB pinned
    dev = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    out["h2d_pinned_GBs"] = round(4 * (1 << 28) / timed(lambda: dev.copy_(host, non_blocking=True), 5) / 1e9, 1)
    out["d2h_pinned_GBs"] = round(4 * (1 << 28) / timed(lambda: host.copy_(dev, non_blocking=True), 5) / 1e9, 1)
    del host, dev
    M, N, K = 16384, 49152, 12288
    a = torch.randn((M, K), dtype=torch.float16, device="cuda")
    b = torch.randn((K, N), dtype=torch.float16, device="cuda")
    c = torch.empty((M, N), dtype=torch.float16, device="cuda")
    t = timed(lambda: torch.matmul(a, b, out=c), 5)
    out["library_fp16_gemm_TFLOPs"] = round(2.0 * M * N * K / t / 1e12, 1)
    out["library_fp16_gemm_shape"] = [M, N, K]
    return out


def kernel_only(fq, synth, torch, cfg, args):
    if args.kernel_only == "gemm_prefill":
        return kernel_only_gemm(fq, synth, torch, cfg, args, prefill=True)
    if args.kernel_only == "gemm_decode":
        return kernel_only_gemm(fq, synth, torch, cfg, args, prefill=False)
    return kernel_only_decode_attention(fq, synth, torch, cfg, args)


def kernel_only_decode_attention(fq, synth, torch, cfg, args):
    """Decode attention of one layer at three cache lengths of the workload's
    decode steps (first, middle, last): B sequences x H heads over a packed
    cache of capacity P + G - 1 (contents are seeded random codes and
    {min, scale} pairs; the traffic does not depend on them)."""
    h, H, B, P, G = cfg["hidden"], cfg["heads"], cfg["batch"], cfg["prompt"], cfg["gen"]
    d, S = h // H, P + G - 1
    gen = torch.Generator(device="cuda").manual_seed(args.seed)
    kc = torch.randint(0, 256, (B, H, S, d // 2), dtype=torch.uint8, device="cuda", generator=gen)
    vc = torch.randint(0, 256, (B, H, S, d // 2), dtype=torch.uint8, device="cuda", generator=gen)
    km = torch.empty((B, H, S, d // 64, 2), dtype=torch.float16, device="cuda")
    km[..., 0], km[..., 1] = -0.05, 0.006
    vm = km.clone()
    kv = fq.kv_layer_view(kc, km.view(torch.int16), vc, vm.view(torch.int16))
    q = torch.empty((B, 3 * h), dtype=torch.float16, device="cuda")
    fq.fq_synth_normal_f16(q, args.seed, synth.STREAM["aux"], 1.0)
    out = torch.empty((B, h), dtype=torch.float16, device="cuda")
    launches = []
    for length in (P + 1, P + G // 2, P + G - 1):
        fq.fq_decode_attention(q, kv, 0, B, length, out, ldq=3 * h)
        launches.append([B, H, length, d])
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": args.kernel_only, "launches": launches}), flush=True)


def kernel_only_gemm(fq, synth, torch, cfg, args, prefill):
    """The projection GEMMs of one layer, exactly as the prompt pass (prefill)
    or one decode step launches them: the batch's B*P prompt rows in chunks of
    whole sequences of at most --max-tokens rows (or the B rows of a decode
    step), each chunk through the QKV (bias, query scaling, K/V appended to a
    4-bit cache), out (bias, residual), FC1 (bias, ReLU) and FC2 (bias,
    residual) products of that layer's packed weights.  Every layer of the
    workload repeats this launch list."""
    h, F, B, P, H = cfg["hidden"], cfg["ffn"], cfg["batch"], cfg["prompt"], cfg["heads"]
    d = h // H
    model = fq.Model(h, cfg["heads"], F, 1, vocab=cfg["vocab"], max_pos=P + cfg["gen"] + 2,
                     compress_weight=True, max_tokens=args.max_tokens)
    model.init_random(args.seed)
    shapes = {0: (3 * h, h), 1: (h, h), 2: (F, h), 3: (h, F)}
    W = {i: fq.fq_weight(fq.FQ_WEIGHT_PACKED4, model.packed_weight(0, i), None, n, k)
         for i, (n, k) in shapes.items()}
    total = B * P if prefill else B  # a decode step runs every sequence's one new row
    T = P if prefill else 1
    chunk = max(1, args.max_tokens // T) * T  # rows per launch: whole sequences
    rows = min(total, chunk)
    cap = P + cfg["gen"] - 1
    cache = [torch.zeros((B, H, cap, d // 2), dtype=torch.uint8, device="cuda"),
             torch.zeros((B, H, cap, d // 64, 2), dtype=torch.float16, device="cuda")]
    cache += [torch.zeros_like(cache[0]), torch.zeros_like(cache[1])]
    kv = fq.kv_layer_view(*cache)
    def act(cols, stream):
        t = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
        fq.fq_synth_normal_f16(t, args.seed, stream, 1.0)
        return t

    x, att, x1, h1 = (act(h, synth.STREAM["aux"] + i) for i in range(4))
    qkv, f = act(3 * h, synth.STREAM["aux"] + 4), act(F, synth.STREAM["aux"] + 5)
    bias = torch.zeros(max(3 * h, F), dtype=torch.float16, device="cuda")
    E = fq
    launches = []
    for r0 in range(0, total, chunk):
        M = min(chunk, total - r0)
        fq.fq_qkv_gemm_append(h1[:M], W[0], bias[:3 * h], d ** -0.5, kv, r0 // T, M // T, T, 0 if prefill else P,
                              qkv[:M])
        fq.fq_dequant_gemm(att[:M], W[1], x1[:M], bias=bias, residual=x[:M],
                           epilogue=E.FQ_EPI_BIAS | E.FQ_EPI_RESIDUAL)
        fq.fq_dequant_gemm(h1[:M], W[2], f[:M], bias=bias, epilogue=E.FQ_EPI_BIAS | E.FQ_EPI_RELU)
        fq.fq_dequant_gemm(f[:M], W[3], x[:M], bias=bias, residual=x1[:M], epilogue=E.FQ_EPI_BIAS | E.FQ_EPI_RESIDUAL)
        launches += [(M, n, k) for n, k in shapes.values()]
    torch.cuda.synchronize()
    model.close()
    print(json.dumps({"kernel_only": args.kernel_only, "launches": [list(t) for t in launches]}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the batch dimension would shard over "
              f"GPUs with no exchange, which this program does not launch.", file=sys.stderr)
        sys.exit(2)
    cfg = CONFIGS[args.config]
    if args.cpu_baseline_only:
        print(json.dumps({"cpu_baseline": cpu_baseline(cfg, args.seed)}))
        return
    import numpy as np
    import torch

    import bit_weight_kv_amd as fq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # an elementwise kernel: reads and writes BYTES each
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 copies of {4 * n} bytes")
        del src, dst
        torch.cuda.empty_cache()
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(torch)}), flush=True)
        return
    if args.kernel_only:
        kernel_only(fq, synth, torch, cfg, args)
        return
    B, P, G = cfg["batch"], cfg["prompt"], cfg["gen"]
    t0 = time.time()
    model = fq.Model(cfg["hidden"], cfg["heads"], cfg["ffn"], cfg["layers"], vocab=cfg["vocab"], max_pos=P + G + 2,
                     compress_weight=cfg["compress_weight"], resident_layers=cfg.get("resident_layers", -1),
                     host_layers=cfg.get("host_layers", 0), overlap=True, max_tokens=args.max_tokens,
                     compress_cache=cfg.get("compress_cache", True),
                     cache_resident_layers=cfg.get("cache_resident_layers", -1))
    model.init_random(args.seed)
    kv = fq.KVCache(model, B, P + G)
    last = [time.time()]

    def progress(done, total):  # generations of several minutes report each completed token every ~20 s
        if time.time() - last[0] > 20 or done == 1 and time.time() - last[0] > 5:
            log(f"[bench] token {done}/{total} done")
            last[0] = time.time()

    fq.fq_set_progress(progress)
    ids = synth.token_ids(args.seed, synth.STREAM["prompt"], (B, P), cfg["vocab"])
    torch.cuda.synchronize()
    log(f"[bench] {args.config}: model + cache ready in {time.time() - t0:.1f} s")
    for w in range(args.warmup):
        out, st = fq.fq_generate(model, kv, ids, G)
        log(f"[bench] warmup {w}: {st.tokens_per_s:.2f} tok/s (prefill {st.prefill_s:.2f} s, decode {st.decode_s:.2f} s)")
    torch.cuda.synchronize()
    fq.fq_timing_start()
    stats = []
    t_start = time.perf_counter()
    for s in range(args.steps):
        out, st = fq.fq_generate(model, kv, ids, G)
        stats.append((st.prefill_s, st.decode_s, st.h2d_bytes, st.h2d_s, st.kv_h2d_bytes, st.kv_d2h_bytes))
        log(f"[bench] step {s}: {st.tokens_per_s:.2f} tok/s (prefill {st.prefill_s:.2f} s, decode {st.decode_s:.2f} s)")
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    kstats = fq.fq_timing_stop()
    ms_per_step = t_total / args.steps * 1e3
    value = B * G * args.steps / t_total
    _, roof = roofline(kstats, args.config)
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": (round(value / PAGES_T4_TOKS[args.config], 1) if args.config in PAGES_T4_TOKS else None),
        "dtype": "f16", "data": "synthetic (seeded random-init weights and uniform prompt ids)",
        "config": {"workload": cfg["desc"], "config": args.config, "layers": cfg["layers"], "hidden": cfg["hidden"],
                   "heads": cfg["heads"], "ffn": cfg["ffn"], "vocab": cfg["vocab"], "global_batch": B,
                   "prompt": P, "gen": G, "group": 64, "parallelism": "single GPU"},
        "phases": {"prefill_s": round(float(np.mean([s[0] for s in stats])), 3),
                   "decode_s": round(float(np.mean([s[1] for s in stats])), 3),
                   "h2d_GB": round(float(np.mean([s[2] for s in stats])) / 1e9, 2),
                   "h2d_busy_s": round(float(np.mean([s[3] for s in stats])), 3),
                   "kv_h2d_GB": round(float(np.mean([s[4] for s in stats])) / 1e9, 2),
                   "kv_d2h_GB": round(float(np.mean([s[5] for s in stats])) / 1e9, 2)},
        "roofline": roof,
        "kernels": kernel_table(kstats, args.config),
    }
    kv.close()
    model.close()
    del kv, model
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        res["cpu_baseline"] = cpu_baseline(cfg, args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
