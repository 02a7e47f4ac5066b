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

Single-layer workloads (--config tiny-layer, opt6.7b-layer): one OPT-style
layer over a batch of seeded hidden states, prefill of the prompt then T
teacher-forced decode steps; throughput is the per-layer form of the same
metric, B*T / (layer prefill + T decode steps).

Prints one JSON line.  The warmup steps record every kernel launch's device
time (HIP events on the launching stream) for the per-class kernel table;
the timed steps record only the launches of the dominant kernel class, whose
average launch time gives the roofline figure.  The CPU oracle is timed on
the host cores: on a bounded sample of a full-model workload, or in full for
the single-layer workloads.
"""
import argparse
import json
import subprocess
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
    "tiny-layer": dict(hidden=256, heads=4, ffn=1024, layers=1, vocab=0, batch=8, prompt=64, gen=4,
                       compress_weight=True, layer_only=True,
                       desc="tiny OPT-style layer (hidden 256, 4 heads x 64, FFN 1024), 4-bit g64 weights + 4-bit "
                            "KV, batch 8, prompt 64, 4 teacher-forced decode steps"),
    "opt6.7b-layer": dict(hidden=4096, heads=32, ffn=16384, layers=1, vocab=0, batch=64, prompt=512, gen=32,
                          compress_weight=True, layer_only=True,
                          desc="one OPT-6.7B-shaped layer (hidden 4096, 32 heads x 128, FFN 16384), 4-bit g64 "
                               "weights + 4-bit KV, batch 64, prompt 512, 32 teacher-forced decode steps"),
}
METRIC = "generation tokens/s (prompt 512, gen 32) at batch 144-256; % HBM/MFMA roofline"
PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak (published)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak (published)


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
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="host threads for the oracle sample (default: the host share of one GPU, 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the run, copy a BYTES-sized device buffer three times (a plain copy kernel of known "
                         "size, for scaling hardware byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure this GPU's practical ceilings (HBM copy stream, pinned host<->device copies, "
                         "the vendor library's fp16 GEMM at the prefill shape) and print them as one JSON line")
    ap.add_argument("--kernel-only", choices=["gemm_prefill", "gemm_decode", "decode_attention", "prefill_attention",
                                              "quantize"], default=None,
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
                                    [csrc + "attention.hip", csrc + "common.h"]),
               "prefill_attention": ("profiles/prefill_attention_opt175b_4bit_b144.md",
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


def roofline(name, st, config):
    """One kernel class's launches against that kernel's own roofline: algorithmic
    work per launch / average launch duration."""
    if not st or st["launches"] == 0 or st["seconds"] <= 0:
        return None
    per_launch_s = st["seconds"] / st["launches"]
    if name.startswith("gemm") or name in ("lm_head", "prefill_attention"):
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
    return r


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
        if st.get("dropped"):
            e["untimed_launches"] = st["dropped"]
        if config == "opt175b-4bit":
            t = measured_traffic(name)
            if t is not None:
                e["traffic_per_launch"] = t
        out[name] = e
    return out


def host_description():
    """The host the oracle runs on: logical CPUs, the ones this process may use,
    the CPU model, and the BLAS threads NumPy runs with."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "blas_threads": blas}


def _oracle_layer_params(cfg, seed, workers):
    """The oracle's layer 0 of this shape: seeded fp16 parameters (OPT-style init:
    biases 0, LayerNorm gain 1) and the weights as the GEMMs read them."""
    import oracle
    lcfg = oracle.LayerConfig(cfg["hidden"], cfg["heads"], cfg["ffn"], compress_weight=cfg["compress_weight"],
                              compress_cache=cfg.get("compress_cache", True))
    params = oracle.layer_params(seed, lcfg, 0, workers=workers)
    return lcfg, params, oracle.pack_layer(params, lcfg, workers=workers)


def _oracle_layer_run(lcfg, params, packed, x, P, T):
    """Prefill of P tokens then T single-token steps of one layer; seconds taken."""
    import oracle
    cache = oracle.new_cache(lcfg, x.shape[0], P + T)
    t = time.time()
    oracle.layer_step(x[:, :P], params, packed, cache, lcfg, 0)
    for i in range(T):
        oracle.layer_step(x[:, P + i:P + i + 1], params, packed, cache, lcfg, P + i)
    return time.time() - t


def cpu_baseline(cfg, seed, workers=0):
    """The CPU oracle on the host cores.

    Full-model workloads: a bounded sample -- three sequences through one layer
    of this shape, prefill of the prompt and the gen-1 decode steps -- scaled to
    the whole model (every layer costs the same; cost is linear in the batch):
    tokens/s = 3 * gen / (t * layers).  Single-layer workloads: the whole
    workload (every sequence, prefill and every decode step), and for the tiny
    layer also on one thread."""
    import synth
    workers = workers or min(16, os.cpu_count() or 1)  # the host share of one GPU
    t0 = time.time()
    lcfg, params, packed = _oracle_layer_params(cfg, seed, workers)
    setup_s = time.time() - t0
    h, P, G = cfg["hidden"], cfg["prompt"], cfg["gen"]
    hostd = host_description()
    if cfg.get("layer_only"):
        B, T = cfg["batch"], G
        x = synth.normal_f16(seed, synth.STREAM["hidden"], (B, P + T, h), 1.0)
        t = _oracle_layer_run(lcfg, params, packed, x, P, T)
        r = {"value": B * T / t, "unit": "tokens/s", "cores": hostd["blas_threads"], "kind": "oracle",
             "sample": f"the whole workload: {B} sequences, prefill of {P} tokens + {T} decode steps of the layer, "
                       f"{t:.2f} s on the host; tokens/s = B*T/t; weight generation and packing ({setup_s:.0f} s, "
                       f"load-time) not timed",
             "sample_seconds": round(t, 3), "host": hostd}
        if B * (P + T) * h <= (1 << 22):  # small enough to repeat on one thread
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                t1 = _oracle_layer_run(lcfg, params, packed, x, P, T)
            r["single_thread"] = {"value": B * T / t1, "sample_seconds": round(t1, 3), "cores": 1}
        return r
    S = 3  # sequences in the sample (about 10-15 s of host time at the OPT-175B shape)
    x = synth.normal_f16(seed, synth.STREAM["hidden"], (S, P + G - 1, h), 1.0)
    t = _oracle_layer_run(lcfg, params, packed, x, P, G - 1)
    value = S * G / (t * cfg["layers"])
    return {"value": value, "unit": "tokens/s", "cores": hostd["blas_threads"], "kind": "oracle",
            "sample": f"{S} sequences x 1 layer of the {cfg['desc']} shape: prefill of {P} tokens + {G - 1} decode "
                      f"steps, {t:.1f} s on the host; scaled to the {cfg['layers']}-layer model (every layer "
                      f"costs the same, and the oracle's cost is linear in the batch): tokens/s = "
                      f"{S}*gen/(t*layers); weight generation and packing ({setup_s:.0f} s, load-time) not timed",
            "sample_seconds": round(t, 2), "host": hostd}


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
    if args.kernel_only == "quantize":
        return kernel_only_quantize(fq, synth, torch, cfg, args)
    if args.kernel_only == "prefill_attention":
        return kernel_only_prefill_attention(fq, synth, torch, cfg, args)
    return kernel_only_decode_attention(fq, synth, torch, cfg, args)


def kernel_only_quantize(fq, synth, torch, cfg, args):
    """Load-time quantisation of the largest weight of a layer (FC1, [ffn, hidden]
    fp16 ~ N(0, 0.02) from the seeded generator), three launches."""
    n, k = cfg["ffn"], cfg["hidden"]
    w = torch.empty((n, k), dtype=torch.float16, device="cuda")
    from synth.gen import layer_stream
    fq.fq_synth_normal_f16(w, args.seed, layer_stream(0, "w_fc1"), 0.02)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device="cuda")
    for _ in range(3):
        fq.fq_quantize(w, codes, meta.view(torch.int16))
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": args.kernel_only, "launches": [[n, k]] * 3}), flush=True)


def kernel_only_prefill_attention(fq, synth, torch, cfg, args):
    """Causal attention of one prompt chunk as the prefill launches it: the
    sequences of one --max-tokens chunk x all heads x the prompt, over a packed
    cache (seeded random codes; the {min, scale} pairs are constant) -- three
    launches."""
    h, H, P, G = cfg["hidden"], cfg["heads"], cfg["prompt"], cfg["gen"]
    d, S = h // H, P + G - 1
    B = max(1, min(cfg["batch"], args.max_tokens // P))
    gen = torch.Generator(device="cuda").manual_seed(args.seed)
    kc = torch.randint(0, 256, (B, H, S, d // 2), dtype=torch.uint8, device="cuda", generator=gen)
    vc = torch.randint(0, 256, (B, H, S, d // 2), dtype=torch.uint8, device="cuda", generator=gen)
    km = torch.empty((B, H, S, d // 64, 2), dtype=torch.float16, device="cuda")
    km[..., 0], km[..., 1] = -0.05, 0.006
    vm = km.clone()
    kv = fq.kv_layer_view(kc, km.view(torch.int16), vc, vm.view(torch.int16))
    q = torch.empty((B * P, 3 * h), dtype=torch.float16, device="cuda")
    fq.fq_synth_normal_f16(q, args.seed, synth.STREAM["aux"], 1.0)
    out = torch.empty((B * P, h), dtype=torch.float16, device="cuda")
    for _ in range(3):
        fq.fq_prefill_attention(q, kv, 0, B, P, 0, out, ldq=3 * h)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": args.kernel_only, "launches": [[B, H, P, d]] * 3}), flush=True)


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


class GenerationRun:
    """One step = one greedy generation of the workload (fq_generate)."""

    def __init__(self, fq, synth, torch, cfg, args):
        self.fq, self.cfg = fq, cfg
        B, P, G = cfg["batch"], cfg["prompt"], cfg["gen"]
        self.model = fq.Model(cfg["hidden"], cfg["heads"], cfg["ffn"], cfg["layers"], vocab=cfg["vocab"],
                              max_pos=P + G + 2, compress_weight=cfg["compress_weight"],
                              resident_layers=cfg.get("resident_layers", -1), host_layers=cfg.get("host_layers", 0),
                              overlap=True, max_tokens=args.max_tokens, compress_cache=cfg.get("compress_cache", True),
                              cache_resident_layers=cfg.get("cache_resident_layers", -1))
        self.model.init_random(args.seed)
        self.kv = fq.KVCache(self.model, B, P + G)
        self.ids = synth.token_ids(args.seed, synth.STREAM["prompt"], (B, P), cfg["vocab"])
        self.tokens = B * G
        last = [time.time()]

        def progress(done, total):  # generations of several minutes report a completed token every ~20 s
            if time.time() - last[0] > 20 or done == 1 and time.time() - last[0] > 5:
                log(f"[bench] token {done}/{total} done")
                last[0] = time.time()

        fq.fq_set_progress(progress)

    def step(self):
        _, st = self.fq.fq_generate(self.model, self.kv, self.ids, self.cfg["gen"])
        return {"prefill_s": st.prefill_s, "decode_s": st.decode_s, "h2d_bytes": st.h2d_bytes, "h2d_s": st.h2d_s,
                "kv_h2d_bytes": st.kv_h2d_bytes, "kv_d2h_bytes": st.kv_d2h_bytes}

    def close(self):
        self.fq.fq_set_progress(None)
        self.kv.close()
        self.model.close()


class LayerRun:
    """One step = one layer over the batch: prefill of the prompt (all sequences in
    one call), then `gen` decode steps, each consuming the next seeded hidden state
    of every sequence (teacher-forced).  Timed with HIP events on the stream the
    layer runs on."""

    def __init__(self, fq, synth, torch, cfg, args):
        self.fq, self.torch, self.cfg = fq, torch, cfg
        B, P, T, h = cfg["batch"], cfg["prompt"], cfg["gen"], cfg["hidden"]
        self.model = fq.Model(h, cfg["heads"], cfg["ffn"], 1, compress_weight=cfg["compress_weight"],
                              max_tokens=B * P, compress_cache=cfg.get("compress_cache", True))
        self.model.init_random(args.seed)
        self.kv = fq.KVCache(self.model, B, P + T)
        hidden = torch.empty((B, P + T, h), dtype=torch.float16, device="cuda")
        fq.fq_synth_normal_f16(hidden, args.seed, synth.STREAM["hidden"], 1.0)
        self.x = hidden[:, :P].reshape(B * P, h).contiguous()
        self.xt = [hidden[:, P + t].contiguous() for t in range(T)]
        self.y = torch.empty_like(self.x)
        self.yt = torch.empty_like(self.xt[0])
        self.tokens = B * T

    def step(self):
        torch, fq, c = self.torch, self.fq, self.cfg
        B, P, T = c["batch"], c["prompt"], c["gen"]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        fq.fq_layer_step(self.model, 0, self.kv, 0, B, P, 0, self.x, self.y)
        ev[1].record()
        for t in range(T):
            fq.fq_layer_step(self.model, 0, self.kv, 0, B, 1, P + t, self.xt[t], self.yt)
        ev[2].record()
        ev[2].synchronize()
        return {"prefill_s": ev[0].elapsed_time(ev[1]) / 1e3, "decode_s": ev[1].elapsed_time(ev[2]) / 1e3}

    def close(self):
        self.kv.close()
        self.model.close()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the batch dimension would shard over "
              f"GPUs with no exchange, which this program does not launch.", file=sys.stderr)
        sys.exit(2)
    cfg = CONFIGS[args.config]
    if args.cpu_baseline_only:
        print(json.dumps({"cpu_baseline": cpu_baseline(cfg, args.seed, args.cpu_workers)}), flush=True)
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
    t0 = time.time()
    run = (LayerRun if cfg.get("layer_only") else GenerationRun)(fq, synth, torch, cfg, args)
    torch.cuda.synchronize()
    log(f"[bench] {args.config}: model + cache ready in {time.time() - t0:.1f} s")
    # The CPU oracle sample runs in a child process (no GPU use) during the
    # untimed warmup steps, on all but one of the host share's cores (the other
    # stays with this process, which launches the GPU work), and is collected
    # before the timed steps start.
    oracle_proc = None
    if not args.no_cpu_baseline:
        nw = max(1, min(16, os.cpu_count() or 1) - 1)
        env = dict(os.environ, OMP_NUM_THREADS=str(nw), OPENBLAS_NUM_THREADS=str(nw), MKL_NUM_THREADS=str(nw))
        oracle_proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--config",
                                        args.config, "--seed", str(args.seed), "--cpu-workers", str(nw)],
                                       stdout=subprocess.PIPE, env=env, text=True)
        log(f"[bench] CPU oracle sample started ({nw} host threads, during the warmup steps)")
    # warmup steps: every launch timed (the per-class table comes from the last one)
    table = None
    for w in range(args.warmup):
        fq.fq_timing_start()
        st = run.step()
        table = fq.fq_timing_stop()
        log(f"[bench] warmup {w}: {run.tokens / (st['prefill_s'] + st['decode_s']):.2f} tok/s "
            f"(prefill {st['prefill_s']:.3f} s, decode {st['decode_s']:.3f} s)")
    cpu_res = None
    if oracle_proc is not None:
        out, _ = oracle_proc.communicate()
        try:
            if oracle_proc.returncode != 0:
                raise RuntimeError(f"exit status {oracle_proc.returncode}")
            cpu_res = json.loads(out.strip().splitlines()[-1])["cpu_baseline"]
            cpu_res["sample"] += "; run in a child process during the GPU's untimed warmup steps"
            log(f"[bench] CPU oracle sample: {cpu_res['sample_seconds']} s")
        except Exception as e:  # the GPU measurement stands without it
            log(f"[bench] CPU oracle sample failed ({e}); no cpu_baseline")
            cpu_res = None
    # timed steps: only the dominant class's launches carry events
    dominant = max(table.items(), key=lambda kv: kv[1]["seconds"])[0] if table else "gemm_prefill"
    torch.cuda.synchronize()
    fq.fq_timing_start([dominant])
    stats = []
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        st = run.step()
        stats.append(st)
        log(f"[bench] step {s_}: {run.tokens / (st['prefill_s'] + st['decode_s']):.2f} tok/s "
            f"(prefill {st['prefill_s']:.3f} s, decode {st['decode_s']:.3f} s)")
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    kstats = fq.fq_timing_stop()
    ms_per_step = t_total / args.steps * 1e3
    value = run.tokens * args.steps / t_total
    mean = lambda k: float(np.mean([st[k] for st in stats]))
    phases = {"prefill_s": round(mean("prefill_s"), 4), "decode_s": round(mean("decode_s"), 4)}
    if not cfg.get("layer_only"):
        phases.update({"h2d_GB": round(mean("h2d_bytes") / 1e9, 2), "h2d_busy_s": round(mean("h2d_s"), 3),
                       "kv_h2d_GB": round(mean("kv_h2d_bytes") / 1e9, 2),
                       "kv_d2h_GB": round(mean("kv_d2h_bytes") / 1e9, 2)})
    c = cfg
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded random-init weights, uniform prompt ids / seeded hidden states)",
        "config": {"workload": c["desc"], "config": args.config, "layers": c["layers"], "hidden": c["hidden"],
                   "heads": c["heads"], "ffn": c["ffn"], "vocab": c["vocab"], "global_batch": c["batch"],
                   "prompt": c["prompt"], ("decode_steps" if c.get("layer_only") else "gen"): c["gen"], "group": 64,
                   "parallelism": "single GPU"},
        "phases": phases,
        "roofline": roofline(dominant, kstats.get(dominant), args.config),
        "kernels": kernel_table(table, args.config) if table else None,
    }
    if c.get("layer_only"):
        res["metric_form"] = "per layer: B*T / (layer prefill + T decode steps)"
    run.close()
    del run
    torch.cuda.empty_cache()
    if cpu_res is not None:
        res["cpu_baseline"] = cpu_res
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
