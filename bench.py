"""Benchmark of the NVFP4 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

Headline step (one JSON line on stdout): NVFP4 quantize + dequantize of 64
MoE expert weight matrices [2048 x 7168] bf16 (N(0, 0.02) with 0.1% x50
outliers), one FP32 tensor scale per expert, inputs resident in HBM.
value = algorithmic bytes of the step (each input byte read once, each
output byte written once) / wall time per step, in GB/s.

Extra records in the same line ("rows"): the single 1024x1024 tensor, the
16384 x 7168 activation quantize (two-kernel and fused), the 32x8x128 KV
cache (512 appends of 256 tokens, decode QK over 131072 tokens, 32 query
heads, plus decode attention), the 8192 x 2048 x 7168 block-scaled GEMM and
the grouped MoE GEMM (16384 tokens routed top-8 over 64 experts) in TFLOP/s,
MXFP4 against NVFP4 on the same data (codec and GEMM speed, error), and the
training-recipe quantize variants (2D weight scales, column-wise RHT + SR
Wgrad operands) --
each with its roofline fraction.  Every kernel time comes from HIP events recorded on
the stream the kernels run on.

cpu_baseline: the CPU oracle (the parity reference, not tuned) timed on a
bounded sample of the headline workload on this host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA, TFLOP/s
# What an MFMA-only loop sustains on this device (16 independent chains of
# v_mfma_f32_32x32x16_f16, or of the scaled fp4 32x32x64 MFMA, per wave; the
# shader clock then runs at about 2.0 GHz, not the 2.4 GHz of the spec).
# Context next to the spec peak, not a roofline.
MEASURED_F16_MFMA_TFLOPS = 2190.0
MEASURED_FP4_MFMA_TFLOPS = 8500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-extras", action="store_true", help="headline step only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--rows-only", default="",
                   help="comma list of extra rows to run (experts,single,acts,kv,gemm,moe,mx,train,steady)")
    p.add_argument("--traffic-kernels", action="store_true",
                   help="only launch every benchmarked kernel on its benchmarked shape (3 times each) and a "
                        "1 GiB device copy: the workload of the rocprofv3 --pmc counter runs")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class EventTimer:
    """HIP events on the current stream, one per kernel: each launch is timed
    from the event recorded after the previous launch to the event recorded
    after it, so consecutive kernels share a boundary and only one event
    marker sits between two launches.  The first launch after mark() (the
    stream idle) is not timed: its interval would hold the host's launch
    latency.  Mean milliseconds."""

    def __init__(self, torch):
        self.torch = torch
        self.last = None
        self.pairs = {}

    def _event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def mark(self):
        self.last = None

    def lap(self, name):
        e = self._event()
        if self.last is not None:
            self.pairs.setdefault(name, []).append((self.last, e))
        self.last = e

    def mean_ms(self, name):
        v = [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]
        return sum(v) / len(v) if v else None

    def reset(self):
        self.pairs = {}
        self.last = None


# The sources the headline kernels (quantize and dequantize) are built from.
HEADLINE_SOURCES = ("codec.hip", "common.hpp")


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_block_scaled_06_amd", "csrc")
    for f in HEADLINE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken from the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- workloads
def bytes_quantize(n_elem, n_tensors):
    return n_elem * 2 + n_elem // 2 + n_elem // 16 + 4 * n_tensors


def bytes_dequant(n_elem, n_tensors):
    return n_elem // 2 + n_elem // 16 + 4 * n_tensors + 2 * n_elem


def run_headline(nv, synth, torch, steps, warmup, steady_steps=0, steady_skip=20):
    """The headline step on the 64 experts.  With steady_steps > 0 the same
    step first runs that many times as its own row (per-launch laps over
    all but the first steady_skip), on the same tensors and with no other
    GPU work between it and the headline's W + K steps: a device that has
    just come from idle or from other kernels runs this alternation's first
    ~20-25 quantize launches up to 45% slower before it settles, so the row
    both reports the settled step and leaves the device settled.
    Returns (headline, steady row or None)."""
    E, R, C = 64, 2048, 7168
    log(f"headline: experts {E}x{R}x{C}: generating inputs on the GPU")
    x = synth.experts(E, R, C, device="cuda")
    n = E * R * C
    q = torch.empty((E, R, C // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((E, R, C // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty((E,), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    ws = nv.make_workspace(E, R, C)
    flags = "fused"               # single persistent launch, each input byte read once; both modes are timed in "rows"
    bq, bd = bytes_quantize(n, E), bytes_dequant(n, E)
    timer = EventTimer(torch)

    def step():
        nv.quantize(x, flags=flags, workspace=ws, out=(q, sf, g))
        timer.lap("quantize")
        nv.dequantize(q, sf, g, out=y)
        timer.lap("dequantize")

    steady = None
    if steady_steps > 0:
        timer.mark()
        for i in range(steady_steps):
            if i == steady_skip:
                timer.pairs = {}              # drop the first laps, keep the boundary event
            step()
        torch.cuda.synchronize()
        mq, md = timer.mean_ms("quantize"), timer.mean_ms("dequantize")
        steady = {"steps": steady_steps, "timed": steady_steps - steady_skip,
                  "quantize": {"ms": mq, **roof(bq, mq, HBM_PEAK_GBS, "GB/s")},
                  "dequantize": {"ms": md, **roof(bd, md, HBM_PEAK_GBS, "GB/s")},
                  "step": {"ms": mq + md, **roof(bq + bd, mq + md, HBM_PEAK_GBS, "GB/s")}}
        log("steady row done:", json.dumps(steady))
        timer.reset()
    timer.mark()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.mark()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    res = {
        "ms_per_step": ms_step,
        "value_gbs": (bq + bd) / (ms_step * 1e-3) / 1e9,
        "quantize_ms": timer.mean_ms("quantize"),
        "dequantize_ms": timer.mean_ms("dequantize"),
        "quantize_bytes": bq,
        "dequantize_bytes": bd,
        "flags": flags,
    }
    del x, q, sf, g, y, ws
    torch.cuda.empty_cache()
    return res, steady


def _fused_ok(nv):
    """True when the library accepts the persistent single-launch mode."""
    import torch
    x = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")
    try:
        nv.quantize(x, flags="fused")
        torch.cuda.synchronize()
        return True
    except nv.NVFP4Error:
        return False


def flush_caches(torch, buf):
    """Evicts L2 and the 256 MB Infinity Cache by reading a 512 MiB buffer.
    A read leaves clean lines behind, so the timed kernel pays for no
    write-back of the flush itself."""
    buf.view(torch.int64).sum()


def hold_stream(torch):
    """Keeps the stream busy for some tens of microseconds (a spin kernel), so
    that an event recorded next fires when the GPU reaches it, after the host
    has already queued the call being timed: the pair then brackets the GPU
    work, not the host's marshalling and launch latency."""
    torch.cuda._sleep(100_000)


def timed(torch, fn, reps, flush=None, warm=2):
    for _ in range(warm):
        fn()
    ms = []
    for _ in range(reps):
        if flush is not None:
            flush()
        hold_stream(torch)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2]


def roof(bytes_or_flops, ms, peak, unit):
    ach = bytes_or_flops / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    return {"achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4)}


def run_extras(nv, synth, torch, which):
    rows = {}
    fbuf = torch.ones(512 * 2 ** 20, dtype=torch.uint8, device="cuda")
    flush = lambda: flush_caches(torch, fbuf)
    fused = _fused_ok(nv)
    if "experts" in which:
        x = synth.experts(device="cuda")
        ws = nv.make_workspace(64, 2048, 7168)
        q, sf, g = nv.quantize(x, workspace=ws)
        n = x.numel()
        r = {}
        for fl in (["two_kernel", "fused"] if fused else ["two_kernel"]):
            m = timed(torch, lambda: nv.quantize(x, flags=fl, workspace=ws, out=(q, sf, g)), 10)
            r[fl] = {"ms": m, **roof(bytes_quantize(n, 64), m, HBM_PEAK_GBS, "GB/s")}
        rows["experts_64x2048x7168_quantize_modes"] = r
        del x, q, sf, g
        torch.cuda.empty_cache()
    if "single" in which:
        x = synth.single(device="cuda")
        ws = nv.make_workspace(1, 1024, 1024)
        q, sf, g = nv.quantize(x, workspace=ws)
        y = torch.empty_like(x)
        n = 1024 * 1024
        mq = timed(torch, lambda: nv.quantize(x, workspace=ws, out=(q, sf, g)), 50)
        mf = timed(torch, lambda: nv.quantize(x, flags="fused", workspace=ws, out=(q, sf, g)), 50) if fused else None
        md = timed(torch, lambda: nv.dequantize(q, sf, g, out=y), 50)
        rows["single_1024x1024"] = {
            "note": "2.7 MB working set: launch-bound and cache-resident; warm medians of HIP events around "
                    "one call with preallocated outputs (the stream held busy first, so host latency is excluded)",
            "quantize": {"ms": mq, **roof(bytes_quantize(n, 1), mq, HBM_PEAK_GBS, "GB/s")},
            "dequantize": {"ms": md, **roof(bytes_dequant(n, 1), md, HBM_PEAK_GBS, "GB/s")}}
        if mf is not None:
            rows["single_1024x1024"]["quantize_fused"] = {"ms": mf, **roof(bytes_quantize(n, 1), mf, HBM_PEAK_GBS,
                                                                           "GB/s")}
        del x, q, sf, g, y
    if "acts" in which:
        x = synth.activations(device="cuda")
        n = x.numel()
        ws = nv.make_workspace(1, 16384, 7168)
        q, sf, g = nv.quantize(x, workspace=ws)
        r = {}
        for fl in (["two_kernel", "fused"] if fused else ["two_kernel"]):
            m = timed(torch, lambda: nv.quantize(x, flags=fl, workspace=ws, out=(q, sf, g)), 20, flush)
            r[fl] = {"ms": m, **roof(bytes_quantize(n, 1), m, HBM_PEAK_GBS, "GB/s")}
        rows["activations_16384x7168_quantize"] = r
        del x, q, sf, g
    if "kv" in which:
        L, H, D, T, C = 32, 8, 128, 131072, 256
        log("kv: generating 512 chunks of K/V on the GPU (16 GiB bf16)")
        chunks = [synth.kv_chunk(c, device="cuda") for c in range(T // C)]
        kg, vg = calibrate_kv_scales(nv, torch, chunks, L, H)        # untimed
        cache = nv.KVCache(L, H, D, T, kg, vg, device="cuda")
        qv = synth.kv_query(device="cuda")
        logits = torch.empty((L, 4 * H, T), dtype=torch.float32, device="cuda")

        def appends():
            for c, (k, v) in enumerate(chunks):
                cache.append(c * C, k, v)
        ma = timed(torch, appends, 5, flush, warm=1)
        side = [torch.cuda.Stream(), torch.cuda.Stream()]       # default priority

        def appends_two_streams():
            # consecutive appends write disjoint token ranges: alternate two
            # streams so one launch's ramp overlaps the other's tail
            main = torch.cuda.current_stream()
            for sd in side:
                sd.wait_stream(main)
            for c, (k, v) in enumerate(chunks):
                cache.append(c * C, k, v, stream=side[c & 1])
            for sd in side:
                main.wait_stream(sd)
        ma2 = timed(torch, appends_two_streams, 5, flush, warm=1)
        mqk = timed(torch, lambda: cache.decode_qk(qv, T, out=logits), 20, flush)
        att = torch.empty((L, 4 * H, D), dtype=torch.float32, device="cuda")
        aws = torch.empty(max(cache.attention_workspace_bytes(4 * H, T), 16), dtype=torch.uint8, device="cuda")
        matt = timed(torch, lambda: cache.decode_attention(qv, T, D ** -0.5, out=att, workspace=aws), 20, flush)
        RL = 4                                         # kv_read: K and V of 4 layers, every token, to bf16
        kr = torch.empty((RL, H, T, D), dtype=torch.bfloat16, device="cuda")
        vr = torch.empty_like(kr)
        mrd = timed(torch, lambda: cache.read(0, RL, 0, T, k_out=kr, v_out=vr), 20, flush)
        del kr, vr
        nvals = L * H * D * T
        app_bytes = 2 * nvals * 2 + 2 * (nvals // 2 + nvals // 16)
        qk_bytes = nvals // 2 + nvals // 16 + L * 4 * H * T * 4 + qv.numel() * 2
        att_bytes = 2 * (nvals // 2 + nvals // 16) + qv.numel() * 2 + att.numel() * 4   # K and V once
        rvals = RL * H * D * T
        rd_bytes = 2 * (rvals // 2 + rvals // 16) + 2 * rvals * 2                        # codes + scales in, bf16 out
        rows["kv_32x8x128_131072"] = {
            "append_512x256": {"ms": ma, "ms_per_chunk": ma / (T // C), **roof(app_bytes, ma, HBM_PEAK_GBS, "GB/s")},
            "append_512x256_two_streams": {"ms": ma2, "ms_per_chunk": ma2 / (T // C),
                                           **roof(app_bytes, ma2, HBM_PEAK_GBS, "GB/s")},
            "decode_qk_32q": {"ms": mqk, **roof(qk_bytes, mqk, HBM_PEAK_GBS, "GB/s")},
            "decode_attention_32q": {"ms": matt, **roof(att_bytes, matt, HBM_PEAK_GBS, "GB/s")},
            "read_4_layers_all_tokens": {"ms": mrd, **roof(rd_bytes, mrd, HBM_PEAK_GBS, "GB/s")},
            "cache_bytes": cache.nbytes()}
        del chunks, cache, logits
        torch.cuda.empty_cache()
    if "gemm" in which:
        a, b = synth.gemm_operands(device="cuda")
        aq, asf, ag = nv.quantize(a)
        bq, bsf, bg = nv.quantize(b)
        c = torch.empty((8192, 2048), dtype=torch.float32, device="cuda")
        m = timed(torch, lambda: nv.gemm(aq, asf, ag, bq, bsf, bg, out=c), 20)
        flops = 2 * 8192 * 2048 * 7168
        r = roof(flops, m, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s")
        rows["gemm_8192x2048x7168"] = {"ms": m, "bound": "mfma", **r,
                                       "measured_mfma_only_tflops": MEASURED_F16_MFMA_TFLOPS,
                                       "frac_of_measured": round(r["achieved"] / MEASURED_F16_MFMA_TFLOPS, 4)}
        del a, b, aq, bq, c
    if "moe" in which:
        rows["moe_grouped_gemm_16384x8_64x2048x7168"] = run_moe(nv, synth, torch)
    if "mx" in which:
        rows["mxfp4_vs_nvfp4"] = run_mx(nv, synth, torch)
    if "train" in which:
        rows["training_variants"] = run_train(nv, synth, torch)
    del fbuf
    torch.cuda.empty_cache()
    return rows


def calibrate_kv_scales(nv, torch, chunks, L, H):
    """Per-(layer, KV head) tensor scales of K and V, fixed at cache creation
    from a calibration pass over the whole stream: the codec's tensor-scale
    rule g = RN32(amax / 2688), applied by nvfp4_quantize to one 16-value
    block per (layer, head) that holds the head's amax over every chunk."""
    kmax = torch.zeros((L, H), dtype=torch.bfloat16, device="cuda")
    vmax = torch.zeros_like(kmax)
    for k, v in chunks:
        kmax = torch.maximum(kmax, k.abs().amax(dim=(1, 3)))
        vmax = torch.maximum(vmax, v.abs().amax(dim=(1, 3)))
    blocks = torch.zeros((2 * L * H, 1, 16), dtype=torch.bfloat16, device="cuda")
    blocks[:, 0, 0] = torch.cat([kmax.reshape(-1), vmax.reshape(-1)])
    _, _, g = nv.quantize(blocks)
    return g[:L * H].reshape(L, H).clone(), g[L * H:].reshape(L, H).clone()


def run_moe(nv, synth, torch):
    """Grouped NVFP4 GEMM of MoE expert linears: 16384 tokens routed top-8 over
    64 experts [2048 x 7168] (seeded uniform routing, 8 distinct experts per
    token), routed activations sorted by expert."""
    T, E, top, N, K = 16384, 64, 8, 2048, 7168
    gen = torch.Generator().manual_seed(106)
    choice = torch.rand((T, E), generator=gen).argsort(dim=1)[:, :top]       # 8 distinct experts per token
    counts = torch.bincount(choice.flatten(), minlength=E)
    offsets = torch.cat([torch.zeros(1, dtype=torch.int64), counts.cumsum(0)]).to(torch.int32).cuda()
    M = int(counts.sum())
    a = synth.activations(tokens=M, channels=K, seed=107, device="cuda")      # routed rows
    aq, asf, ag = nv.quantize(a)
    del a
    w = synth.experts(E, N, K, device="cuda")
    bq, bsf, bg = nv.quantize(w)
    del w
    torch.cuda.empty_cache()
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    m = timed(torch, lambda: nv.grouped_gemm(aq, asf, ag, bq, bsf, bg, offsets, out=c), 10)
    flops = 2 * M * N * K
    res = {"ms": m, "rows": M, "experts": E, "min_rows": int(counts.min()), "max_rows": int(counts.max()),
           "bound": "mfma", **roof(flops, m, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s")}
    del aq, asf, bq, bsf, c
    torch.cuda.empty_cache()
    return res


def _rel_err(torch, y, x):
    d = (y.float() - x.float()).double()
    return float(d.square().sum().sqrt() / x.double().square().sum().sqrt())


def run_mx(nv, synth, torch):
    """MXFP4 against NVFP4 on the same synthetic data: the 64 x 2048 x 7168
    experts tensor through quantize and dequantize (speed and round-trip
    relative Frobenius error), and the 8192 x 2048 x 7168 GEMM (speed, and the
    relative error of C on 64 sampled rows against the fp32 product of the
    unquantized bf16 operands)."""
    res = {}
    x = synth.experts(device="cuda")
    n = x.numel()
    mq_bytes = 2 * n + n // 2 + n // 32
    q, sf = nv.mxfp4_quantize(x)
    y = nv.mxfp4_dequantize(q, sf)
    mq = timed(torch, lambda: nv.mxfp4_quantize(x, out=(q, sf)), 10)
    md = timed(torch, lambda: nv.mxfp4_dequantize(q, sf, out=y), 10)
    mx_err = _rel_err(torch, y, x)
    del q, sf
    ws = nv.make_workspace(64, 2048, 7168)
    nq, nsf, ng = nv.quantize(x, workspace=ws)
    nvfp4_err = _rel_err(torch, nv.dequantize(nq, nsf, ng, out=y), x)
    del nq, nsf, ng, y, x
    torch.cuda.empty_cache()
    res["experts_64x2048x7168"] = {
        "mxfp4_quantize": {"ms": mq, **roof(mq_bytes, mq, HBM_PEAK_GBS, "GB/s")},
        "mxfp4_dequantize": {"ms": md, **roof(mq_bytes, md, HBM_PEAK_GBS, "GB/s")},
        "round_trip_rel_err": {"mxfp4": round(mx_err, 6), "nvfp4": round(nvfp4_err, 6)},
        "bits_per_value": {"mxfp4": 4.25, "nvfp4": 4.5}}
    a, b = synth.gemm_operands(device="cuda")
    rows = torch.from_numpy(__import__("numpy").random.default_rng(4).choice(8192, 64, replace=False)).cuda()
    ref = a[rows].float() @ b.float().T
    c = torch.empty((8192, 2048), dtype=torch.float32, device="cuda")
    aq, asf = nv.mxfp4_quantize(a)
    bq, bsf = nv.mxfp4_quantize(b)
    mg = timed(torch, lambda: nv.mxfp4_gemm(aq, asf, bq, bsf, out=c), 20)
    mx_gerr = _rel_err(torch, c[rows], ref)
    del aq, asf, bq, bsf
    aq, asf, ag = nv.quantize(a)
    bq, bsf, bg = nv.quantize(b)
    ng = timed(torch, lambda: nv.gemm(aq, asf, ag, bq, bsf, bg, out=c), 20)
    nv_gerr = _rel_err(torch, c[rows], ref)
    flops = 2 * 8192 * 2048 * 7168
    res["gemm_8192x2048x7168"] = {
        "mxfp4": {"ms": mg, "bound": "mfma", "peak_dtype": "fp4", **roof(flops, mg, FP4_MFMA_PEAK_TFLOPS, "TFLOP/s"),
                  "measured_mfma_only_tflops": MEASURED_FP4_MFMA_TFLOPS,
                  "frac_of_measured": round(flops / (mg * 1e-3) / 1e12 / MEASURED_FP4_MFMA_TFLOPS, 4)},
        "nvfp4": {"ms": ng, "bound": "mfma", "peak_dtype": "bf16/f16",
                  **roof(flops, ng, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s")},
        "rel_err_vs_bf16_inputs": {"mxfp4": round(mx_gerr, 6), "nvfp4": round(nv_gerr, 6)}}
    del a, b, aq, asf, bq, bsf, c, ref
    torch.cuda.empty_cache()
    return res


def run_train(nv, synth, torch):
    """Training-recipe quantize variants: the 64 x 2048 x 7168 expert weights
    with 16x16 2D scales (and their transposes), and the 16384 x 7168
    activations as a Wgrad operand (column-wise, RHT, stochastic rounding).
    Algorithmic bytes count one read of x and one write of the outputs; the
    variant path reads x twice (amax pass, encode pass)."""
    res = {}
    x = synth.experts(device="cuda")
    n = x.numel()
    ws = torch.empty(nv.lib().nvfp4_quantize_ex_workspace_bytes(64), dtype=torch.uint8, device="cuda")
    for name, v in (("2d", nv.VAR_2D), ("2d_colwise", nv.VAR_2D | nv.VAR_COLWISE)):
        out = nv.quantize_ex(x, v, workspace=ws)
        m = timed(torch, lambda: nv.quantize_ex(x, v, workspace=ws, out=out), 10)
        res[f"experts_64x2048x7168_{name}"] = {"ms": m, **roof(bytes_quantize(n, 64), m, HBM_PEAK_GBS, "GB/s")}
        del out
    del x
    torch.cuda.empty_cache()
    a = synth.activations(device="cuda")
    n = a.numel()
    for name, v in (("rowwise_sr", nv.VAR_SR), ("colwise_rht_sr", nv.VAR_COLWISE | nv.VAR_RHT | nv.VAR_SR)):
        out = nv.quantize_ex(a, v, rht_signs=0x6A3C, seed=77, workspace=ws)
        m = timed(torch, lambda: nv.quantize_ex(a, v, rht_signs=0x6A3C, seed=77, workspace=ws, out=out), 10)
        res[f"activations_16384x7168_{name}"] = {"ms": m, **roof(bytes_quantize(n, 1), m, HBM_PEAK_GBS, "GB/s")}
        del out
    del a, ws
    torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(synth, torch):
    """The oracle, untouched, on the whole headline workload: quantize +
    dequantize of all 64 expert matrices, two passes (about 10 s of CPU work
    on a 16-core host)."""
    import numpy as np
    import oracle
    E, reps = 64, 2
    x = synth.experts(E, 2048, 7168, device="cuda")
    xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
    del x
    torch.cuda.empty_cache()
    n = E * 2048 * 7168
    t0 = time.perf_counter()
    for _ in range(reps):
        q, sf, g = oracle.quantize(xb)
        oracle.dequantize(q, sf, g)
        del q, sf, g
    dt = time.perf_counter() - t0
    nbytes = reps * (bytes_quantize(n, E) + bytes_dequant(n, E))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"quantize+dequantize of all {E} expert matrices ({E}x2048x7168), {reps} passes, "
                      f"{dt:.2f} s wall"}


def traffic_kernels(nv, synth, torch):
    """The workload of the rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE,
    MFMA and VALU busy cycles): every benchmarked kernel on its benchmarked
    shape, three launches each unless stated, and a plain 1 GiB
    device-to-device copy whose byte counts (1 GiB read, 1 GiB written)
    calibrate the HBM byte counters.  A kernel's workload is told apart in
    the counter files by its grid size."""
    E, R, C = 64, 2048, 7168
    x = synth.experts(E, R, C, device="cuda")
    ws = nv.make_workspace(E, R, C)
    q, sf, g = nv.quantize(x, flags="fused", workspace=ws)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for fl in ("fused", "two_kernel"):
        for _ in range(3):
            nv.quantize(x, flags=fl, workspace=ws, out=(q, sf, g))
    for _ in range(3):
        nv.dequantize(q, sf, g, out=y)
    xw = torch.empty(nv.lib().nvfp4_quantize_ex_workspace_bytes(64), dtype=torch.uint8, device="cuda")
    for v in (nv.VAR_2D, nv.VAR_2D | nv.VAR_COLWISE):
        out = nv.quantize_ex(x, v, workspace=xw)
        for _ in range(2):
            nv.quantize_ex(x, v, workspace=xw, out=out)
        del out
    mq, msf = nv.mxfp4_quantize(x)
    for _ in range(3):
        nv.mxfp4_quantize(x, out=(mq, msf))
    for _ in range(3):
        nv.mxfp4_dequantize(mq, msf, out=y)
    torch.cuda.synchronize()
    del x, y, q, sf, g, ws, mq, msf
    torch.cuda.empty_cache()
    log("traffic: experts done")
    a = synth.activations(device="cuda")
    ws = nv.make_workspace(1, 16384, 7168)
    q, sf, g = nv.quantize(a, workspace=ws)
    for fl in ("fused", "two_kernel"):
        for _ in range(3):
            nv.quantize(a, flags=fl, workspace=ws, out=(q, sf, g))
    for v in (nv.VAR_SR, nv.VAR_COLWISE | nv.VAR_RHT | nv.VAR_SR):
        out = nv.quantize_ex(a, v, rht_signs=0x6A3C, seed=77, workspace=xw)
        for _ in range(2):
            nv.quantize_ex(a, v, rht_signs=0x6A3C, seed=77, workspace=xw, out=out)
        del out
    torch.cuda.synchronize()
    del a, q, sf, g, ws, xw
    torch.cuda.empty_cache()
    log("traffic: activations done")
    L, H, D, T, CH = 32, 8, 128, 131072, 256
    chunks = [synth.kv_chunk(c, device="cuda") for c in range(T // CH)]
    kg, vg = calibrate_kv_scales(nv, torch, chunks, L, H)
    cache = nv.KVCache(L, H, D, T, kg, vg, device="cuda")
    for c, (k, v) in enumerate(chunks):                  # 512 appends
        cache.append(c * CH, k, v)
    del chunks
    torch.cuda.empty_cache()
    qv = synth.kv_query(device="cuda")
    logits = torch.empty((L, 4 * H, T), dtype=torch.float32, device="cuda")
    att = torch.empty((L, 4 * H, D), dtype=torch.float32, device="cuda")
    aws = torch.empty(max(cache.attention_workspace_bytes(4 * H, T), 16), dtype=torch.uint8, device="cuda")
    kr = torch.empty((4, H, T, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.empty_like(kr)
    for _ in range(3):
        cache.decode_qk(qv, T, out=logits)
    for _ in range(3):
        cache.decode_attention(qv, T, D ** -0.5, out=att, workspace=aws)
    for _ in range(3):
        cache.read(0, 4, 0, T, k_out=kr, v_out=vr)
    torch.cuda.synchronize()
    del cache, logits, att, aws, kr, vr
    torch.cuda.empty_cache()
    log("traffic: kv done")
    a, b = synth.gemm_operands(device="cuda")
    aq, asf, ag = nv.quantize(a)
    bq, bsf, bg = nv.quantize(b)
    c = torch.empty((8192, 2048), dtype=torch.float32, device="cuda")
    for _ in range(3):
        nv.gemm(aq, asf, ag, bq, bsf, bg, out=c)
    maq, masf = nv.mxfp4_quantize(a)
    mbq, mbsf = nv.mxfp4_quantize(b)
    for _ in range(3):
        nv.mxfp4_gemm(maq, masf, mbq, mbsf, out=c)
    torch.cuda.synchronize()
    del a, b, aq, asf, bq, bsf, maq, masf, mbq, mbsf, c
    torch.cuda.empty_cache()
    Tm, top, N, K = 16384, 8, 2048, 7168
    gen = torch.Generator().manual_seed(106)
    choice = torch.rand((Tm, E), generator=gen).argsort(dim=1)[:, :top]
    counts = torch.bincount(choice.flatten(), minlength=E)
    offsets = torch.cat([torch.zeros(1, dtype=torch.int64), counts.cumsum(0)]).to(torch.int32).cuda()
    M = int(counts.sum())
    ra = synth.activations(tokens=M, channels=K, seed=107, device="cuda")
    raq, rasf, rag = nv.quantize(ra)
    del ra
    w = synth.experts(E, N, K, device="cuda")
    wq, wsf, wg = nv.quantize(w)
    del w
    torch.cuda.empty_cache()
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for _ in range(2):
        nv.grouped_gemm(raq, rasf, rag, wq, wsf, wg, offsets, out=c)
    torch.cuda.synchronize()
    del raq, rasf, wq, wsf, c
    torch.cuda.empty_cache()
    log("traffic: gemms done")
    src = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("traffic kernels done")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the multi-GPU design "
              "is documented, not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_block_scaled_06_amd as nv
    import synth
    nv.lib()                       # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.traffic_kernels:
        traffic_kernels(nv, synth, torch)
        return
    # The CPU leg first (the GPU idles meanwhile), then the extra rows, then
    # the headline step: a freshly started device takes some tens of
    # milliseconds of this traffic before its memory and clock state settle
    # (the fused quantize's first ~40 launches after a start vary between
    # 0.42 and 0.53 ms, then hold at 0.415-0.42 ms), so the headline runs on
    # the settled device.  With --no-extras it runs first.
    cpu = None if args.no_cpu else cpu_baseline(synth, torch)
    rows = {}
    which = []
    if not args.no_extras:
        which = (args.rows_only.split(",") if args.rows_only
                 else ["experts", "single", "acts", "kv", "gemm", "moe", "mx", "train", "steady"])
        rows = run_extras(nv, synth, torch, which)
        log("extras done")
    head, steady = run_headline(nv, synth, torch, args.steps, args.warmup, 60 if "steady" in which else 0)
    if steady is not None:
        rows["experts_quantize_dequantize_steady"] = steady
    log("headline done:", json.dumps(head))
    dom = "quantize" if head["quantize_ms"] >= head["dequantize_ms"] else "dequantize"
    dom_bytes = head[f"{dom}_bytes"]
    dom_ms = head[f"{dom}_ms"]
    kname = {"quantize": "fused_reg8_kernel<14> (nvfp4_quantize, fused)" if head["flags"] == "fused"
             else "nvfp4_quantize (two_kernel)", "dequantize": "dequant_kernel"}[dom]
    r = roof(dom_bytes, dom_ms, HBM_PEAK_GBS, "GB/s")
    line = {
        "metric": "NVFP4 quantize/dequant GB/s (% of 8 TB/s HBM); block-scaled GEMM TFLOPS",
        "value": round(head["value_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; N(0,0.02) with Bernoulli(0.001) x50 outliers)",
        "config": {"workload": "moe_expert_weights_quantize_dequantize", "experts": 64, "rows": 2048,
                   "cols": 7168, "block": 16, "quantize_flags": head["flags"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": r["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r["frac"], "traffic": traffic_for(dom),
                     "ms_per_launch": round(dom_ms, 4), "algorithmic_bytes_per_launch": dom_bytes},
        "cpu_baseline": cpu,
        "kernels_ms": {"quantize": round(head["quantize_ms"], 4), "dequantize": round(head["dequantize_ms"], 4)},
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
