"""Benchmark of the canvas denoising hot path on one MI355X.

Workload (one bench "step" = one pass of the whole path): the full-width synthetic decoder
(30 layers, d_model 2816, 16/8 heads of 256, 128 experts top-8 + 1 shared with inner width 704,
262,144-entry vocabulary, about 25B parameters, bf16, random N(0, 0.02^2) weights) with a
256-token canvas against an 8,192-token N(0,1) cached prompt: canvas 1 runs up to 48
entropy-bound steps with adaptive stop, is encoded and appended to the cache, then canvas 2 runs
the same on the 8,448-token cache and is appended.  Inputs are resident in HBM before timing.

Reported: denoising steps/s (value), tokens/s, the HBM roofline fraction of the MoE gate/up
kernel (the dominant kernel) from HIP events recorded around its launches in the timed region,
and the plain CPU oracle timed on a bounded sample of the same step on the host cores.  Besides,
from HIP events in an untimed pass: the MFMA fraction of the LM head and of attention (algorithmic
flops), the HBM fraction of the MoE down product, and the HBM fraction of the standalone EB
sampler's statistics kernel on the standalone sampler workload (bf16 logits [256 x 262144]:
30% peaked rows with one logit 12 over N(0,1), 40% N(0,2) rows, 30% N(0,0.1) rows).
Also, outside the timed region: the native generation loop (dg_generate) for 512 tokens on the
same cache (`generate`), and the chunked prefill of an 8,192-token prompt in 2,048-token calls
with its MFMA fraction from exact flops (`prefill`; `--prefill-only` runs just that).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "canvas denoise steps/s + tokens/s (256-tok canvas, 1 GPU), % of roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)
HBM_PEAK_GBS = 8000.0
GATEUP_SAMPLE_EVERY = 8
MFMA_BF16_PEAK_TFS = 2500.0
MFMA_FP8_PEAK_TFS = 5000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--cache", type=int, default=8192)
    ap.add_argument("--canvases", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=1)
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill measurement (one JSON object) and exit")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill line")
    ap.add_argument("--no-generate", action="store_true", help="skip the generation-loop line")
    ap.add_argument("--no-sampler", action="store_true",
                    help="skip the standalone sampler line and the measured ceilings")
    ap.add_argument("--long-fp8-only", action="store_true",
                    help="run only the long-context batched fp8 workload (one JSON object)")
    ap.add_argument("--no-long-fp8", action="store_true",
                    help="skip the long-context batched fp8 line")
    ap.add_argument("--long-kv", choices=("e4m3", "bf16"), default="e4m3",
                    help="KV cache type of the long-context batched fp8 line")
    ap.add_argument("--decoder-only", action="store_true",
                    help="only the decoder steps and appends (for hardware-counter runs: no "
                         "prefill, generation loop, standalone sampler, ceilings or CPU oracle)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run only the library's plain copy kernel on buffers of this many MiB "
                         "(known bytes, to scale hardware byte counters) and exit")
    return ap.parse_args()


def copy_calibration(mib, launches=4):
    """Plain device copy of `mib` MiB, `launches` times: each launch reads and writes exactly
    mib MiB, the yardstick for FETCH_SIZE / WRITE_SIZE of the other kernels."""
    import torch
    from block_diffusion_decoding_canvas_amd import driver
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        driver.copy_bytes(dst, src, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    print(json.dumps(dict(copy_bytes_per_launch=n, launches=launches)))


def measured_peaks(driver, mib=1024, launches=5, mfma_iters=20000):
    """Measured ceilings, timed with events on the stream the kernels run on, after one untimed
    launch each: a plain read stream and a plain copy of `mib` MiB buffers (larger than the
    256 MB last-level cache), in bytes moved per second, and the bf16 MFMA loop in flop/s."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    blocks = driver.mfma_loop_blocks()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / launches
    t_read = timed(lambda: driver.read_stream(src, n, word, stream))
    t_copy = timed(lambda: driver.copy_bytes(dst, src, n, stream))
    t_mfma = timed(lambda: driver.mfma_loop(mfma_iters, out, stream))
    assert int(word.item()) == 0   # an even number of words of 0x01010101
    mfma_flops = blocks * 4 * mfma_iters * 8 * 2.0 * 16 * 16 * 32
    del src, dst
    return dict(hbm_read_gbs=round(n / t_read / 1e9, 1), hbm_copy_gbs=round(2.0 * n / t_copy / 1e9, 1),
                mfma_bf16_tfs=round(mfma_flops / t_mfma / 1e12, 1),
                note=("library kernels: read stream and copy on 1 GiB buffers (bytes moved / s), "
                      "16x16x32 bf16 MFMA loop at 2 waves per SIMD; frac_of_measured in the "
                      "roofline lines divides by the read stream (GB/s) or the MFMA loop"))


def moe_gateup_bytes(dims, n_touched):
    """Algorithmic HBM bytes of one gate/up launch: each touched expert's [2F, d] weights and
    the shared expert's once, the token rows once, the SwiGLU activations written once."""
    d, f, fs, k, t = dims["d"], dims["F"], dims["Fs"], dims["top_k"], dims["C"]
    weights = (n_touched * 2 * f * d + 2 * fs * d) * 2
    acts = t * d * 2 + (t * k * f + t * fs) * 2
    return weights + acts


def moe_down_bytes(dims, n_touched):
    """Algorithmic HBM bytes of one down launch: each touched expert's [d, F] weights and the
    shared expert's once, the SwiGLU activations read once, the expert outputs written once."""
    d, f, fs, k, t = dims["d"], dims["F"], dims["Fs"], dims["top_k"], dims["C"]
    weights = (n_touched * d * f + d * fs) * 2
    acts = (t * k * f + t * fs) * 2 + (t * k + t) * d * 2
    return weights + acts


def attention_flops(dims, cache_len, causal):
    """Algorithmic flops of one layer's canvas attention: QK^T and PV over the visible keys (the
    cache, then the canvas: all of it for the decoder, the causal prefix for the encoder)."""
    c, hq, dh = dims["C"], dims["hq"], dims["dh"]
    keys = cache_len + ((c + 1) / 2 if causal else c)
    return 4.0 * hq * c * keys * dh


def prefill_flops(dims, prompt, chunk):
    """Algorithmic flops of the chunked prefill of a `prompt`-token prompt on an empty cache: per
    token and layer the QKV product, causal attention over the cache and the chunk's earlier
    tokens, and (every layer but the last, whose keys and values are all an append adds) the O
    product, the router and the top-k + shared SwiGLU experts."""
    d, hq, hkv, dh = dims["d"], dims["hq"], dims["hkv"], dims["dh"]
    e, k, f, fs, nl = dims["E"], dims["top_k"], dims["F"], dims["Fs"], dims["n_layers"]
    qkv = 2.0 * d * (hq + 2 * hkv) * dh
    rest = 2.0 * d * hq * dh + 2.0 * d * e + k * 6.0 * d * f + 6.0 * d * fs
    keys = prompt * (prompt + 1) / 2.0          # sum over tokens of the keys each one sees
    attn = 4.0 * hq * dh * keys
    return nl * (prompt * qkv + attn) + (nl - 1) * prompt * rest


def prefill_measure(driver, model, dims, dev, prompt=8192, chunk=2048, reps=2):
    """Chunked prefill of a `prompt`-token prompt into an empty cache, `chunk` tokens per call;
    the mean wall time of `reps` timed prefills after one untimed."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    tokens = torch.randint(0, dims["V"], (1, prompt), generator=g, device=dev, dtype=torch.int32)
    kv = driver.KVCache(dims, 1, prompt, dev)
    ws = driver.workspace(model.append_workspace_bytes(1, chunk), dev)

    def run():
        kv.len[0] = 0
        for c0 in range(0, prompt, chunk):
            driver.kv_append_tokens(model, kv, tokens[:, c0:c0 + chunk].contiguous(), ws)
    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / reps
    flops = prefill_flops(dims, prompt, chunk)
    tf = flops / t / 1e12
    del kv, ws
    return dict(workload=f"{prompt}-token prompt into an empty cache, {chunk}-token chunks, "
                         f"{dims['n_layers']} layers", tokens_per_s=round(prompt / t, 1),
                ms=round(t * 1e3, 2), reps=reps,
                roofline=dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFS,
                              unit="TFLOP/s", frac=round(tf / MFMA_BF16_PEAK_TFS, 4),
                              flops=round(flops)))


def generate_measure(driver, model, kv, params, dims, dev, cache_len, gen_length=512):
    """The native generation loop (dg_generate) for gen_length tokens on the benchmark's cache:
    canvases of up to 48 steps with the done flags read after every step, each appended."""
    import torch
    state = driver.SamplerState(1, dims["C"], dev)
    out = driver.StepOut(1, dims["C"], dims["V"], dev)
    ws = driver.workspace(driver._lib.load().dg_generate_workspace_bytes(model.handle, 1), dev)
    kv.len[0] = cache_len
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, n, steps = driver.generate(model, kv, params, state, out, gen_length, ws=ws)
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    kv.len[0] = cache_len
    return dict(workload=f"{gen_length} tokens after a {cache_len}-token cache, "
                         f"{dims['n_layers']} layers, adaptive stop on",
                tokens_per_s=round(n * dims["C"] / t, 2), ms=round(t * 1e3, 1), canvases=n,
                steps_per_canvas=steps)


def sampler_roofline(driver, timer, dev, vocab, steps=8):
    """The standalone EB sampler (dg_eb_sample) on the standalone sampler workload: HBM rate of
    its statistics kernel (one read of the logits) and the time of the whole call."""
    import torch
    rows = 256
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    cls = torch.randperm(rows, generator=g, device=dev)
    z = torch.randn((rows, vocab), generator=g, device=dev)
    peaked, moderate = cls[:77], cls[77:77 + 102]
    z[moderate] *= 2.0 ** 0.5
    flat = cls[179:]
    z[flat] *= 0.1 ** 0.5
    pos = torch.randint(0, vocab, (77,), generator=g, device=dev)
    z[peaked, pos] = 12.0
    logits = z.to(torch.bfloat16).view(1, rows, vocab)
    del z
    params = driver.eb_params()
    state = driver.SamplerState(1, rows, dev)
    out = driver.StepOut(1, rows, vocab, dev)
    driver.canvas_init(params, state, vocab)
    ws = driver.eb_sample(logits, 0, params, state, out)
    torch.cuda.synchronize()
    names = ["logit_stats", "stats_merge", "eb_commit", "candidates", "cand_apply"]
    timer.reset()
    timer.enable(names)
    for s in range(steps):
        driver.eb_sample(logits, s, params, state, out, ws)
    torch.cuda.synchronize()
    timer.enable([])
    ms = {n: timer.read(n) for n in names}
    t_stats = ms["logit_stats"][0] / max(ms["logit_stats"][1], 1) * 1e-3
    total = sum(v[0] for v in ms.values()) / steps * 1e-3
    nbytes = rows * vocab * 2
    gbs = nbytes / t_stats / 1e9
    return dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), kernel="logit_stats",
                bytes_per_launch=nbytes, avg_launch_us=round(t_stats * 1e6, 2),
                sampler_call_us=round(total * 1e6, 2),
                workload="bf16 logits [256 x 262144]: 30% peaked, 40% N(0,2), 30% N(0,0.1) rows")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed PMC summary (FETCH_SIZE + WRITE_SIZE, each
    scaled by the copy-kernel yardstick), or None when the kernel sources no longer hash to the
    ones the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decoder_step_pmc_traffic.txt")
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                      if ": " in line and not line.startswith(" "))
        csrc = os.path.join(ROOT, "block_diffusion_decoding_canvas_amd", "csrc")
        src = b"".join(open(os.path.join(csrc, f), "rb").read()
                       for f in ("k_moe.hip", "dg_internal.h"))
        if hashlib.sha256(src).hexdigest() != fields["kernel_source_sha256"].strip():
            return None
        return int(fields["moe_gateup_traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def touched_experts(driver, model, kv, state, embed, params, dims, ws, cache_len, canvases):
    """(step, distinct routed experts) of every expert launch of one pass, in launch order: the
    pass is replayed, and before each decoder step the layer chain runs on the step's canvas with
    top-k traces (the chain's expert sets are the step's own)."""
    import torch
    B, C, k, V = kv.batch, dims["C"], dims["top_k"], dims["V"]
    out = driver.StepOut(B, C, V, "cuda")
    h = torch.empty((B * C, dims["d"]), dtype=torch.float32, device="cuda")
    ti = torch.empty((B * C, k), dtype=torch.int32, device="cuda")
    counts = []
    kv.len[0] = cache_len
    for _ in range(canvases):
        driver.canvas_init(params, state, V)
        for s in range(params.max_steps):
            ids = state.canvas.view(-1).long().clamp(0, V - 1)
            h.copy_(torch.index_select(embed, 0, ids).float())
            for layer in range(dims["n_layers"]):
                driver.layer_forward(model, kv, layer, 0, h, ws, None, ti, None)
                counts.append((s, int(torch.unique(ti).numel())))
            driver.decoder_step(model, kv, s, params, state, out, ws)
            if bool(state.done.all()):
                break
        driver.kv_append_canvas(model, kv, state.canvas, ws)
    torch.cuda.synchronize()
    kv.len[0] = cache_len
    return counts


def attention_flops_windowed(dims, cache_len, window, causal):
    """Algorithmic flops of one sliding-window layer's attention: canvas query i sees the cache
    positions less than `window` back from its absolute position, and the canvas (all of it, or
    the causal prefix)."""
    c, hq, dh = dims["C"], dims["hq"], dims["dh"]
    keys = 0.0
    for i in range(c):
        keys += min(cache_len, max(window - 1 - i, 0)) + ((i + 1) if causal else c)
    return 4.0 * hq * keys * dh


def long_fp8_measure(driver, dev, layers=30, batch=4, cache=131072, steps=1, warmup=1,
                     cpu=True, kv_dtype="e4m3"):
    """The long-context batched fp8 workload: the full-width decoder with e4m3 expert and LM-head
    weights (per-row fp32 scales), 4 canvases of 256 tokens each on its own 131,072-token cache
    (kv_dtype "e4m3": e4m3 rows with fp32 row scales, QK^T on the e4m3 MFMA and P V on the bf16
    one; "bf16": N(0,1) bf16 rows), 5 sliding-window (1,024) layers to 1 global; one bench step =
    every canvas's EB steps (48, adaptive stop on) + the append of the 4 canvases.  Returns one
    JSON-able dict."""
    import torch
    from block_diffusion_decoding_canvas_amd import synth
    dims = synth.dims_long(n_layers=layers)
    kv8 = kv_dtype == "e4m3"
    if kv8:
        dims["kv_dtype"] = "e4m3"
    B, C, V = batch, dims["C"], dims["V"]
    log(f"long fp8: drawing the model and {batch} x {cache}-token {kv_dtype} caches")
    w = synth.make_model_device(dims, dev, seed=0)
    model = driver.Model(w, wdtype="e4m3")
    cap = cache + C
    if kv8:
        kc, vc, ks, vs = synth.make_cache_fp8_device(dims, B, cap, cache, dev, seed=1)
        kv = driver.KVCache(dims, B, cap, dev, kc, vc, [cache] * B, ks, vs)
    else:
        kc, vc = synth.make_cache_device(dims, B, cap, cache, dev, seed=1)
        kv = driver.KVCache(dims, B, cap, dev, kc, vc, [cache] * B)
    ws = driver.workspace(model.workspace_bytes(B), dev)
    params = driver.eb_params()
    state = driver.SamplerState(B, C, dev)
    out = driver.StepOut(B, C, V, dev)
    timer = driver.KernelTimer()
    torch.cuda.synchronize()

    def one_pass():
        for b in range(B):
            kv.len[b] = cache
        driver.canvas_init(params, state, V)
        n = 0
        for s in range(params.max_steps):
            driver.decoder_step(model, kv, s, params, state, out, ws)
            n += 1
            if bool(state.done.all()):
                break
        driver.kv_append_canvas(model, kv, state.canvas, ws)
        return n

    for _ in range(warmup):
        one_pass()
    torch.cuda.synchronize()
    log("long fp8: timing")
    t0 = time.perf_counter()
    n_steps = sum(one_pass() for _ in range(steps))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-class pass: attention and the fp8 expert stream
    timer.reset()
    timer.enable(["attention", "moe_gateup", "lmhead"])
    n_pass = one_pass()
    torch.cuda.synchronize()
    timer.enable([])
    ms_at, n_at = timer.read("attention")
    ms_gu, n_gu = timer.read("moe_gateup")
    at_flops = 0.0
    for layer in range(layers):
        glob = (layer + 1) % dims["global_every"] == 0
        f_dec = (attention_flops(dims, cache, False) if glob else
                 attention_flops_windowed(dims, cache, dims["window"], False))
        f_app = (attention_flops(dims, cache, True) if glob else
                 attention_flops_windowed(dims, cache, dims["window"], True))
        at_flops += B * (n_pass * f_dec + f_app)
    t_at = ms_at * 1e-3
    at_tf = at_flops / t_at / 1e12
    # fp8 expert bytes per gate/up launch: every expert is touched at 1,024 routed tokens x 8
    d, f, fs, k = dims["d"], dims["F"], dims["Fs"], dims["top_k"]
    T = B * C
    gu_bytes = (dims["E"] * 2 * f * d + 2 * fs * d) + T * d + (T * k * f + T * fs) * 4
    gu_t = ms_gu / max(n_gu, 1) * 1e-3
    gu_gbs = gu_bytes / gu_t / 1e9
    # attention peak: bf16 MFMA; with the e4m3 cache, half the flops (QK^T) run on the e4m3
    # MFMA at twice the rate, so the attainable peak is the harmonic mix 2 / (1/5.0 + 1/2.5) PF/s
    at_peak = (2.0 / (1.0 / MFMA_FP8_PEAK_TFS + 1.0 / MFMA_BF16_PEAK_TFS) if kv8
               else MFMA_BF16_PEAK_TFS)
    res = dict(
        workload=(f"{layers}-layer full-width decoder, e4m3 experts + LM head, {B} x 256-token "
                  f"canvases on {cache}-token {kv_dtype} KV caches each, 5 sliding-window (1024) "
                  f": 1 global layers, 48 EB steps max (adaptive stop) + append per bench step"),
        steps_per_s=round(n_steps / elapsed, 3), tokens_per_s=round(B * C * steps / elapsed, 2),
        ms_per_bench_step=round(elapsed / steps * 1e3, 1), decoder_steps=n_steps,
        bench_steps=steps, warmup=warmup, kv_cache=kv_dtype,
        dtype=("e4m3 experts, LM head and KV cache (QK^T e4m3, P V bf16)" if kv8 else
               "e4m3 experts and LM head, bf16 attention"),
        roofline=dict(bound="mfma", achieved=round(at_tf, 1), peak=round(at_peak, 1),
                      unit="TFLOP/s", frac=round(at_tf / at_peak, 4),
                      kernel="attention (+ split merge): global and windowed layers",
                      launches=n_at, ms_per_pass=round(ms_at, 2)),
        moe_gateup_fp8=dict(bound="hbm", achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS,
                            unit="GB/s", frac=round(gu_gbs / HBM_PEAK_GBS, 4),
                            bytes_per_launch=gu_bytes, avg_launch_us=round(gu_t * 1e6, 2),
                            launches=n_gu))
    del model, w, kv, kc, vc, ws, out
    if kv8:
        del ks, vs
    torch.cuda.empty_cache()
    if cpu:
        res["cpu_baseline"] = cpu_baseline_long(dims, B, cache)
    return res


def cpu_baseline_long(dims, batch, cache_len):
    """The oracle on a bounded sample of the long-context fp8 step: one global and one windowed
    full-width layer (e4m3 experts) over one 256-token canvas on a cache of `cache_len`, the fp8
    LM head and the EB sampler; per step = batch x (global layers x global + windowed layers x
    windowed + LM head + sampler)."""
    import numpy as np
    from block_diffusion_decoding_canvas_amd import synth
    from oracle import model as om
    from oracle import sampler as osamp
    from oracle.numerics import quantize_rows_e4m3, round_bf16
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    C, d = dims["C"], dims["d"]
    h = synth.hidden_states(C, d, seed=1).astype(np.float64)[None]
    times = {}
    for name, layer in (("windowed", 0), ("global", dims["global_every"] - 1)):
        lw = om.quantize_layer_e4m3({k: v.astype(np.float64)
                                     for k, v in synth.make_layer(dims, rng).items()})
        n_keys = cache_len if name == "global" else dims["window"] - 1
        cache = synth.make_cache(dict(dims, n_layers=1), 1, n_keys, n_keys, seed=1)
        kc, vc = cache["k"][0].astype(np.float64), cache["v"][0].astype(np.float64)
        t0 = time.perf_counter()
        om.layer_forward(h, lw, dims, layer, kc, vc, np.array([n_keys]), causal=False)
        times[name] = time.perf_counter() - t0
        log(f"oracle {name} layer: {times[name]:.1f} s")
        del lw, kc, vc
    w_lm = synth.to_bf16_values(rng.standard_normal((dims["V"], d), dtype=np.float32) * 0.02)
    wq, s_lm = quantize_rows_e4m3(w_lm.astype(np.float64))
    del w_lm
    t0 = time.perf_counter()
    z = om.fp8_linear(om.rms_norm(h, np.ones(d), dims["eps"]), wq, s_lm)
    zr = round_bf16(z)
    t_lm = time.perf_counter() - t0
    del wq, z
    st = osamp.new_state(osamp.init_canvas(2, [0], C, dims["V"]))
    t0 = time.perf_counter()
    osamp.eb_step(zr, 0, osamp.default_params(), st, 2, [0])
    t_samp = time.perf_counter() - t0
    n_glob = dims["n_layers"] // dims["global_every"]
    per_canvas = (n_glob * times["global"] + (dims["n_layers"] - n_glob) * times["windowed"] +
                  t_lm + t_samp)
    return dict(value=1.0 / (batch * per_canvas), unit="steps/s", cores=cores, kind="oracle",
                sample=(f"one global ({times['global']:.1f} s, {cache_len} cached keys) and one "
                        f"windowed ({times['windowed']:.1f} s) full-width e4m3 layer, the fp8 LM "
                        f"head ({t_lm:.1f} s) and the EB sampler ({t_samp:.1f} s) for one 256-token "
                        f"canvas, fp64 numpy; per step = {batch} canvases x ({n_glob} global + "
                        f"{dims['n_layers'] - n_glob} windowed layers + LM head + sampler)"))


def cpu_baseline(dims, n_layers_sample, cache_len):
    """The oracle (fp64 numpy) on a bounded sample of one decoder step: `n_layers_sample`
    full-width layers over the 256-token canvas with the N(0,1) cache, the LM head and the EB
    sampler; the per-step time is scaled to the full depth."""
    import numpy as np
    from block_diffusion_decoding_canvas_amd import synth
    from oracle import model as om
    from oracle import sampler as osamp
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    C, d = dims["C"], dims["d"]
    h = synth.hidden_states(C, d, seed=1).astype(np.float64)[None]
    t_layers = 0.0
    for _ in range(n_layers_sample):
        lw = {k: v.astype(np.float64) for k, v in synth.make_layer(dims, rng).items()}
        cache = synth.make_cache(dict(dims, n_layers=1), 1, cache_len, cache_len, seed=1)
        kc = cache["k"][0].astype(np.float64)
        vc = cache["v"][0].astype(np.float64)
        t0 = time.perf_counter()
        h, _, _, _ = om.layer_forward(h, lw, dims, 0, kc, vc, cache["len"], causal=False)
        t_layers += time.perf_counter() - t0
        log(f"oracle layer: {t_layers:.1f} s")
        del lw, kc, vc
    w_lm = synth.to_bf16_values(rng.standard_normal((dims["V"], d), dtype=np.float32) * 0.02)
    w_lm = w_lm.astype(np.float64)
    fn = np.ones(d)
    t0 = time.perf_counter()
    z = om.rms_norm(h, fn, dims["eps"]) @ w_lm.T
    from oracle.numerics import round_bf16
    zr = round_bf16(z)
    t_lm = time.perf_counter() - t0
    del w_lm, z
    st = osamp.new_state(osamp.init_canvas(2, [0], C, dims["V"]))
    t0 = time.perf_counter()
    osamp.eb_step(zr, 0, osamp.default_params(), st, 2, [0])
    t_samp = time.perf_counter() - t0
    per_step = t_layers / n_layers_sample * dims["n_layers"] + t_lm + t_samp
    return dict(value=1.0 / per_step, unit="steps/s", cores=cores, kind="oracle",
                sample=(f"{n_layers_sample} full-width layer(s) ({t_layers:.1f} s) + LM head "
                        f"({t_lm:.1f} s) + EB sampler ({t_samp:.1f} s) of one 256-token step on "
                        f"a {cache_len}-token cache, fp64 numpy; per-step time = layers scaled "
                        f"to {dims['n_layers']} + LM head + sampler"))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library does not "
              f"shard the path across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    import numpy as np
    import torch
    from block_diffusion_decoding_canvas_amd import driver, synth

    dev = "cuda"
    dims = synth.dims_full(n_layers=args.layers)
    if args.prefill_only:
        pmodel = driver.Model(synth.make_model_device(dims, dev, seed=0))
        print(json.dumps(prefill_measure(driver, pmodel, dims, dev)))
        return
    if args.long_fp8_only:
        print(json.dumps(long_fp8_measure(driver, dev, layers=args.layers,
                                          cpu=not args.no_cpu_baseline, kv_dtype=args.long_kv)))
        return
    C, B = dims["C"], 1
    cap = args.cache + C * args.canvases
    weights = synth.make_model_device(dims, dev, seed=0)
    kc, vc = synth.make_cache_device(dims, B, cap, args.cache, dev, seed=1)
    model = driver.Model(weights)
    kv = driver.KVCache(dims, B, cap, dev, kc, vc, [args.cache])
    ws = driver.workspace(model.workspace_bytes(B), dev)
    params = driver.eb_params()        # the model card's sampler constants, adaptive stop on
    state = driver.SamplerState(B, C, dev)
    out = driver.StepOut(B, C, dims["V"], dev)
    timer = driver.KernelTimer()
    torch.cuda.synchronize()

    def one_pass(per_canvas=None, sample_gateup=0):
        """Generate `canvases` canvases back to back; returns decoder steps run (and appends the
        steps of each canvas to `per_canvas`).  With `sample_gateup` = n, HIP events bracket the
        MoE gate/up launches of every n-th step only."""
        kv.len[0] = args.cache
        steps = 0
        for _ in range(args.canvases):
            driver.canvas_init(params, state, dims["V"])
            n = 0
            for s in range(params.max_steps):
                if sample_gateup:
                    timer.enable(["moe_gateup"] if s % sample_gateup == 0 else [])
                driver.decoder_step(model, kv, s, params, state, out, ws)
                n += 1
                if bool(state.done.all()):
                    break
            steps += n
            if per_canvas is not None:
                per_canvas.append(n)
            driver.kv_append_canvas(model, kv, state.canvas, ws)
        return steps

    log("model and cache resident; warming up")
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    log("warmup done; timing")
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total_steps = 0
    for i in range(args.steps):
        # events only around the dominant kernel, on every 8th step: an event pair around every
        # launch costs about 0.17 ms per step of GPU time, 1/8 of them stays in the noise
        total_steps += one_pass(sample_gateup=GATEUP_SAMPLE_EVERY)
        log(f"timed pass {i + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timer.enable([])
    ms_gu, n_gu = timer.read("moe_gateup")
    # per-kernel breakdown from one more (untimed) pass with every class timed
    timer.reset()
    timer.enable()
    per_canvas = []
    one_pass(per_canvas)
    torch.cuda.synchronize()
    timer.enable([])
    per_class = {n: timer.read(n) for n in timer.names}

    # experts touched by each timed gate/up launch: the passes are deterministic (same seed,
    # canvas ids and cache lengths), so one more pass replays the sampled steps exactly; before
    # each of them the GPU layer chain (dg_layer_forward, the step's own kernels) yields every
    # layer's expert sets
    every_step = touched_experts(driver, model, kv, state, weights["embed"], params, dims, ws,
                                 args.cache, args.canvases)
    touched = [n for s_, n in every_step if s_ % GATEUP_SAMPLE_EVERY == 0]
    avg_gu = ms_gu / max(n_gu, 1) * 1e-3
    per_pass = len(touched)
    assert n_gu == per_pass * args.steps, (n_gu, per_pass)
    bytes_gu = sum(moe_gateup_bytes(dims, n) for n in touched) / per_pass
    achieved = bytes_gu / avg_gu / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                    kernel="moe_gateup", bytes_per_launch=round(bytes_gu),
                    avg_launch_us=round(avg_gu * 1e6, 2), launches=n_gu,
                    launches_sampled=(f"every {GATEUP_SAMPLE_EVERY}th decoder step of the timed "
                                      f"region, every layer"),
                    experts_touched=dict(min=min(touched), max=max(touched),
                                         mean=round(sum(touched) / per_pass, 2)))
    # the down product is timed over every launch of the per-class pass: every step's counts
    n_touched = sum(n for _, n in every_step) / len(every_step)
    kernel_ms = {n: round(v[0], 3) for n, v in per_class.items() if v[1]}

    # the other kernels of the path with a roofline line, from the per-class pass (HIP events per
    # launch)
    def rate(name):
        ms, n = per_class[name]
        return ms / max(n, 1) * 1e-3, n
    t_lm, n_lm = rate("lmhead")
    lm_flops = 2.0 * B * C * dims["V"] * dims["d"]
    t_at, n_at = rate("attention")
    at_flops = 0.0
    for i, n in enumerate(per_canvas):
        length = args.cache + i * C
        at_flops += args.layers * (n * attention_flops(dims, length, False) +
                                   attention_flops(dims, length, True))
    t_dn, n_dn = rate("moe_down")
    dn_bytes = moe_down_bytes(dims, n_touched)

    def mfma_line(flops, t, n, kernel):
        tf = flops / t / 1e12
        return dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                    frac=round(tf / MFMA_BF16_PEAK_TFS, 4), kernel=kernel,
                    avg_launch_us=round(t * 1e6, 2), launches=n)
    rooflines = dict(
        moe_gateup=roofline,
        moe_down=dict(bound="hbm", achieved=round(dn_bytes / t_dn / 1e9, 1), peak=HBM_PEAK_GBS,
                      unit="GB/s", frac=round(dn_bytes / t_dn / 1e9 / HBM_PEAK_GBS, 4),
                      kernel="moe_down", bytes_per_launch=dn_bytes,
                      avg_launch_us=round(t_dn * 1e6, 2), launches=n_dn),
        lmhead=mfma_line(lm_flops, t_lm, n_lm, "lmhead (bf16 GEMM + tempered softmax statistics)"),
        attention=dict(mfma_line(at_flops / max(n_at, 1), t_at, n_at,
                                 "attention (+ split merge), averaged over the pass"),
                       flops_per_launch=round(at_flops / max(n_at, 1))))
    gen = prefill = peaks = None
    if not (args.no_generate or args.decoder_only):
        log("timing the native generation loop")
        gen = generate_measure(driver, model, kv, params, dims, dev, args.cache)
    if not (args.no_prefill or args.decoder_only):
        log("timing the chunked prefill")
        prefill = prefill_measure(driver, model, dims, dev)
    if not (args.no_sampler or args.decoder_only):
        log("timing the standalone EB sampler")
        rooflines["eb_sampler"] = sampler_roofline(driver, timer, dev, dims["V"])
        # what the library's plain read stream and MFMA loop reach on this machine: each line's rate
        # over that ceiling, beside its fraction of the nominal peak
        peaks = measured_peaks(driver)
        for line_ in [roofline] + list(rooflines.values()):
            ceiling = (peaks["hbm_read_gbs"] if line_.get("unit") == "GB/s"
                       else peaks["mfma_bf16_tfs"])
            line_["frac_of_measured"] = round(line_["achieved"] / ceiling, 4)

    long_fp8 = None
    if not (args.no_long_fp8 or args.decoder_only):
        log("freeing the bf16 model; timing the long-context fp8 workload")
        del model, weights, kv, kc, vc, ws, out, state
        torch.cuda.empty_cache()
        long_fp8 = long_fp8_measure(driver, dev, layers=args.layers,
                                    cpu=not args.no_cpu_baseline, kv_dtype=args.long_kv)

    cpu = None
    if not (args.no_cpu_baseline or args.decoder_only):
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(dims, args.cpu_layers, args.cache)

    steps_per_s = total_steps / elapsed
    tokens = B * C * args.canvases * args.steps
    line = dict(
        metric=METRIC, value=round(steps_per_s, 3), unit="steps/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(elapsed / args.steps * 1e3, 2),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic: random-init N(0,0.02^2) weights, N(0,1) bf16 KV cache, Philox canvases",
        config=dict(workload=(f"{args.layers}-layer full-width decoder, 128 experts top-8 + "
                              f"shared, V 262144, B {B} x 256-token canvas, {args.cache}-token "
                              f"cache, {args.canvases} canvases (48 EB steps max each, adaptive "
                              f"stop) + append per step"),
                    layers=args.layers, canvas=C, batch=B, cache=args.cache,
                    canvases_per_step=args.canvases, decoder_steps=total_steps),
        tokens_per_s=round(tokens / elapsed, 2),
        decoder_step_ms=round(elapsed / total_steps * 1e3, 3),
        roofline=roofline, cpu_baseline=cpu, rooflines=rooflines,
        measured_peaks=peaks, prefill=prefill, generate=gen, long_fp8=long_fp8,
        kernel_ms_per_bench_step=kernel_ms)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
