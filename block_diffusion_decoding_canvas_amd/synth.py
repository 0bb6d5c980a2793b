"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and stores them in the device's storage type (bf16); it
holds none of the method's arithmetic.  Both the HIP path and the oracle read the arrays it makes.

Shapes follow the model card's dimension table (DiffusionGemma model card, "Model overview":
30 layers, 8 of 128 experts active plus 1 shared, 256-token canvas, ~262K vocabulary, 1,024-token
sliding window).  The width dimensions (d_model 2816, 16/8 heads of 256, expert width 704) are
synthetic stand-ins; the pages do not give them.

Seeds: weights from numpy ``default_rng(seed)`` (default 0) in the fixed order of
``weight_order``; inputs (hidden states, caches, logits, prompt ids) from ``default_rng(1)``;
the sampler's Philox key defaults to 2 and canvas b has canvas id b.
"""
import numpy as np
import torch

WEIGHT_STD = 0.02      # weights ~ N(0, 0.02^2)


def dims_tiny():
    """2-layer toy decoder: d 64, 4 heads of 16, 8 experts top-2 + shared, F 128, V 512, C 16."""
    return dict(n_layers=2, d=64, hq=4, hkv=4, dh=16, E=8, top_k=2, F=128, Fs=128, V=512, C=16,
                window=0, global_every=1, eps=1e-6)


def dims_full(n_layers=30, vocab=262144):
    """Full-width synthetic decoder: d 2816, 16/8 heads of 256, 128 experts top-8 + shared,
    F 704, V 262,144, canvas 256."""
    return dict(n_layers=n_layers, d=2816, hq=16, hkv=8, dh=256, E=128, top_k=8, F=704, Fs=704,
                V=vocab, C=256, window=0, global_every=1, eps=1e-6)


def dims_long(n_layers=30):
    """Full-width decoder with the 5 sliding-window (1,024) : 1 global layer pattern."""
    d = dims_full(n_layers)
    d.update(window=1024, global_every=6)
    return d


def to_bf16_values(x):
    """Round float values to bf16 storage (torch CPU cast, RNE); returned as float32 numpy."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def weight_order(dims):
    """(name, shape) of every weight tensor, in generation order."""
    d, hq, hkv, dh = dims["d"], dims["hq"], dims["hkv"], dims["dh"]
    e, f, fs, v = dims["E"], dims["F"], dims["Fs"], dims["V"]
    layer = [("attn_norm", (d,)), ("w_qkv", ((hq + 2 * hkv) * dh, d)), ("w_o", (d, hq * dh)),
             ("ffn_norm", (d,)), ("w_router", (e, d)), ("w_gate_up", (e, 2 * f, d)),
             ("w_down", (e, d, f)), ("ws_gate_up", (2 * fs, d)), ("ws_down", (d, fs))]
    return layer, [("embed", (v, d)), ("final_norm", (d,)), ("w_lm", (v, d))]


def make_layer(dims, rng, norm_gain_std=0.0, lm_std=None):
    layer_spec, _ = weight_order(dims)
    out = {}
    for name, shape in layer_spec:
        if name.endswith("norm"):
            g = np.ones(shape, dtype=np.float32)
            if norm_gain_std > 0:
                g = g + rng.standard_normal(shape, dtype=np.float32) * norm_gain_std
            out[name] = to_bf16_values(g)
        else:
            out[name] = to_bf16_values(rng.standard_normal(shape, dtype=np.float32) * WEIGHT_STD)
    return out


def make_model(dims, seed=0, norm_gain_std=0.0, lm_std=WEIGHT_STD, embed_std=WEIGHT_STD):
    """All weights as float32 numpy arrays holding bf16 values.

    ``norm_gain_std`` > 0 draws norm gains 1 + N(0, std^2) instead of ones (to exercise the gain);
    ``lm_std`` lets a test use a sharper LM head (the tiny "hot" variant uses 1.0).
    """
    rng = np.random.default_rng(seed)
    layers = [make_layer(dims, rng, norm_gain_std) for _ in range(dims["n_layers"])]
    v, d = dims["V"], dims["d"]
    embed = to_bf16_values(rng.standard_normal((v, d), dtype=np.float32) * embed_std)
    fn = np.ones((d,), dtype=np.float32)
    if norm_gain_std > 0:
        fn = fn + rng.standard_normal((d,), dtype=np.float32) * norm_gain_std
    final_norm = to_bf16_values(fn)
    w_lm = to_bf16_values(rng.standard_normal((v, d), dtype=np.float32) * lm_std)
    return dict(dims=dict(dims), layers=layers, embed=embed, final_norm=final_norm, w_lm=w_lm)


def make_cache(dims, batch, cap, length, seed=1):
    """Per-layer K, V [B, Hkv, cap, dh] with N(0,1) bf16 entries in [0, length), zeros after."""
    rng = np.random.default_rng(seed)
    ks, vs = [], []
    for _ in range(dims["n_layers"]):
        k = np.zeros((batch, dims["hkv"], cap, dims["dh"]), dtype=np.float32)
        v = np.zeros_like(k)
        k[:, :, :length] = to_bf16_values(
            rng.standard_normal((batch, dims["hkv"], length, dims["dh"]), dtype=np.float32))
        v[:, :, :length] = to_bf16_values(
            rng.standard_normal((batch, dims["hkv"], length, dims["dh"]), dtype=np.float32))
        ks.append(k)
        vs.append(v)
    return dict(k=ks, v=vs, len=np.full(batch, length, dtype=np.int64))


# e4m3 cache rows are drawn as codes, not by quantising anything: the exponent field e (0..15)
# with weight 2^(e - 14) up to 14 and 0.35 for the top binade, the 3 mantissa bits uniform (the
# top binade stops at mantissa 6: code 0x7F is NaN), the sign uniform.  That puts most codes in
# the upper binades, as in a row scaled so that its largest magnitude is 448.  Row scales are
# log-uniform in [2/448, 4/448], so a row's values are of order 1.
_E4M3_EXP_W = np.array([2.0 ** (e - 14) for e in range(15)] + [0.35])
_E4M3_EXP_W = _E4M3_EXP_W / _E4M3_EXP_W.sum()


def e4m3_codes(rng, shape):
    """Random e4m3 codes (uint8, never NaN) with the distribution described above."""
    e = rng.choice(16, size=shape, p=_E4M3_EXP_W)
    m = rng.integers(0, 8, size=shape)
    m = np.where(e == 15, np.minimum(m, 6), m)
    sign = rng.integers(0, 2, size=shape)
    return ((sign << 7) | (e << 3) | m).astype(np.uint8)


def row_scales(rng, shape):
    return (np.exp(rng.uniform(np.log(2.0), np.log(4.0), size=shape)) / 448.0).astype(np.float32)


def make_cache_fp8(dims, batch, cap, length, seed=1):
    """Per-layer e4m3 K, V codes [B, Hkv, cap, dh] (uint8) and fp32 row scales [B, Hkv, cap]
    in [0, length) (codes 0 and scale 1 after)."""
    rng = np.random.default_rng(seed)
    out = dict(k=[], v=[], k_scale=[], v_scale=[])
    for _ in range(dims["n_layers"]):
        for n in ("k", "v"):
            c = np.zeros((batch, dims["hkv"], cap, dims["dh"]), dtype=np.uint8)
            sc = np.ones((batch, dims["hkv"], cap), dtype=np.float32)
            c[:, :, :length] = e4m3_codes(rng, (batch, dims["hkv"], length, dims["dh"]))
            sc[:, :, :length] = row_scales(rng, (batch, dims["hkv"], length))
            out[n].append(c)
            out[n + "_scale"].append(sc)
    out["len"] = np.full(batch, length, dtype=np.int64)
    return out


def empty_cache_fp8(dims, batch, cap):
    shape = (batch, dims["hkv"], cap, dims["dh"])
    out = {n: [np.zeros(shape, dtype=np.uint8) for _ in range(dims["n_layers"])]
           for n in ("k", "v")}
    for n in ("k_scale", "v_scale"):
        out[n] = [np.ones(shape[:-1], dtype=np.float32) for _ in range(dims["n_layers"])]
    out["len"] = np.zeros(batch, dtype=np.int64)
    return out


def empty_cache(dims, batch, cap):
    z = [np.zeros((batch, dims["hkv"], cap, dims["dh"]), dtype=np.float32)
         for _ in range(dims["n_layers"])]
    return dict(k=z, v=[a.copy() for a in z], len=np.zeros(batch, dtype=np.int64))


def prompt_ids(n, vocab, seed=1):
    return np.random.default_rng(seed).integers(0, vocab, size=n).astype(np.int64)


def hidden_states(ntok, d, seed=1):
    return np.random.default_rng(seed).standard_normal((ntok, d), dtype=np.float32)


def sampler_logits(rows=256, vocab=262144, seed=1, peak=12.0, frac=(0.30, 0.40, 0.30)):
    """Sampler workload: a seeded permutation splits the rows into peaked rows (N(0,1) with one
    logit set to ``peak`` at a seeded position), moderate rows N(0, 2) and near-flat rows
    N(0, 0.1) (second argument = variance).  Returns (bf16 values as float32 [rows, vocab],
    class per row: 0 peaked, 1 moderate, 2 near-flat)."""
    rng = np.random.default_rng(seed)
    n_peak = int(round(frac[0] * rows))
    n_mod = int(round(frac[1] * rows))
    cls = np.full(rows, 2, dtype=np.int64)
    perm = rng.permutation(rows)
    cls[perm[:n_peak]] = 0
    cls[perm[n_peak:n_peak + n_mod]] = 1
    z = rng.standard_normal((rows, vocab), dtype=np.float32)
    scale = np.where(cls == 0, 1.0, np.where(cls == 1, np.sqrt(2.0), np.sqrt(0.1)))
    z *= scale.astype(np.float32)[:, None]
    peak_pos = rng.integers(0, vocab, size=rows)
    for r in np.nonzero(cls == 0)[0]:
        z[r, peak_pos[r]] = peak
    return to_bf16_values(z), cls


# ---- device copies (torch owns device memory; the values are the arrays above) --------------

def to_device_bf16(x, device):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        device=device, dtype=torch.bfloat16)


def model_to_device(model, device):
    dev = dict(dims=model["dims"], layers=[])
    for lw in model["layers"]:
        dev["layers"].append({k: to_device_bf16(v, device) for k, v in lw.items()})
    for k in ("embed", "final_norm", "w_lm"):
        dev[k] = to_device_bf16(model[k], device)
    return dev


def model_to_f64(model):
    out = dict(dims=model["dims"], layers=[])
    for lw in model["layers"]:
        out["layers"].append({k: v.astype(np.float64) for k, v in lw.items()})
    for k in ("embed", "final_norm", "w_lm"):
        out[k] = model[k].astype(np.float64)
    return out


def make_model_device(dims, device, seed=0, lm_std=WEIGHT_STD):
    """Timing-size model drawn directly on the device with a seeded torch generator (bf16).

    Used where only shapes and value distributions matter (the 25B-parameter benchmark model)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    layer_spec, _ = weight_order(dims)

    def normal(shape, std):
        t = torch.empty(shape, device=device, dtype=torch.bfloat16)
        t.normal_(0.0, std, generator=g)
        return t

    layers = []
    for _ in range(dims["n_layers"]):
        lw = {}
        for name, shape in layer_spec:
            lw[name] = (torch.ones(shape, device=device, dtype=torch.bfloat16)
                        if name.endswith("norm") else normal(shape, WEIGHT_STD))
        layers.append(lw)
    return dict(dims=dict(dims), layers=layers,
                embed=normal((dims["V"], dims["d"]), WEIGHT_STD),
                final_norm=torch.ones((dims["d"],), device=device, dtype=torch.bfloat16),
                w_lm=normal((dims["V"], dims["d"]), lm_std))


def make_cache_fp8_device(dims, batch, cap, length, device, seed=1, chunk=1 << 26):
    """Timing-size e4m3 cache drawn on the device with a seeded torch generator: codes with the
    distribution of e4m3_codes (exponent field by inverse CDF of a uniform draw), row scales
    log-uniform in [2/448, 4/448], rows [0, length) of every canvas (codes 0, scale 1 after).
    Returns (k, v, k_scale, v_scale)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    L, hkv, dh = dims["n_layers"], dims["hkv"], dims["dh"]
    shape = (L, batch, hkv, cap, dh)
    cdf = torch.tensor(np.cumsum(_E4M3_EXP_W), device=device, dtype=torch.float32)

    def codes(n):
        out = torch.empty(n, dtype=torch.uint8, device=device)
        for o in range(0, n, chunk):
            m = min(chunk, n - o)
            u = torch.rand(m, device=device, generator=g)
            e = torch.searchsorted(cdf, u, right=True).clamp_(max=15)
            mant = torch.randint(0, 8, (m,), device=device, generator=g)
            mant = torch.where(e == 15, mant.clamp(max=6), mant)
            sign = torch.randint(0, 2, (m,), device=device, generator=g)
            out[o:o + m] = ((sign << 7) | (e << 3) | mant).to(torch.uint8)
        return out

    res = []
    for _ in range(2):
        c = torch.zeros(shape, dtype=torch.uint8, device=device)
        for l in range(L):
            for b in range(batch):
                c[l, b, :, :length] = codes(hkv * length * dh).view(hkv, length, dh)
        res.append(c)
    for _ in range(2):
        sc = torch.ones(shape[:-1], dtype=torch.float32, device=device)
        u = torch.rand((L, batch, hkv, length), device=device, generator=g)
        sc[:, :, :, :length] = torch.exp(np.log(2.0) + u * np.log(2.0)) / 448.0
        res.append(sc)
    return tuple(res)


def make_cache_device(dims, batch, cap, length, device, seed=1):
    """Timing-size KV cache drawn on the device: N(0,1) bf16 in [0, length)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (dims["n_layers"], batch, dims["hkv"], cap, dims["dh"])
    k = torch.zeros(shape, device=device, dtype=torch.bfloat16)
    v = torch.zeros(shape, device=device, dtype=torch.bfloat16)
    k[:, :, :, :length].normal_(0.0, 1.0, generator=g)
    v[:, :, :, :length].normal_(0.0, 1.0, generator=g)
    return k, v
