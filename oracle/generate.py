"""The outer generation loop over canvases, written plainly on top of the oracle's decoder, encoder
and sampler.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix (diffusers DiffusionGemmaPipeline docs, the ``__call__`` parameters and
"Adaptive stopping"; DiffusionGemma model card, "Model overview"):
  * ``gen_length`` tokens are generated, rounded up to a whole number of canvases;
  * each canvas is denoised for at most ``num_inference_steps`` steps; a sample freezes on its own
    (adaptive stop) and the canvas's loop ends once every sample is frozen;
  * a finished canvas is run through the encoder and appended to the KV cache before the next
    canvas starts;
  * with ``eos_early_stop`` (the default), no further canvas is started once every sequence has
    produced the EOS token.

Readings taken where the pages are silent:
  * "has produced EOS" means the EOS id occurs at any position of any finished canvas of that
    sequence; the canvas that contains it is still kept and appended; a negative EOS id never
    stops the loop;
  * canvas c of sequence b draws its Philox noise with canvas id c * B + b, so that every
    (sequence, canvas) pair has its own streams;
  * the prompt is already in the cache when the loop starts (the chunked prefill writes it).
"""
import numpy as np

from . import model as om
from . import sampler as osamp


def n_canvases(gen_length, canvas_len):
    """Canvases needed for gen_length tokens: gen_length rounded up to a multiple of C."""
    return -(-int(gen_length) // int(canvas_len))


def generate(model, cache, params, seed, gen_length, eos_id=-1, eos_early_stop=True):
    """Runs the canvas loop on a cache that holds the prompt (updated in place).

    Returns dict(tokens [B, n * C] int64 for the n canvases generated, steps: list of decoder steps
    per canvas, canvases: n).
    """
    dims = model["dims"]
    clen = dims["C"]
    bsz = int(np.asarray(cache["len"]).shape[0])
    total = n_canvases(gen_length, clen)
    out, steps = [], []
    has_eos = np.zeros(bsz, dtype=bool)
    for c in range(total):
        ids = [c * bsz + b for b in range(bsz)]
        state = osamp.new_state(osamp.init_canvas(seed, ids, clen, dims["V"]))
        n = 0
        for s in range(int(params["max_steps"])):
            z, _, _ = om.decoder_forward(state["canvas"], model, cache)
            osamp.eb_step(z, s, params, state, seed, ids)
            n += 1
            if state["done"].all():
                break
        canvas = state["canvas"].copy()
        om.encoder_append(canvas, model, cache)
        out.append(canvas)
        steps.append(n)
        if eos_id >= 0:
            has_eos |= (canvas == eos_id).any(axis=1)
            if eos_early_stop and has_eos.all():
                break
    return dict(tokens=np.concatenate(out, axis=1), steps=steps, canvases=len(out))
