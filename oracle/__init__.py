"""Plain, slow CPU oracle of the canvas denoising step (fp64, numpy).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run anything under ``oracle/``.  The HIP library never calls it, and
the two share no code; only the seeded input generators feed both.

Modules:
  philox    Philox4x32-10 from its published definition (SC'11).
  numerics  bf16 rounding of float64 values (storage precision).
  sampler   the entropy-bound sampler step, initial canvas, renoise and Gumbel-max candidates.
  model     RMSNorm, joint canvas/cache attention, routed + shared SwiGLU MoE, decoder forward
            and encoder append.

Parity pins: every function is checked in ``tests/test_oracle_*.py`` against closed forms,
invariants, brute force on tiny inputs and library routines (torch CPU, rocRAND's host Philox).
The model internals are readings of the pages, not the released network: parity against the real
DiffusionGemma weights is unpinned (no weights are available); parity here is oracle-internal.
"""
from . import numerics, philox, sampler, model  # noqa: F401
