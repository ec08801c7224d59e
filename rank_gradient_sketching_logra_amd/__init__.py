"""LoGRA low-rank gradient sketch hot path for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI of
``liblogra.so`` (``include/logra.h``); ``binding`` is its thin ctypes layer.
``synth`` holds the seeded synthetic workloads.  Build the library with
``python -m rank_gradient_sketching_logra_amd.build``.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    Key, LograError, key, merge, predicted_kl_q, project_input, regen_A, rowadam,
    sketch_accumulate, sketch_accumulate_grouped, sketch_bytes, step_alpha, step_alpha_dev,
    version,
)
