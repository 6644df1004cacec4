"""Seeded synthetic inputs for the canvas denoise step.

This package is the ONE module shared by the CPU oracle (under ``oracle/``)
and the HIP path (``uniform_state_discrete_amd``): it only draws numbers and
stores them in the storage precision.  It holds none of the method's
arithmetic (no attention, no softmax, no renoising, no random token draws:
the method's own uniform token draws are computed on each side from the
published Philox4x64-10 definition).
"""
from .configs import Config, CONFIGS, config_by_name, tau_schedule  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_from_f32, f32_from_bf16_bits, to_storage, from_storage,
    gen_embedding, gen_weights, gen_cache, gen_hidden, gen_problem, Problem,
    signal_amplitude,
)
