"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

Input generation only: Philox4x32-10 uniforms, Gaussian logit rows shaped like
the benchmark configurations, and Gumbel-max drafted tokens.  Nothing here
computes any part of the verification step.
"""

from .philox import philox4x32_10, open_unit_f32, uniforms  # noqa: F401
from .synth import (  # noqa: F401
    VerifyCase, LMHeadCase, gaussian_case, config1, config2, config3, config4, config5,
    f32_to_bf16_bits, bf16_bits_to_f32, as_f32, make_uniforms,
)
