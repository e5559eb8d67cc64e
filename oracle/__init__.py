"""Plain CPU oracle of the latent KV cache path (test infrastructure only).

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  The HIP library and its Python binding never do.
"""
from .oracle import *  # noqa: F401,F403
