"""Seeded synthetic inputs for batched speculative-decoding verification.

This module only makes inputs (logits, drafted tokens, uniforms). It holds none
of the verification arithmetic; both the HIP library and the CPU oracle consume
what it produces.
"""

from .gen import (CONFIGS, Config, make_inputs, mc_inputs, const_alpha_inputs,  # noqa: F401
                  to_host_f64, window_edge_inputs)
