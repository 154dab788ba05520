"""Seeded synthetic inputs of the LowRAM decode step.

Workload shapes (``configs``) and random draws (``draws``).  Holds none of the
decode step's arithmetic; the CPU oracle and the GPU tests both read their
inputs from here.
"""
from .configs import BY_ID, C0, C1, C2, C3, C3_BATCHES, C4, CONFIGS, Config  # noqa: F401
from .draws import (basis, evicted_chunks, exact_keys, key_noise, latents, layer_cols,  # noqa: F401
                    mixing, mlp_weights, needle_chunks, plant_needle, queries, rng,
                    survivors, value_noise, value_spikes)
