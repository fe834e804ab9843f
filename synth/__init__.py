"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side
tests/bench.  Holds no quantization or attention arithmetic."""

from .inputs import CONFIGS, make_inputs, sample_rows, rng  # noqa: F401
