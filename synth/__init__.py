"""Seeded synthetic inputs shared by the oracle's tests and the GPU path.

``configs``   -- the workload shapes.
``generator`` -- host (numpy) Philox4x32-10 generator of activations, router weights, router
                 bias and fp32 expert weights.
``device``    -- the same generator on the GPU (``libmoe_synth.so``), bit-identical, for
                 filling multi-GB expert banks without a host round trip.
"""
from . import configs, generator  # noqa: F401
