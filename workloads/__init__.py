"""Seeded synthetic inputs for the HySparse2 attention hot path.

This package is shared by the tests, the benchmark and the oracle's callers. It
draws random numbers, rounds them to the stored dtype and lays them out; it holds
none of the method's arithmetic (no attention, no scoring, no selection, no
projection). Both the GPU path and the fp64 oracle consume exactly the stored
values produced here.
"""
from .gen import (  # noqa: F401
    bf16_round,
    bf16_to_f32,
    normal_f32,
    stored_to_f64,
)
from .configs import (  # noqa: F401
    BlockInputs,
    BridgeInputs,
    CONFIGS,
    make_block_inputs,
    make_bridge_inputs,
    block_config,
)
