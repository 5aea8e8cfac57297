"""Seeded synthetic workloads shared by the oracle (tests) and the HIP library.

Holds input data only: presets and generators.  No step of the decode method
is computed here.
"""
from .configs import DecodeCfg, ModelCfg, WorkloadCfg, PRESETS, PRESET_ORDER, preset  # noqa: F401
from .generate import (make_weights, make_requests, make_logits, normal, sub_seed,  # noqa: F401
                       torch_dtype)
