"""Tiered KV-cache decode attention for MI355X (gfx950).

The computation lives in ``libqkv.so`` (hand-written HIP, C ABI in
``include/qkv.h``); :mod:`._lib` is its thin ctypes binding.
"""
from ._lib import (Cache, QkvConfig, QkvError, make_config, plan_capacities, quantize_status, quantize_window,
                   rank_tiers, workspace_bytes)

__all__ = ["Cache", "QkvConfig", "QkvError", "make_config", "plan_capacities", "quantize_window", "quantize_status",
           "rank_tiers", "workspace_bytes"]
