"""Seeded synthetic inputs for the MAC-Attention decode workloads.

This package holds none of the method's arithmetic: only shapes, random draws,
the bf16 rounding of those draws and the page scatter of a logical KV cache.
Both the HIP path and the CPU oracle take their inputs from here.
"""
from .synth import (CONFIGS, Workload, get_config, scaled, queries, rho_values, kv_logical,
                    page_table, to_paged, bf16_bits)

__all__ = ["CONFIGS", "Workload", "get_config", "scaled", "queries", "rho_values",
           "kv_logical", "page_table", "to_paged", "bf16_bits"]
