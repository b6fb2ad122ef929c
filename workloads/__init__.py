"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks."""
from .gen import (CONFIGS, CFG4_PATIENCE_SWEEP, ORDER_GIVEN, ORDER_NATURAL, ORDER_RECENT_FIRST,
                  READINGS, Spec, Workload, bf16_bits_to_f32, config, draw_unit, f32_to_bf16_bits,
                  make_workload, multi_row_queries, scaled, storage_to_f64)
