"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks."""
from .workloads import (CONFIG_ORDER, PAGE, SPECS, F64View, Workload, WorkloadSpec, bf16_bits_to_f32, oracle_inputs,
                        budget_for, f32_to_bf16_bits, make_workload, num_pages, small_spec,
                        to_f64)

__all__ = ["CONFIG_ORDER", "PAGE", "SPECS", "F64View", "oracle_inputs", "Workload", "WorkloadSpec", "bf16_bits_to_f32",
           "budget_for", "f32_to_bf16_bits", "make_workload", "num_pages", "small_spec",
           "to_f64"]
