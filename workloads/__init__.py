"""Seeded synthetic inputs for the decode step.

This package is shared by the GPU harness and the oracle-based tests.  It
holds none of the method's arithmetic: it draws random numbers, rounds them to
their storage formats (bf16, and OCP E4M3FN with a per-64-token-block fp32
scale, both through torch's conversions), lays rows out in paged pools with
block tables, and sets up residency tables.  It imports neither ``oracle`` nor
the HIP binding.
"""

from .gen import (Workload, tiny_fp32, resident_fp8, mixed_128k, mtp3_agentic,  # noqa: F401
                  norescache_1m, build_pool, by_name, CONFIG_NAMES)
