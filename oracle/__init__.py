"""CPU oracle of the MoE route/dispatch/combine transform -- test
infrastructure only (tests, the smoke check and the benchmark's CPU-baseline
leg); never imported by the product path."""
from . import moe_oracle  # noqa: F401
