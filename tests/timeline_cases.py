"""Workloads that tests/test_timeline_gpu.py runs on both builds."""
import workloads

CASES = {
    "bf16": (workloads.custom([150, 150, 40], [700, 700, 300], 3, 128, seed=7600), "bf16"),
    "fp8": (workloads.custom([150, 40], [700, 300], 2, 128, seed=7700, dtype="fp8"), "fp8"),
}
