"""CPU oracle for the mixed-adapter LoRA linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark, never by the product path. It shares
no code with the HIP library (its own C source, its own bf16 decode, its own
planner).
"""
from .oracle import (  # noqa: F401
    build,
    lora_rows,
    lora_merged,
    lora_grouped,
    decode_bf16,
    threads,
    set_threads,
)
from .plan import plan, work_list  # noqa: F401
