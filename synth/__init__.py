"""Seeded synthetic inputs for paged FP8-KV attention (input generation only)."""

from .workloads import (  # noqa: F401
    CONFIGS,
    PAGE_SIZE,
    POISON_BYTE,
    Workload,
    custom_workload,
    empty_pages,
    k_to_layout,
    make_workload,
    v_to_layout,
)
