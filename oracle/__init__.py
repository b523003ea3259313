"""CPU oracle for the fused attention forward and its gradients (test
infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the GPU library or its Python binding.
"""
from .attention import (  # noqa: F401
    admitted, attention, attention_backward, kv_head_of, modified_scores, pair_count,
    tile_classes,
)
