"""CPU oracle (test infrastructure only): see oracle.lora_oracle."""
from .lora_oracle import (  # noqa: F401
    decode, build_addressing, expert_keys, build_addressing_experts, shrink, gather_shrink,
    expand, base_projection,
    shrink_all_slots, apply_scalar, run_target, within_tolerance,
)
