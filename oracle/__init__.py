"""CPU oracle for the sparse MoE layer forward (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
does, and the two share no code.
"""
from .moe_ref import (  # noqa: F401
    Dispatch,
    Routing,
    RoutingStats,
    capacity,
    capacity_dispatch,
    combine,
    expert_choice_dispatch,
    expert_ffn_rows,
    expert_slots_out,
    gelu,
    moe_forward,
    moe_forward_expert_choice,
    renormalise_survivors,
    route_topk,
    routing_stats,
    shared_expert_out,
    router_logits,
    to_f64,
)
