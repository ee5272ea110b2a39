"""CPU oracle of the routed MoE layer and its slot cache.

TEST INFRASTRUCTURE: only tests/, the smoke check in __graft_entry__ and the
bench's cpu_baseline leg may import this package.  It shares no code with the
HIP library (expert_ffn_execution_router_amd) and never imports it.

  formats  exact decoding of bf16 / OCP E4M3FN / OCP MX (E2M1, E8M0)
  moe      routing, grouping, SwiGLU experts, the layer (exact and mirrored)
  cache    global LRU slot model, q* split, link-bound prefill time

Every function is pinned by tests/test_oracle_*.py against values that do not
come from the oracle itself (format definitions, hand-computed worked
examples, a dense brute force, closed forms and invariants).  The end-to-end
layer output has no worked example on the pages: it is pinned only by the
brute force and the invariants.
"""
from . import cache, formats, moe  # noqa: F401
