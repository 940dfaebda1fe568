"""fp64 CPU oracle of the Multi-head Latent Attention forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP library never calls it and shares no code with it.

Sources (web pages, cited by title and section):
  * "MLA(Multi-Head Latent Attention)" blog walk-through of vLLM's MLA code
    (the projection, cache-update, forward_mha / forward_mqa and cache-spec
    listings),
  * SpecForge PR "Add config-selectable MLA draft attention" (Summary,
    Structure) and PR "extract GQA/MLA attention into reusable layers"
    (Modifications, Accuracy Test).

The gradient of the expanded layer (training form) is in oracle.backward.

Parity status: every function is pinned by the CPU tests (tests/oracle_pins.py,
run by tests/test_oracle.py) except the
choices the pages leave open (RMSNorm eps value, softmax scale, RoPE theta,
output-gate form), which are "parity unpinned" conventions shared with the
library.
"""
from .mla import (  # noqa: F401
    MASK_CAUSAL, MASK_FULL, MASK_SLIDING, ROPE_INTERLEAVED, ROPE_NEOX,
    apply_rope, attention_core, brute_force_forward, expand_kv, forward_sequence,
    mla_forward, project_tokens, rms_norm, rope_pairs, visible_interval,
)
