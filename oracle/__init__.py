"""Plain fp64 CPU oracle of one tree-verification step.  TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, links or calls it, and it shares no code with that path: the
only thing both sides use is the seeded input generator in ``workloads``.

Source of the method: JetSpec GitHub README, "JetSpec > Overview" (the target
verifies the whole draft tree in one forward pass under a tree-causal mask;
the accepted path follows the target's own logits, which makes decoding
lossless), and the EQSPEC/EXSPEC abstract (arXiv 2510.22876, on the RSS reader
page) for output equivalence with step-by-step greedy decoding and for the
per-sequence KV state of a ragged batch.

Every function here is the plain definition written out, with library
primitives (matmul, argmax, partition) as single steps.  Pins that tie each
function to something other than itself live in tests/test_oracle_pins.py.
"""
from .verify import (  # noqa: F401
    ancestors,
    decode,
    kv_commit_slots,
    kv_compact,
    kv_compact_paged,
    lm_head_argmax,
    paged_to_contiguous,
    round_bf16,
    lm_logits,
    tree_accept,
    tree_attention,
    tree_attention_paged,
    verify_step,
)
from .tree_build import accum_logp_tree, accum_logp_tree_paths, topk_tokens  # noqa: F401
from .model import (  # noqa: F401
    ar_decode,
    kv_compact_layers,
    node_positions,
    rms_norm,
    rope,
    silu,
    verify_pass,
)
