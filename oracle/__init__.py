"""CPU oracle for one ISD decode step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the HIP path computes.  Only the
tests, `__graft_entry__.smoke()` and the benchmark's CPU-baseline leg may import it;
the product path never does.  It shares no code with the HIP library or its binding.

Modules:
  stored     exact decoding of stored values (bf16 bit patterns, float32) to float64
  attention  strictly causal GQA attention of the 2N-1 strided rows over a paged cache
  verify     anchor p / proposal q distributions, min(1, p/q) walk, residual resampling
  proj       R-ISD gated-LoRA projection
  layer      an R-ISD decoder layer: seven gated linears around the block's attention
  lm_head    logits of the block rows (nearest bf16 of the product), then verification
  chain      tokens-per-forward closed form, hot/cold chain simulation, estimator

Pins (tests/test_oracle_*.py) tie each function to something other than itself:
brute force on tiny inputs, library special cases, exact laws (chi-square), closed
forms and the values the pages print.  Nothing here is "parity unpinned".
"""
from . import attention, chain, layer, lm_head, proj, stored, verify  # noqa: F401
from .attention import attention_step  # noqa: F401
from .chain import efficiency, renewal_estimate, simulate_chain, tpf_closed_form  # noqa: F401
from .layer import decoder_layer  # noqa: F401
from .lm_head import lm_head_logits, lm_head_verify  # noqa: F401
from .proj import gated_lora_proj  # noqa: F401
from .verify import commit as commit_step  # noqa: F401
from .verify import verify as verify_step  # noqa: F401
