"""CPU oracle for batched draft-block verification -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the hot path computes, step by
step, in the order and notation of the pages.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from it.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path never does.

Sources (cited by page title and section):

* "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion
  Drafters" (arXiv 2607.19223) -- Section 2.1 (acceptance test, first-rejection
  truncation, residual resample, closed form of the expected output length),
  Section 3.1 (entry-wise clipped reverse-KL equation; the hard-label cross-entropy
  and the mixture OPD loss), Section 3.2 (the adaptive length head and its loss; per-request
  verification length), Section 3.3 (packed batch of total length sum k_i),
  Appendix B.1 (greedy decoding default, reverse-KL temperature 1).
* "AdaFlash reading notes" (zhongzhuzhou.org blog) -- steps 3-4 of the basic
  speculative-decoding recipe (normalised residual max(0, p - q)); Algorithm 2
  (entry-wise clipped reverse-KL); the complete numeric example for one toy
  position.
* "D3D: Decoupled Diffusion Drafting for Asynchronous Speculative Decoding" review page --
  Methodology, inference paragraph (prepared successor blocks, the packed budget
  B((C - 1) F + 2), cache hits on a matching verified prefix).
* "DFlash: Block Diffusion for Flash Speculative Decoding" notes
  (zhangshuibai.github.io) -- Section 3.1 step 6 (a bonus token when every draft
  is accepted, m + 1 tokens per round); Section 5.2 (rejection sampling with the
  drafter's per-position marginals; worked example #4, greedy verification).

Every function is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, library routines and brute force.  Conventions the pages
leave open are fixed here and listed in the repository's design notes:

* acceptance is ``u < min(1, p/q)`` (equality rejects), u in [0, 1);
* the uniform slot ``k_b`` of a request drives its single final-token draw;
* the final token is the smallest id whose cumulative (unnormalised) mass
  exceeds ``u * Z``; if rounding leaves none, the largest id with positive mass;
* a residual with zero mass (possible only through rounding) falls back to p_T;
* temperature 0 is greedy: accept iff the draft equals the target argmax, the
  final token is the target argmax, ties go to the lowest id;
* the clipped reverse-KL always uses temperature 1 and applies min(delta, .)
  per entry, so negative entries pass unchanged and R may be negative;
* for temperature-0 requests the reported p(x), q(x) are the temperature-1
  probabilities.

Parity status: the inverse-CDF tie conventions above (which id a given u maps
to at a bin edge, the zero-mass fallback) are fixed by choice, not by the
pages; the losslessness tests pin only their law.  Everything else is pinned.
"""

from .verify import (  # noqa: F401
    widen_logits,
    log_softmax,
    greedy_argmax,
    acceptance,
    inverse_cdf,
    final_token_distribution,
    verify_request,
    verify_block,
    expected_tau,
)
from .rkl import clipped_rkl_row, clipped_rkl  # noqa: F401
from .opd import hard_ce_row, opd_loss, clipped_rkl_grad_row, opd_grad  # noqa: F401
from .length_head import (  # noqa: F401
    length_head,
    length_loss,
    packed_offsets,
    silu,
    truncate,
    truncation_margin,
)
from .branch import branch_lookup, final_tokens  # noqa: F401
from .tree import tree_valid, verify_tree_block, verify_tree_greedy  # noqa: F401
