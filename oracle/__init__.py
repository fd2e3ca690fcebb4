"""CPU oracle for the DSpark draft -> schedule -> verify step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
restatement of what the method computes, written from the pages that describe
DSpark.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the HIP path (the package
``draft_verify_schedule_amd``) and never imports it; the HIP path never imports
this package.

Sources, cited by page title and section:

* "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
  Generation" (bilingual PaperTrace copy of the paper): section 2.1 (accept
  rule, left-to-right verification), section 3.1 (semi-autoregressive
  factorisation, Markov head), section 3.2.2 (Algorithm 1), section 5.2
  (asynchronous capacity, dynamic top-K), Appendix A (selection-bias
  counterexample).
* Paperglide simplified reader of the same paper: the two-request scheduling
  example ("The DSpark Architecture"), the clean restatement of Algorithm 1,
  and the Appendix A numbers ("Theoretical Caveats and Selection Bias").
* "Speculative decoding, from zero to DSpark" (The Information Bottleneck):
  section 2 (acceptance rule, residual distribution, TV identity), section 6
  (the factorised Markov bias), section 8 (objective, survival products,
  greedy admission), Appendix A1 (why the rejection rule is exact), A4
  (dimensions of W1 and W2), A6 (empty-system limit).
* The glean.smartcoder article on DSpark: the five-step description of the
  verification routine (target probabilities, min(1, p/q) test against a
  uniform, prefix truncation, residual-or-bonus sample, concatenation).

Randomness is fixed by one counter-based uniform per decision (``philox``);
every categorical draw is an inverse-CDF draw in ascending token-id order.

Modules:
  philox    -- Philox4x32-10 and the per-decision uniform
  draft     -- sequential Markov-head drafter (draft_ref, independent_draft_ref)
  rnn       -- sequential RNN-head drafter (rnn_cell_ref, rnn_draft_ref)
  schedule  -- Algorithm 1 and its modes (schedule_ref), brute force
  verify    -- rejection-sampling verification (verify_ref)
  step      -- the composed step (run_step)
"""

from .philox import philox4x32_10, uniform, PURPOSE_DRAFT, PURPOSE_ACCEPT, PURPOSE_RESAMPLE
from .draft import draft_ref, independent_draft_ref
from .schedule import (schedule_ref, schedule_async_ref, schedule_bruteforce, SCHED_EARLY_STOP,
                       SCHED_GLOBAL, SCHED_TOPK)
from .verify import verify_ref
from .label import acceptance_label_ref
from .confidence import confidence_head_ref, confidence_logits_ref, ece_ref, sts_fit_ref
from .rnn import rnn_cell_ref, rnn_draft_ref
from .step import run_step

__all__ = [
    "philox4x32_10", "uniform", "PURPOSE_DRAFT", "PURPOSE_ACCEPT", "PURPOSE_RESAMPLE",
    "draft_ref", "independent_draft_ref",
    "schedule_ref", "schedule_async_ref", "schedule_bruteforce", "SCHED_EARLY_STOP", "SCHED_GLOBAL",
    "SCHED_TOPK",
    "verify_ref", "run_step", "acceptance_label_ref",
    "confidence_head_ref", "confidence_logits_ref", "ece_ref", "sts_fit_ref",
    "rnn_cell_ref", "rnn_draft_ref",
]
