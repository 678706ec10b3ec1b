"""Plain CPU oracle for batched speculative-decoding verification and paged KV bookkeeping.

TEST INFRASTRUCTURE. This package is the slow, obviously-correct reference that the HIP
library is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the HIP path
(``rejection_sampling_verify_specdec_amd``) and imports nothing from it.

Arithmetic is fp64 (NumPy) or exact (``fractions.Fraction``) where the functions are
written generically. Sources, cited by page title and section:

* "Speculative decoding: accelerate LLM generation without changing its answers"
  (chaowen.tw daily lesson), section 2 "Draft, verify, correct", section 3 "Why this
  preserves the target distribution", section 5 "Reproducible toy lab" and its two
  variations, section 6 "Production failures" (stable softmax, identical transforms).
* "Walk through KV-cache updates when speculative decoding rejects some draft tokens"
  (zenaique.com), both paragraphs: provisional append, left-to-right test, paged free /
  contiguous rewind.
* "Keep cache validity aligned with the committed token history"
  (study.greatitself.com), paragraphs 1-4: pending-token convention, partial validity,
  block tables / refcounts, shared-prefix isolation and copy-on-write.
* "rejected speculative tokens remain in KV" (archcrux.com): partial-block validity and
  the per-step record.

Where the pages leave a step open the reading taken is stated at the function.
"""

from .verify import (  # noqa: F401
    ERR_TOKEN, ERR_K, ERR_NONFINITE, ERR_QZERO, ERR_ZFALLBACK, ERR_UNIFORM, ERR_PARAM,
    params_ok, bf16_bits_to_f64, Transformed, transform, accept, residual_weights,
    inverse_cdf, inverse_cdf_np, verify_probs, verify_request, verify_batch,
    BatchResult,
)
from .analytics import (  # noqa: F401
    acceptance_rate, expected_emitted, acceptance_batch,
)
from .tree import (  # noqa: F401
    ERR_TREE, children_of, tree_verify_probs, tree_verify_request, tree_verify_batch,
    tree_commit,
)
from .kv import (  # noqa: F401
    KV_ERR_NOMEM, KV_ERR_APPEND, KV_ERR_ROLLBACK,
    PagedKV, ContiguousKV,
)
