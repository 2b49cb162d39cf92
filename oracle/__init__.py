"""CPU oracle for lossless draft verification and confidence-scheduled lengths.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check in
`__graft_entry__.smoke()` and the CPU-baseline leg of the benchmark use it.  The HIP
library never routes through it and shares no code with it.

It is a plain, slow, fp64 restatement of what the method computes, written
from the DSpark pages:

  * `verify`        -- rejection-sampling verification with the correction /
                       bonus token (DSpark paper, §1 and §2.1; appendix
                       counterexample for a length of zero);
  * `verify_greedy` -- the greedy (argmax) verification rule;
  * `verify_left_to_right` -- the same verification taken position by
                       position, stopping at the first rejection (§2.1);
                       what it never reaches is never examined;
  * `schedule`      -- survival products and the budgeted length selector
                       (DSpark paper, §3.2.2; Algorithm 1 as printed in the
                       Chinese translation of the paper);
  * `capacity`, `schedule_topk` -- the asynchronous scheduler of §5.2 (a
                       capacity from an earlier step, top-K admission now);
  * `overlap_mass`  -- the per-position overlap sum_v min(p_t, p_d) of the
                       target and draft distributions (DSpark paper, §3.2.1,
                       Eq. 8);
  * `markov_draft`  -- the Markov-head sequential draft sampler and the
                       confidence head (DSpark paper, §3.1 Eq. 4-5, §3.2.1
                       Eq. 7);
  * `sts_fit`, `sts_apply` -- Sequential Temperature Scaling of the
                       confidences (DSpark paper, §3.2.1, post-hoc
                       calibration);
  * `philox`        -- the counter-based generator the draws come from
                       (Philox4x64-10, Salmon et al., SC'11).

Every function states the passage it follows.  Pins that tie it to facts
outside itself live in tests/test_oracle_*.py.
"""

from .philox import draft_uniform, philox4x64_10, uniforms  # noqa: F401
from .verification import (  # noqa: F401
    STATUS_BAD_LENGTH,
    STATUS_BAD_TEMPERATURE,
    STATUS_BAD_TOKEN,
    STATUS_BAD_TOPK,
    STATUS_NONFINITE,
    FLAG_ACCEPT_WINDOW,
    FLAG_EMIT_WINDOW,
    inverse_cdf,
    kept_mask,
    log_probs,
    verify,
    verify_greedy,
    verify_left_to_right,
)
from .overlap import overlap_mass  # noqa: F401
from .drafting import markov_draft, round_bf16  # noqa: F401
from .calibration import ece, sts_apply, sts_fit  # noqa: F401
from .scheduling import (  # noqa: F401
    capacity,
    survival,
    schedule,
    schedule_bruteforce,
    schedule_topk,
    theta_path,
)
