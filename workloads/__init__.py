"""Seeded synthetic inputs for lossless draft verification.

This module only *makes inputs*: logits, draft tokens, temperatures, top-k
sizes, RNG seeds, per-position confidences and the engine cost table.  It
holds none of the verification or scheduling arithmetic: no softmax, no
log-sum-exp, no acceptance test, no residual, no survival product and no
throughput objective.  Both the HIP path and the CPU oracle consume the very
tensors built here, and nothing else is shared between them.

The drafter is simulated: a draft token is drawn from the draft logits with
the Gumbel-max trick (argmax of logits/T plus Gumbel noise, restricted to the
top-k set where one applies).  That is the drafter's job upstream of the
verifier, so it lives with the inputs.

`workloads.drafting` makes the draft sampler's inputs (base logits, the
Markov head's weights, anchors, hidden states); it too holds random numbers
only.

Shapes follow the statement of the problem in the DSpark paper, §2.1
(gamma draft tokens per request, target and draft distributions per draft
position over a vocabulary) plus one extra target row per request for the
token the target appends after the block (DSpark paper, §1; §3.2.2 counts
1 + l_r target tokens per request).
"""

from .configs import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    make_verify_inputs,
    make_greedy_inputs,
    make_confidences,
    make_sps_table,
    sample_draft_tokens,
)
from .drafting import DraftInputs, make_draft_inputs  # noqa: F401
from .calibration import make_sts_inputs, tau_grid  # noqa: F401
