"""Plain, slow, float64 CPU oracle for the sampled-token logprob and the
REINFORCE Zero loss and gradient.

TEST INFRASTRUCTURE. Only the test suite, the smoke check of the package
entry point and the benchmark's CPU-baseline leg may import this package.
The product path (the HIP library and its Python binding) never imports,
calls or links anything here, and nothing here imports the product path.

Sources (web pages, cited by title and section):

* "vLLM says aligned kernels make asynchronous RL stable at lag 64",
  section "REINFORCE Zero removes the mismatch first": the rollout records
  each sampled token's logprob, the learner divides its own probability by
  that record (token-level importance ratio, no clipping), the advantage is
  the response's reward minus its group's mean reward, tokens are averaged
  within a response, and the objective is plain REINFORCE.
* "vLLM Train-Inference Consistency Release Notes", sections "Overview" and
  "Achieving Bitwise Consistency": logprobs of the sampled tokens are the
  quantity rollout and learner must agree on.

The pages never write the logprob as a formula. The oracle takes the plain
definition of a token's log-probability under a softmax output head:
z = W h (an LM-head contraction), lp = z[y] - log sum_v exp(z[v]).

Every function evaluates its definition in float64 on the exact values of
its inputs: bfloat16 bit patterns (numpy uint16) and float32 numbers both
convert to float64 without rounding.

The mismatch diagnostics (oracle/diagnostics.py) follow the pages' split of
the learner/rollout logprob gap into weight lag and kernel mismatch; their
readings and pins are listed in that module.

Pins (see tests/test_oracle_*.py): brute force in 60-digit decimal
arithmetic on tiny vocabularies, exact rational dot products, closed forms
(uniform logits, one dominant logit), shift invariance, lp <= 0, the
softmax summing to one, advantages summing to zero per group, ratio == 1
exactly at zero lag, the loss reducing to plain REINFORCE at zero lag,
central finite differences of the loss for the gradient, and torch float64
autograd. The end-to-end numbers the pages report are not recomputable from
any inputs: parity against the pages' own figures is unpinned.
"""

from .lmhead import to_f64, logits, log_softmax_at, lmhead_logprob
from .diagnostics import STAT_NAMES, mismatch_stats
from .fp8 import e4m3_decode, e4m3_encode, quantize_rows_fp8, lmhead_logprob_fp8
from .fp8 import e2m1_decode, e2m1_encode, quantize_rows_mxfp4, mxfp4_decode, lmhead_logprob_mxfp4
from .reinforce_zero import (
    group_advantage,
    importance_ratio,
    reinforce_zero_loss,
    reinforce_zero_backward,
    reinforce_zero_backward_rows,
    reinforce_zero_objective,
)

__all__ = [
    "to_f64",
    "logits",
    "log_softmax_at",
    "lmhead_logprob",
    "group_advantage",
    "importance_ratio",
    "reinforce_zero_loss",
    "reinforce_zero_backward",
    "reinforce_zero_backward_rows",
    "reinforce_zero_objective",
    "STAT_NAMES",
    "mismatch_stats",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_rows_fp8",
    "lmhead_logprob_fp8",
    "e2m1_decode",
    "e2m1_encode",
    "quantize_rows_mxfp4",
    "mxfp4_decode",
    "lmhead_logprob_mxfp4",
]
