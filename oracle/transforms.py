"""Input transforms some callers leave to the operator, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

* q/k L2 normalisation: the K3 README page's test-status table lists the chunk
  kernels (rows L3/L4) as run on L2-normalised q and k, normalised inside the
  operator. Each (token, head) vector x of K channels becomes
  ``x / sqrt(sum(x^2) + EPS)``. The pages state no epsilon; EPS = 1e-6 keeps a
  zero vector at zero and changes a unit vector by under 1e-6 relatively.
* beta sigmoid: the KDA CUDA Trainer README's usage notes name a CUDA path that
  applies the sigmoid to beta itself; with it, the operator receives the logit
  and uses ``1 / (1 + exp(-beta))``.

``recurrent`` and ``decode_step`` take ``qk_l2norm`` / ``beta_sigmoid`` flags and
apply these before the recurrence.
"""

import numpy as np

EPS = 1e-6


def l2_normalize(x):
    """x / sqrt(sum over the last axis of x^2 + EPS), float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def sigmoid(x):
    """1 / (1 + exp(-x)), float64, computed without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
