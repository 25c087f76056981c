"""CPU oracle for the Kimi Delta Attention (KDA) forward operator.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
path (``gated_delta_rule_67_amd``) and imports nothing from it.

Three independent CPU formulations, all in float64 numpy:

* ``recurrent`` / ``decode_step`` (O1, the oracle proper): the token-by-token
  recurrence as stated in the K3 README page ("KDA 训练 → 推理 手写实现"),
  roadmap table (实现路线表) row L1, with the order of operations given in the
  KDA CUDA Trainer README's model paragraph (decay, then the delta-rule write
  against the decayed state, then the read from the updated state).
* ``chunked`` (O2): the chunk-wise form in the four steps listed by the K3
  README's roadmap row L2 (in-chunk cumsum of g, decay-weighted lower
  triangular system, triangular solve, state passed between chunks).
* ``brute`` (O3): each token written as an affine map of the state, composed
  explicitly with K x K matrices. Only for tiny shapes.
* ``recurrent_bwd``: gradients of O1 by reverse-mode differentiation of each
  token step, written out (K3 README roadmap rows L1/L4).
* ``gate`` / ``gate_bwd``: the decay gate that produces g from the gate input,
  A_log and dt_bias (standard and safe, K3 README roadmap row L5), and its
  gradients.
* ``transforms``: the optional in-operator input transforms (q/k L2
  normalisation, beta sigmoid) that ``recurrent`` / ``decode_step`` apply on
  request.

Pins (tests/test_oracle_*.py) tie these to each other and to closed forms, a
hand-worked example, invariants and brute force. No function here is
"parity unpinned".
"""

from .recurrent import decode_step, recurrent
from .chunked import chunked, forward_substitution_inverse
from .brute import brute
from .transforms import l2_normalize, sigmoid
from .backward import recurrent_bwd
from .gate import gate, gate_bwd

__all__ = [
    "decode_step",
    "recurrent",
    "chunked",
    "forward_substitution_inverse",
    "brute",
    "l2_normalize",
    "sigmoid",
    "recurrent_bwd",
    "gate",
    "gate_bwd",
]
