"""CPU oracle for the LiSA forward and backward passes -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 NumPy statement of what the LiSA
(Linear Stochastic Attention) forward pass computes, written from the paper
"LiSA: Linear Stochastic Attention for Long-Range Visual Modeling"
(arXiv:2611.04216v2) as described by its reading note, sections 2.1-2.5.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls into it, and it
shares no code with the GPU library: no kernels, helpers, tables or constants.
The only thing both sides consume is the seeded synthetic input generator,
which holds none of the method's arithmetic and which this package does not
import.

``oracle.backward`` holds the exact derivative of that forward pass
(gradients for Q, K, V, the adaptive weights and alpha), pinned by
``tests/test_oracle_backward_pins.py`` (finite differences, explicit n x n
powers of S, branch isolation, planted mistakes).

``oracle.predictor`` holds the per-token walk-weight predictor (a two-layer
MLP on concat(Q_i, K_i) and a softmax), pinned by
``tests/test_oracle_predictor_pins.py``.

``oracle.layer`` holds a LiSA attention layer (QKV projection, heads, the
operator, output projection), pinned by ``tests/test_oracle_layer_pins.py``.

Every function of ``oracle.lisa`` is pinned by ``tests/test_oracle_pins.py``
to facts other than itself (brute force on tiny grids, closed forms,
invariants, hand-derived examples under ``tests/golden/``).  The one place
where parity is unpinned is stated in ``oracle.lisa``'s module docstring.
"""

from .lisa import (  # noqa: F401
    feature_map,
    geometric_weights,
    walk_weights,
    normaliser,
    stats,
    global_branch,
    local_branch,
    local_branch_loop,
    mix,
    lisa_forward,
    lisa_bruteforce,
    neighbour_offsets,
)
from .predictor import predicted_weights, lisa_forward_mlp  # noqa: F401
from .layer import lisa_layer  # noqa: F401
from .backward import (  # noqa: F401
    global_branch_backward,
    local_branch_backward,
    lisa_backward,
)
