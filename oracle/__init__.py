"""CPU oracle (test infrastructure only; see ``sketch_oracle``)."""
from .sketch_oracle import (  # noqa: F401
    adam_step,
    backward_dlut,
    backward_dlut_loop,
    backward_dx,
    dequantize,
    forward,
    forward_multi,
    group_of_column,
    pack_indices,
    rel_err,
    sgd_step,
    unpack_indices,
    weight_gradient,
)
