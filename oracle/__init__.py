"""Float64 CPU oracle for the RWKV-4 WKV operator.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the libwkv C-ABI
library and its Python binding) imports, links or calls this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.

It evaluates what the pages define, slowly and plainly:

* ``wkv_direct``      -- the defining sums of the WKV equation, O(T^2)
* ``wkv_direct_at``   -- the same sums for single (lane, t) samples
* ``wkv_recurrent``   -- the RNN-mode form with an (A, B) state, O(T)
* ``wkv_step_ref``    -- one RNN-mode step from a given (a, b, p) state
* ``wkv_mp``          -- the defining sums at 50 significant digits (mpmath)
* ``wkv_backward_direct`` -- gradients of the defining sums, O(T^2)
* ``wkv_backward_recurrent`` -- the same gradients by forward and reverse recurrences, O(T)
* ``token_shift``, ``token_shift_backward`` -- the time-mixing token shift (lerp of
  x_t and x_{t-1}) and its gradients
* ``wkv_gated``, ``wkv_gated_backward`` -- the output gate sigmoid(r) * wkv and its gradients
  (``*_recurrent``: the same from the O(T) forms, for long sequences)
* ``linear_attention_direct``, ``linear_attention_recurrent`` -- causal linear attention
  (the linear-transformer page), masked sums and cumulative-state forms
* ``scaled_error``    -- the scale-normalised error used as the parity gate

Citations name the page ("Reinventing RNNs for the Transformer Era: RWKV",
a paper review on velog, or the linear-transformer review "Transformers are
RNNs: ...") and its section/equation.
"""
from .wkv_oracle import (  # noqa: F401
    EMPTY_P,
    scaled_error,
    wkv_direct,
    wkv_direct_at,
    wkv_recurrent,
    wkv_step_ref,
    state_log_b,
    state_ratio,
)
from .wkv_mp import wkv_mp  # noqa: F401
from .wkv_grad import wkv_backward_direct, wkv_backward_recurrent  # noqa: F401
from .linear_attention import elu_feature, linear_attention_direct, linear_attention_recurrent  # noqa: F401
from .wkv_mix import (  # noqa: F401
    sigmoid,
    token_shift,
    token_shift_backward,
    wkv_gated,
    wkv_gated_backward,
    wkv_gated_backward_recurrent,
    wkv_gated_recurrent,
)
