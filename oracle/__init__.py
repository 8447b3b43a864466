"""fp64 CPU oracle of the Hyena operator -- TEST INFRASTRUCTURE ONLY.

Importable from the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg; never from the product path.
"""
from .hyena_oracle import (  # noqa: F401
    modal_filter, conv_direct, conv_fft, causal_conv, hyena_fwd, fir_fwd,
    modal_state, chunk_fwd, next_pow2, modal_decode, fir_fwd_window,
    modal_filter_cpx, hyena_fwd_cpx, modal_state_cpx, chunk_fwd_cpx, modal_decode_cpx,
    tokmajor_streams, chunk_fwd_tokmajor, fir_fwd_tokmajor,
)
from .metrics import (compare, passes, channel_stats, from_stats,  # noqa: F401
                      REL_L2_MAX, ELEM_REL_MAX, TAU)
