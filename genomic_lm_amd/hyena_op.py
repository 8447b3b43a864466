"""The four core calls of the Hyena operator under short names.

    hyena_op.fftconv(x1, x2, v, log_poles, residues, skip) -> y
    hyena_op.fir(x1, x2, v, taps, skip)                     -> y
    hyena_op.chunk(x1, x2, v, log_poles, residues, C, skip, state_in=None)
                                                            -> (y, state_out)
    hyena_op.modal_filter(log_poles, residues, L)           -> h

They are the functions of the package binding (hyena_fftconv_fwd,
hyena_fir_fwd, hyena_chunk_fwd, hyena_modal_filter of libhyena.so), which
only check and marshal their arguments.
"""
from . import chunk_fwd as chunk
from . import fftconv_fwd as fftconv
from . import fir_fwd as fir
from . import modal_filter

__all__ = ["fftconv", "fir", "chunk", "modal_filter"]
