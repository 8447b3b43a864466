"""Index arithmetic of the on-chip Stockham FFT (genomic_lm_amd/csrc/fft.hpp),
checked on the host for every transform shape the kernels instantiate.

The LDS exchange of each pass pads every 32-element row by one element
(lds_pad(i) = i + i/32).  The kernels compute one padded base per butterfly
and reach its other elements through constant offsets, which is valid only if
lds_pad(base + r*NS) = lds_pad(base) + r*NS + (r*NS >> 5) for all of a pass's
indices.  This test walks every thread of every pass (stores and the next
pass's loads) and checks that identity, and that the stores of a pass write
each of the S elements exactly once.
"""
import pytest


def pad(i):
    return i + (i >> 5)


def radix(S, T, NS):
    P = min(S // T, 16)
    return P if S // NS >= P else S // NS


# (S, T) of every instantiation: fftconv.hip (two-half kernels S <= 4096,
# one-half kernels S = 8192, 16384), chunk_fft.hip (S = C/2), and
# fftconv_large.hip (size-256 column transforms; row transforms S1 = 128 ..
# 1024, forward with S1/8 threads, inverse with S1/4)
SHAPES = sorted({(256, 64), (512, 64), (1024, 128), (2048, 256), (4096, 512), (8192, 512),
                 (16384, 1024),
                 (1024, 64), (2048, 128), (4096, 256),
                 (256, 32), (128, 16), (256, 32), (512, 64), (1024, 128),
                 (128, 32), (256, 64), (512, 128), (1024, 256)})


@pytest.mark.parametrize("S,T", SHAPES)
def test_pass_offsets_affine(S, T):
    P = S // T
    NS = 1
    while NS < S:
        R = radix(S, T, NS)
        NB = P // R
        written = set()
        for t in range(T):
            for b in range(NB):
                j = t + T * b
                base = (j // NS) * NS * R + (j & (NS - 1))
                for r in range(R):
                    idx = base + r * NS
                    assert pad(idx) == pad(base) + r * NS + ((r * NS) >> 5), (S, T, NS, t, b, r)
                    assert idx not in written
                    written.add(idx)
        assert len(written) == S
        if NS * R < S:
            R2 = radix(S, T, NS * R)
            Q = S // R2
            for t in range(T):
                for b in range(P // R2):
                    jp = t + T * b
                    for r in range(R2):
                        assert pad(jp + r * Q) == pad(jp) + r * Q + ((r * Q) >> 5), (S, T, NS, t, b, r)
        NS *= R
