"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

Only calls whose arguments fail validation are made here; those return before
any HIP call.  The last test checks that the benchmark refuses to run on more
than one GPU before it touches one."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import genomic_lm_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyena.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(G.LIB_PATH):
        from genomic_lm_amd import build
        build.build()
    yield


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(hyena_[a-z0-9_]+)\s*\(", text))


def test_header_declares_the_binding_set():
    assert declared_functions() == set(G.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = declared_functions() - syms
    assert not missing, missing
    lib = G.lib()
    for name in declared_functions():
        assert hasattr(lib, name)


def test_version_and_status_strings():
    assert G.abi_version() == 8
    for st in range(5):
        assert G.status_string(st).startswith("HYENA_")
    assert "UNKNOWN" in G.status_string(99)


P = ctypes.c_void_p
FAKE = P(0x10000)            # never dereferenced: every call below fails validation first
MISALIGNED = P(0x10001)


def test_modal_filter_validation():
    f = G.lib().hyena_modal_filter
    assert f(None, None, 4, 16, 8, None, None) == G.ERR_INVALID_ARG
    assert f(FAKE, FAKE, -1, 16, 8, FAKE, None) == G.ERR_INVALID_ARG
    assert f(FAKE, FAKE, 4, 0, 8, FAKE, None) == G.ERR_INVALID_ARG
    assert f(FAKE, FAKE, 4, 65, 8, FAKE, None) == G.ERR_INVALID_ARG
    assert f(FAKE, MISALIGNED, 4, 16, 8, FAKE, None) == G.ERR_INVALID_ARG
    assert f(None, None, 0, 16, 8, None, None) == G.OK          # empty: nothing to do
    assert f(None, None, 4, 16, 0, None, None) == G.OK


def test_fir_validation():
    f = G.lib().hyena_fir_fwd
    good = (FAKE, FAKE, FAKE, FAKE, 7, None, FAKE, 1, 4, 64, G.BF16, None)
    bad = list(good); bad[0] = None
    assert f(*bad) == G.ERR_INVALID_ARG
    bad = list(good); bad[4] = 0
    assert f(*bad) == G.ERR_INVALID_ARG
    bad = list(good); bad[4] = 1025
    assert f(*bad) == G.ERR_UNSUPPORTED
    bad = list(good); bad[10] = 7
    assert f(*bad) == G.ERR_INVALID_ARG
    bad = list(good); bad[9] = -3
    assert f(*bad) == G.ERR_INVALID_ARG
    bad = list(good); bad[1] = MISALIGNED
    assert f(*bad) == G.ERR_INVALID_ARG
    bad = list(good); bad[3] = None
    assert f(*bad) == G.ERR_INVALID_ARG
    empty = list(good); empty[9] = 0; empty[0] = None
    assert f(*empty) == G.OK


def test_fir_window_validation():
    f = G.lib().hyena_fir_fwd_window
    # x1 x2 v taps K skip win_in win_out y B D L io stream
    good = [FAKE, FAKE, FAKE, FAKE, 7, None, None, FAKE, FAKE, 1, 4, 64, G.BF16, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (3, None, G.ERR_INVALID_ARG),
                           (4, 0, G.ERR_INVALID_ARG), (4, 1025, G.ERR_UNSUPPORTED),
                           (7, None, G.ERR_INVALID_ARG),          # window_out needed when K > 1
                           (7, MISALIGNED, G.ERR_INVALID_ARG), (6, MISALIGNED, G.ERR_INVALID_ARG),
                           (11, -1, G.ERR_INVALID_ARG), (12, 5, G.ERR_INVALID_ARG)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[10] = 0; a[0] = None                     # D = 0: nothing to do
    assert f(*a) == G.OK
    a = list(good); a[4] = 1; a[7] = None; a[11] = 0; a[0] = None   # K = 1, L = 0: no window
    assert f(*a) == G.OK


def test_modal_decode_validation():
    f = G.lib().hyena_modal_decode
    # x1 x2 v lam res N skip s_in s_out y B D io stream
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, None, FAKE, FAKE, 1, 4, G.BF16, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (3, None, G.ERR_INVALID_ARG),
                           (5, 0, G.ERR_INVALID_ARG), (5, 65, G.ERR_INVALID_ARG),
                           (8, None, G.ERR_INVALID_ARG), (7, MISALIGNED, G.ERR_INVALID_ARG),
                           (9, MISALIGNED, G.ERR_INVALID_ARG), (11, -2, G.ERR_INVALID_ARG),
                           (12, 9, G.ERR_INVALID_ARG)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[10] = 0; a[0] = None
    assert f(*a) == G.OK


def test_fftconv_validation():
    f = G.lib().hyena_fftconv_fwd
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, FAKE, 1, 4, 1024, G.BF16, None, 0, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (3, None, G.ERR_INVALID_ARG),
                           (5, 0, G.ERR_INVALID_ARG), (5, 65, G.ERR_INVALID_ARG),
                           (10, -1, G.ERR_INVALID_ARG), (11, 2, G.ERR_INVALID_ARG),
                           (10, 1 << 20, G.ERR_UNSUPPORTED)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    ws = G.lib().hyena_fftconv_workspace_size
    assert ws(1, 4, 1024, 16, G.BF16) == 0                     # on-chip path, no workspace
    assert ws(1, 4, 4096, 16, G.BF16) == 0
    # 4096 < L <= 32768: two on-chip launches, the even half's result
    # (S = 4096 ... 16384 complex fp32 per row) through the workspace, up to
    # 1 GiB of rows
    assert ws(1, 4, 4097, 16, G.BF16) == 4 * 8 * 4096
    assert ws(1, 4, 8192, 16, G.BF16) == 4 * 8 * 4096
    assert ws(1, 4, 8193, 16, G.BF16) == 4 * 8 * 8192
    assert ws(1, 4, 16384, 16, G.BF16) == 4 * 8 * 8192
    assert ws(1, 4, 16385, 16, G.BF16) == 4 * 8 * 16384
    assert ws(1, 4, 32768, 16, G.F32) == 4 * 8 * 16384
    assert ws(1, 4096, 32768, 16, G.BF16) == 4096 * 8 * 16384
    assert ws(4, 4096, 32768, 16, G.BF16) == 8192 * 8 * 16384
    assert ws(0, 4, 1024, 16, G.BF16) == 0
    # four-step path from L > 32768: 32 S bytes per row (u and h, two parity
    # halves, complex fp32), rows batched up to 1 GiB
    assert ws(1, 4, 32769, 16, G.BF16) == 4 * 32 * 32768
    assert ws(2, 3, 65536, 16, G.F32) == 6 * 32 * 32768
    assert ws(1, 4096, 262144, 16, G.BF16) == 256 * 32 * 131072
    assert ws(1, 4096, 1 << 19, 16, G.BF16) == 128 * 32 * 262144
    assert ws(1, 4, (1 << 19) + 1, 16, G.BF16) == 0             # beyond the largest FFT
    # missing, short or misaligned workspace is refused before any launch
    big = list(good); big[10] = 40000
    assert f(*big) == G.ERR_WORKSPACE
    need = ws(1, 4, 40000, 16, G.BF16)
    big[12] = FAKE; big[13] = need - 1
    assert f(*big) == G.ERR_WORKSPACE
    big[12] = P(0x10008); big[13] = need
    assert f(*big) == G.ERR_WORKSPACE
    # the same for the two-launch on-chip range
    mid = list(good); mid[10] = 20000
    assert f(*mid) == G.ERR_WORKSPACE
    mid[12] = FAKE; mid[13] = ws(1, 4, 20000, 16, G.BF16) - 1
    assert f(*mid) == G.ERR_WORKSPACE


def test_fftconv_noalloc_validation():
    """The scratch-free single pass validates like hyena_fftconv_fwd, before
    it looks up its scratch or launches anything."""
    f = G.lib().hyena_fftconv_fwd_noalloc
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, FAKE, 1, 4, 1024, G.BF16, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (3, None, G.ERR_INVALID_ARG),
                           (5, 0, G.ERR_INVALID_ARG), (5, 65, G.ERR_INVALID_ARG),
                           (10, -1, G.ERR_INVALID_ARG), (11, 2, G.ERR_INVALID_ARG),
                           (1, MISALIGNED, G.ERR_INVALID_ARG),
                           (10, 1 << 20, G.ERR_UNSUPPORTED)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[9] = 0; a[0] = None                     # D = 0: nothing to do
    assert f(*a) == G.OK
    assert _declaration("hyena_fftconv_fwd_noalloc")[-1] == ("hipStream_t", "stream")


def test_chunk_validation():
    f = G.lib().hyena_chunk_fwd
    # x1 x2 v lam res N skip s_in s_out y B D L C io stream  (AUTO algorithm)
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, None, FAKE, FAKE, 1, 4, 1024, 1024,
            G.BF16, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (8, None, G.ERR_INVALID_ARG),
                           (13, 0, G.ERR_INVALID_ARG), (14, 3, G.ERR_INVALID_ARG),
                           (5, 65, G.ERR_INVALID_ARG), (8, MISALIGNED, G.ERR_INVALID_ARG)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[5] = 33; a[13] = 16384; a[12] = 16384   # AUTO: > 32 modes take FFT chunks
    assert f(*a) == G.ERR_UNSUPPORTED                          # ... of at most 8192
    a = list(good); a[10] = 0                                  # empty batch
    assert f(*a) == G.OK
    # the same with the algorithm chosen: one more argument before the stream
    fa = G.lib().hyena_chunk_fwd_algo
    ga = good[:15] + [0, None]
    a = list(ga); a[15] = 3
    assert fa(*a) == G.ERR_INVALID_ARG
    a = list(ga); a[5] = 33; a[15] = G.ALGOS["mfma"]          # MFMA kernel holds <= 32 modes
    assert fa(*a) == G.ERR_UNSUPPORTED
    a = list(ga); a[13] = 16384; a[15] = G.ALGOS["fft"]; a[12] = 16384
    assert fa(*a) == G.ERR_UNSUPPORTED                         # FFT chunk > 8192
    a = list(ga); a[13] = 16384; a[15] = G.ALGOS["auto"]; a[12] = 16384; a[8] = None
    assert fa(*a) == G.ERR_INVALID_ARG
    a = list(ga); a[10] = 0
    assert fa(*a) == G.OK


def test_chunk_cpx_validation():
    f = G.lib().hyena_chunk_fwd_cpx_algo
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, None, None, FAKE, FAKE, 1, 4, 1024, 1024,
            G.BF16, 0, None]
    a = list(good); a[5] = 17; a[15] = G.ALGOS["mfma"]        # 17 complex modes: 34 real lanes
    assert f(*a) == G.ERR_UNSUPPORTED
    a = list(good); a[15] = 3
    assert f(*a) == G.ERR_INVALID_ARG
    a = list(good); a[5] = 0
    assert f(*a) == G.ERR_INVALID_ARG
    a = list(good); a[10] = 0                                  # empty batch
    assert f(*a) == G.OK
    fa = G.lib().hyena_chunk_fwd_cpx                           # AUTO, no algorithm argument
    a = good[:15] + [None]
    a[5] = 0
    assert fa(*a) == G.ERR_INVALID_ARG
    a[5] = 8; a[10] = 0
    assert fa(*a) == G.OK


def _declaration(name):
    """Parameter list of `name` in the header, as [(type, name)]."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = []
    if m.group(1).strip() == "void":
        return params
    for p in m.group(1).split(","):
        p = " ".join(p.split())
        typ, nm = p.rsplit(" ", 1)
        while nm.startswith("*"):
            typ, nm = typ + "*", nm[1:]
        params.append((typ.replace(" *", "*"), nm))
    return params


def test_chunk_fwd_has_the_scope_table_signature():
    """hyena_chunk_fwd takes exactly the boundary's parameter list: the
    activations, the modal parameters, the state in and out, the sizes, the
    chunk length, the I/O type and a HIP stream -- no algorithm selector."""
    want = [("const void*", "x1"), ("const void*", "x2"), ("const void*", "v"),
            ("const float*", "log_poles"), ("const float*", "residues"), ("int64_t", "N"),
            ("const float*", "skip"), ("const float*", "state_in"), ("float*", "state_out"),
            ("void*", "y"), ("int64_t", "B"), ("int64_t", "D"), ("int64_t", "L"),
            ("int64_t", "C"), ("hyena_dtype_t", "io"), ("hipStream_t", "stream")]
    assert _declaration("hyena_chunk_fwd") == want
    assert _declaration("hyena_chunk_fwd_algo") == want[:15] + [
        ("hyena_chunk_algo_t", "algo"), ("hipStream_t", "stream")]
    assert _declaration("hyena_fftconv_fwd")[-1] == ("hipStream_t", "stream")
    assert _declaration("hyena_fir_fwd") == [
        ("const void*", "x1"), ("const void*", "x2"), ("const void*", "v"),
        ("const float*", "taps"), ("int64_t", "K"), ("const float*", "skip"), ("void*", "y"),
        ("int64_t", "B"), ("int64_t", "D"), ("int64_t", "L"), ("hyena_dtype_t", "io"),
        ("hipStream_t", "stream")]
    # every entry point that launches work takes its stream as a hipStream_t
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    assert "void* stream" not in text
    for name in declared_functions():
        params = _declaration(name)
        if any(n == "stream" for _, n in params):
            assert params[-1] == ("hipStream_t", "stream"), name


def test_python_names_follow_the_boundary():
    from genomic_lm_amd import hyena_op
    assert hyena_op.fftconv is G.fftconv_fwd and hyena_op.chunk is G.chunk_fwd
    assert hyena_op.fir is G.fir_fwd and hyena_op.modal_filter is G.modal_filter
    for name in declared_functions() - {"hyena_abi_version", "hyena_status_string",
                                        "hyena_chunk_fwd_algo", "hyena_chunk_fwd_cpx_algo",
                                        "hyena_chunk_fwd_tokmajor_algo"}:
        assert callable(getattr(G, name)), name


def test_chunk_tokmajor_validation():
    f = G.lib().hyena_chunk_fwd_tokmajor
    # xin, pos x3, lam, res, N, skip, state_in, state_out, y, B, D, L, io, ws, ws_bytes, stream
    good = [FAKE, 0, 1, 2, FAKE, FAKE, 16, None, None, FAKE, FAKE, 1, 4, 64, G.BF16, None, 0,
            None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (10, None, G.ERR_INVALID_ARG),
                           (9, None, G.ERR_INVALID_ARG), (4, None, G.ERR_INVALID_ARG),
                           (1, 1, G.ERR_INVALID_ARG), (3, 3, G.ERR_INVALID_ARG),
                           (2, -1, G.ERR_INVALID_ARG), (6, 0, G.ERR_INVALID_ARG),
                           (6, 65, G.ERR_INVALID_ARG), (0, MISALIGNED, G.ERR_INVALID_ARG),
                           (14, 2, G.ERR_INVALID_ARG), (11, 65536, G.ERR_UNSUPPORTED),
                           (13, -1, G.ERR_INVALID_ARG)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[11] = 0                                  # empty batch
    assert f(*a) == G.OK
    ws = G.lib().hyena_chunk_tokmajor_workspace_size
    # one workgroup of 256 channels per channel group and segment; segments
    # of at least 64 tokens (a multiple of the tile) are cut so that about
    # 1024 workgroups run; B * P * D * N fp32 slots, none for one segment
    assert ws(1, 4, 64, 16, G.BF16) == 0                        # one segment
    assert ws(1, 4, 65, 16, G.BF16) == 1 * 2 * 4 * 16 * 4       # P = 2 segments of 64
    assert ws(1, 4, 4096, 16, G.BF16) == 64 * 4 * 16 * 4
    assert ws(1, 4096, 32768, 16, G.BF16) == 64 * 4096 * 16 * 4  # 16 groups x 64 segments of 512
    assert ws(1, 8192, 32768, 16, G.BF16) == 32 * 8192 * 16 * 4
    assert ws(2, 300, 1000, 3, G.F32) == 2 * 16 * 300 * 3 * 4
    assert ws(1, 4, 64, 0, G.BF16) == 0
    big = list(good); big[13] = 4096                           # needs a workspace
    assert f(*big) == G.ERR_WORKSPACE
    need = ws(1, 4, 4096, 16, G.BF16)
    big[15] = FAKE; big[16] = need - 1
    assert f(*big) == G.ERR_WORKSPACE
    big[15] = P(0x10008); big[16] = need
    assert f(*big) == G.ERR_WORKSPACE
    # the same arguments with the evaluation named (algo after io)
    fa = G.lib().hyena_chunk_fwd_tokmajor_algo
    ga = good[:15] + [0] + good[15:]
    for algo, want in [(1, G.ERR_UNSUPPORTED), (4, G.ERR_INVALID_ARG), (-1, G.ERR_INVALID_ARG)]:
        a = list(ga); a[15] = algo
        assert fa(*a) == want, algo
    # D = 4 is not a multiple of 8: the matrix-core evaluation does not apply
    a = list(ga); a[15] = 2
    assert fa(*a) == G.ERR_UNSUPPORTED
    # the recurrence, named or taken by AUTO, still asks for its workspace
    a = list(ga); a[15] = 3; a[13] = 4096
    assert fa(*a) == G.ERR_WORKSPACE
    a = list(ga); a[15] = 0; a[13] = 4096
    assert fa(*a) == G.ERR_WORKSPACE


def test_fir_tokmajor_validation():
    f = G.lib().hyena_fir_fwd_tokmajor
    # xin, pos x3, taps, K, skip, window_in, window_out, y, B, D, L, io, stream
    good = [FAKE, 0, 1, 2, FAKE, 7, None, None, None, FAKE, 1, 4, 64, G.BF16, None]
    for idx, val, want in [(0, None, G.ERR_INVALID_ARG), (4, None, G.ERR_INVALID_ARG),
                           (9, None, G.ERR_INVALID_ARG), (5, 0, G.ERR_INVALID_ARG),
                           (5, 129, G.ERR_UNSUPPORTED), (1, 1, G.ERR_INVALID_ARG),
                           (3, 5, G.ERR_INVALID_ARG), (10, 65536, G.ERR_UNSUPPORTED),
                           (13, 2, G.ERR_INVALID_ARG), (0, MISALIGNED, G.ERR_INVALID_ARG),
                           (7, MISALIGNED, G.ERR_INVALID_ARG), (8, MISALIGNED, G.ERR_INVALID_ARG),
                           (12, -1, G.ERR_INVALID_ARG)]:
        a = list(good); a[idx] = val
        assert f(*a) == want, (idx, val)
    a = list(good); a[10] = 0                                  # empty batch
    assert f(*a) == G.OK
    a = list(good); a[12] = 0                                  # no token, no window kept
    assert f(*a) == G.OK


def test_binding_rejects_cpu_tensors_before_any_call():
    import torch
    x = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        G.fir_fwd(x, x, x, torch.zeros(2, 7))
    with pytest.raises(ValueError):
        G.chunk_fwd(x, x, x, torch.zeros(2, 16), torch.zeros(2, 16), 4)


def test_bench_refuses_more_than_one_gpu():
    # one GPU's throughput is the measured value; a request for several exits before any work
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
