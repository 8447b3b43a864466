"""hyena_fftconv_fwd_noalloc, the single pass through the library's own
device scratch, against hyena_fftconv_fwd with a caller workspace, both
called through the C ABI.  Each test makes two calls in a row, the second
with a smaller input, so the second runs on what the first left in the
scratch; rows go through it in several batches (the scratch holds 512 rows
of L <= 32768 and 32 rows of L <= 65536), and both results must be the same
bits.  Free device memory must not drop across a call."""
import ctypes

import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import workloads as W
from tests.gpu_util import DevWorkload, gate, log, oracle_modal, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    # the first call on a device loads the code object that holds the
    # scratch (and looks up its address); later calls allocate nothing
    d = DevWorkload(W.make("7b_layer_set", D=1, L=5000))
    _noalloc_call(d, torch.empty_like(d.x1))
    torch.cuda.synchronize()
    yield


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _workspace_call(d, y):
    B, D, L = d.x1.shape
    io = G.BF16 if d.x1.dtype == torch.bfloat16 else G.F32
    need = G.lib().hyena_fftconv_workspace_size(B, D, L, d.lam.shape[1], io)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=d.x1.device)
    st = G.lib().hyena_fftconv_fwd(_p(d.x1), _p(d.x2), _p(d.v), _p(d.lam), _p(d.res),
                                   d.lam.shape[1], _p(d.skip), _p(y), B, D, L, io, _p(ws),
                                   ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == G.OK, G.status_string(st)


def _noalloc_call(d, y):
    B, D, L = d.x1.shape
    io = G.BF16 if d.x1.dtype == torch.bfloat16 else G.F32
    st = G.lib().hyena_fftconv_fwd_noalloc(
        _p(d.x1), _p(d.x2), _p(d.v), _p(d.lam), _p(d.res), d.lam.shape[1], _p(d.skip), _p(y),
        B, D, L, io, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == G.OK, G.status_string(st)


def _run(name, B, D, L):
    w = W.make(name, B=B, D=D, L=L)
    d = DevWorkload(w)
    y_ws = torch.full_like(d.x1, float("nan"))
    _workspace_call(d, y_ws)
    y_na = torch.full_like(d.x1, float("nan"))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _noalloc_call(d, y_na)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    log(f"noalloc {name} B={B} D={D} L={L}: free device memory {free0} -> {free1}")
    assert free1 >= free0 - (1 << 20), (free0, free1)
    assert torch.isfinite(y_na.float()).all()
    bits = torch.equal(y_na.view(torch.int16) if y_na.dtype == torch.bfloat16 else y_na.view(torch.int32),
                       y_ws.view(torch.int16) if y_ws.dtype == torch.bfloat16 else y_ws.view(torch.int32))
    assert bits, "noalloc and workspace results differ"
    rows = sample_rows(w.D, k=4)
    ref, _ = oracle_modal(w, rows)
    gate(y_na, ref, w.io, rows, label=f"noalloc {name} L={L}")


def test_noalloc_two_launch_rows_then_smaller():
    # 600 rows of S = 16384 (128 KiB of scratch each): batches of 512 + 88;
    # then 3 rows of S = 4096 in one batch
    _run("7b_layer_set", 2, 300, 20000)
    _run("tiny", 1, 3, 5000)


def test_noalloc_four_step_rows_then_smaller():
    # 70 rows of S = 65536 (2 MiB each): batches of 32 + 32 + 6; then 2 rows
    # of S = 32768 in one batch
    _run("7b_layer_set", 1, 70, 70000)
    _run("7b_layer_set", 1, 2, 40000)
