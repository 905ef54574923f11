"""The allocation-free entry point convtranspose_nd_noalloc, through the C ABI: its output
must equal, bit for bit, that of convtranspose_nd_with_kernel (the entry point it is a
variant of, given a caller workspace) on the same inputs, on two calls in a row with the
second one smaller (the shared device workspace keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import transposed_convolution_amd as T
    T.load_library()
    return T


def _inputs(xs, ws, cl, seed):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.normal(size=xs).astype(np.float16)).to(dev)
    if cl:
        x = x.to(memory_format=torch.channels_last if len(xs) == 4 else torch.channels_last_3d)
    w = torch.from_numpy((rng.normal(size=ws) * 0.05).astype(np.float16)).to(dev)
    b = torch.from_numpy(rng.normal(size=ws[1]).astype(np.float16)).to(dev)
    return x, w, b


def _with_kernel(T, x, w, b, y, cl, attrs):
    """convtranspose_nd_with_kernel with a workspace of the size it reports."""
    lib = T.load_library()
    nsp, xp, xs, wp, ws, bp, yp, at = T._call_args(x, w, b, y, attrs)
    nbytes = ctypes.c_size_t(0)
    assert lib.convtranspose_workspace_size(0, 1, nsp, int(cl), xp, xs, ws, *at, ctypes.byref(nbytes)) == 0
    scratch = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=x.device)
    st = lib.convtranspose_nd_with_kernel(0, 1, nsp, int(cl), xp, xs, wp, ws, bp, yp, T._i64(tuple(y.shape)), *at,
                                          ctypes.c_void_p(scratch.data_ptr()), nbytes.value,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, T.convtranspose_last_error()
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
def test_noalloc_matches_workspace_entry_point(T, cl):
    cases = [
        # a C4-like decoder layer (packed weights 1 MiB), then a smaller 3-D one
        ((2, 256, 16, 16), (256, 128, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
        ((1, 32, 5, 6, 8), (32, 48, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1])),
    ]
    for i, (xs, ws, attrs) in enumerate(cases):
        print(f"[case] noalloc call {i} x{xs} w{ws} cl={cl}", flush=True)
        x, w, b = _inputs(xs, ws, cl, seed=40 + i)
        assert T.convtranspose_select_kernel(x, w, b, channels_last=cl, **attrs) == "igemm"
        ys, _ = T.convtranspose_output_shape(xs, ws, **attrs)
        mk = (lambda: T.channels_last_empty(ys, torch.float16, x.device)) if cl else \
            (lambda: torch.empty(ys, dtype=torch.float16, device=x.device))
        want = _with_kernel(T, x, w, b, mk().fill_(7.0), cl, attrs)
        got = mk().fill_(-3.0)
        T.convtranspose_nd_noalloc(x, w, b, out=got, channels_last=cl, **attrs)
        torch.cuda.synchronize()
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), f"call {i}: {(got != want).sum().item()} elements differ"


def test_noalloc_without_workspace_families(T):
    """Families that need no workspace (float32 MFMA, grouped, gather) run unchanged."""
    dev = torch.device("cuda:0")
    for wl in (W.C1, W.C2, W.C3.with_(x_shape=(2, 32, 14, 16), w_shape=(32, 1, 4, 4), attrs=dict(W.C3.attrs, group=32))):
        x, w, b = W.make_inputs(wl)
        tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
        tb = None if b is None else torch.from_numpy(b).to(dev)
        ys, _ = T.convtranspose_output_shape(x.shape, w.shape, **wl.attrs)
        want = T.convtranspose_nd(tx, tw, tb, **wl.attrs)
        got = torch.empty(ys, dtype=tx.dtype, device=dev)
        T.convtranspose_nd_noalloc(tx, tw, tb, out=got, **wl.attrs)
        torch.cuda.synchronize()
        assert torch.equal(got, want), wl.name
