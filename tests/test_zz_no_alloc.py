"""The allocation-free Hessian entry point against gptq_hessian_accumulate
(needs an MI355X).

Calls go through the C ABI (ctypes binding).  Two calls in a row on the same
GPU scratch array, the second with a smaller input, each compared with the
regular entry point on the same inputs:
* a narrow layer (d = 1024, 40000 bf16 tokens: its regular plan wants more
  partial tiles than the array holds, so the windows differ: float64
  rounding only, element-wise within 1e-12 of sum_t |x_ti x_tj|, and the
  diagonal within 1e-13 relative);
* then a smaller one (d = 300, 3000 fp16 tokens, rows not 16-byte aligned:
  copied through the array; the regular plan fits it: bit-identical).
A wide aligned layer (no scratch at all) and a misaligned input too wide for
the array's copy (GPTQ_ERR_WORKSPACE) complete the cases.
"""
import ctypes

import numpy as np
import pytest
import torch

import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import _lib, synth

from _util import to_torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(X):
    d = X.shape[1]
    Hr = torch.zeros((d, d), dtype=torch.float64, device=DEV)
    P.hessian_accumulate(Hr, X)
    Hn = torch.zeros((d, d), dtype=torch.float64, device=DEV)
    P.hessian_accumulate_noalloc(Hn, X)
    torch.cuda.synchronize()
    return Hr.cpu().numpy(), Hn.cpu().numpy()


def test_noalloc_matches_regular_entry_point_twice():
    L = synth.make_layer(4, 1024, 40000, dtype="bf16", sigma_w=0.02, dist="t4", outlier_frac=0.01,
                         outlier_scale=30.0, config=90, layer=501)
    X = to_torch(L.X, "bf16")
    Hr, Hn = _both(X)
    iu = np.triu_indices(1024)
    x = np.abs(L.X_f64())
    A = 2.0 * (x.T @ x)
    assert np.all(np.abs(Hn - Hr)[iu] <= 1e-12 * A[iu])
    np.testing.assert_allclose(np.diag(Hn), np.diag(Hr), rtol=1e-13)
    # second call on the same array, smaller and misaligned (odd row stride)
    L2 = synth.make_layer(4, 300, 3000, dtype="f16", sigma_w=0.02, dist="t4", outlier_frac=0.01,
                          outlier_scale=30.0, config=90, layer=502)
    big = torch.zeros((3000, 301), dtype=torch.float16, device=DEV)
    big[:, :300] = to_torch(L2.X, "f16")
    X2 = big[:, :300]
    assert X2.stride(0) == 301
    Hr2, Hn2 = _both(X2)
    iu2 = np.triu_indices(300)
    assert np.array_equal(Hn2[iu2], Hr2[iu2])


def test_noalloc_wide_layer_and_limit():
    L = synth.make_layer(4, 4096, 3000, dtype="bf16", sigma_w=0.02, dist="t4", outlier_frac=0.01,
                         outlier_scale=30.0, config=90, layer=503)
    Hr, Hn = _both(to_torch(L.X, "bf16"))
    iu = np.triu_indices(4096)
    assert np.array_equal(Hn[iu], Hr[iu])
    # a misaligned input too wide for a 256-token copy in a quarter of the array
    lib = P.load()
    d = 40001
    H = torch.zeros(1, dtype=torch.float64, device=DEV)   # never touched: rejected before any launch
    X = torch.zeros(8, dtype=torch.float16, device=DEV)
    st = lib.gptq_hessian_accumulate_noalloc(ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(X.data_ptr()),
                                             _lib.F16, 256, d, d, ctypes.c_void_p(0))
    assert st == _lib.ERR_WORKSPACE
