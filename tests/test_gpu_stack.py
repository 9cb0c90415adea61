"""A stack of decoder blocks quantized in sequence on the GPU
(post_weight_quantization_accum_amd.sequential) against the oracle's block
chain (needs an MI355X).

Two blocks of hidden 256 / ffn 1024 on 16384 tokens, in the recipes of
workload 5 (fp16, 3-bit g128, natural order) and workload 3 (bf16, 4-bit
g128, act-order: the products gather activations through perm).  Every
layer is checked on the GPU's own activations (handed to the oracle as
data):
* given the GPU's Hessian of them, codes >= 99.99% identical, loss to 1e-6;
* from the oracle's float64 Hessian: >= 99.9% of codes identical, every
  difference <= 1, layer loss within 1e-3; every differing code is a
  rounding tie decided the other way or follows from one (tie replay), and
  after the replay scales are within 1e-5 relative and zero points equal;
* each block's output equals the float64 recomputation from the GPU's own
  intermediate activations and packed layers, to the dtype's rounding plus
  the product's float32 bound.
The oracle's own two-block chain reaches the same total loss within 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import sequential as S
from post_weight_quantization_accum_amd import synth

from _util import assert_from_x_parity, compare_codes, to_torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _product_bound(X64, q, bits, gs, perm):
    """(96 + 32 nb) u sum_k |x_a(k)| s (c + z + 2^(b+1)) (float32 product bound)."""
    d_in = X64.shape[1]
    codes = q["codes"]
    if perm is not None:
        codes = codes[:, perm]
        Xs = X64[:, perm]
    else:
        Xs = X64
    g = np.arange(d_in) // gs
    S_ = q["scales"].astype(np.float64)[g].T
    Z = q["zeros"].astype(np.float64)[g].T
    A = np.abs(Xs) @ (S_ * (codes.astype(np.float64) + Z + 2.0 ** (bits + 1))).T
    nb = -(-(-(-d_in // 32)) // 256)
    return (96 + 32 * nb) * 2.0 ** -24 * A


@pytest.mark.parametrize("dtype,bits,act", [("f16", 3, False), ("bf16", 4, True)])
def test_two_block_stack(dtype, bits, act):
    gs, h, ffn, n, nblocks = 128, 256, 1024, 16384, 2
    cfg = P.make_config(bits=bits, group_size=gs, act_order=act, block=128, damp=0.01)
    X0, _, _ = synth.gen_activations(n, h, "t4", dtype, seed=6001, outlier_count=1, outlier_scale=50.0)
    shapes = (("q", h, h), ("k", h, h), ("v", h, h), ("out", h, h), ("fc1", ffn, h), ("fc2", h, ffn))
    Wnp = [{name: synth.gen_weights(d_out, d_in, 0.02, dtype, 6100 + 10 * b + i)
            for i, (name, d_out, d_in) in enumerate(shapes)} for b in range(nblocks)]
    blocks = [S.Block(**{k: to_torch(v, dtype) for k, v in w.items()}) for w in Wnp]
    X0d = to_torch(X0, dtype)
    results, Xout = S.quantize_stack(blocks, X0d, cfg)
    torch.cuda.synchronize()

    q = dict(bits=bits, group_size=gs, act_order=act, block=128, damp=0.01)
    total_gpu = 0.0
    X_in = X0d
    for b, (res, inputs) in enumerate(results):
        W64 = {k: synth.to_f64(v, dtype) for k, v in Wnp[b].items()}
        got = {name: {k: v.cpu().numpy() for k, v in res[name].items()} for name in S.LAYERS}
        for name in S.LAYERS:
            Xd = inputs[name]
            Xl = _to_f64(Xd)
            Hg = torch.zeros((Xl.shape[1], Xl.shape[1]), dtype=torch.float64, device=DEV)
            P.hessian_accumulate(Hg, Xd)
            Hg = Hg.cpu().numpy()
            Hg = np.triu(Hg) + np.triu(Hg, 1).T
            ref_h = O.gptq_quantize(W64[name], Hg, **q)
            same_h, mx_h = compare_codes(got[name]["codes"], ref_h["codes"])
            lg_h = O.layer_loss(W64[name], got[name]["w_hat"].astype(np.float64), Hg).sum()
            assert same_h >= 0.9999 and mx_h <= 1, (b, name)
            assert abs(lg_h - ref_h["loss"].sum()) <= 1e-6 * ref_h["loss"].sum(), (b, name)
            rp = assert_from_x_parity(O, W64[name], O.hessian(Xl), got[name], bits, gs, act,
                                      name=f"block {b} {name} from X")
            assert rp["same_raw"] >= 0.999 and rp["maxdiff_raw"] <= 1, (b, name)
            assert abs(rp["loss_gpu"] - rp["loss_oracle"]) <= 1e-3 * rp["loss_oracle"], (b, name)
            total_gpu += rp["loss_gpu"]
        # the block's output from the GPU's own intermediates, in float64
        X64 = _to_f64(X_in)
        h1 = X64.copy()
        r64 = _to_f64(inputs["fc2"])
        A64 = _to_f64(inputs["out"])
        tol = np.zeros((n, h))
        for name, Xa in (("out", A64), ("fc2", r64)):
            perm = got[name]["perm"] if act else None
            words = got[name]["packed"].view(np.uint32)
            kw = dict(perm=perm, group_size=gs) if act else dict(group_size=gs)
            h1 = h1 + O.dequant_matmul(Xa, words, bits, Xa.shape[1], got[name]["scales"], got[name]["zeros"], **kw)
            tol += _product_bound(Xa, got[name], bits, gs, perm)
        got_out = _to_f64(Xout if b == nblocks - 1 else results[b + 1][1]["q"])
        err = np.abs(got_out - h1)
        assert np.all(err <= 2 * EPS[dtype] * np.abs(h1) + 2 * tol + 1e-6 * EPS[dtype]), b
        X_in = Xout if b == nblocks - 1 else results[b + 1][1]["q"]

    # the oracle's own chain
    Xo = synth.to_f64(X0, dtype)
    total_o = 0.0
    for b in range(nblocks):
        W64 = {k: synth.to_f64(v, dtype) for k, v in Wnp[b].items()}
        res_o, _, Xo = O.quantize_block_chain(W64, Xo, dtype, **q)
        total_o += sum(res_o[name]["loss"].sum() for name in S.LAYERS)
    print(f"stack loss gpu {total_gpu:.6g} oracle chain {total_o:.6g}", flush=True)
    assert abs(total_gpu - total_o) <= 1e-3 * total_o
