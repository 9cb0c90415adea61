"""Quantize a stack of decoder blocks in sequence (true-sequential).

"GPTQ量化算法深度解析" §3.1: layers are quantized one after another, each
from calibration activations; "GPTQ论文复现指南" §3.2: --true-sequential
quantizes inside a transformer block in order, so that every layer sees
the outputs of the layers before it already quantized.

The pages give no attention or normalisation details, so a block is the
plainest chain those passages support (identity attention, residuals, no
layer norm, ReLU as in OPT):

    q, k, v  <- H(X)                      (one Hessian, one factorisation)
    A  = X  W_v^T                         out <- H(A)
    h1 = X  + A W_out^T                   fc1 <- H(h1)
    r  = relu(h1 W_fc1^T)                 fc2 <- H(r)
    X' = h1 + r W_fc2^T                   (the next block's input)

Every product uses the already-quantized weights, computed by
gptq_dequant_matmul from the packed words (with act-order: packed in
quantization order, activations gathered into that order first).  Products come out
in float32; residual sums are taken in float32 and every activation that
feeds a Hessian or a product is rounded to the stack's dtype.  All steps of
the method run in the library; this module only sequences the calls and
does the elementwise glue (residual, ReLU, dtype rounding).
"""
from __future__ import annotations

import dataclasses

from . import (dequant_matmul, factored_supported, gather_columns, hessian_accumulate, load, pack, pack_permuted,
               prepare_hinv, prepare_hinv_factored, quantize_layer, quantize_layer_factored)

LAYERS = ("q", "k", "v", "out", "fc1", "fc2")


@dataclasses.dataclass
class Block:
    """Weights of one block (device tensors, d_out x d_in, fp16/bf16/fp32):
    q, k, v, out: hidden x hidden; fc1: ffn x hidden; fc2: hidden x ffn."""
    q: object
    k: object
    v: object
    out: object
    fc1: object
    fc2: object


def _torch():
    import torch
    return torch


def _hessian(X):
    torch = _torch()
    d = X.shape[1]
    H = torch.zeros((d, d), dtype=torch.float64, device=X.device)
    hessian_accumulate(H, X)
    return H


def _quantize_shared(Ws: dict, X, cfg, stats: dict | None, want_w_hat: bool = True):
    """Quantize the layers of Ws (all reading X) from one Hessian of X."""
    torch = _torch()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if stats is not None else None
    if ev:
        ev[0].record()
    H = _hessian(X)
    if ev:
        ev[1].record()
    d_in = H.shape[0]
    factored = all(factored_supported(W.shape[0], d_in, cfg) for W in Ws.values())
    perm = (prepare_hinv_factored if factored else prepare_hinv)(H, cfg)
    res = {}
    for name, W in Ws.items():
        out = (quantize_layer_factored if factored else quantize_layer)(W, H, perm, cfg, want_w_hat=want_w_hat)
        out["perm"] = perm
        if cfg.act_order:
            out["packed"] = pack_permuted(out["codes"], cfg.bits, perm)
        else:
            out["packed"] = pack(out["codes"], cfg.bits)
        res[name] = out
    if ev:
        ev[2].record()
        torch.cuda.synchronize()
        stats["hessian_ms"] += ev[0].elapsed_time(ev[1])
        stats["solver_ms"] += ev[1].elapsed_time(ev[2])
    return res


def _product(X, q, cfg, stats: dict | None):
    """X W_hat^T (float32) from the packed layer."""
    torch = _torch()
    if stats is not None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
    if cfg.act_order and X.shape[0] >= 128:
        # many tokens: gather once into quantization order, then the matrix-core route
        Y = dequant_matmul(gather_columns(X, q["perm"]), q["packed"], cfg.bits, q["scales"], q["zeros"],
                           group_size=cfg.group_size)
    elif cfg.act_order:
        Y = dequant_matmul(X, q["packed"], cfg.bits, q["scales"], q["zeros"], perm=q["perm"],
                           group_size=cfg.group_size)
    else:
        Y = dequant_matmul(X, q["packed"], cfg.bits, q["scales"], q["zeros"], group_size=cfg.group_size)
    if stats is not None:
        e1.record()
        torch.cuda.synchronize()
        stats["product_ms"] += e0.elapsed_time(e1)
    return Y


def quantize_block(block: Block, X, cfg, stats: dict | None = None, want_w_hat: bool = True):
    """Quantize one block from its input activations X (tokens x hidden,
    device, fp16/bf16).  Returns (per-layer outputs of quantize_layer plus
    perm and packed, the activations each layer was quantized on, the next
    block's input X').  want_w_hat=False skips the float32 reconstructions
    (4 bytes per weight)."""
    dt = X.dtype
    res, inputs = {}, {}
    res.update(_quantize_shared({"q": block.q, "k": block.k, "v": block.v}, X, cfg, stats, want_w_hat))
    for n in ("q", "k", "v"):
        inputs[n] = X
    A = _product(X, res["v"], cfg, stats).to(dt)
    inputs["out"] = A
    res.update(_quantize_shared({"out": block.out}, A, cfg, stats, want_w_hat))
    h1f = X.float() + _product(A, res["out"], cfg, stats)
    h1 = h1f.to(dt)
    inputs["fc1"] = h1
    res.update(_quantize_shared({"fc1": block.fc1}, h1, cfg, stats, want_w_hat))
    r = _torch().relu(_product(h1, res["fc1"], cfg, stats)).to(dt)
    inputs["fc2"] = r
    res.update(_quantize_shared({"fc2": block.fc2}, r, cfg, stats, want_w_hat))
    X_next = (h1f + _product(r, res["fc2"], cfg, stats)).to(dt)
    return res, inputs, X_next


def quantize_stack(blocks, X0, cfg, stats: dict | None = None, want_w_hat: bool = True):
    """Quantize the blocks in order; block b+1 is calibrated on the output of
    the already-quantized block b.  Returns a list of (outputs, inputs) per
    block and the stack's output activations."""
    load()
    out = []
    X = X0
    for b in blocks:
        res, inputs, X = quantize_block(b, X, cfg, stats, want_w_hat)
        out.append((res, inputs))
    return out, X


def new_stats() -> dict:
    return {"hessian_ms": 0.0, "solver_ms": 0.0, "product_ms": 0.0}


__all__ = ["Block", "LAYERS", "quantize_block", "quantize_stack", "new_stats"]
