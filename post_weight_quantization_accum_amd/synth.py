"""Seeded synthetic layer inputs (weights W and calibration activations X).

This module holds no step of the quantization method: it only draws numbers.
The HIP path and the fp64 oracle both consume the arrays it returns, byte for
byte, so a parity comparison always starts from identical inputs.

Recipe (numpy PCG64, all draws in float32, then cast with round-to-nearest-
even to the layer's dtype):

* W ~ N(0, sigma_w^2), d_out x d_in.
* X is drawn in chunks of ``CHUNK`` tokens; chunk i uses the i-th child of
  ``SeedSequence(seed_x)``, so any chunk can be regenerated alone and the
  chunks can be drawn in parallel.
* "t4": i.i.d. Student-t with 4 degrees of freedom per element, drawn as
  Z / sqrt((E1 + E2) / 2) with Z standard normal and E1, E2 standard
  exponential (chi-square with 4 degrees of freedom is 2 * (E1 + E2)).
* "gauss_mix": X = Z A with Z ~ N(0, 1) and A ~ N(0, 1/d_in) (d_in x d_in),
  a Gaussian with a random correlation.
* Outlier channels: k = round(frac * d_in) columns chosen without replacement
  by ``Generator(PCG64(seed_o)).choice``; those columns are multiplied by
  ``outlier_scale`` after drawing.
* fp16 values are clamped to +-65504 before the cast (the number of clamps
  is reported); bf16 is kept as its uint16 bit pattern.

Seeds: seed_w = 1000*config + 10*layer, seed_x = seed_w + 1,
seed_o = seed_w + 2.

Packed layers (inputs of the product with quantized weights), from
``Generator(PCG64(seed))`` in this order: codes uniform on [0, 2^bits)
(uint8, d_out x d_in); scales log-uniform on [1e-3, 5e-2] (float32,
[n_groups][d_out]); zero points uniform integers on [0, 2^bits) (stored as
float32); a uniformly random permutation of the d_in columns (int32, the
column order of an act-order layer).  Activations: ``gen_activations`` with
seed + 1 (Student-t, 1% outlier channels x 20 by default).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

CHUNK = 8192

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Layer:
    """Host arrays of one synthetic layer.

    ``W`` and ``X`` hold the stored representation of ``dtype``: float32,
    float16, or uint16 bf16 bit patterns.  ``as_f64`` widens them exactly.
    """
    W: np.ndarray
    X: np.ndarray
    dtype: str
    outliers: np.ndarray
    clamps: int = 0

    def W_f64(self) -> np.ndarray:
        return to_f64(self.W, self.dtype)

    def X_f64(self) -> np.ndarray:
        return to_f64(self.X, self.dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def _cast(a32: np.ndarray, dtype: str):
    if dtype == "f32":
        return a32, 0
    if dtype == "f16":
        lim = np.float32(65504.0)
        n = int(np.count_nonzero(np.abs(a32) > lim))
        if n:
            a32 = np.clip(a32, -lim, lim)
        return a32.astype(np.float16), n
    if dtype == "bf16":
        return f32_to_bf16_bits(a32), 0
    raise ValueError(f"unknown dtype {dtype}")


def _stored_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def gen_weights(d_out: int, d_in: int, sigma: float, dtype: str, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(sigma)
    return _cast(w, dtype)[0]


def _t4_chunk(rng: np.random.Generator, n: int, d_in: int) -> np.ndarray:
    z = rng.standard_normal((n, d_in), dtype=np.float32)
    e = rng.standard_exponential((n, d_in), dtype=np.float32)
    e += rng.standard_exponential((n, d_in), dtype=np.float32)
    e *= np.float32(0.5)
    np.sqrt(e, out=e)
    z /= e
    return z


def gen_activations(n_tok: int, d_in: int, dist: str, dtype: str, seed: int,
                    outlier_frac: float = 0.0, outlier_count: int | None = None,
                    outlier_scale: float = 1.0, seed_outliers: int | None = None,
                    threads: int | None = None):
    """Return (X stored as ``dtype``, outlier column indices, fp16 clamp count)."""
    if outlier_count is None:
        outlier_count = int(round(outlier_frac * d_in))
    ro = np.random.Generator(np.random.PCG64(seed_outliers if seed_outliers is not None else seed + 1))
    outl = np.sort(ro.choice(d_in, outlier_count, replace=False)) if outlier_count else np.zeros(0, np.int64)

    out = np.empty((n_tok, d_in), dtype=_stored_dtype(dtype))
    n_chunks = -(-n_tok // CHUNK)
    children = np.random.SeedSequence(seed).spawn(n_chunks + 1)
    A = None
    if dist == "gauss_mix":
        ra = np.random.Generator(np.random.PCG64(children[-1]))
        A = ra.standard_normal((d_in, d_in), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_in))
    elif dist != "t4":
        raise ValueError(f"unknown distribution {dist}")
    oscale = np.float32(outlier_scale)
    clamps = [0] * n_chunks

    def work(i):
        t0, t1 = i * CHUNK, min(n_tok, (i + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(children[i]))
        if dist == "t4":
            x = _t4_chunk(rng, t1 - t0, d_in)
        else:
            x = rng.standard_normal((t1 - t0, d_in), dtype=np.float32) @ A
        if len(outl):
            x[:, outl] *= oscale
        out[t0:t1], clamps[i] = _cast(x, dtype)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    if n_chunks == 1 or nthreads == 1:
        for i in range(n_chunks):
            work(i)
    else:
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(n_chunks)))
    return out, outl, sum(clamps)


def make_layer(d_out: int, d_in: int, n_tok: int, *, dtype: str, sigma_w: float,
               dist: str, outlier_frac: float = 0.0, outlier_count: int | None = None,
               outlier_scale: float = 1.0, config: int = 0, layer: int = 0,
               x_layer: int | None = None, threads: int | None = None) -> Layer:
    """One layer's (W, X).  Layers sharing an input pass the same ``x_layer``."""
    seed_w = 1000 * config + 10 * layer
    xl = layer if x_layer is None else x_layer
    seed_x = 1000 * config + 10 * xl + 1
    W = gen_weights(d_out, d_in, sigma_w, dtype, seed_w)
    X, outl, clamps = gen_activations(n_tok, d_in, dist, dtype, seed_x,
                                      outlier_frac=outlier_frac, outlier_count=outlier_count,
                                      outlier_scale=outlier_scale, seed_outliers=seed_x + 1,
                                      threads=threads)
    return Layer(W=W, X=X, dtype=dtype, outliers=outl, clamps=clamps)


@dataclasses.dataclass
class PackedLayer:
    """Host arrays of a quantized layer: integer codes (uint8 d_out x d_in),
    scales and zeros (float32 [n_groups][d_out]), a column permutation
    (int32 d_in) and activations ``X`` in the stored form of ``dtype``."""
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    perm: np.ndarray
    X: np.ndarray
    dtype: str

    def X_f64(self) -> np.ndarray:
        return to_f64(self.X, self.dtype)


def make_packed_layer(d_out: int, d_in: int, n_tok: int, *, bits: int, group_size: int, dtype: str,
                      dist: str = "t4", outlier_frac: float = 0.01, outlier_scale: float = 20.0,
                      seed: int = 0) -> PackedLayer:
    rng = np.random.Generator(np.random.PCG64(seed))
    n_groups = -(-d_in // group_size) if 0 < group_size < d_in else 1
    codes = rng.integers(0, 1 << bits, size=(d_out, d_in), dtype=np.uint8)
    scales = np.exp(rng.uniform(np.log(1e-3), np.log(5e-2), size=(n_groups, d_out))).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, size=(n_groups, d_out)).astype(np.float32)
    perm = rng.permutation(d_in).astype(np.int32)
    X, _, _ = gen_activations(n_tok, d_in, dist, dtype, seed + 1, outlier_frac=outlier_frac,
                              outlier_scale=outlier_scale)
    return PackedLayer(codes=codes, scales=scales, zeros=zeros, perm=perm, X=X, dtype=dtype)
