"""Product with the packed layer: HIP path vs the fp64 oracle (needs an MI355X).

Calls go through the C ABI (ctypes binding).  Inputs come from
``synth.make_packed_layer``; the oracle packs the codes itself and computes
Y = X W_hat^T in float64 from its own unpacking.

Tolerance (float32 arithmetic, u = 2^-24).  With
A[t, r] = sum_k |x_t,a(k)| * s[g(k), r] * (c_r(k) + z[g(k), r] + 2^(b+1)),
every intermediate the kernel forms is bounded by A, and the number of
roundings along any path to one output is at most
  block route: 16 chained v_dot2 (<= 2 roundings each) for sum x (2^b + c),
  the same for sum x, one FMA removing the offset, one FMA per 32-column
  block into the thread's sum (<= nb blocks per thread), 6 exchange levels
  in the wave and 4 additions across waves;
  column route: one rounding forming the weight, 32 * nb chained FMAs, the
  same reduction.
So |Y - Y_exact| <= (96 + 32 nb) u A elementwise, nb = ceil(ceil(d_in/32) / 256).
Integer-valued inputs (integer activations, power-of-two scales) make every
partial sum exact: there the comparison is bit-exact, which pins the
indexing (pairs, permutation, groups, tails) independently of the bound.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import synth

from _util import to_torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
U32 = 2.0 ** -24


def _g_idx(perm, group_size, d_in):
    """Original-order group index of each column when the quantization order is perm."""
    gs = group_size if 0 < group_size < d_in else d_in
    g = np.empty(d_in, dtype=np.int32)
    g[perm] = np.arange(d_in) // gs
    return g


def _stream_order(L, mode, group_size):
    """(codes in stream order, group of each stream position, activation column of each position)."""
    d_in = L.codes.shape[1]
    gs = group_size if 0 < group_size < d_in else d_in
    if mode == "perm":
        return L.codes[:, L.perm], np.arange(d_in) // gs, L.perm.astype(np.int64)
    if mode == "g_idx":
        return L.codes, _g_idx(L.perm, group_size, d_in).astype(np.int64), np.arange(d_in)
    return L.codes, np.arange(d_in) // gs, np.arange(d_in)


MM_MIN_TOKENS = 2     # natural order, block route: the matrix-core routes from this many tokens


def _mfma_route(L, mode, group_size, dtype, bits):
    d_in = L.codes.shape[1]
    block = dtype != "f32" and not (dtype == "bf16" and bits == 8) and mode != "g_idx" and \
        (group_size <= 0 or group_size >= d_in or group_size % 32 == 0)
    return block and mode == "natural" and L.X.shape[0] >= MM_MIN_TOKENS


def _bound(L, X64, mode, group_size, bits, dtype=None):
    c, g, a = _stream_order(L, mode, group_size)
    S = L.scales.astype(np.float64)[g].T            # d_out x d_in, stream order
    Z = L.zeros.astype(np.float64)[g].T
    mag = S * (c.astype(np.float64) + Z + 2.0 ** (bits + 1))
    A = np.abs(X64[:, a]) @ mag.T
    d_in = L.codes.shape[1]
    dtype = L.dtype if dtype is None else dtype
    if _mfma_route(L, mode, group_size, dtype, bits):
        # matrix cores: a group's products summed in float32 (<= glen
        # roundings), its sum of x by v_dot2 (<= glen), two FMAs, one addition
        # per group; under 128 tokens a group may be cut in two parts (one
        # more correction) and eight partial tiles are added at the end
        glen = group_size if 0 < group_size < d_in else d_in
        ng = -(-d_in // glen)
        return (2 * glen + ng + 16) * U32 * A
    nb = -(-(-(-d_in // 32)) // 256)
    return (96 + 32 * nb) * U32 * A


def _run(L, mode, bits, group_size, x_view=None):
    """GPU product through the C ABI; returns (Y_gpu, oracle Y, X as float64)."""
    d_out, d_in = L.codes.shape
    codes = torch.from_numpy(L.codes).to(DEV)
    perm = torch.from_numpy(L.perm).to(DEV)
    if mode == "perm":
        packed = P.pack_permuted(codes, bits, perm)
        words_ref = O.pack_permuted(L.codes, bits, L.perm)
    else:
        packed = P.pack(codes, bits)
        words_ref = O.pack(L.codes, bits)
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), words_ref)
    X = to_torch(L.X, L.dtype) if x_view is None else x_view
    scales = torch.from_numpy(L.scales).to(DEV)
    zeros = torch.from_numpy(L.zeros).to(DEV)
    kw = {}
    okw = {}
    if mode == "perm":
        kw = dict(perm=perm, group_size=group_size)
        okw = dict(perm=L.perm, group_size=group_size)
    elif mode == "g_idx":
        gi = _g_idx(L.perm, group_size, d_in)
        kw = dict(g_idx=torch.from_numpy(gi).to(DEV))
        okw = dict(g_idx=gi)
    else:
        kw = dict(group_size=group_size)
        okw = dict(group_size=group_size)
    Y = P.dequant_matmul(X, packed, bits, scales, zeros, **kw)
    torch.cuda.synchronize()
    X64 = L.X_f64()
    ref = O.dequant_matmul(X64, words_ref, bits, d_in, L.scales, L.zeros, **okw)
    return Y.cpu().numpy().astype(np.float64), ref, X64


CASES = [
    # bits, dtype, mode, group_size, n_tok, d_out, d_in
    (4, "bf16", "perm", 128, 1, 72, 1000),      # block route, gather, ragged last block
    (4, "bf16", "natural", 128, 5, 37, 4100),   # few-token matrix cores, ragged rows and last block
    (3, "f16", "natural", 64, 1, 40, 777),      # 3-bit pairs, straddling codes
    (2, "bf16", "perm", 32, 3, 16, 2048),
    (8, "f16", "natural", -1, 2, 24, 513),      # 8-bit in f16 pairs, one group
    (3, "bf16", "perm", 96, 4, 48, 2000),
    (4, "bf16", "natural", 128, 9, 64, 8192),   # few-token matrix cores, aligned vector loads
    (4, "bf16", "perm", 128, 1, 64, 16384),     # two blocks per thread
    (8, "bf16", "natural", 128, 1, 16, 640),    # column route (8-bit codes, bf16)
    (4, "bf16", "g_idx", 128, 3, 33, 1500),     # column route, act-order original order
    (3, "f32", "natural", 128, 2, 20, 900),     # column route, fp32 activations
    (4, "f16", "natural", 25, 1, 19, 500),      # column route, group size not a multiple of 32
    (2, "f32", "perm", 16, 4, 8, 300),          # column route with the gather
    (4, "f16", "g_idx", 32, 2, 9, 33),          # tiny: one full block plus one column
    # a few tokens in natural order: 32 rows x 32 tokens per workgroup, the
    # row's blocks split over eight waves (groups cut between waves)
    (4, "bf16", "natural", 128, 16, 4096, 11008 // 4),
    (3, "f16", "natural", 64, 33, 70, 1000),        # two token tiles, ragged
    (2, "bf16", "natural", -1, 31, 45, 700),        # one group per row, cut eight ways
    (8, "f16", "natural", 32, 7, 33, 129),          # fewer blocks than waves
    (4, "f16", "natural", 96, 127, 100, 1200),
    (4, "bf16", "natural", 128, 2, 300, 4096 + 8),
    (4, "bf16", "natural", 128, 50, 40, 1001),     # four 16-token tiles per workgroup, element-wise loads
    (3, "bf16", "natural", 32, 20, 18, 515),       # two tiles, ragged
    # many tokens in natural order: the matrix-core route (128x128 tiles)
    (4, "bf16", "natural", 128, 300, 200, 1000),    # ragged token, row and column tiles
    (3, "f16", "natural", 64, 129, 130, 777),
    (2, "bf16", "natural", -1, 128, 64, 96),
    (8, "f16", "natural", 128, 256, 72, 640),
    (4, "f16", "natural", 32, 1000, 384, 2048),
    (3, "bf16", "natural", 96, 170, 257, 2000),
]


@pytest.mark.parametrize("bits,dtype,mode,gs,n_tok,d_out,d_in", CASES)
def test_dequant_matmul_matches_oracle(bits, dtype, mode, gs, n_tok, d_out, d_in):
    print(f"dequant b{bits} {dtype} {mode} g{gs} n{n_tok} {d_out}x{d_in}", flush=True)
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype=dtype,
                                seed=bits * 1000 + d_in)
    Y, ref, X64 = _run(L, mode, bits, gs)
    tol = _bound(L, X64, mode, gs, bits, dtype)
    err = np.abs(Y - ref)
    assert np.all(np.isfinite(Y))
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"


def test_dequant_matmul_strided_unaligned_activations():
    # row stride not a multiple of 8 elements: the element-wise activation loads
    bits, gs, n_tok, d_out, d_in = 4, 128, 3, 40, 1024
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype="bf16", seed=77)
    big = torch.zeros((n_tok, d_in + 3), dtype=torch.bfloat16, device=DEV)
    big[:, 1:1 + d_in] = to_torch(L.X, "bf16")
    view = big[:, 1:1 + d_in]
    assert view.stride(0) == d_in + 3
    for mode in ("natural", "g_idx"):
        Y, ref, X64 = _run(L, mode, bits, gs, x_view=view)
        assert np.all(np.abs(Y - ref) <= _bound(L, X64, mode, gs, bits))


@pytest.mark.parametrize("bits,dtype,mode,gs,d_in", [
    (4, "bf16", "perm", 128, 1111), (4, "bf16", "natural", 64, 1280), (3, "f16", "perm", 32, 1111),
    (2, "bf16", "natural", -1, 1280), (8, "f16", "natural", 128, 1280), (3, "f16", "natural", 64, 1280),
    (4, "bf16", "natural", 128, 1111), (8, "f16", "perm", 128, 1111),
    (4, "bf16", "g_idx", 128, 1111), (8, "bf16", "natural", 128, 1280), (3, "f32", "perm", 40, 1111),
])
@pytest.mark.parametrize("n_tok", [5, 200])
def test_dequant_matmul_exact_on_integer_data(bits, dtype, mode, gs, d_in, n_tok):
    # integer activations in [-8, 8] and scales 2^-3 or 2^-5: every partial
    # sum is a multiple of 2^-5 below 2^19, exact in float32 and float64.
    # d_in = 1280 keeps the activation rows 16-byte aligned (vector loads and
    # byte permutes), 1111 takes the element-wise loads and a ragged block;
    # 200 tokens take the matrix-core route in natural order.
    d_out = 29
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype=dtype, seed=500 + bits)
    rng = np.random.default_rng(900 + bits)
    xi = rng.integers(-8, 9, size=(n_tok, d_in)).astype(np.float32)
    L.X = synth._cast(xi, dtype)[0]
    L.scales = np.where(rng.random(L.scales.shape) < 0.5, 2.0 ** -3, 2.0 ** -5).astype(np.float32)
    Y, ref, _ = _run(L, mode, bits, gs)
    assert np.array_equal(Y, ref)


@pytest.mark.parametrize("n_tok", [16, 64])
def test_dequant_matmul_headline_layer_few_tokens(n_tok):
    # 4096 x 11008, 4-bit g128, natural order (static groups or no act-order):
    # the few-token matrix-core route, every output compared
    d_out, d_in, bits, gs = 4096, 11008, 4, 128
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype="bf16", seed=77 + n_tok)
    Y, ref, X64 = _run(L, "natural", bits, gs)
    err = np.abs(Y - ref)
    tol = _bound(L, X64, "natural", gs, bits, "bf16")
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"
    assert np.median(err / np.maximum(np.abs(ref), 1e-30)) < 1e-5


def test_dequant_matmul_headline_layer_many_tokens():
    # 4096 x 11008, 4-bit g128, natural order, 512 tokens: the matrix-core route
    d_out, d_in, bits, gs, n_tok = 4096, 11008, 4, 128, 512
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype="bf16", seed=512)
    Y, ref, X64 = _run(L, "natural", bits, gs)
    err = np.abs(Y - ref)
    tol = _bound(L, X64, "natural", gs, bits, "bf16")
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"
    assert np.median(err / np.maximum(np.abs(ref), 1e-30)) < 1e-5


@pytest.mark.parametrize("mode", ["perm", "g_idx"])
def test_dequant_matmul_headline_layer(mode):
    # 4096 x 11008 (the down projection of a 7B decoder), 4-bit, g128,
    # act-order; decode batches of 1 and 4 tokens, every output compared
    d_out, d_in, bits, gs = 4096, 11008, 4, 128
    for n_tok in (1, 4):
        print(f"dequant headline {mode} n{n_tok}", flush=True)
        L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype="bf16", seed=11008 + n_tok)
        Y, ref, X64 = _run(L, mode, bits, gs)
        err = np.abs(Y - ref)
        tol = _bound(L, X64, mode, gs, bits)
        assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"
        # typical error far inside the bound
        assert np.median(err / np.maximum(np.abs(ref), 1e-30)) < 1e-5


def test_dequant_matmul_bad_indices_give_nan():
    bits, gs, d_out, d_in = 4, 128, 16, 512
    L = synth.make_packed_layer(d_out, d_in, 2, bits=bits, group_size=gs, dtype="bf16", seed=3)
    codes = torch.from_numpy(L.codes).to(DEV)
    X = to_torch(L.X, "bf16")
    scales = torch.from_numpy(L.scales).to(DEV)
    zeros = torch.from_numpy(L.zeros).to(DEV)
    perm = L.perm.copy()
    perm[17] = d_in + 5
    pt = torch.from_numpy(perm).to(DEV)
    Y = P.dequant_matmul(X, P.pack_permuted(codes, bits, pt), bits, scales, zeros, perm=pt, group_size=gs)
    assert torch.isnan(Y).all()
    gi = _g_idx(L.perm, gs, d_in)
    gi[100] = 7
    Y = P.dequant_matmul(X, P.pack(codes, bits), bits, scales, zeros, g_idx=torch.from_numpy(gi).to(DEV))
    assert torch.isnan(Y).all()
    torch.cuda.synchronize()


def test_pack_permuted_matches_oracle():
    for bits, d_in in ((4, 1000), (3, 257), (2, 64), (8, 33)):
        rng = np.random.default_rng(bits + d_in)
        codes = rng.integers(0, 1 << bits, size=(21, d_in)).astype(np.uint8)
        perm = rng.permutation(d_in).astype(np.int32)
        got = P.pack_permuted(torch.from_numpy(codes).to(DEV), bits, torch.from_numpy(perm).to(DEV))
        assert np.array_equal(got.cpu().numpy().view(np.uint32), O.pack_permuted(codes, bits, perm))


def test_quantized_layer_product_end_to_end():
    # quantize on the GPU with act-order, pack in quantization order, multiply:
    # the product equals X W_hat^T with the sweep's own reconstruction
    L = synth.make_layer(96, 640, 4096, dtype="bf16", sigma_w=0.02, dist="t4", outlier_frac=0.01,
                         outlier_scale=20.0, config=91, layer=1)
    cfg = P.make_config(bits=4, group_size=128, act_order=True)
    out = P.quantize(to_torch(L.W, "bf16"), X=to_torch(L.X, "bf16"), cfg=cfg, packed=False)
    Xd = to_torch(L.X[:3], "bf16")
    packed = P.pack_permuted(out["codes"], 4, out["perm"])
    Y = P.dequant_matmul(Xd, packed, 4, out["scales"], out["zeros"], perm=out["perm"], group_size=128)
    Y2 = P.dequant_matmul(Xd, P.pack(out["codes"], 4), 4, out["scales"], out["zeros"], g_idx=out["g_idx"])
    torch.cuda.synchronize()
    want = L.X_f64()[:3] @ out["w_hat"].double().cpu().numpy().T
    scale = np.abs(L.X_f64()[:3]) @ np.abs(out["w_hat"].double().cpu().numpy()).T
    for got in (Y, Y2):
        assert np.all(np.abs(got.double().cpu().numpy() - want) <= 1e-5 * scale)


@pytest.mark.parametrize("dtype,n_tok", [("bf16", 37), ("f16", 37), ("f32", 37), ("bf16", 1030)])
def test_gather_columns_exact(dtype, n_tok):
    # 37 tokens: tiles of 4 rows x 512 columns; 1030: 16 rows x 4096; ragged both ways
    d_in = 5000
    L = synth.make_packed_layer(4, d_in, n_tok, bits=4, group_size=128, dtype=dtype, seed=41)
    X = to_torch(L.X, dtype)
    perm = torch.from_numpy(L.perm).to(DEV)
    G = P.gather_columns(X, perm)
    torch.cuda.synchronize()
    want = X.cpu()[:, torch.from_numpy(L.perm).long()]
    assert torch.equal(G.cpu().view(torch.int16) if dtype != "f32" else G.cpu(),
                       want.view(torch.int16) if dtype != "f32" else want)
    bad = L.perm.copy()
    bad[123] = d_in
    G = P.gather_columns(X, torch.from_numpy(bad).to(DEV)).float().cpu()
    assert torch.isnan(G[:, 123]).all() and not torch.isnan(G[:, :123]).any()


def test_act_order_many_tokens_through_gather():
    # act-order layer packed in quantization order, 300 tokens: gather the
    # activations, then the matrix-core route without perm; equals the
    # oracle's product with perm
    bits, gs, n_tok, d_out, d_in = 4, 128, 300, 200, 1536
    L = synth.make_packed_layer(d_out, d_in, n_tok, bits=bits, group_size=gs, dtype="bf16", seed=300)
    codes = torch.from_numpy(L.codes).to(DEV)
    perm = torch.from_numpy(L.perm).to(DEV)
    packed = P.pack_permuted(codes, bits, perm)
    X = to_torch(L.X, "bf16")
    scales = torch.from_numpy(L.scales).to(DEV)
    zeros = torch.from_numpy(L.zeros).to(DEV)
    Y = P.dequant_matmul(P.gather_columns(X, perm), packed, bits, scales, zeros, group_size=gs)
    torch.cuda.synchronize()
    X64 = L.X_f64()
    ref = O.dequant_matmul(X64, O.pack_permuted(L.codes, bits, L.perm), bits, d_in, L.scales, L.zeros,
                           perm=L.perm, group_size=gs)
    # bound of the matrix-core route on the gathered activations (stream order)
    Xs = X64[:, L.perm]
    g = np.arange(d_in) // gs
    S = L.scales.astype(np.float64)[g].T
    Z = L.zeros.astype(np.float64)[g].T
    A = np.abs(Xs) @ (S * (L.codes[:, L.perm].astype(np.float64) + Z + 2.0 ** (bits + 1))).T
    tol = (2 * gs + d_in // gs + 8) * U32 * A
    assert np.all(np.abs(Y.cpu().numpy() - ref) <= tol)
