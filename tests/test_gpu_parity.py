"""HIP path vs the fp64 oracle on identical seeded inputs (needs an MI355X).

Every call goes through the C ABI (via the ctypes binding).  Shapes span
several tiles/blocks and ragged tails.  Tolerances:

* Hessian: bf16/fp16 products are exact in float32; the matrix cores sum
  them in float32 over runs of 256 tokens (16 MFMA steps of 16 tokens), and
  the runs are added in float64.  A run's float32 sum is off by at most
  (32 roundings) x 2^-24 x its sum of |products| (every MFMA step rounds
  once, the summation inside one step at most once more), so element-wise
  |H_gpu - H| <= 32 * 2^-24 * 2 * sum_t |x_ti x_tj| (+ float64 slack); the
  diagonal is summed from exact float64 squares: relative error <= 1e-12.
* prepare_hinv and the sweep run in float64, like the oracle: U within 1e-9
  relative (rounding order only); codes bit-identical when both sides get the
  same U; scales/zeros equal after rounding to float32 (1 ulp allowed).
* End to end from X: >= 99.9% codes identical and every difference <= 1
  (the pages' tolerance), loss within 1e-3 relative; every differing code is
  a rounding tie or follows from one (tie replay), and after the replay the
  scales are within 1e-5 relative and the zero points equal.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import synth

from _util import assert_from_x_parity, compare_codes, to_torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _layer(d_out, d_in, n_tok, dtype="bf16", dist="t4", frac=0.01, scale=30.0, seed=1, sigma=0.02):
    return synth.make_layer(d_out, d_in, n_tok, dtype=dtype, sigma_w=sigma, dist=dist,
                            outlier_frac=frac, outlier_scale=scale, config=90, layer=seed)


def _gpu_hessian(L):
    X = to_torch(L.X, L.dtype)
    d = X.shape[1]
    H = torch.zeros((d, d), dtype=torch.float64, device=DEV)
    P.hessian_accumulate(H, X)
    torch.cuda.synchronize()
    return H


# ---------------------------------------------------------------------------
# Hessian
# ---------------------------------------------------------------------------

# Cases: narrow layers (partial tiles summed by a second kernel), inputs whose
# rows are not 16-byte aligned (copied to an aligned buffer first), and wide
# layers (>= 256 tiles, every window added to H directly) with a ragged last
# tile over two or more 32768-token windows, aligned (4200) and not (4203).
@pytest.mark.parametrize("dtype,d,n", [("bf16", 300, 9000), ("f16", 257, 4500), ("f32", 130, 2100),
                                       ("bf16", 128, 32), ("bf16", 1, 7), ("f16", 383, 8200),
                                       ("bf16", 300, 70001), ("f16", 257, 65600), ("bf16", 1024, 5000),
                                       ("bf16", 4200, 40000), ("f16", 4203, 33000)])
def test_hessian_matches_oracle(dtype, d, n):
    print(f"hessian {dtype} d={d} n={n}", flush=True)
    L = _layer(4, d, n, dtype=dtype, seed=d)
    X64 = L.X_f64()
    Href = O.hessian(X64)
    Hg = _gpu_hessian(L).cpu().numpy()
    A = 2.0 * (np.abs(X64).T @ np.abs(X64))
    iu = np.triu_indices(d, 1)
    err = np.abs(Hg - Href)[iu]
    bound = 32 * 2.0 ** -24 * A[iu] + 1e-12 * A[iu] + 1e-300
    if err.size:
        print(f"  max |err| / bound {np.max(err / bound):.3e}, max |err| / sqrt(Hii Hjj) "
              f"{np.max(err / np.sqrt(np.outer(np.diag(Href), np.diag(Href))[iu] + 1e-300)):.3e}", flush=True)
    assert np.all(err <= bound)
    dg = np.diag(Hg)
    np.testing.assert_allclose(dg, np.diag(Href), rtol=1e-12, atol=0)
    dg = np.abs(np.diag(Hg) - np.diag(Href)) / np.abs(np.diag(Href)).max()
    assert dg.max() <= 1e-12
    assert np.all(np.tril(Hg, -1) == 0.0)  # strict lower untouched


def test_hessian_accumulates_over_calls_and_odd_stride():
    L = _layer(4, 200, 6000, dtype="bf16", seed=5)
    X = to_torch(L.X, "bf16")
    H1 = torch.zeros((200, 200), dtype=torch.float64, device=DEV)
    P.hessian_accumulate(H1, X[:2500])
    P.hessian_accumulate(H1, X[2500:])
    # odd row stride: a column slice of a wider buffer
    wide = torch.zeros((6000, 201), dtype=torch.bfloat16, device=DEV)
    wide[:, :200] = X
    H2 = torch.zeros((200, 200), dtype=torch.float64, device=DEV)
    P.hessian_accumulate(H2, wide[:, :200])
    Href = O.hessian(L.X_f64())
    iu = np.triu_indices(200)
    for H in (H1, H2):
        Hg = H.cpu().numpy()
        assert np.linalg.norm((Hg - Href)[iu]) / np.linalg.norm(Href[iu]) <= 1e-6


def test_hessian_deterministic():
    L = _layer(4, 260, 5000, dtype="bf16", seed=6)
    a = _gpu_hessian(L).cpu().numpy()
    b = _gpu_hessian(L).cpu().numpy()
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# prepare_hinv: order, damping, U
# ---------------------------------------------------------------------------

def _gpu_prepare(Hfull, cfg):
    d = Hfull.shape[0]
    H = torch.from_numpy(np.triu(Hfull)).to(DEV)
    perm = P.prepare_hinv(H, cfg)
    torch.cuda.synchronize()
    return H.cpu().numpy(), perm.cpu().numpy()


@pytest.mark.parametrize("d,act", [(1, False), (2, True), (63, True), (64, False), (65, True),
                                   (200, True), (333, False)])
def test_prepare_hinv_matches_oracle(d, act):
    print(f"prepare_hinv d={d} act={act}", flush=True)
    L = _layer(4, d, max(3 * d, 500), dtype="f32", dist="gauss_mix", frac=0.0, seed=d + 1)
    H = O.hessian(L.X_f64())
    cfg = P.make_config(act_order=act, damp=0.01)
    Ug, perm = _gpu_prepare(H, cfg)
    p = O.act_order_permutation(H) if act else np.arange(d)
    assert np.array_equal(perm, p)
    Uref = O.inverse_hessian_upper(O.damp_hessian(H[np.ix_(p, p)], 0.01))
    assert np.all(np.tril(Ug, -1) == 0.0)
    err = np.abs(Ug - Uref).max() / np.abs(Uref).max()
    assert err <= 1e-9, err


@pytest.mark.parametrize("d,act", [(2100, True), (4700, False)])
def test_prepare_hinv_large_matches_oracle(d, act):
    # sizes whose top products run on the LDS-tiled GEMM (64- and
    # 128-column tiles, triangular K ranges, XCD-balanced tile lists)
    print(f"prepare_hinv d={d} act={act}", flush=True)
    L = _layer(4, d, d + 300, dtype="f32", dist="gauss_mix", frac=0.0, seed=d + 1)
    H = O.hessian(L.X_f64())
    cfg = P.make_config(act_order=act, damp=0.01)
    Ug, perm = _gpu_prepare(H, cfg)
    p = O.act_order_permutation(H) if act else np.arange(d)
    assert np.array_equal(perm, p)
    Uref = O.inverse_hessian_upper(O.damp_hessian(H[np.ix_(p, p)], 0.01))
    assert np.all(np.tril(Ug, -1) == 0.0)
    err = np.abs(Ug - Uref).max() / np.abs(Uref).max()
    assert err <= 1e-9, err


def test_act_order_ties_and_dead_channels():
    d = 150
    # three tie classes, one of them all-zero (dead channels)
    H = np.diag(np.repeat([5.0, 3.0, 0.0], 50)[np.random.default_rng(1).permutation(d)])
    cfg = P.make_config(act_order=True, damp=0.1)
    Ug, perm = _gpu_prepare(H, cfg)
    assert np.array_equal(perm, O.act_order_permutation(H))


def test_not_pd_and_nonfinite():
    cfg = P.make_config(damp=0.01)
    with pytest.raises(P.NotPositiveDefinite):
        _gpu_prepare(np.zeros((70, 70)), cfg)
    bad = np.eye(40)
    bad[3, 5] = bad[5, 3] = 2.0
    with pytest.raises(P.NotPositiveDefinite):
        _gpu_prepare(bad, P.make_config(damp=0.0))
    nan = np.eye(40)
    nan[2, 30] = np.nan
    with pytest.raises(P.NonFinite):
        _gpu_prepare(nan, cfg)


# ---------------------------------------------------------------------------
# Column sweep fed the oracle's U
# ---------------------------------------------------------------------------

def _sweep_case(d_out, d_in, bits, g, act, sym=False, block=128, dtype="bf16", seed=0, static_groups=False):
    L = _layer(d_out, d_in, max(2 * d_in, 1000), dtype=dtype, seed=100 + seed)
    H = O.hessian(L.X_f64())
    ref = O.gptq_quantize(L.W_f64(), H, bits=bits, group_size=g, sym=sym, act_order=act, block=block,
                          static_groups=static_groups)
    cfg = P.make_config(bits=bits, group_size=g, sym=sym, act_order=act, block=block, static_groups=static_groups)
    W = to_torch(L.W, dtype)
    U = torch.from_numpy(ref["U"]).to(DEV)
    perm = torch.from_numpy(ref["perm"].astype(np.int32)).to(DEV)
    out = P.quantize_layer(W, U, perm, cfg)
    torch.cuda.synchronize()
    return ref, {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("d_out,d_in,bits,g,act,sym,block", [
    (100, 300, 4, 128, True, False, 128),
    (64, 256, 4, -1, False, False, 128),
    (130, 384, 3, 64, True, False, 128),
    (70, 200, 2, 32, False, False, 64),
    (33, 259, 4, 256, True, False, 128),   # group spans two blocks; ragged tail
    (40, 96, 4, 16, False, True, 32),      # symmetric
    (20, 75, 8, 25, False, False, 25),     # odd sizes: sub-block width 1
    (5, 40, 3, 12, True, False, 4),        # sub-block width 4
    # block and group widths that do not divide one another: groups begin
    # inside a block and run past its end
    (96, 1000, 4, 96, True, False, 128),   # superblocks of lcm multiples, ragged tail
    (64, 700, 3, 48, False, False, 128),
    (50, 600, 4, 200, True, False, 128),   # group wider than a block, across two block ends
    (40, 333, 2, 100, True, False, 64),
    (30, 250, 4, 30, False, True, 32),     # symmetric, sub-block width 2
    (12, 60, 3, 12, False, False, 5),      # odd block, sub-block width 1
    (9, 21, 3, 6, True, False, 1),         # one column per block
    (7, 50, 4, 10, False, False, 3),       # block 3, group 10
    # lcm(B, g) beyond the superblock cap: superblocks of one block, groups
    # crossing superblock ends while far updates are pending (d_in > 3B)
    (64, 1000, 4, 100, True, False, 128),
    (48, 900, 3, 120, False, False, 128),
    (40, 700, 4, 64, False, False, 100),
])
def test_sweep_matches_oracle_given_U(d_out, d_in, bits, g, act, sym, block):
    print(f"sweep {d_out}x{d_in} b{bits} g{g} act{act} sym{sym} B{block}", flush=True)
    ref, got = _sweep_case(d_out, d_in, bits, g, act, sym, block, seed=d_in)
    assert np.array_equal(got["codes"], ref["codes"])
    assert np.array_equal(got["g_idx"], ref["g_idx"])
    np.testing.assert_allclose(got["scales"], ref["scales"].astype(np.float32), rtol=2e-7)
    np.testing.assert_array_equal(got["zeros"], ref["zeros"].astype(np.float32))
    np.testing.assert_allclose(got["w_hat"], ref["w_hat"].astype(np.float32), rtol=2e-7, atol=1e-30)
    np.testing.assert_allclose(got["row_loss"], ref["row_loss"], rtol=1e-9)


@pytest.mark.parametrize("d_out,d_in,bits,g,act,sym,block", [
    (100, 300, 4, 128, True, False, 128),  # ragged last group
    (130, 384, 3, 64, True, False, 128),
    (40, 96, 4, 16, False, True, 32),      # symmetric, natural order
    (96, 1000, 4, 96, True, False, 128),   # groups crossing block ends, ragged tail
    (50, 600, 4, 200, True, False, 128),   # group wider than a block
    (64, 1000, 4, 100, True, False, 128),  # groups crossing superblock ends
    (20, 75, 8, 25, False, False, 25),     # 8-bit, partial blocks
    (9, 21, 3, 6, True, False, 1),         # one column per block
    (64, 256, 4, -1, True, False, 128),    # per-row: the same as the default grouping
])
def test_static_groups_sweep_matches_oracle_given_U(d_out, d_in, bits, g, act, sym, block):
    """Static groups: parameters per group of original columns from W as
    given, act-order only ordering the sweep, g_idx = j // g."""
    print(f"static sweep {d_out}x{d_in} b{bits} g{g} act{act} sym{sym} B{block}", flush=True)
    ref, got = _sweep_case(d_out, d_in, bits, g, act, sym, block, seed=d_in + 1, static_groups=True)
    assert np.array_equal(got["codes"], ref["codes"])
    assert np.array_equal(got["g_idx"], ref["g_idx"])
    if g > 0:
        assert np.array_equal(got["g_idx"], np.arange(d_in) // g)
    np.testing.assert_allclose(got["scales"], ref["scales"].astype(np.float32), rtol=2e-7)
    np.testing.assert_array_equal(got["zeros"], ref["zeros"].astype(np.float32))
    np.testing.assert_allclose(got["w_hat"], ref["w_hat"].astype(np.float32), rtol=2e-7, atol=1e-30)
    np.testing.assert_allclose(got["row_loss"], ref["row_loss"], rtol=1e-9)
    if act and g > 0 and d_out * d_in >= 10000:
        dyn = O.gptq_quantize(_layer(d_out, d_in, max(2 * d_in, 1000), seed=100 + d_in + 1).W_f64(), H=ref["H"],
                              bits=bits, group_size=g, sym=sym, act_order=act, block=block)
        assert not np.array_equal(dyn["codes"], got["codes"])   # the option changes the result


@pytest.mark.parametrize("bits,g,sym", [(4, 32, False), (3, 64, True), (2, -1, False)])
def test_sweep_zero_and_one_signed_groups(bits, g, sym):
    # rows 0-3 all zero (every group all-zero: xmin = -1, xmax = 1 in the
    # asymmetric grid, amax = 1 in the symmetric one; codes = zero point);
    # rows 4-7 all positive and rows 8-11 all negative (the range widened to
    # include 0); the rest Gaussian.  U from correlated activations, so the
    # compensation is real.
    d_out, d_in = 40, 160
    L = _layer(d_out, d_in, 1500, seed=77)
    rng = np.random.default_rng(78)
    W = L.W_f64().copy()
    W[0:4] = 0.0
    W[4:8] = rng.uniform(0.5, 1.0, (4, d_in))
    W[8:12] = -rng.uniform(0.5, 1.0, (4, d_in))
    H = O.hessian(L.X_f64())
    ref = O.gptq_quantize(W, H, bits=bits, group_size=g, sym=sym, act_order=True)
    cfg = P.make_config(bits=bits, group_size=g, sym=sym, act_order=True)
    out = P.quantize_layer(torch.from_numpy(W.astype(np.float32)).to(DEV), torch.from_numpy(ref["U"]).to(DEV),
                           torch.from_numpy(ref["perm"].astype(np.int32)).to(DEV), cfg)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    # the float32 copy of W is exact for the Gaussian rows (bf16 values) but
    # not for the uniform ones: the oracle quantizes the same float32 values
    ref = O.gptq_quantize(W.astype(np.float32).astype(np.float64), H, bits=bits, group_size=g, sym=sym,
                          act_order=True)
    assert np.array_equal(got["codes"], ref["codes"])
    np.testing.assert_allclose(got["scales"], ref["scales"].astype(np.float32), rtol=2e-7)
    np.testing.assert_array_equal(got["zeros"], ref["zeros"].astype(np.float32))
    zero_pt = 2 ** (bits - 1)   # sym: 2^(b-1); asym all-zero: rint(maxq / 2) = 2^(b-1), ties to even
    assert np.all(got["codes"][0:4] == zero_pt)
    assert np.all(got["w_hat"][0:4] == 0.0)
    if not sym:
        assert np.all(got["zeros"][:, 4:8] == 0.0)                  # xmin = 0: zero point 0
        assert np.all(got["zeros"][:, 8:12] == 2 ** bits - 1)       # xmax = 0: zero point maxq


def test_sweep_exact_ties_round_half_even():
    # One-hot tokens make H, and so U, diagonal: no compensation crosses
    # columns and every weight reaches the quantizer as written.  Each
    # 128-column group holds 0 and 15 (4-bit asym: scale 1, zero 0) and
    # otherwise k + 0.5, so every other quotient is an exact tie, decided
    # half-to-even as in the oracle.
    d_out, d_in = 24, 256
    rng = np.random.default_rng(5)
    W = rng.integers(0, 15, size=(d_out, d_in)).astype(np.float64) + 0.5
    W[:, 0::128] = 0.0
    W[:, 1::128] = 15.0
    H = O.hessian(np.eye(d_in))
    ref = O.gptq_quantize(W, H, bits=4, group_size=128, act_order=False)
    assert np.array_equal(ref["codes"], np.rint(W).astype(ref["codes"].dtype))
    cfg = P.make_config(bits=4, group_size=128, act_order=False)
    out = P.quantize_layer(torch.from_numpy(W.astype(np.float32)).to(DEV), torch.from_numpy(ref["U"]).to(DEV),
                           torch.from_numpy(ref["perm"].astype(np.int32)).to(DEV), cfg)
    torch.cuda.synchronize()
    assert np.array_equal(out["codes"].cpu().numpy(), ref["codes"])


def test_sweep_fp16_and_fp32_weights():
    for dtype in ("f16", "f32"):
        ref, got = _sweep_case(48, 256, 4, 128, True, dtype=dtype, seed=7)
        assert np.array_equal(got["codes"], ref["codes"]), dtype


def test_sweep_nonfinite_weight():
    L = _layer(8, 128, 500)
    H = O.hessian(L.X_f64())
    ref = O.gptq_quantize(L.W_f64(), H)
    W = to_torch(L.W, "bf16")
    W[3, 7] = float("nan")
    with pytest.raises(P.NonFinite):
        P.quantize_layer(W, torch.from_numpy(ref["U"]).to(DEV),
                         torch.from_numpy(ref["perm"].astype(np.int32)).to(DEV), P.make_config())


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_in", [1, 31, 100, 257, 1024])
def test_pack_matches_oracle(bits, d_in):
    rng = np.random.default_rng(bits * 7 + d_in)
    codes = rng.integers(0, 2 ** bits, size=(37, d_in)).astype(np.uint8)
    got = P.pack(torch.from_numpy(codes).to(DEV), bits).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, O.pack(codes, bits))


# ---------------------------------------------------------------------------
# End to end from X
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,n,dtype,bits,g,act", [
    (256, 256, 2048, "f32", 4, -1, False),      # workload 1, full size
    (192, 640, 8192, "bf16", 4, 128, True),     # workload-3 recipe, reduced
    (150, 512, 8192, "f16", 3, 128, False),     # workload-2/5 recipe, reduced
    (96, 448, 6000, "bf16", 2, 64, True),       # workload-4 recipe, reduced
    (128, 600, 6000, "bf16", 3, 96, True),      # group 96 with block 128: groups cross block ends
])
def test_end_to_end(d_out, d_in, n, dtype, bits, g, act):
    print(f"e2e {d_out}x{d_in} n={n} {dtype} b{bits} g{g} act{act}", flush=True)
    if dtype == "f32":
        L = synth.make_layer(d_out, d_in, n, dtype="f32", sigma_w=0.02, dist="gauss_mix",
                             outlier_count=4, outlier_scale=20.0, config=1, layer=0)
    else:
        L = _layer(d_out, d_in, n, dtype=dtype, frac=0.005, scale=50.0, seed=d_in)
    ref = O.gptq_quantize(L.W_f64(), X=L.X_f64(), bits=bits, group_size=g, act_order=act)
    cfg = P.make_config(bits=bits, group_size=g, act_order=act)
    out = P.quantize(to_torch(L.W, dtype), X=to_torch(L.X, dtype), cfg=cfg)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    same, mx = compare_codes(got["codes"], ref["codes"])
    assert same >= 0.999 and mx <= 1, (same, mx)
    loss_g = O.layer_loss(L.W_f64(), got["w_hat"].astype(np.float64), ref["H"]).sum()
    assert abs(loss_g - ref["loss"].sum()) <= 1e-3 * ref["loss"].sum()
    words = got["packed"].view(np.uint32)
    assert np.array_equal(words, O.pack(got["codes"], bits))
    assert_from_x_parity(O, L.W_f64(), ref["H"], got, bits, g, act, name=f"{d_out}x{d_in}")
    print(f"  identical {same:.6f} max diff {mx}", flush=True)


@pytest.mark.parametrize("d_out,d_in,n,dtype,bits,g", [
    (192, 640, 8192, "bf16", 4, 128),   # workload-3 recipe, reduced
    (96, 448, 6000, "bf16", 2, 64),     # workload-4 recipe, reduced
    (128, 600, 6000, "f16", 3, 96),     # groups crossing block ends, ragged last group
])
def test_static_groups_end_to_end(d_out, d_in, n, dtype, bits, g):
    """Static groups with act-order from X: the same acceptance as the
    default grouping, and the product from the packed words needs no
    gather (g_idx = j // g: the plain original-order product)."""
    print(f"static e2e {d_out}x{d_in} n={n} {dtype} b{bits} g{g}", flush=True)
    L = _layer(d_out, d_in, n, dtype=dtype, frac=0.005, scale=50.0, seed=d_in + 3)
    ref = O.gptq_quantize(L.W_f64(), X=L.X_f64(), bits=bits, group_size=g, act_order=True, static_groups=True)
    cfg = P.make_config(bits=bits, group_size=g, act_order=True, static_groups=True)
    out = P.quantize(to_torch(L.W, dtype), X=to_torch(L.X, dtype), cfg=cfg)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    same, mx = compare_codes(got["codes"], ref["codes"])
    assert same >= 0.999 and mx <= 1, (same, mx)
    rp = assert_from_x_parity(O, L.W_f64(), ref["H"], got, bits, g, True, name=f"static {d_out}x{d_in}",
                              static_groups=True)
    assert rp["same_raw"] >= 0.999
    Xt = to_torch(L.X[:300], dtype)
    Y = P.dequant_matmul(Xt, out["packed"], bits, out["scales"], out["zeros"], group_size=g)
    torch.cuda.synchronize()
    want = O.dequant_matmul(L.X_f64()[:300], O.pack(got["codes"], bits), bits, d_in, got["scales"].astype(np.float64),
                            got["zeros"].astype(np.float64), g_idx=np.arange(d_in) // g)
    # float32 error bound of the product (either route: the matrix-core one
    # sums a group's products in float32, the block route chains v_dot2 and
    # FMAs), elementwise with A = sum_k |x_k| s_k (c_k + z_k + 2^(b+1))
    S = got["scales"].astype(np.float64)[np.arange(d_in) // g].T
    Z = got["zeros"].astype(np.float64)[np.arange(d_in) // g].T
    A = np.abs(L.X_f64()[:300]) @ (S * (got["codes"] + Z + 2.0 ** (bits + 1))).T
    ng = -(-d_in // g)
    nb = -(-(-(-d_in // 32)) // 256)
    tol = (max(2 * g + ng + 8, 96 + 32 * nb)) * 2.0 ** -24 * A
    assert np.all(np.abs(Y.cpu().numpy() - want) <= tol)


@pytest.mark.parametrize("factored", [True, False])
@pytest.mark.parametrize("d_out,d_in,n,dtype,bits,g,act", [
    (1, 256, 1024, "bf16", 4, 128, True),    # one row: one workgroup with a single live row
    (3, 128, 300, "f16", 3, 64, False),      # one block: no lazy update at all
    (2, 128, 200, "bf16", 2, -1, True),      # one block, one group per row
])
def test_degenerate_layers(d_out, d_in, n, dtype, bits, g, act, factored):
    print(f"degenerate {d_out}x{d_in} n={n} {dtype} b{bits} g{g} act{act} factored {factored}", flush=True)
    L = _layer(d_out, d_in, n, dtype=dtype, frac=0.01, scale=30.0, seed=d_in + d_out)
    ref = O.gptq_quantize(L.W_f64(), X=L.X_f64(), bits=bits, group_size=g, act_order=act)
    cfg = P.make_config(bits=bits, group_size=g, act_order=act)
    out = P.quantize(to_torch(L.W, dtype), X=to_torch(L.X, dtype), cfg=cfg, factored=factored)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    assert got["codes"].shape == (d_out, d_in)
    assert np.array_equal(got["packed"].view(np.uint32), O.pack(got["codes"], bits))
    assert_from_x_parity(O, L.W_f64(), ref["H"], got, bits, g, act, name=f"degenerate {d_out}x{d_in}")


def test_hessian_empty_and_single_token():
    # no tokens: H unchanged (nothing launched); one token: the outer product
    L = _layer(4, 200, 1, seed=5)
    X1 = to_torch(L.X, "bf16")
    H = torch.full((200, 200), 0.25, dtype=torch.float64, device=DEV)
    P.hessian_accumulate(H, X1[:0])
    torch.cuda.synchronize()
    assert torch.all(H == 0.25)
    P.hessian_accumulate(H, X1)
    torch.cuda.synchronize()
    x = L.X_f64()[0]
    want = 0.25 + 2.0 * np.outer(x, x)
    got = H.cpu().numpy()
    iu = np.triu_indices(200)
    # bf16 products are exact in float32 and one token is one product per entry
    np.testing.assert_allclose(got[iu], want[iu], rtol=1e-15, atol=0)


def test_scale_invariance_and_row_subset_on_gpu():
    L = _layer(64, 256, 3000, seed=11)
    H = O.hessian(L.X_f64())
    cfg = P.make_config(bits=4, group_size=64, act_order=True)
    W = to_torch(L.W, "bf16")
    outs = []
    for f in (1.0, 4.0):
        Ht = torch.from_numpy(np.triu(H) * f).to(DEV)
        outs.append({k: v.cpu().numpy() for k, v in P.quantize(W, H=Ht, cfg=cfg).items()})
    for k in ("codes", "scales", "zeros", "perm", "g_idx"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
    rows = torch.tensor([5, 63, 0, 17], device=DEV)
    sub = P.quantize(W[rows].contiguous(), H=torch.from_numpy(np.triu(H)).to(DEV), cfg=cfg)
    assert np.array_equal(sub["codes"].cpu().numpy(), outs[0]["codes"][rows.cpu().numpy()])


def test_sweep_rejects_bad_perm():
    L = _layer(8, 64, 500)
    H = O.hessian(L.X_f64())
    ref = O.gptq_quantize(L.W_f64(), H, group_size=32, block=32)
    W = to_torch(L.W, "bf16")
    U = torch.from_numpy(ref["U"]).to(DEV)
    cfg = P.make_config(group_size=32, block=32)
    dup = torch.arange(64, dtype=torch.int32, device=DEV)
    dup[5] = 6
    with pytest.raises(P.InvalidArgument):
        P.quantize_layer(W, U, dup, cfg)
    oob = torch.arange(64, dtype=torch.int32, device=DEV)
    oob[9] = 64
    with pytest.raises(P.InvalidArgument):
        P.quantize_layer(W, U, oob, cfg)
