"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the oracle to a hand-worked example, a closed form, a special
case that reduces to a simpler textbook procedure, a brute-force rendering of
the pages' OBS formula, or an exact identity of the method, chosen so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_pd(rng, d, cond_spread=1.0):
    A = rng.standard_normal((d, 2 * d + 3))
    D = np.exp(cond_spread * rng.standard_normal(d))
    A = A * D[:, None]
    return 2.0 * A @ A.T


# ---------------------------------------------------------------------------
# Hand-worked examples (tests/golden)
# ---------------------------------------------------------------------------

def test_hand_two_column_example():
    g = _load("hand_2col.json")
    out = O.gptq_quantize(np.array(g["W"]), np.array(g["H"]), bits=g["bits"],
                          group_size=g["group_size"], sym=g["sym"],
                          act_order=g["act_order"], block=g["block"], damp=g["damp"])
    np.testing.assert_array_equal(out["codes"], np.array(g["codes"]))
    np.testing.assert_allclose(out["scales"], g["scales"], rtol=1e-15)
    np.testing.assert_array_equal(out["zeros"], g["zeros"])
    np.testing.assert_allclose(out["w_hat"], g["w_hat"], rtol=1e-15)
    np.testing.assert_allclose(out["row_loss"], g["row_loss"], rtol=1e-13)
    np.testing.assert_allclose(out["U"], g["U"], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(out["loss"], g["row_loss"], rtol=1e-13)


def test_quant_grid_hand_cases():
    for case in _load("quant_grid.json")["cases"]:
        w = np.array([case["w"]])
        s, z = O.quant_params(w, case["bits"], case["sym"])
        assert s[0] == pytest.approx(case["scale"], rel=1e-15), case["note"]
        assert z[0] == case["zero"], case["note"]
        codes = [int(O.quantize_column(np.array([x]), s, z, case["bits"])[0][0]) for x in case["w"]]
        assert codes == case["codes"], case["note"]


def test_pack_hand_cases():
    for case in _load("pack_examples.json")["cases"]:
        codes = np.array(case["codes"])
        words = O.pack(codes, case["bits"])
        assert words.tolist() == case["words"], case["note"]
        back = O.unpack(words, case["bits"], codes.shape[1])
        np.testing.assert_array_equal(back, codes)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_in", [1, 31, 32, 33, 96, 257])
def test_pack_roundtrip(bits, d_in):
    rng = np.random.default_rng(bits * 1000 + d_in)
    codes = rng.integers(0, 2 ** bits, size=(5, d_in))
    words = O.pack(codes, bits)
    assert words.shape == (5, -(-d_in * bits // 32))
    np.testing.assert_array_equal(O.unpack(words, bits, d_in), codes)
    # bits past the last code stay zero
    total = d_in * bits
    if total % 32:
        assert np.all(words[:, -1] >> np.uint32(total % 32) == 0)


def test_pack_4bit_is_base16_digits():
    """4-bit words are the base-16 numbers whose digits are the codes, low first."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(3, 64))
    words = O.pack(codes, 4)
    for r in range(3):
        for m in range(8):
            expect = sum(int(codes[r, 8 * m + t]) * 16 ** t for t in range(8))
            assert int(words[r, m]) == expect


# ---------------------------------------------------------------------------
# Hessian
# ---------------------------------------------------------------------------

def test_hessian_explicit_loops():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((7, 4))
    H = O.hessian(X)
    for i in range(4):
        for j in range(4):
            s = 0.0
            for t in range(7):
                s += X[t, i] * X[t, j]
            assert H[i, j] == pytest.approx(2.0 * s, rel=1e-14, abs=1e-14)


def test_hessian_chunks_and_psd():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((300, 20))
    H1 = O.hessian(X)
    H2 = O.hessian([X[:100], X[100:257], X[257:]])
    np.testing.assert_allclose(H1, H2, rtol=1e-13, atol=1e-12)
    np.testing.assert_array_equal(H1, H1.T)
    assert np.linalg.eigvalsh(H1).min() > -1e-9 * np.abs(H1).max()


# ---------------------------------------------------------------------------
# The Cholesky form of the inverse
# ---------------------------------------------------------------------------

def test_U_is_upper_factor_of_inverse():
    rng = np.random.default_rng(5)
    H = _rand_pd(rng, 30, 1.0)
    Hd = O.damp_hessian(H, 0.01)
    U = O.inverse_hessian_upper(Hd)
    assert np.allclose(np.tril(U, -1), 0.0)
    assert np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(30), atol=1e-10)


def test_U_reverse_cholesky_identity():
    """U = J chol(J H_d J)^{-1} J, J the reversal: the 'UL' route to the same factor."""
    rng = np.random.default_rng(6)
    for d in (1, 2, 9, 40):
        Hd = O.damp_hessian(_rand_pd(rng, d, 1.5), 0.01)
        U = O.inverse_hessian_upper(Hd)
        J = np.eye(d)[::-1]
        Lr = np.linalg.cholesky(J @ Hd @ J)
        U2 = J @ np.linalg.inv(Lr) @ J
        np.testing.assert_allclose(U, U2, rtol=1e-10, atol=1e-12 * np.abs(U).max())


def test_damp_hand_values():
    g = _load("damp_hand.json")["damp_only"]
    Hd = O.damp_hessian(np.array(g["H"]), g["damp"])
    np.testing.assert_allclose(Hd, np.array(g["Hd"]), rtol=1e-15, atol=0)


def test_damp_hand_sweep():
    # a two-column layer swept with damp 0.5: lambda shows in U and row_loss
    g = _load("damp_hand.json")["sweep"]
    out = O.gptq_quantize(np.array(g["W"]), np.array(g["H"]), bits=g["bits"], group_size=-1,
                          act_order=False, block=128, damp=g["damp"])
    np.testing.assert_allclose(out["U"], np.array(g["U"]), rtol=1e-14, atol=1e-17)
    np.testing.assert_array_equal(out["codes"], np.array(g["codes"]))
    np.testing.assert_allclose(out["scales"], np.array(g["scales"]), rtol=1e-15)
    np.testing.assert_array_equal(out["zeros"], np.array(g["zeros"]))
    np.testing.assert_allclose(out["w_hat"], np.array(g["w_hat"]), rtol=1e-15)
    np.testing.assert_allclose(out["row_loss"], g["row_loss"], rtol=1e-13)
    np.testing.assert_allclose(out["loss"], g["loss"], rtol=1e-13)


def test_damp_shifts_the_spectrum():
    # H + lambda*I has the eigenvalues of H shifted by lambda = damp * tr(H) / d
    rng = np.random.default_rng(3)
    H = _rand_pd(rng, 7, 1.0)
    ev = np.linalg.eigvalsh(H)
    evd = np.linalg.eigvalsh(O.damp_hessian(H, 0.01))
    np.testing.assert_allclose(evd - ev, 0.01 * np.trace(H) / 7, rtol=1e-12)


# ---------------------------------------------------------------------------
# P-RTN: with a diagonal H there is nothing to compensate.
# ---------------------------------------------------------------------------

def _rtn_in_test(W, bits, g, sym):
    """Round-to-nearest per group from the untouched weights, written out here."""
    d_out, d_in = W.shape
    maxq = 2 ** bits - 1
    codes = np.zeros_like(W, dtype=np.int64)
    for s in range(0, d_in, g):
        blk = W[:, s:s + g]
        lo = np.minimum(blk.min(1), 0)
        hi = np.maximum(blk.max(1), 0)
        if sym:
            a = np.maximum(-lo, hi)
            a[a == 0] = 1
            scale = 2 * a / maxq
            zero = np.full(d_out, 2 ** (bits - 1))
        else:
            both0 = (lo == 0) & (hi == 0)
            lo[both0], hi[both0] = -1, 1
            scale = (hi - lo) / maxq
            zero = np.rint(-lo / scale)
        codes[:, s:s + g] = np.clip(np.rint(blk / scale[:, None]) + zero[:, None], 0, maxq)
    return codes


@pytest.mark.parametrize("bits,g,sym", [(4, -1, False), (3, 16, False), (2, 8, True), (4, 64, False)])
def test_identity_hessian_reduces_to_rtn(bits, g, sym):
    rng = np.random.default_rng(10 + bits)
    W = 0.02 * rng.standard_normal((9, 64))
    H = 3.0 * np.eye(64)
    out = O.gptq_quantize(W, H, bits=bits, group_size=g, sym=sym, block=32, damp=0.01)
    gg = 64 if g <= 0 else g
    np.testing.assert_array_equal(out["codes"], _rtn_in_test(W, bits, gg, sym))


def test_diagonal_hessian_act_order_is_rtn_on_sorted_columns():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((6, 48))
    dg = rng.permutation(np.arange(1, 49)).astype(float)
    out = O.gptq_quantize(W, np.diag(dg), bits=3, group_size=16, act_order=True, block=16)
    order = np.argsort(-dg, kind="stable")
    np.testing.assert_array_equal(out["perm"], order)
    expect = np.empty_like(out["codes"])
    expect[:, order] = _rtn_in_test(W[:, order], 3, 16, False)
    np.testing.assert_array_equal(out["codes"], expect)
    np.testing.assert_array_equal(out["g_idx"][order], np.arange(48) // 16)


# ---------------------------------------------------------------------------
# P-OBS: brute-force fixed-order OBS with explicit inverses.
# ---------------------------------------------------------------------------

def _obs_bruteforce(W, Hd, bits, g, sym):
    """Fixed-order OBS: after each column, re-invert H_d over the remaining set F."""
    W = W.astype(float).copy()
    d_out, d = W.shape
    maxq = 2 ** bits - 1
    codes = np.zeros((d_out, d), dtype=np.int64)
    qv = np.zeros((d_out, d))
    for q in range(d):
        if q % g == 0:
            blk = W[:, q:q + g]
            lo = np.minimum(blk.min(1), 0)
            hi = np.maximum(blk.max(1), 0)
            if sym:
                a = np.maximum(-lo, hi)
                a[a == 0] = 1
                scale, zero = 2 * a / maxq, np.full(d_out, 2.0 ** (bits - 1))
            else:
                both0 = (lo == 0) & (hi == 0)
                lo[both0], hi[both0] = -1, 1
                scale = (hi - lo) / maxq
                zero = np.rint(-lo / scale)
        c = np.clip(np.rint(W[:, q] / scale) + zero, 0, maxq)
        val = scale * (c - zero)
        codes[:, q], qv[:, q] = c, val
        F = list(range(q, d))
        Hinv = np.linalg.inv(Hd[np.ix_(F, F)])
        # delta_F = -(w_q - q) / [H_F^-1]_qq * [H_F^-1]_{:, q}
        delta = -np.outer((W[:, q] - val) / Hinv[0, 0], Hinv[:, 0])
        W[:, F] += delta
        W[:, q] = val
    return codes, qv


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("g", [-1, 2, 4])
def test_matches_bruteforce_obs(seed, g):
    rng = np.random.default_rng(100 + seed)
    d = 2 + seed  # 2..7 columns
    W = rng.standard_normal((5, d))
    H = _rand_pd(rng, d, 0.8)
    for act in (False, True):
        out = O.gptq_quantize(W, H, bits=2, group_size=g, act_order=act, block=2, damp=0.01)
        perm = out["perm"]
        Hd = O.damp_hessian(H[np.ix_(perm, perm)], 0.01)
        gg = d if g <= 0 else g
        if g > 0 and 2 % g and g % 2:
            continue
        c_bf, q_bf = _obs_bruteforce(W[:, perm], Hd, 2, gg, False)
        np.testing.assert_array_equal(out["codes"][:, perm], c_bf)
        np.testing.assert_allclose(out["w_hat"][:, perm], q_bf, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P-B: lazy batching changes nothing.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("g", [-1, 16, 12])
def test_block_size_invariance(g):
    """Any block size, also one that neither divides nor is divided by the
    group width (groups then begin inside a block and run past its end):
    the codes do not change, since lazy batching is the per-column
    algorithm reordered (B = 1 is the unbatched sweep)."""
    rng = np.random.default_rng(20)
    X = rng.standard_normal((400, 96)) @ (rng.standard_normal((96, 96)) / 10)
    W = 0.02 * rng.standard_normal((11, 96))
    ref = O.gptq_quantize(W, X=X, bits=3, group_size=g, block=1)
    for B in (5, 7, 8, 16, 20, 32, 48, 96):
        out = O.gptq_quantize(W, X=X, bits=3, group_size=g, block=B)
        np.testing.assert_array_equal(out["codes"], ref["codes"])
        np.testing.assert_allclose(out["w_hat"], ref["w_hat"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(out["scales"], ref["scales"], rtol=1e-12)


def test_group_crossing_block_end_uses_compensated_values():
    """Worked by hand: d_in = 4, block 3, groups {0, 1} and {2, 3}, 2-bit
    asymmetric, U = I except U[0][3] = 5, one row w = (0.22, 0.3, 0, 0).
    Group {0, 1}: scale 0.3/3 = 0.1, zero 0; column 0 gets code 2, error
    0.02, so column 3 (past the block) holds 0 - 5 * 0.02 = -0.1 by the time
    group {2, 3} begins at column 2: range [-0.1, 0] -> scale 0.1/3, zero 3;
    column 2 -> code 3, column 3 -> code 0.  With the uncompensated value the
    group would be all zeros (scale 2/3, zero 2)."""
    U = np.eye(4)
    U[0, 3] = 5.0
    W = np.array([[0.22, 0.3, 0.0, 0.0]])
    codes, scales, zeros, w_hat, _ = O.sweep(W, U, 2, 2, False, block=3)
    np.testing.assert_allclose(scales[:, 0], [0.1, 0.1 / 3.0], rtol=1e-12)
    np.testing.assert_array_equal(zeros[:, 0], [0.0, 3.0])
    np.testing.assert_array_equal(codes[0], [2, 3, 3, 0])
    np.testing.assert_allclose(w_hat[0], [0.2, 0.3, 0.0, -0.1], rtol=1e-12, atol=1e-15)


def test_invalid_block_size():
    W = np.zeros((2, 48))
    with pytest.raises(O.InvalidArgument):
        O.gptq_quantize(W, np.eye(48), group_size=12, block=0)


# ---------------------------------------------------------------------------
# P-loss: the sweep's running loss equals the quadratic form of the change.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", [False, True])
def test_loss_identity(act):
    rng = np.random.default_rng(30)
    X = rng.standard_normal((500, 70)) @ (np.eye(70) + 0.3 * rng.standard_normal((70, 70)))
    W = 0.05 * rng.standard_normal((13, 70))
    out = O.gptq_quantize(W, X=X, bits=3, group_size=-1, act_order=act, block=16)
    p = out["perm"]
    Hd = O.damp_hessian(out["H"][np.ix_(p, p)], 0.01)
    dW = out["w_hat"][:, p] - W[:, p]
    quad = 0.5 * np.einsum("ij,jk,ik->i", dW, Hd, dW)
    np.testing.assert_allclose(out["row_loss"], quad, rtol=1e-9)


# ---------------------------------------------------------------------------
# P-range and dequantization.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,g,sym", [(2, 8, False), (3, 16, False), (4, -1, False), (4, 32, True), (8, 16, False)])
def test_code_range_and_dequant(bits, g, sym):
    rng = np.random.default_rng(40 + bits)
    X = rng.standard_t(4, size=(300, 64))
    W = 0.02 * rng.standard_normal((10, 64))
    out = O.gptq_quantize(W, X=X, bits=bits, group_size=g, sym=sym, act_order=True, block=16)
    maxq = 2 ** bits - 1
    assert out["codes"].min() >= 0 and out["codes"].max() <= maxq
    assert np.all(out["scales"] > 0)
    assert np.all(out["zeros"] == np.rint(out["zeros"]))
    assert np.all((out["zeros"] >= 0) & (out["zeros"] <= maxq))
    np.testing.assert_array_equal(
        O.dequantize(out["codes"], out["scales"], out["zeros"], out["g_idx"]), out["w_hat"])


# ---------------------------------------------------------------------------
# Invariances: scale of H, rows, act-order as a relabelling.
# ---------------------------------------------------------------------------

def test_hessian_scale_by_four_is_bit_identical():
    rng = np.random.default_rng(50)
    X = rng.standard_normal((256, 48))
    H = O.hessian(X)
    W = 0.02 * rng.standard_normal((7, 48))
    a = O.gptq_quantize(W, H, bits=4, group_size=16, act_order=True, block=16)
    b = O.gptq_quantize(W, 4.0 * H, bits=4, group_size=16, act_order=True, block=16)
    for k in ("codes", "scales", "zeros", "w_hat", "perm", "g_idx"):
        np.testing.assert_array_equal(a[k], b[k])


def test_rows_are_independent():
    rng = np.random.default_rng(60)
    X = rng.standard_normal((300, 40))
    W = 0.02 * rng.standard_normal((12, 40))
    full = O.gptq_quantize(W, X=X, bits=3, group_size=8, block=8)
    rows = np.array([9, 2, 2, 7, 0])
    sub = O.gptq_quantize(W[rows], X=X, bits=3, group_size=8, block=8)
    np.testing.assert_array_equal(sub["codes"], full["codes"][rows])
    np.testing.assert_allclose(sub["w_hat"], full["w_hat"][rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sub["scales"], full["scales"][:, rows], rtol=1e-12)


def test_act_order_is_natural_order_on_permuted_problem():
    rng = np.random.default_rng(70)
    X = rng.standard_normal((300, 40)) * np.exp(rng.standard_normal(40))
    W = 0.02 * rng.standard_normal((6, 40))
    H = O.hessian(X)
    a = O.gptq_quantize(W, H, bits=4, group_size=8, act_order=True, block=8)
    p = a["perm"]
    assert np.all(np.diff(np.diag(H)[p]) <= 0)
    b = O.gptq_quantize(W[:, p], H[np.ix_(p, p)], bits=4, group_size=8, act_order=False, block=8)
    np.testing.assert_array_equal(a["codes"][:, p], b["codes"])
    np.testing.assert_array_equal(a["w_hat"][:, p], b["w_hat"])
    np.testing.assert_array_equal(a["scales"], b["scales"])


def test_act_order_ties_go_to_lower_index():
    H = np.diag([1.0, 3.0, 3.0, 2.0, 3.0])
    np.testing.assert_array_equal(O.act_order_permutation(H), [1, 2, 4, 3, 0])
    # many ties: the order is (descending key, ascending index), by definition
    rng = np.random.default_rng(5)
    keys = rng.integers(0, 7, size=500).astype(float)
    expect = sorted(range(500), key=lambda j: (-keys[j], j))
    np.testing.assert_array_equal(O.act_order_permutation(np.diag(keys)), expect)


# ---------------------------------------------------------------------------
# Ragged shapes and degenerate inputs.
# ---------------------------------------------------------------------------

def test_ragged_tail_blocks_and_groups():
    rng = np.random.default_rng(80)
    X = rng.standard_normal((400, 75))
    W = 0.02 * rng.standard_normal((4, 75))
    a = O.gptq_quantize(W, X=X, bits=4, group_size=16, block=32)
    b = O.gptq_quantize(W, X=X, bits=4, group_size=16, block=16)
    assert a["scales"].shape == (5, 4)
    np.testing.assert_array_equal(a["codes"], b["codes"])


def test_dead_channel_is_kept():
    rng = np.random.default_rng(81)
    X = rng.standard_normal((200, 10))
    X[:, 3] = 0.0
    W = rng.standard_normal((3, 10))
    out = O.gptq_quantize(W, X=X, bits=4, group_size=-1, act_order=True)
    assert out["perm"][-1] == 3  # energy 0 is swept last
    assert np.all(np.isfinite(out["w_hat"]))


def test_errors():
    with pytest.raises(O.NotPositiveDefinite):
        O.gptq_quantize(np.ones((2, 3)), np.zeros((3, 3)), damp=0.01)
    with pytest.raises(O.NotPositiveDefinite):
        O.gptq_quantize(np.ones((2, 2)), np.array([[1.0, 2.0], [2.0, 1.0]]), damp=0.0)
    with pytest.raises(O.NonFinite):
        O.gptq_quantize(np.array([[np.nan, 1.0]]), np.eye(2))
    with pytest.raises(O.NonFinite):
        O.hessian(np.array([[np.inf, 1.0]]))
    with pytest.raises(O.InvalidArgument):
        O.gptq_quantize(np.ones((2, 3)), np.eye(3), bits=5)


# ---------------------------------------------------------------------------
# Quality sanity (the method's purpose, not an exact pin).
# ---------------------------------------------------------------------------

def test_gptq_not_worse_than_rtn_on_correlated_inputs():
    rng = np.random.default_rng(90)
    X = rng.standard_normal((1000, 64)) @ rng.standard_normal((64, 64))
    W = 0.02 * rng.standard_normal((32, 64))
    H = O.hessian(X)
    out = O.gptq_quantize(W, H, bits=3, group_size=-1, block=16)
    s, z = O.quant_params(W, 3, False)
    rtn = s[:, None] * (np.clip(np.rint(W / s[:, None]) + z[:, None], 0, 7) - z[:, None])
    assert out["loss"].sum() < 0.5 * O.layer_loss(W, rtn, H).sum()
    out8 = O.gptq_quantize(W, H, bits=8, group_size=-1, block=16)
    assert out8["loss"].sum() < 1e-3 * out["loss"].sum()


# ---------------------------------------------------------------------------
# Product with the packed layer (inference side of the packed format).
# ---------------------------------------------------------------------------

def test_dequant_matmul_hand_example():
    g = _load("dequant_hand.json")
    codes = np.array(g["codes"])
    words = O.pack(codes, g["bits"])
    assert words.shape == (1, 1) and int(words[0, 0]) == int(g["word_hex"], 16)
    n = codes.shape[1]
    g_idx = np.arange(n) // g["group_size"]
    W_hat = O.dequantize(codes, np.array(g["scales"]), np.array(g["zeros"]), g_idx)
    assert np.array_equal(W_hat, np.array(g["w_hat"]))
    for kw in (dict(group_size=g["group_size"]), dict(g_idx=g_idx)):
        y = O.dequant_matmul(np.array(g["x"]), words, g["bits"], n, np.array(g["scales"]),
                             np.array(g["zeros"]), **kw)
        assert np.array_equal(y, np.array(g["y"]))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_matmul_unit_tokens_brute_force(bits):
    # one-hot tokens pick single columns: Y[j, r] is the weight of column j in
    # row r, checked element by element from the integer codes (no unpacking)
    rng = np.random.default_rng(300 + bits)
    d_out, d_in, n_groups = 5, 37, 4
    codes = rng.integers(0, 1 << bits, size=(d_out, d_in))
    g_idx = rng.integers(0, n_groups, size=d_in)
    scales = rng.uniform(0.01, 2.0, size=(n_groups, d_out))
    zeros = rng.integers(0, 1 << bits, size=(n_groups, d_out)).astype(np.float64)
    Y = O.dequant_matmul(np.eye(d_in), O.pack(codes, bits), bits, d_in, scales, zeros, g_idx=g_idx)
    for j in range(d_in):
        for r in range(d_out):
            want = scales[g_idx[j], r] * (int(codes[r, j]) - zeros[g_idx[j], r])
            assert Y[j, r] == want


def test_dequant_matmul_integer_exact():
    # integer activations, unit scales: every sum is an exact integer,
    # compared with Python integers
    rng = np.random.default_rng(311)
    bits, d_out, d_in, gs = 3, 4, 50, 16
    codes = rng.integers(0, 8, size=(d_out, d_in))
    ng = -(-d_in // gs)
    zeros = rng.integers(0, 8, size=(ng, d_out)).astype(np.float64)
    X = rng.integers(-9, 10, size=(3, d_in)).astype(np.float64)
    Y = O.dequant_matmul(X, O.pack(codes, bits), bits, d_in, np.ones((ng, d_out)), zeros, group_size=gs)
    for t in range(3):
        for r in range(d_out):
            want = sum(int(X[t, j]) * (int(codes[r, j]) - int(zeros[j // gs, r])) for j in range(d_in))
            assert Y[t, r] == want


@pytest.mark.parametrize("bits,gs", [(4, 16), (3, 8), (2, -1)])
def test_dequant_matmul_reproduces_solver_weights(bits, gs):
    # the packed words with scales/zeros/g_idx reproduce the weights the
    # column sweep chose (w_hat = scale*(code - zero) taken inside the sweep),
    # in the original order with g_idx and in the sorted order with perm
    rng = np.random.default_rng(320 + bits)
    d_out, d_in = 6, 48
    X = rng.standard_normal((200, d_in)) * np.exp(rng.standard_normal(d_in))
    W = rng.standard_normal((d_out, d_in))
    out = O.gptq_quantize(W, X=X, bits=bits, group_size=gs, act_order=True, block=16)
    assert not np.array_equal(out["perm"], np.arange(d_in))
    want = X @ out["w_hat"].T
    y1 = O.dequant_matmul(X, O.pack(out["codes"], bits), bits, d_in, out["scales"], out["zeros"],
                          g_idx=out["g_idx"])
    y2 = O.dequant_matmul(X, O.pack_permuted(out["codes"], bits, out["perm"]), bits, d_in, out["scales"],
                          out["zeros"], perm=out["perm"], group_size=gs)
    np.testing.assert_allclose(y1, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    np.testing.assert_allclose(y2, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # sorted packing = packing of the permuted code matrix, read back position by position
    back = O.unpack(O.pack_permuted(out["codes"], bits, out["perm"]), bits, d_in)
    assert np.array_equal(back, out["codes"][:, out["perm"]])


# ---------------------------------------------------------------------------
# Layers in sequence.
# ---------------------------------------------------------------------------

def _on_grid_weights(rng, d_out, d_in, s):
    # every row holds codes 0..15 around zero point 8, so min/max of the row
    # map exactly onto the 4-bit grid: quantization (and compensation) is exact
    c = rng.integers(0, 16, size=(d_out, d_in))
    c[:, 0], c[:, 1] = 0, 15
    return s * (c - 8.0)


@pytest.mark.parametrize("act_order", [False, True])
def test_block_chain_reduces_to_float_block_when_lossless(act_order):
    rng = np.random.default_rng(700)
    h, ffn, n = 16, 32, 400
    s = 2.0 ** -6
    Ws = {"q": _on_grid_weights(rng, h, h, s), "k": _on_grid_weights(rng, h, h, s),
          "v": _on_grid_weights(rng, h, h, s), "out": _on_grid_weights(rng, h, h, s),
          "fc1": _on_grid_weights(rng, ffn, h, s), "fc2": _on_grid_weights(rng, h, ffn, s)}
    X = O.round_to_dtype(rng.standard_normal((n, h)), "f16")
    res, inputs, out = O.quantize_block_chain(Ws, X, "f16", bits=4, group_size=-1, act_order=act_order,
                                              block=8, damp=0.01)
    for name in Ws:
        assert np.array_equal(res[name]["w_hat"], Ws[name]), name
    # the float block written out directly
    r16 = lambda a: a.astype(np.float16).astype(np.float64)  # noqa: E731
    A = r16(X @ Ws["v"].T)
    h1 = X + A @ Ws["out"].T
    h1r = r16(h1)
    r = r16(np.maximum(h1r @ Ws["fc1"].T, 0.0))
    want = r16(h1 + r @ Ws["fc2"].T)
    assert np.array_equal(inputs["out"], A)
    assert np.array_equal(inputs["fc1"], h1r)
    assert np.array_equal(inputs["fc2"], r)
    assert np.array_equal(out, want)


def test_round_to_dtype_bf16_ties_and_range():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (even: 1);
    # 1 + 3 * 2^-8 ties up to 1 + 2^-6 (even mantissa)
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5])
    got = O.round_to_dtype(v, "bf16")
    assert np.array_equal(got, [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5])


# ---------------------------------------------------------------------------
# Diagnostics used by the GPU parity tests: tie margins and forced decisions
# ---------------------------------------------------------------------------

def test_tie_margin_hand_values():
    w = np.array([0.25, 0.3, 0.35, -0.25, 0.1])
    s = np.full(5, 0.1)
    # w/scale = 2.5 (tie), 3.0 (grid point), 3.5 (tie), -2.5 (tie), 1.0
    np.testing.assert_allclose(O.tie_margin(w, s), [0.0, 0.5, 0.0, 0.0, 0.5], atol=1e-12)
    np.testing.assert_allclose(O.tie_margin(np.array([0.275]), np.array([0.1])), [0.25], atol=1e-12)


def test_forced_natural_codes_change_nothing():
    rng = np.random.default_rng(21)
    W = rng.normal(0, 0.02, (6, 40))
    H = _rand_pd(rng, 40, 1.0)
    U = O.inverse_hessian_upper(O.damp_hessian(H, 0.01))
    base = O.sweep(W, U, 3, 16, False, 16)
    force = {c: (np.arange(6), base[0][:, c].astype(np.float64)) for c in (0, 7, 19, 39)}
    out = O.sweep(W, U, 3, 16, False, 16, force=force)
    for a, b in zip(base, out):
        np.testing.assert_array_equal(a, b)


def test_forced_code_with_diagonal_hessian_changes_only_that_code():
    # H proportional to I: no compensation, so a forced code changes only
    # itself (and its reconstruction); every other code stays round-to-nearest
    rng = np.random.default_rng(22)
    W = rng.normal(0, 0.02, (4, 32))
    U = O.inverse_hessian_upper(O.damp_hessian(3.0 * np.eye(32), 0.0))
    base = O.sweep(W, U, 4, 16, False, 16)
    c0 = base[0][2, 5]
    alt = c0 + 1 if c0 < 15 else c0 - 1
    out = O.sweep(W, U, 4, 16, False, 16, force={5: (np.array([2]), np.array([float(alt)]))})
    want = base[0].copy()
    want[2, 5] = alt
    np.testing.assert_array_equal(out[0], want)
    assert out[3][2, 5] == pytest.approx(base[1][0, 2] * (alt - base[2][0, 2]), rel=1e-15)


def test_tie_replay_explains_a_planted_tie_and_rejects_a_non_tie():
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from _util import tie_replay
    rng = np.random.default_rng(23)
    W = rng.normal(0, 0.02, (12, 96))
    H = _rand_pd(rng, 96, 1.5)
    U = O.inverse_hessian_upper(O.damp_hessian(H, 0.01))
    base = O.sweep(W, U, 3, 32, False, 32, margins=True)
    codes, m = base[0], base[5]
    inner = (codes > 0) & (codes < 7)
    r, c = np.unravel_index(np.argmin(np.where(inner, m, 1.0)), m.shape)
    alt = codes[r, c] + (1 if W[r, c] > 0 else -1)
    # another sweep that decided (r, c) the other way: explained by one tie
    other_sweep = O.sweep(W, U, 3, 32, False, 32, force={int(c): (np.array([r]), np.array([float(alt)]))})
    rp = tie_replay(O, W, U, other_sweep[0], 3, 32, block=32, tau=max(2 * m[r, c], 1e-12))
    assert rp["other"] == [] and len(rp["ties"]) >= 1 and rp["ties"][0][:2] == (r, c)
    assert np.array_equal(rp["codes"], other_sweep[0])
    # a code off by one far from any tie is not explained
    bad = codes.copy()
    far = np.argmax(np.where(inner, m, -1.0))
    rb, cb = np.unravel_index(far, m.shape)
    bad[rb, cb] += 1
    rp = tie_replay(O, W, U, bad, 3, 32, block=32)
    assert rp["other"] and rp["other"][0][:2] == (rb, cb)


# ---------------------------------------------------------------------------
# Static groups: groups of g consecutive ORIGINAL columns, parameters from the
# untouched weights before the sweep, act-order only ordering the sweep.
# ---------------------------------------------------------------------------

def test_static_groups_hand_examples():
    g = _load("static_groups_hand.json")
    a = g["case_a"]
    out = O.gptq_quantize(np.array(a["W"]), np.diag(a["H_diag"]), bits=a["bits"], group_size=a["group_size"],
                          sym=a["sym"], act_order=a["act_order"], block=a["block"], damp=a["damp"],
                          static_groups=True)
    np.testing.assert_array_equal(out["perm"], a["perm"])
    np.testing.assert_array_equal(out["codes"], a["codes"])
    np.testing.assert_allclose(out["w_hat"], a["w_hat"], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(out["scales"], a["scales"], rtol=1e-15)
    np.testing.assert_array_equal(out["zeros"], a["zeros"])
    np.testing.assert_array_equal(out["g_idx"], a["g_idx"])
    np.testing.assert_allclose(out["row_loss"], a["row_loss"], rtol=1e-13)
    np.testing.assert_allclose(out["loss"], a["loss"], rtol=1e-13)
    # the default grouping of the same problem differs (sweep-order groups)
    dyn = O.gptq_quantize(np.array(a["W"]), np.diag(a["H_diag"]), bits=2, group_size=2, act_order=True)
    assert not np.array_equal(dyn["codes"], out["codes"])

    b = g["case_b"]
    W = np.array(b["W"])
    s, z = O.static_group_params(W, b["bits"], b["group_size"], b["sym"])
    np.testing.assert_allclose(s, b["scales"], rtol=1e-15)
    np.testing.assert_array_equal(z, b["zeros"])
    codes, scales, zeros, w_hat, row_loss = O.sweep(W, np.array(b["U"]), b["bits"], b["group_size"], b["sym"],
                                                    b["block"], static=(s, z, np.array(b["col_group"])))
    np.testing.assert_array_equal(codes, b["codes"])
    np.testing.assert_allclose(w_hat, b["w_hat"], rtol=1e-15)
    np.testing.assert_allclose(row_loss, b["row_loss"], rtol=1e-13)
    np.testing.assert_allclose(scales, b["scales"], rtol=1e-15)


@pytest.mark.parametrize("bits,g,sym", [(4, 16, False), (3, 8, True), (2, 12, False)])
def test_static_groups_diagonal_hessian_is_rtn_in_original_order(bits, g, sym):
    """With nothing to compensate, static groups are plain round-to-nearest
    over consecutive original columns, whatever order the sweep takes."""
    rng = np.random.default_rng(30 + bits)
    W = rng.standard_normal((7, 48))
    dg = rng.permutation(np.arange(1, 49)).astype(float)
    out = O.gptq_quantize(W, np.diag(dg), bits=bits, group_size=g, sym=sym, act_order=True, block=16,
                          static_groups=True)
    np.testing.assert_array_equal(out["codes"], _rtn_in_test(W, bits, g, sym))
    np.testing.assert_array_equal(out["g_idx"], np.arange(48) // g)
    assert not np.array_equal(out["perm"], np.arange(48))


def _grid_in_test(blk, bits, sym):
    maxq = 2 ** bits - 1
    lo = np.minimum(blk.min(1), 0)
    hi = np.maximum(blk.max(1), 0)
    if sym:
        a = np.maximum(-lo, hi)
        a[a == 0] = 1
        return 2 * a / maxq, np.full(len(blk), 2.0 ** (bits - 1))
    both0 = (lo == 0) & (hi == 0)
    lo[both0], hi[both0] = -1, 1
    scale = (hi - lo) / maxq
    return scale, np.rint(-lo / scale)


def _obs_bruteforce_fixed_grid(W, Hd, bits, col_params):
    """Fixed-order OBS with explicit inverses, column q quantized on the given grid."""
    W = W.astype(float).copy()
    d_out, d = W.shape
    maxq = 2 ** bits - 1
    codes = np.zeros((d_out, d), dtype=np.int64)
    qv = np.zeros((d_out, d))
    for q in range(d):
        scale, zero = col_params[q]
        c = np.clip(np.rint(W[:, q] / scale) + zero, 0, maxq)
        val = scale * (c - zero)
        codes[:, q], qv[:, q] = c, val
        F = list(range(q, d))
        Hinv = np.linalg.inv(Hd[np.ix_(F, F)])
        W[:, F] -= np.outer((W[:, q] - val) / Hinv[0, 0], Hinv[:, 0])
        W[:, q] = val
    return codes, qv


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("g", [2, 3])
def test_static_groups_match_bruteforce_obs(seed, g):
    rng = np.random.default_rng(200 + seed)
    d = 4 + seed
    W = rng.standard_normal((5, d))
    H = _rand_pd(rng, d, 0.8)
    for act in (False, True):
        out = O.gptq_quantize(W, H, bits=2, group_size=g, act_order=act, block=2, damp=0.01, static_groups=True)
        perm = out["perm"]
        Hd = O.damp_hessian(H[np.ix_(perm, perm)], 0.01)
        grids = [_grid_in_test(W[:, s:s + g], 2, False) for s in range(0, d, g)]
        col_params = [grids[perm[k] // g] for k in range(d)]
        c_bf, q_bf = _obs_bruteforce_fixed_grid(W[:, perm], Hd, 2, col_params)
        np.testing.assert_array_equal(out["codes"][:, perm], c_bf)
        np.testing.assert_allclose(out["w_hat"][:, perm], q_bf, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(out["g_idx"], np.arange(d) // g)


def test_static_groups_per_row_and_block_invariance():
    """Per-row grouping takes its one group from the untouched row either
    way; and lazy batching still changes nothing."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((300, 40)) @ (rng.standard_normal((40, 40)) / 6)
    W = 0.05 * rng.standard_normal((6, 40))
    for act in (False, True):
        a = O.gptq_quantize(W, X=X, bits=3, group_size=-1, act_order=act, static_groups=True)
        b = O.gptq_quantize(W, X=X, bits=3, group_size=-1, act_order=act)
        np.testing.assert_array_equal(a["codes"], b["codes"])
        ref = O.gptq_quantize(W, X=X, bits=3, group_size=8, act_order=act, block=1, static_groups=True)
        for B in (3, 8, 13, 40):
            out = O.gptq_quantize(W, X=X, bits=3, group_size=8, act_order=act, block=B, static_groups=True)
            np.testing.assert_array_equal(out["codes"], ref["codes"])
