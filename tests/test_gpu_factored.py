"""The factored form of the solver (prepare_hinv_factored and
quantize_layer_factored) against the fp64 oracle (needs an MI355X).

The factored form keeps U's diagonal 128-blocks and replaces its
off-diagonal blocks by F[K_k, K_l] = R[K_k, K_l] U_ll with R = U^{-1}; the
lazy updates then add (W0 - Q) F instead of subtracting Err U.  The
expected F is formed here from the oracle's U (R by triangular solves in
float64), never from the GPU's.  The sweep's codes are decided in float64 on
both sides but from differently rounded running weights, so the bar for
codes is the tie bar: every difference is a rounding tie decided the other
way or follows from one in its row (tie replay), and after the replay codes
are identical, scales within 1e-5 relative and zero points equal.
"""
import numpy as np
import pytest
import scipy.linalg as sla
import torch

import oracle as O
import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import synth

from _util import assert_from_x_parity, tie_replay, to_torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
B = 128


def _layer(d_out, d_in, n_tok, dtype="bf16", seed=1, frac=0.01, scale=30.0):
    return synth.make_layer(d_out, d_in, n_tok, dtype=dtype, sigma_w=0.02, dist="t4", outlier_frac=frac,
                            outlier_scale=scale, config=91, layer=seed)


def _oracle_u(H, act, damp=0.01):
    perm = O.act_order_permutation(H) if act else np.arange(H.shape[0])
    return perm, O.inverse_hessian_upper(O.damp_hessian(H[np.ix_(perm, perm)], damp))


def _f_block(U, R_cols, k, l):
    """F[K_k, K_l] = R[K_k, K_l] U[K_l, K_l] (k < l), or U's block (k == l)."""
    if k == l:
        return U[k * B:(k + 1) * B, l * B:(l + 1) * B]
    return R_cols[l][k * B:(k + 1) * B] @ U[l * B:(l + 1) * B, l * B:(l + 1) * B]


def _r_cols(U, blocks):
    """Block columns of R = U^{-1} (one triangular solve each)."""
    d = U.shape[0]
    out = {}
    for l in blocks:
        E = np.zeros((d, B))
        E[l * B:(l + 1) * B] = np.eye(B)
        out[l] = sla.solve_triangular(U, E, lower=False)
    return out


def _f_reference(U):
    nb = U.shape[0] // B
    Rc = _r_cols(U, range(nb))
    F = np.zeros_like(U)
    for l in range(nb):
        for k in range(l + 1):
            F[k * B:(k + 1) * B, l * B:(l + 1) * B] = _f_block(U, Rc, k, l)
    return F


def _assert_f_close(Fg, Fr, rtol=1e-9):
    nb = Fr.shape[0] // B
    for l in range(nb):
        for k in range(l + 1):
            r = Fr[k * B:(k + 1) * B, l * B:(l + 1) * B]
            g = Fg[k * B:(k + 1) * B, l * B:(l + 1) * B]
            err = np.abs(g - r).max() / max(np.abs(r).max(), 1e-300)
            assert err <= rtol, (k, l, err)
    assert np.all(np.tril(Fg, -1) == 0.0)


# ---------------------------------------------------------------------------
# prepare_hinv_factored: F against the oracle's U
# ---------------------------------------------------------------------------

# d / 128 leaves: one leaf; small nodes only (<= 8 leaves, where the
# recursion's right spine skips its inverse products inside one launch
# pair); odd leaf counts; nodes above 512 + 512 (side stream, T products on
# the left children only)
@pytest.mark.parametrize("d,act", [(128, True), (256, False), (384, True), (640, True), (1152, False),
                                   (2048, True), (3200, True)])
def test_prepare_factored_matches_oracle(d, act):
    print(f"prepare factored d={d} act={act}", flush=True)
    L = _layer(4, d, 3 * d, dtype="f32", seed=d + 3, frac=0.0)
    H = O.hessian(L.X_f64())
    cfg = P.make_config(act_order=act, damp=0.01)
    Hg = torch.from_numpy(np.triu(H)).to(DEV)
    perm_g = P.prepare_hinv_factored(Hg, cfg)
    torch.cuda.synchronize()
    perm, U = _oracle_u(H, act)
    assert np.array_equal(perm_g.cpu().numpy(), perm)
    _assert_f_close(Hg.cpu().numpy(), _f_reference(U))


def test_prepare_factored_rejects_ragged_width():
    H = torch.eye(200, dtype=torch.float64, device=DEV)
    with pytest.raises(P.Unsupported):
        P.prepare_hinv_factored(H, P.make_config())


# ---------------------------------------------------------------------------
# quantize_layer_factored fed F formed from the oracle's U
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,bits,g,act,sym,static", [
    (100, 384, 4, 128, True, False, False),
    (64, 256, 4, -1, False, False, False),
    (130, 640, 3, 64, True, False, False),
    (70, 512, 2, 32, False, False, False),
    (40, 768, 4, 16, True, True, False),     # symmetric: every group's largest weight sits on a tie
    (33, 384, 8, 8, True, False, False),
    (96, 1152, 4, 128, True, False, False),  # superblocks: far updates on the second stream
    (48, 2304, 3, 128, False, False, False),
    (64, 640, 4, 256, True, False, True),    # static groups wider than a block
    (50, 1024, 4, 64, True, True, True),
])
def test_factored_sweep_matches_oracle_given_u(d_out, d_in, bits, g, act, sym, static):
    print(f"factored sweep {d_out}x{d_in} b{bits} g{g} act{act} sym{sym} static{static}", flush=True)
    L = _layer(d_out, d_in, max(2 * d_in, 1000), seed=d_in + bits)
    H = O.hessian(L.X_f64())
    perm, U = _oracle_u(H, act)
    F = _f_reference(U)
    cfg = P.make_config(bits=bits, group_size=g, sym=sym, act_order=act, block=B, static_groups=static)
    out = P.quantize_layer_factored(to_torch(L.W, "bf16"), torch.from_numpy(F).to(DEV),
                                    torch.from_numpy(perm.astype(np.int32)).to(DEV), cfg)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    W64 = L.W_f64()
    st = None
    if static and g > 0:
        st_s, st_z = O.static_group_params(W64, bits, g, sym)
        st = (st_s, st_z, perm // g)
    rp = tie_replay(O, W64[:, perm], U, got["codes"][:, perm], bits, g, sym, B, static=st)
    print(f"  identical {rp['same_raw']:.6f}, rows differing {rp['rows_differing']}, ties {len(rp['ties'])}",
          flush=True)
    assert not rp["other"], rp["other"][:5]
    assert np.array_equal(rp["codes"], got["codes"][:, perm].astype(np.int64))
    np.testing.assert_allclose(got["scales"].astype(np.float64), rp["scales"], rtol=1e-5, atol=0)
    np.testing.assert_array_equal(got["zeros"].astype(np.float64), rp["zeros"])
    ref_gidx = np.arange(d_in) // g if (static and g > 0) else (
        np.argsort(perm) // g if g > 0 else np.zeros(d_in, np.int64))
    assert np.array_equal(got["g_idx"], ref_gidx)
    np.testing.assert_allclose(got["row_loss"], rp["row_loss"], rtol=1e-9)
    if not sym:
        # no group has a weight on a tie by construction: the codes are the oracle's
        assert rp["same_raw"] == 1.0


# ---------------------------------------------------------------------------
# end to end from X through the factored form
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,n,dtype,bits,g,act", [
    (192, 640, 8192, "bf16", 4, 128, True),
    (150, 768, 8192, "f16", 3, 128, False),
    (96, 1152, 6000, "bf16", 2, 64, True),
    (64, 2304, 9000, "bf16", 4, -1, True),
])
def test_factored_end_to_end(d_out, d_in, n, dtype, bits, g, act):
    print(f"factored e2e {d_out}x{d_in} n={n} {dtype} b{bits} g{g} act{act}", flush=True)
    L = _layer(d_out, d_in, n, dtype=dtype, seed=d_in + 7, frac=0.005, scale=50.0)
    cfg = P.make_config(bits=bits, group_size=g, act_order=act)
    out = P.quantize(to_torch(L.W, dtype), X=to_torch(L.X, dtype), cfg=cfg, factored=True)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    H = O.hessian(L.X_f64())
    rp = assert_from_x_parity(O, L.W_f64(), H, got, bits, g, act, name=f"factored {d_out}x{d_in}")
    assert rp["same_raw"] >= 0.999 and rp["maxdiff_raw"] <= 1
    assert np.array_equal(got["packed"].view(np.uint32), O.pack(got["codes"], bits))


def test_factored_and_u_paths_agree_on_gpu_hessian():
    """Both forms from one GPU Hessian: same order, U's diagonal blocks, and
    the same codes (asymmetric 4-bit: no weight on a tie)."""
    L = _layer(256, 1536, 8192, seed=5)
    X = to_torch(L.X, "bf16")
    H = torch.zeros((1536, 1536), dtype=torch.float64, device=DEV)
    P.hessian_accumulate(H, X)
    cfg = P.make_config(bits=4, group_size=128, act_order=True)
    W = to_torch(L.W, "bf16")
    a = P.quantize(W, H=H.clone(), cfg=cfg, factored=False)
    b = P.quantize(W, H=H.clone(), cfg=cfg, factored=True)
    torch.cuda.synchronize()
    for k in ("perm", "codes", "g_idx", "zeros"):
        assert torch.equal(a[k], b[k]), k
    torch.testing.assert_close(b["scales"], a["scales"], rtol=1e-6, atol=0)
    torch.testing.assert_close(b["row_loss"], a["row_loss"], rtol=1e-9, atol=0)
