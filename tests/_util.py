"""Helpers shared by the tests (no step of the method lives here)."""
import numpy as np


def to_torch(arr, dtype: str, device="cuda"):
    """Host array in the generator's stored form -> torch tensor of that dtype on device."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def upper_to_full(Hu: np.ndarray) -> np.ndarray:
    """Symmetric matrix from its upper triangle."""
    return np.triu(Hu) + np.triu(Hu, 1).T


def compare_codes(got: np.ndarray, ref: np.ndarray):
    """(fraction identical, max |difference|)."""
    got = got.astype(np.int64)
    ref = ref.astype(np.int64)
    same = float(np.mean(got == ref))
    mx = int(np.abs(got - ref).max()) if got.size else 0
    return same, mx


def tie_replay(O, Wp, U, codes_gpu_p, bits, group_size, sym=False, block=128, tau=1e-4, max_forces=32,
               static=None):
    """Classify GPU-vs-oracle code differences by rounding ties and replay.

    Wp, codes_gpu_p: weights and GPU codes in sweep order (columns permuted
    by perm); U: the oracle's own factor.  Rows are independent given U, so
    the differing rows are replayed together: the oracle sweep is re-run
    taking the GPU's code at each row's first remaining difference, which is
    accepted only if the oracle's value there lies within ``tau`` code units
    of a rounding boundary and the codes differ by one (a tie decided the
    other way); repeated until every row agrees or shows a difference that
    is not such a tie.  Returns a dict:
      same_raw, maxdiff_raw, rows_differing: the raw comparison;
      ties: [(row, col, margin)] forced decisions; other: [(row, col, margin,
      delta)] differences that are not ties (a failure);
      codes, scales, zeros, w_hat, row_loss: the oracle's outputs (sweep
      order) after the replay, every row included.
    ``static``: the oracle sweep's static-groups argument (scales, zeros,
    group of each sweep column), for every row of Wp.
    """
    import numpy as np
    codes_gpu_p = np.asarray(codes_gpu_p).astype(np.int64)
    base = O.sweep(Wp, U, bits, group_size, sym, block, margins=True, static=static)
    codes, scales, zeros, w_hat, row_loss, margin = [np.array(a, copy=True) for a in base]
    same_raw = float(np.mean(codes == codes_gpu_p))
    maxdiff_raw = int(np.abs(codes - codes_gpu_p).max()) if codes.size else 0
    rows = np.nonzero((codes != codes_gpu_p).any(axis=1))[0]
    ties, other = [], []
    if rows.size:
        Wr, gr = Wp[rows], codes_gpu_p[rows]
        st_r = None if static is None else (static[0][:, rows], static[1][:, rows], static[2])
        cr, mr = codes[rows], margin[rows]
        forced = {}                       # column -> {local row: code}
        active = np.ones(rows.size, dtype=bool)
        out = None
        for _ in range(max_forces):
            new = False
            for k in np.nonzero(active)[0]:
                d = np.nonzero(cr[k] != gr[k])[0]
                if d.size == 0:
                    active[k] = False
                    continue
                c = int(d[0])
                delta = int(gr[k, c] - cr[k, c])
                m = float(mr[k, c])
                if abs(delta) != 1 or m >= tau or c in forced and k in forced[c]:
                    other.append((int(rows[k]), c, m, delta))
                    active[k] = False
                    continue
                ties.append((int(rows[k]), c, m))
                forced.setdefault(c, {})[k] = float(gr[k, c])
                new = True
            if not new:
                break
            force = {c: (np.array(list(v)), np.array(list(v.values()))) for c, v in forced.items()}
            out = O.sweep(Wr, U, bits, group_size, sym, block, force=force, margins=True, static=st_r)
            cr, mr = out[0], out[5]
        if out is not None:
            codes[rows], w_hat[rows], row_loss[rows] = out[0], out[3], out[4]
            scales[:, rows], zeros[:, rows] = out[1], out[2]
    return dict(same_raw=same_raw, maxdiff_raw=maxdiff_raw, rows_differing=int(rows.size), ties=ties,
                other=other, codes=codes, scales=scales, zeros=zeros, w_hat=w_hat, row_loss=row_loss)


def assert_from_x_parity(O, W64, H, got, bits, group_size, act_order, sym=False, block=128, damp=0.01, name="",
                         static_groups=False):
    """The GPU layer (got: original-order outputs) against the oracle run from
    the same activations' float64 Hessian H, step by step as the oracle's
    gptq_quantize takes them (order, damping, U, sweep): every differing code
    is a rounding tie decided the other way (or follows from one in its row,
    as the replay shows); after the replay the codes are identical, scales
    within 1e-5 relative, zero points equal, and the layer loss within 1e-3
    relative.  Returns the replay summary (raw numbers included).
    ``static_groups``: the static-groups option (groups of original columns,
    parameters from W64 as given)."""
    import time

    import numpy as np
    t0 = time.time()
    d_in = H.shape[0]
    perm = O.act_order_permutation(H) if act_order else np.arange(d_in)
    assert np.array_equal(np.asarray(got["perm"]).astype(np.int64), perm), name
    U = O.inverse_hessian_upper(O.damp_hessian(H[np.ix_(perm, perm)], damp))
    print(f"{name}: oracle order and U in {time.time() - t0:.1f} s", flush=True)
    static = None
    if static_groups and group_size > 0:
        st_s, st_z = O.static_group_params(W64, bits, group_size, sym)
        static = (st_s, st_z, perm // group_size)
        assert np.array_equal(np.asarray(got["g_idx"]), np.arange(d_in) // group_size), name
    t0 = time.time()
    rp = tie_replay(O, W64[:, perm], U, np.asarray(got["codes"])[:, perm], bits, group_size, sym, block,
                    static=static)
    print(f"{name}: oracle sweep of {W64.shape[0]} rows and tie replay in {time.time() - t0:.1f} s", flush=True)
    assert not rp["other"], (name, rp["other"][:5])
    assert np.array_equal(rp["codes"], np.asarray(got["codes"])[:, perm].astype(np.int64)), name
    sc_g = np.asarray(got["scales"]).astype(np.float64)
    np.testing.assert_allclose(sc_g, rp["scales"], rtol=1e-5, atol=0, err_msg=name)
    np.testing.assert_array_equal(np.asarray(got["zeros"]).astype(np.float64), rp["zeros"], err_msg=name)
    base = O.sweep(W64[:, perm], U, bits, group_size, sym, block, static=static) if rp["rows_differing"] else None
    loss_g = O.layer_loss(W64, np.asarray(got["w_hat"]).astype(np.float64), H).sum()
    w_hat_o = np.empty_like(rp["w_hat"])
    w_hat_o[:, perm] = rp["w_hat"]
    loss_o = O.layer_loss(W64, w_hat_o, H).sum()
    if base is not None:
        w_raw = np.empty_like(base[3])
        w_raw[:, perm] = base[3]
        loss_raw = O.layer_loss(W64, w_raw, H).sum()
    else:
        loss_raw = loss_o
    assert abs(loss_g - loss_o) <= 1e-3 * loss_o, (name, loss_g, loss_o)
    rp.update(loss_gpu=float(loss_g), loss_replayed=float(loss_o), loss_oracle=float(loss_raw))
    print(f"{name}: identical {rp['same_raw']:.6f} (max diff {rp['maxdiff_raw']}, rows differing "
          f"{rp['rows_differing']}, ties replayed {len(rp['ties'])}, min tie margin "
          f"{min([t[2] for t in rp['ties']], default=float('nan')):.2e}); loss gpu {loss_g:.6g} oracle "
          f"{loss_raw:.6g} replayed {loss_o:.6g}", flush=True)
    return rp
