"""GPTQ per-layer quantization solver -- plain fp64 oracle (numpy / LAPACK).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources, cited by page title and section:

* "GPTQ量化算法深度解析：从Hessian曲率到大模型单卡部署" (sheratonhq.com) --
  §2.1 (second-order objective), §2.2 (OBS compensation formula), §2.4
  (fixed order, lazy batch update, Cholesky), §3.1 (the four-step per-layer
  flow: H = 2XX^T + lambda*I, Cholesky, blocks of 128 columns with
  per-column scale / round / error accumulation and one update of the later
  columns per block, save codes + scale/zero), §3.3 (group size, desc_act,
  damp_percent = 0.01).
* "通义千问1.5-1.8B-Chat-GPTQ-Int4模型压缩技术解析" (deepseek.csdn.net) --
  §2.1 (min/max range split into 2^b levels), §2.2 (scale and zero point per
  layer or group).
* ai.lansai.wang GPTQ guide, section "bits、group_size、sym 与 desc_act
  分别影响什么" (the quantize_config field table).
* "gptq-for-llama" article (ainews.cool), "工程细节" (four 4-bit codes packed
  per 16-bit integer; matrix products run on the packed codes).
* Inference with the packed layer: "通义千问..." §2.2 (codes are turned back
  into weights with their group's scale and zero point for the computation)
  and "GPTQ量化算法深度解析" §3.3 (act-order costs a gather at inference).

Notation: W is d_out x d_in (row = output channel, column = input channel);
X is tokens x d_in; b = bits, maxq = 2^b - 1; g = group size; B = block size.

Readings taken where the pages are silent or garbled (each is listed in the
design notes of the repository):

* H is the sum 2 * sum_t x_t x_t^T (no mean); lambda = damp * mean(diag H)
  is added to every diagonal entry.
* The compensation uses U, the upper Cholesky factor of H_d^{-1}
  (H_d^{-1} = U^T U): err_c = (w_c - q_c) / U_cc and w_j -= err_c * U_cj for
  the later columns j, which is the OBS update of §2.2 with the quantized
  value restored in its numerator.
* Asymmetric grid: xmin = min(0, min w), xmax = max(0, max w) over the
  group's current values, scale = (xmax - xmin)/maxq, zero = rint(-xmin/scale);
  an all-zero group uses xmin = -1, xmax = +1.  Symmetric grid:
  amax = max(|xmin|, xmax) (1 if zero), scale = 2*amax/maxq, zero = 2^(b-1).
* code = clip(rint(w / scale) + zero, 0, maxq) with round-half-to-even and a
  true division; q = scale * (code - zero).
* Group parameters are taken when the sweep reaches the group's first column,
  from the group's current (already compensated) values; per-row
  quantization is one group per row, taken at column 0.
* act-order: perm = stable argsort of -diag(H) (undamped H); groups are g
  consecutive columns in sweep order; g_idx[perm[k]] = k // g.
* Static groups (an option; the field table's desc_act row notes that the
  order choice can change compatibility and execution cost, and
  "GPTQ量化算法深度解析" §3.3 says act-order costs a gather at inference):
  groups are g consecutive columns in the ORIGINAL order, g_idx[j] = j // g,
  and every group's (scale, zero) is taken before the sweep from the
  weights as given (nothing compensated yet); act-order then only decides
  the order of the sweep, and each column is quantized with the parameters
  of its original-order group.
* Outputs are returned in the original column order.
* Packing: each output row is a little-endian bit stream along d_in; code k
  occupies bits [b*k, b*k + b) of that stream, held in 32-bit words.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


class NotPositiveDefinite(ArithmeticError):
    """The damped Hessian is not positive definite (Cholesky failed)."""


class NonFinite(ArithmeticError):
    """An input held NaN or Inf."""


class InvalidArgument(ValueError):
    """Shapes or configuration outside what the method defines."""


# ---------------------------------------------------------------------------
# Step 1: the Hessian of the layer-reconstruction objective.
# ---------------------------------------------------------------------------

def hessian(X) -> np.ndarray:
    """H = 2 * X^T X in float64, X given tokens-major (n_tok x d_in).

    "GPTQ量化算法深度解析" §3.1 step 1 writes H = 2XX^T + lambda*I with X laid
    out d_in x tokens; the same matrix is 2 * sum_t x_t x_t^T.  The damping
    term is applied separately (damp_hessian).  ``X`` may be one array or an
    iterable of token chunks; every chunk is widened to float64 exactly before
    the product, so bf16/fp16/fp32 inputs lose nothing on the way in.
    """
    chunks = [X] if isinstance(X, np.ndarray) else X
    H = None
    for chunk in chunks:
        x = np.asarray(chunk, dtype=np.float64)
        if x.ndim != 2:
            raise InvalidArgument("X must be 2-D (tokens x d_in)")
        if not np.all(np.isfinite(x)):
            raise NonFinite("X holds NaN or Inf")
        if H is None:
            H = np.zeros((x.shape[1], x.shape[1]), dtype=np.float64)
        H += 2.0 * (x.T @ x)
    if H is None:
        raise InvalidArgument("no token chunks given")
    return H


# ---------------------------------------------------------------------------
# act-order (desc_act): the column order.
# ---------------------------------------------------------------------------

def act_order_permutation(H: np.ndarray) -> np.ndarray:
    """Column order for act-order: descending diag(H), ties to the lower index.

    "GPTQ量化算法深度解析" §3.3 (desc_act): the columns are processed in order
    of their activation magnitude, most influential first.  The key is
    diag(H)_j = 2 * sum_t x_tj^2, the channel's activation energy, taken from
    the undamped H (damping shifts every key equally).  perm[k] is the
    original index of the k-th swept column.
    """
    return np.argsort(-np.diag(H), kind="stable").astype(np.int64)


# ---------------------------------------------------------------------------
# Step 2: damping and the Cholesky form of the inverse Hessian.
# ---------------------------------------------------------------------------

def damp_hessian(H: np.ndarray, damp: float) -> np.ndarray:
    """H_d = H + lambda * I with lambda = damp * mean(diag H).

    "GPTQ量化算法深度解析" §3.1 step 1 (the lambda*I term keeps H invertible
    and stable) and §3.3 (damp_percent is a ratio on the diagonal, default
    0.01, raised to 0.1 when H is near-singular).
    """
    d = H.shape[0]
    lam = damp * np.mean(np.diag(H))
    return H + lam * np.eye(d)


def inverse_hessian_upper(Hd: np.ndarray) -> np.ndarray:
    """U, upper triangular with positive diagonal, such that H_d^{-1} = U^T U.

    "GPTQ量化算法深度解析" §2.4 (a Cholesky factorisation replaces repeated,
    unstable inversion) and §3.1 step 2 (factor H once, lower triangular, and
    reuse the factor).  Taken in three plain steps: L = chol(H_d) lower;
    H_d^{-1} = L^{-T} L^{-1}; U = chol(H_d^{-1})^T.
    """
    if not np.all(np.isfinite(Hd)):
        raise NonFinite("H holds NaN or Inf")
    try:
        L = np.linalg.cholesky(Hd)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from None
    d = Hd.shape[0]
    Linv = scipy.linalg.solve_triangular(L, np.eye(d), lower=True)
    Hinv = Linv.T @ Linv
    try:
        Lh = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from None
    return np.ascontiguousarray(Lh.T)


# ---------------------------------------------------------------------------
# Step 3: the quantizer (scale / zero, rounding).
# ---------------------------------------------------------------------------

def quant_params(wg: np.ndarray, bits: int, sym: bool):
    """Per-row (scale, zero) of one group, wg being d_out x (group width).

    "通义千问...GPTQ-Int4..." §2.1: take the range from min and max and split it
    into 2^b equal levels; §2.2: one scale and zero point per layer or group.
    ai.lansai.wang guide, field table: ``sym`` picks a range symmetric about 0
    or an asymmetric one with a zero point.
    """
    maxq = 2 ** bits - 1
    xmin = np.minimum(wg.min(axis=1), 0.0)
    xmax = np.maximum(wg.max(axis=1), 0.0)
    if sym:
        amax = np.maximum(np.abs(xmin), xmax)
        amax = np.where(amax == 0.0, 1.0, amax)
        scale = 2.0 * amax / maxq
        zero = np.full_like(scale, float(2 ** (bits - 1)))
    else:
        dead = (xmin == 0.0) & (xmax == 0.0)
        xmin = np.where(dead, -1.0, xmin)
        xmax = np.where(dead, 1.0, xmax)
        scale = (xmax - xmin) / maxq
        zero = np.rint(-xmin / scale)
    return scale, zero


def quantize_column(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int):
    """code = clip(rint(w/scale) + zero, 0, maxq); q = scale * (code - zero).

    "GPTQ量化算法深度解析" §3.1 step 3 (round the column to the grid) and
    "通义千问...GPTQ-Int4..." §2.2 (dequantize with scale and zero point).
    """
    maxq = 2 ** bits - 1
    code = np.clip(np.rint(w / scale) + zero, 0.0, float(maxq))
    q = scale * (code - zero)
    return code, q


def tie_margin(w: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Distance of w/scale from the nearest rounding boundary (a
    half-integer), in code units: 0 at an exact tie, 1/2 on a grid point.

    Diagnostic for comparing two implementations: a code can only differ
    between two correct sweeps whose compensated values differ by rounding
    if this margin is that small.
    """
    y = w / scale
    return 0.5 - np.abs(y - np.rint(y))


# ---------------------------------------------------------------------------
# Step 3: the blocked column sweep with error compensation.
# ---------------------------------------------------------------------------

def _check_block_group(d_in: int, group_size: int, block: int) -> int:
    """Effective group width; per-row (group_size <= 0) is one group per row.
    Any positive block works with any group width (lazy batching is exact)."""
    if block <= 0:
        raise InvalidArgument("block size must be positive")
    if group_size <= 0:
        return d_in
    return group_size


def static_group_params(W: np.ndarray, bits: int, group_size: int, sym: bool):
    """(scales, zeros), each [n_groups][d_out], of the static-groups option:
    group G holds original columns G*g .. min((G+1)*g, d_in) - 1 and takes
    its parameters from W as given, before the sweep (reading stated in the
    module docstring; the grid itself is quant_params')."""
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    g = d_in if group_size <= 0 else group_size
    n_groups = -(-d_in // g)
    scales = np.zeros((n_groups, d_out))
    zeros = np.zeros((n_groups, d_out))
    for G in range(n_groups):
        scales[G], zeros[G] = quant_params(W[:, G * g:min((G + 1) * g, d_in)], bits, sym)
    return scales, zeros


def sweep(W: np.ndarray, U: np.ndarray, bits: int, group_size: int, sym: bool,
          block: int = 128, force=None, margins: bool = False, static=None):
    """Quantize the columns of W (already in sweep order) left to right.

    "GPTQ量化算法深度解析" §2.4 (fixed order; lazy batch update: errors are
    collected inside a block and the later columns updated once per block)
    and §3.1 step 3 (blocks of 128 columns; inside a block, per column:
    scale, round, accumulate the error; after the block, one update of the
    later columns).  The per-column compensation is §2.2's OBS update written
    with U (upper Cholesky factor of H_d^{-1}).

    Returns (codes, scales, zeros, w_hat, row_loss), all in sweep order;
    scales/zeros are [n_groups][d_out]; row_loss[r] = sum_c (w_c - q_c)^2 /
    (2 U_cc^2).

    Two diagnostics for comparisons with another implementation (they leave
    the arithmetic above untouched): ``margins=True`` appends the tie margin
    of every code (tie_margin of the value quantized, d_out x d_in);
    ``force`` maps a sweep column c to (rows, codes): those rows take the
    given codes at column c instead of their rounded value, and the sweep
    continues from the resulting quantized value, which replays another
    implementation's decision at a rounding tie.

    ``static = (scales, zeros, col_group)`` selects the static-groups option:
    sweep column c is quantized with scales[col_group[c]], zeros[col_group[c]]
    (fixed before the sweep, see static_group_params) and no parameters are
    taken during the sweep; the returned scales / zeros are the given ones.
    """
    if bits not in (2, 3, 4, 8):
        raise InvalidArgument("bits must be 2, 3, 4 or 8")
    W = np.array(W, dtype=np.float64, copy=True)
    d_out, d_in = W.shape
    g = _check_block_group(d_in, group_size, block)
    n_groups = -(-d_in // g)
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    w_hat = np.zeros((d_out, d_in), dtype=np.float64)
    scales = np.zeros((n_groups, d_out), dtype=np.float64)
    zeros = np.zeros((n_groups, d_out), dtype=np.float64)
    row_loss = np.zeros(d_out, dtype=np.float64)
    margin = np.zeros((d_out, d_in), dtype=np.float64) if margins else None
    scale = zero = None
    if static is not None:
        st_scales, st_zeros, col_group = static
        scales = np.array(st_scales, dtype=np.float64, copy=True)
        zeros = np.array(st_zeros, dtype=np.float64, copy=True)

    for i1 in range(0, d_in, block):
        i2 = min(i1 + block, d_in)
        W1 = W[:, i1:i2].copy()              # the block being swept
        Err = np.zeros((d_out, i2 - i1))     # accumulated scaled errors
        for c in range(i1, i2):
            k = c - i1
            if static is not None:
                scale, zero = scales[col_group[c]], zeros[col_group[c]]
            elif c % g == 0:
                # The group's current values: the part inside this block sits
                # in W1 (already compensated by earlier columns of the block);
                # the part past the block sits in W, which holds every earlier
                # block's lazy update but not yet this block's, so the errors
                # of this block's finished columns are applied to it here.
                # Lazy batching thus stays exactly the per-column algorithm
                # for any block size, also when a group crosses the block end.
                end = min(c + g, d_in)
                past = W[:, i2:max(end, i2)] - Err[:, :k] @ U[i1:c, i2:max(end, i2)]
                cur = np.hstack([W1[:, k:min(end, i2) - i1], past])
                scale, zero = quant_params(cur, bits, sym)
                scales[c // g] = scale
                zeros[c // g] = zero
            w = W1[:, k]
            code, q = quantize_column(w, scale, zero, bits)
            if margins:
                margin[:, c] = tie_margin(w, scale)
            if force is not None and c in force:
                rows, fc = force[c]
                code[rows] = fc
                q[rows] = scale[rows] * (code[rows] - zero[rows])
            codes[:, c] = code.astype(np.int64)
            w_hat[:, c] = q
            ucc = U[c, c]
            err = (w - q) / ucc
            W1[:, k + 1:] -= np.outer(err, U[c, c + 1:i2])
            Err[:, k] = err
            row_loss += (w - q) ** 2 / (2.0 * ucc * ucc)
        # lazy batch update of every later column
        W[:, i2:] -= Err @ U[i1:i2, i2:]
    if margins:
        return codes, scales, zeros, w_hat, row_loss, margin
    return codes, scales, zeros, w_hat, row_loss


# ---------------------------------------------------------------------------
# The whole per-layer solver (steps 1-4).
# ---------------------------------------------------------------------------

def gptq_quantize(W, H=None, *, X=None, bits=4, group_size=128, sym=False,
                  act_order=False, block=128, damp=0.01, static_groups=False):
    """Quantize one linear layer; returns a dict of outputs in original order.

    "GPTQ量化算法深度解析" §3.1 (the four steps per layer) with §3.3's
    options.  Give either H (d_in x d_in, the undamped 2 X^T X) or X.

    Keys: codes (int64 d_out x d_in), scales / zeros ([n_groups][d_out]),
    g_idx (d_in), perm (d_in, perm[k] = original column swept k-th), w_hat
    (d_out x d_in), row_loss (sum_c (w_c-q_c)^2 / (2 U_cc^2) per row),
    loss (||(W - W_hat) X^T||_F^2 = 1/2 tr(dW H dW^T) with the undamped H),
    U (sweep order), H (undamped, original order).  ``static_groups``: the
    static-groups option (module docstring): g_idx[j] = j // g.
    """
    W0 = np.asarray(W, dtype=np.float64)
    if W0.ndim != 2:
        raise InvalidArgument("W must be 2-D")
    if not np.all(np.isfinite(W0)):
        raise NonFinite("W holds NaN or Inf")
    if H is None:
        if X is None:
            raise InvalidArgument("give H or X")
        H = hessian(X)
    H = np.asarray(H, dtype=np.float64)
    d_out, d_in = W0.shape
    if H.shape != (d_in, d_in):
        raise InvalidArgument("H must be d_in x d_in")
    if not np.all(np.isfinite(H)):
        raise NonFinite("H holds NaN or Inf")

    if act_order:
        perm = act_order_permutation(H)
    else:
        perm = np.arange(d_in, dtype=np.int64)
    Wp = W0[:, perm]
    Hp = H[np.ix_(perm, perm)]

    U = inverse_hessian_upper(damp_hessian(Hp, damp))
    g = d_in if group_size <= 0 else group_size
    static = None
    if static_groups:
        st_scales, st_zeros = static_group_params(W0, bits, group_size, sym)
        static = (st_scales, st_zeros, perm // g)
    codes_s, scales, zeros, w_hat_s, row_loss = sweep(Wp, U, bits, group_size, sym, block, static=static)

    codes = np.empty_like(codes_s)
    w_hat = np.empty_like(w_hat_s)
    codes[:, perm] = codes_s
    w_hat[:, perm] = w_hat_s
    g_idx = np.empty(d_in, dtype=np.int64)
    if static_groups:
        g_idx[:] = np.arange(d_in) // g
    else:
        g_idx[perm] = np.arange(d_in) // g
    return dict(codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, perm=perm,
                w_hat=w_hat, row_loss=row_loss, loss=layer_loss(W0, w_hat, H),
                U=U, H=H)


def dequantize(codes, scales, zeros, g_idx) -> np.ndarray:
    """W_hat[r, j] = scale[g_idx[j], r] * (code[r, j] - zero[g_idx[j], r]).

    "通义千问...GPTQ-Int4..." §2.2 (dequantize back with scale and zero point);
    "GPTQ量化算法深度解析" §3.3 (act-order needs a gather at inference, here
    the g_idx lookup).
    """
    codes = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)[np.asarray(g_idx)].T
    z = np.asarray(zeros, dtype=np.float64)[np.asarray(g_idx)].T
    return s * (codes - z)


def layer_loss(W, W_hat, H) -> np.ndarray:
    """Per-row reconstruction error 1/2 * (w - w_hat) H (w - w_hat)^T.

    With H = 2 X^T X this is ||(w - w_hat) X^T||^2, the layer-output error
    that "GPTQ量化算法深度解析" §2.1 puts at the centre of the objective.
    """
    dW = np.asarray(W_hat, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    # row r: 1/2 * (dW H)_r . dW_r, the product dW H by the library's matmul
    return 0.5 * np.einsum("ij,ij->i", dW @ np.asarray(H, dtype=np.float64), dW)


# ---------------------------------------------------------------------------
# Step 4: packing.
# ---------------------------------------------------------------------------

def words_per_row(d_in: int, bits: int) -> int:
    return -(-(d_in * bits) // 32)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes into little-endian bit streams of 32-bit words.

    "gptq-for-llama" article, "工程细节": four 4-bit codes share one 16-bit
    integer.  Generalised to b bits: per output row, code k occupies bits
    [b*k, b*k + b) of a bit stream whose bit 0 is the LSB of word 0; a 3-bit
    code may straddle two words.  Returns uint32 [d_out][words_per_row].
    """
    if bits not in (2, 3, 4, 8):
        raise InvalidArgument("bits must be 2, 3, 4 or 8")
    c = np.asarray(codes)
    if c.min(initial=0) < 0 or c.max(initial=0) >= (1 << bits):
        raise InvalidArgument("code outside [0, 2^bits)")
    d_out, d_in = c.shape
    nw = words_per_row(d_in, bits)
    out = np.zeros((d_out, nw), dtype=np.uint64)
    c = c.astype(np.uint64)
    for k in range(d_in):
        pos = bits * k
        wi, sh = divmod(pos, 32)
        out[:, wi] |= (c[:, k] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            out[:, wi + 1] |= c[:, k] >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    """Inverse of pack: read code k from bits [b*k, b*k + b) of the row stream."""
    w = np.asarray(words).astype(np.uint64)
    d_out = w.shape[0]
    out = np.zeros((d_out, d_in), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for k in range(d_in):
        pos = bits * k
        wi, sh = divmod(pos, 32)
        v = w[:, wi] >> np.uint64(sh)
        if sh + bits > 32:
            v |= w[:, wi + 1] << np.uint64(32 - sh)
        out[:, k] = (v & mask).astype(np.int64)
    return out


# ---------------------------------------------------------------------------
# Inference: the product with the packed layer.
# ---------------------------------------------------------------------------

def pack_permuted(codes: np.ndarray, bits: int, perm) -> np.ndarray:
    """Pack the columns in the order perm: stream position k of every row
    holds the code of column perm[k].

    With act-order ("GPTQ量化算法深度解析" §3.3) the columns of one group are
    scattered over the original order; in the quantization order they are
    consecutive again, and inference gathers the activations instead.
    """
    return pack(np.asarray(codes)[:, np.asarray(perm)], bits)


def dequant_matmul(X, words, bits: int, d_in: int, scales, zeros, *, g_idx=None,
                   perm=None, group_size: int = -1) -> np.ndarray:
    """Y = X W_hat^T with W_hat read back from packed words, in float64.

    "通义千问..." §2.2: the integer codes with the per-group scale and zero
    point are turned back into weights (W_hat = scale * (code - zero)) for the
    computation, the activations keep their precision; "gptq-for-llama"
    article, "工程细节": the product runs on the packed codes.

    Stream position k of a packed row holds the code of activation column
    a(k), in group g(k):
      g_idx given:  a(k) = k,       g(k) = g_idx[k]   (original order);
      perm given:   a(k) = perm[k], g(k) = k // group_size (sorted order);
      neither:      a(k) = k,       g(k) = k // group_size.
    group_size <= 0 (or >= d_in) means one group.  X: tokens x d_in.
    """
    if g_idx is not None and perm is not None:
        raise InvalidArgument("give g_idx or perm, not both")
    codes = unpack(words, bits, d_in)
    k = np.arange(d_in)
    if g_idx is not None:
        g = np.asarray(g_idx, dtype=np.int64)
    elif 0 < group_size < d_in:
        g = k // group_size
    else:
        g = np.zeros(d_in, dtype=np.int64)
    W_stream = dequantize(codes, scales, zeros, g)
    X64 = np.asarray(X, dtype=np.float64)
    if perm is not None:
        X64 = X64[:, np.asarray(perm, dtype=np.int64)]
    return X64 @ W_stream.T


# ---------------------------------------------------------------------------
# Layers in sequence.
# ---------------------------------------------------------------------------

def round_to_dtype(a, dtype: str) -> np.ndarray:
    """Round float64 values to the activation dtype and back (nearest, ties
    to even): "f32", "f16", or "bf16" (through float32, then the upper 16
    bits of the float32 pattern with round-to-nearest-even)."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    f = a.astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return (r.astype(np.uint32)).view(np.float32).astype(np.float64)


def quantize_block_chain(Ws: dict, X, dtype: str, **q):
    """One decoder block quantized in sequence ("GPTQ量化算法深度解析" §3.1,
    layers one after another; "GPTQ论文复现指南" §3.2, --true-sequential:
    each layer sees the already-quantized outputs of the layers before it).
    With no attention or normalisation details on the pages the block is a
    plain chain: q, k, v on H(X); A = X W_v^T -> out; h1 = X + A W_out^T ->
    fc1; r = relu(h1 W_fc1^T) -> fc2; the block's output h1 + r W_fc2^T.
    Products use the quantized weights in float64; every activation that
    feeds a Hessian or a product is rounded to `dtype`.
    Returns (per-layer gptq_quantize outputs, per-layer inputs, output)."""
    X = np.asarray(X, dtype=np.float64)
    res, inputs = {}, {}
    H = hessian(X)
    for n in ("q", "k", "v"):
        res[n] = gptq_quantize(Ws[n], H, **q)
        inputs[n] = X
    A = round_to_dtype(X @ res["v"]["w_hat"].T, dtype)
    res["out"] = gptq_quantize(Ws["out"], X=A, **q)
    inputs["out"] = A
    h1 = X + A @ res["out"]["w_hat"].T
    h1r = round_to_dtype(h1, dtype)
    res["fc1"] = gptq_quantize(Ws["fc1"], X=h1r, **q)
    inputs["fc1"] = h1r
    r = round_to_dtype(np.maximum(h1r @ res["fc1"]["w_hat"].T, 0.0), dtype)
    res["fc2"] = gptq_quantize(Ws["fc2"], X=r, **q)
    inputs["fc2"] = r
    out = round_to_dtype(h1 + r @ res["fc2"]["w_hat"].T, dtype)
    return res, inputs, out
