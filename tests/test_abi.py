"""The C ABI: the library loads, exports every declared symbol, validates arguments.

CPU only: no call here reaches a kernel launch (every call is rejected by
argument validation, which happens before any HIP call).
"""
import ctypes
import os
import re

import pytest

import post_weight_quantization_accum_amd as P
from post_weight_quantization_accum_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(gptq_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = P.load()
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTS) == declared


def test_status_strings_and_version():
    for st in range(7):
        assert isinstance(P.status_string(st), str) and P.status_string(st)
    assert re.match(r"^\d+\.\d+\.\d+$", P.version())


def test_config_default():
    lib = P.load()
    c = P.Config()
    c.static_groups = 7   # overwritten by the default
    lib.gptq_config_default(ctypes.byref(c))
    assert (c.bits, c.group_size, c.sym, c.act_order, c.block_size, c.static_groups, c.damp) == \
        (4, 128, 0, 0, 128, 0, 0.01)
    assert ctypes.sizeof(P.Config) == 32 and P.Config.damp.offset == 24


def test_workspace_queries():
    lib = P.load()
    c = P.make_config(bits=4, group_size=128, block=128)
    assert lib.gptq_prepare_hinv_workspace(11008) >= 11008 * 11008 * 8
    assert lib.gptq_quantize_layer_workspace(4096, 11008, ctypes.byref(c)) >= 4096 * 11008 * 9
    assert lib.gptq_prepare_hinv_workspace(0) == 0
    mixed = P.make_config(group_size=96, block=128)   # neither divides the other: accepted
    assert lib.gptq_quantize_layer_workspace(8, 384, ctypes.byref(mixed)) >= 8 * 384 * 9
    assert lib.gptq_quantize_layer_workspace(8, 384, ctypes.byref(P.make_config(block=0))) == 0
    bad = P.make_config()
    bad.static_groups = 2
    assert lib.gptq_quantize_layer_workspace(8, 384, ctypes.byref(bad)) == 0
    st = P.make_config(group_size=96, block=128, static_groups=True)
    assert lib.gptq_quantize_layer_workspace(8, 384, ctypes.byref(st)) >= 8 * 384 * 9
    # factored form: workspace 0 where unsupported; the sweep's plus a float64 copy of W otherwise
    assert lib.gptq_prepare_hinv_factored_workspace(1000) == 0
    assert lib.gptq_prepare_hinv_factored_workspace(1024) >= lib.gptq_prepare_hinv_workspace(1024)
    c128 = P.make_config(group_size=128)
    assert lib.gptq_quantize_layer_factored_workspace(8, 1024, ctypes.byref(c128)) >= \
        lib.gptq_quantize_layer_workspace(8, 1024, ctypes.byref(c128)) + 8 * 1024 * 8
    for g, ok in ((128, True), (64, True), (8, True), (-1, True), (4096, True), (96, False), (256, False),
                  (4, False)):
        cg = P.make_config(group_size=g)
        assert (lib.gptq_quantize_layer_factored_workspace(8, 1024, ctypes.byref(cg)) > 0) == ok, g
    assert lib.gptq_quantize_layer_factored_workspace(
        8, 1024, ctypes.byref(P.make_config(group_size=256, static_groups=True))) > 0
    assert lib.gptq_quantize_layer_factored_workspace(8, 1024, ctypes.byref(P.make_config(block=64))) == 0
    assert lib.gptq_packed_words_per_row(11, 3) == 2
    assert lib.gptq_packed_words_per_row(8, 4) == 1
    assert lib.gptq_packed_words_per_row(8, 5) == -1


def test_argument_validation_before_any_launch():
    lib = P.load()
    c = P.make_config()
    n = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.gptq_hessian_accumulate(n, fake, 2, 10, 10, 10, n, 0, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_hessian_accumulate(fake, fake, 7, 10, 10, 10, n, 0, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_hessian_accumulate(fake, fake, 2, 10, 10, 5, n, 0, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_prepare_hinv(n, 10, ctypes.byref(c), fake, fake, 1 << 30, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_prepare_hinv(fake, 10, ctypes.byref(c), fake, n, 0, n) == _lib.ERR_WORKSPACE
    assert lib.gptq_prepare_hinv(fake, 10, ctypes.byref(c), fake, fake, 16, n) == _lib.ERR_WORKSPACE
    b5 = P.make_config(bits=5)
    assert lib.gptq_prepare_hinv(fake, 10, ctypes.byref(b5), fake, fake, 1 << 30, n) == _lib.ERR_INVALID_ARG
    big_b = P.make_config(group_size=256, block=256)
    assert lib.gptq_prepare_hinv(fake, 10, ctypes.byref(big_b), fake, fake, 1 << 30, n) == _lib.ERR_UNSUPPORTED
    b0 = P.make_config(group_size=96, block=0)
    args = [fake, 2, 8, 384, 384, fake, fake, ctypes.byref(b0), fake, fake, fake, fake, n, n, fake, 1 << 30, n]
    assert lib.gptq_quantize_layer(*args) == _lib.ERR_INVALID_ARG
    args = [fake, 2, 8, 384, 100, fake, fake, ctypes.byref(c), fake, fake, fake, fake, n, n, fake, 1 << 30, n]
    assert lib.gptq_quantize_layer(*args) == _lib.ERR_INVALID_ARG  # ld_w < d_in
    args = [fake, 2, 8, 384, 384, fake, fake, ctypes.byref(c), fake, fake, fake, fake, n, n, fake, 10, n]
    assert lib.gptq_quantize_layer(*args) == _lib.ERR_WORKSPACE
    neg = P.make_config(damp=-0.1)
    args = [fake, 2, 8, 384, 384, fake, fake, ctypes.byref(neg), fake, fake, fake, fake, n, n, fake, 1 << 30, n]
    assert lib.gptq_quantize_layer(*args) == _lib.ERR_INVALID_ARG
    # the factored form: 128-column blocks only, every group inside one block
    assert lib.gptq_prepare_hinv_factored(fake, 1000, ctypes.byref(c), fake, fake, 1 << 40, n) == \
        _lib.ERR_UNSUPPORTED
    assert lib.gptq_prepare_hinv_factored(n, 1024, ctypes.byref(c), fake, fake, 1 << 40, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_prepare_hinv_factored(fake, 1024, ctypes.byref(c), fake, fake, 16, n) == _lib.ERR_WORKSPACE
    for bad_cfg in (P.make_config(group_size=96), P.make_config(block=64), P.make_config(group_size=4)):
        args = [fake, 2, 8, 1024, 1024, fake, fake, ctypes.byref(bad_cfg), fake, fake, fake, fake, n, n, fake,
                1 << 40, n]
        assert lib.gptq_quantize_layer_factored(*args) == _lib.ERR_UNSUPPORTED
    args = [fake, 2, 8, 1000, 1000, fake, fake, ctypes.byref(c), fake, fake, fake, fake, n, n, fake, 1 << 40, n]
    assert lib.gptq_quantize_layer_factored(*args) == _lib.ERR_UNSUPPORTED   # d_in not a multiple of 128
    args = [fake, 2, 8, 1024, 1024, fake, fake, ctypes.byref(c), fake, fake, fake, fake, n, n, fake, 10, n]
    assert lib.gptq_quantize_layer_factored(*args) == _lib.ERR_WORKSPACE
    assert lib.gptq_pack(n, 4, 8, 4, fake, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_pack(fake, 4, 8, 5, fake, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_pack(fake, 0, 8, 4, fake, n) == _lib.ERR_INVALID_ARG
    assert lib.gptq_pack_permuted(fake, 4, 8, 4, n, fake, n) == _lib.ERR_INVALID_ARG  # perm missing
    assert lib.gptq_pack_permuted(fake, 4, 8, 3 + 3, fake, fake, n) == _lib.ERR_INVALID_ARG


def _dq(**kw):
    # gptq_dequant_matmul with valid arguments unless overridden
    fake = ctypes.c_void_p(0x1000)
    a = dict(X=fake, dt=2, n_tok=1, d_in=256, ld_x=256, packed=fake, bits=4, scales=fake, zeros=fake,
             n_groups=2, g_idx=None, perm=None, gs=128, d_out=64, Y=fake, ld_y=64)
    a.update(kw)
    return P.load().gptq_dequant_matmul(a["X"], a["dt"], a["n_tok"], a["d_in"], a["ld_x"], a["packed"], a["bits"],
                                        a["scales"], a["zeros"], a["n_groups"], a["g_idx"], a["perm"], a["gs"],
                                        a["d_out"], a["Y"], a["ld_y"], None)


def test_dequant_matmul_validation_before_any_launch():
    fake = ctypes.c_void_p(0x1000)
    assert P.dequant_max_groups() == 2048
    assert _dq(bits=5) == _lib.ERR_INVALID_ARG
    assert _dq(dt=7) == _lib.ERR_INVALID_ARG
    assert _dq(ld_x=255) == _lib.ERR_INVALID_ARG
    assert _dq(ld_y=63) == _lib.ERR_INVALID_ARG
    assert _dq(d_in=0) == _lib.ERR_INVALID_ARG
    assert _dq(n_tok=-1) == _lib.ERR_INVALID_ARG
    assert _dq(g_idx=fake, perm=fake) == _lib.ERR_INVALID_ARG
    assert _dq(n_groups=3) == _lib.ERR_INVALID_ARG            # ceil(256 / 128) = 2
    assert _dq(gs=-1, n_groups=2) == _lib.ERR_INVALID_ARG     # one group
    assert _dq(g_idx=fake, n_groups=0) == _lib.ERR_INVALID_ARG
    assert _dq(X=None) == _lib.ERR_INVALID_ARG
    assert _dq(Y=None) == _lib.ERR_INVALID_ARG
    # the per-column route keeps [group][row] scales of 8 rows in LDS: bounded group count
    assert _dq(d_in=8192, ld_x=8192, g_idx=fake, n_groups=4096) == _lib.ERR_UNSUPPORTED
    # the column gather
    lib = P.load()
    assert lib.gptq_gather_columns(fake, 7, 4, 8, 8, fake, fake, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.gptq_gather_columns(fake, 2, 4, 8, 7, fake, fake, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.gptq_gather_columns(fake, 2, 4, 8, 8, None, fake, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.gptq_gather_columns(fake, 2, 0, 8, 8, fake, fake, 8, None) == _lib.OK
    # empty products launch nothing
    assert _dq(n_tok=0) == _lib.OK
    assert _dq(d_out=0, ld_y=0) == _lib.OK


def test_python_errors_map_status():
    with pytest.raises(P.InvalidArgument):
        _lib.check(_lib.ERR_INVALID_ARG, "x")
    with pytest.raises(P.NotPositiveDefinite):
        _lib.check(_lib.ERR_NOT_PD, "x")
    with pytest.raises(P.NonFinite):
        _lib.check(_lib.ERR_NONFINITE, "x")


def test_hessian_workspace_required_for_16bit_inputs():
    lib = P.load()
    fake = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    assert lib.gptq_hessian_workspace(100, 11008) >= 11008 * 8
    assert lib.gptq_hessian_accumulate(fake, fake, _lib.BF16, 10, 16, 16, n, 0, n) == _lib.ERR_WORKSPACE
    assert lib.gptq_hessian_accumulate(fake, fake, _lib.F16, 10, 16, 16, fake, 8, n) == _lib.ERR_WORKSPACE
