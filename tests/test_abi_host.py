"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/moe.h declares, and rejects bad arguments before launching anything.
No kernel is launched here (no GPU needed): each call below fails validation."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_51_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# fake, 256-byte aligned device addresses: never dereferenced, validation fails first
A = 0x7F0000000000


def fake(i=0):
    return ctypes.c_void_p(A + 0x100000 * (i + 1))


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.lib_path()):
        from sparse_mixture_experts_51_amd import build
        build.build()
    return moe.load()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert set(syms) == set(moe.EXPORTED)
    for s in syms:
        assert hasattr(L, s), s


def test_exports_nothing_from_the_oracle(L):
    for s in ("oracle_route", "oracle_layer", "oracle_combine"):
        assert not hasattr(L, s)


def shape(**kw):
    base = dict(tokens=512, d_model=384, n_experts=16, top_k=4, hidden=256, shared_hidden=256,
                seq_len=256)
    base.update(kw)
    return moe.Shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=17), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(tokens=-1), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(seq_len=300), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(n_experts=2000, top_k=4), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=64, top_k=33), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_model=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(shared_hidden=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(tokens=1 << 29, top_k=4), moe.MOE_ERR_UNSUPPORTED),
])
def test_bad_shapes(L, kw, code):
    s = shape(**kw)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_bytes(ctypes.byref(s.c()), ctypes.byref(n)) == code
    ws = fake(20)
    assert L.moe_route(ctypes.byref(s.c()), fake(0), fake(1), fake(2), fake(3), fake(4), None,
                       None, ctypes.c_float(1e-4), ws, 1 << 40, None) == code
    assert L.moe_update_bias(ctypes.byref(s.c()), fake(0), fake(1), ctypes.c_float(1e-3),
                             None) == code


def test_null_shape_and_bytes(L):
    assert L.moe_workspace_bytes(None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_route(None, fake(0), fake(1), fake(2), fake(3), fake(4), None, None,
                       ctypes.c_float(0), fake(5), 1 << 30, None) == moe.MOE_ERR_INVALID_ARGUMENT


def test_workspace_size_monotone_and_layout(L):
    small = moe.moe_workspace_bytes(shape(tokens=256))
    big = moe.moe_workspace_bytes(shape(tokens=4096))
    assert 0 < small < big and small % 256 == 0 and big % 256 == 0
    # the hidden activations dominate: T*k*H + T*Hs bf16
    s = shape(tokens=4096, seq_len=0)
    assert moe.moe_workspace_bytes(s) >= 2 * (4096 * 4 * 256 + 4096 * 256)


def test_route_argument_checks(L):
    s = shape().c()
    need = moe.moe_workspace_bytes(shape())
    f = ctypes.c_float(1e-4)
    # null required pointers
    for i in range(5):
        args = [fake(j) for j in range(5)]
        args[i] = None
        assert L.moe_route(ctypes.byref(s), *args, None, None, f, fake(9), need, None) == \
            moe.MOE_ERR_INVALID_ARGUMENT
    # misaligned x
    assert L.moe_route(ctypes.byref(s), ctypes.c_void_p(A + 2), fake(1), fake(2), fake(3),
                       fake(4), None, None, f, fake(9), need, None) == moe.MOE_ERR_INVALID_ARGUMENT
    # workspace missing / too small / misaligned
    args = [fake(j) for j in range(5)]
    assert L.moe_route(ctypes.byref(s), *args, None, None, f, None, need, None) == \
        moe.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(s), *args, None, None, f, fake(9), need - 1, None) == \
        moe.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(s), *args, None, None, f, ctypes.c_void_p(A + 64), need,
                       None) == moe.MOE_ERR_WORKSPACE


def test_route_zero_tokens_is_noop(L):
    s = shape(tokens=0, seq_len=0).c()
    # returns OK without touching any pointer
    assert L.moe_route(ctypes.byref(s), None, None, None, None, None, None, None,
                       ctypes.c_float(0), None, 0, None) == moe.MOE_OK
    assert L.moe_grouped_ffn(ctypes.byref(s), *([None] * 12), None, 0, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(s), *([None] * 6), None) == moe.MOE_OK


def test_permute_argument_checks(L):
    s = shape().c()
    need = moe.moe_workspace_bytes(shape())
    base = [fake(j) for j in range(5)]
    for i in range(5):
        args = list(base)
        args[i] = None
        assert L.moe_permute(ctypes.byref(s), *args, None, None, fake(9), need, None) == \
            moe.MOE_ERR_INVALID_ARGUMENT
    # x without x_perm (and the reverse)
    assert L.moe_permute(ctypes.byref(s), *base, fake(6), None, fake(9), need, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_permute(ctypes.byref(s), *base, None, fake(6), fake(9), need, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_permute(ctypes.byref(s), *base, None, None, fake(9), 16, None) == \
        moe.MOE_ERR_WORKSPACE


def test_grouped_ffn_argument_checks(L):
    s = shape().c()
    need = moe.moe_workspace_bytes(shape())
    x, xp, ps, off, w1, w3, w2, s1, s3, s2, yp, ys = [fake(j) for j in range(12)]
    ok_args = [x, None, ps, off, w1, w3, w2, s1, s3, s2, yp, ys]
    # shared expert present in the shape but a shared pointer missing
    for i in (7, 8, 9, 11):
        args = list(ok_args)
        args[i] = None
        assert L.moe_grouped_ffn(ctypes.byref(s), *args, fake(20), need, None) == \
            moe.MOE_ERR_INVALID_ARGUMENT
    # no shared expert in the shape but shared pointers given
    s0 = shape(shared_hidden=0)
    need0 = moe.moe_workspace_bytes(s0)
    assert L.moe_grouped_ffn(ctypes.byref(s0.c()), *ok_args, fake(20), need0, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # misaligned weight
    args = list(ok_args)
    args[4] = ctypes.c_void_p(A + 8)
    assert L.moe_grouped_ffn(ctypes.byref(s), *args, fake(20), need, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_grouped_ffn(ctypes.byref(s), *ok_args, fake(20), need - 256, None) == \
        moe.MOE_ERR_WORKSPACE


def test_combine_and_bias_argument_checks(L):
    s = shape().c()
    for i in (0, 2, 3, 5):
        args = [fake(j) for j in range(6)]
        args[i] = None
        assert L.moe_combine(ctypes.byref(s), *args, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_update_bias(ctypes.byref(s), None, fake(1), ctypes.c_float(1e-3), None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_update_bias(ctypes.byref(s), fake(0), None, ctypes.c_float(1e-3), None) == \
        moe.MOE_ERR_INVALID_ARGUMENT


def test_status_strings(L):
    for code in range(5):
        assert moe.status_str(code).startswith("MOE_")
    assert moe.status_str(99) == "unknown moe_status"


def test_binding_raises_on_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "libmoe.so"))
    with pytest.raises(ImportError):
        moe.load()


def test_probe_library_exports_its_declared_symbols():
    from sparse_mixture_experts_51_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    syms = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))
    assert syms == ["moe_probe_hbm_read", "moe_probe_hbm_read_nt"]
    P = ctypes.CDLL(build.PROBE_LIB)
    L = moe.load()
    for name in syms:
        assert hasattr(P, name)
        # the MoE library itself does not carry the probes
        assert not hasattr(L, name)


def test_probe_rejects_unusable_sizes_before_launching():
    from sparse_mixture_experts_51_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    P = ctypes.CDLL(build.PROBE_LIB)
    mib = 1 << 20
    for name in ("moe_probe_hbm_read", "moe_probe_hbm_read_nt"):
        fn = getattr(P, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        for buf, n, sink in ((fake(0), mib + 1, fake(1)), (fake(0), 0, fake(1)), (fake(0), -mib, fake(1)),
                             (None, mib, fake(1)), (fake(0), mib, None)):
            assert fn(buf, n, sink, None) == 1, name
