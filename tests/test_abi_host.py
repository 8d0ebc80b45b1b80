"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/moe.h and include/mla.h declare, and rejects bad arguments before
launching anything.
No kernel is launched here (no GPU needed): each call below fails validation."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_51_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe.h", "mla.h")]
DECL = r"\b((?:moe|mla)_[a-z_]+)\s*\("

# fake, 256-byte aligned device addresses: never dereferenced, validation fails first
A = 0x7F0000000000


def fake(i=0):
    return ctypes.c_void_p(A + 0x100000 * (i + 1))


def header_text():
    text = "".join(open(h).read() for h in HEADERS)
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def declared_symbols():
    return sorted(set(m for m in re.findall(DECL, header_text()) if m not in ("moe_status",)))


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


def declared_prototypes():
    """name -> list of parameter type strings, from the headers."""
    out = {}
    for m in re.finditer(r"\b((?:moe|mla)_[a-z_]+)\s*\(([^)]*)\)\s*;", header_text()):
        params = [q.strip() for q in m.group(2).split(",") if q.strip()]
        out[m.group(1)] = params
    return out


def test_binding_argtypes_match_the_header(L):
    """Every ctypes prototype of the binding has the header's parameter count,
    and size_t / float / int parameters sit where the header puts them."""
    protos = declared_prototypes()
    assert set(protos) == set(moe.EXPORTED)
    for name, params in protos.items():
        argtypes = getattr(L, name).argtypes
        assert len(argtypes) == len(params), (name, len(argtypes), len(params))
        for ctype, decl in zip(argtypes, params):
            if "*" in decl:
                assert ctype not in (ctypes.c_size_t, ctypes.c_float, ctypes.c_int), (name, decl)
            elif decl.startswith("size_t"):
                assert ctype is ctypes.c_size_t, (name, decl)
            elif decl.startswith("float"):
                assert ctype is ctypes.c_float, (name, decl)
            else:
                assert decl.startswith("int "), (name, decl)
                assert ctype is ctypes.c_int, (name, decl)


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


def test_operand_offset_limits(L):
    """The forward GEMMs address x_perm and h per tile, so a V3-wide layer above
    2 GiB of x_perm is accepted; x itself and one expert's weights must stay
    below 2 GiB, and the backward keeps the whole-operand limit."""
    n = ctypes.c_size_t(0)
    v3 = dict(d_model=7168, n_experts=256, top_k=8, hidden=2048, shared_hidden=2048, seq_len=0)
    big = shape(tokens=32768, **v3)  # x_perm 3.8 GB, h 1.2 GB
    assert L.moe_workspace_bytes(ctypes.byref(big.c()), ctypes.byref(n)) == moe.MOE_OK
    assert n.value >= 2 * (32768 * 8 * 2048 + 32768 * 2048)
    assert L.moe_backward_workspace_bytes(ctypes.byref(big.c()), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED
    ok_bwd = shape(tokens=18723, **v3)  # 2*T*k*d just below 2^31
    assert L.moe_backward_workspace_bytes(ctypes.byref(ok_bwd.c()), ctypes.byref(n)) == moe.MOE_OK
    x_at_2g = shape(tokens=(1 << 30) // 7168 + 1, **v3)  # x reaches 2 GiB
    assert L.moe_workspace_bytes(ctypes.byref(x_at_2g.c()), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED
    x_below = shape(tokens=(1 << 30) // 7168, **v3)
    assert L.moe_workspace_bytes(ctypes.byref(x_below.c()), ctypes.byref(n)) == moe.MOE_OK
    w_2g = shape(tokens=64, d_model=1 << 15, n_experts=8, top_k=2, hidden=1 << 15,
                 shared_hidden=0, seq_len=0)  # one expert's weights: 2 GiB
    assert L.moe_workspace_bytes(ctypes.byref(w_2g.c()), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED


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
    # misaligned outputs: the GEMM epilogue writes 16-byte chunks of y_perm and y_shared
    for i in (10, 11):
        args = list(ok_args)
        args[i] = ctypes.c_void_p(A + 0x100000 * (i + 1) + 8)
        assert L.moe_grouped_ffn(ctypes.byref(s), *args, fake(20), need, None) == \
            moe.MOE_ERR_INVALID_ARGUMENT, i


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


def test_permute_noalloc_argument_checks_and_scratch_limit(L):
    """moe_permute_noalloc checks like moe_permute and refuses shapes beyond its
    2 MiB static scratch before touching the GPU."""
    s = shape().c()
    base = [fake(j) for j in range(5)]
    for i in range(5):
        args = list(base)
        args[i] = None
        assert L.moe_permute_noalloc(ctypes.byref(s), *args, None, None, None) == \
            moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_permute_noalloc(ctypes.byref(s), *base, fake(6), None, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # two tables of 4 * ceil(T/256) * E bytes: 2 x 4 MiB here
    big = shape(tokens=1 << 20, n_experts=256, top_k=8, seq_len=0, d_model=64, hidden=64,
                shared_hidden=0).c()
    assert L.moe_permute_noalloc(ctypes.byref(big), *base, None, None, None) == \
        moe.MOE_ERR_SCRATCH_LIMIT
    assert moe.status_str(moe.MOE_ERR_SCRATCH_LIMIT).startswith("MOE_ERR_SCRATCH_LIMIT")


def test_rmsnorm_argument_checks(L):
    s = shape().c()
    f = ctypes.c_float
    for i in range(3):
        args = [fake(0), fake(1), fake(2)]
        args[i] = None
        assert L.moe_rmsnorm(ctypes.byref(s), args[0], args[1], f(1e-6), args[2], None) == \
            moe.MOE_ERR_INVALID_ARGUMENT
    for eps in (-1.0, float("nan"), float("inf")):
        assert L.moe_rmsnorm(ctypes.byref(s), fake(0), fake(1), f(eps), fake(2), None) == \
            moe.MOE_ERR_INVALID_ARGUMENT, eps
    for i in range(3):  # every array 16-byte aligned
        args = [fake(0), fake(1), fake(2)]
        args[i] = ctypes.c_void_p(A + 0x100000 * (i + 1) + 4)
        assert L.moe_rmsnorm(ctypes.byref(s), args[0], args[1], f(1e-6), args[2], None) == \
            moe.MOE_ERR_INVALID_ARGUMENT, i
    z = shape(tokens=0, seq_len=0).c()
    assert L.moe_rmsnorm(ctypes.byref(z), None, None, f(1e-6), None, None) == moe.MOE_OK
    assert L.moe_rmsnorm(ctypes.byref(shape(d_model=100).c()), fake(0), fake(1), f(1e-6), fake(2),
                         None) == moe.MOE_ERR_UNSUPPORTED


def test_status_strings(L):
    for code in range(6):
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
    assert syms == ["moe_probe_hbm_read", "moe_probe_hbm_read_nt", "moe_probe_hbm_read_write"]
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
    fn = P.moe_probe_hbm_read_write
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    misaligned = ctypes.c_void_p(fake(2).value + 8)
    for buf, n, row, out, per, sink in (
            (fake(0), mib + 1, 4096, fake(2), 4096, fake(1)),        # not whole pieces
            (fake(0), 0, 4096, fake(2), 4096, fake(1)),
            (fake(0), mib, 14336, fake(2), 4096, fake(1)),           # 1 MiB is no whole 3.5 MiB piece
            (fake(0), mib, 100, fake(2), 4096, fake(1)),             # row not a multiple of 128
            (fake(0), 2 * mib * 256, 2 * mib, fake(2), 4096, fake(1)),  # row above 1 MiB
            (None, mib, 4096, fake(2), 4096, fake(1)), (fake(0), mib, 4096, None, 4096, fake(1)),
            (fake(0), mib, 4096, fake(2), 4096, None), (fake(0), mib, 4096, fake(2), 0, fake(1)),
            (fake(0), mib, 4096, fake(2), 24, fake(1)), (fake(0), mib, 4096, fake(2), mib + 16, fake(1)),
            (fake(0), mib, 4096, misaligned, 4096, fake(1))):
        assert fn(buf, n, row, out, per, sink, None) == 1, (n, row, per)


def mla_shape(**kw):
    base = dict(batch=2, seq_len=64, max_len=128, d_model=384, n_heads=6, d_latent=128,
                d_nope=32, d_rope=16, d_v=32, rope_base=10000.0)
    base.update(kw)
    return moe.MlaShapeC(*[base[f] for f, _ in moe.MlaShapeC._fields_])


def test_mla_workspace_and_shape_checks(L):
    n = ctypes.c_size_t(0)
    assert L.mla_workspace_bytes(ctypes.byref(mla_shape()), 0, ctypes.byref(n)) == moe.MOE_OK
    T, H = 2 * 64, 6
    assert n.value >= 2 * T * H * (48 + 64 + 32)
    assert L.mla_workspace_bytes(ctypes.byref(mla_shape()), 1, ctypes.byref(n)) == moe.MOE_OK
    assert L.mla_workspace_bytes(ctypes.byref(mla_shape()), 0, None) == moe.MOE_ERR_INVALID_ARGUMENT
    bad = [dict(seq_len=200), dict(max_len=0), dict(rope_base=1.0), dict(n_heads=0)]
    for kw in bad:
        assert L.mla_workspace_bytes(ctypes.byref(mla_shape(**kw)), 0, ctypes.byref(n)) == \
            moe.MOE_ERR_INVALID_ARGUMENT, kw
    unsupported = [dict(d_model=100), dict(d_latent=96), dict(d_latent=192), dict(d_latent=320),
                   dict(d_v=24),
                   dict(d_nope=100, d_rope=40), dict(n_heads=17, d_v=64), dict(d_rope=12)]
    for kw in unsupported:
        assert L.mla_workspace_bytes(ctypes.byref(mla_shape(**kw)), 0, ctypes.byref(n)) == \
            moe.MOE_ERR_UNSUPPORTED, kw


def test_mla_calls_refuse_bad_arguments(L):
    s = ctypes.byref(mla_shape())
    ws = fake(20)
    w = [fake(i) for i in range(6)]
    # a missing weight, a misaligned output, a small workspace, no positions
    assert L.mla_prefill(s, fake(7), None, *w[1:], None, fake(8), fake(9), fake(10), ws, 1 << 30,
                         None) == moe.MOE_ERR_INVALID_ARGUMENT
    odd = ctypes.c_void_p(A + 2)
    assert L.mla_prefill(s, fake(7), *w, None, fake(8), fake(9), odd, ws, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.mla_prefill(s, fake(7), *w, None, fake(8), fake(9), fake(10), ws, 16, None) == \
        moe.MOE_ERR_WORKSPACE
    assert L.mla_decode(s, fake(7), None, *w, None, fake(8), fake(9), fake(10), ws, 1 << 30,
                        None) == moe.MOE_ERR_INVALID_ARGUMENT
    # nothing to do: no launch, OK
    empty = ctypes.byref(mla_shape(batch=0))
    assert L.mla_prefill(empty, None, *w, None, None, None, None, None, 0, None) == moe.MOE_OK
