"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Needs an MI355X and a built libmoe.so.

Small shapes are compared element by element on every output; the full-size
workloads (the launch configuration bench.py times) are compared on every
routing decision and on sampled token outputs, since the oracle computes a
token at a time.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import (bits, check_bf16_close, check_routing, f32, gpu_host, host, host_params,
                    inputs, run_layer, say)
from sparse_mixture_experts_51_amd import moe, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()  # raises if the HIP library is missing


def custom(**kw):
    return workloads.custom(**kw)


ROUTE_CASES = {
    "mini_2048": workloads.WORKLOADS["mini_2048"],
    "ragged_T1000_S250": custom(tokens=1000, seq_len=250, cfg_id=91),
    "small_cfg_E8_k2": custom(tokens=777, n_experts=8, top_k=2, cfg_id=92),
    "odd_E3_k2_d64": custom(tokens=129, d_model=64, n_experts=3, top_k=2, cfg_id=93,
                            router_std=0.2),
    "E100_k6": custom(tokens=300, seq_len=100, d_model=128, n_experts=100, top_k=6, cfg_id=94,
                      router_std=0.1),
    "v3_router_T256": custom(tokens=256, seq_len=256, d_model=7168, n_experts=256, top_k=8,
                             hidden=2048, shared_hidden=2048, cfg_id=95, w_std=0.006,
                             router_std=0.006, bias_range=0.01),
    "max_E1024_k32": custom(tokens=200, seq_len=50, d_model=64, n_experts=1024, top_k=32,
                            cfg_id=96, router_std=0.1),
    "k_equals_E": custom(tokens=100, d_model=64, n_experts=8, top_k=8, cfg_id=97),
    "k1": custom(tokens=300, n_experts=16, top_k=1, cfg_id=98),
    # fewer experts than the router's 4-expert W_r pieces (a tile of 4, two
    # of them absent)
    "E2_k1": custom(tokens=300, seq_len=150, d_model=64, n_experts=2, top_k=1, cfg_id=175,
                    router_std=0.2),
    "T1": custom(tokens=1, n_experts=16, top_k=4, cfg_id=99),
    # two 16-lane rows per token in the selection: separate select kernel
    # (250-token sequences do not split into whole blocks) and fused routing
    "E24_k3": custom(tokens=500, seq_len=250, d_model=128, n_experts=24, top_k=3, cfg_id=117,
                     router_std=0.1),
    "E24_k3_fused": custom(tokens=512, seq_len=256, d_model=128, n_experts=24, top_k=3,
                           cfg_id=119, router_std=0.1),
    # a whole wave per token, one expert per lane
    "E64_k8": custom(tokens=320, seq_len=160, d_model=128, n_experts=64, top_k=8, cfg_id=118,
                     router_std=0.1),
    # logits on the fp32 matrix cores (many tokens, E a multiple of 64): a
    # ragged last block of tokens, and the V3 expert count
    "mfma_T1100_E128": custom(tokens=1100, seq_len=550, d_model=256, n_experts=128, top_k=8,
                              cfg_id=120, router_std=0.1),
    "mfma_T2048_E256": custom(tokens=2048, seq_len=1024, d_model=384, n_experts=256, top_k=8,
                              cfg_id=121, router_std=0.05),
}


def route_gpu(wl, x, w_r, b, alpha=1e-4):
    shape = moe.Shape.of(wl)
    bufs = moe.alloc_buffers(shape, DEV)
    moe.moe_route(shape, x, w_r, b, bufs["topk_idx"], bufs["topk_gate"], bufs["margin"],
                  bufs["seq_balance"], alpha, bufs["workspace"])
    torch.cuda.synchronize()
    return bufs


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_matches_oracle(name):
    wl = ROUTE_CASES[name]
    say(f"[route] {name} T={wl.tokens} d={wl.d_model} E={wl.n_experts} k={wl.top_k} S={wl.seq_len}")
    x = workloads.tokens(wl, 0, DEV)
    w_r = workloads.router(wl, 0, DEV)
    b = workloads.bias(wl, 0, DEV)
    bufs = route_gpu(wl, x, w_r, b)
    g = gpu_host(bufs)
    ref = oracle.route(bits(x), host(w_r), host(b), wl.top_k)
    check_routing(g, ref, name)
    if wl.top_k == 1:
        assert np.all(g["topk_gate"] == 1.0)
    if wl.seq_len:
        L = oracle.seq_balance(ref["scores"], g["topk_idx"], wl.seq_len, 1e-4)
        rel = np.abs(g["seq_balance"].astype(np.float64) - L) / np.abs(L)
        say(f"  seq_balance: max rel err {rel.max():.2e} over {len(L)} sequences")
        assert rel.max() <= 1e-5


def test_route_nan_token_and_bias_only_moves_choice():
    wl = custom(tokens=64, n_experts=16, top_k=4, cfg_id=101)
    x = workloads.tokens(wl, 0, DEV)
    w_r = workloads.router(wl, 0, DEV)
    b = workloads.bias(wl, 0, DEV)
    x[5, 7] = float("nan")
    g = gpu_host(route_gpu(wl, x, w_r, b))
    ref = oracle.route(bits(x), host(w_r), host(b), 4)
    assert list(g["topk_idx"][5]) == [0, 1, 2, 3] == list(ref["idx"][5])
    assert np.all(np.isnan(g["topk_gate"][5]))
    keep = np.arange(64) != 5
    assert np.array_equal(g["topk_idx"][keep], ref["idx"][keep])
    # a second bias: tokens whose choices do not change keep bit-identical gates
    b2 = b + 0.03 * torch.sin(torch.arange(16, device=DEV, dtype=torch.float32))
    g2 = gpu_host(route_gpu(wl, x, w_r, b2))
    same = np.all(g["topk_idx"] == g2["topk_idx"], 1) & keep
    assert same.any() and not same.all()
    assert np.array_equal(g["topk_gate"][same], g2["topk_gate"][same])


PERM_CASES = [(2048, 16, 4), (1000, 16, 4), (4096, 256, 8), (300, 1024, 32), (1, 8, 2),
              (777, 8, 2), (64, 256, 8)]
# every case with and without the x_perm copy, plus the mini model's shape, a
# single expert and eight choices per token without it
# count tables of more than 16384 (block, expert) entries go through the
# separate single-block scan kernel instead of the scan inside the scatter:
# 79 token blocks x 256 experts and 20 x 1024
PERM_SCAN_CASES = [(20000, 256, 8), (5000, 1024, 8)]
PERM_RUNS = ([(T, E, k, True) for T, E, k in PERM_CASES] + [(T, E, k, False) for T, E, k in PERM_CASES]
             + [(8192, 16, 4, False), (500, 1, 1, False), (3000, 16, 8, False)]
             + [(T, E, k, g) for T, E, k in PERM_SCAN_CASES for g in (True, False)])


@pytest.mark.parametrize("T,E,k,gather", PERM_RUNS)
def test_permute_matches_oracle(T, E, k, gather):
    say(f"[permute] T={T} E={E} k={k} x_perm={gather}")
    gen = torch.Generator().manual_seed(T * 131 + E)
    idx = torch.stack([torch.randperm(E, generator=gen)[:k] for _ in range(T)]).to(torch.int32)
    d = 128
    shape = moe.Shape(T, d, E, k, 64, 0, 0)
    bufs = moe.alloc_buffers(shape, DEV, x_perm=gather)
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    idx_d = idx.to(DEV)
    bufs["perm_src"].fill_(-7)
    bufs["pos"].fill_(-7)
    moe.moe_permute(shape, idx_d, bufs["counts"], bufs["offsets"], bufs["perm_src"], bufs["pos"],
                    x if gather else None, bufs["x_perm"] if gather else None, bufs["workspace"])
    torch.cuda.synchronize()
    ref = oracle.permute(idx.numpy(), E)
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(host(bufs[key]), ref[key]), key
    if gather:
        xp = bits(bufs["x_perm"])
        assert np.array_equal(xp, bits(x)[ref["perm_src"]])


def test_permute_skips_malformed_choices_and_gathers_the_rest():
    """Choices outside [0, E) (only a malformed caller produces them) are left
    out of the loads, offsets and rows; every other row is placed and copied.
    Checked by properties, with no oracle call: the oracle is never fed such
    input."""
    T, E, k, d = 700, 16, 4, 128
    say(f"[permute] malformed choices T={T} E={E} k={k} x_perm=True")
    gen = torch.Generator().manual_seed(4242)
    idx = torch.stack([torch.randperm(E, generator=gen)[:k] for _ in range(T)]).to(torch.int32)
    bad = torch.rand(T, k, generator=gen) < 0.07
    idx[bad] = torch.where(torch.rand(T, k, generator=gen) < 0.5, -1, E + 3).to(torch.int32)[bad]
    shape = moe.Shape(T, d, E, k, 64, 0, 0)
    bufs = moe.alloc_buffers(shape, DEV, x_perm=True)
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    bufs["x_perm"].fill_(0)
    moe.moe_permute(shape, idx.to(DEV), bufs["counts"], bufs["offsets"], bufs["perm_src"], bufs["pos"],
                    x, bufs["x_perm"], bufs["workspace"])
    torch.cuda.synchronize()
    ids = idx.numpy()
    valid = (ids >= 0) & (ids < E)
    counts, offsets = host(bufs["counts"]), host(bufs["offsets"])
    assert np.array_equal(counts, np.bincount(ids[valid], minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[E] == valid.sum()
    pos, src = host(bufs["pos"]), host(bufs["perm_src"])
    assert np.all(pos[~valid] == -1)
    n = int(offsets[E])
    assert sorted(pos[valid].tolist()) == list(range(n))  # a bijection onto the filled rows
    for t, j in zip(*np.nonzero(valid)):
        e, r = ids[t, j], pos[t, j]
        assert src[r] == t and offsets[e] <= r < offsets[e + 1]
    for e in range(E):  # ascending tokens inside each group
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    xp, xb = bits(bufs["x_perm"]), bits(x)
    assert np.array_equal(xp[:n], xb[src[:n]])
    assert not xp[n:].any()  # rows past the filled ones are not written


def test_hbm_probe_reads_and_leaves_the_sink():
    import ctypes

    from sparse_mixture_experts_51_amd import build
    P = ctypes.CDLL(build.PROBE_LIB)
    buf = torch.ones(8 << 20, dtype=torch.bfloat16, device=DEV)  # 16 MiB
    sink = torch.full((4096,), 7, dtype=torch.int32, device=DEV)
    for name in ("moe_probe_hbm_read", "moe_probe_hbm_read_nt"):
        say(f"[probe] {name} over 16 MiB")
        fn = getattr(P, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        assert fn(buf.data_ptr(), 16 << 20, sink.data_ptr(), None) == 0
        torch.cuda.synchronize()
        assert torch.all(sink == 7), name
    fn = P.moe_probe_hbm_read_write
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    per = 4096
    for row, n in ((4096, 16 << 20), (14336, 14 << 20)):
        say(f"[probe] moe_probe_hbm_read_write over {n >> 20} MiB, rows of {row} bytes, {per} bytes per piece")
        pieces = n // (256 * row)
        out = torch.zeros(pieces * per // 4, dtype=torch.int32, device=DEV)
        assert fn(buf.data_ptr(), n, row, out.data_ptr(), per, sink.data_ptr(), None) == 0
        torch.cuda.synchronize()
        assert torch.all(sink == 7)
        # piece p wrote its 16-byte chunks c at p * per, each holding (.., p, c, 0)
        words = out.view(pieces, per // 16, 4).cpu()
        assert torch.equal(words[:, :, 1], torch.arange(pieces).view(-1, 1).expand(pieces, per // 16).int())
        assert torch.equal(words[:, :, 2], torch.arange(per // 16).view(1, -1).expand(pieces, per // 16).int())
        assert torch.all(words[:, :, 3] == 0)


def test_permute_zero_tokens_writes_zero_loads():
    shape = moe.Shape(0, 64, 16, 4, 64, 0, 0)
    bufs = moe.alloc_buffers(shape, DEV)
    bufs["counts"].fill_(7)
    bufs["offsets"].fill_(7)
    moe.moe_permute(shape, bufs["topk_idx"], bufs["counts"], bufs["offsets"], bufs["perm_src"],
                    bufs["pos"], None, None, bufs["workspace"])
    torch.cuda.synchronize()
    assert torch.all(bufs["counts"] == 0) and torch.all(bufs["offsets"] == 0)


FFN_CASES = {
    "mini_2048": workloads.WORKLOADS["mini_2048"],
    "ragged_T333": custom(tokens=333, cfg_id=111),
    "no_shared": custom(tokens=500, shared_hidden=0, cfg_id=112),
    "shared_wider": custom(tokens=300, shared_hidden=512, cfg_id=113),
    "v3_dims_T16": custom(tokens=16, d_model=7168, n_experts=16, top_k=4, hidden=2048,
                          shared_hidden=2048, cfg_id=114, w_std=0.006, router_std=0.006,
                          bias_range=0.01),
    # hundreds of rows per expert (the 256x256 tile), ragged row tails
    "big_ragged_T3001": custom(tokens=3001, n_experts=8, top_k=4, cfg_id=115),
    # ... with partial column tiles (H = 320, d = 448) and odd K-step counts
    "big_H320_d448": custom(tokens=2500, d_model=448, n_experts=8, top_k=4, hidden=320,
                            shared_hidden=192, cfg_id=116),
}


# the gathered x_perm input is exercised on the mini shapes; every case runs
# with the in-kernel gather through perm_src
FFN_RUNS = [(n, False) for n in FFN_CASES] + [("mini_2048", True), ("ragged_T333", True)]


@pytest.mark.parametrize("name,use_x_perm", FFN_RUNS)
def test_grouped_ffn_matches_oracle(name, use_x_perm):
    wl = FFN_CASES[name]
    say(f"[ffn] {name} x_perm={use_x_perm} T={wl.tokens} d={wl.d_model} E={wl.n_experts} "
        f"k={wl.top_k} H={wl.hidden} Hs={wl.shared_hidden}")
    shape = moe.Shape.of(wl)
    x, p = inputs(wl, DEV)
    bufs = run_layer(shape, x, p, use_x_perm=use_x_perm)
    g = gpu_host(bufs)
    hp = host_params(p)
    # the oracle's own grouping of the GPU's choices (integer work, checked exactly)
    pm = oracle.permute(g["topk_idx"], wl.n_experts)
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(g[key], pm[key]), key
    ref = oracle.grouped_ffn(bits(x), pm["perm_src"], pm["offsets"], hp["w1"], hp["w3"], hp["w2"],
                             hp.get("ws1"), hp.get("ws3"), hp.get("ws2"))
    check_bf16_close(g["y_perm"], ref["y_perm"], f"{name}.y_perm")
    if wl.shared_hidden:
        check_bf16_close(g["y_shared"], ref["y_shared"], f"{name}.y_shared")
    out = oracle.combine(g["y_perm"], g.get("y_shared"), g["topk_gate"], g["topk_idx"], g["pos"])
    check_bf16_close(g["out"], out, f"{name}.out(from gpu y)")


def test_combine_matches_oracle_with_residual():
    T, d, E, k = 700, 384, 16, 4
    shape = moe.Shape(T, d, E, k, 256, 256, 0)
    gen = torch.Generator(device=DEV).manual_seed(121)
    y_perm = torch.randn(T * k, d, device=DEV, generator=gen).to(torch.bfloat16)
    y_sh = torch.randn(T, d, device=DEV, generator=gen).to(torch.bfloat16)
    res = torch.randn(T, d, device=DEV, generator=gen).to(torch.bfloat16)
    gate = torch.rand(T, k, device=DEV, generator=gen)
    gate = gate / gate.sum(1, keepdim=True)
    cpu_gen = torch.Generator().manual_seed(122)
    idx = torch.stack([torch.randperm(E, generator=cpu_gen)[:k] for _ in range(T)]).to(torch.int32)
    pos_np = oracle.permute(idx.numpy(), E)["pos"]
    pos = torch.from_numpy(pos_np).to(DEV)
    out = torch.empty(T, d, device=DEV, dtype=torch.bfloat16)
    for r, ys in ((res, y_sh), (None, y_sh), (None, None)):
        moe.moe_combine(shape, y_perm, ys, gate, pos, r, out)
        torch.cuda.synchronize()
        ref = oracle.combine(bits(y_perm), None if ys is None else bits(ys), host(gate),
                             idx.numpy(), host(pos), None if r is None else bits(r))
        g = f32(bits(out)).astype(np.float64)
        rr = f32(ref).astype(np.float64)
        # magnitude of the summed terms, for the fp32-vs-fp64 accumulation bound
        yp = f32(bits(y_perm)).astype(np.float64)
        mag = np.abs(host(gate)).astype(np.float64)[:, :, None] * np.abs(yp[pos_np])
        mag = mag.sum(1)
        if ys is not None:
            mag += np.abs(f32(bits(ys)).astype(np.float64))
        if r is not None:
            mag += np.abs(f32(bits(r)).astype(np.float64))
        # Both sides round once to bf16.  Before rounding they differ by the
        # GPU's fp32 accumulation error, at most (k+2) * 2^-24 * sum|terms|
        # (k+2 rounded additions, each off by at most 2^-24 of a partial sum
        # no larger than sum|terms|); two roundings of values that close land
        # at most one bf16 ulp (<= 2^-7 |ref|) apart.  Asserted:
        #   |gpu - ref| <= 2^-7 |ref| + 2 (k+3) 2^-24 sum|terms|
        # i.e. twice (2^-8 |ref| + (k+3) 2^-24 sum|terms|), the accumulation
        # term with one spare rounding and a factor 2 of headroom.
        bound = np.abs(rr) * 2.0 ** -8 + (k + 3) * 2.0 ** -24 * mag + 1e-30
        assert np.all(np.abs(g - rr) <= 2 * bound)
        assert (g == rr).mean() > 0.99


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 steps between two arrays of finite bf16 bit patterns."""
    def key(b):
        b = np.asarray(b).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


# (T, d): one chunk per lane and less (d = 64, 384), 2, 4, 8 and 16 chunks per
# lane in registers (d = 1024 ... 8192, the V3 width among them), and the
# re-reading path (d = 16384); ragged row counts against four rows per block
NORM_CASES = [(1000, 384), (33, 64), (5, 1024), (4096, 7168), (7, 8192), (3, 16384), (1, 128)]


@pytest.mark.parametrize("T,d", NORM_CASES)
def test_rmsnorm_matches_oracle(T, d):
    say(f"[rmsnorm] T={T} d={d}")
    gen = torch.Generator(device=DEV).manual_seed(T * 7 + d)
    x = torch.randn(T, d, device=DEV, generator=gen).to(torch.bfloat16)
    if T > 2:
        x[1] = 0.0      # a zero row: eps keeps it finite
        x[2] = -0.375   # a constant row
    gain = 1.0 + 0.3 * torch.randn(d, device=DEV, generator=gen)
    out = torch.empty_like(x)
    shape = moe.Shape(T, d, 8, 2, 64, 0, 0)
    moe.moe_rmsnorm(shape, x, gain, 1e-6, out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(bits(x), host(gain), 1e-6)
    g = bits(out)
    diff = bf16_ulp_diff(g, ref)
    # fp32 sum and product against the oracle's fp64: the roundings to bf16
    # may differ by one step where the value lies within ~2^-23 of a midpoint
    say(f"  max bf16 steps {diff.max()}, differing elements {(diff > 0).mean():.2e}")
    assert diff.max() <= 1
    assert (diff > 0).mean() < 1e-3
    if T > 2:
        assert not (g[1] & 0x7FFF).any()  # +-0 (a negative gain gives -0)


def test_small_config_blocks_teacher_forced():
    """The pages' small configuration (4 layers, 8 experts, top-2, 128-token
    sequences) as pre-norm residual blocks, two steps with the bias update in
    between.  Each layer's oracle input is the GPU's layer input (teacher
    forcing); the norm, routing, loads and bias are compared exactly (the
    norm to one bf16 step), the block outputs on sampled tokens."""
    wl = workloads.WORKLOADS["small_block_4096x4"]
    shape = moe.Shape.of(wl)
    params = [workloads.layer_params(wl, l, DEV) for l in range(wl.layers)]
    bufs = [moe.alloc_buffers(shape, DEV) for _ in range(wl.layers)]
    sample = np.arange(0, wl.tokens, 37)
    for step in range(2):
        x = workloads.tokens(wl, step, DEV)
        for l in range(wl.layers):
            say(f"[small] step {step} layer {l}")
            b_before = host(params[l]["bias"]).copy()
            moe.block_forward(shape, x, params[l], bufs[l])
            torch.cuda.synchronize()
            g = gpu_host(bufs[l])
            hp = host_params(params[l])
            hp["bias"] = b_before
            xb = bits(x)
            xn_ref = oracle.rmsnorm(xb, hp["norm"], 1e-6)
            assert bf16_ulp_diff(g["xn"], xn_ref).max() <= 1
            # routing on the GPU's normalised rows, exact
            ref = oracle.route(g["xn"], hp["w_router"], b_before, wl.top_k)
            check_routing(g, ref, f"step{step}.layer{l}")
            pm = oracle.permute(g["topk_idx"], wl.n_experts)
            for key in ("counts", "offsets", "perm_src", "pos"):
                assert np.array_equal(g[key], pm[key]), key
            L = oracle.seq_balance(ref["scores"], g["topk_idx"], wl.seq_len, 1e-4)
            assert np.abs(g["seq_balance"] - L).max() / np.abs(L).max() <= 1e-5
            lo = oracle.layer(g["xn"][sample], hp, wl.top_k, residual=xb[sample])
            check_bf16_close(g["out"][sample], lo["out"], f"step{step}.layer{l}.out")
            x = bufs[l]["out"].clone()
        for l in range(wl.layers):
            b_before = host(params[l]["bias"]).copy()
            moe.moe_update_bias(shape, bufs[l]["counts"], params[l]["bias"], 1e-3)
            torch.cuda.synchronize()
            ref_b = oracle.update_bias(host(bufs[l]["counts"]), b_before, wl.tokens, wl.top_k)
            assert np.array_equal(host(params[l]["bias"]), ref_b)


def test_update_bias_matches_oracle_bit_exact():
    for T, E, k in ((8192, 16, 4), (4096, 256, 8), (10, 1000, 3)):
        gen = torch.Generator().manual_seed(E)
        counts = torch.randint(0, 2 * T * k // E + 2, (E,), generator=gen, dtype=torch.int32)
        counts[0] = T * k // E if (T * k) % E == 0 else counts[0]
        bias = (torch.rand(E, generator=gen) - 0.5) * 0.1
        shape = moe.Shape(T, 64, E, k, 64, 0, 0)
        b_d = bias.to(DEV)
        moe.moe_update_bias(shape, counts.to(DEV), b_d, 1e-3)
        torch.cuda.synchronize()
        ref = oracle.update_bias(counts.numpy(), bias.numpy(), T, k, 1e-3)
        assert np.array_equal(host(b_d).view(np.uint32), ref.view(np.uint32))


def test_layer_end_to_end_mini_2048_and_dense_formulation():
    wl = workloads.WORKLOADS["mini_2048"]
    shape = moe.Shape.of(wl)
    x, p = inputs(wl, DEV)
    g = gpu_host(run_layer(shape, x, p))
    hp = host_params(p)
    ref = oracle.layer(bits(x), hp, wl.top_k, wl.seq_len)
    check_routing(g, ref)
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(g[key], ref[key]), key
    check_bf16_close(g["out"], ref["out"], "mini_2048.out")
    rel = np.abs(g["seq_balance"] - ref["seq_balance"]) / ref["seq_balance"]
    assert rel.max() <= 1e-5
    # the pages' dense formulation (every expert on every token, masked) on a sample
    sample = np.arange(0, wl.tokens, 32)
    dense = oracle.dense_masked(bits(x)[sample], ref["gate"][sample], ref["idx"][sample],
                                hp["w1"], hp["w3"], hp["w2"], hp["ws1"], hp["ws3"], hp["ws2"])
    assert np.array_equal(dense, ref["out"][sample])
    check_bf16_close(g["out"][sample], dense, "mini_2048.out vs dense-masked")


# Degenerate shapes of the whole layer: one expert (k = E = 1, every gate
# exactly 1), one token, the narrowest dims the kernels take (d = H = 64), no
# shared expert, a shared expert narrower than the routed ones, every token
# in one sequence of odd length, and a ragged number of tokens around the
# 256-token permutation block.
DEGENERATE = {
    "E1_k1": custom(tokens=300, seq_len=100, d_model=64, n_experts=1, top_k=1, hidden=64,
                    shared_hidden=64, cfg_id=171, router_std=0.1),
    "T1_no_shared": custom(tokens=1, seq_len=1, d_model=128, n_experts=4, top_k=2, hidden=64,
                           shared_hidden=0, cfg_id=172, router_std=0.1),
    "E2_k2_d64": custom(tokens=257, seq_len=257, d_model=64, n_experts=2, top_k=2, hidden=128,
                        shared_hidden=64, cfg_id=173, router_std=0.1),
    "narrow_shared_T513": custom(tokens=513, seq_len=171, d_model=192, n_experts=12, top_k=3,
                                 hidden=192, shared_hidden=64, cfg_id=174, router_std=0.1),
}


@pytest.mark.parametrize("name", list(DEGENERATE))
def test_layer_degenerate_shapes(name):
    wl = DEGENERATE[name]
    say(f"[degenerate] {name}: T={wl.tokens} S={wl.seq_len} d={wl.d_model} E={wl.n_experts} "
        f"k={wl.top_k} H={wl.hidden} Hs={wl.shared_hidden}")
    shape = moe.Shape.of(wl)
    x, p = inputs(wl, DEV)
    g = gpu_host(run_layer(shape, x, p))
    ref = oracle.layer(bits(x), host_params(p), wl.top_k, wl.seq_len)
    check_routing(g, ref, name)
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(g[key], ref[key]), key
    if wl.top_k == 1:
        assert np.all(g["topk_gate"] == 1.0)
    check_bf16_close(g["out"], ref["out"], f"{name}.out")
    if wl.seq_len:
        rel = np.abs(g["seq_balance"] - ref["seq_balance"]) / np.abs(ref["seq_balance"])
        assert rel.max() <= 1e-5, rel.max()


def test_layer_is_deterministic_and_residual_path():
    wl = custom(tokens=1536, seq_len=256, cfg_id=131)
    shape = moe.Shape.of(wl)
    x, p = inputs(wl, DEV)
    a = gpu_host(run_layer(shape, x, p, residual=x))
    b = gpu_host(run_layer(shape, x, p, residual=x))
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    sample = np.arange(0, wl.tokens, 7)
    ref = oracle.layer(bits(x)[sample], host_params(p), wl.top_k, residual=bits(x)[sample])
    check_bf16_close(a["out"][sample], ref["out"], "residual.out")


# --------------------------------------------------------------------------
# Full-size workloads, in the launch configuration that bench.py times

def sampled_outputs(x, p_gpu, tokens, ref_idx, ref_gate, residual=None, cache=None):
    """Oracle outputs for a few tokens, copying only the experts they use."""
    import concurrent.futures as cf
    cache = {} if cache is None else cache

    def expert(e):
        if e not in cache:
            cache[e] = tuple(bits(p_gpu[n][e]) for n in ("w1", "w3", "w2"))
        return cache[e]

    xb = bits(x)
    shared = tuple(bits(p_gpu[n]) for n in ("ws1", "ws3", "ws2")) if "ws1" in p_gpu else None
    jobs = []
    for t in tokens:
        for j in range(ref_idx.shape[1]):
            jobs.append((t, j, ref_idx[t, j]))
    for _, _, e in jobs:
        expert(e)
    with cf.ThreadPoolExecutor(oracle.default_threads()) as ex:
        ys = list(ex.map(lambda job: oracle.expert_ffn(xb[job[0]], *expert(job[2])), jobs))
        ysh = list(ex.map(lambda t: oracle.expert_ffn(xb[t], *shared), tokens)) if shared else None
    k = ref_idx.shape[1]
    y_perm = np.stack(ys)
    pos = np.arange(len(tokens) * k, dtype=np.int32).reshape(len(tokens), k)
    res = None if residual is None else bits(residual)[tokens]
    return oracle.combine(y_perm, None if ysh is None else np.stack(ysh), ref_gate[tokens],
                          ref_idx[tokens], pos, res)


@pytest.fixture(scope="module")
def v3_weights():
    wl = workloads.WORKLOADS["v3_prefill_4096"]
    say("[v3] drawing 22.5 GB of expert weights on the GPU")
    p = workloads.layer_params(wl, 0, DEV)
    torch.cuda.synchronize()
    yield p
    del p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["v3_prefill_4096", "v3_decode_64"])
def test_v3_full_size(name, v3_weights):
    full_size_check(name, v3_weights)


def test_v3_local32_full_size():
    """The matrix-core-bound shape (about 1024 rows per expert)."""
    wl = workloads.WORKLOADS["v3_local32_4096"]
    say("[v3] drawing the 32 experts of v3_local32_4096 on the GPU")
    p = workloads.layer_params(wl, 0, DEV)
    full_size_check(wl.name, p)


def full_size_check(name, p):
    wl = workloads.WORKLOADS[name]
    shape = moe.Shape.of(wl)
    say(f"[v3] {name} T={wl.tokens}")
    x = workloads.tokens(wl, 0, DEV)
    bufs = run_layer(shape, x, p)
    g = gpu_host(bufs)
    ref = oracle.route(bits(x), host(p["w_router"]), host(p["bias"]), wl.top_k)
    same = check_routing(g, ref, name)
    idx_used = np.where(same[:, None], ref["idx"], g["topk_idx"])  # adopt GPU's near-tie choices
    pm = oracle.permute(idx_used, wl.n_experts)
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(g[key], pm[key]), key
    if wl.seq_len:
        L = oracle.seq_balance(ref["scores"], g["topk_idx"], wl.seq_len, 1e-4)
        assert np.abs(g["seq_balance"] - L).max() / np.abs(L).max() <= 1e-5
    sample = np.unique(np.linspace(0, wl.tokens - 1, 12).astype(int))
    sample = sample[same[sample]]
    out = sampled_outputs(x, p, sample, ref["idx"], ref["gate"])
    check_bf16_close(g["out"][sample], out, f"{name}.out[sampled {len(sample)} tokens]")
    assert g["y_perm"].shape == (wl.tokens * wl.top_k, wl.d_model)
    # every row of the largest, the smallest and a median expert group (each
    # group is one m-tile of the weight-streaming tile at prefill), so that
    # all of a tile's row passes and output columns are compared
    counts = g["counts"]
    used = np.nonzero(counts)[0]
    order = used[np.argsort(counts[used], kind="stable")]
    xb = bits(x)
    for e in sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])}):
        lo, hi = int(g["offsets"][e]), int(g["offsets"][e + 1])
        rows = g["perm_src"][lo:hi]
        ref_e = oracle.grouped_ffn(xb[rows], np.arange(hi - lo, dtype=np.int32),
                                   np.array([0, hi - lo], np.int32), bits(p["w1"][e])[None],
                                   bits(p["w3"][e])[None], bits(p["w2"][e])[None])
        check_bf16_close(g["y_perm"][lo:hi], ref_e["y_perm"], f"{name}.y_perm[expert {e}, {hi - lo} rows]")
    # shared-expert rows spread over all of its m-tiles (at prefill it runs as
    # a launch of its own)
    if wl.shared_hidden:
        rows = np.unique(np.linspace(0, wl.tokens - 1, 16).astype(int))
        shared = tuple(bits(p[n]) for n in ("ws1", "ws3", "ws2"))
        ysh = np.stack([oracle.expert_ffn(xb[t], *shared) for t in rows])
        check_bf16_close(g["y_shared"][rows], ysh, f"{name}.y_shared[{len(rows)} rows]")


# Layers whose x_perm and y_perm (and in the first case h) exceed 2 GiB: the
# grouped GEMM addresses a tile's own rows of x_perm and h from the tile's
# first row, so 32-bit offsets suffice however large those buffers are.
#   wide_k_eq_E: every token to all 8 experts, 80 000 tokens at d = 7168,
#     H = 2048: x_perm and y_perm 9.2 GB, h 2.6 GB, the 256x128 loader-wave tile;
#   wide_stream: 1024 experts of H = 256 (weights 11.3 GB), 200 rows each:
#     the weight-streaming tile, x_perm 2.9 GB.
WIDE_CASES = {
    "wide_k_eq_E": custom(tokens=80000, d_model=7168, n_experts=8, top_k=8, hidden=2048,
                          shared_hidden=2048, cfg_id=161, w_std=0.006, router_std=0.006,
                          bias_range=0.01),
    "wide_stream": custom(tokens=25600, d_model=7168, n_experts=1024, top_k=8, hidden=256,
                          shared_hidden=256, cfg_id=162, w_std=0.006, router_std=0.006,
                          bias_range=0.01),
}


@pytest.mark.parametrize("name", list(WIDE_CASES))
def test_forward_beyond_32bit_operand_offsets(name):
    wl = WIDE_CASES[name]
    x, p = inputs(wl, DEV)
    wide_layer_check(wl, x, p)


def test_v3_prefill_32768_sampled(v3_weights):
    """The V3 layer over 32768 tokens (about 1024 rows per expert), on the
    prefill's weights: routing and permutation of every token against the
    oracle's integer work, sampled tokens and rows against the oracle."""
    wl = workloads.WORKLOADS["v3_prefill_32768"]
    assert wl.weight_cfg_id == workloads.WORKLOADS["v3_prefill_4096"].weight_cfg_id
    x = workloads.tokens(wl, 0, DEV)
    wide_layer_check(wl, x, v3_weights)


def wide_layer_check(wl, x, p):
    """Run the layer with x_perm and with the gather through perm_src (the two
    must agree bit for bit), then compare sampled tokens' routing and outputs
    and y_perm rows on both sides of x_perm's 2 GiB byte offset with the oracle."""
    shape = moe.Shape.of(wl)
    name = wl.name
    T, d, k = wl.tokens, wl.d_model, wl.top_k
    assert 2 * T * k * d >= 1 << 31  # refused before the per-tile descriptors
    say(f"[wide] {name}: T={T} E={wl.n_experts} k={k} H={wl.hidden}, x_perm "
        f"{2 * T * k * d / 1e9:.1f} GB")
    bufs = run_layer(shape, x, p, use_x_perm=True)
    y_perm_xp = bufs["y_perm"].clone()
    out_xp = bufs["out"].clone()
    run_layer(shape, x, p, use_x_perm=False, bufs=bufs)  # rows gathered through perm_src
    assert torch.equal(bufs["y_perm"], y_perm_xp) and torch.equal(bufs["out"], out_xp)
    del y_perm_xp, out_xp
    idx = host(bufs["topk_idx"])
    perm_src = host(bufs["perm_src"])
    offsets = host(bufs["offsets"])
    pm = oracle.permute(idx, wl.n_experts)  # the oracle's grouping of the GPU's choices
    for key in ("counts", "offsets", "perm_src", "pos"):
        assert np.array_equal(host(bufs[key]), pm[key]), key
    xb = bits(x)
    if wl.seq_len:  # the last sequence: every token's routing and its balance statistic
        S = wl.seq_len
        last = oracle.route(xb[T - S:], host(p["w_router"]), host(p["bias"]), k)
        g_last = {key: host(bufs[key])[T - S:] for key in ("topk_idx", "topk_gate", "margin")}
        check_routing(g_last, last, f"{name}.route[last sequence]")
        L = oracle.seq_balance(last["scores"], idx[T - S:], S, 1e-4)
        got = host(bufs["seq_balance"])[-1:]
        assert np.abs(got - L).max() / np.abs(L).max() <= 1e-5, (got, L)
    # routing of sampled tokens, and their whole layer output
    sample = np.unique(np.linspace(0, T - 1, 9).astype(int))
    ref = oracle.route(xb[sample], host(p["w_router"]), host(p["bias"]), k)
    near = ref["margin"] < 1e-6
    same = np.all(idx[sample] == ref["idx"], axis=1)
    assert (same | near).all()
    sample, ref_idx = sample[same], ref["idx"][same]
    ref_gate = np.zeros((T, k), np.float32)
    full_idx = np.zeros((T, k), np.int32)
    ref_gate[sample], full_idx[sample] = ref["gate"][same], ref_idx
    out = sampled_outputs(x, p, sample, full_idx, ref_gate)
    got = bits(bufs["out"][torch.as_tensor(sample, device=DEV)])
    check_bf16_close(got, out, f"{name}.out[sampled {len(sample)} tokens]")
    # y_perm rows at both sides of the 2 GiB byte offset of x_perm and at the end
    edge = (1 << 31) // (2 * d)
    rows = sorted({0, edge - 1, edge, edge + 1, T * k - 1})
    ys = []
    for r in rows:
        e = int(np.searchsorted(offsets, r, side="right") - 1)
        ys.append(oracle.expert_ffn(xb[perm_src[r]], bits(p["w1"][e]), bits(p["w3"][e]),
                                    bits(p["w2"][e])))
    got = bits(bufs["y_perm"][torch.as_tensor(rows, device=DEV)])
    check_bf16_close(got, np.stack(ys), f"{name}.y_perm[rows {rows}]")


def test_mini_train_stacked_layers_teacher_forced():
    """Six stacked layers with the residual stream, two steps with the bias
    update in between; the oracle is fed the GPU's layer inputs and biases."""
    wl = workloads.WORKLOADS["mini_train_8192x6"]
    shape = moe.Shape.of(wl)
    params = [workloads.layer_params(wl, l, DEV) for l in range(wl.layers)]
    bufs = [moe.alloc_buffers(shape, DEV) for _ in range(wl.layers)]
    sample = np.arange(0, wl.tokens, 61)
    for step in range(2):
        x = workloads.tokens(wl, step, DEV)
        for l in range(wl.layers):
            say(f"[stack] step {step} layer {l}")
            b_before = host(params[l]["bias"]).copy()
            moe.layer_forward(shape, x, params[l], bufs[l], residual=x)
            torch.cuda.synchronize()
            g = gpu_host(bufs[l])
            hp = host_params(params[l])
            hp["bias"] = b_before
            ref = oracle.route(bits(x), hp["w_router"], b_before, wl.top_k)
            check_routing(g, ref, f"step{step}.layer{l}")
            pm = oracle.permute(g["topk_idx"], wl.n_experts)
            assert np.array_equal(g["counts"], pm["counts"])
            lo = oracle.layer(bits(x)[sample], hp, wl.top_k, residual=bits(x)[sample])
            check_bf16_close(g["out"][sample], lo["out"], f"step{step}.layer{l}.out")
            x = bufs[l]["out"].clone()
        for l in range(wl.layers):
            b_before = host(params[l]["bias"]).copy()
            moe.moe_update_bias(shape, bufs[l]["counts"], params[l]["bias"], 1e-3)
            torch.cuda.synchronize()
            ref_b = oracle.update_bias(host(bufs[l]["counts"]), b_before, wl.tokens, wl.top_k)
            assert np.array_equal(host(params[l]["bias"]), ref_b)


def test_imbalanced_bias_chain_200_steps():
    """Routing + loads + bias update for 200 steps on the imbalanced workload.
    Bias bit-exact every step (teacher-forced); the load spread narrows."""
    wl = workloads.WORKLOADS["mini_imbalanced_8192"]
    shape = moe.Shape.of(wl)
    w_r = workloads.router(wl, 0, DEV)
    bias = workloads.bias(wl, 0, DEV)
    bufs = moe.alloc_buffers(shape, DEV)
    w_host = host(w_r)
    shares = []
    near_total = 0
    for step in range(wl.steps):
        x = workloads.tokens(wl, step, DEV)
        b_before = host(bias).copy()
        moe.moe_route(shape, x, w_r, bias, bufs["topk_idx"], bufs["topk_gate"], bufs["margin"],
                      None, 1e-4, bufs["workspace"])
        moe.moe_permute(shape, bufs["topk_idx"], bufs["counts"], bufs["offsets"],
                        bufs["perm_src"], bufs["pos"], None, None, bufs["workspace"])
        moe.moe_update_bias(shape, bufs["counts"], bias, 1e-3)
        torch.cuda.synchronize()
        g = {"topk_idx": host(bufs["topk_idx"]), "topk_gate": host(bufs["topk_gate"]),
             "margin": host(bufs["margin"])}
        ref = oracle.route(bits(x), w_host, b_before, wl.top_k)
        near = ref["margin"] < 1e-6
        near_total += int(near.sum())
        same = np.all(g["topk_idx"] == ref["idx"], 1)
        assert np.all(same | near), step
        idx_used = np.where(same[:, None], ref["idx"], g["topk_idx"])
        counts = np.bincount(idx_used.ravel(), minlength=wl.n_experts).astype(np.int32)
        assert np.array_equal(counts, host(bufs["counts"])), step
        ref_b = oracle.update_bias(counts, b_before, wl.tokens, wl.top_k)
        assert np.array_equal(host(bias).view(np.uint32), ref_b.view(np.uint32)), step
        shares.append(counts / (wl.tokens * wl.top_k))
    s0, s1 = shares[0], shares[-1]
    say(f"  expert share step 0: {s0.min():.4f}..{s0.max():.4f}; step {wl.steps - 1}: "
        f"{s1.min():.4f}..{s1.max():.4f}; near-tie tokens {near_total}")
    assert s0.min() < 0.01 and s0.max() > 0.15          # strongly imbalanced at the start
    assert s1.max() - s1.min() < 0.5 * (s0.max() - s0.min())  # bias pulls loads together
