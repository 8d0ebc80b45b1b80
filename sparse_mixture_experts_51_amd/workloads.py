"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module only *draws* tensors: token activations, router weights, the
per-expert balancing bias and the expert weights, for five named workloads
and for ad-hoc test shapes.  It holds none of the layer's arithmetic.  Both
the HIP path and the CPU oracle receive their inputs from here, so that the
two sides never share anything but the data they are compared on.

Workload shapes follow the pages:
  * the mini model: 16 routed experts, top-4, one always-on shared expert
    (190行JAX复刻DeepSeek V3, section 190行代码到底装进了什么; DeepSeek V3 viết
    lại bằng 190 dòng JAX thuần, section Những gì có trong 190 dòng code);
    training batches of 256-token sequences (same page, comparison table in
    先说结论);
  * the official DeepSeek-V3 shape: 256 routed experts, 8 per token, one
    shared expert (190行JAX复刻DeepSeek V3, comparison table in 先说结论).
Sizes that the pages leave open (d_model, hidden sizes, value
distributions) are fixed here and listed with their reasons in the design
notes.

Seeds: seed = 51000 + 100*cfg + 10*layer + role + 1000*(expert+1)
             + 10_000_000*step
where role is one of the ROLE_* constants and expert is -1 for tensors that
are not per-expert.  Every expert is drawn from its own generator, so any
single expert can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

ROLE_X = 0
ROLE_ROUTER = 1
ROLE_BIAS = 2
ROLE_W1 = 3
ROLE_W3 = 4
ROLE_W2 = 5
ROLE_WS1 = 6
ROLE_WS3 = 7
ROLE_WS2 = 8
ROLE_IMBALANCE = 9
ROLE_NORM = 10


def seed_of(cfg: int, layer: int, role: int, expert: int = -1, step: int = 0) -> int:
    return 51000 + 100 * cfg + 10 * layer + role + 1000 * (expert + 1) + 10_000_000 * step


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int          # seed namespace of the activations
    weight_cfg_id: int   # seed namespace of the weights (decode reuses prefill's)
    tokens: int
    seq_len: int         # 0: no sequence structure (balance statistic off)
    d_model: int
    n_experts: int
    top_k: int
    hidden: int
    shared_hidden: int   # 0: no shared expert
    layers: int
    steps: int
    x_std: float
    w_std: float
    router_std: float
    bias_kind: str       # "zero" or "uniform"
    bias_range: float
    imbalance: float     # 0: none; else half-width c of the per-expert logit offsets
    description: str = ""
    norm: bool = False   # pre-norm residual block: x + MoE(RMSNorm(x))

    @property
    def rows(self) -> int:
        """Routed rows T*k plus shared rows T."""
        return self.tokens * self.top_k + (self.tokens if self.shared_hidden else 0)


WORKLOADS = {
    "mini_2048": Workload(
        "mini_2048", 1, 1, 2048, 256, 384, 16, 4, 256, 256, 1, 1,
        1.0, 0.02, 0.02, "zero", 0.0, 0.0,
        "mini DeepSeekMoE layer, 8 seqs x 256 tokens, bias 0"),
    "mini_train_8192x6": Workload(
        "mini_train_8192x6", 2, 2, 8192, 256, 384, 16, 4, 256, 256, 6, 10,
        1.0, 0.02, 0.02, "uniform", 0.05, 0.0,
        "mini-model training batch, 32 seqs x 256 tokens, 6 stacked layers"),
    "mini_imbalanced_8192": Workload(
        "mini_imbalanced_8192", 3, 3, 8192, 256, 384, 16, 4, 256, 256, 1, 200,
        1.0, 0.02, 0.02, "zero", 0.0, 0.7,
        "imbalanced routing stress: per-expert logit offsets, 200 bias steps"),
    "v3_prefill_4096": Workload(
        "v3_prefill_4096", 4, 4, 4096, 4096, 7168, 256, 8, 2048, 2048, 1, 1,
        1.0, 0.006, 0.006, "uniform", 0.01, 0.0,
        "DeepSeek-V3-shaped prefill layer, one 4096-token sequence"),
    "v3_decode_64": Workload(
        "v3_decode_64", 5, 4, 64, 0, 7168, 256, 8, 2048, 2048, 1, 1,
        1.0, 0.006, 0.006, "uniform", 0.01, 0.0,
        "DeepSeek-V3-shaped decode step, 64 independent tokens"),
    # The same V3-shaped layer (the prefill's weights) over eight 4096-token
    # sequences: about 1024 rows per expert, past the ridge of the bf16
    # matrix cores (about 1100 FLOP per byte of weights), so the whole layer,
    # not only one GPU's expert-parallel share, is matrix-core-bound.
    "v3_prefill_32768": Workload(
        "v3_prefill_32768", 8, 4, 32768, 4096, 7168, 256, 8, 2048, 2048, 1, 1,
        1.0, 0.006, 0.006, "uniform", 0.01, 0.0,
        "DeepSeek-V3-shaped prefill layer, 8 sequences x 4096 tokens (~1024 rows per expert)"),
    # The grouped-FFN shape one GPU holds under 8-way expert parallelism of the
    # V3 layer (32 of the 256 experts, about 1024 rows each, the shared expert
    # on the GPU's own 4096 tokens), built as a layer of 32 experts with top-8
    # routing over 4096 tokens: the matrix-core-bound regime of the layer.
    "v3_local32_4096": Workload(
        "v3_local32_4096", 6, 6, 4096, 4096, 7168, 32, 8, 2048, 2048, 1, 1,
        1.0, 0.006, 0.006, "uniform", 0.01, 0.0,
        "V3 dims, 32 local experts top-8 over 4096 tokens (~1024 rows per expert)"),
    # The pages' small configuration: 4 layers, 8 experts, top-2 routing and a
    # 128-token context (190行JAX复刻DeepSeek V3, section 如何在Mac上复现), as
    # pre-norm residual blocks over 32 sequences; d_model and the expert
    # sizes are the mini model's (the pages do not give them).
    "small_block_4096x4": Workload(
        "small_block_4096x4", 7, 7, 4096, 128, 384, 8, 2, 256, 256, 4, 10,
        1.0, 0.02, 0.02, "uniform", 0.05, 0.0,
        "small configuration: 4 pre-norm blocks, 8 experts top-2, 32 seqs x 128 tokens",
        norm=True),
}

DEFAULT_BENCH_WORKLOAD = "v3_prefill_4096"


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) draws in fp32, then cast (bf16 casts round to nearest even)."""
    g = _gen(device, seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    t = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def tokens(wl: Workload, step: int = 0, device="cpu", layer: int = 0) -> torch.Tensor:
    """x[T, d] bf16.  The imbalance workload pins channel d-1 to 1.0 so that the
    router's last row acts as a per-expert logit offset."""
    x = normal((wl.tokens, wl.d_model), wl.x_std,
               seed_of(wl.cfg_id, layer, ROLE_X, step=step), device, torch.bfloat16)
    if wl.imbalance:
        x[:, wl.d_model - 1] = 1.0
    return x


def router(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """W_r[d, E] fp32; with imbalance, row d-1 holds a seeded permutation of
    linspace(-c, c, E)."""
    w = normal((wl.d_model, wl.n_experts), wl.router_std,
               seed_of(wl.weight_cfg_id, layer, ROLE_ROUTER), device)
    if wl.imbalance:
        c = wl.imbalance
        lin = torch.linspace(-c, c, wl.n_experts, dtype=torch.float32)
        perm = torch.randperm(wl.n_experts, generator=_gen("cpu", seed_of(
            wl.weight_cfg_id, layer, ROLE_IMBALANCE)))
        w[wl.d_model - 1] = lin[perm].to(device)
    return w


def bias(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    if wl.bias_kind == "zero":
        return torch.zeros(wl.n_experts, dtype=torch.float32, device=device)
    r = wl.bias_range
    return uniform((wl.n_experts,), -r, r, seed_of(wl.weight_cfg_id, layer, ROLE_BIAS), device)


def expert_weights(wl: Workload, layer: int = 0, device="cpu",
                   experts: Optional[list] = None) -> dict:
    """Routed expert weights: w1, w3 [E, H, d] and w2 [E, d, H], bf16.
    Each expert comes from its own generator.  `experts` restricts the draw to
    a subset (the others stay zero), for host copies of a few experts."""
    E, H, d = wl.n_experts, wl.hidden, wl.d_model
    out = {}
    for name, role, shape in _EXPERT_ROLES:
        t = torch.zeros((E,) + shape(H, d), dtype=torch.bfloat16, device=device)
        for e in (range(E) if experts is None else experts):
            t[e] = normal(shape(H, d), wl.w_std, seed_of(wl.weight_cfg_id, layer, role, e),
                          device, torch.bfloat16)
        out[name] = t
    return out


_EXPERT_ROLES = (("w1", ROLE_W1, lambda H, d: (H, d)), ("w3", ROLE_W3, lambda H, d: (H, d)),
                 ("w2", ROLE_W2, lambda H, d: (d, H)))


def one_expert(wl: Workload, e: int, layer: int = 0, device="cpu") -> dict:
    """Expert e's w1, w3 [H, d] and w2 [d, H] alone: the same values as
    expert_weights(...)[name][e], without the [E, ...] tensors."""
    H, d = wl.hidden, wl.d_model
    return {name: normal(shape(H, d), wl.w_std, seed_of(wl.weight_cfg_id, layer, role, e),
                         device, torch.bfloat16) for name, role, shape in _EXPERT_ROLES}


def shared_weights(wl: Workload, layer: int = 0, device="cpu") -> dict:
    """Shared expert weights ws1, ws3 [Hs, d] and ws2 [d, Hs], bf16 (empty dict
    when the workload has no shared expert)."""
    if not wl.shared_hidden:
        return {}
    Hs, d = wl.shared_hidden, wl.d_model
    return {
        "ws1": normal((Hs, d), wl.w_std, seed_of(wl.weight_cfg_id, layer, ROLE_WS1), device, torch.bfloat16),
        "ws3": normal((Hs, d), wl.w_std, seed_of(wl.weight_cfg_id, layer, ROLE_WS3), device, torch.bfloat16),
        "ws2": normal((d, Hs), wl.w_std, seed_of(wl.weight_cfg_id, layer, ROLE_WS2), device, torch.bfloat16),
    }


def norm_gain(wl: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """RMSNorm gain [d] fp32, N(1, 0.1^2): the spread of a trained gain, so
    that a gain applied to the wrong column shows."""
    g = normal((wl.d_model,), 0.1, seed_of(wl.weight_cfg_id, layer, ROLE_NORM), device)
    return g.add_(1.0)


def layer_params(wl: Workload, layer: int = 0, device="cpu") -> dict:
    p = {"w_router": router(wl, layer, device), "bias": bias(wl, layer, device)}
    if wl.norm:
        p["norm"] = norm_gain(wl, layer, device)
    p.update(expert_weights(wl, layer, device))
    p.update(shared_weights(wl, layer, device))
    return p


def custom(name: str = "custom", tokens: int = 1000, seq_len: int = 0, d_model: int = 384,
           n_experts: int = 16, top_k: int = 4, hidden: int = 256, shared_hidden: int = 256,
           cfg_id: int = 90, x_std: float = 1.0, w_std: float = 0.02, router_std: float = 0.02,
           bias_kind: str = "uniform", bias_range: float = 0.05, imbalance: float = 0.0) -> Workload:
    """An ad-hoc shape for tests (ragged tails, edge cases)."""
    return Workload(name, cfg_id, cfg_id, tokens, seq_len, d_model, n_experts, top_k, hidden,
                    shared_hidden, 1, 1, x_std, w_std, router_std, bias_kind, bias_range,
                    imbalance, "test shape")


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Reinterpret a bf16 tensor as its uint16 bit patterns (int16 storage)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


# ---------------------------------------------------------------- MLA attention

ROLE_MLA_X = 20
ROLE_MLA_W = 21   # + index into MLA_WEIGHT_ROLES
ROLE_MLA_RES = 28
ROLE_MLA_POS = 29
MLA_WEIGHT_ROLES = ("w_q", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")


@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    """The attention half of the mini block: 6 heads, a 128-number latent
    and a 16-number shared rotary key per token, 32-number content keys and
    values per head, 256-token context (190行JAX复刻DeepSeek V3, sections
    190行代码到底装进了什么 and 先说结论); d_model 384 as for the MoE."""
    name: str
    cfg_id: int
    batch: int           # sequences
    seq_len: int         # prefill: tokens per sequence; decode: cached tokens before the new one
    max_len: int
    decode: bool
    d_model: int = 384
    n_heads: int = 6
    d_latent: int = 128
    d_nope: int = 32
    d_rope: int = 16
    d_v: int = 32
    x_std: float = 1.0
    w_std: float = 0.05
    description: str = ""

    @property
    def tokens(self) -> int:
        """Token rows of one call."""
        return self.batch if self.decode else self.batch * self.seq_len


MLA_WORKLOADS = {
    "mla_prefill_32x256": MlaWorkload(
        "mla_prefill_32x256", 30, 32, 256, 256, False,
        description="MLA prefill of a mini training batch: 32 sequences x 256 tokens"),
    "mla_decode_256x256": MlaWorkload(
        "mla_decode_256x256", 31, 256, 255, 256, True,
        description="MLA decode step of 256 sequences at position 255 (255 cached tokens each)"),
    # A long context, where reading the 144-number-per-token cache dominates
    # the step (256 x 4096 x 144 bf16 = 302 MB).
    "mla_decode_256x4096": MlaWorkload(
        "mla_decode_256x4096", 32, 256, 4095, 4096, True,
        description="MLA decode step of 256 sequences at position 4095 (4095 cached tokens each)"),
}


def mla_custom(name="mla_custom", cfg_id=40, batch=2, seq_len=70, max_len=80, decode=False, **kw):
    return MlaWorkload(name, cfg_id, batch, seq_len, max_len, decode, **kw)


def mla_params(wl: MlaWorkload, layer: int = 0, device="cpu") -> dict:
    """The six MLA weights, bf16, N(0, w_std^2), stored [N, K]."""
    H, d = wl.n_heads, wl.d_model
    shapes = {"w_q": (H * (wl.d_nope + wl.d_rope), d), "w_dkv": (wl.d_latent, d),
              "w_kr": (wl.d_rope, d), "w_uk": (H * wl.d_nope, wl.d_latent),
              "w_uv": (H * wl.d_v, wl.d_latent), "w_o": (d, H * wl.d_v)}
    return {k: normal(shapes[k], wl.w_std, seed_of(wl.cfg_id, layer, ROLE_MLA_W + i), device,
                      torch.bfloat16)
            for i, k in enumerate(MLA_WEIGHT_ROLES)}


def mla_tokens(wl: MlaWorkload, rows: int, step: int = 0, device="cpu") -> torch.Tensor:
    """Token rows (bf16, N(0, x_std^2)) for a prefill of rows tokens or a
    decode step of rows sequences."""
    return normal((rows, wl.d_model), wl.x_std, seed_of(wl.cfg_id, 0, ROLE_MLA_X, step=step),
                  device, torch.bfloat16)


def mla_residual(wl: MlaWorkload, rows: int, device="cpu") -> torch.Tensor:
    return normal((rows, wl.d_model), 1.0, seed_of(wl.cfg_id, 0, ROLE_MLA_RES), device,
                  torch.bfloat16)
