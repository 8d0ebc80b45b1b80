"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
on seeded inputs, hand the same inputs to the oracle, compare.

Tolerances (the layer's float outputs are bf16 with fp32 accumulation):
  max|err| <= 2e-2 * max|ref|  and  mean|err| <= 2e-3
Indices, counts, offsets, permutation and bias: bit-exact.  Tokens whose
k-th/(k+1)-th key margin is below 1e-6 are reported and left out of the
index check; gates: |diff| <= 1e-6.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_mixture_experts_51_amd import moe, workloads

NEAR_TIE = 1e-6
GATE_TOL = 1e-6
MAX_REL = 2e-2
MEAN_ABS = 2e-3


def bits(t: torch.Tensor) -> np.ndarray:
    return oracle.as_bf16_bits(t)


def f32(b: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(b)


def host(t):
    return None if t is None else t.detach().cpu().numpy()


def say(*a):
    print(*a, flush=True)


def check_bf16_close(gpu_bits, ref_bits, what: str):
    g = f32(np.asarray(gpu_bits)).astype(np.float64)
    r = f32(np.asarray(ref_bits)).astype(np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(r).all() and np.isfinite(g).all(), what
    err = np.abs(g - r)
    mx, mean = err.max(initial=0.0), err.mean() if err.size else 0.0
    ref_max = np.abs(r).max(initial=0.0)
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    say(f"  {what}: max|err|={mx:.3e} (bound {MAX_REL * ref_max:.3e}) mean|err|={mean:.3e} "
        f"rel_l2={rel_l2:.3e}")
    assert mx <= MAX_REL * ref_max + 1e-30, what
    assert mean <= MEAN_ABS, what
    return {"max_err": mx, "mean_err": mean, "rel_l2": rel_l2}


def check_routing(gpu: dict, ref: dict, what: str = "route"):
    """idx exact outside near-ties, gates within 1e-6, margin exact where the
    choices agree.  Returns the mask of tokens whose choices agree."""
    idx_g, idx_r = gpu["topk_idx"], ref["idx"]
    near = ref["margin"] < NEAR_TIE
    same = np.all(idx_g == idx_r, axis=1)
    bad = ~same & ~near
    say(f"  {what}: tokens={len(same)} near-ties={int(near.sum())} "
        f"differing(outside near-ties)={int(bad.sum())} differing(near-ties)={int((~same & near).sum())}")
    assert not bad.any(), np.nonzero(bad)[0][:10]
    gd = np.abs(gpu["topk_gate"][same] - ref["gate"][same])
    assert (gd.max(initial=0.0) <= GATE_TOL), gd.max()
    mg, mr = gpu["margin"][same], ref["margin"][same]
    assert np.array_equal(np.isnan(mg), np.isnan(mr))
    ok = ~np.isnan(mr)
    assert np.array_equal(mg[ok], mr[ok])
    return same


def inputs(wl, device="cuda", layer: int = 0, step: int = 0) -> tuple:
    x = workloads.tokens(wl, step, device, layer)
    p = workloads.layer_params(wl, layer, device)
    return x, p


def host_params(p: dict) -> dict:
    out = {}
    for k, v in p.items():
        out[k] = bits(v) if v.dtype == torch.bfloat16 else host(v)
    return out


def run_layer(shape: moe.Shape, x, p, residual=None, use_x_perm=False, bufs=None) -> dict:
    bufs = bufs or moe.alloc_buffers(shape, x.device, x_perm=use_x_perm)
    moe.layer_forward(shape, x, p, bufs, residual=residual, use_x_perm=use_x_perm)
    torch.cuda.synchronize()
    return bufs


def gpu_host(bufs: dict) -> dict:
    out = {}
    for k, v in bufs.items():
        if v is None or k == "workspace":
            continue
        out[k] = bits(v) if v.dtype == torch.bfloat16 else host(v)
    return out
