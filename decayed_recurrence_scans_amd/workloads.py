"""Seeded synthetic inputs for the decayed-recurrence workloads.

This module holds none of the method's arithmetic: only random draws, dtype
casts (round-to-nearest-even into bfloat16), and -- for the continuation
workload -- the synthesis of a carried state from a random preceding segment
by a plain matrix product and a plain sum.  It is the one module that both the
HIP path's callers and the fp64 oracle's callers share, so that both sides see
bit-identical inputs.

Every draw comes from ``torch.Generator('cpu').manual_seed(seed)`` in a fixed
order (q, k, v, then decay / w / u / outlier masks, then any prefix segment),
so a (config, seed) pair names one exact input.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

__all__ = [
    "LAConfig", "WKVConfig", "EMAConfig", "LA_CONFIGS", "WKV_CONFIGS", "EMA_CONFIGS",
    "la_inputs", "wkv_inputs", "ema_inputs", "retention_gammas", "to_dtype", "output_gradients",
]


@dataclass(frozen=True)
class LAConfig:
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    dtype: str            # "f32" | "bf16"
    mode: str             # "none" | "head" | "step" | "elem"
    normalize: bool
    dist: str             # "quarter" | "scaled" | "elu1"
    seed: int
    prefix: int = 0       # length of the preceding segment summarised into S0/cum_k0
    reverse: tuple = (False,)
    chunk: int = 64
    random_state: bool = False   # S0 ~ N(0,1), cum_k0 ~ |N(0,1)| * Dk
    bidirectional: bool = False  # forward + reverse, summed
    in_place: bool = False       # state_out / cum_k_out are state_in / cum_k_in
    backward: bool = False       # the gradients, given dy ~ N(0,1)
    description: str = ""


@dataclass(frozen=True)
class WKVConfig:
    name: str
    B: int
    T: int
    C: int
    seed: int
    outlier_frac: float = 0.01
    outlier: float = 60.0
    backward: bool = False       # the gradients, given dy ~ N(0,1)
    description: str = ""


@dataclass(frozen=True)
class EMAConfig:
    name: str
    B: int
    T: int
    C: int
    dtype: str            # "f32" | "bf16"
    seed: int
    reverse: tuple = (False, True)
    bidirectional: bool = False  # forward + reverse, summed
    description: str = ""


LA_CONFIGS = {
    "plain_f32": LAConfig(
        "plain_f32", B=2, H=2, T=64, Dk=16, Dv=16, dtype="f32", mode="none",
        normalize=False, dist="quarter", seed=1,
        description="plain causal linear attention, fp32, q/k/v ~ N(0,1)/4, zero state"),
    "retention_bf16": LAConfig(
        "retention_bf16", B=8, H=8, T=2048, Dk=64, Dv=64, dtype="bf16", mode="head",
        normalize=False, dist="scaled", seed=2, reverse=(False, True),
        description="retention, scalar per-head decay 1-2^(-5-h), bf16 q/k/v ~ N(0,1)/sqrt(Dk), "
                    "zero state, forward and reverse scans"),
    "normalized_bf16": LAConfig(
        "normalized_bf16", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16", mode="none",
        normalize=True, dist="elu1", seed=3, prefix=1024,
        description="normalized linear attention, q/k = elu(N)+1, v ~ N(0,1), bf16, continuing "
                    "from S0/cum_k0 summed over a preceding random 1024-token segment"),
    "step_decay_bf16": LAConfig(
        "step_decay_bf16", B=4, H=16, T=16384, Dk=128, Dv=128, dtype="bf16", mode="step",
        normalize=False, dist="scaled", seed=5,
        description="data-dependent per-step decay sigmoid(N(3,1)), bf16 q/k/v ~ N(0,1)/sqrt(Dk), "
                    "fp32 state, chunk 64, zero state"),
    # One generation step (the cached-state case of flash-linear-attention issue
    # #268): a batch of 64 sequences at the normalized workload's head shape, each
    # feeding one new token with its carried fp32 state and key sum.
    "decode_bf16": LAConfig(
        "decode_bf16", B=64, H=16, T=1, Dk=128, Dv=128, dtype="bf16", mode="head",
        normalize=True, dist="elu1", seed=7, random_state=True, in_place=True,
        description="decode step: T=1, normalized, per-head decay 1-2^(-5-h), q/k = elu(N)+1, "
                    "v ~ N(0,1), bf16, carried fp32 state ~ N(0,1) and key sum |N|*Dk, updated in place"),
    # Per-key-channel decay (a factor per (b, h, t, channel), cumulative_ema's
    # factors of the values' own shape) at the normalized workload's head shape.
    "elem_decay_bf16": LAConfig(
        "elem_decay_bf16", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16", mode="elem",
        normalize=False, dist="scaled", seed=11,
        description="per-key-channel decay sigmoid(N(3,1)) per (b,h,t,channel) fp32, bf16 q/k/v ~ "
                    "N(0,1)/sqrt(Dk), zero state"),
    # The backward of the retention workload (both directions), with an output
    # gradient dy ~ N(0,1) in bf16.
    "backward_retention_bf16": LAConfig(
        "backward_retention_bf16", B=8, H=8, T=2048, Dk=64, Dv=64, dtype="bf16", mode="head",
        normalize=False, dist="scaled", seed=10, reverse=(False, True), backward=True,
        description="retention backward: dq, dk, dv, per-head decay gradient and initial-state gradient "
                    "for the forward and the reverse scan, bf16 q/k/v ~ N(0,1)/sqrt(Dk), dy ~ N(0,1), zero state"),
    # The backward of the normalized workload (its dq, dk, dv, the initial state's and
    # key sum's gradients), with final-state and key-sum gradients ~ N(0,1).
    "backward_normalized_bf16": LAConfig(
        "backward_normalized_bf16", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16", mode="none",
        normalize=True, dist="elu1", seed=3, prefix=1024, backward=True,
        description="normalized linear attention backward: dq, dk, dv and the gradients of S0 and cum_k0, "
                    "q/k = elu(N)+1, v ~ N(0,1), bf16, continuing from a 1024-token prefix, "
                    "dy, dS_final, dz_final ~ N(0,1)"),
    # The backward of the per-key-channel decay workload (with the factors' gradient).
    "backward_elem_bf16": LAConfig(
        "backward_elem_bf16", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16", mode="elem",
        normalize=False, dist="scaled", seed=11, backward=True,
        description="per-key-channel decay backward: dq, dk, dv and the gradient of every factor, "
                    "sigmoid(N(3,1)) factors per (b,h,t,channel), bf16 q/k/v ~ N(0,1)/sqrt(Dk), "
                    "dy ~ N(0,1), zero state"),
    # The bidirectional encoder (RetNet issue #21) at the retention workload's shape.
    "bidir_retention_bf16": LAConfig(
        "bidir_retention_bf16", B=8, H=8, T=2048, Dk=64, Dv=64, dtype="bf16", mode="head",
        normalize=False, dist="scaled", seed=8, bidirectional=True,
        description="bidirectional retention (forward + reverse summed), per-head decay 1-2^(-5-h), "
                    "bf16 q/k/v ~ N(0,1)/sqrt(Dk), zero state"),
}

WKV_CONFIGS = {
    "wkv_f32": WKVConfig(
        "wkv_f32", B=8, T=1024, C=4096, seed=4,
        description="RWKV-4 WKV, fp32, w=-exp(N), u~N, k~5N with 1% set to +-60, v~N, zero state"),
    "backward_wkv_f32": WKVConfig(
        "backward_wkv_f32", B=8, T=1024, C=4096, seed=4, backward=True,
        description="RWKV-4 WKV backward (dw, du, dk, dv) at the WKV workload's inputs, dy ~ N(0,1) fp32"),
}

# The pages give no sizes for the gated EMA (a BERT-sized toy experiment); this
# workload takes the WKV workload's channel count and a longer sequence, in bf16
# as a layer would feed it, scanned in both directions (a bidirectional encoder).
EMA_CONFIGS = {
    "ema_bf16": EMAConfig(
        "ema_bf16", B=8, T=2048, C=4096, dtype="bf16", seed=6,
        description="gated EMA, bf16 x~N(0,1), f=sigmoid(N(2,1)), zero state, forward and reverse scans"),
    "bidir_ema_bf16": EMAConfig(
        "bidir_ema_bf16", B=8, T=2048, C=4096, dtype="bf16", seed=9, reverse=(False,),
        bidirectional=True,
        description="bidirectional gated EMA (forward + reverse summed), bf16 x~N(0,1), "
                    "f=sigmoid(N(2,1)), zero state"),
}


def to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast to the named storage dtype (round-to-nearest-even for bf16)."""
    if dtype == "f32":
        return x.to(torch.float32).contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(f"unknown dtype {dtype!r}")


def retention_gammas(H: int) -> torch.Tensor:
    """Per-head decay schedule 1 - 2^(-5-h), h = 0..H-1 (fp32)."""
    return torch.tensor([1.0 - 2.0 ** (-5 - h) for h in range(H)], dtype=torch.float32)


def _draw(gen, shape, dist: str, Dk: int, role: str):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if dist == "quarter":
        return x / 4.0
    if dist == "scaled":
        return x * (Dk ** -0.5)
    if dist == "elu1":
        # positive feature map elu(x) + 1 for queries and keys; values stay N(0,1)
        return torch.nn.functional.elu(x) + 1.0 if role in ("q", "k") else x
    raise ValueError(f"unknown dist {dist!r}")


def la_inputs(B, H, T, Dk, Dv, dtype="bf16", mode="none", normalize=False, dist="scaled",
              seed=0, prefix=0, random_state=False, gamma=None, return_prefix=False):
    """Seeded inputs for ``la_forward``.

    Returns a dict of CPU tensors: q, k [B,H,T,Dk] and v [B,H,T,Dv] in ``dtype``;
    ``decay`` (fp32, [H] for mode 'head', [B,H,T] for 'step', [B,H,T,Dk] for
    'elem' (one factor per key channel), else None);
    ``state_in`` [B,H,Dk,Dv] and ``cum_k_in`` [B,H,Dk] (fp32 or None).

    prefix > 0: S0 = sum over a preceding random segment of k v^T and
    cum_k0 = sum of its keys, both accumulated in fp64 from the bf16/fp32-rounded
    prefix and then rounded to fp32 (the same rounded values go to both sides).
    random_state: S0 ~ N(0,1) (and cum_k0 ~ |N(0,1)|*Dk when normalising).
    gamma: optional decay override (fp32 tensor of the mode's shape); by default
    mode 'head' uses 1 - 2^(-5-h); modes 'step' and 'elem' draw sigmoid(N(3,1))
    per factor.
    return_prefix: also return the prefix segment's rounded keys and values
    (``prefix_k``, ``prefix_v``) so a caller can rebuild the concatenation.
    """
    gen = torch.Generator().manual_seed(int(seed))
    q = to_dtype(_draw(gen, (B, H, T, Dk), dist, Dk, "q"), dtype)
    k = to_dtype(_draw(gen, (B, H, T, Dk), dist, Dk, "k"), dtype)
    v = to_dtype(_draw(gen, (B, H, T, Dv), dist, Dk, "v"), dtype)
    decay = None
    if mode == "head":
        decay = retention_gammas(H) if gamma is None else gamma.to(torch.float32)
    elif mode == "step":
        if gamma is None:
            decay = torch.sigmoid(torch.randn(B, H, T, generator=gen) + 3.0).to(torch.float32)
        else:
            decay = gamma.to(torch.float32).contiguous()
    elif mode == "elem":
        if gamma is None:
            decay = torch.sigmoid(torch.randn(B, H, T, Dk, generator=gen) + 3.0).to(torch.float32)
        else:
            decay = gamma.to(torch.float32).contiguous()
    elif mode != "none":
        raise ValueError(mode)
    state_in = cum_k_in = None
    extra = {}
    if prefix:
        kp_r = to_dtype(_draw(gen, (B, H, prefix, Dk), dist, Dk, "k"), dtype)
        vp_r = to_dtype(_draw(gen, (B, H, prefix, Dv), dist, Dk, "v"), dtype)
        kp, vp = kp_r.double(), vp_r.double()
        state_in = torch.matmul(kp.transpose(-1, -2), vp).to(torch.float32).contiguous()
        if normalize:
            cum_k_in = kp.sum(dim=2).to(torch.float32).contiguous()
        if return_prefix:
            extra = dict(prefix_k=kp_r, prefix_v=vp_r)
    elif random_state:
        state_in = torch.randn(B, H, Dk, Dv, generator=gen, dtype=torch.float32)
        if normalize:
            cum_k_in = (torch.randn(B, H, Dk, generator=gen).abs() * Dk).to(torch.float32)
    return dict(q=q, k=k, v=v, decay=decay, state_in=state_in, cum_k_in=cum_k_in, **extra)


def la_config_inputs(cfg: LAConfig, seed=None):
    return la_inputs(cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv, dtype=cfg.dtype, mode=cfg.mode,
                     normalize=cfg.normalize, dist=cfg.dist,
                     seed=cfg.seed if seed is None else seed, prefix=cfg.prefix,
                     random_state=cfg.random_state)


def wkv_inputs(B, T, C, seed=0, outlier_frac=0.01, outlier=60.0, random_state=False,
               k_scale=5.0):
    """Seeded fp32 inputs for ``wkv_forward``.

    Draw order: k ~ N(0,1)*k_scale, v ~ N(0,1), w = -exp(N(0,1)) [C], u ~ N(0,1) [C],
    then an i.i.d. Bernoulli(outlier_frac) mask and a fair sign: masked keys are
    set to +-outlier (after the scaling).  random_state gives a carried state
    (aa ~ N, bb ~ |N|+0.5, pp ~ 3N); otherwise state_in is None (zero sums and
    pp = -1e38).
    """
    gen = torch.Generator().manual_seed(int(seed))
    k = torch.randn(B, T, C, generator=gen) * k_scale
    v = torch.randn(B, T, C, generator=gen)
    w = -torch.exp(torch.randn(C, generator=gen))
    u = torch.randn(C, generator=gen)
    if outlier_frac > 0:
        hit = torch.rand(B, T, C, generator=gen) < outlier_frac
        sign = torch.where(torch.rand(B, T, C, generator=gen) < 0.5, -1.0, 1.0)
        k = torch.where(hit, sign * outlier, k)
    state_in = None
    if random_state:
        aa = torch.randn(B, C, generator=gen)
        bb = torch.randn(B, C, generator=gen).abs() + 0.5
        pp = torch.randn(B, C, generator=gen) * 3.0
        state_in = torch.stack([aa, bb, pp]).to(torch.float32).contiguous()
    f = lambda x: x.to(torch.float32).contiguous()
    return dict(w=f(w), u=f(u), k=f(k), v=f(v), state_in=state_in)


def wkv_config_inputs(cfg: WKVConfig, seed=None):
    return wkv_inputs(cfg.B, cfg.T, cfg.C, seed=cfg.seed if seed is None else seed,
                      outlier_frac=cfg.outlier_frac, outlier=cfg.outlier)


def la_tokens(cfg: LAConfig) -> int:
    return cfg.B * cfg.H * cfg.T


def ema_inputs(B, T, C, dtype="f32", seed=0, random_state=False, f_mean=2.0, f_std=1.0):
    """Seeded inputs for ``ema_forward``.

    Draw order: x ~ N(0,1) [B,T,C], factor logits ~ N(f_mean, f_std) [B,T,C]
    (factors = sigmoid of them, as the layer that feeds the scan produces them),
    then, with random_state, the carried state ~ N(0,1) [B,C] (fp32).  x and f
    are rounded to `dtype` (RNE for bf16); the oracle sees the rounded values.
    """
    gen = torch.Generator().manual_seed(int(seed))
    x = torch.randn(B, T, C, generator=gen)
    f = torch.sigmoid(torch.randn(B, T, C, generator=gen) * f_std + f_mean)
    state_in = torch.randn(B, C, generator=gen).to(torch.float32).contiguous() if random_state else None
    return dict(x=to_dtype(x, dtype), f=to_dtype(f, dtype), state_in=state_in)


def ema_config_inputs(cfg: EMAConfig, seed=None):
    return ema_inputs(cfg.B, cfg.T, cfg.C, dtype=cfg.dtype, seed=cfg.seed if seed is None else seed)


def output_gradients(B, H, T, Dk, Dv, dtype="bf16", seed=0, with_state=False):
    """Seeded gradients for a linear-attention backward: dy ~ N(0,1) [B,H,T,Dv] in
    ``dtype`` and, with_state, dstate_out ~ N(0,1) [B,H,Dk,Dv] fp32 (else None)."""
    gen = torch.Generator().manual_seed(int(seed) + 7919)
    dy = to_dtype(torch.randn(B, H, T, Dv, generator=gen), dtype)
    dsf = torch.randn(B, H, Dk, Dv, generator=gen).to(torch.float32) if with_state else None
    return dy, dsf
