"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side
tests/bench.

This module holds random draws, scaling and dtype casts only -- none of the
method's arithmetic -- so that the oracle and the HIP path can consume the very
same stored arrays while sharing no code.

Recipe (every workload): ``numpy.random.default_rng(seed)`` (PCG64), draws in
float64 in the order q, k, v, g, then the initial key/value states (when the
workload has them); each draw is then scaled/shifted and cast to its storage
dtype.  bf16 storage rounds float64 -> float32 -> bfloat16, both steps
round-to-nearest-even.  The float64 view the oracle consumes is the exact
upcast of the stored values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Stored", "bf16_bits", "bf16_to_f64", "stored", "gsa_inputs", "gla_inputs",
    "decode_inputs", "varlen_lengths", "varlen_inputs", "WORKLOADS", "to_dev", "to_np",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest-even, via float32) and return the raw uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Stored:
    """A tensor as stored for the device: ``raw`` is float32 or uint16 (bf16 bits);
    ``f64`` is its exact float64 upcast for the oracle."""
    raw: np.ndarray
    dtype: str  # "f32" | "bf16"

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_to_f64(self.raw)
        return self.raw.astype(np.float64)

    @property
    def shape(self):
        return self.raw.shape


def stored(x: np.ndarray, dtype: str) -> Stored:
    if dtype == "bf16":
        return Stored(bf16_bits(x), "bf16")
    if dtype == "f32":
        return Stored(np.ascontiguousarray(x, dtype=np.float32), "f32")
    raise ValueError(dtype)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float64)


def gsa_inputs(B, H, T, dk, dv, m, dtype="bf16", seed=0, qkv_scale=None,
               g_shift=0.0, init_std=None, fast_slots=0, fast_shift=0.0):
    """q,k,v ~ N(0,1)*qkv_scale [B,H,T,d]; g ~ N(0,1)+g_shift [B,H,T,m];
    optional K0 [B,H,m,dk], V0 [B,H,m,dv] ~ N(0, init_std) stored as float32.
    fast_slots > 0: the logits of the first fast_slots slots are shifted by
    fast_shift in addition (a set of fast-forgetting slots)."""
    rng = np.random.default_rng(seed)
    if qkv_scale is None:
        qkv_scale = 1.0 / math.sqrt(dk)
    q = _normal(rng, (B, H, T, dk)) * qkv_scale
    k = _normal(rng, (B, H, T, dk)) * qkv_scale
    v = _normal(rng, (B, H, T, dv)) * qkv_scale
    g = _normal(rng, (B, H, T, m)) + g_shift
    if fast_slots:
        g[..., :fast_slots] += fast_shift
    out = dict(q=stored(q, dtype), k=stored(k, dtype), v=stored(v, dtype),
               g=stored(g, dtype), k0=None, v0=None)
    if init_std is not None:
        out["k0"] = stored(_normal(rng, (B, H, m, dk)) * init_std, "f32")
        out["v0"] = stored(_normal(rng, (B, H, m, dv)) * init_std, "f32")
    return out


def gsa_grad_inputs(B, H, T, dk, dv, m, dtype="bf16", seed=0, final_std=None):
    """Upstream gradients for a GSA backward: dO ~ N(0,1) [B,H,T,dv] in dtype;
    optional final-state gradients dKf [B,H,m,dk], dVf [B,H,m,dv] ~ N(0,
    final_std) stored as float32."""
    rng = np.random.default_rng(seed)
    out = dict(do=stored(_normal(rng, (B, H, T, dv)), dtype), dkf=None, dvf=None)
    if final_std is not None:
        out["dkf"] = stored(_normal(rng, (B, H, m, dk)) * final_std, "f32")
        out["dvf"] = stored(_normal(rng, (B, H, m, dv)) * final_std, "f32")
    return out


def gla_inputs(B, H, T, dk, dv, dtype="bf16", seed=0, qkv_scale=None,
               g_shift=0.0, init_std=None, log_decay_scale=None):
    """q,k ~ N(0,1)*qkv_scale [B,H,T,dk]; v [B,H,T,dv]; g ~ N(0,1)+g_shift
    [B,H,T,dk] (one logit per key dim); optional S0 [B,H,dk,dv] ~ N(0,init_std).
    With log_decay_scale, g is instead -|N(0,1)| * log_decay_scale (gates given
    as log-decays: non-positive, half-normal)."""
    rng = np.random.default_rng(seed)
    if qkv_scale is None:
        qkv_scale = 1.0 / math.sqrt(dk)
    q = _normal(rng, (B, H, T, dk)) * qkv_scale
    k = _normal(rng, (B, H, T, dk)) * qkv_scale
    v = _normal(rng, (B, H, T, dv)) * qkv_scale
    g = _normal(rng, (B, H, T, dk))
    g = -np.abs(g) * log_decay_scale if log_decay_scale is not None else g + g_shift
    out = dict(q=stored(q, dtype), k=stored(k, dtype), v=stored(v, dtype),
               g=stored(g, dtype), s0=None)
    if init_std is not None:
        out["s0"] = stored(_normal(rng, (B, H, dk, dv)) * init_std, "f32")
    return out


def decode_inputs(N, H, dk, dv, m, dtype="bf16", seed=0, qkv_scale=None,
                  state_std=0.1):
    """Key/value slot states [N,H,m,d] ~ N(0,state_std) float32, then one token
    per sequence: q,k,v ~ N(0,1)*qkv_scale [N,H,d], g ~ N(0,1) [N,H,m]."""
    rng = np.random.default_rng(seed)
    if qkv_scale is None:
        qkv_scale = 1.0 / math.sqrt(dk)
    q = _normal(rng, (N, H, dk)) * qkv_scale
    k = _normal(rng, (N, H, dk)) * qkv_scale
    v = _normal(rng, (N, H, dv)) * qkv_scale
    g = _normal(rng, (N, H, m))
    ks = _normal(rng, (N, H, m, dk)) * state_std
    vs = _normal(rng, (N, H, m, dv)) * state_std
    return dict(q=stored(q, dtype), k=stored(k, dtype), v=stored(v, dtype),
                g=stored(g, dtype), kstate=stored(ks, "f32"), vstate=stored(vs, "f32"))


def varlen_lengths(n, lo, hi, seed=0):
    """n sequence lengths, log-uniform in [lo, hi] (a prompt-length mix with
    many short and few long sequences), from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(round(math.exp(t))) for t in x]


def varlen_inputs(lengths, H, dk, dv, m, dtype="bf16", seed=0, qkv_scale=None,
                  g_shift=0.0, init_std=None):
    """A packed batch of len(lengths) sequences, head-major: cu_seqlens [n+1]
    (int32 offsets, cu[0] = 0); q,k ~ N(0,1)*qkv_scale [H,total,dk]; v
    [H,total,dv]; g ~ N(0,1)+g_shift [H,total,m]; optional K0 [n,H,m,dk],
    V0 [n,H,m,dv] ~ N(0, init_std) stored as float32.  Draw order as for
    gsa_inputs."""
    rng = np.random.default_rng(seed)
    if qkv_scale is None:
        qkv_scale = 1.0 / math.sqrt(dk)
    n = len(lengths)
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    total = int(cu[-1])
    q = _normal(rng, (H, total, dk)) * qkv_scale
    k = _normal(rng, (H, total, dk)) * qkv_scale
    v = _normal(rng, (H, total, dv)) * qkv_scale
    g = _normal(rng, (H, total, m)) + g_shift
    out = dict(cu_seqlens=cu, q=stored(q, dtype), k=stored(k, dtype), v=stored(v, dtype),
               g=stored(g, dtype), k0=None, v0=None)
    if init_std is not None:
        out["k0"] = stored(_normal(rng, (n, H, m, dk)) * init_std, "f32")
        out["v0"] = stored(_normal(rng, (n, H, m, dv)) * init_std, "f32")
    return out


def varlen_grad_inputs(lengths, H, dk, dv, m, dtype="bf16", seed=0, final_std=None):
    """Upstream gradients for the backward of a packed batch: dO ~ N(0,1)
    [H,total,dv] in dtype; optional dKf [n,H,m,dk], dVf [n,H,m,dv] ~ N(0,
    final_std) stored as float32."""
    rng = np.random.default_rng(seed)
    n, total = len(lengths), int(np.sum(np.asarray(lengths, dtype=np.int64)))
    out = dict(do=stored(_normal(rng, (H, total, dv)), dtype), dkf=None, dvf=None)
    if final_std is not None:
        out["dkf"] = stored(_normal(rng, (n, H, m, dk)) * final_std, "f32")
        out["dvf"] = stored(_normal(rng, (n, H, m, dv)) * final_std, "f32")
    return out


# The five workloads: sizes, dtypes and value distributions of the method's
# configurations (GSA: tau = 8 per the paper's Sec. 3.3; the standalone GLA
# case uses tau = 16).
WORKLOADS = {
    "gsa_f32_small": dict(op="gsa", B=1, H=2, T=256, dk=64, dv=64, m=32, C=64, tau=8.0,
                          dtype="f32", qkv_scale=1 / 8.0, g_shift=0.0, init_std=None),
    "gsa_bf16_train_T2048": dict(op="gsa", B=8, H=4, T=2048, dk=128, dv=128, m=64, C=64,
                                 tau=8.0, dtype="bf16", qkv_scale=1 / math.sqrt(128),
                                 g_shift=0.0, init_std=None),
    # the training shape with 8 of the 64 slots forgetting fast (logits
    # N(-6, 1): log alpha ~ -0.75 per token, about -48 over a 64-token chunk)
    "gsa_bf16_train_T2048_fast_forget": dict(op="gsa", B=8, H=4, T=2048, dk=128, dv=128, m=64,
                                             C=64, tau=8.0, dtype="bf16",
                                             qkv_scale=1 / math.sqrt(128), g_shift=0.0,
                                             init_std=None, fast_slots=8, fast_shift=-6.0),
    # the same with logits N(-10, 1): log alpha ~ -1.25 per token, about -80
    # over a 64-token chunk
    "gsa_bf16_train_T2048_rapid_forget": dict(op="gsa", B=8, H=4, T=2048, dk=128, dv=128, m=64,
                                              C=64, tau=8.0, dtype="bf16",
                                              qkv_scale=1 / math.sqrt(128), g_shift=0.0,
                                              init_std=None, fast_slots=8, fast_shift=-10.0),
    # the same with logits N(-40, 1): log alpha ~ -5 per token, so that even a
    # 16-token sub-chunk decays below the factorised range (the exact walk)
    "gsa_bf16_train_T2048_extreme_forget": dict(op="gsa", B=8, H=4, T=2048, dk=128, dv=128, m=64,
                                                C=64, tau=8.0, dtype="bf16",
                                                qkv_scale=1 / math.sqrt(128), g_shift=0.0,
                                                init_std=None, fast_slots=8, fast_shift=-40.0),
    # the training shape with 128 slots (the largest slot count the pages
    # measure training throughput at)
    "gsa_bf16_train_T2048_m128": dict(op="gsa", B=8, H=4, T=2048, dk=128, dv=128, m=128, C=64,
                                      tau=8.0, dtype="bf16", qkv_scale=1 / math.sqrt(128),
                                      g_shift=0.0, init_std=None),
    "gla_bf16_T4096": dict(op="gla", B=8, H=16, T=4096, dk=128, dv=128, C=64, tau=16.0,
                           dtype="bf16", qkv_scale=1 / math.sqrt(128), g_shift=0.0,
                           init_std=None),
    # the same GLA with the gate given as per-token log-decays, half-normal with
    # mean -0.048 (the tau = 16 logit gate's mean log-decay is -0.050)
    "gla_bf16_T4096_log_decay": dict(op="gla", B=8, H=16, T=4096, dk=128, dv=128, C=64,
                                     tau=16.0, dtype="bf16", qkv_scale=1 / math.sqrt(128),
                                     g_shift=0.0, init_std=None, log_decay_scale=0.06),
    "gsa_bf16_long_T16384": dict(op="gsa", B=1, H=8, T=16384, dk=128, dv=128, m=64, C=64,
                                 tau=8.0, dtype="bf16", qkv_scale=1 / math.sqrt(128),
                                 g_shift=2.0, init_std=0.1),
    "gsa_decode_N256": dict(op="decode", N=256, H=16, dk=128, dv=128, m=64, tau=8.0,
                            dtype="bf16", qkv_scale=1 / math.sqrt(128), state_std=0.1),
    "gsa_decode_N256_m128": dict(op="decode", N=256, H=16, dk=128, dv=128, m=128, tau=8.0,
                                 dtype="bf16", qkv_scale=1 / math.sqrt(128), state_std=0.1),
    # serving: the prefill of the decode batch's 256 sequences (prompt lengths
    # log-uniform in [16, 1024]) as one packed variable-length call, then decode
    # steps from its final states
    "gsa_bf16_serve_N256": dict(op="serve", N=256, H=16, dk=128, dv=128, m=64, C=64, tau=8.0,
                                dtype="bf16", qkv_scale=1 / math.sqrt(128), g_shift=0.0,
                                len_lo=16, len_hi=1024),
}


def to_dev(st, torch):
    """Stored -> device tensor with identical stored bits (data movement only)."""
    if st is None:
        return None
    if st.dtype == "bf16":
        t = torch.from_numpy(st.raw.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(st.raw, dtype=np.float32))
    return t.to("cuda")


def to_np(t):
    """Device tensor -> float64 numpy array (exact upcast)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)
