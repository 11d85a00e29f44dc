"""Seeded synthetic decode workloads (inputs only; no quantization arithmetic).

This module is the single source of inputs for both the CPU oracle and the HIP
path.  It draws fp16 keys, values and queries shaped like one attention layer
of a Llama-3-8B / Qwen3-8B style model (head_dim 128, grouped-query heads) and
holds none of the method's arithmetic.

Distribution (stands in for the Qwen3 / LLaMA3 activations the Kitty paper
evaluates on, "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with
Dynamic Channel-wise Precision Boost", Abstract):

* per KV head and channel j, a key scale sigma_k[h, j] drawn log-uniform in
  ``k_sigma``; ``k_outliers`` distinct channels per head are multiplied by
  ``k_outlier_factor`` (the strongly non-uniform channel variance the
  precision boost targets);
* value scales sigma_v[h, j] log-uniform in ``v_sigma``, no outliers;
* K = N(0,1) * sigma_k and V = N(0,1) * sigma_v drawn in float32 and rounded
  to float16 (round-to-nearest-even); queries Q ~ N(0,1) rounded to float16.

Streams: the scales come from ``default_rng([seed, TAG_SCALES])``; sequence b
draws from ``default_rng([seed, TAG_SEQUENCE, b])`` in the order K, V, Q, then
the decode-step tokens (k, v, q per step).  Each sequence has its own stream,
so a smaller batch is a prefix of a larger one.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 32

TAG_SCALES = 7001
TAG_SEQUENCE = 7002


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    ctx: int
    hi_fraction: float = 0.25
    k_sigma: tuple = (0.05, 4.0)
    k_outliers: int = 4
    k_outlier_factor: float = 20.0
    v_sigma: tuple = (0.05, 4.0)
    decode_steps: int = 0
    head_dim: int = HEAD_DIM
    sweep: tuple = field(default=())

    @property
    def n_hi(self) -> int:
        return n_hi_for(self.hi_fraction, self.head_dim)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def n_hi_for(hi_fraction: float, head_dim: int = HEAD_DIM) -> int:
    """Boosted channels per page: hi_fraction * head_dim, rounded half-to-even."""
    return int(np.rint(hi_fraction * head_dim))


# The five workloads: a tiny correctness case, Llama-3-8B and Qwen3-8B decode
# shapes, a batch sweep at a fixed memory shape, and a prefill precision sweep.
TINY = Workload("tiny_b1_h1_ctx256", seed=0, batch=1, n_kv_heads=1, n_q_heads=1, ctx=256)
LLAMA3_8B = Workload("llama3_8b_b16_ctx4096", seed=1, batch=16, n_kv_heads=8, n_q_heads=32, ctx=4096)
QWEN3_8B = Workload("qwen3_8b_b4_ctx32768_append64", seed=2, batch=4, n_kv_heads=8, n_q_heads=32,
                    ctx=32768, decode_steps=64)
BATCH_SWEEP = Workload("batch_sweep_ctx8192", seed=3, batch=8, n_kv_heads=8, n_q_heads=32, ctx=8192,
                       sweep=(8, 16, 32, 64, 128))
PREFILL_SWEEP = Workload("prefill_b8_s16384", seed=4, batch=8, n_kv_heads=8, n_q_heads=32, ctx=16384,
                         k_sigma=(0.01, 8.0), k_outliers=8, k_outlier_factor=30.0,
                         sweep=(0.0, 0.125, 0.25, 0.5))

WORKLOADS = [TINY, LLAMA3_8B, QWEN3_8B, BATCH_SWEEP, PREFILL_SWEEP]


def to_f16(x):
    """float32 -> float16 round-to-nearest-even.  Uses torch's vectorized CPU
    conversion when torch is importable (bit-identical to numpy's, which is
    ~40x slower); numpy otherwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
    except ImportError:  # pragma: no cover
        return x.astype(np.float16)
    return torch.from_numpy(x).to(torch.float16).numpy()


def _log_uniform(rng, lo, hi, shape):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))


def scales(w: Workload):
    """Per-(KV head, channel) standard deviations of K and V, float64."""
    rng = np.random.default_rng([w.seed, TAG_SCALES])
    sk = _log_uniform(rng, *w.k_sigma, (w.n_kv_heads, w.head_dim))
    for h in range(w.n_kv_heads):
        out = rng.choice(w.head_dim, size=w.k_outliers, replace=False)
        sk[h, out] *= w.k_outlier_factor
    sv = _log_uniform(rng, *w.v_sigma, (w.n_kv_heads, w.head_dim))
    return sk, sv


def sequence(w: Workload, b: int, ctx: int | None = None, steps: int | None = None):
    """Inputs of sequence b: fp16 k, v [Hkv, ctx, D], q [Hq, D] and the decode
    tokens k_new, v_new [steps, Hkv, D], q_new [steps, Hq, D]."""
    ctx = w.ctx if ctx is None else ctx
    steps = w.decode_steps if steps is None else steps
    sk, sv = scales(w)
    rng = np.random.default_rng([w.seed, TAG_SEQUENCE, b])
    H, D, Hq = w.n_kv_heads, w.head_dim, w.n_q_heads
    k = to_f16(rng.standard_normal((H, ctx, D), dtype=np.float32) * sk[:, None, :].astype(np.float32))
    v = to_f16(rng.standard_normal((H, ctx, D), dtype=np.float32) * sv[:, None, :].astype(np.float32))
    q = to_f16(rng.standard_normal((Hq, D), dtype=np.float32))
    kn = np.empty((steps, H, D), np.float16)
    vn = np.empty((steps, H, D), np.float16)
    qn = np.empty((steps, Hq, D), np.float16)
    for t in range(steps):
        kn[t] = to_f16(rng.standard_normal((H, D), dtype=np.float32) * sk.astype(np.float32))
        vn[t] = to_f16(rng.standard_normal((H, D), dtype=np.float32) * sv.astype(np.float32))
        qn[t] = to_f16(rng.standard_normal((Hq, D), dtype=np.float32))
    return dict(k=k, v=v, q=q, k_new=kn, v_new=vn, q_new=qn)


def batch(w: Workload, batch: int | None = None, ctx: int | None = None, steps: int | None = None):
    """Stack sequences 0..batch-1: k, v [B, Hkv, ctx, D]; q [B, Hq, D];
    k_new, v_new [steps, B, Hkv, D]; q_new [steps, B, Hq, D]."""
    B = w.batch if batch is None else batch
    workers = max(1, min(16, os.cpu_count() or 1, B))
    with ThreadPoolExecutor(workers) as ex:   # per-sequence streams: order-independent
        seqs = list(ex.map(lambda b: sequence(w, b, ctx, steps), range(B)))
    out = {}
    for key in ("k", "v", "q"):
        out[key] = np.stack([s[key] for s in seqs])
    for key in ("k_new", "v_new", "q_new"):
        out[key] = np.stack([s[key] for s in seqs], axis=1)
    return out


def planted_page(seed: int, n_tokens: int = PAGE_TOKENS, head_dim: int = HEAD_DIM):
    """A [n_tokens, head_dim] fp16 block with a wide spread of channel scales,
    used by small unit cases."""
    rng = np.random.default_rng([seed, 9001])
    sig = _log_uniform(rng, 0.05, 4.0, head_dim)
    return to_f16((rng.standard_normal((n_tokens, head_dim)) * sig).astype(np.float32))
