"""Key reconstruction error of the two ranking modes on the five synthetic
workloads; writes ranking_mse.txt beside this file.

Calls only the oracle and the input generator.  For each workload it
quantizes a seeded sample of sequences twice, once with each ranking mode
("page": each page ranked by its own variance; "running": [Velox] "How it
works" Prefill step 1 and Decode phase steps 1-2, a page ranked by the
variance of its head over all tokens stored when it is sealed), appends the
workload's decode tokens, and measures over every sealed page the Key
reconstruction error sum (k^ - k)^2 / sum k^2 and the share of channel
slots on which the two modes boost the same channel.

The synthetic workloads draw every token of a head from the same channel
scales.  One more case, "drift", redraws the scales every 1024 tokens (the
llama3_8b shape, one sequence of 4096 tokens plus 64 appends; scales
log-uniform over [0.05, 4] with 4 channels x20, seeded), where a ranking
over the whole history lags behind the current page.

Run from the repository root:  python tests/golden/ranking_mse.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from mixed_precision_bit_kitty_amd import synth  # noqa: E402

# (workload, hi_fraction override, sequences sampled, decode steps)
CASES = [
    (synth.TINY, None, 1, 64),
    (synth.LLAMA3_8B, None, 2, 40),
    (synth.QWEN3_8B, None, 1, 64),
    (synth.BATCH_SWEEP, None, 2, 0),
    (synth.PREFILL_SWEEP, 0.125, 1, 0),
    (synth.PREFILL_SWEEP, 0.25, 1, 0),
    (synth.PREFILL_SWEEP, 0.5, 1, 0),
]


def drift_inputs(ctx=4096, steps=64, period=1024, seed=11):
    """One sequence (batch 1), 8 KV heads, whose channel scales change every
    `period` tokens."""
    rng = np.random.default_rng([seed, 9100])
    H, D = 8, 128
    total = ctx + steps
    k = np.empty((H, total, D), np.float32)
    for s0 in range(0, total, period):
        sig = np.exp(rng.uniform(np.log(0.05), np.log(4.0), (H, D)))
        for h in range(H):
            sig[h, rng.choice(D, 4, replace=False)] *= 20.0
        n = min(period, total - s0)
        k[:, s0:s0 + n] = rng.standard_normal((H, n, D)).astype(np.float32) * sig[:, None, :].astype(np.float32)
    k = synth.to_f16(k)
    v = synth.to_f16(rng.standard_normal((H, total, D)).astype(np.float32))
    x = dict(k=k[None, :, :ctx], v=v[None, :, :ctx],
             k_new=np.ascontiguousarray(np.transpose(k[:, ctx:], (1, 0, 2))[:, None]),
             v_new=np.ascontiguousarray(np.transpose(v[:, ctx:], (1, 0, 2))[:, None]))
    return x


def sealed_keys(x, b, steps):
    """Keys of sequence b in storage order: the prefill, then the appended tokens."""
    ks = [x["k"][b]]
    if steps:
        ks.append(np.transpose(x["k_new"][:steps, b], (1, 0, 2)))
    return np.concatenate(ks, axis=1)          # [Hkv, T, D]


def measure(w, hf, n_seq, steps, lo_bit=2, x=None):
    if hf is not None:
        w = w.with_(hi_fraction=hf)
    n_hi = w.n_hi
    x = synth.batch(w, batch=n_seq, steps=steps) if x is None else x
    err = {}
    idx = {}
    for mode in O.RANK_MODES:
        c = O.quantize_pages(x["k"], x["v"], n_hi, lo_bit=lo_bit, rank_mode=mode)
        for t in range(steps):
            O.append_token(c, x["k_new"][t], x["v_new"][t])
        num = den = 0.0
        idx[mode] = []
        for b in range(n_seq):
            P = c.n_pages(b)
            kh, _ = c.dequant_sequence(b)
            k = sealed_keys(x, b, steps)[:, :P * 32].astype(np.float64)
            d = kh[:, :P * 32].astype(np.float64) - k
            num += float((d * d).sum())
            den += float((k * k).sum())
            idx[mode].append(c.k[b]["mask"])
        err[mode] = num / den
    same = np.mean([(a & b_).sum() / max(1, a.sum()) for a, b_ in zip(idx["page"], idx["running"])]) if n_hi else 1.0
    return w, n_hi, err, same


def main():
    lines = ["# Key reconstruction error by ranking mode (hi_bit 4 / lo_bit 2), oracle, synthetic inputs",
             "# written by tests/golden/ranking_mse.py",
             "# workload | n_hi | sequences | decode steps | rel. error page | rel. error running | running / page"
             " | boosted channels shared"]
    for w, hf, n_seq, steps in CASES:
        w2, n_hi, err, same = measure(w, hf, n_seq, steps)
        ratio = err["running"] / err["page"]
        lines.append(f"{w2.name} | {n_hi} | {n_seq} | {steps} | {err['page']:.5e} | {err['running']:.5e} | "
                     f"{ratio:.4f} | {same:.3f}")
        print(lines[-1], flush=True)
    w2, n_hi, err, same = measure(synth.LLAMA3_8B.with_(name="drift_h8_ctx4096_append64"), None, 1, 64,
                                  x=drift_inputs())
    lines.append(f"{w2.name} | {n_hi} | 1 | 64 | {err['page']:.5e} | {err['running']:.5e} | "
                 f"{err['running'] / err['page']:.4f} | {same:.3f}")
    print(lines[-1], flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "ranking_mse.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
