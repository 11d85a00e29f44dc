"""The shared input generator: shapes, streams and the fp16 conversion."""
import numpy as np

from mixed_precision_bit_kitty_amd import synth


def test_fast_f16_conversion_is_round_to_nearest_even():
    # every finite fp16 value, every midpoint between neighbours and the
    # float32 values just around each midpoint: identical to numpy's RNE cast
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = np.sort(h[np.isfinite(h)].astype(np.float32))
    h = np.unique(h)
    mid = ((h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2).astype(np.float32)
    x = np.concatenate([h, mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf)),
                        np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 1e-5])
    assert np.array_equal(synth.to_f16(x).view(np.uint16), x.astype(np.float16).view(np.uint16))


def test_workload_shapes():
    assert [w.n_hi for w in synth.WORKLOADS] == [32, 32, 32, 32, 32]
    assert synth.PREFILL_SWEEP.sweep == (0.0, 0.125, 0.25, 0.5)
    assert [synth.n_hi_for(f) for f in synth.PREFILL_SWEEP.sweep] == [0, 16, 32, 64]
    s = synth.sequence(synth.TINY, 0)
    assert s["k"].shape == (1, 256, 128) and s["q"].shape == (1, 128)
    s = synth.sequence(synth.QWEN3_8B, 1, ctx=64, steps=3)
    assert s["k_new"].shape == (3, 8, 128) and s["q_new"].shape == (3, 32, 128)
