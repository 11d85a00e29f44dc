"""GPU parity at boosted-channel counts that are not a multiple of 16
(hi_fraction x 128 rounded half to even, e.g. hi_fraction 0.1 -> 13), for
both bit-width pairs: prefill and append records (padded to the next
multiple of 16 boost slots) and tails bit-exact against the oracle, decode
attention and the fused step within 2e-3."""
import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

from _gpu_util import compare_decode, compare_records, compare_tails, dev, new_cache, step_twins

pytestmark = pytest.mark.gpu

WIDTHS = [1, 8, 13, 17, 38, 45, 100, 127]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_bit_kitty_amd import binding as B
    B.load()


@pytest.mark.parametrize("lo_bit", [2, 4])
@pytest.mark.parametrize("n_hi", WIDTHS)
def test_prefill_and_decode(n_hi, lo_bit):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x = synth.batch(w, batch=2, ctx=100, steps=0)
    lens = [100, 45]
    cache = new_cache(2, 2, n_hi, 100, lo_bit=lo_bit)
    assert cache.record_bytes == O.record_bytes(n_hi, lo_bit=lo_bit)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit)
    compare_records(cache, oc)
    compare_tails(cache, oc)
    err, _ = compare_decode(cache, oc, x["q"])
    print(f"n_hi {n_hi}, lo_bit {lo_bit}: max abs err {err:.3g}")


@pytest.mark.parametrize("lo_bit", [2, 4])
@pytest.mark.parametrize("n_hi", [13, 127])
def test_append_stream(n_hi, lo_bit):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    steps = 40
    x = synth.batch(w, batch=3, ctx=40, steps=steps)
    lens = [0, 20, 40]
    cache = new_cache(3, 2, n_hi, 40 + steps + 32, lo_bit=lo_bit)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit)
    for t in range(steps):
        cache.append_token(dev(x["k_new"][t]), dev(x["v_new"][t]))
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        if any(int(oc.seq_len[b]) % 32 == 0 for b in range(3)) or t == steps - 1:
            compare_records(cache, oc)
            compare_tails(cache, oc)
    compare_decode(cache, oc, x["q_new"][steps - 1])


@pytest.mark.parametrize("lo_bit", [2, 4])
def test_fused_step_across_seals(lo_bit):
    # hi_fraction 0.1: 13 boosted channels; two head groups (G = 6)
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=12, hi_fraction=0.1)
    assert w.n_hi == 13
    worst = step_twins(w, [0, 31, 45, 63], 36, 64, n_hi=w.n_hi, lo_bit=lo_bit)
    print(f"fused step, n_hi 13, lo_bit {lo_bit}: max abs err {worst:.3g}")


def test_several_workgroups():
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x = synth.batch(w, batch=2, ctx=2000, steps=0)
    for n_hi, lo_bit in ((45, 2), (100, 4)):
        cache = new_cache(2, 2, n_hi, 2000, lo_bit=lo_bit)
        cache.quantize_pages(dev(x["k"]), dev(x["v"]))
        oc = O.quantize_pages(x["k"], x["v"], n_hi, lo_bit=lo_bit)
        err, _ = compare_decode(cache, oc, x["q"], max_seq_len=2000)
        print(f"n_hi {n_hi}, lo_bit {lo_bit}, 2000 tokens: max abs err {err:.3g}")
