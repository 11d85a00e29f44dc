"""GPU parity of the running ranking mode (KITTY_RANK_RUNNING; "Kitty --
Dynamic Channel-wise Mixed-Precision Keys", How it works: Prefill steps 1
and 5, Decode phase steps 1-2) against the CPU oracle: the exact running
sums (state bytes) and the prefill ranking equal to the oracle's, page
records and tails bit-exact after prefill, appends and fused steps,
attention within 2e-3, for both bit-width pairs and several boost widths."""
import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

from _gpu_util import compare_decode, compare_records, compare_state, compare_tails, dev, host, new_cache, step_twins

pytestmark = pytest.mark.gpu
RUN = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_bit_kitty_amd import binding as B
    B.load()


@pytest.mark.parametrize("n_hi,lo_bit", [(32, 2), (0, 2), (13, 2), (128, 2), (32, 4), (100, 4)])
def test_prefill(n_hi, lo_bit):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    lens = [200, 45, 0, 33]
    x = synth.batch(w, batch=4, ctx=200, steps=0)
    cache = new_cache(4, 2, n_hi, 200, lo_bit=lo_bit, rank_mode=RUN)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit, rank_mode="running")
    compare_state(cache, oc, masks=True)
    compare_records(cache, oc)
    compare_tails(cache, oc)
    err, _ = compare_decode(cache, oc, x["q"])
    print(f"running prefill n_hi {n_hi} lo_bit {lo_bit}: max abs err {err:.3g}")


def test_prefill_leaves_negative_slots_alone():
    import torch
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x = synth.batch(w, batch=2, ctx=64, steps=0)
    cache = new_cache(2, 2, 32, 64, rank_mode=RUN)
    cache.key_stats.copy_(torch.arange(2 * 2 * 8192, device="cuda").reshape(2, 2, 8192).to(torch.uint8))
    before = host(cache.key_stats)[1].copy()
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array([64, -1], np.int32)))
    assert np.array_equal(host(cache.key_stats)[1], before)
    oc = O.quantize_pages(x["k"][:1], x["v"][:1], 32, rank_mode="running")
    compare_state(cache, oc, masks=True)


@pytest.mark.parametrize("n_hi,lo_bit", [(32, 2), (45, 4)])
def test_append_stream(n_hi, lo_bit):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    steps = 70
    x = synth.batch(w, batch=3, ctx=40, steps=steps)
    lens = [0, 20, 40]
    cache = new_cache(3, 2, n_hi, 40 + steps + 32, lo_bit=lo_bit, rank_mode=RUN)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit, rank_mode="running")
    for t in range(steps):
        cache.append_token(dev(x["k_new"][t]), dev(x["v_new"][t]))
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        compare_state(cache, oc)
        if any(int(oc.seq_len[b]) % 32 == 0 for b in range(3)) or t == steps - 1:
            compare_records(cache, oc)
            compare_tails(cache, oc)
    compare_decode(cache, oc, x["q_new"][steps - 1])


@pytest.mark.parametrize("hkv,hq", [(2, 8), (2, 12), (1, 2)])
def test_fused_step_across_seals(hkv, hq):
    # G = 6: the second head group ranks its seal copy from the same sums
    w = synth.LLAMA3_8B.with_(n_kv_heads=hkv, n_q_heads=hq)
    worst = step_twins(w, [0, 31, 45, 63], 40, 64, rank_mode="running")
    print(f"running fused step Hkv {hkv} Hq {hq}: max abs err {worst:.3g}")


@pytest.mark.parametrize("n_hi,lo_bit", [(13, 2), (32, 4)])
def test_fused_step_widths(n_hi, lo_bit):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    step_twins(w, [30, 62], 4, 64, n_hi=n_hi, lo_bit=lo_bit, rank_mode="running")


def test_fused_step_several_workgroups():
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    worst = step_twins(w, [2015, 1500, 7], 36, 2015, check_every=5, rank_mode="running")
    print(f"running fused step, several workgroups: max abs err {worst:.3g}")


def test_fused_step_idle_slot():
    # an idle slot (seq_lens -1) appends nothing and its sums stay as they are
    import torch
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x = synth.batch(w, batch=2, ctx=63, steps=2)
    cache = new_cache(2, 2, 32, 128, rank_mode=RUN)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]))
    oc = O.quantize_pages(x["k"][:1], x["v"][:1], 32, rank_mode="running")
    cache.seq_lens[1] = -1
    before = host(cache.key_stats)[1].copy()
    for t in range(2):
        out = host(cache.decode_step(dev(x["k_new"][t]), dev(x["v_new"][t]), dev(x["q_new"][t])))
        O.append_token(oc, x["k_new"][t][:1], x["v_new"][t][:1])
        ref = O.decode_attention(oc, x["q_new"][t][:1])[0]
        assert float(np.abs(out[0] - ref).max()) <= 2e-3
        assert not out[1].any()
    assert np.array_equal(host(cache.key_stats)[1], before)
    compare_state(cache, oc, seq_map={0: 0})
    compare_records(cache, oc, seq_map={0: 0})
