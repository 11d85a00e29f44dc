"""The fused decode step (append + decode attention in one launch) against
the two separate calls and against the oracle.

Each case runs twin caches from the same prefill: one through
kitty_decode_step, one through kitty_append_token then
kitty_decode_attention.  Page records, tails and lengths must match byte
for byte after every step.  Outputs must match bit for bit on steps where
no sequence seals a page (the same waves compute the same sums), and on
every step they must lie within 2e-3 of the oracle, which appends and
attends on its own."""
import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

from _gpu_util import ATOL, compare_records, compare_tails, dev, host, new_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_bit_kitty_amd import binding as B
    B.load()


def _twins(w, lens, steps, ctx, n_hi=32):
    batch = len(lens)
    x = synth.batch(w, batch=batch, ctx=ctx, steps=steps)
    cap = max(lens) + steps + 32
    caches = [new_cache(batch, w.n_kv_heads, n_hi, cap) for _ in range(2)]
    for c in caches:
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens)
    return x, caches, oc


def _run(w, lens, steps, ctx, msl=None, check_every=1, n_hi=32):
    torch = pytest.importorskip("torch")
    x, (fused, split), oc = _twins(w, lens, steps, ctx, n_hi)
    hq = w.n_q_heads
    msl = max(lens) + steps if msl is None else msl
    outs = [torch.zeros((len(lens), hq, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    worst = 0.0
    for t in range(steps):
        k, v, q = dev(x["k_new"][t]), dev(x["v_new"][t]), dev(x["q_new"][t])
        seals = [b for b in range(len(lens)) if int(oc.seq_len[b]) % 32 == 31]
        fused.decode_step(k, v, q, max_seq_len=msl, out=outs[0])
        split.append_token(k, v)
        split.decode_attention(q, max_seq_len=msl, out=outs[1])
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        a, b = host(outs[0]), host(outs[1])
        assert np.all(np.isfinite(a))
        if not seals:
            assert np.array_equal(a, b), f"step {t}: fused and separate outputs differ without a seal"
        assert np.array_equal(host(fused.seq_lens), host(split.seq_lens)), f"step {t}"
        assert np.array_equal(host(fused.tail_k), host(split.tail_k)), f"step {t}"
        assert np.array_equal(host(fused.tail_v), host(split.tail_v)), f"step {t}"
        if seals or t % check_every == 0 or t == steps - 1:
            assert np.array_equal(host(fused.pool), host(split.pool)), f"step {t}: page pools differ"
            compare_tails(fused, oc)
            ref = O.decode_attention(oc, x["q_new"][t], max_len=msl)
            err = float(np.abs(a - ref).max())
            worst = max(worst, err)
            assert err <= ATOL, f"step {t}: max abs err {err}"
    compare_records(fused, oc)
    return worst


@pytest.mark.parametrize("hkv,hq", [(2, 8), (2, 12), (1, 2)])
def test_step_ragged_batch_across_seals(hkv, hq):
    # lengths 0 (first token into an empty cache), 31 (the first step seals
    # page 0), 45, 63; G = 4, 6 (two head groups: one seals into the pool,
    # one into the workspace) and 2
    w = synth.LLAMA3_8B.with_(n_kv_heads=hkv, n_q_heads=hq)
    worst = _run(w, [0, 31, 45, 63], 40, 64)
    print(f"fused step Hkv {hkv} Hq {hq}: max abs err {worst:.3g}")


def test_step_several_workgroups():
    # long sequences: every unit is split over several workgroups
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    worst = _run(w, [2015, 1500, 7], 36, 2015, check_every=5)
    print(f"fused step, several workgroups: max abs err {worst:.3g}")


def test_step_packed_workgroups():
    # 40 sequences x 8 KV heads = 320 units, more than the 256 CUs hold at
    # one workgroup each: the plan packs 4-wave workgroups, three per CU
    from mixed_precision_bit_kitty_amd import binding as B
    rng = np.random.default_rng(41)
    lens = [int(n) for n in rng.integers(250, 300, 40)]
    steps = 34
    assert B.kitty_decode_plan(B.config(8, 32), 40, 32, max(lens) + steps)[:2] == (1, 4)
    worst = _run(synth.LLAMA3_8B, lens, steps, 300, check_every=8)
    print(f"fused step, packed 4-wave workgroups: max abs err {worst:.3g}")


def test_step_capacity_bound():
    # the default bound (cache capacity) plans another split than the tight one
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x, (fused, split), oc = _twins(w, [95, 300], 3, 300)
    for t in range(3):
        k, v, q = dev(x["k_new"][t]), dev(x["v_new"][t]), dev(x["q_new"][t])
        a = host(fused.decode_step(k, v, q))
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        ref = O.decode_attention(oc, x["q_new"][t])
        assert float(np.abs(a - ref).max()) <= ATOL
    compare_records(fused, oc)
    compare_tails(fused, oc)


def test_step_bound_below_length():
    # a bound below the new length: the first 40 tokens are attended, in both
    # paths alike and as the oracle truncated at the bound, also on the step
    # that seals page 1 (63 -> 64) and once page 1 is sealed (the bound then
    # cuts a sealed page, not the tail)
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    _run(w, [60, 20], 6, 64, msl=40)


@pytest.mark.parametrize("msl", [31, 32, 64, 75, 100])
def test_step_bound_inside_sealed_pages(msl):
    # sequences of 130-200 tokens (four to six sealed pages) under a bound
    # that falls inside an older sealed page, on a page boundary or inside
    # the tail: exactly the first min(length, bound) tokens are attended
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    _run(w, [130, 200, 95, 20], 5, 200, msl=msl)


@pytest.mark.parametrize("n_hi", [0, 16, 128])
def test_step_boost_widths(n_hi):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    _run(w, [30, 62], 4, 64, n_hi=n_hi)


@pytest.mark.parametrize("rank_mode", [0, 1])
def test_step_graph_replays_match_eager(rank_mode):
    """The fused step captured in a HIP graph replays like eager launches
    (bitwise), with eager work and synchronizations between replays; in
    both ranking modes (the running mode's sums alternate between two
    copies from step to step)."""
    torch = pytest.importorskip("torch")
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=12)
    steps = 40
    lens = [1000, 700, 31]
    x = synth.batch(w, batch=3, ctx=1000, steps=steps)
    caches = [new_cache(3, 2, 32, 1000 + steps + 32, rank_mode=rank_mode) for _ in range(2)]
    msl = 1000 + steps
    k_buf, v_buf, q_buf = dev(x["k_new"][0]), dev(x["v_new"][0]), dev(x["q_new"][0])
    outs = [torch.zeros((3, 12, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    wss = [c.workspace(12, msl) for c in caches]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        caches[0].decode_step(k_buf, v_buf, q_buf, max_seq_len=msl, out=outs[0], workspace=wss[0])
    torch.cuda.synchronize()
    for c in caches:  # capture does not run the step; prefill after it
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    torch.cuda.synchronize()
    for t in range(steps):
        k_buf.copy_(dev(x["k_new"][t]))
        v_buf.copy_(dev(x["v_new"][t]))
        q_buf.copy_(dev(x["q_new"][t]))
        g.replay()
        torch.cuda.synchronize()
        caches[1].decode_step(k_buf, v_buf, q_buf, max_seq_len=msl, out=outs[1], workspace=wss[1])
        torch.cuda.synchronize()
        assert np.array_equal(host(outs[0]), host(outs[1])), f"step {t}: outputs differ"
        assert np.array_equal(host(caches[0].seq_lens), host(caches[1].seq_lens))
    assert np.array_equal(host(caches[0].pool), host(caches[1].pool))
    assert np.array_equal(host(caches[0].tail_k), host(caches[1].tail_k))
    assert np.array_equal(host(caches[0].tail_v), host(caches[1].tail_v))
    if rank_mode:
        assert np.array_equal(host(caches[0].key_stats), host(caches[1].key_stats))
