"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
small and edge-case inputs: page record bytes, fp16 tails and sequence
lengths bit-exact; decode attention within 2e-3 max abs error."""
import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

from _gpu_util import ATOL, compare_decode, compare_records, compare_tails, dev, host, new_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_bit_kitty_amd import binding as B
    B.load()


def _prefill(w, batch, ctx, n_hi, lens=None, max_tokens=None):
    x = synth.batch(w, batch=batch, ctx=ctx, steps=0)
    cache = new_cache(batch, w.n_kv_heads, n_hi, max_tokens or max(ctx, 32))
    lt = None if lens is None else dev(np.array(lens, np.int32))
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=lt)
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens)
    return x, cache, oc


def test_tiny_workload():
    w = synth.TINY
    x, cache, oc = _prefill(w, 1, w.ctx, w.n_hi)
    assert compare_records(cache, oc) == 8
    compare_tails(cache, oc)
    err, _ = compare_decode(cache, oc, x["q"])
    print(f"tiny: max abs err {err:.3g}")


@pytest.mark.parametrize("n_hi", [0, 16, 32, 48, 64, 96, 128])
def test_boost_widths(n_hi):
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x, cache, oc = _prefill(w, 2, 100, n_hi, lens=[100, 45])
    compare_records(cache, oc)
    compare_tails(cache, oc)
    compare_decode(cache, oc, x["q"])


@pytest.mark.parametrize("hq", [2, 6, 8, 12, 16])
def test_query_group_sizes(hq):
    # G = 1, 3, 4, 6, 8: one or two head groups of up to 4 queries per KV head
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=hq)
    x, cache, oc = _prefill(w, 2, 200, 32)
    compare_decode(cache, oc, x["q"])


def test_edge_lengths():
    lens = [0, 1, 31, 32, 33, 64]
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=4)
    x, cache, oc = _prefill(w, len(lens), 64, 32, lens=lens)
    compare_records(cache, oc)
    compare_tails(cache, oc)
    err, out = compare_decode(cache, oc, x["q"])
    assert np.all(out[0] == 0)


def test_edge_values():
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((1, 2, 96, 128)) * 2).astype(np.float16)
    v = (rng.standard_normal((1, 2, 96, 128)) * 2).astype(np.float16)
    k[0, 0, :32, 3] = np.float16(-2.5)                       # constant channel
    k[0, 0, :32, 4] = np.float16(0.0)                        # all zero
    k[0, 0, :32, 5] = np.float16(-0.0)                       # signed zeros
    k[0, 0, 7, 5] = np.float16(1.0)
    k[0, 0, :32, 6] = np.float16(1.0)                        # tiny range -> subnormal step
    k[0, 0, 9, 6] = np.nextafter(np.float16(1.0), np.float16(2.0))
    k[0, 0, :32, 7] = np.float16(0.0)
    k[0, 0, 3, 7] = np.float16(21 * 2.0 ** -24)              # step rounds down -> clamp
    k[0, 1, 32:64, :] = (rng.standard_normal((32, 128)) * 60000 / 4).clip(-60000, 60000).astype(np.float16)
    v[0, 1, 32:64, :] = (rng.standard_normal((32, 128)) * 60000 / 4).clip(-60000, 60000).astype(np.float16)
    v[0, 0, 40, :] = np.float16(3.0)                         # constant value group row
    v[0, 0, 41, :32] = np.float16(-0.0)
    v[0, 0, 42, :32] = np.float16(0.0)
    v[0, 0, 42, 5] = np.float16(7 * 2.0 ** -24)              # value step rounds down -> clamp
    k[0, 0, 64:96, :] = k[0, 0, 64:65, :]                     # identical tokens in a page
    q = (rng.standard_normal((1, 8, 128))).astype(np.float16)
    for n_hi in (0, 32, 128):
        cache = new_cache(1, 2, n_hi, 96)
        cache.quantize_pages(dev(k), dev(v))
        oc = O.quantize_pages(k, v, n_hi)
        compare_records(cache, oc)
    # attention on the moderate-range head only (the +-60000 head overflows
    # any fp32 softmax test tolerance by construction)
    k2, v2 = k.copy(), v.copy()
    k2[0, 1], v2[0, 1] = k2[0, 0], v2[0, 0]
    cache = new_cache(1, 2, 32, 96)
    cache.quantize_pages(dev(k2), dev(v2))
    oc = O.quantize_pages(k2, v2, 32)
    compare_decode(cache, oc, q)


def test_append_stream_matches_oracle():
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    steps = 70
    x = synth.batch(w, batch=3, ctx=40, steps=steps)
    lens = [0, 20, 40]
    cache = new_cache(3, 2, 32, 40 + steps + 32)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], 32, batch_lens=lens)
    for t in range(steps):
        cache.append_token(dev(x["k_new"][t]), dev(x["v_new"][t]))
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        compare_tails(cache, oc)
        sealed = any(int(oc.seq_len[b]) % 32 == 0 for b in range(3))
        if sealed or t % 9 == 0 or t == steps - 1:
            compare_records(cache, oc)
            compare_decode(cache, oc, x["q_new"][t])


def test_permuted_block_table():
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x = synth.batch(w, batch=3, ctx=160, steps=0)
    rng = np.random.default_rng(3)
    n_pages = 40
    perm = rng.permutation(n_pages)[:15].reshape(3, 5).astype(np.int32)
    cache = new_cache(3, 2, 32, 160, block_table=perm, n_pages=n_pages)
    cache.quantize_pages(dev(x["k"]), dev(x["v"]))
    oc = O.quantize_pages(x["k"], x["v"], 32)
    compare_records(cache, oc)
    compare_decode(cache, oc, x["q"])


def test_determinism():
    w = synth.LLAMA3_8B.with_(n_kv_heads=4, n_q_heads=16)
    x = synth.batch(w, batch=2, ctx=300, steps=0)
    outs, pools = [], []
    for _ in range(2):
        cache = new_cache(2, 4, 32, 300)
        cache.quantize_pages(dev(x["k"]), dev(x["v"]))
        pools.append(host(cache.pool))
        outs.append(host(cache.decode_attention(dev(x["q"]))))
    assert np.array_equal(pools[0], pools[1])
    assert np.array_equal(outs[0], outs[1])


def test_max_seq_len_bounds_grid():
    # a grid sized for the exact longest sequence gives the same output as
    # the default (capacity-sized) one
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    x, cache, oc = _prefill(w, 2, 257, 32, lens=[257, 100], max_tokens=1024)
    a = host(cache.decode_attention(dev(x["q"]), max_seq_len=257))
    b = host(cache.decode_attention(dev(x["q"])))
    ref = O.decode_attention(oc, x["q"])
    assert np.abs(a - ref).max() <= ATOL and np.abs(b - ref).max() <= ATOL


@pytest.mark.parametrize("batch,hkv,hq,ctx,lens", [
    (2, 2, 8, 2000, [2000, 700]),      # several workgroups per (sequence, KV head), ragged lengths
    (1, 1, 4, 4113, None),              # one long sequence: 129 pages and a tail over 11 workgroups
    (3, 1, 6, 900, [900, 17, 416]),     # two head groups (G = 6); a sequence of only a tail
])
def test_multi_workgroup_merge(batch, hkv, hq, ctx, lens):
    w = synth.LLAMA3_8B.with_(n_kv_heads=hkv, n_q_heads=hq)
    x, cache, oc = _prefill(w, batch, ctx, 32, lens=lens)
    err, _ = compare_decode(cache, oc, x["q"])
    # the same cache under a loose bound (another workgroup plan) agrees too
    err2, _ = compare_decode(cache, oc, x["q"], max_seq_len=4 * ctx)
    print(f"multi-workgroup {batch}x{hkv}x{hq} ctx {ctx}: max abs err {err:.3g} / {err2:.3g}")


def test_maximum_length():
    # the longest supported sequence: 4096 sealed pages and a 31-token tail
    # (131,103 tokens), prefilled one token short and completed by a fused
    # step; records bit-exact, attention under the tight and the capacity
    # bound within 2e-3
    n = 4096 * 32 + 31
    w = synth.LLAMA3_8B.with_(n_kv_heads=1, n_q_heads=4)
    x = synth.batch(w, batch=1, ctx=n, steps=0)
    cache = new_cache(1, 1, 32, 4096 * 32)
    assert cache.max_pages == 4096 and cache.default_max_seq_len() == n
    cache.quantize_pages(dev(x["k"][:, :, :n - 1]), dev(x["v"][:, :, :n - 1]))
    out = host(cache.decode_step(dev(np.ascontiguousarray(x["k"][:, :, n - 1])),
                                 dev(np.ascontiguousarray(x["v"][:, :, n - 1])), dev(x["q"]), max_seq_len=n))
    oc = O.quantize_pages(x["k"], x["v"], 32)
    assert int(host(cache.seq_lens)[0]) == n
    compare_records(cache, oc)
    compare_tails(cache, oc)
    ref = O.decode_attention(oc, x["q"])
    err = float(np.abs(out - ref).max())
    assert err <= ATOL, err
    err2, _ = compare_decode(cache, oc, x["q"], max_seq_len=n)
    err3, _ = compare_decode(cache, oc, x["q"])
    print(f"maximum length {n}: fused step {err:.3g}, decode {err2:.3g} / {err3:.3g}")
