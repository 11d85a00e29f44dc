"""A decode step captured in a HIP graph (append + decode attention through
the C ABI on torch's capture stream) replays exactly like eager launches:
every replay is checked bitwise against an eager twin cache, with eager work
and synchronizations between the replays."""
import numpy as np
import pytest

from mixed_precision_bit_kitty_amd import synth

from _gpu_util import dev, host, new_cache

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch = pytest.importorskip("torch")
    w = synth.LLAMA3_8B.with_(n_kv_heads=2, n_q_heads=8)
    steps = 40  # crosses a seal (ctx 1000 + 24 = 1024)
    x = synth.batch(w, batch=3, ctx=1000, steps=steps)
    caches = [new_cache(3, 2, 32, 1000 + steps + 32) for _ in range(2)]
    for c in caches:
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array([1000, 700, 31], np.int32)))
    msl = 1000 + steps + 1
    k_buf, v_buf = dev(x["k_new"][0]), dev(x["v_new"][0])
    q_buf = dev(x["q_new"][0])
    outs = [torch.zeros((3, 8, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    wss = [c.workspace(8, msl) for c in caches]
    caches[0].decode_attention(q_buf, max_seq_len=msl, out=outs[0], workspace=wss[0])  # warm launch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        caches[0].append_token(k_buf, v_buf)
        caches[0].decode_attention(q_buf, max_seq_len=msl, out=outs[0], workspace=wss[0])
    torch.cuda.synchronize()
    # capture does not run the step: restore the pre-capture state on both caches
    for c in caches:
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array([1000, 700, 31], np.int32)))
    torch.cuda.synchronize()
    for t in range(steps):
        k_buf.copy_(dev(x["k_new"][t]))
        v_buf.copy_(dev(x["v_new"][t]))
        q_buf.copy_(dev(x["q_new"][t]))
        g.replay()
        torch.cuda.synchronize()
        caches[1].append_token(k_buf, v_buf)
        caches[1].decode_attention(q_buf, max_seq_len=msl, out=outs[1], workspace=wss[1])
        torch.cuda.synchronize()
        assert np.array_equal(host(outs[0]), host(outs[1])), f"step {t}: outputs differ"
        assert np.array_equal(host(caches[0].seq_lens), host(caches[1].seq_lens))
    assert np.array_equal(host(caches[0].pool), host(caches[1].pool))
    assert np.array_equal(host(caches[0].tail_k), host(caches[1].tail_k))
    assert np.array_equal(host(caches[0].tail_v), host(caches[1].tail_v))
