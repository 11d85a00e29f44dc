"""The allocation-free fused decode step (kitty_decode_step_noalloc, for
callers that cannot allocate) against the fused step with a caller
workspace (kitty_decode_step): twin caches, calls in a row through the C
ABI, the later ones on smaller shapes, so the scratch layout moves between
calls.  Outputs, records, tails and lengths bit-equal to the workspace
version's; outputs within 2e-3 of the oracle."""
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


def _twin_steps(hkv, hq, lens, steps, n_hi=32, lo_bit=2):
    """`steps` fused steps on twin caches: one through the allocation-free
    entry point, one through kitty_decode_step with its own workspace."""
    import torch
    from mixed_precision_bit_kitty_amd import binding as B
    w = synth.LLAMA3_8B.with_(n_kv_heads=hkv, n_q_heads=hq)
    batch = len(lens)
    x = synth.batch(w, batch=batch, ctx=max(lens), steps=steps)
    cap = max(lens) + steps + 32
    a, b = [new_cache(batch, hkv, n_hi, cap, lo_bit=lo_bit) for _ in range(2)]
    for c in (a, b):
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit)
    msl = max(lens) + steps
    out_a = torch.full((batch, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    out_b = torch.zeros((batch, hq, 128), dtype=torch.float32, device="cuda")
    ws = b.workspace(hq, msl)
    worst = 0.0
    for t in range(steps):
        k, v, q = dev(x["k_new"][t]), dev(x["v_new"][t]), dev(x["q_new"][t])
        B.kitty_decode_step_noalloc(a.cfg, a.view, k, v, q, hq, msl, out_a)
        B.kitty_decode_step(b.cfg, b.view, k, v, q, hq, msl, out_b, ws)
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        ga, gb = host(out_a), host(out_b)
        assert np.array_equal(ga, gb), f"step {t}: outputs differ from the workspace version"
        assert np.array_equal(host(a.seq_lens), host(b.seq_lens)), f"step {t}"
        assert np.array_equal(host(a.tail_k), host(b.tail_k)) and np.array_equal(host(a.tail_v), host(b.tail_v))
        ref = O.decode_attention(oc, x["q_new"][t])
        err = float(np.abs(ga - ref).max())
        assert err <= ATOL, f"step {t}: max abs err {err}"
        worst = max(worst, err)
    assert np.array_equal(host(a.pool), host(b.pool)), "page pools differ"
    compare_records(a, oc)
    compare_tails(a, oc)
    return worst


def test_noalloc_step_matches_workspace_step_then_a_smaller_shape():
    # first: 3 sequences up to 2015 tokens (several workgroups per unit: the
    # split partials and arrival counters are used), G = 6 (two head groups:
    # the second seals into the scratch's record area), seals at 31 -> 32;
    # then a smaller shape (fewer sequences, heads and tokens): the scratch
    # layout shrinks, and the counters it reuses start from zero again
    w1 = _twin_steps(4, 24, [2015, 1500, 31], 34)
    w2 = _twin_steps(2, 8, [95, 40], 3)
    print(f"noalloc step: max abs err {w1:.3g} (large shape), {w2:.3g} (smaller shape)", flush=True)
