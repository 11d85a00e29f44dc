"""GPU parity of decode under packed workgroup plans: more (sequence, KV
head, head group) units than CUs, so the split plan picks workgroups of 3, 4
or 12 waves.  Both bit-width pairs and both ranking modes; the fused step and
append + decode attention against each other and against the oracle (records
bit-exact, attention within 2e-3)."""
import numpy as np
import pytest

from mixed_precision_bit_kitty_amd import synth

from _gpu_util import step_twins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_bit_kitty_amd import binding as B
    B.load()


def _plan(batch, hkv, hq, msl, n_hi, lo_bit):
    from mixed_precision_bit_kitty_amd import binding as B
    n_wg, waves, _ = B.kitty_decode_plan(B.config(hkv, n_hi, lo_bit=lo_bit), batch, hq, msl)
    return n_wg, waves


# (batch, KV heads, query heads, longest prompt, n_hi, lo_bit, ranking, waves per workgroup)
CASES = [
    (20, 16, 32, 200, 32, 2, "page", 3),
    (20, 16, 32, 200, 32, 4, "running", 3),
    (33, 8, 32, 3470, 13, 2, "page", 12),
    (24, 16, 64, 660, 100, 4, "page", 4),
    (80, 4, 16, 360, 0, 2, "running", 4),
    (36, 8, 48, 860, 45, 4, "page", 4),
    (300, 1, 4, 460, 32, 2, "page", 4),
]


@pytest.mark.parametrize("batch,hkv,hq,ctx,n_hi,lo_bit,mode,waves", CASES)
def test_packed_plans(batch, hkv, hq, ctx, n_hi, lo_bit, mode, waves):
    steps = 4
    rng = np.random.default_rng([batch, hkv, ctx, 77])
    lens = [int(n) for n in rng.integers(ctx // 2, ctx + 1, batch)]
    lens[0] = ctx
    assert _plan(batch, hkv, hq, ctx + steps, n_hi, lo_bit) == (1, waves)
    w = synth.LLAMA3_8B.with_(n_kv_heads=hkv, n_q_heads=hq)
    worst = step_twins(w, lens, steps, ctx, n_hi=n_hi, check_every=2, lo_bit=lo_bit, rank_mode=mode)
    print(f"packed plan {batch}x{hkv}x{hq} ctx {ctx} n_hi {n_hi} lo_bit {lo_bit} {mode}: "
          f"{waves}-wave workgroups, max abs err {worst:.3g}")
