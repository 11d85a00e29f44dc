"""Pins of the oracle at boosted-channel counts that are not a multiple of 16
(hi_fraction x 128 rounded half to even, e.g. hi_fraction 0.1 -> 13).

The record keeps the shape of the next multiple of 16 (the boost slots); the
padding slots carry code 0 and index 0.  Pinned by: byte positions worked
out by hand from the layout rules, ranking against brute force, the padded
record against the record of the same page at that multiple of 16 with the
extra channels' boost codes zeroed, dequantization from the unpacked record
against the definition, and attention against a float64 brute force."""
import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

WIDTHS = [1, 8, 13, 17, 45, 100, 127]


def _page(seed):
    rng = np.random.default_rng([seed, 5151])
    sig = np.exp(rng.uniform(np.log(0.05), np.log(4.0), 128))
    sig[rng.choice(128, 5, replace=False)] *= 20.0
    return (rng.standard_normal((32, 128)) * sig).astype(np.float32).astype(np.float16)


def test_hi_fraction_rounding():
    # hi_fraction 0.1 -> 12.8 -> 13; 0.3 -> 38.4 -> 38; 0.0625 -> 8 exactly
    assert synth.n_hi_for(0.1) == 13
    assert synth.n_hi_for(0.3) == 38
    assert synth.n_hi_for(0.0625) == 8


@pytest.mark.parametrize("k", WIDTHS)
def test_rank_bruteforce(k):
    rng = np.random.default_rng([k, 77])
    for trial in range(3):
        m2 = rng.integers(0, 5 if trial else 1000, 128).astype(np.float32)
        idx, mask = O.rank_channels(m2, k)
        # H = {c : #{c' ranked above c} < k}, ranked above = larger m2 or equal m2 and lower index
        want = [c for c in range(128)
                if sum(1 for c2 in range(128) if m2[c2] > m2[c] or (m2[c2] == m2[c] and c2 < c)) < k]
        assert list(idx) == want and mask.sum() == k


def test_padding_positions_by_hand():
    # n_hi = 13 -> 16 slots, one half block (lanes 0..31), 3072 + 144 bytes.
    # Every boost code of the 13 real slots is 3: in chunk c = 16w + u (w =
    # slot // 8 for slots 0..15) element e of combo A sits at bit
    # 16*(e // 4) + 4*(e % 2) + 2*((e // 2) % 2), of combo B 8 higher.
    # Chunks 16..31 (w = 1) hold slots 8..15: elements 5, 6, 7 (slots 13, 14,
    # 15) are padding, at bits 20, 18, 22 (A) and 28, 26, 30 (B); all other
    # bits of those words are ones.  Chunks 0..15 (slots 0..7) are all ones.
    n = 13
    kf = dict(base=np.zeros((32, 128), np.uint8), boost=np.full((32, n), 3, np.uint8),
              kscale=np.zeros(128, np.float16), kmin=np.zeros(128, np.float16),
              idx=np.arange(100, 100 + n, dtype=np.uint8))
    vf = dict(a=np.zeros((32, 128), np.uint8), vscale=np.zeros((32, 4), np.float16),
              vmin=np.zeros((32, 4), np.float16))
    r = O.pack_record(kf, vf)
    assert r.size == 3072 + 9 * 16
    words = r[1024:1024 + 128].view("<u4")
    pad = 0
    for b in (20, 18, 22, 28, 26, 30):
        pad |= 3 << b
    for c in range(32):
        want = 0xFFFFFFFF if c < 16 else 0xFFFFFFFF & ~pad
        assert words[c] == want, (c, hex(words[c]))
    # the boost plane is 8 * 16 bytes; V codes follow at 1024 + 128
    assert not r[1024 + 128:2048 + 128].any()
    # idx: 13 entries, then 3 zero bytes
    o = 2048 + 128 + 1024
    assert list(r[o:o + 16]) == list(range(100, 113)) + [0, 0, 0]


@pytest.mark.parametrize("lo_bit", [2, 4])
@pytest.mark.parametrize("n", WIDTHS)
def test_padded_record_equals_zeroed_wider_record(n, lo_bit):
    # The record at width n equals the record of the logical fields at the
    # next multiple of 16 whose extra slots have boost code 0 and index 0.
    x, y = _page(n), _page(n + 200)
    kf = O.quant_k_page(x, n, lo_bit)
    vf = O.quant_v_page(y, lo_bit)
    s = O.boost_slots(n)
    wide = dict(kf)
    wide["boost"] = np.concatenate([kf["boost"], np.zeros((32, s - n), np.uint8)], axis=1)
    wide["idx"] = np.concatenate([kf["idx"], np.zeros(s - n, np.uint8)])
    r = O.pack_record(kf, vf)
    assert r.size == O.record_bytes(n, lo_bit=lo_bit) == O.record_bytes(s, lo_bit=lo_bit)
    assert np.array_equal(r, O.pack_record(wide, vf))


@pytest.mark.parametrize("lo_bit", [2, 4])
@pytest.mark.parametrize("n", WIDTHS)
def test_roundtrip_and_dequant(n, lo_bit):
    x, y = _page(3 * n), _page(3 * n + 1)
    kf = O.quant_k_page(x, n, lo_bit)
    vf = O.quant_v_page(y, lo_bit)
    kf2, vf2 = O.unpack_record(O.pack_record(kf, vf), n, lo_bit)
    for key in ("base", "boost", "kscale", "kmin", "idx"):
        assert np.array_equal(kf[key], kf2[key]), key
    for key in vf2:
        assert np.array_equal(vf[key], vf2[key]), key
    # dequantization from the unpacked record: the definition written out,
    # q = 2^lo_bit base + boost at step kscale / 2^lo_bit on the n ranked
    # channels, q = base at step kscale elsewhere; k^ = q * step + kmin
    k_hat = O.dequant_k(kf2["base"], kf2["boost"], kf2["kscale"], kf2["kmin"], kf2["idx"], lo_bit)
    step = kf2["kscale"].astype(np.float64)
    q = kf2["base"].astype(np.float64)
    sc = float(1 << lo_bit)
    for j, c in enumerate(kf2["idx"]):
        q[:, c] = sc * q[:, c] + kf2["boost"][:, j]
        step[c] = step[c] / sc
    want = q * step[None, :] + kf2["kmin"].astype(np.float64)[None, :]
    assert np.allclose(k_hat, want, rtol=2 ** -23, atol=0)
    # and the ranked channels reconstruct better than a uniform lo_bit code would
    lo_l, hi_l = O.levels(lo_bit)
    assert kf["q"][:, kf["idx"]].max() <= hi_l and kf["q"].max() <= hi_l


@pytest.mark.parametrize("n", [13, 45])
def test_attention_fp64_and_append(n):
    w = synth.TINY.with_(n_kv_heads=2, n_q_heads=4)
    x = synth.batch(w, batch=2, ctx=80)
    pre = O.quantize_pages(x["k"], x["v"], n)
    st = O.OracleCache(2, 2, n)
    for t in range(80):
        O.append_token(st, x["k"][:, :, t], x["v"][:, :, t])
    for b in range(2):
        for key in ("base", "boost", "kscale", "kmin", "idx"):
            assert np.array_equal(pre.k[b][key], st.k[b][key])
    out = O.decode_attention(pre, x["q"])
    assert np.array_equal(out, O.decode_attention(st, x["q"]))
    # float64 brute force over the dequantized sequence
    for b in range(2):
        kh, vh = pre.dequant_sequence(b)
        kh, vh = kh.astype(np.float64), vh.astype(np.float64)
        for hq in range(4):
            h = hq // 2
            s = (x["q"][b, hq].astype(np.float64) @ kh[h].T) / np.sqrt(128.0)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ vh[h]
            assert np.abs(out[b, hq] - ref).max() < 2e-5
