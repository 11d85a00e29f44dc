"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare against the CPU oracle on the same seeded inputs."""
import numpy as np

import oracle as O

ATOL = 2e-3  # max abs error of decode attention against the oracle's fp32 attention


def torch_mod():
    import torch
    return torch


def dev(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def new_cache(batch, n_kv_heads, n_hi, max_tokens, **kw):
    from mixed_precision_bit_kitty_amd import binding as B
    return B.KittyCache(batch, n_kv_heads, n_hi, max_tokens, **kw)


def host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _diff_fields(got, want, n_hi, lo_bit):
    gk, gv = O.unpack_record(got, n_hi, lo_bit)
    wk, wv = O.unpack_record(want, n_hi, lo_bit)
    out = []
    for key in gk:
        d = int(np.sum(np.atleast_1d(gk[key]).view(np.uint8) != np.atleast_1d(wk[key]).view(np.uint8)))
        if d:
            out.append(f"{key}:{d}")
    for key in gv:
        d = int(np.sum(np.atleast_1d(gv[key]).view(np.uint8) != np.atleast_1d(wv[key]).view(np.uint8)))
        if d:
            out.append(f"{key}:{d}")
    return out


def compare_records(cache, oc, samples=None, seq_map=None, pool=None):
    """Byte-compare GPU page records with the oracle's packed records.

    samples: (b_oracle, page, head) triples, default all sealed pages.
    seq_map: oracle sequence index -> GPU sequence index (default identity)."""
    pool = host(cache.pool) if pool is None else pool
    bt = host(cache.block_table)
    rb = cache.record_bytes
    if samples is None:
        samples = [(b, j, h) for b in range(oc.batch) for j in range(oc.n_pages(b)) for h in range(oc.n_kv_heads)]
    bad = []
    for (b, j, h) in samples:
        gb = b if seq_map is None else seq_map[b]
        got = pool[bt[gb, j], h * rb:(h + 1) * rb]
        want = O.pack_record(*oc.page_fields(b, h, j))
        if not np.array_equal(got, want):
            bad.append(((b, j, h), _diff_fields(got, want, oc.n_hi, oc.lo_bit)))
    assert not bad, f"{len(bad)} of {len(samples)} records differ, first: {bad[:5]}"
    return len(samples)


def compare_tails(cache, oc, seq_map=None):
    tk, tv, sl = host(cache.tail_k), host(cache.tail_v), host(cache.seq_lens)
    for b in range(oc.batch):
        gb = b if seq_map is None else seq_map[b]
        n = int(oc.seq_len[b])
        assert int(sl[gb]) == n, (b, int(sl[gb]), n)
        nt = n % 32
        assert np.array_equal(tk[gb, :, :nt].view(np.uint16), oc.tail_k[b, :, :nt].view(np.uint16))
        assert np.array_equal(tv[gb, :, :nt].view(np.uint16), oc.tail_v[b, :, :nt].view(np.uint16))


def compare_decode(cache, oc, q, max_seq_len=None, seq_map=None, atol=ATOL):
    """GPU decode attention on all sequences; oracle attention on the oracle's
    sequences (all, or the subset seq_map names).  Returns the max error."""
    out = host(cache.decode_attention(dev(q), max_seq_len=max_seq_len))
    qo = q if seq_map is None else q[[seq_map[b] for b in range(oc.batch)]]
    ref = O.decode_attention(oc, qo)
    got = out if seq_map is None else out[[seq_map[b] for b in range(oc.batch)]]
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= atol, f"max abs error {err} > {atol}"
    return err, out


def oracle_state_bytes(oc, b, h, with_mask=None):
    """One copy of the library's running-mode sums of (sequence b, head h)
    from the oracle's exact sums: int64 s1[128], uint64 low / high halves of
    the 128-bit s2[128] (3072 bytes), and, if given, the uint32 mask[4] of a
    ranking (16 more bytes)."""
    out = np.zeros(3088, np.uint8)
    s1 = np.array([int(x) for x in oc.s1[b, h]], dtype=object)
    s2 = np.array([int(x) for x in oc.s2[b, h]], dtype=object)
    out[0:1024] = np.array([int(x) & (2 ** 64 - 1) for x in s1], dtype=np.uint64).view(np.uint8)
    out[1024:2048] = np.array([int(x) & (2 ** 64 - 1) for x in s2], dtype=np.uint64).view(np.uint8)
    out[2048:3072] = np.array([int(x) >> 64 for x in s2], dtype=np.uint64).view(np.uint8)
    if with_mask is not None:
        words = np.zeros(4, np.uint32)
        for c in np.nonzero(with_mask)[0]:
            words[c >> 5] |= np.uint32(1 << (c & 31))
        out[3072:3088] = words.view(np.uint8)
    return out


def compare_state(cache, oc, seq_map=None, masks=False):
    """Current running sums (copy seq_len & 1) of every (sequence, head)
    byte-equal to the oracle's; with masks=True also the stored prefill
    ranking (byte 6144)."""
    ks = host(cache.key_stats)
    for b in range(oc.batch):
        gb = b if seq_map is None else seq_map[b]
        o = 3072 * (int(oc.seq_len[b]) & 1)
        for h in range(oc.n_kv_heads):
            m = oc.running_mask(b)[h] if masks else None
            want = oracle_state_bytes(oc, b, h, m)
            assert np.array_equal(ks[gb, h, o:o + 3072], want[:3072]), f"sums of sequence {b} head {h} differ"
            if masks:
                assert np.array_equal(ks[gb, h, 6144:6160], want[3072:3088]), f"ranking of sequence {b} head {h}"


def step_twins(w, lens, steps, ctx, n_hi=32, msl=None, check_every=1, lo_bit=2, rank_mode="page"):
    """Twin caches: one through the fused step, one through append +
    decode attention; pools, tails, lengths byte-equal after every step,
    outputs bit-equal on steps without a seal, both within 2e-3 of the
    oracle."""
    import torch
    from mixed_precision_bit_kitty_amd import synth
    batch = len(lens)
    x = synth.batch(w, batch=batch, ctx=ctx, steps=steps)
    cap = max(lens) + steps + 32
    rm = 1 if rank_mode == "running" else 0
    fused, split = [new_cache(batch, w.n_kv_heads, n_hi, cap, lo_bit=lo_bit, rank_mode=rm) for _ in range(2)]
    for c in (fused, split):
        c.quantize_pages(dev(x["k"]), dev(x["v"]), lens=dev(np.array(lens, np.int32)))
    oc = O.quantize_pages(x["k"], x["v"], n_hi, batch_lens=lens, lo_bit=lo_bit, rank_mode=rank_mode)
    msl = max(lens) + steps if msl is None else msl
    outs = [torch.zeros((batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    worst = 0.0
    for t in range(steps):
        k, v, q = dev(x["k_new"][t]), dev(x["v_new"][t]), dev(x["q_new"][t])
        seals = [b for b in range(batch) if int(oc.seq_len[b]) % 32 == 31]
        fused.decode_step(k, v, q, max_seq_len=msl, out=outs[0])
        split.append_token(k, v)
        split.decode_attention(q, max_seq_len=msl, out=outs[1])
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        a, b = host(outs[0]), host(outs[1])
        if not seals:
            assert np.array_equal(a, b), f"step {t}: fused and separate outputs differ without a seal"
        assert np.array_equal(host(fused.seq_lens), host(split.seq_lens)), f"step {t}"
        assert np.array_equal(host(fused.tail_k), host(split.tail_k)), f"step {t}"
        if rm:  # the current copy of the sums (the other copy holds older sums in both)
            ka, kb_ = host(fused.key_stats), host(split.key_stats)
            for bb in range(batch):
                o = 3072 * (int(oc.seq_len[bb]) & 1)
                assert np.array_equal(ka[bb, :, o:o + 3072], kb_[bb, :, o:o + 3072]), f"step {t}: running sums differ"
        if seals or t % check_every == 0 or t == steps - 1:
            assert np.array_equal(host(fused.pool), host(split.pool)), f"step {t}: page pools differ"
            compare_tails(fused, oc)
            if rm:
                compare_state(fused, oc)
            ref = O.decode_attention(oc, x["q_new"][t])
            err = float(np.abs(a - ref).max())
            worst = max(worst, err)
            assert err <= ATOL, f"step {t}: max abs err {err}"
    compare_records(fused, oc)
    return worst
