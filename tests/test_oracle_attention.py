"""Pins of the attention oracle (no GPU): brute force, a library routine, closed forms."""
import math

import numpy as np
import torch

from oracle import attention, codec
from oracle.cache import OracleCache


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rand_bf16(rng, shape, scale=1.0):
    return _bf16(rng.standard_normal(shape) * scale)


def test_matches_pure_python_brute_force():
    rng = np.random.default_rng(10)
    for trial in range(6):
        hkv, group, t, d = 2, int(rng.integers(1, 5)), int(rng.integers(1, 20)), 8
        q = _rand_bf16(rng, (hkv * group, d))
        k = _rand_bf16(rng, (t, hkv, d))
        v = _rand_bf16(rng, (t, hkv, d))
        scale = 0.3
        got = attention.attention_fp64(q, k, v, scale)
        qf, kf, vf = (codec.bf16_bits_to_f64(a) for a in (q, k, v))
        for h in range(hkv * group):
            g = h // group
            logits = []
            for tt in range(t):
                acc = 0.0
                for dd in range(d):
                    acc += float(qf[h, dd]) * float(kf[tt, g, dd])
                logits.append(scale * acc)
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            den = sum(w)
            for dd in range(d):
                num = sum(w[tt] * float(vf[tt, g, dd]) for tt in range(t))
                assert abs(got[h, dd] - num / den) <= 1e-12 * (1 + abs(num / den))


def test_matches_torch_sdpa_float64():
    """torch.nn.functional.scaled_dot_product_attention (CPU, float64) with the KV head of each
    query group repeated."""
    rng = np.random.default_rng(11)
    hkv, group, t = 2, 4, 300
    q = _rand_bf16(rng, (hkv * group, 128))
    k = _rand_bf16(rng, (t, hkv, 128), 2.0)
    v = _rand_bf16(rng, (t, hkv, 128))
    scale = 1 / math.sqrt(128)
    got = attention.attention_fp64(q, k, v, scale)
    qt = torch.from_numpy(codec.bf16_bits_to_f64(q))[:, None, :]                  # [Hq,1,D]
    kt = torch.from_numpy(codec.bf16_bits_to_f64(k)).permute(1, 0, 2)             # [Hkv,T,D]
    vt = torch.from_numpy(codec.bf16_bits_to_f64(v)).permute(1, 0, 2)
    kt = kt.repeat_interleave(group, dim=0)
    vt = vt.repeat_interleave(group, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :]
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(12)
    t = 50
    k = _rand_bf16(rng, (t, 1, 128))
    v = _rand_bf16(rng, (t, 1, 128))
    # q = 0: uniform weights -> mean of V
    q0 = np.zeros((4, 128), dtype=np.uint16)
    np.testing.assert_allclose(attention.attention_fp64(q0, k, v, 0.1),
                               np.repeat(codec.bf16_bits_to_f64(v).mean(axis=0), 4, axis=0),
                               rtol=1e-13, atol=1e-15)
    # constant V -> that V
    vc = np.repeat(v[:1], t, axis=0)
    q = _rand_bf16(rng, (4, 128))
    np.testing.assert_allclose(attention.attention_fp64(q, k, vc, 0.1),
                               np.repeat(codec.bf16_bits_to_f64(v[0]), 4, axis=0), rtol=1e-13)
    # one dominant logit -> that token's V
    kd = k.copy()
    kd[17, 0, :] = _bf16(np.full(128, 64.0) * np.sign(codec.bf16_bits_to_f64(q[0])))
    got = attention.attention_fp64(q[:1], kd, v, 1.0)
    np.testing.assert_allclose(got[0], codec.bf16_bits_to_f64(v[17, 0]), rtol=1e-12)
    # a single token -> its V
    np.testing.assert_allclose(attention.attention_fp64(q, k[:1], v[:1], 0.1),
                               np.repeat(codec.bf16_bits_to_f64(v[0]), 4, axis=0), rtol=1e-13)
    # empty sequence -> zeros (reading)
    assert not attention.attention_fp64(q, k[:0], v[:0], 0.1).any()


def test_softmax_weights_closed_forms_and_brute_force():
    rng = np.random.default_rng(15)
    t = 40
    k = _rand_bf16(rng, (t, 2, 128))
    # q = 0: every key weighs 1/T
    w0 = attention.softmax_weights_fp64(np.zeros((4, 128), dtype=np.uint16), k, 0.1)
    np.testing.assert_allclose(w0, np.full((4, t), 1.0 / t), rtol=1e-14)
    # one dominant logit: one-hot on that key, for the heads of its KV group only
    q = _rand_bf16(rng, (4, 128))
    kd = k.copy()
    kd[9, 0, :] = _bf16(np.full(128, 64.0) * np.sign(codec.bf16_bits_to_f64(q[0])))
    w = attention.softmax_weights_fp64(q, kd, 1.0)
    assert w[0, 9] == 1.0 and w[0].sum() == 1.0
    assert w[2].max() < 1.0
    # brute force (pure Python exp over the scores)
    qf, kf = codec.bf16_bits_to_f64(q), codec.bf16_bits_to_f64(k)
    w = attention.softmax_weights_fp64(q, k, 0.2)
    for h in range(4):
        g = h // 2
        s = [0.2 * sum(float(qf[h, d]) * float(kf[tt, g, d]) for d in range(128)) for tt in range(t)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        for tt in range(t):
            assert abs(w[h, tt] - e[tt] / sum(e)) <= 1e-13


def test_paged_compressed_cache_equals_dense_attention():
    """Compressed pages read through the block table plus a ragged tail give exactly the
    attention of the plain dense K/V (one softmax over both, GAAC 'Attention with
    On-the-Fly Decompression')."""
    rng = np.random.default_rng(13)
    bsz, hkv, group, n_phys = 3, 2, 4, 12
    seq_lens = [16 * 3 + 5, 16 * 4, 7]
    n_comp = [3, 4, 0]
    max_pages = 5
    pages = _rand_bf16(rng, (n_phys, 2, hkv, 16, 128), 3.0)
    cache = OracleCache(1 << 20)
    # item order: (phys page, kv head, K/V)
    flat = pages.transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)
    kinds = [n % 2 for n in range(flat.shape[0])]
    metas = cache.encode(flat, kinds)
    meta_table = [[[metas[(p * hkv + g) * 2 + kv] for kv in range(2)] for g in range(hkv)]
                  for p in range(n_phys)]
    perm = rng.permutation(n_phys)
    block_table = np.zeros((bsz, max_pages), dtype=np.int32)
    used = 0
    for b in range(bsz):
        block_table[b, :n_comp[b]] = perm[used:used + n_comp[b]]
        used += n_comp[b]
    tail = _rand_bf16(rng, (bsz, 2, hkv, 16, 128), 3.0)
    q = _rand_bf16(rng, (bsz, hkv * group, 128))
    got = attention.decode_attention(q, cache.arena, meta_table, block_table, seq_lens,
                                     n_comp, tail, 0.125)
    for b in range(bsz):
        ks, vs = [], []
        for p in range(n_comp[b]):
            ks.append(pages[block_table[b, p], 0].transpose(1, 0, 2))
            vs.append(pages[block_table[b, p], 1].transpose(1, 0, 2))
        nt = seq_lens[b] - 16 * n_comp[b]
        ks.append(tail[b, 0, :, :nt].transpose(1, 0, 2))
        vs.append(tail[b, 1, :, :nt].transpose(1, 0, 2))
        ref = attention.attention_fp64(q[b], np.concatenate(ks), np.concatenate(vs), 0.125)
        np.testing.assert_array_equal(got[b], ref)


def test_non_finite_propagates():
    rng = np.random.default_rng(14)
    k = _rand_bf16(rng, (10, 1, 128))
    v = _rand_bf16(rng, (10, 1, 128))
    q = _rand_bf16(rng, (2, 128))
    v[3, 0, 5] = 0x7FC0
    out = attention.attention_fp64(q, k, v, 0.1)
    assert np.isnan(out[:, 5]).all() and np.isfinite(np.delete(out, 5, axis=1)).all()
    k[4, 0, 0] = 0x7FC0
    assert np.isnan(attention.attention_fp64(q, k, v, 0.1)).all()
