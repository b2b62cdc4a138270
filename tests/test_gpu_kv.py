"""GPU parity: NVFP4 KV cache append / read (bit-exact vs the oracle) and the
decode-step QK sweep (relative Frobenius error <= 1e-5 vs the fp64 oracle)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, np_, rel_frobenius

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")
QK_TOL = 1e-5


def _cache(L, H, D, cap, seed):
    gen = torch.Generator().manual_seed(seed)
    kg = (torch.rand((L, H), generator=gen) * 0.003 + 0.0005).float()
    vg = (torch.rand((L, H), generator=gen) * 0.003 + 0.0005).float()
    return nv.KVCache(L, H, D, cap, kg, vg, device="cuda"), np_(kg), np_(vg)


def _oracle_cache(cache, k, v, kg, vg):
    """The oracle's encoding of tokens [0, n) appended from k, v ([L][n][H][D]
    bf16).  The cache's bytes must agree, and the expected values are then
    computed from the oracle's encoding alone."""
    n = k.shape[1]
    kq, ks = oracle.kv_encode(bits(k), kg)
    vq, vs = oracle.kv_encode(bits(v), vg)
    for got, want, what in ((cache.k, kq, "K codes"), (cache.k_sf, ks, "K scales"), (cache.v, vq, "V codes"),
                            (cache.v_sf, vs, "V scales")):
        assert np.array_equal(np_(got[:, :, :n]), want), what
    return kq, ks, vq, vs


@pytest.mark.parametrize("D,grp", [(128, 4), (64, 2), (32, 1), (256, 8), (16, 4), (128, 16), (64, 3), (256, 5),
                                   (128, 1), (128, 8), (64, 4), (64, 8), (128, 2)])
def test_append_read_qk_small(D, grp):
    print("case: kv small D", D, "grp", grp, flush=True)
    L, H, cap = 3, 2, 300
    cache, kg, vg = _cache(L, H, D, cap, D + grp)
    gen = torch.Generator().manual_seed(11 * D + grp)
    ks, vs = [], []
    bounds = [0, 1, 8, 100, 257, 300]
    for a, b in zip(bounds, bounds[1:]):
        k = (torch.randn((L, b - a, H, D), generator=gen) * 2).to(torch.bfloat16)
        v = torch.randn((L, b - a, H, D), generator=gen).to(torch.bfloat16)
        cache.append(a, k.cuda(), v.cuda())
        ks.append(bits(k))
        vs.append(bits(v))
    torch.cuda.synchronize()
    kall = np.concatenate(ks, axis=1)
    vall = np.concatenate(vs, axis=1)
    okq, oks = oracle.kv_encode(kall, kg)
    ovq, ovs = oracle.kv_encode(vall, vg)
    assert np.array_equal(np_(cache.k), okq) and np.array_equal(np_(cache.k_sf), oks)
    assert np.array_equal(np_(cache.v), ovq) and np.array_equal(np_(cache.v_sf), ovs)
    # read a window of layers / tokens
    kr, vr = cache.read(1, 2, 5, 250)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kr), oracle.kv_read(okq[1:3, :, 5:255], oks[1:3, :, 5:255], kg[1:3]))
    assert np.array_equal(bits(vr), oracle.kv_read(ovq[1:3, :, 5:255], ovs[1:3, :, 5:255], vg[1:3]))
    # decode QK over the first n tokens
    qv = torch.randn((L, H * grp, D), generator=gen).to(torch.bfloat16)
    for n in (1, 77, 300):
        logits = cache.decode_qk(qv.cuda(), n)
        torch.cuda.synchronize()
        want = oracle.decode_qk_f64(bits(qv), okq[:, :, :n], oks[:, :, :n], kg)
        err = rel_frobenius(np_(logits), want)
        assert err <= QK_TOL, f"n={n}: rel Frobenius {err:.3e}"


def test_append_on_two_streams():
    """Consecutive 256-token appends alternating between two streams (they
    write disjoint token ranges, so they may run at once), joined at the end:
    every cache byte against the oracle."""
    print("case: kv append on two streams", flush=True)
    L, H, D, cap, C = 3, 2, 128, 16 * 256, 256
    cache, kg, vg = _cache(L, H, D, cap, 77)
    gen = torch.Generator().manual_seed(77)
    ks, vs, chunks = [], [], []
    for c in range(cap // C):
        k = (torch.randn((L, C, H, D), generator=gen) * 2).to(torch.bfloat16)
        v = torch.randn((L, C, H, D), generator=gen).to(torch.bfloat16)
        chunks.append((k.cuda(), v.cuda()))
        ks.append(bits(k))
        vs.append(bits(v))
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    main = torch.cuda.current_stream()
    for s in side:
        s.wait_stream(main)
    for c, (k, v) in enumerate(chunks):
        cache.append(c * C, k, v, stream=side[c % 2])
    for s in side:
        main.wait_stream(s)
    torch.cuda.synchronize()
    okq, oks = oracle.kv_encode(np.concatenate(ks, axis=1), kg)
    ovq, ovs = oracle.kv_encode(np.concatenate(vs, axis=1), vg)
    assert np.array_equal(np_(cache.k), okq) and np.array_equal(np_(cache.k_sf), oks)
    assert np.array_equal(np_(cache.v), ovq) and np.array_equal(np_(cache.v_sf), ovs)


def test_append_read_non_pow2_head_dim():
    """head_dim 48: three blocks per row (the non-power-of-two append path);
    the decode sweep reports the documented ENOTSUP for it."""
    L, H, D, cap = 2, 3, 48, 70
    cache, kg, vg = _cache(L, H, D, cap, 48)
    gen = torch.Generator().manual_seed(48)
    k = (torch.randn((L, 70, H, D), generator=gen) * 3).to(torch.bfloat16)
    v = torch.randn((L, 70, H, D), generator=gen).to(torch.bfloat16)
    cache.append(0, k[:, :33].contiguous().cuda(), v[:, :33].contiguous().cuda())
    cache.append(33, k[:, 33:].contiguous().cuda(), v[:, 33:].contiguous().cuda())
    torch.cuda.synchronize()
    okq, oks = oracle.kv_encode(bits(k), kg)
    ovq, ovs = oracle.kv_encode(bits(v), vg)
    assert np.array_equal(np_(cache.k), okq) and np.array_equal(np_(cache.k_sf), oks)
    assert np.array_equal(np_(cache.v), ovq) and np.array_equal(np_(cache.v_sf), ovs)
    kr, vr = cache.read(0, 2, 3, 60)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kr), oracle.kv_read(okq[:, :, 3:63], oks[:, :, 3:63], kg))
    qv = torch.randn((L, 2 * H, D), generator=gen).to(torch.bfloat16).cuda()
    with pytest.raises(nv.NVFP4Error):
        cache.decode_qk(qv, 10)


@pytest.mark.parametrize("D,grp", [(128, 4), (64, 2), (32, 1), (256, 8), (16, 4), (128, 1), (128, 16), (64, 3),
                                   (256, 5)])
def test_decode_attention_small(D, grp):
    """Decode attention (QK, softmax, P.V) against the fp64 oracle for token
    counts that leave ragged splits, including a single token."""
    print("case: kv attention D", D, "grp", grp, flush=True)
    L, H, cap = 2, 3, 700
    cache, kg, vg = _cache(L, H, D, cap, 7 * D + grp)
    gen = torch.Generator().manual_seed(3 * D + grp)
    k = (torch.randn((L, cap, H, D), generator=gen) * 2).to(torch.bfloat16)
    v = torch.randn((L, cap, H, D), generator=gen).to(torch.bfloat16)
    cache.append(0, k.cuda(), v.cuda())
    qv = torch.randn((L, H * grp, D), generator=gen).to(torch.bfloat16)
    kq, ks, vq, vs = _oracle_cache(cache, k, v, kg, vg)
    scale = 1.0 / np.sqrt(D)
    for n in (1, 63, 300, 700):
        out = cache.decode_attention(qv.cuda(), n, scale)
        torch.cuda.synchronize()
        want = oracle.decode_attention_f64(bits(qv), kq[:, :, :n], ks[:, :, :n], kg, vq[:, :, :n], vs[:, :, :n],
                                           vg, scale)
        err = rel_frobenius(np_(out), want)
        assert err <= QK_TOL, f"n={n}: rel Frobenius {err:.3e}"


@pytest.mark.parametrize("D,grp", [(128, 4), (64, 2), (32, 2)])
@pytest.mark.parametrize("scale_kind", ["negative", "zero", "large"])
def test_decode_attention_scale_sign_and_size(D, grp, scale_kind):
    """Softmax scales that are negative (the running max is then taken on
    the negated logits), zero (uniform weights over the tokens) or large
    (near one-hot weights), against the fp64 oracle, on the MFMA kernel
    (head_dim 64, 128) and the VALU kernel (head_dim 32)."""
    print("case: kv attention scale", scale_kind, "D", D, "grp", grp, flush=True)
    L, H, cap = 2, 2, 333
    cache, kg, vg = _cache(L, H, D, cap, 5 * D + grp)
    gen = torch.Generator().manual_seed(13 * D + grp)
    k = (torch.randn((L, cap, H, D), generator=gen) * 2).to(torch.bfloat16)
    v = torch.randn((L, cap, H, D), generator=gen).to(torch.bfloat16)
    cache.append(0, k.cuda(), v.cuda())
    qv = torch.randn((L, H * grp, D), generator=gen).to(torch.bfloat16)
    kq, ks, vq, vs = _oracle_cache(cache, k, v, kg, vg)
    scale = {"negative": -1.0 / np.sqrt(D), "zero": 0.0, "large": 8.0}[scale_kind]
    for n in (1, 200, 333):
        out = cache.decode_attention(qv.cuda(), n, scale)
        torch.cuda.synchronize()
        want = oracle.decode_attention_f64(bits(qv), kq[:, :, :n], ks[:, :, :n], kg, vq[:, :, :n], vs[:, :, :n],
                                           vg, scale)
        err = rel_frobenius(np_(out), want)
        assert err <= QK_TOL, f"n={n}: rel Frobenius {err:.3e}"


@pytest.mark.parametrize("k", [-100, -20, 0, 30, 100])
def test_decode_attention_query_magnitudes(k):
    """Queries scaled by 2^k (with the softmax scale taking 2^-k back) and a
    head whose elements span 40 binades: the per-head power-of-two scaling
    of q keeps the logits exact enough for the 1e-5 bar."""
    print("case: kv attention q magnitude 2^", k, flush=True)
    L, H, D, grp, cap = 1, 2, 128, 4, 200
    cache, kg, vg = _cache(L, H, D, cap, 1000 + k)
    gen = torch.Generator().manual_seed(77 + k)
    kk = (torch.randn((L, cap, H, D), generator=gen) * 2).to(torch.bfloat16)
    vv = torch.randn((L, cap, H, D), generator=gen).to(torch.bfloat16)
    cache.append(0, kk.cuda(), vv.cuda())
    qf = torch.randn((L, H * grp, D), generator=gen) * 2.0 ** k
    qf[0, 1] *= torch.exp2(torch.randint(-40, 1, (D,), generator=gen).float())   # mixed binades in one head
    qv = qf.to(torch.bfloat16)
    scale = 2.0 ** -k / np.sqrt(D)
    out = cache.decode_attention(qv.cuda(), cap, scale)
    torch.cuda.synchronize()
    kq, ks, vq, vs = _oracle_cache(cache, kk, vv, kg, vg)
    want = oracle.decode_attention_f64(bits(qv), kq, ks, kg, vq, vs, vg, scale)
    err = rel_frobenius(np_(out), want)
    assert err <= QK_TOL, f"rel Frobenius {err:.3e}"


@pytest.mark.parametrize("k", [-100, -20, 0, 30, 100])
def test_decode_qk_query_magnitudes(k):
    """Queries scaled by 2^k and a head whose elements span 40 binades: the
    decode-QK forms fp32 dot products of the bf16 queries with the E2M1
    values (exact products) and applies the block and tensor scales to the
    partial sums, with no rounding of q, so the logits stay within the 1e-5
    bar at any magnitude."""
    print("case: kv decode-QK q magnitude 2^", k, flush=True)
    L, H, D, grp, cap = 1, 2, 128, 4, 200
    cache, kg, vg = _cache(L, H, D, cap, 2000 + k)
    gen = torch.Generator().manual_seed(99 + k)
    kk = (torch.randn((L, cap, H, D), generator=gen) * 2).to(torch.bfloat16)
    cache.append(0, kk.cuda(), kk.cuda())
    qf = torch.randn((L, H * grp, D), generator=gen) * 2.0 ** k
    qf[0, 1] *= torch.exp2(torch.randint(-40, 1, (D,), generator=gen).float())   # mixed binades in one head
    qv = qf.to(torch.bfloat16)
    logits = cache.decode_qk(qv.cuda(), 197)
    torch.cuda.synchronize()
    kq, ks, _, _ = _oracle_cache(cache, kk, kk, kg, vg)
    want = oracle.decode_qk_f64(bits(qv), kq[:, :, :197], ks[:, :, :197], kg)
    err = rel_frobenius(np_(logits), want)
    assert err <= QK_TOL, f"rel Frobenius {err:.3e}"


def test_decode_attention_rejects_unsupported_shapes():
    cache, kg, vg = _cache(1, 2, 48, 10, 1)
    with pytest.raises(nv.NVFP4Error):
        cache.decode_attention(torch.zeros((1, 2, 48), dtype=torch.bfloat16, device="cuda"), 5, 0.1)
    cache, kg, vg = _cache(1, 2, 32, 10, 1)
    with pytest.raises(nv.NVFP4Error):                 # head_dim 32 runs 1, 2, 4 or 8 query heads per KV head
        cache.decode_attention(torch.zeros((1, 6, 32), dtype=torch.bfloat16, device="cuda"), 5, 0.1)
    cache, kg, vg = _cache(1, 2, 64, 10, 1)
    with pytest.raises(nv.NVFP4Error):                 # more than 16 query heads per KV head
        cache.decode_attention(torch.zeros((1, 34, 64), dtype=torch.bfloat16, device="cuda"), 5, 0.1)
    with pytest.raises(nv.NVFP4Error):                 # n = 0: a softmax over no tokens
        cache.decode_attention(torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda"), 0, 0.1)


def test_read_only_k_or_v():
    cache, kg, vg = _cache(2, 2, 64, 40, 3)
    k = torch.randn((2, 40, 2, 64)).to(torch.bfloat16)
    v = torch.randn((2, 40, 2, 64)).to(torch.bfloat16)
    cache.append(0, k.cuda(), v.cuda())
    kr, vr = cache.read(0, 2, 0, 40, want_v=False)
    torch.cuda.synchronize()
    assert vr is None
    okq, oks = oracle.kv_encode(bits(k), kg)
    assert np.array_equal(bits(kr), oracle.kv_read(okq, oks, kg))


def calibrated_kv_scales(L, H, T, C):
    """Per-(layer, KV head) tensor scales of K and V, fixed at cache creation
    from a calibration pass over the whole seeded stream: the codec's own
    tensor-scale rule g = RN32(amax / 2688), applied by nvfp4_quantize to one
    16-value block per (layer, head) holding that head's amax over every
    chunk (the amax of bf16 values is a bf16 value)."""
    kmax = torch.zeros((L, H), dtype=torch.bfloat16, device="cuda")
    vmax = torch.zeros_like(kmax)
    for c in range(T // C):
        k, v = synth.kv_chunk(c, device="cuda")
        kmax = torch.maximum(kmax, k.abs().amax(dim=(1, 3)))
        vmax = torch.maximum(vmax, v.abs().amax(dim=(1, 3)))
    blocks = torch.zeros((2 * L * H, 1, 16), dtype=torch.bfloat16, device="cuda")
    blocks[:, 0, 0] = torch.cat([kmax.reshape(-1), vmax.reshape(-1)])
    _, _, g = nv.quantize(blocks)
    return g[:L * H].reshape(L, H).clone(), g[L * H:].reshape(L, H).clone()


SAMPLED_CHUNKS = (0, 1, 2, 63, 64, 100, 127, 128, 255, 256, 257, 383, 384, 450, 510, 511)


def test_full_context_sampled():
    """32 layers x 8 KV heads x 128 dims, 131072 tokens appended in 512 chunks of
    256, with calibrated per-(layer, head, K|V) tensor scales.  Every chunk's
    append is checked byte for byte (the whole 4.5 GiB cache); decode QK for 32 query heads
    (GQA 4:1) on every token and full decode attention on sampled
    (layer, KV head) pairs against fp64; kv_read of layers 0-3 over every token
    (the benchmarked read) bit for bit on the sampled tokens.  Every expected
    value is computed from the oracle's own encoding of the input chunks."""
    print("case: kv full context 32x8x128x131072", flush=True)
    L, H, D, T, C = 32, 8, 128, 131072, 256
    kg, vg = calibrated_kv_scales(L, H, T, C)
    cache = nv.KVCache(L, H, D, T, kg, vg, device="cuda")
    pairs = ((0, 0), (5, 3), (11, 6), (17, 5), (20, 1), (26, 2), (29, 4), (31, 7))   # every KV head once
    kin = {p: [] for p in pairs}
    vin = {p: [] for p in pairs}
    kgn, vgn = np_(kg), np_(vg)
    qv = synth.kv_query(device="cuda")
    qb = bits(qv)
    want_qk = np.empty((L, 4 * H, T), dtype=np.float64)   # fp64 logits from the oracle's encoding, chunk by chunk
    for c in range(T // C):
        k, v = synth.kv_chunk(c, device="cuda")
        cache.append(c * C, k, v)
        for (l, h) in pairs:                          # inputs of the attention check
            kin[(l, h)].append(bits(k[l:l + 1, :, h:h + 1].contiguous()))
            vin[(l, h)].append(bits(v[l:l + 1, :, h:h + 1].contiguous()))
        # every chunk's append, byte for byte (the whole cache over the run)
        sl = slice(c * C, (c + 1) * C)
        okq, oks = oracle.kv_encode(bits(k), kgn)
        ovq, ovs = oracle.kv_encode(bits(v), vgn)
        want_qk[:, :, sl] = oracle.decode_qk_f64(qb, okq, oks, kgn)
        assert np.array_equal(np_(cache.k[:, :, sl]), okq), f"chunk {c} K codes"
        assert np.array_equal(np_(cache.k_sf[:, :, sl]), oks), f"chunk {c} K scales"
        assert np.array_equal(np_(cache.v[:, :, sl]), ovq), f"chunk {c} V codes"
        assert np.array_equal(np_(cache.v_sf[:, :, sl]), ovs), f"chunk {c} V scales"
    torch.cuda.synchronize()
    enc = {}
    for c in SAMPLED_CHUNKS:                          # the oracle's encoding of the sampled chunks
        k, v = synth.kv_chunk(c, device="cuda")
        enc[c] = oracle.kv_encode(bits(k), kgn) + oracle.kv_encode(bits(v), vgn)
    toks = np.concatenate([np.arange(c * C, (c + 1) * C) for c in SAMPLED_CHUNKS])
    okq, oks, ovq, ovs = (np.concatenate([enc[c][i] for c in SAMPLED_CHUNKS], axis=2) for i in range(4))
    logits = cache.decode_qk(qv, T)                   # every logit of the 131072-token sweep
    torch.cuda.synchronize()
    err = rel_frobenius(np_(logits), want_qk)
    assert err <= QK_TOL, f"rel Frobenius {err:.3e}"
    del logits, want_qk
    kr, vr = cache.read(0, 4, 0, T)
    assert np.array_equal(bits(kr[:, :, toks]), oracle.kv_read(okq[0:4], oks[0:4], kgn[0:4])), "kv_read K"
    assert np.array_equal(bits(vr[:, :, toks]), oracle.kv_read(ovq[0:4], ovs[0:4], vgn[0:4])), "kv_read V"
    del kr, vr
    # full decode attention over all 131072 tokens, checked on sampled (layer, KV head) pairs
    out = np_(cache.decode_attention(qv, T, 1.0 / np.sqrt(D)))
    for (l, h) in pairs:
        pkq, pks = oracle.kv_encode(np.concatenate(kin[(l, h)], axis=1), kgn[l:l + 1, h:h + 1])
        pvq, pvs = oracle.kv_encode(np.concatenate(vin[(l, h)], axis=1), vgn[l:l + 1, h:h + 1])
        want = oracle.decode_attention_f64(bits(qv)[l:l + 1, 4 * h:4 * h + 4], pkq, pks, kgn[l:l + 1, h:h + 1],
                                           pvq, pvs, vgn[l:l + 1, h:h + 1], 1.0 / np.sqrt(D))
        err = rel_frobenius(out[l:l + 1, 4 * h:4 * h + 4], want)
        assert err <= QK_TOL, f"attention l={l} h={h}: rel Frobenius {err:.3e}"
    del cache
