"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.

  * codes, bit planes, QJL bits and fp16 norms: bit-exact except coordinates within 1e-6
    of a decision boundary (see tests/parity.py), at most 1e-6 of all codes;
  * decode attention: max-abs 2e-3 against the oracle attending over the same packed cache
    (the oracle's own packing, uploaded), and end-to-end against oracle encode + attend;
  * search: top-10 identical up to swaps of near-equal scores (|diff| <= 1e-6).
Small cases span several tiles and ragged tails; the full-size cases use the launch
configuration bench.py times and compare sampled (batch, kv-head) units.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

from oracle import tq_oracle as O
from vector_quantization_rope_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vector_quantization_rope_amd import tq as _tq
    return _tq


@pytest.fixture(scope="module")
def P():
    import parity
    return parity


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build(tq, w, K, V, chunks=None, capacity=None):
    B, H, T, d = K.shape
    codec = tq.Codec(d, w.bits_k, w.bits_v, w.m, seed=0)
    cache = tq.PackedCache(B, H, d, capacity or T, w.bits_k, w.bits_v, w.m)
    chunks = chunks or [(0, T)]
    for s, e in chunks:
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, s:e].contiguous(),
                       V[:, :, s:e].contiguous() if V is not None else None, s, w.rope_base)
    return codec, cache


def decode(tq, codec, cache, q, length, q_pos, rope_base, splits=0, want_scores=True):
    B, Hq, d = q.shape
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    scores = torch.empty((B, Hq, max(1, length)), dtype=torch.float32, device="cuda") if want_scores else None
    nws = tq.decode_workspace_bytes(cache.desc, Hq, length, splits=splits)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    tq.decode_attend(cache.desc, codec.dev, cache.buf, length, q, q_pos, rope_base, out,
                     scores=scores, ws=ws, splits=splits)
    torch.cuda.synchronize()
    return out, scores


def oracle_side(P, w, K, V, q, length, codec_o):
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    T = Kd.shape[2]
    fields = P.oracle_encode_unitwise(Kd, Vd, codec_o, np.arange(T), w.rope_base)
    out, scores = O.attend(fields, P.to_f64(q), codec_o, q_pos=w.q_pos, rope_base=w.rope_base,
                           scale=0.0, kv_heads=K.shape[1], length=length)
    return fields, out, scores


def check_case(tq, P, w, K, V, q, chunks=None, splits=0, label=""):
    """Full check of one small case: codes, decode over the oracle's cache, end to end."""
    B, H, T, d = K.shape
    say(f"[case] {label} B={B} Hkv={H} Hq={q.shape[1]} T={T} d={d} chunks={chunks} splits={splits}")
    codec, cache = build(tq, w, K.cuda(), V.cuda(), chunks)
    codec_o = O.make_codec(d, w.bits_k, w.bits_v, w.m, 0)
    fields, out_o, sc_o = oracle_side(P, w, K, V, q, T, codec_o)
    rep = {}
    P.compare_codes(P.gpu_fields(cache, T), fields, codec_o, rep)
    # decode over the oracle's packed cache
    img = P.oracle_image(cache.desc.as_dict(), fields)
    ocache = tq.PackedCache(B, H, d, T, w.bits_k, w.bits_v, w.m)
    ocache.buf.copy_(torch.from_numpy(img))
    out, sc = decode(tq, codec, ocache, q.cuda(), T, w.q_pos, w.rope_base, splits=splits)
    e_out = P.max_abs(out.cpu().numpy(), out_o)
    e_sc = P.max_abs(sc.cpu().numpy()[:, :, :T], sc_o)
    # end to end: the GPU's own cache
    out2, _ = decode(tq, codec, cache, q.cuda(), T, w.q_pos, w.rope_base, splits=splits, want_scores=False)
    e_e2e = P.max_abs(out2.cpu().numpy(), out_o)
    say(f"    codes {rep} | out {e_out:.2e} scores {e_sc:.2e} e2e {e_e2e:.2e}")
    assert e_out <= TOL and e_sc <= TOL
    if rep["excused"] == 0:
        assert e_e2e <= TOL
    return rep


# ------------------------------------------------------------------ small cases
def test_single_head_workload_full(tq, P):
    """Single head, d 128, 1024 fp32 N(0,1) keys/values with 4 channels x20, no RoPE."""
    w = W.SINGLE_HEAD
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    check_case(tq, P, w, K, V, q, label="single_head")


@pytest.mark.parametrize("d,G,T,chunks", [
    (128, 4, 1000, [(0, 100), (100, 237), (237, 1000)]),
    (128, 8, 777, None),
    (64, 1, 333, [(0, 31), (31, 64), (64, 333)]),
    (64, 4, 2100, None),
])
def test_gqa_ragged_and_appends(tq, P, d, G, T, chunks):
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    check_case(tq, P, w, K, V, q, chunks=chunks, label=f"gqa d{d} G{G}")


@pytest.mark.parametrize("bk,d,G,T,dist", [
    (1, 128, 8, 700, "laplace"),
    (3, 128, 8, 700, "laplace"),
    (1, 64, 4, 500, "laplace"),
    (3, 64, 2, 530, "laplace"),
    (3, 64, 1, 1024, "student_t3"),
    # groups of at most 4 query heads at d = 128 take the 16-row key-score kernel
    (1, 128, 4, 640, "laplace"),
    (3, 128, 2, 650, "normal"),
    (2, 128, 3, 515, "laplace"),
    (3, 128, 1, 333, "normal"),
])
def test_mfma_key_widths(tq, P, bk, d, G, T, dist):
    """1-bit and 3-bit keys (+ QJL) with 3-bit values on the MFMA decode path: for 3-bit
    codes the code term is split over the three bit planes and their parity."""
    w = W.LONG_CONTEXT.scaled(batch=1, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=bk,
                              dist=dist, outliers=3 if dist == "student_t3" else 4,
                              outlier_scale=15.0 if dist == "student_t3" else 20.0,
                              rope_base=10000.0 if dist == "student_t3" else 500000.0)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    check_case(tq, P, w, K, V, q, label=f"mfma keys {bk}-bit d{d} G{G} {dist}")


@pytest.mark.parametrize("bk,bv,d,G,T", [
    (2, 3, 128, 8, 1300), (3, 3, 128, 4, 700), (1, 3, 64, 8, 530), (3, 3, 64, 2, 300), (3, 4, 128, 4, 300),
])
def test_logits_only(tq, P, bk, bv, d, G, T):
    """out = NULL: the scores alone (the MFMA key formats run a logits-only kernel; other
    formats the full split kernel without the merge), against the oracle's scores and the
    scores of a full decode."""
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=bk, bits_v=bv)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    codec, cache = build(tq, w, K.cuda(), V.cuda())
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    fields, _, sc_o = oracle_side(P, w, K, V, q, T, codec_o)
    img = P.oracle_image(cache.desc.as_dict(), fields)
    ocache = tq.PackedCache(w.batch, w.kv_heads, d, T, w.bits_k, w.bits_v, w.m)
    ocache.buf.copy_(torch.from_numpy(img))
    B, Hq = q.shape[0], q.shape[1]
    sc = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.decode_workspace_bytes(ocache.desc, Hq, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(ocache.desc, codec.dev, ocache.buf, T, q.cuda(), w.q_pos, w.rope_base, None,
                     scores=sc, ws=ws)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    assert np.isfinite(got).all()
    e = P.max_abs(got, sc_o)
    _, sc_full = decode(tq, codec, ocache, q.cuda(), T, w.q_pos, w.rope_base)
    full = sc_full.cpu().numpy()[:, :, :T]
    e_full = P.max_abs(got, full)
    say(f"    logits only k{bk} v{bv} d{d} G{G}: vs oracle {e:.2e}, vs full decode {e_full:.2e}")
    # the full decode forms scale * score and divides the scale out again: a few fp32 ulps
    assert e <= TOL and e_full <= 1e-6 * max(1.0, float(np.abs(full).max()))


@pytest.mark.parametrize("bk,bv,d,G,L,Wn,cap,dt", [
    (2, 3, 128, 8, 700, 45, 64, "bf16"),   # MFMA path, partial window
    (3, 3, 64, 2, 300, 64, 64, "bf16"),    # full window
    (2, 3, 128, 4, 0, 100, 128, "bf16"),   # window only
    (2, 3, 64, 4, 257, 0, 32, "bf16"),     # empty window
    (1, 3, 64, 8, 130, 200, 256, "f32"),   # fp32 inputs, window longer than the packed part
    (3, 4, 128, 4, 190, 70, 80, "f32"),    # fp32 decode path
    (2, 3, 64, 16, 150, 600, 640, "f16"),  # f16, 16 q-heads per kv-head (fp32 decode path), 10 chunks
    (2, 3, 128, 16, 260, 90, 128, "bf16"), # d 128 with 16 head slots
    (2, 3, 128, 12, 200, 64, 64, "f32"),   # d 128, fp32 window, 12 q-heads per kv-head (not a power of two)
    (3, 3, 64, 16, 100, 33, 64, "f32"),    # d 64, fp32 window with 16 head slots
])
def test_window_attention(tq, P, bk, bv, d, G, L, Wn, cap, dt):
    """Packed tokens [0, L) plus a full-precision window of Wn raw tokens (NSNQuant's
    residual): outputs and scores against the oracle over the same packed fields; logits
    only; and, for a full window, the flush through tq_quantize_kv."""
    T = L + Wn
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=bk, bits_v=bv,
                              dtype=dt)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    codec_o = O.make_codec(d, bk, bv, d, 0)
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    fields = P.oracle_encode_unitwise(Kd[:, :, :L], Vd[:, :, :L], codec_o, np.arange(L), w.rope_base)
    out_o, sc_o = O.attend_window(fields, Kd[:, :, L:], Vd[:, :, L:], P.to_f64(q), codec_o, q_pos=w.q_pos,
                                  rope_base=w.rope_base, scale=0.0, kv_heads=w.kv_heads, length=L, win_len=Wn)
    codec = tq.Codec(d, bk, bv, d, seed=0)
    cap_t = max(T, 1)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, cap_t, bk, bv, d)
    if L > 0:
        cache.buf.copy_(torch.from_numpy(P.oracle_image(cache.desc.as_dict(), fields)))
    wk = torch.zeros((w.batch, w.kv_heads, cap, d), dtype=K.dtype)
    wv = torch.zeros_like(wk)
    wk[:, :, :Wn] = K[:, :, L:]
    wv[:, :, :Wn] = V[:, :, L:]
    wk, wv = wk.cuda(), wv.cuda()
    B, Hq = q.shape[0], q.shape[1]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, max(T, 1)), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.decode_window_workspace_bytes(cache.desc, Hq, L), dtype=torch.uint8, device="cuda")
    tq.decode_attend_window(cache.desc, codec.dev, cache.buf, L, wk, wv, Wn, q.cuda(), w.q_pos, w.rope_base,
                            out, scores=sc, ws=ws)
    torch.cuda.synchronize()
    e_out = P.max_abs(out.cpu().numpy(), out_o)
    e_sc = P.max_abs(sc.cpu().numpy()[:, :, :T], sc_o)
    # logits only
    sc2 = torch.full_like(sc, float("nan"))
    tq.decode_attend_window(cache.desc, codec.dev, cache.buf, L, wk, wv, Wn, q.cuda(), w.q_pos, w.rope_base,
                            None, scores=sc2, ws=ws)
    torch.cuda.synchronize()
    e_lg = P.max_abs(sc2.cpu().numpy()[:, :, :T], sc_o)
    say(f"    window k{bk} v{bv} d{d} G{G} L{L} W{Wn} {dt}: out {e_out:.2e} scores {e_sc:.2e} logits-only {e_lg:.2e}")
    assert e_out <= TOL and e_sc <= TOL and e_lg <= TOL
    if Wn == cap and L > 0:
        # flush the full window into the packed cache, then a plain decode over L + Wn
        # tokens matches the oracle over the GPU-encoded cache
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, wk, wv, L, w.rope_base)
        out3, _ = decode(tq, codec, cache, q.cuda(), T, w.q_pos, w.rope_base, want_scores=False)
        g = P.gpu_fields(cache, T)
        o3, _ = O.attend(g, P.to_f64(q), codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                         kv_heads=w.kv_heads, length=T)
        e3 = P.max_abs(out3.cpu().numpy(), o3)
        say(f"    after flush: out {e3:.2e}")
        assert e3 <= TOL


@pytest.mark.parametrize("bk,d,G,L0,T,dist", [
    (2, 128, 8, 700, 900, "laplace"),      # MFMA path, means from a prefill, ragged append
    (3, 64, 4, 300, 530, "student_t3"),
    (1, 128, 2, 64, 64, "normal"),         # means over the whole cache
])
def test_nsn_codes_and_decode(tq, P, bk, d, G, L0, T, dist):
    """NSN caches (NSNQuant section 1): the means over the prefill, codes and s1 of every
    token against the oracle's NSN encode; decode and logits over the oracle's NSN cache
    and end to end over the GPU's own."""
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=bk, bits_v=3,
                              dist=dist)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    codec_o = O.make_codec(d, bk, 3, d, 0)
    means = P.oracle_means(Kd[:, :, :L0], Vd[:, :, :L0], np.arange(L0), w.rope_base)
    fields = P.oracle_encode_unitwise(Kd, Vd, codec_o, np.arange(T), w.rope_base, means)
    codec = tq.Codec(d, bk, 3, d, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, bk, 3, d, nsn=1)
    Kc, Vc = K.cuda(), V.cuda()
    ws = torch.empty(tq.nsn_means_workspace_bytes(cache.desc, L0), dtype=torch.uint8, device="cuda")
    tq.nsn_set_means(cache.desc, codec.dev, cache.buf, Kc[:, :, :L0].contiguous(), Vc[:, :, :L0].contiguous(), 0,
                     w.rope_base, ws)
    for s0, s1 in ((0, L0), (L0, T)):
        if s1 > s0:
            tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kc[:, :, s0:s1].contiguous(),
                           Vc[:, :, s0:s1].contiguous(), s0, w.rope_base)
    torch.cuda.synchronize()
    rep = {}
    P.compare_codes(P.gpu_fields(cache, T), fields, codec_o, rep)
    ocache = tq.PackedCache(w.batch, w.kv_heads, d, T, bk, 3, d, nsn=1)
    ocache.buf.copy_(torch.from_numpy(P.oracle_image(ocache.desc.as_dict(), fields)))
    out, sc = decode(tq, codec, ocache, q.cuda(), T, w.q_pos, w.rope_base)
    out_o, sc_o = O.attend(fields, P.to_f64(q), codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                           kv_heads=w.kv_heads, length=T)
    e_out = P.max_abs(out.cpu().numpy(), out_o)
    e_sc = P.max_abs(sc.cpu().numpy()[:, :, :T], sc_o)
    out2, _ = decode(tq, codec, cache, q.cuda(), T, w.q_pos, w.rope_base, want_scores=False)
    e_e2e = P.max_abs(out2.cpu().numpy(), out_o)
    sc3 = torch.full((w.batch, w.q_heads, T), float("nan"), dtype=torch.float32, device="cuda")
    ws3 = torch.empty(tq.decode_workspace_bytes(ocache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(ocache.desc, codec.dev, ocache.buf, T, q.cuda(), w.q_pos, w.rope_base, None, scores=sc3, ws=ws3)
    torch.cuda.synchronize()
    e_lg = P.max_abs(sc3.cpu().numpy(), sc_o)
    say(f"    nsn k{bk} d{d} G{G} L0 {L0} T {T} {dist}: codes {rep} | out {e_out:.2e} scores {e_sc:.2e} "
        f"e2e {e_e2e:.2e} logits {e_lg:.2e}")
    assert e_out <= TOL and e_sc <= TOL and e_lg <= TOL
    if rep["excused"] == 0:
        assert e_e2e <= TOL


@pytest.mark.parametrize("d,dt,T", [(128, torch.float32, 333), (64, torch.float16, 260)])
def test_nsn_means_input_dtypes(tq, P, d, dt, T):
    """NSN means (and the shifted codes) from fp32 and fp16 inputs, whose element loads in
    the means kernel differ from the bf16 ones: the means over the whole cache, every code,
    norm and s1 against the oracle on the same input values."""
    w = W.LONG_CONTEXT.scaled(batch=1, kv_heads=2, q_heads=4, d=d, m=d, context=T, bits_k=2, bits_v=3)
    K, V = W.gen_kv(w)
    K, V = K.to(dt).contiguous(), V.to(dt).contiguous()
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    codec_o = O.make_codec(d, 2, 3, d, 0)
    means = P.oracle_means(Kd, Vd, np.arange(T), w.rope_base)
    fields = P.oracle_encode_unitwise(Kd, Vd, codec_o, np.arange(T), w.rope_base, means)
    codec = tq.Codec(d, 2, 3, d, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, 2, 3, d, nsn=1)
    Kc, Vc = K.cuda(), V.cuda()
    ws = torch.empty(tq.nsn_means_workspace_bytes(cache.desc, T), dtype=torch.uint8, device="cuda")
    tq.nsn_set_means(cache.desc, codec.dev, cache.buf, Kc, Vc, 0, w.rope_base, ws)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kc, Vc, 0, w.rope_base)
    torch.cuda.synchronize()
    rep = {}
    P.compare_codes(P.gpu_fields(cache, T), fields, codec_o, rep)
    say(f"    nsn means d{d} {dt}: codes {rep}")


@pytest.mark.parametrize("d,G,T,chunks,dist", [
    (128, 8, 700, [(0, 300), (300, 700)], "laplace"),   # two appends, a ragged tail
    (64, 4, 530, None, "student_t3"),
    (128, 2, 64, None, "normal"),
    (128, 5, 33, None, "normal"),                       # odd head count, one step and a token
    (64, 8, 97, [(0, 40), (40, 97)], "laplace"),        # d 64 with 8 heads, appends off the 32 grid
    (128, 1, 1, None, "normal"),                        # a single token and head
])
def test_polar_codes_and_decode(tq, P, d, G, T, chunks, dist):
    """PolarQuant caches ([TurboQuant] "PolarQuant" as stage 1, QJL on the key residual):
    every angle code, norm and QJL bit against the oracle's polar encode; decode and logits
    over the oracle's polar cache; decode end to end over the GPU's own."""
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=3, bits_v=3,
                              dist=dist)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    codec_o = O.make_codec(d, 3, 3, d, 0)
    fields = P.oracle_encode_polar(Kd, Vd, codec_o, np.arange(T), w.rope_base)
    codec = tq.Codec(d, 3, 3, d, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, 3, 3, d, polar=1)
    Kc, Vc = K.cuda(), V.cuda()
    for s0, s1 in chunks or [(0, T)]:
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kc[:, :, s0:s1].contiguous(), Vc[:, :, s0:s1].contiguous(),
                       s0, w.rope_base)
    torch.cuda.synchronize()
    rep = {}
    P.compare_polar_codes(P.gpu_fields(cache, T), fields, codec_o, rep)
    ocache = tq.PackedCache(w.batch, w.kv_heads, d, T, 3, 3, d, polar=1)
    ocache.buf.copy_(torch.from_numpy(P.oracle_image(ocache.desc.as_dict(), fields)))
    out, sc = decode(tq, codec, ocache, q.cuda(), T, w.q_pos, w.rope_base)
    out_o, sc_o = O.attend(fields, P.to_f64(q), codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                           kv_heads=w.kv_heads, length=T)
    e_out = P.max_abs(out.cpu().numpy(), out_o)
    e_sc = P.max_abs(sc.cpu().numpy()[:, :, :T], sc_o)
    out2, _ = decode(tq, codec, cache, q.cuda(), T, w.q_pos, w.rope_base, want_scores=False)
    e_e2e = P.max_abs(out2.cpu().numpy(), out_o)
    sc3 = torch.full((w.batch, w.q_heads, T), float("nan"), dtype=torch.float32, device="cuda")
    ws3 = torch.empty(tq.decode_workspace_bytes(ocache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(ocache.desc, codec.dev, ocache.buf, T, q.cuda(), w.q_pos, w.rope_base, None, scores=sc3, ws=ws3)
    torch.cuda.synchronize()
    e_lg = P.max_abs(sc3.cpu().numpy(), sc_o)
    say(f"    polar d{d} G{G} T {T} {dist}: codes {rep} | out {e_out:.2e} scores {e_sc:.2e} e2e {e_e2e:.2e} "
        f"logits {e_lg:.2e}")
    assert e_out <= TOL and e_sc <= TOL and e_lg <= TOL
    if rep["excused"] == 0:
        assert e_e2e <= TOL


@pytest.mark.parametrize("bk,bv,d,G,L0,cap,steps,dt,nsn", [
    (2, 3, 128, 4, 300, 16, 40, "bf16", 0),   # MFMA path, two flushes
    (3, 4, 64, 8, 0, 8, 20, "f32", 0),        # fp32 path, starting from an empty cache
    (2, 3, 128, 4, 200, 32, 70, "bf16", 1),   # NSN cache: flushes shifted by the prefill means
])
def test_decode_step_loop(tq, P, bk, bv, d, G, L0, cap, steps, dt, nsn):
    """A generation loop through tq_decode_step (flush of a full window, append inside the
    window kernel, attention) against the oracle's decode_step, step by step; then the
    packed cache the flushes wrote against the oracle's codes, and the window rows."""
    T = L0 + steps
    w = W.LONG_CONTEXT.scaled(batch=2, kv_heads=2, q_heads=2 * G, d=d, m=d, context=T, bits_k=bk, bits_v=bv,
                              dtype=dt)
    K, V = W.gen_kv(w)
    Kd, Vd = P.to_f64(K), P.to_f64(V)
    codec_o = O.make_codec(d, bk, bv, d, 0)
    codec = tq.Codec(d, bk, bv, d, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, bk, bv, d, nsn=nsn)
    means = P.oracle_means(Kd[:, :, :L0], Vd[:, :, :L0], np.arange(L0), w.rope_base) if nsn else None
    fields = P.oracle_encode_unitwise(Kd[:, :, :L0], Vd[:, :, :L0], codec_o, np.arange(L0), w.rope_base, means)
    if L0 > 0:
        cache.buf.copy_(torch.from_numpy(P.oracle_image(cache.desc.as_dict(), fields)))
    st = {"fields": fields, "length": L0, "win_k": np.zeros((w.batch, w.kv_heads, cap, d)),
          "win_v": np.zeros((w.batch, w.kv_heads, cap, d)), "win_len": 0}
    wk = torch.zeros((w.batch, w.kv_heads, cap, d), dtype=K.dtype, device="cuda")
    wv = torch.zeros_like(wk)
    Kc, Vc = K.cuda(), V.cuda()
    Hq = w.q_heads
    ws = torch.empty(tq.decode_window_workspace_bytes(cache.desc, Hq, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, Hq, d), dtype=torch.float32, device="cuda")
    sc = torch.empty((w.batch, Hq, T), dtype=torch.float32, device="cuda")
    L, Wn, worst = L0, 0, 0.0
    for s in range(steps):
        n = L0 + s + 1
        q = W.gen_q(w, seed=100 + s)
        nk, nv = Kc[:, :, n - 1].contiguous(), Vc[:, :, n - 1].contiguous()
        L, Wn = tq.decode_step(cache.desc, codec.dev, cache.buf, L, wk, wv, Wn, nk, nv, q.cuda(), n - 1,
                               w.rope_base, out, scores=sc, ws=ws)
        o_o, s_o = O.decode_step(st, Kd[:, :, n - 1], Vd[:, :, n - 1], P.to_f64(q), codec_o, q_pos=n - 1,
                                 rope_base=w.rope_base, scale=0.0, kv_heads=w.kv_heads)
        assert (L, Wn) == (st["length"], st["win_len"])
        torch.cuda.synchronize()
        e_out = P.max_abs(out.cpu().numpy(), o_o)
        e_sc = P.max_abs(sc.view(-1)[:w.batch * Hq * n].view(w.batch, Hq, n).cpu().numpy(), s_o)
        worst = max(worst, e_out, e_sc)
        assert e_out <= TOL and e_sc <= TOL, (s, e_out, e_sc)
    rep = {}
    P.compare_codes(P.gpu_fields(cache, L), P.oracle_encode_unitwise(Kd[:, :, :L], Vd[:, :, :L], codec_o,
                                                                    np.arange(L), w.rope_base, means), codec_o, rep)
    assert torch.equal(wk[:, :, :Wn].cpu(), K[:, :, L:L + Wn]) and torch.equal(wv[:, :, :Wn].cpu(), V[:, :, L:L + Wn])
    say(f"    step loop k{bk} v{bv} d{d} G{G} L0 {L0} cap {cap} nsn {nsn}: {steps} steps, final ({L}, {Wn}), "
        f"worst {worst:.2e}, codes {rep}")


@pytest.mark.parametrize("bk,bv,m", [(1, 2, 64), (3, 4, 128), (4, 1, 32), (2, 3, 0), (2, 3, 96), (2, 3, 256)])
def test_other_bit_widths(tq, P, bk, bv, m):
    w = W.LLAMA3_8B.scaled(batch=1, kv_heads=2, q_heads=4, context=300, bits_k=bk, bits_v=bv, m=m)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    check_case(tq, P, w, K, V, q, label=f"bits k{bk} v{bv} m{m}")


def test_split_counts_and_determinism(tq, P):
    w = W.LLAMA3_8B.scaled(batch=1, kv_heads=2, q_heads=8, context=1500)
    K, V = W.gen_kv(w)
    q = W.gen_q(w)
    codec, cache = build(tq, w, K.cuda(), V.cuda())
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    fields, out_o, _ = oracle_side(P, w, K, V, q, 1500, codec_o)
    outs = []
    for s in (1, 3, 7, 0):
        out, _ = decode(tq, codec, cache, q.cuda(), 1500, w.q_pos, w.rope_base, splits=s)
        outs.append(out.cpu().numpy())
        assert P.max_abs(outs[-1], out_o) <= TOL
    out_again, _ = decode(tq, codec, cache, q.cuda(), 1500, w.q_pos, w.rope_base, splits=0)
    assert np.array_equal(out_again.cpu().numpy(), outs[-1])
    # quantize is deterministic too
    _, cache2 = build(tq, w, K.cuda(), V.cuda())
    assert torch.equal(cache.buf, cache2.buf)


def test_edge_cases_zero_overflow_empty(tq, P):
    w = W.LLAMA3_8B.scaled(batch=1, kv_heads=1, q_heads=2, context=64)
    K, V = W.gen_kv(w)
    K = K.float()
    V = V.float()
    K[0, 0, 5] = 0.0
    V[0, 0, 6] = 0.0
    K[0, 0, 9] = 3.0e4          # norm far beyond fp16 range
    w32 = w.scaled(dtype="f32")
    q = W.gen_q(w32)
    codec, cache = build(tq, w32, K.cuda(), V.cuda())
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    fields = P.oracle_encode_unitwise(P.to_f64(K), P.to_f64(V), codec_o, np.arange(64), w.rope_base)
    g = P.gpu_fields(cache, 64)
    P.compare_codes(g, fields, codec_o)
    assert g["flags"] & 1, "fp16 norm saturation must set the header flag"
    assert g["n16"][0, 0, 9] == 65504.0
    assert np.all(g["bits"][0, 0, 5] == 1) and g["n16"][0, 0, 5] == 0 and g["rn16"][0, 0, 5] == 0
    # n_new = 0 is a no-op; length = 0 gives zeros
    before = cache.buf.clone()
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, :0].cuda(), V[:, :, :0].cuda(), 3, w.rope_base)
    torch.cuda.synchronize()
    assert torch.equal(before, cache.buf)
    out, _ = decode(tq, codec, cache, q.cuda(), 0, 0, w.rope_base, want_scores=False)
    assert torch.all(out == 0)
    # a single cached token: out = Pi^T (n_v c_v[code]) of that token (oracle)
    out1, _ = decode(tq, codec, cache, q.cuda(), 1, 1, w.rope_base)
    o1, _ = O.attend(fields, P.to_f64(q), codec_o, q_pos=1, rope_base=w.rope_base, scale=0.0,
                     kv_heads=1, length=1)
    assert P.max_abs(out1.cpu().numpy(), o1) <= TOL
    # cache_init clears the flag
    tq.cache_init(cache.desc, cache.buf)
    torch.cuda.synchronize()
    assert P.gpu_fields(cache, 0)["flags"] == 0


def test_esm2_all_layers(tq, P):
    """ESM-2-650M-shaped: 33 layers x 20 heads x d 64, 1024 tokens, bf16 Student-t, RoPE."""
    w = W.ESM2_650M
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    tot = {"codes": 0, "excused": 0, "dependent": 0}
    worst = worst_e2e = 0.0
    for layer in range(w.layers):
        K, V = W.gen_kv(w, layer)
        q = W.gen_q(w, layer)
        codec, cache = build(tq, w, K.cuda(), V.cuda())
        fields, out_e2e, _ = oracle_side(P, w, K, V, q, w.context, codec_o)
        gf = P.gpu_fields(cache, w.context)
        rep = P.compare_codes(gf, fields, codec_o)
        for kk in tot:
            tot[kk] += rep[kk]
        out, _ = decode(tq, codec, cache, q.cuda(), w.context, w.q_pos, w.rope_base, want_scores=False)
        out = out.cpu().numpy()
        # the oracle attending over the same (GPU-produced) packed cache
        out_o, _ = O.attend(gf, P.to_f64(q), codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                            kv_heads=w.kv_heads, length=w.context)
        worst = max(worst, P.max_abs(out, out_o))
        # end to end (the oracle's own encode) only where no code was excused: an excused
        # code changes its token's score by a whole code step
        if rep["excused"] == 0:
            worst_e2e = max(worst_e2e, P.max_abs(out, out_e2e))
    say(f"[esm2] codes {tot} worst out {worst:.2e} worst e2e (layers without excused codes) {worst_e2e:.2e}")
    assert tot["excused"] <= 1e-6 * tot["codes"]
    assert worst <= TOL and worst_e2e <= TOL


# ------------------------------------------------------------------ search
def test_search_small(tq, P):
    w = W.VECTOR_SEARCH.scaled(n_db=3000, nq=16)
    db, qs = W.gen_search(w)
    codec = tq.Codec(w.d, w.bits, 0, w.m, seed=0)
    cache = tq.PackedCache(1, 1, w.d, w.n_db, w.bits, 0, w.m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, db.cuda()[None, None], None, 0, 0.0)
    codec_o = O.make_codec(w.d, w.bits, 0, w.m, 0)
    enc = O.encode(db.double().numpy(), codec_o, kind="db")
    g = O.unpack_cache(cache.buf.cpu().numpy(), cache.desc.as_dict(), w.n_db)
    orc = {"kcodes": enc["codes"][None, None], "n16": enc["n16"][None, None], "rn16": enc["rn16"][None, None],
           "bits": enc["bits"][None, None], "ku": enc["u"][None, None], "kn": enc["n"][None, None],
           "krn": enc["rn"][None, None], "kz": enc["z"][None, None]}
    rep = P.compare_codes(g, orc, codec_o)
    say(f"[search db] {rep}")
    # search over the oracle's packed database
    fields = {"kcodes": enc["codes"], "n16": enc["n16"], "rn16": enc["rn16"], "bits": enc["bits"]}
    img = O.pack_cache(cache.desc.as_dict(), {k: v[None, None] for k, v in fields.items()})
    ocache = tq.PackedCache(1, 1, w.d, w.n_db, w.bits, 0, w.m)
    ocache.buf.copy_(torch.from_numpy(img))
    s_o = O.search_scores(fields, qs.double().numpy(), codec_o)
    idx_o, val_o = O.topk(s_o, w.k)
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device="cuda")
    val = torch.empty((w.nq, w.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.search_workspace_bytes(ocache.desc, w.n_db, w.nq, w.k), dtype=torch.uint8, device="cuda")
    tq.search_topk(ocache.desc, codec.dev, ocache.buf, w.n_db, qs.cuda(), w.k, idx, val, ws)
    torch.cuda.synchronize()
    check_topk(idx.cpu().numpy(), val.cpu().numpy(), s_o, idx_o, val_o)


@pytest.mark.parametrize("d,bits,m", [(256, 3, 256), (512, 2, 512), (1024, 3, 512), (1536, 3, 1536), (2048, 1, 2048)])
def test_db_codes_widths(tq, P, d, bits, m):
    """Database vectors at every width the wide-vector encoder serves (one wave per vector;
    S r on fp16 MFMA in groups of 24 up to d = 1536, on fp32 MFMA in groups of 16 at
    2048): every code, norm, QJL bit and residual norm against the oracle's encode under
    the boundary rule; 40 vectors, so the last group is ragged."""
    w = W.VECTOR_SEARCH.scaled(n_db=40, nq=1, d=d, bits=bits, m=m)
    db, _ = W.gen_search(w)
    codec = tq.Codec(d, bits, 0, m, seed=3)
    cache = tq.PackedCache(1, 1, d, w.n_db, bits, 0, m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, db.cuda()[None, None], None, 0, 0.0)
    torch.cuda.synchronize()
    codec_o = O.make_codec(d, bits, 0, m, 3)
    enc = O.encode(db.double().numpy(), codec_o, kind="db")
    g = O.unpack_cache(cache.buf.cpu().numpy(), cache.desc.as_dict(), w.n_db)
    orc = {"kcodes": enc["codes"][None, None], "n16": enc["n16"][None, None], "rn16": enc["rn16"][None, None],
           "bits": enc["bits"][None, None], "ku": enc["u"][None, None], "kn": enc["n"][None, None],
           "krn": enc["rn"][None, None], "kz": enc["z"][None, None]}
    rep = P.compare_codes(g, orc, codec_o)
    say(f"[db d={d} bits={bits} m={m}] {rep}")


def check_topk(idx, val, s_o, idx_o, val_o, tie=1e-6, stol=1e-4):
    """Top-k identical except swaps among entries whose oracle scores differ by <= tie."""
    nq, k = idx.shape
    for i in range(nq):
        # returned scores agree with the oracle's score of the returned index
        np.testing.assert_allclose(val[i], s_o[i, idx[i]], atol=stol)
        if np.array_equal(idx[i], idx_o[i]):
            continue
        kth = val_o[i, -1]
        for r in range(k):
            if idx[i, r] != idx_o[i, r]:
                # the two entries at this rank must be near-tied in the oracle's scores
                assert abs(s_o[i, idx[i, r]] - val_o[i, r]) <= tie, (i, r)
        # any index outside the oracle's list must tie with its k-th score
        for j in set(idx[i]) - set(idx_o[i]):
            assert abs(s_o[i, j] - kth) <= tie
