"""GPU parity at full workload sizes, on sampled outputs the oracle computes one by one.

  * long context (1 layer, 64 q-heads / 8 kv-heads, d 128, batch 4, 131072 tokens): the
    cache is built exactly as bench.py builds it (prefill [0, 126976), append of the last
    4096 positions as a separate call) and decoded with the library's default split count,
    without the scores output, as bench.py times it.  For sampled (batch, kv-head) units,
    every code, bit and norm of all 131072 tokens is compared with the oracle's encode, and
    the unit's 8 q-head outputs with the oracle attending over the GPU-produced cache.
  * Llama-3-8B-shaped layer (batch 16, 32 q / 8 kv heads, 32768 tokens): the same checks
    on sampled units of one layer.
  * the same long-context shape as an NSN cache (means over the prefill), as a PolarQuant
    cache, and with its last 128 tokens as a full-precision window, as bench.py's sections
    build them: a sampled unit's codes and outputs against the oracle.
  * vector search (10^6 x 1536 database, 1024 queries, 3-bit + QJL m = 1536, top-10):
    codes of sampled database vectors; the returned scores of sampled queries against the
    oracle's estimate of the returned vectors; and, for two queries, the complete top-10
    against the oracle's scores of all 10^6 packed vectors.
"""
from __future__ import annotations

import sys
import time

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


def unit_oracle(P, w, K, V, b, g, codec_o):
    Kd = K[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    Vd = V[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    T = Kd.shape[2]
    return P.oracle_encode_unitwise(Kd, Vd, codec_o, np.arange(T), w.rope_base)


def check_units(tq, P, w, K, V, q, cache, out, units, label):
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    G = w.q_heads // w.kv_heads
    T = w.context
    for (b, g) in units:
        t0 = time.time()
        unit = b * w.kv_heads + g
        gf = P.unit_fields(cache, unit, T)
        assert gf["flags"] == 0
        orc = unit_oracle(P, w, K, V, b, g, codec_o)
        rep = P.compare_codes(gf, orc, codec_o)
        qd = q[b:b + 1, g * G:(g + 1) * G].to("cpu").to(torch.float64).numpy()
        out_o, _ = O.attend(gf, qd, codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                            kv_heads=1, length=T)
        err = P.max_abs(out[b, g * G:(g + 1) * G].cpu().numpy(), out_o[0])
        say(f"[{label}] unit (b={b}, kv={g}) codes {rep} out max-abs {err:.2e} ({time.time() - t0:.1f} s)")
        assert err <= TOL


def test_long_context_full_size_bench_config(tq, P):
    w = W.LONG_CONTEXT
    T, A = w.context, w.append
    pre = T - A
    say(f"[long_context] B={w.batch} Hkv={w.kv_heads} Hq={w.q_heads} T={T} append={A}")
    K, V = W.gen_kv(w, device="cuda")
    q = W.gen_q(w, device="cuda")
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous(),
                   0, w.rope_base)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous(),
                   pre, w.rope_base)
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=ws)
    torch.cuda.synchronize()
    say(f"    decode splits {tq.decode_splits(cache.desc, w.q_heads, T)}")
    assert torch.isfinite(out).all()
    check_units(tq, P, w, K, V, q, cache, out, [(0, 0), (3, 5)], "long_context")


def _long_context_inputs(tq, w):
    K, V = W.gen_kv(w, device="cuda")
    q = W.gen_q(w, device="cuda")
    return K, V, q


def test_long_context_nsn_full_size(tq, P):
    """NSN cache at the long-context shape, built as bench.py's NSN section builds it
    (means over the 126976-token prefill, prefill, 4096-token append) and decoded with the
    default split count; a sampled unit's means, codes, s1 and outputs against the oracle."""
    w = W.LONG_CONTEXT
    T, A = w.context, w.append
    pre = T - A
    K, V, q = _long_context_inputs(tq, w)
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m, nsn=1)
    Kp, Vp = K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous()
    ws = torch.empty(tq.nsn_means_workspace_bytes(cache.desc, pre), dtype=torch.uint8, device="cuda")
    tq.nsn_set_means(cache.desc, codec.dev, cache.buf, Kp, Vp, 0, w.rope_base, ws)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kp, Vp, 0, w.rope_base)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous(),
                   pre, w.rope_base)
    del Kp, Vp
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device="cuda")
    wsd = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=wsd)
    torch.cuda.synchronize()
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    G = w.q_heads // w.kv_heads
    b, g = 2, 3
    t0 = time.time()
    gf = P.unit_fields(cache, b * w.kv_heads + g, T)
    Kd = K[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    Vd = V[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    means = P.oracle_means(Kd[:, :, :pre], Vd[:, :, :pre], np.arange(pre), w.rope_base)
    orc = P.oracle_encode_unitwise(Kd, Vd, codec_o, np.arange(T), w.rope_base, means)
    rep = P.compare_codes(gf, orc, codec_o)
    qd = q[b:b + 1, g * G:(g + 1) * G].to("cpu").to(torch.float64).numpy()
    out_o, _ = O.attend(gf, qd, codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0, kv_heads=1, length=T)
    err = P.max_abs(out[b, g * G:(g + 1) * G].cpu().numpy(), out_o[0])
    say(f"[long_context nsn] unit (b={b}, kv={g}) codes {rep} out max-abs {err:.2e} ({time.time() - t0:.1f} s)")
    assert err <= TOL


def test_long_context_polar_full_size(tq, P):
    """PolarQuant cache at the long-context shape (prefill, 4096-token append, default
    split count, as bench.py's PolarQuant section): a sampled unit's angle codes, norms,
    QJL bits and outputs against the oracle."""
    w = W.LONG_CONTEXT
    T, A = w.context, w.append
    pre = T - A
    K, V, q = _long_context_inputs(tq, w)
    d = w.d
    codec = tq.Codec(d, 3, 3, d, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, 3, 3, d, polar=1)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous(), 0,
                   w.rope_base)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous(),
                   pre, w.rope_base)
    out = torch.empty((w.batch, w.q_heads, d), dtype=torch.float32, device="cuda")
    wsd = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=wsd)
    torch.cuda.synchronize()
    codec_o = O.make_codec(d, 3, 3, d, 0)
    G = w.q_heads // w.kv_heads
    b, g = 1, 6
    t0 = time.time()
    gf = P.unit_fields(cache, b * w.kv_heads + g, T)
    Kd = K[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    Vd = V[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    orc = P.oracle_encode_polar(Kd, Vd, codec_o, np.arange(T), w.rope_base)
    rep = P.compare_polar_codes(gf, orc, codec_o)
    qd = q[b:b + 1, g * G:(g + 1) * G].to("cpu").to(torch.float64).numpy()
    out_o, _ = O.attend(gf, qd, codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0, kv_heads=1, length=T)
    err = P.max_abs(out[b, g * G:(g + 1) * G].cpu().numpy(), out_o[0])
    say(f"[long_context polar] unit (b={b}, kv={g}) codes {rep} out max-abs {err:.2e} ({time.time() - t0:.1f} s)")
    assert err <= TOL


def test_long_context_window_full_size(tq, P):
    """The long-context cache with its last 128 tokens as a full-precision window (bench.py's
    window section: 130944 packed tokens + 128 raw ones): a sampled unit's outputs against
    the oracle attending over the GPU-produced packed part and the raw window."""
    w = W.LONG_CONTEXT
    T, cap = w.context, 128
    L = T - cap
    K, V, q = _long_context_inputs(tq, w)
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, :L].contiguous(), V[:, :, :L].contiguous(), 0,
                   w.rope_base)
    wk, wv = K[:, :, L:].contiguous(), V[:, :, L:].contiguous()
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.decode_window_workspace_bytes(cache.desc, w.q_heads, L), dtype=torch.uint8, device="cuda")
    tq.decode_attend_window(cache.desc, codec.dev, cache.buf, L, wk, wv, cap, q, w.q_pos, w.rope_base, out, ws=ws)
    torch.cuda.synchronize()
    codec_o = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    G = w.q_heads // w.kv_heads
    b, g = 3, 1
    t0 = time.time()
    gf = P.unit_fields(cache, b * w.kv_heads + g, L)
    qd = q[b:b + 1, g * G:(g + 1) * G].to("cpu").to(torch.float64).numpy()
    wkd = wk[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    wvd = wv[b:b + 1, g:g + 1].to("cpu").to(torch.float64).numpy()
    out_o, _ = O.attend_window(gf, wkd, wvd, qd, codec_o, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0,
                               kv_heads=1, length=L, win_len=cap)
    err = P.max_abs(out[b, g * G:(g + 1) * G].cpu().numpy(), out_o[0])
    say(f"[long_context window] unit (b={b}, kv={g}) out max-abs {err:.2e} ({time.time() - t0:.1f} s)")
    assert err <= TOL


def test_llama3_8b_layer_sampled_units(tq, P):
    w = W.LLAMA3_8B
    T = w.context
    say(f"[llama3_8b] layer 0: B={w.batch} Hkv={w.kv_heads} Hq={w.q_heads} T={T}")
    K, V = W.gen_kv(w, 0, device="cuda")
    q = W.gen_q(w, 0, device="cuda")
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K, V, 0, w.rope_base)
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device="cuda")
    tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_units(tq, P, w, K, V, q, cache, out, [(0, 0), (11, 6)], "llama3_8b")


def _db_rows_fields(kbits_cpu, knorm_cpu, desc, rows):
    """Oracle-unpacked fields of the database vectors `rows` (indices or a slice), read
    from copies of the two key regions."""
    kb = (desc["bits_k"] * desc["d"] + desc["m"]) // 8
    recs = kbits_cpu.reshape(-1, kb)[rows]
    norms = knorm_cpu.reshape(-1, 4)[rows]
    n = recs.shape[0]
    sub = dict(desc, capacity=n)
    sl = O.cache_layout(1, 1, sub["d"], n, sub["bits_k"], 0, sub["m"])
    img = np.zeros(sl["total"], dtype=np.uint8)
    img[sl["kbits"]: sl["kbits"] + n * kb] = recs.reshape(-1)
    img[sl["knorm"]: sl["knorm"] + n * 4] = norms.reshape(-1)
    f = O.unpack_cache(img, sub, n)
    return {k: f[k][0, 0] for k in ("kcodes", "n16", "rn16", "bits")}


def test_vector_search_full_size(tq, P):
    from test_gpu_parity import check_topk

    w = W.VECTOR_SEARCH
    say(f"[search] n_db={w.n_db} d={w.d} nq={w.nq} bits={w.bits} m={w.m} k={w.k}")
    db, qs = W.gen_search(w, device="cuda")
    codec = tq.Codec(w.d, w.bits, 0, w.m, seed=0)
    cache = tq.PackedCache(1, 1, w.d, w.n_db, w.bits, 0, w.m)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, db[None, None], None, 0, 0.0)
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device="cuda")
    val = torch.empty((w.nq, w.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.search_workspace_bytes(cache.desc, w.n_db, w.nq, w.k), dtype=torch.uint8, device="cuda")
    tq.search_topk(cache.desc, codec.dev, cache.buf, w.n_db, qs, w.k, idx, val, ws)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    desc = cache.desc.as_dict()
    lay = O.cache_layout(1, 1, w.d, w.n_db, w.bits, 0, w.m)
    kb = lay["kbytes"]
    kbits = cache.buf[lay["kbits"]: lay["kbits"] + w.n_db * kb].cpu().numpy()
    knorm = cache.buf[lay["knorm"]: lay["knorm"] + w.n_db * 4].cpu().numpy()
    assert int(cache.buf[8:12].cpu().numpy().view(np.uint32)[0]) == 0
    codec_o = O.make_codec(w.d, w.bits, 0, w.m, 0)

    # codes of sampled database vectors
    rng = np.random.default_rng(7)
    samp = np.sort(rng.choice(w.n_db, 4096, replace=False))
    x = db[torch.from_numpy(samp).cuda()].double().cpu().numpy()
    enc = O.encode(x, codec_o, kind="db")
    gpu = {k: v[None, None] for k, v in _db_rows_fields(kbits, knorm, desc, samp).items()}
    orc = {"kcodes": enc["codes"][None, None], "n16": enc["n16"][None, None], "rn16": enc["rn16"][None, None],
           "bits": enc["bits"][None, None], "ku": enc["u"][None, None], "kn": enc["n"][None, None],
           "krn": enc["rn"][None, None], "kz": enc["z"][None, None]}
    rep = P.compare_codes(gpu, orc, codec_o)
    say(f"    sampled database codes {rep}")

    # returned scores of sampled queries against the oracle's estimate of those vectors
    qsel = rng.choice(w.nq, 16, replace=False)
    for i in qsel:
        f = _db_rows_fields(kbits, knorm, desc, idx[i].astype(np.int64))
        s = O.search_scores(f, qs[i:i + 1].double().cpu().numpy(), codec_o)[0]
        assert np.all(np.diff(val[i]) <= 0)
        assert len(set(idx[i].tolist())) == w.k
        np.testing.assert_allclose(val[i], s, atol=1e-6)

    # complete top-10 of 64 queries (the 16 above and 48 more) over all 10^6 packed vectors
    rest = np.setdiff1d(np.arange(w.nq), qsel)
    q64 = np.concatenate([qsel, rng.choice(rest, 48, replace=False)]).astype(np.int64)
    qd = qs[torch.from_numpy(q64).cuda()].double().cpu().numpy()
    scores = np.empty((len(q64), w.n_db))
    t0 = time.time()
    step = 4096
    for i0 in range(0, w.n_db, step):
        i1 = min(w.n_db, i0 + step)
        scores[:, i0:i1] = O.search_scores(_db_rows_fields(kbits, knorm, desc, slice(i0, i1)), qd, codec_o)
        if i0 % (step * 64) == 0:
            say(f"    oracle scoring: {i1} of {w.n_db} vectors, {time.time() - t0:.1f} s")
    idx_o, val_o = O.topk(scores, w.k)
    say(f"    oracle scored {len(q64)} queries x {w.n_db} vectors in {time.time() - t0:.1f} s")
    check_topk(idx[q64], val[q64], scores, idx_o, val_o, stol=1e-6)
