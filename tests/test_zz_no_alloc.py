"""tq_decode_attend_noalloc: the decode with the library's own device scratch, called
through the C ABI and checked against tq_decode_attend on the same inputs.

Outputs must be bitwise equal (same kernels, same split count), on two calls in a row
whose second has a smaller shape, so the scratch still holds the first call's contents."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from vector_quantization_rope_amd import workloads as W


@pytest.fixture(scope="module")
def tq():
    from vector_quantization_rope_amd import tq as _tq
    return _tq


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(tq, batch, kv_heads, G, T, bits_k, dtype, seed, polar=0):
    w = W.LONG_CONTEXT.scaled(batch=batch, kv_heads=kv_heads, q_heads=G * kv_heads, context=T, bits_k=bits_k,
                              dtype=dtype, **({"bits_v": 3, "m": 128} if polar else {}))
    K, V = W.gen_kv(w, device="cuda")
    q = W.gen_q(w, device="cuda")
    codec = tq.Codec(w.d, bits_k, w.bits_v, w.m, seed=seed)
    cache = tq.PackedCache(batch, kv_heads, w.d, T, bits_k, w.bits_v, w.m, polar=polar)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K.contiguous(), V.contiguous(), 0, w.rope_base)
    return w, q, codec, cache


@pytest.mark.gpu
def test_noalloc_decode_equals_decode_attend(tq):
    # (batch, kv_heads, G, context, key bits, dtype, polar): the MFMA path at two shapes, the
    # second smaller, then the fp32 path (16 q-heads per kv-head) smaller still, then a
    # PolarQuant cache (its own decode kernel; logits on the same kernel)
    cases = [(2, 4, 8, 5000, 2, "bf16", 0), (1, 2, 4, 700, 2, "bf16", 0), (1, 1, 16, 300, 3, "f32", 0),
             (1, 2, 8, 260, 3, "bf16", 1)]
    for i, (B, H, G, T, bk, dt, pol) in enumerate(cases):
        say(f"[noalloc] case {i}: batch {B} kv_heads {H} G {G} context {T} keys {bk}-bit {dt} polar {pol}")
        w, q, codec, cache = _case(tq, B, H, G, T, bk, dt, seed=i, polar=pol)
        Hq = G * H
        assert tq.decode_workspace_bytes(cache.desc, Hq, T) <= tq.NOALLOC_SCRATCH_BYTES
        out_ref = torch.empty((B, Hq, w.d), dtype=torch.float32, device="cuda")
        sc_ref = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
        ws = torch.empty(tq.decode_workspace_bytes(cache.desc, Hq, T), dtype=torch.uint8, device="cuda")
        tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out_ref, scores=sc_ref, ws=ws)
        out = torch.full_like(out_ref, float("nan"))
        sc = torch.full_like(sc_ref, float("nan"))
        tq.decode_attend_noalloc(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, scores=sc)
        # logits only (its own kernel on the MFMA path) against tq_decode_attend's logits only
        lg_ref = torch.empty_like(sc_ref)
        tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, None, scores=lg_ref, ws=ws)
        lg = torch.full_like(sc_ref, float("nan"))
        tq.decode_attend_noalloc(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, None, scores=lg)
        torch.cuda.synchronize()
        assert torch.isfinite(out_ref).all() and torch.isfinite(lg_ref).all()
        assert torch.equal(out, out_ref), float((out - out_ref).abs().max())
        assert torch.equal(sc, sc_ref), float((sc - sc_ref).abs().max())
        assert torch.equal(lg, lg_ref), float((lg - lg_ref).abs().max())
        say(f"[noalloc] case {i}: outputs and scores bitwise equal to tq_decode_attend")


def test_noalloc_rejects_shapes_beyond_the_scratch(tq):
    # host-side: a workspace above TQ_NOALLOC_SCRATCH_BYTES is TQ_ENOSPACE before any device
    # call (the fake pointers are never used), and malformed calls get the usual statuses
    P = 0x1000
    big = tq.CacheDesc(64, 64, 128, 4096, 2, 3, 128)
    assert tq.decode_workspace_bytes(big, 64 * 8, 4096) > tq.NOALLOC_SCRATCH_BYTES
    assert tq._decode_attend_noalloc(ctypes.byref(big), P, P, 4096, P, 1, 64 * 8, 0, 0.0, 0.0, P, None,
                                     None) == tq.TQ_ENOSPACE
    bad = tq.CacheDesc(1, 1, 100, 64, 2, 3, 128)
    assert tq._decode_attend_noalloc(ctypes.byref(bad), P, P, 10, P, 1, 1, 0, 0.0, 0.0, P, None,
                                     None) == tq.TQ_EUNSUPPORTED
    good = tq.CacheDesc(1, 1, 128, 64, 2, 3, 128)
    assert tq._decode_attend_noalloc(ctypes.byref(good), P, P, 10, P, 1, 0, 0, 0.0, 0.0, P, None,
                                     None) == tq.TQ_EINVAL
    assert tq._decode_attend_noalloc(None, P, P, 10, P, 1, 1, 0, 0.0, 0.0, P, None, None) == tq.TQ_EINVAL
