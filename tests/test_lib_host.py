"""Host-side checks of libtq that need no GPU: the library loads and exports every
declared symbol, the host codec tables equal the oracle's, buffer sizes follow the
format, and argument errors come back as status codes with nothing enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    from vector_quantization_rope_amd import tq as _tq
    return _tq


def test_header_declarations_are_all_exported(tq):
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    names = set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", hdr))
    assert names, "no declarations parsed"
    lib = ctypes.CDLL(tq.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in tq.h but not exported"
    assert names == set(tq.EXPORTS)
    assert "format 1" in tq.version()


@pytest.mark.parametrize("d,bits", [(8, 1), (8, 2), (64, 2), (64, 3), (128, 2), (128, 3), (1536, 3)])
def test_codebook_matches_oracle(tq, O, d, bits):
    c64, t64 = tq.make_codebook_f64(d, bits)
    cb = O.make_codebook(d, bits)
    # both iterations stop at a 1e-13 step; the fixed point is reached to ~1e-11 (sqrt(d) units)
    np.testing.assert_allclose(c64, cb.c64, rtol=0, atol=1e-11 / np.sqrt(d))
    c, t = tq.make_codebook(d, bits)
    np.testing.assert_array_equal(c.astype(np.float64), cb.c)
    np.testing.assert_array_equal(t.astype(np.float64), cb.t)


@pytest.mark.parametrize("d,m,seed", [(64, 64, 0), (128, 128, 0), (128, 96, 12345), (1536, 1536, 0)])
def test_codec_tables_match_oracle(tq, O, d, m, seed):
    desc = tq.CodecDesc(d, 3 if d == 1536 else 2, 0 if d == 1536 else 3, m, seed)
    blob = tq.codec_build(desc)
    hdr = blob[:256].view(np.uint32)
    assert hdr[0] == 0x44435154 and hdr[1] == 1
    # section offsets as laid out by the library (header, 4 x 16 floats, D, S, S^T, ...)
    off_d = 256 + 256
    D = blob[off_d:off_d + 4 * d].view(np.float32)
    np.testing.assert_array_equal(D.astype(np.float64), O.rotation_signs(d, seed))
    off_s = off_d + ((4 * d + 255) // 256) * 256
    S = blob[off_s:off_s + 4 * m * d].view(np.float32).reshape(m, d)
    So = O.gaussian_projection(m, d, seed)
    mism = np.count_nonzero(S != So)
    if d <= 128:
        assert mism == 0
    else:
        # independent libm implementations may differ in the last fp64 bit, which can
        # flip an fp32 rounding; allow a handful of 1-ulp differences
        assert mism <= 8
        if mism:
            diff = np.abs(S.view(np.int32).astype(np.int64) - So.view(np.int32).astype(np.int64))
            assert diff.max() <= 1
    off_st = off_s + ((4 * m * d + 255) // 256) * 256
    ST = blob[off_st:off_st + 4 * m * d].view(np.float32).reshape(d, m)
    np.testing.assert_array_equal(ST, S.T)
    # three fp16 parts after S^T, each the nearest fp16 of what is left: their sum is S
    # exactly where |S| >= 1/2 (the last remainder is a multiple of the fp16 subnormal
    # step 2^-24) and within half that step elsewhere
    off_b = off_st + ((4 * m * d + 255) // 256) * 256
    step = ((2 * m * d + 255) // 256) * 256
    parts = [blob[off_b + i * step: off_b + i * step + 2 * m * d].view(np.float16).reshape(m, d)
             .astype(np.float64) for i in range(3)]
    S64 = S.astype(np.float64)
    rest = S64.copy()
    for p in parts:
        np.testing.assert_array_equal(p, rest.astype(np.float16).astype(np.float64))
        rest = rest - p
    total = parts[0] + parts[1] + parts[2]
    big = np.abs(S64) >= 0.5
    np.testing.assert_array_equal(total[big], S64[big])
    assert np.all(np.abs(total - S64) <= 2.0 ** -25)


def test_cache_layout_matches_oracle(tq, O):
    for args in [(1, 1, 128, 1024, 2, 3, 128), (3, 5, 64, 100, 2, 3, 64), (1, 1, 1536, 1000, 3, 0, 1536),
                 (2, 2, 128, 33, 4, 1, 32)]:
        desc = tq.CacheDesc(*args)
        assert tq.cache_bytes(desc) == O.cache_layout(*args)["total"]
    # NSN caches: wider norm records and the per-unit means region
    for args in [(1, 1, 128, 1024, 2, 3, 128), (3, 5, 64, 100, 3, 4, 64), (2, 2, 128, 33, 1, 3, 128)]:
        assert tq.cache_bytes(tq.CacheDesc(*args, 1)) == O.cache_layout(*args, 1)["total"]
    # PolarQuant caches: the same region sizes as 3-bit keys and values (token records)
    for args in [(1, 1, 128, 1024, 3, 3, 128), (3, 5, 64, 100, 3, 3, 64), (2, 2, 128, 33, 3, 0, 64)]:
        assert tq.cache_bytes(tq.CacheDesc(*args, 0, 1)) == O.cache_layout(*args, 0, 1)["total"]
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 128, 64, 2, 3, 128, 0, 1)) == 0    # bits must be 3
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 128, 64, 3, 3, 128, 1, 1)) == 0    # not with NSN
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 256, 64, 3, 0, 256, 0, 1)) == 0    # d = 64 or 128
    # NSN needs values and d = 64 or 128
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 128, 64, 2, 0, 128, 1)) == 0
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 256, 64, 2, 3, 256, 1)) == 0
    assert tq.cache_bytes(tq.CacheDesc(1, 1, 128, 64, 2, 3, 128, 2)) == 0
    assert tq.nsn_means_workspace_bytes(tq.CacheDesc(2, 4, 128, 64, 2, 3, 128, 1), 5000) > 0
    assert tq.nsn_means_workspace_bytes(tq.CacheDesc(2, 4, 128, 64, 2, 3, 128), 5000) == 0


def test_argument_errors_return_status(tq):
    good = tq.CacheDesc(1, 1, 128, 64, 2, 3, 128)
    bad_d = tq.CacheDesc(1, 1, 100, 64, 2, 3, 128)
    assert tq.cache_bytes(bad_d) == 0
    assert tq.codec_bytes(tq.CodecDesc(128, 5, 3, 128, 0)) == 0
    assert tq.codec_bytes(tq.CodecDesc(128, 2, 3, 100, 0)) == 0
    with pytest.raises(tq.TQError) as e:
        tq.make_codebook(4, 2)
    assert e.value.status == tq.TQ_EUNSUPPORTED
    # device entry points: every check runs before anything is enqueued (no GPU needed)
    P = 0x1000  # never dereferenced: each call fails validation first
    nsn = tq.CacheDesc(1, 1, 128, 64, 2, 3, 128, 1)
    cases = [
        (lambda: tq._quantize_kv(ctypes.byref(good), None, P, P, P, 0, 0, 1, 0.0, None), tq.TQ_EINVAL),
        (lambda: tq._quantize_kv(ctypes.byref(good), P, P, P, P, 0, 60, 5, 0.0, None), tq.TQ_ECAPACITY),
        (lambda: tq._quantize_kv(ctypes.byref(good), P, P, P, None, 0, 0, 1, 0.0, None), tq.TQ_EINVAL),
        (lambda: tq._quantize_kv(ctypes.byref(good), P, P, P, P, 7, 0, 1, 0.0, None), tq.TQ_EINVAL),
        (lambda: tq._quantize_kv(ctypes.byref(good), P, P, P, P, 0, -1, 1, 0.0, None), tq.TQ_EINVAL),
        (lambda: tq._quantize_kv(ctypes.byref(bad_d), P, P, P, P, 0, 0, 1, 0.0, None), tq.TQ_EUNSUPPORTED),
        (lambda: tq._decode_attend_splits(ctypes.byref(good), P, P, 65, P, 0, 1, 0, 0.0, 0.0, P, None, 0, P,
                                          1 << 30, None), tq.TQ_ECAPACITY),
        (lambda: tq._decode_attend_splits(ctypes.byref(tq.CacheDesc(1, 2, 128, 64, 2, 3, 128)), P, P, 10, P,
                                          0, 3, 0, 0.0, 0.0, P, None, 0, P, 1 << 30, None), tq.TQ_EINVAL),
        (lambda: tq._decode_attend_splits(ctypes.byref(good), P, P, 10, P, 0, 1, 0, 0.0, 0.0, P, None, 0, P,
                                          16, None), tq.TQ_ENOSPACE),
        (lambda: tq._decode_attend_splits(ctypes.byref(good), P, P, 10, P, 0, 32, 0, 0.0, 0.0, P, None, 0, P,
                                          1 << 30, None), tq.TQ_EUNSUPPORTED),
        (lambda: tq._decode_attend_splits(ctypes.byref(good), P, P, 10, None, 0, 1, 0, 0.0, 0.0, P, None, 0,
                                          P, 1 << 30, None), tq.TQ_EINVAL),
        (lambda: tq._search_topk(ctypes.byref(good), P, P, 10, P, 4, 10, P, P, P, 1 << 30, None), tq.TQ_EINVAL),
        # NSN: means only on NSN caches, n >= 1, enough workspace; decode on the MFMA path only
        (lambda: tq._nsn_set(ctypes.byref(good), P, P, P, P, 1, 0, 10, 0.0, P, 1 << 30, None), tq.TQ_EINVAL),
        (lambda: tq._nsn_set(ctypes.byref(nsn), P, P, P, P, 1, 0, 0, 0.0, P, 1 << 30, None), tq.TQ_EINVAL),
        (lambda: tq._nsn_set(ctypes.byref(nsn), P, P, P, P, 1, 0, 10, 0.0, P, 8, None), tq.TQ_ENOSPACE),
        (lambda: tq._decode_attend_splits(ctypes.byref(tq.CacheDesc(1, 1, 128, 64, 4, 3, 128, 1)), P, P, 10, P,
                                          0, 1, 0, 0.0, 0.0, P, None, 0, P, 1 << 30, None), tq.TQ_EUNSUPPORTED),
        (lambda: tq._search_topk(ctypes.byref(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128)), P, P, 65, P, 4, 10,
                                 P, P, P, 1 << 30, None), tq.TQ_ECAPACITY),
        (lambda: tq._search_topk(ctypes.byref(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128)), P, P, 10, P, 4, 65,
                                 P, P, P, 1 << 30, None), tq.TQ_EINVAL),
        (lambda: tq._search_topk(ctypes.byref(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128)), P, P, 10, P, 4, 10,
                                 P, P, P, 8, None), tq.TQ_ENOSPACE),
    ]
    for fn, want in cases:
        assert fn() == want
    assert tq.status_str(tq.TQ_ECAPACITY) == "beyond cache capacity"


def test_decode_split_choice_and_workspace(tq):
    d = tq.CacheDesc(4, 8, 128, 131072, 2, 3, 128)
    s = tq.decode_splits(d, 64, 131072)
    assert s >= 1
    assert tq.decode_workspace_bytes(d, 64, 131072) == tq.decode_workspace_bytes(d, 64, 0, splits=s)


@pytest.mark.parametrize("level", [1, 2, 3, 4, 5, 6, 7])
def test_polar_grids_match_oracle(tq, O, level):
    # two independent Lloyd iterations (C++ Gauss-Legendre cells, scipy quadrature) agree
    c, t = tq.make_polar_grid(level)
    co, to = O.polar_level_codebook(level)
    np.testing.assert_allclose(c, co, rtol=0, atol=1e-12)
    np.testing.assert_allclose(t, to, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_codec_polar_tables_match_oracle(tq, O, d):
    # the codec table's stored cos / sin (fp32) and boundaries (fp64) of every level of d
    blob = tq.codec_build(tq.CodecDesc(d, 3, 3, d, 0))
    pc = O.make_polar_codebook(d)
    al = lambda n: (n + 255) // 256 * 256
    pt_off = len(blob) - al(11 * 16 * 8)              # fp64 boundaries, the last section
    pcs_off = pt_off - al(11 * 16 * 2 * 4)            # fp32 cos / sin just before
    pt = blob[pt_off:pt_off + 11 * 16 * 8].view(np.float64).reshape(11, 16)
    pcs = blob[pcs_off:pcs_off + 11 * 16 * 2 * 4].view(np.float32).reshape(11, 16, 2)
    for lv in range(1, pc.L + 1):
        K = 16 if lv == 1 else 4
        assert np.count_nonzero(pcs[lv - 1, :K, 0] != pc.cos[lv]) == 0
        assert np.count_nonzero(pcs[lv - 1, :K, 1] != pc.sin[lv]) == 0
        np.testing.assert_allclose(pt[lv - 1, :K - 1], pc.t[lv], rtol=0, atol=1e-12)


def test_binding_rejects_bad_tensors_before_the_call(tq):
    # the binding checks shapes, contiguity and dtypes on the host; each case below fails
    # there, so no pointer reaches the library (CPU tensors, no GPU needed)
    import torch
    desc = tq.CacheDesc(2, 4, 128, 64, 2, 3, 128)
    k = torch.zeros((2, 4, 8, 128), dtype=torch.bfloat16)
    cases = [
        lambda: tq.quantize_kv(desc, 1, 1, k.transpose(2, 3).contiguous().transpose(2, 3), k, 0, 0.0),
        lambda: tq.quantize_kv(desc, 1, 1, k[:, :3], k[:, :3], 0, 0.0),                    # kv_heads 3
        lambda: tq.quantize_kv(desc, 1, 1, k, k.float(), 0, 0.0),                           # mixed dtypes
        lambda: tq.quantize_kv(desc, 1, 1, k, None, 0, 0.0),                                # no values
        lambda: tq.quantize_kv(desc, 1, 1, k[:, :, ::2], k[:, :, ::2], 0, 0.0),             # strided
        lambda: tq.decode_attend(desc, 1, 1, 64, torch.zeros((2, 16, 64)), 64, 0.0,
                                 torch.zeros((2, 16, 128)), ws=1, ws_bytes=1 << 20),        # q of d 64
        lambda: tq.decode_attend(desc, 1, 1, 64, torch.zeros((2, 16, 128)), 64, 0.0,
                                 torch.zeros((2, 16, 127)), ws=1, ws_bytes=1 << 20),        # short out
        lambda: tq.decode_attend(desc, 1, 1, 64, torch.zeros((2, 16, 128)), 64, 0.0,
                                 torch.zeros((2, 16, 128), dtype=torch.float64), ws=1, ws_bytes=1 << 20),
        lambda: tq.decode_attend(desc, 1, 1, 64, torch.zeros((2, 16, 128)), 64, 0.0,
                                 torch.zeros((2, 16, 128)), scores=torch.zeros((2, 16, 63)), ws=1,
                                 ws_bytes=1 << 20),                                         # short scores
        lambda: tq.search_topk(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128), 1, 1, 64, torch.zeros((4, 128)), 10,
                               torch.zeros((4, 10), dtype=torch.int64), torch.zeros((4, 10)), 1, ws_bytes=1),
        lambda: tq.search_topk(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128), 1, 1, 64, torch.zeros((4, 128)), 10,
                               torch.zeros((4, 9), dtype=torch.int32), torch.zeros((4, 10)), 1, ws_bytes=1),
        lambda: tq.search_topk(tq.CacheDesc(1, 1, 128, 64, 3, 0, 128), 1, 1, 64,
                               torch.zeros((128, 4)).t(), 10, torch.zeros((4, 10), dtype=torch.int32),
                               torch.zeros((4, 10)), 1, ws_bytes=1),                        # strided queries
    ]
    for i, fn in enumerate(cases):
        with pytest.raises(ValueError):
            fn()
            pytest.fail(f"case {i} was not rejected")
