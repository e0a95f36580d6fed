"""Parity helpers shared by the GPU tests: run the library and the oracle on the same
seeded inputs and compare under the codec's parity rule.

Codes and bits must equal the oracle's.  The only mismatches excused are
  * a scalar code whose oracle coordinate u_j lies within 1e-6 of a decision boundary,
  * a QJL bit whose oracle |z_i| / ||r|| <= 1e-6,
  * an fp16 norm whose fp64 value lies within 1e-6 (relative) of an fp16 rounding midpoint,
and these must number at most 1e-6 of all codes.  A token with an excused scalar-code or
norm mismatch has a different residual on the two sides, so its residual norm and QJL
bits are compared only when its codes and norm agree.  NSN caches: the stored means agree
to fp32 rounding (relative 2.4e-7), an fp16 s1 may differ only next to an fp16 midpoint
(excused, counted), and a token whose s1 differs is shifted differently on the two sides,
so its codes and norms are left out of the comparison.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import tq_oracle as O
from vector_quantization_rope_amd import tq

MARGIN = 1e-6


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_means(K, V, positions, rope_base):
    """NSN means of every unit over the tokens K, V (fp64 [B, H, n, d]), fp32 [B, H, d]."""
    B, H = K.shape[:2]
    ok = np.stack([[O.nsn_mean(K[b, h], positions=positions, rope_base=rope_base) for h in range(H)]
                   for b in range(B)])
    ov = np.stack([[O.nsn_mean(V[b, h]) for h in range(H)] for b in range(B)])
    return ok.astype(np.float32), ov.astype(np.float32)


def oracle_encode_unitwise(K, V, codec, positions, rope_base, means=None):
    """K, V: fp64 [B, H, T, d] -> dict of oracle fields for all units; means = (o_K, o_V)
    fp32 [B, H, d] for an NSN cache."""
    B, H, T, d = K.shape
    rows = lambda o: None if o is None else np.repeat(o.reshape(B * H, 1, d), T, axis=1).reshape(-1, d)
    ok, ov = means if means is not None else (None, None)
    ke = O.encode(K.reshape(-1, d), codec, kind="key",
                  positions=np.tile(positions, B * H), rope_base=rope_base, nsn_o=rows(ok))
    out = {
        "kcodes": ke["codes"].reshape(B, H, T, d), "n16": ke["n16"].reshape(B, H, T),
        "rn16": ke["rn16"].reshape(B, H, T), "bits": ke["bits"].reshape(B, H, T, codec.m),
        "ku": ke["u"].reshape(B, H, T, d), "kn": ke["n"].reshape(B, H, T),
        "krn": ke["rn"].reshape(B, H, T), "kz": ke["z"].reshape(B, H, T, codec.m),
        "overflow": ke["overflow"].reshape(B, H, T),
    }
    if V is not None:
        ve = O.encode(V.reshape(-1, d), codec, kind="value", nsn_o=rows(ov))
        out.update(vcodes=ve["codes"].reshape(B, H, T, d), vn16=ve["n16"].reshape(B, H, T),
                   vu=ve["u"].reshape(B, H, T, d), vn=ve["n"].reshape(B, H, T))
        out["overflow"] = out["overflow"] | ve["overflow"].reshape(B, H, T)
        if means is not None:
            out.update(vs1=ve["s1_16"].reshape(B, H, T), vs1x=ve["s1"].reshape(B, H, T), ov=ov,
                       pov=O.nsn_rotated_mean(ov.reshape(-1, d), codec).reshape(B, H, d))
    if means is not None:
        out.update(ks1=ke["s1_16"].reshape(B, H, T), ks1x=ke["s1"].reshape(B, H, T), ok=ok,
                   pok=O.nsn_rotated_mean(ok.reshape(-1, d), codec).reshape(B, H, d))
    return out


def oracle_encode_polar(K, V, codec, positions, rope_base):
    """PolarQuant fields of every unit: kpc / vpc {level: [B, H, T, d / 2^level]}, norms,
    QJL bits, plus the oracle's angles and exact norms for the parity rule."""
    B, H, T, d = K.shape
    ke = O.polar_encode(K.reshape(-1, d), codec, kind="key", positions=np.tile(positions, B * H),
                        rope_base=rope_base)
    ve = O.polar_encode(V.reshape(-1, d), codec, kind="value")
    rs = lambda a: np.asarray(a).reshape((B, H, T) + np.asarray(a).shape[1:])
    return {"kpc": {lv: rs(c) for lv, c in ke["pcodes"].items()}, "kang": {lv: rs(c) for lv, c in ke["angles"].items()},
            "n16": rs(ke["n16"]), "kn": rs(ke["n"]), "rn16": rs(ke["rn16"]), "krn": rs(ke["rn"]),
            "bits": rs(ke["bits"]), "kz": rs(ke["z"]),
            "vpc": {lv: rs(c) for lv, c in ve["pcodes"].items()}, "vang": {lv: rs(c) for lv, c in ve["angles"].items()},
            "vn16": rs(ve["n16"]), "vn": rs(ve["n"])}


def compare_polar_codes(gpu: dict, orc: dict, codec, report=None):
    """PolarQuant records under the parity rule: an angle code may differ only when the
    oracle's angle lies within 1e-6 rad of one of its level's boundaries (for level 1 also
    the wrap-around at 0 = 2 pi), a norm only next to
    an fp16 midpoint; a key whose codes or norm differ has a different residual, so its QJL
    bits and residual norm are compared only when they agree."""
    pc = O.make_polar_codebook(codec.d)
    res = {"codes": 0, "excused": 0, "dependent": 0}
    shape = orc["n16"].shape
    for side in ("k", "v"):
        pcs, ang = orc[side + "pc"], orc[side + "ang"]
        tok_bad = np.zeros(shape, bool)
        for lv in pcs:
            bad = gpu[side + "pc"][lv] != pcs[lv]
            res["codes"] += pcs[lv].size
            if np.any(bad):
                # level-1 angles live on a circle: 0 = 2 pi is a decision boundary as well
                tb = np.concatenate(([0.0], pc.t[lv], [2 * math.pi])) if lv == 1 else pc.t[lv]
                near = np.min(np.abs(ang[lv][..., None] - tb), axis=-1) <= MARGIN
                assert np.all(near[bad]), f"{int(np.sum(bad & ~near))} {side} angle codes (level {lv}) differ away from a boundary"
                res["excused"] += int(np.sum(bad))
                tok_bad |= np.any(bad, axis=-1)
        nf, nx = ("n16", "kn") if side == "k" else ("vn16", "vn")
        nb = gpu[nf] != orc[nf]
        if np.any(nb):
            ok = _near_fp16_midpoint(orc[nx])
            assert np.all(ok[nb]), f"{int(np.sum(nb & ~ok))} {side} norms differ"
            res["excused"] += int(np.sum(nb))
            tok_bad |= nb
        if side == "k" and codec.m > 0:
            same = ~tok_bad
            b_bad = (gpu["bits"] != orc["bits"]) & same[..., None]
            res["codes"] += orc["bits"].size
            if np.any(b_bad):
                scale = np.where(orc["krn"] > 0, orc["krn"], 1.0)[..., None]
                ok = np.abs(orc["kz"]) / scale <= MARGIN
                assert np.all(ok[b_bad]), f"{int(np.sum(b_bad & ~ok))} QJL bits differ away from zero"
                res["excused"] += int(np.sum(b_bad))
            rn_bad = (gpu["rn16"] != orc["rn16"]) & same
            if np.any(rn_bad):
                ok = _near_fp16_midpoint(orc["krn"])
                assert np.all(ok[rn_bad]), f"{int(np.sum(rn_bad & ~ok))} residual norms differ"
                res["excused"] += int(np.sum(rn_bad))
            res["dependent"] += int(np.sum((gpu["bits"] != orc["bits"]) & ~same[..., None]))
    assert res["excused"] <= MARGIN * res["codes"], f"excused mismatches over budget: {res}"
    if report is not None:
        report.update(res)
    return res


def _near_boundary(u, t):
    return np.min(np.abs(u[..., None] - t), axis=-1) <= MARGIN


def _near_fp16_midpoint(x):
    """fp64 norm within 1e-6 relative of a midpoint between adjacent fp16 values."""
    x = np.asarray(x, dtype=np.float64)
    h = x.astype(np.float16).astype(np.float64)
    up = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([(h + up) / 2, (h + dn) / 2], -1)
    return np.min(np.abs(mids - x[..., None]), -1) <= MARGIN * np.maximum(np.abs(x), 1e-30)


def compare_codes(gpu: dict, orc: dict, codec, report=None):
    """gpu: unpacked GPU cache fields for the same tokens; orc: oracle_encode_unitwise.
    Returns a dict of counts; raises AssertionError on any non-excused mismatch."""
    cbk = codec.cb_k
    res = {"codes": 0, "excused": 0, "dependent": 0}
    # NSN: the means agree to fp32 rounding; an fp16 s1 may differ only next to an fp16
    # midpoint, and such a token (its shift differs) is left out of the code comparisons
    kskip = np.zeros(orc["kcodes"].shape[:3], bool)
    vskip = np.zeros(orc["kcodes"].shape[:3], bool)
    if "ks1" in orc:
        for f in ("ok", "ov", "pok", "pov"):
            g, o = np.asarray(gpu[f], np.float64), np.asarray(orc[f], np.float64)
            assert np.all(np.abs(g - o) <= 2.4e-7 * np.maximum(np.abs(o), 1e-30)), f"NSN mean {f} differs"
        for f, fx, skip in (("ks1", "ks1x", kskip), ("vs1", "vs1x", vskip)):
            bad = gpu[f] != orc[f]
            if np.any(bad):
                ok = _near_fp16_midpoint(orc[fx])
                assert np.all(ok[bad]), f"{int(np.sum(bad & ~ok))} NSN s1 values differ away from an fp16 midpoint"
                res["excused"] += int(np.sum(bad))
                skip |= bad
        res["codes"] += 2 * kskip.size
    kc_bad = (gpu["kcodes"] != orc["kcodes"]) & ~kskip[..., None]
    res["codes"] += orc["kcodes"].size
    if np.any(kc_bad):
        ok = _near_boundary(orc["ku"], cbk.t)
        assert np.all(ok[kc_bad]), f"{int(np.sum(kc_bad & ~ok))} key codes differ away from a boundary"
        res["excused"] += int(np.sum(kc_bad))
    n_bad = (gpu["n16"] != orc["n16"]) & ~kskip
    if np.any(n_bad):
        ok = _near_fp16_midpoint(orc["kn"])
        assert np.all(ok[n_bad]), f"{int(np.sum(n_bad & ~ok))} key norms differ away from an fp16 midpoint"
        res["excused"] += int(np.sum(n_bad))
    # tokens whose residual is defined the same way on both sides
    same_tok = ~(np.any(kc_bad, axis=-1) | n_bad | kskip)
    if codec.m > 0:
        b_bad = (gpu["bits"] != orc["bits"]) & same_tok[..., None]
        res["codes"] += orc["bits"].size
        if np.any(b_bad):
            scale = np.where(orc["krn"] > 0, orc["krn"], 1.0)[..., None]
            ok = np.abs(orc["kz"]) / scale <= MARGIN
            assert np.all(ok[b_bad]), f"{int(np.sum(b_bad & ~ok))} QJL bits differ away from zero"
            res["excused"] += int(np.sum(b_bad))
        rn_bad = (gpu["rn16"] != orc["rn16"]) & same_tok
        if np.any(rn_bad):
            ok = _near_fp16_midpoint(orc["krn"])
            assert np.all(ok[rn_bad]), f"{int(np.sum(rn_bad & ~ok))} residual norms differ"
            res["excused"] += int(np.sum(rn_bad))
        res["dependent"] += int(np.sum((gpu["bits"] != orc["bits"]) & ~same_tok[..., None]))
    if "vcodes" in orc:
        cbv = codec.cb_v
        vc_bad = (gpu["vcodes"] != orc["vcodes"]) & ~vskip[..., None]
        res["codes"] += orc["vcodes"].size
        if np.any(vc_bad):
            ok = _near_boundary(orc["vu"], cbv.t)
            assert np.all(ok[vc_bad]), f"{int(np.sum(vc_bad & ~ok))} value codes differ away from a boundary"
            res["excused"] += int(np.sum(vc_bad))
        vn_bad = (gpu["vn16"] != orc["vn16"]) & ~vskip
        if np.any(vn_bad):
            ok = _near_fp16_midpoint(orc["vn"])
            assert np.all(ok[vn_bad]), f"{int(np.sum(vn_bad & ~ok))} value norms differ"
            res["excused"] += int(np.sum(vn_bad))
    assert res["excused"] <= MARGIN * res["codes"], f"excused mismatches over budget: {res}"
    if report is not None:
        report.update(res)
    return res


def gpu_fields(cache: "tq.PackedCache", length: int) -> dict:
    img = cache.buf.to("cpu").numpy()
    return O.unpack_cache(img, cache.desc.as_dict(), length)


def oracle_image(desc: dict, fields: dict, start=0) -> np.ndarray:
    return O.pack_cache(desc, fields, start_pos=start)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def unit_fields(cache: "tq.PackedCache", unit: int, length: int) -> dict:
    """Unpacked fields of one (batch, kv-head) unit of a device cache, tokens [0, length).

    Copies only that unit's slices of each region (the layout of the format description,
    as the oracle computes it) into a one-unit image and unpacks it with the oracle."""
    desc = cache.desc.as_dict()
    nsn, polar = desc.get("nsn", 0), desc.get("polar", 0)
    lay = O.cache_layout(desc["batch"], desc["kv_heads"], desc["d"], desc["capacity"],
                         desc["bits_k"], desc["bits_v"], desc["m"], nsn, polar)
    sub = dict(desc, batch=1, kv_heads=1)
    sl = O.cache_layout(1, 1, sub["d"], sub["capacity"], sub["bits_k"], sub["bits_v"], sub["m"], nsn, polar)
    img = np.zeros(sl["total"], dtype=np.uint8)
    img[:256] = cache.buf[:256].cpu().numpy()
    cap = desc["capacity"]
    sizes = {"kbits": cap * lay["kbytes"], "knorm": cap * lay["knrec"]}
    if desc["bits_v"] > 0:
        vbytes = cap * 3 * desc["d"] // 8 if polar else lay["tiles"] * desc["d"] * 4 * desc["bits_v"]
        sizes.update(vcodes=vbytes, vnorm=cap * lay["vnrec"])
    if nsn:
        sizes["nsn"] = 4 * desc["d"] * 4
    for name, n in sizes.items():
        src = cache.buf[lay[name] + unit * n: lay[name] + (unit + 1) * n]
        img[sl[name]: sl[name] + n] = src.cpu().numpy()
    return O.unpack_cache(img, sub, length)


def fields_slice(f: dict, t0: int, t1: int) -> dict:
    """Tokens [t0, t1) of unpacked / oracle fields ([1, 1, T, ...] arrays)."""
    out = {}
    for k, v in f.items():
        out[k] = v[:, :, t0:t1] if isinstance(v, np.ndarray) and v.ndim >= 3 else v
    return out
