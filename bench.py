"""Benchmark: one step of the packed-KV hot path on the long-context GQA workload.

Workload (one GPU's share of a long-context decode): 1 layer, 64 q-heads / 8 kv-heads,
head dim 128, batch 4, context 131072, bf16 unit-variance Laplace keys/values with 4
channels x20, RoPE base 500000, keys 2-bit + 1-bit QJL (m = 128), values 3-bit.
The cache is prefilled with positions [0, 126976) before timing.  One step =
  * append: tq_quantize_kv of the last 4096 positions [126976, 131072) of every
    (batch, kv-head) unit (rewritten each step), and
  * decode: tq_decode_attend of one query per (batch, q-head) over all 131072 tokens.
Inputs (K, V, q) are resident in HBM before timing.  `value` is the decode attention
throughput in GB/s of algorithmic packed-cache bytes (52 B key + 50 B value per token
per kv-head) over the whole decode call.  Extra fields give the append throughput
(Mtokens/s, a token being one position of one sequence with all its kv-heads, K and V),
the roofline of the dominant kernel (split-K decode; its duration comes from HIP
events the library records around that kernel), the CPU oracle timed on a bounded
sample on this host, and -- outside the timed steps -- the vector-search workload
(10^6 x 1536 database build, search of 1024 queries, recall@10).

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--spinup-ms 300] [--no-cpu-baseline]
                    [--sections widths,nsn,polar,window,configs,search] [--no-search]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KEY_RECORD = 52      # bytes per token per kv-head: 2-bit planes 32 + signs 16 + 2 fp16 norms
VALUE_RECORD = 50    # 3-bit codes 48 + fp16 norm
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_lds_long_context_counters.txt")
DEVICE_SRC = os.path.join(ROOT, "vector_quantization_rope_amd", "csrc", "tq_device.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEventCreate / hipEventElapsedTime through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = None
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if self.hip is None:
            raise RuntimeError("libamdhip64.so not found")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def pct_us(ms):
    """p10, median and p90 of a list of durations in ms, in microseconds."""
    v = sorted(ms)
    at = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))] * 1e3
    return [round(at(0.1), 2), round(at(0.5), 2), round(at(0.9), 2)]


# Source regions the decode kernel is built from: the shared helpers at the top of the
# device source, the MFMA decode section (argument block, query prep, k_decode_lds) and the
# host-side launch constants. Counters taken on other sources stay valid while these match.
_DECODE_REGIONS = (("", "// ------------------------------------------------------------------ quantize"),
                   ("// ------------------------------------------------------------------ decode (MFMA path)",
                    "// ------------------------------------------------------------------ full-precision window"),
                   ("// ------------------------------------------------------------------ host-side helpers",
                    "}  // namespace tq"))


def kernel_source_hash() -> str:
    with open(DEVICE_SRC, encoding="utf-8") as f:
        src = f.read()
    h = hashlib.sha256()
    for start, end in _DECODE_REGIONS:
        i = src.index(start) if start else 0
        h.update(src[i:src.index(end, i)].encode())
    return h.hexdigest()[:16]


def traffic_from_counters(launch_bytes: float):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def cpu_baseline(w, K, V, q, units_total: int, n_units: int = 8):
    """Time the CPU oracle on a bounded sample of the same workload: the first `n_units`
    (batch, kv-head) units, each encoded (all its keys and values) and attended by its
    G q-heads over all its tokens."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import tq_oracle as O

    G = w.q_heads // w.kv_heads
    codec = O.make_codec(w.d, w.bits_k, w.bits_v, w.m, 0)
    t_enc = t_att = 0.0
    T = K.shape[2]
    for u in range(n_units):
        b, g = divmod(u, w.kv_heads)
        Kd = K[b, g].to("cpu").to(torch.float64).numpy()
        Vd = V[b, g].to("cpu").to(torch.float64).numpy()
        qd = q[b:b + 1, g * G:(g + 1) * G].to("cpu").to(torch.float64).numpy()
        t0 = time.perf_counter()
        ke = O.encode(Kd, codec, kind="key", positions=np.arange(T), rope_base=w.rope_base)
        ve = O.encode(Vd, codec, kind="value")
        t_enc += time.perf_counter() - t0
        fields = {"kcodes": ke["codes"][None, None], "n16": ke["n16"][None, None],
                  "rn16": ke["rn16"][None, None], "bits": ke["bits"][None, None],
                  "vcodes": ve["codes"][None, None], "vn16": ve["n16"][None, None]}
        del ke, ve
        t0 = time.perf_counter()
        O.attend(fields, qd, codec, q_pos=w.q_pos, rope_base=w.rope_base, scale=0.0, kv_heads=1, length=T)
        t_att += time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    gbs = n_units * T * (KEY_RECORD + VALUE_RECORD) / t_att / 1e9
    # a token is one position of one sequence with all its kv-heads
    mtok = n_units * T / w.kv_heads / t_enc / 1e6
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{n_units} of the {units_total} (batch, kv-head) units: oracle decode attention of "
                   f"their {G} q-heads each over all {T} tokens ({t_att:.1f} s), and oracle encode of "
                   f"their {T} keys and values each ({t_enc:.1f} s)"),
        "quantize_mtokens_s": round(mtok, 6),
        "seconds": round(t_enc + t_att, 2),
    }


def search_bench(tq, W, dev, ev, stream):
    """Vector search workload (10^6 x 1536 database, 1024 queries, 3-bit + QJL m = 1536,
    top-10): database build and search times from HIP events, recall against exact fp32
    inner products.  Reported beside the decode line, outside its timed region."""
    import torch

    w = W.VECTOR_SEARCH
    db, qs = W.gen_search(w, device=dev)
    codec = tq.Codec(w.d, w.bits, 0, w.m, seed=0, device=dev)
    cache = tq.PackedCache(1, 1, w.d, w.n_db, w.bits, 0, w.m, device=dev)
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device=dev)
    val = torch.empty((w.nq, w.k), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.search_workspace_bytes(cache.desc, w.n_db, w.nq, w.k), dtype=torch.uint8, device=dev)
    e = [ev.create() for _ in range(4)]
    build_ms, search_ms = [], []
    for _ in range(3):
        ev.record(e[0], stream)
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, db[None, None], None, 0, 0.0)
        ev.record(e[1], stream)
        tq.search_topk(cache.desc, codec.dev, cache.buf, w.n_db, qs, w.k, idx, val, ws)
        ev.record(e[2], stream)
        build_ms.append(ev.elapsed_ms(e[0], e[1]))
        search_ms.append(ev.elapsed_ms(e[1], e[2]))
    torch.cuda.synchronize()
    exact = []
    for s0 in range(0, w.nq, 128):
        exact.append(torch.topk(qs[s0:s0 + 128] @ db.T, w.k, dim=1).indices)
    exact = torch.cat(exact).cpu()
    got = idx.cpu().long()
    hit = sum(len(set(got[i].tolist()) & set(exact[i].tolist())) for i in range(w.nq))
    top1 = sum(int(exact[i, 0].item() in set(got[i].tolist())) for i in range(w.nq))
    bm, sm = min(build_ms[1:]), min(search_ms[1:])
    pairs = w.nq * w.n_db
    return {
        "workload": (f"vector_search: {w.n_db} database vectors of dim {w.d}, fp32 N(0,1) unit rows, "
                     f"3-bit codes + QJL m={w.m}, {w.nq} unit queries, top-{w.k}"),
        "db_build_ms": round(bm, 3), "db_build_mvec_s": round(w.n_db / bm / 1e3, 3),
        "search_ms": round(sm, 3), "search_gpairs_s": round(pairs / sm / 1e6, 3),
        "search_equiv_tflops": round(pairs * 2 * (w.d + w.m) / sm / 1e9, 2),
        "recall_at_10": round(hit / (w.nq * w.k), 4), "recall_1_at_10": round(top1 / w.nq, 4),
    }


def time_us(fn, ev, stream, reps: int = 20, warm_ms: float = 100.0):
    """p10 / median / p90 (us) of fn() over `reps` calls, each bracketed by HIP events on the
    stream, after `warm_ms` of untimed calls (the clock ramps up under load)."""
    import torch

    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < warm_ms * 1e-3:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    E = [(ev.create(), ev.create()) for _ in range(reps)]
    for e0, e1 in E:
        ev.record(e0, stream)
        fn()
        ev.record(e1, stream)
    torch.cuda.synchronize()
    return pct_us([ev.elapsed_ms(e0, e1) for e0, e1 in E])


def configs_bench(tq, W, dev, ev, stream):
    """The other decode workloads, outside the timed steps (medians of event-timed calls):
      * llama3_8b: one decode step over all 32 layers (32 tq_decode_attend calls, one per
        layer cache, 13.69 GB of packed records), and the quantize of one layer's prefill;
      * esm2_650m: the quantize of all 33 layers' 1024 tokens, and one decode step over
        the 33 layers (36.5 MB of packed records: it fits in the 256 MB last-level cache, so
        the step is latency-bound and reported in us per layer);
      * single_head: quantize of the 1024 fp32 tokens and one decode with its 1024 scores."""
    import torch

    out_rec = {}
    rec_bytes = lambda w: (w.bits_k * w.d + w.m) // 8 + 4 + w.bits_v * w.d // 8 + 2

    # ---- llama3_8b: 32 layers, 16 x 8 units x 32768 tokens
    w = W.LLAMA3_8B
    T, units = w.context, w.batch * w.kv_heads
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0, device=dev)
    caches, qs = [], []
    prefill_us = None
    for layer in range(w.layers):
        K, V = W.gen_kv(w, layer, device=dev)
        c = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m, device=dev)
        if layer == 0:
            prefill_us = time_us(lambda: tq.quantize_kv(c.desc, codec.dev, c.buf, K, V, 0, w.rope_base), ev,
                                 stream, reps=5, warm_ms=50.0)
        tq.quantize_kv(c.desc, codec.dev, c.buf, K, V, 0, w.rope_base)
        del K, V
        caches.append(c)
        qs.append(W.gen_q(w, layer, device=dev))
    torch.cuda.synchronize()
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(caches[0].desc, w.q_heads, T), dtype=torch.uint8, device=dev)

    def llama_step():
        for layer in range(w.layers):
            tq.decode_attend(caches[layer].desc, codec.dev, caches[layer].buf, T, qs[layer], w.q_pos, w.rope_base,
                             out, ws=ws)

    st = time_us(llama_step, ev, stream, reps=20)
    step_bytes = w.layers * units * T * rec_bytes(w)
    out_rec["llama3_8b"] = {
        "workload": ("llama3_8b: 32 layers, 32 q-heads / 8 kv-heads, d 128, batch 16, context 32768, bf16 N(0,1) "
                     "+ 3 channels x10, RoPE 500000; one decode step = one tq_decode_attend per layer"),
        "step_us_p10_p50_p90": st, "layer_us": round(st[1] / w.layers, 2),
        "packed_bytes_per_step": step_bytes,
        "step_gbs": round(step_bytes / (st[1] * 1e-6) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (st[1] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_splits": tq.decode_splits(caches[0].desc, w.q_heads, T),
        "prefill_quantize_us_p10_p50_p90": prefill_us,
        "prefill_quantize_mtokens_s": round(w.batch * T / (prefill_us[1] * 1e-6) / 1e6, 1),
    }
    del caches, qs, out, ws
    torch.cuda.empty_cache()
    log(f"[bench] llama3_8b {out_rec['llama3_8b']}")

    # ---- esm2_650m: 33 layers, 20 heads (G = 1), d 64, 1024 tokens
    w = W.ESM2_650M
    T, units = w.context, w.batch * w.kv_heads
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0, device=dev)
    kvs = [W.gen_kv(w, layer, device=dev) for layer in range(w.layers)]
    qs = [W.gen_q(w, layer, device=dev) for layer in range(w.layers)]
    caches = [tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m, device=dev)
              for _ in range(w.layers)]

    def esm_quantize():
        for layer in range(w.layers):
            tq.quantize_kv(caches[layer].desc, codec.dev, caches[layer].buf, kvs[layer][0], kvs[layer][1], 0,
                           w.rope_base)

    qt = time_us(esm_quantize, ev, stream, reps=10, warm_ms=50.0)
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(caches[0].desc, w.q_heads, T), dtype=torch.uint8, device=dev)

    def esm_step():
        for layer in range(w.layers):
            tq.decode_attend(caches[layer].desc, codec.dev, caches[layer].buf, T, qs[layer], w.q_pos, w.rope_base,
                             out, ws=ws)

    st = time_us(esm_step, ev, stream, reps=20)
    step_bytes = w.layers * units * T * rec_bytes(w)
    out_rec["esm2_650m"] = {
        "workload": ("esm2_650m: 33 layers x 20 heads x d 64, batch 1, 1024 tokens, bf16 Student-t (nu 3) + 3 "
                     "channels x15, RoPE 10000; keys 2-bit + QJL m 64, values 3-bit"),
        "quantize_all_layers_us_p10_p50_p90": qt,
        "quantize_mtokens_s": round(w.layers * T / (qt[1] * 1e-6) / 1e6, 2),
        "step_us_p10_p50_p90": st, "layer_us": round(st[1] / w.layers, 2),
        "packed_bytes_per_step": step_bytes,
        "cache_resident": "MALL (36.5 MB of records in the 256 MB last-level cache): latency-bound, no HBM roofline",
    }
    del kvs, qs, caches, out, ws
    log(f"[bench] esm2_650m {out_rec['esm2_650m']}")

    # ---- single_head: d 128, 1024 fp32 tokens, one query, no RoPE
    w = W.SINGLE_HEAD
    T = w.context
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0, device=dev)
    K, V = W.gen_kv(w, device=dev)
    q = W.gen_q(w, device=dev)
    c = tq.PackedCache(1, 1, w.d, T, w.bits_k, w.bits_v, w.m, device=dev)
    qt = time_us(lambda: tq.quantize_kv(c.desc, codec.dev, c.buf, K, V, 0, 0.0), ev, stream, reps=20)
    out = torch.empty((1, 1, w.d), dtype=torch.float32, device=dev)
    sc = torch.empty((1, 1, T), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(c.desc, 1, T), dtype=torch.uint8, device=dev)
    st = time_us(lambda: tq.decode_attend(c.desc, codec.dev, c.buf, T, q, w.q_pos, 0.0, out, scores=sc, ws=ws),
                 ev, stream, reps=20)
    out_rec["single_head"] = {
        "workload": "single_head: d 128, 1024 fp32 N(0,1) tokens + 4 channels x20, no RoPE, one query",
        "quantize_us_p10_p50_p90": qt, "decode_with_scores_us_p10_p50_p90": st,
    }
    log(f"[bench] single_head {out_rec['single_head']}")
    return out_rec


def timed_calls(fn, ev, stream, E):
    """Median call and kernel times (us) of fn over len(E) back-to-back calls, after 80 ms of
    the same calls (the work before idles the GPU and its clock ramps up again); fn(events)
    records its kernel between the given pair of events, fn(None) records nothing.  Events
    recorded between a call's kernels hold the stream for a few microseconds each, so the
    calls alternate: the odd ones are timed whole with no event inside, the even ones give
    the kernel time."""
    import torch

    med = lambda v: sorted(v)[len(v) // 2]
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.08:
        fn(None)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    for i, e in enumerate(E):
        if i % 2:
            ev.record(e[0], stream)
            fn(None)
            ev.record(e[3], stream)
        else:
            fn((e[1], e[2]))
    torch.cuda.synchronize()
    return (med([ev.elapsed_ms(e[0], e[3]) * 1e3 for i, e in enumerate(E) if i % 2]),
            med([ev.elapsed_ms(e[1], e[2]) * 1e3 for i, e in enumerate(E) if not i % 2]))


def nsn_bench(tq, w, K, V, q, dev, ev, stream, reps: int = 30):
    """NSN cache (normalize-shift-normalize before the codec) on the long-context shape,
    outside the timed steps: the prefill means (tq_nsn_set_means over 126976 tokens per
    unit), the 4096-token append, decode and logits only, medians of back-to-back calls."""
    import torch

    T, A = w.context, w.append
    pre = T - A
    units, G = w.batch * w.kv_heads, w.q_heads // w.kv_heads
    E = [[ev.create() for _ in range(4)] for _ in range(reps)]
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0, device=dev)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m, device=dev, nsn=1)
    Kp, Vp = K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous()
    Ka, Va = K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous()
    wsm = torch.empty(tq.nsn_means_workspace_bytes(cache.desc, pre), dtype=torch.uint8, device=dev)
    def means(e):
        if e:
            ev.record(e[0], stream)
        tq.nsn_set_means(cache.desc, codec.dev, cache.buf, Kp, Vp, 0, w.rope_base, wsm)
        if e:
            ev.record(e[1], stream)

    means_call, _ = timed_calls(means, ev, stream, E[:5])
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kp, Vp, 0, w.rope_base)
    del Kp, Vp
    app_call, app_kern = timed_calls(lambda e: tq.quantize_kv(cache.desc, codec.dev, cache.buf, Ka, Va, pre,
                                                              w.rope_base, events=e), ev, stream, E)
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device=dev)
    sc = torch.empty((w.batch, w.q_heads, T), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device=dev)
    dec_call, dec_kern = timed_calls(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                                w.rope_base, out, ws=ws, events=e), ev, stream, E)
    lg_call, lg_kern = timed_calls(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                              w.rope_base, None, scores=sc, ws=ws, events=e),
                                   ev, stream, E)
    rec = KEY_RECORD + 4 + VALUE_RECORD + 2   # norm records grow by fp16 s1 (+ padding for keys)
    dbytes = units * T * rec
    return {"workload": ("long_context shape, NSN cache: means over the 126976-token prefill, append of "
                         "4096 tokens, decode and logits at 131072; medians over %d calls" % reps),
            "record_bytes_per_token": rec,
            "means_call_us": round(means_call, 1),
            "append_kernel_us": round(app_kern, 2),
            "append_mtokens_s": round(w.batch * A / (app_kern * 1e-6) / 1e6, 1),
            "decode_call_us": round(dec_call, 2), "split_kernel_us": round(dec_kern, 2),
            "split_kernel_gbs": round(dbytes / (dec_kern * 1e-6) / 1e9, 1),
            "split_kernel_hbm_frac": round(dbytes / (dec_kern * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "logits_call_us": round(lg_call, 2), "logits_kernel_us": round(lg_kern, 2)}


def polar_bench(tq, w, K, V, q, dev, ev, stream, reps: int = 20):
    """PolarQuant caches (recursive polar angles as stage 1, QJL on the key residual) on the
    long-context shape, outside the timed steps: the 4096-token append, decode and logits
    only, medians of back-to-back calls.  The decode kernel decodes every key and value
    coordinate from its angle tree and splits it into fp16 hi + lo for the MFMA dot
    products and value sums: it is bound by vector instruction issue, not by its bytes."""
    import torch

    T, A = w.context, w.append
    pre = T - A
    units, d = w.batch * w.kv_heads, w.d
    E = [[ev.create() for _ in range(4)] for _ in range(reps)]
    codec = tq.Codec(d, 3, 3, d, seed=0, device=dev)
    cache = tq.PackedCache(w.batch, w.kv_heads, d, T, 3, 3, d, device=dev, polar=1)
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous(), 0,
                   w.rope_base)
    Ka, Va = K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous()
    app_call, app_kern = timed_calls(lambda e: tq.quantize_kv(cache.desc, codec.dev, cache.buf, Ka, Va, pre,
                                                              w.rope_base, events=e), ev, stream, E)
    out = torch.empty((w.batch, w.q_heads, d), dtype=torch.float32, device=dev)
    sc = torch.empty((w.batch, w.q_heads, T), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device=dev)
    dec_call, dec_kern = timed_calls(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                                w.rope_base, out, ws=ws, events=e), ev, stream, E)
    lg_call, _ = timed_calls(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                         w.rope_base, None, scores=sc, ws=ws, events=e), ev, stream, E)
    rec = 3 * d // 8 + d // 8 + 4 + 3 * d // 8 + 2          # angles + signs + norms, keys and values
    dbytes = units * T * rec
    return {"workload": ("long_context shape, PolarQuant keys (3 - 2/d bits of angles + QJL m = d) and values; "
                         "append of 4096 tokens, decode and logits at 131072; medians over %d calls" % reps),
            "record_bytes_per_token": rec,
            "append_kernel_us": round(app_kern, 2),
            "append_mtokens_s": round(w.batch * A / (app_kern * 1e-6) / 1e6, 1),
            "decode_call_us": round(dec_call, 2), "split_kernel_us": round(dec_kern, 2),
            "split_kernel_gbs": round(dbytes / (dec_kern * 1e-6) / 1e9, 1),
            "split_kernel_hbm_frac": round(dbytes / (dec_kern * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "split_kernel_limiter": ("VALU issue: the angle-tree decode of every coordinate and its fp16 hi + lo "
                                     "split; dots and value sums on MFMA (profiles/decode_polar_long_context.md)"),
            "logits_call_us": round(lg_call, 2)}


def key_width_bench(tq, W, w, K, V, q, dev, ev, stream, reps: int = 30):
    """Key bit-width variants on the same long-context shape, outside the timed steps:
    full decode of 1-, 2- and 3-bit keys (+ QJL, 3-bit values), and attention logits only
    (scores, out = NULL) for packed 3- and 4-bit keys next to the same logits computed from
    unquantized fp32 and bf16 keys with a batched matmul (the pages' "up to 8x" compares
    4-bit keys against 32-bit ones)."""
    import torch

    T, units, G = w.context, w.batch * w.kv_heads, w.q_heads // w.kv_heads
    vrec = w.d * 3 // 8 + 2
    med = lambda v: sorted(v)[len(v) // 2]
    E = [[ev.create() for _ in range(4)] for _ in range(reps)]
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device=dev)
    sc = torch.empty((w.batch, w.q_heads, T), dtype=torch.float32, device=dev)

    def timed(fn):
        return timed_calls(fn, ev, stream, E)

    decode, logits = {}, {}
    for bk in (1, 2, 3):
        codec = tq.Codec(w.d, bk, w.bits_v, w.d, seed=0, device=dev)
        cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, bk, w.bits_v, w.d, device=dev)
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, K, V, 0, w.rope_base)
        ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device=dev)
        krec = (bk + 1) * w.d // 8 + 4
        call, kern = timed(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                       w.rope_base, out, ws=ws, events=e))
        nbytes = units * T * (krec + vrec)
        decode[f"keys_{bk}bit_qjl"] = {
            "bits_per_key_coordinate": bk + 1, "record_bytes_per_token": krec + vrec,
            "decode_call_us": round(call, 2), "split_kernel_us": round(kern, 2),
            "split_kernel_gbs": round(nbytes / (kern * 1e-6) / 1e9, 1),
            "split_kernel_hbm_frac": round(nbytes / (kern * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if bk >= 2:
            call, kern = timed(lambda e: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos,
                                                           w.rope_base, None, scores=sc, ws=ws, events=e))
            lb = units * T * (krec + 4 * G)
            logits[f"packed_{bk + 1}bit_keys"] = {
                "call_us": round(call, 2), "kernel_us": round(kern, 2),
                "kernel_gbs": round(lb / (kern * 1e-6) / 1e9, 1)}
        del cache, ws, codec
    # unquantized keys: scores[u, t, g] = K[u, t, :] . q[u, g, :] as one batched matmul
    qf = q.float().reshape(units, G, w.d).transpose(1, 2).contiguous()
    for name, kdt in (("fp32_keys", torch.float32), ("bf16_keys", torch.bfloat16)):
        Ku = K.reshape(units, T, w.d).to(kdt).contiguous()
        qu = qf.to(kdt).contiguous()
        res = torch.empty((units, T, G), dtype=kdt, device=dev)
        call, _ = timed(lambda e: torch.matmul(Ku, qu, out=res) if e is None else
                        (ev.record(e[0], stream), torch.matmul(Ku, qu, out=res), ev.record(e[1], stream)))
        eb = torch.finfo(kdt).bits // 8
        lb = units * T * (w.d + G) * eb
        logits[name] = {"call_us": round(call, 2), "gbs": round(lb / (call * 1e-6) / 1e9, 1)}
        del Ku, qu, res
    base = logits["fp32_keys"]["call_us"]
    for k in ("packed_3bit_keys", "packed_4bit_keys"):
        logits[k]["speedup_vs_fp32_keys"] = round(base / logits[k]["call_us"], 2)
        logits[k]["speedup_vs_bf16_keys"] = round(logits["bf16_keys"]["call_us"] / logits[k]["call_us"], 2)
    return {"workload": ("long_context shape (4 x 8 units x 131072 tokens, 8 q-heads per kv-head, d 128), "
                         "3-bit values; medians over %d calls" % reps),
            "decode": decode, "logits": logits}


def window_bench(tq, w, K, V, q, cache, codec, dev, ev, stream, cap: int = 128, cycles: int = 3):
    """The full-precision recent-token window on the long-context cache, outside the timed
    steps: (1) the same T tokens attended as T - cap packed + cap raw ones, next to plain
    decode over T packed tokens; (2) a generation loop of tq_decode_step calls (one flush
    of the cap-token window every cap steps, the new token stored by the window kernel),
    per-step call times split into steps with and without the flush.  The loop rewrites
    packed tokens the cache already holds, so the cache stays as it was."""
    import torch

    T, B, Hkv, d = w.context, w.batch, w.kv_heads, w.d
    med = lambda v: sorted(v)[len(v) // 2]
    out = torch.empty((B, w.q_heads, d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_window_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device=dev)
    wk = K[:, :, T - cap:].contiguous()
    wv = V[:, :, T - cap:].contiguous()
    reps = 40
    E = [[ev.create() for _ in range(2)] for _ in range(reps)]

    def timed(fn):
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < 0.3:
            fn()
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        for i in range(reps):
            ev.record(E[i][0], stream)
            fn()
            ev.record(E[i][1], stream)
        torch.cuda.synchronize()
        return med([ev.elapsed_ms(e[0], e[1]) * 1e3 for e in E])

    plain = timed(lambda: tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out,
                                           ws=ws))
    win = timed(lambda: tq.decode_attend_window(cache.desc, codec.dev, cache.buf, T - cap, wk, wv, cap, q,
                                                w.q_pos, w.rope_base, out, ws=ws))
    # generation loop
    n = cap * cycles
    L0 = T - n - cap
    Kn = K[:, :, L0:L0 + n].permute(2, 0, 1, 3).contiguous()
    Vn = V[:, :, L0:L0 + n].permute(2, 0, 1, 3).contiguous()
    bk = torch.zeros((B, Hkv, cap, d), dtype=K.dtype, device=dev)
    bv = torch.zeros_like(bk)
    SE = [[ev.create() for _ in range(2)] for _ in range(n)]

    def loop(events):
        L, Wn = L0, 0
        for s in range(n):
            if events:
                ev.record(SE[s][0], stream)
            L, Wn = tq.decode_step(cache.desc, codec.dev, cache.buf, L, bk, bv, Wn, Kn[s], Vn[s], q, L0 + s,
                                   w.rope_base, out, ws=ws)
            if events:
                ev.record(SE[s][1], stream)
        return L, Wn

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        loop(False)
    torch.cuda.synchronize()
    L, Wn = loop(True)
    torch.cuda.synchronize()
    st = [ev.elapsed_ms(e[0], e[1]) * 1e3 for e in SE]
    flush = [st[s] for s in range(cap, n, cap)]
    plain_steps = [st[s] for s in range(n) if s % cap != 0]
    return {"workload": (f"long_context shape (4 x 8 units, d 128, G 8), {T} tokens; window of {cap} "
                         f"tokens; loop of {n} steps from {L0} packed tokens; medians"),
            "plain_decode_call_us": round(plain, 2),
            "packed_plus_window_call_us": round(win, 2),
            "window_overhead_us": round(win - plain, 2),
            "step_call_us_no_flush": round(med(plain_steps), 2),
            "step_call_us_with_flush": round(med(flush), 2) if flush else None,
            "step_call_us_mean": round(sum(st) / len(st), 2),
            "final_length_window": [L, Wn]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="untimed steps run for this long before the warmup steps, so that the "
                         "timed steps see the GPU at its sustained clock (it ramps up over the "
                         "first tens of milliseconds of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true", help="skip the vector-search measurement")
    ap.add_argument("--sections", default="widths,nsn,polar,window,configs,search",
                    help="comma-separated measurements beside the timed steps (any of widths, nsn, "
                         "polar, window, configs, search; empty for none)")
    ap.add_argument("--copy-calibration", type=int, default=1024,
                    help="size in MiB of the plain streaming copy that is timed (measured HBM "
                         "bandwidth) and whose counters scale the decode kernel's (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the packed-KV path runs on a single device and this "
              "build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 2:
        # odd steps time the decode call, even steps its split kernel
        print("bench.py needs --steps 2 or more", file=sys.stderr)
        sys.exit(2)

    import torch

    from vector_quantization_rope_amd import tq
    from vector_quantization_rope_amd import workloads as W

    w = W.LONG_CONTEXT
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    T, A = w.context, w.append
    pre = T - A
    log(f"[bench] generating {w.name} inputs on the GPU ...")
    K, V = W.gen_kv(w, device=dev)
    q = W.gen_q(w, device=dev)
    codec = tq.Codec(w.d, w.bits_k, w.bits_v, w.m, seed=0, device=dev)
    cache = tq.PackedCache(w.batch, w.kv_heads, w.d, T, w.bits_k, w.bits_v, w.m, device=dev)
    Kp, Vp = K[:, :, :pre].contiguous(), V[:, :, :pre].contiguous()
    Ka, Va = K[:, :, pre:].contiguous(), V[:, :, pre:].contiguous()
    tq.quantize_kv(cache.desc, codec.dev, cache.buf, Kp, Vp, 0, w.rope_base)
    del Kp, Vp
    out = torch.empty((w.batch, w.q_heads, w.d), dtype=torch.float32, device=dev)
    splits = tq.decode_splits(cache.desc, w.q_heads, T)
    ws = torch.empty(tq.decode_workspace_bytes(cache.desc, w.q_heads, T), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] prefill done; decode splits {splits}")

    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    E = {k: [ev.create() for _ in range(args.steps)] for k in
         ("a0", "a1", "k0", "k1", "d0", "d1")}

    def step(i=None):
        if i is None:
            tq.quantize_kv(cache.desc, codec.dev, cache.buf, Ka, Va, pre, w.rope_base)
            tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=ws)
            return
        tq.quantize_kv(cache.desc, codec.dev, cache.buf, Ka, Va, pre, w.rope_base,
                       events=(E["a0"][i], E["a1"][i]))
        # events recorded between the decode call's kernels hold the stream for a few
        # microseconds each: odd steps time the whole call with no event inside it, even
        # steps time its split kernel
        if i % 2:
            ev.record(E["d0"][i], stream)
            tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=ws)
            ev.record(E["d1"][i], stream)
        else:
            tq.decode_attend(cache.desc, codec.dev, cache.buf, T, q, w.q_pos, w.rope_base, out, ws=ws,
                             events=(E["k0"][i], E["k1"][i]))

    t_spin = time.perf_counter()
    spin = 0
    while (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        step()
        spin += 1
        if spin % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"[bench] spin-up: {spin} untimed steps in {(time.perf_counter() - t_spin) * 1e3:.0f} ms")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    append_ms = [ev.elapsed_ms(E["a0"][i], E["a1"][i]) for i in range(args.steps)]
    kern_ms = [ev.elapsed_ms(E["k0"][i], E["k1"][i]) for i in range(0, args.steps, 2)]
    dec_ms = [ev.elapsed_ms(E["d0"][i], E["d1"][i]) for i in range(1, args.steps, 2)]
    mean = lambda v: sum(v) / len(v)
    units = w.batch * w.kv_heads
    dec_bytes = units * T * (KEY_RECORD + VALUE_RECORD)
    dec_gbs = dec_bytes / (mean(dec_ms) * 1e-3) / 1e9
    kern_gbs = dec_bytes / (mean(kern_ms) * 1e-3) / 1e9
    append_tokens = w.batch * A
    append_mtok = append_tokens / (mean(append_ms) * 1e-3) / 1e6
    # append algorithmic bytes: bf16 K and V read + records written
    append_bytes = units * A * (2 * w.d * 2 + KEY_RECORD + VALUE_RECORD)
    log(f"[bench] decode call {mean(dec_ms)*1e3:.1f} us ({dec_gbs:.0f} GB/s), split kernel "
        f"{mean(kern_ms)*1e3:.1f} us ({kern_gbs:.0f} GB/s), append {mean(append_ms)*1e3:.1f} us "
        f"({append_mtok:.1f} Mtokens/s, {append_bytes/(mean(append_ms)*1e-3)/1e9:.0f} GB/s)")

    stream_gbs = None
    if args.copy_calibration:
        # a plain streaming kernel of known traffic (reads n bytes, writes n bytes): its time
        # gives the HBM bandwidth this machine sustains, and its FETCH_SIZE / WRITE_SIZE readings
        # scale the counters of the decode kernel
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        ec = [ev.create() for _ in range(4)]
        ev.record(ec[0], stream)
        for _ in range(3):
            torch.neg(src, out=dst)
        ev.record(ec[1], stream)
        torch.cuda.synchronize()
        stream_gbs = 2 * n * 3 / (ev.elapsed_ms(ec[0], ec[1]) * 1e-3) / 1e9
        del src, dst
        log(f"[bench] streaming copy (elementwise neg, {n} bytes in + out): {stream_gbs:.0f} GB/s")

    sections = set(x for x in args.sections.split(",") if x)
    if args.no_search:
        sections = set()
    widths = None
    if "widths" in sections:
        log("[bench] key bit-width variants and logits-only ...")
        widths = key_width_bench(tq, W, w, K, V, q, dev, ev, stream)
        log(f"[bench] key widths {widths}")

    nsn = None
    if "nsn" in sections:
        log("[bench] NSN cache ...")
        nsn = nsn_bench(tq, w, K, V, q, dev, ev, stream)
        log(f"[bench] nsn {nsn}")

    polar = None
    if "polar" in sections:
        log("[bench] PolarQuant cache ...")
        polar = polar_bench(tq, w, K, V, q, dev, ev, stream)
        log(f"[bench] polar {polar}")

    window = None
    if "window" in sections:
        log("[bench] full-precision window and decode steps ...")
        window = window_bench(tq, w, K, V, q, cache, codec, dev, ev, stream)
        log(f"[bench] window {window}")

    configs = None
    if "configs" in sections:
        log("[bench] other decode workloads (llama3_8b 32 layers, esm2_650m 33 layers, single head) ...")
        configs = configs_bench(tq, W, dev, ev, stream)

    search = None
    if "search" in sections:
        log("[bench] vector search workload ...")
        search = search_bench(tq, W, dev, ev, stream)
        log(f"[bench] search {search}")

    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        base = cpu_baseline(w, K, V, q, units)
        log(f"[bench] cpu baseline {base}")

    rec = {
        "metric": "packed-KV decode attention GB/s & % HBM peak; quantize Mtokens/s",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": ("long_context: 1 layer, 64 q-heads / 8 kv-heads, head dim 128, batch 4, "
                         "context 131072, append 4096, bf16 Laplace K/V + 4 channels x20, RoPE 500000, "
                         "keys 2-bit + QJL m=128, values 3-bit"),
            "batch": w.batch, "context": T, "append_tokens": A, "q_heads": w.q_heads,
            "kv_heads": w.kv_heads, "head_dim": w.d, "decode_splits": splits,
        },
        "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(mean(dec_ms) * 1e3, 2),
        "decode_us_p10_p50_p90": pct_us(dec_ms),
        "append_us": round(mean(append_ms) * 1e3, 2),
        "append_us_p10_p50_p90": pct_us(append_ms),
        "quantize_mtokens_s": round(append_mtok, 2),
        "quantize_gbs": round(append_bytes / (mean(append_ms) * 1e-3) / 1e9, 2),
        "roofline": {
            "kernel": "k_decode_lds<128> (split-K decode over the packed cache)",
            "bound": "hbm",
            "limiter": ("instruction issue, not HBM: VALU + MFMA keep the SIMDs busy 72% of the launch "
                        "with HBM traffic 1.01x the algorithmic bytes "
                        "(profiles/decode_lds_long_context.md)"),
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_counters(dec_bytes),
            "algorithmic_bytes_per_launch": dec_bytes,
            "avg_launch_us": round(mean(kern_ms) * 1e3, 2),
            "launch_us_p10_p50_p90": pct_us(kern_ms),
            "measured_stream_copy_gbs": None if stream_gbs is None else round(stream_gbs, 1),
        },
        "cpu_baseline": base,
        "key_widths": widths,
        "window": window,
        "nsn": nsn,
        "polar": polar,
        "search": search,
        "configs": configs,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
