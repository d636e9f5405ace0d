"""Benchmark of the head-partitioned KV attention hot path on one MI355X.

Decode leg (the headline): the Llama-3-8B-shaped GQA layer at a 128K context (32 query heads,
8 KV heads, head_dim 128, bf16, 4 retrieval KV heads, sink 16 + recent 512). One step is, for
each of ``--layers`` replica layers, one append of the new token and its decode (the fused
``duo_decode_step``; ``--unfused`` times duo_kv_append + duo_attn_decode instead). The
replica layers sit at distinct addresses so that the per-step K/V (>= 2 GB) cannot stay in
the 256 MB Infinity Cache; the time per layer-step is the step time divided by the layers.

Prefill leg: the Llama-2-7B-shaped MHA layer (32 heads, 8 retrieval) pre-filling a 32K
prompt in 4K-token chunks (prefill attention of each chunk, then its append), once with the
per-query sink + recent mask on streaming heads and once with chunk-granular streaming heads
(the pruned cache before the chunk plus the chunk; ``--prefill-modes`` picks the legs).

Gate-mixed leg: the identification-phase attention of the same MHA layer over one 32K-token
sequence processed whole (every head blends its causal and sink + recent outputs).

Head-reorder leg: the one-time permutation of a Llama-3-8B-shaped model's attention
projections (2.68 GB) after binarizing its gates.

Prints one JSON line. ``value`` is the decode K/V bandwidth in GB/s (algorithmic bytes: the
K/V rows the method must read, plus q, out and the appended token). Inputs are resident in
HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s (% HBM peak) + µs/layer-step at 128K ctx; prefill TFLOP/s"
ROPE_THETA = 500000.0  # RoPE base of the Llama-3-8B-shaped workload's pre-RoPE 4-bit leg
PREFILL_ROPE_THETA = 10000.0  # Llama-2's RoPE base (the MHA prefill workload)
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=8, help="replica layers of the decode leg")
    p.add_argument("--workload", default="c3", help="decode workload key (c2, c3, c5, c5q)")
    p.add_argument("--prefill-passes", type=int, default=3)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--prefill-modes", default="window,chunk,mixed,kv4,kv4rope,gqa",
                   help="prefill legs to time: window (per-query sink + recent mask), chunk "
                        "(chunk-granular streaming heads), mixed (gate-mixed attention), kv4 "
                        "(window mode over a 4-bit cache, staged), kv4rope (the same with "
                        "pre-RoPE keys, staged turned), gqa (the prompt on the GQA layer)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-kv4", action="store_true", help="skip the 4-bit full-cache decode leg")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--splits", type=int, default=0, help="force decode splits (0 = automatic)")
    p.add_argument("--unfused", action="store_true", help="time append + decode as two calls")
    p.add_argument("--legs", default="decode,kv4,kv4rope,kv8,c4,prefill,reorder,probe,cpu",
                   help="legs to run: decode (the headline, always run), kv4 (4-bit full "
                        "caches), kv4rope (4-bit with pre-RoPE keys), kv8 (8-bit), c4 (32 layers x batch 8, ragged), prefill (the legs of "
                        "--prefill-modes), reorder, probe (read and copy bandwidth), cpu "
                        "(the oracle on the host)")
    a = p.parse_args()
    legs = set(a.legs.split(","))
    unknown = legs - {"decode", "kv4", "kv4rope", "kv8", "c4", "prefill", "reorder", "probe",
                      "cpu"}
    if unknown:
        p.error(f"unknown legs {sorted(unknown)}")
    a.no_kv4rope = a.no_kv4 or "kv4rope" not in legs
    a.no_kv8 = "kv8" not in legs
    a.no_kv4 = a.no_kv4 or "kv4" not in legs
    a.no_prefill = a.no_prefill or "prefill" not in legs
    a.no_cpu = a.no_cpu or "cpu" not in legs
    a.no_c4 = "c4" not in legs
    a.no_reorder = "reorder" not in legs
    a.no_probe = "probe" not in legs
    return a


def source_sha(name: str) -> str:
    with open(os.path.join(ROOT, "head_split_kv_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_record(kernel_file: str, key: str):
    """The rocprofv3 counter record ``key`` of profiles/traffic.json when it was taken on the
    current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(key)
    if not rec or rec.get("source_sha") != source_sha(kernel_file):
        return None
    return rec


def committed_traffic(kernel_file: str, key: str):
    """HBM bytes per launch measured with rocprofv3 counters for the current kernel source,
    or None when the counters were taken on another version of the kernel."""
    rec = committed_record(kernel_file, key)
    return None if rec is None else rec.get("bytes_per_launch")


def committed_mfma(kernel_file: str, key: str):
    """Matrix-core counters of the current kernel source (SQ_VALU_MFMA_BUSY_CYCLES against
    GRBM_GUI_ACTIVE, executed MFMA work against the algorithmic work), or None."""
    rec = committed_record(kernel_file, key)
    if rec is None or "mfma_busy_frac_active" not in rec:
        return None
    return {k: rec[k] for k in ("mfma_busy_frac_active", "mfma_busy_frac_at_peak_clock",
                                "executed_over_algorithmic", "clock_ghz")}


class Timer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def decode_leg(args, torch, hsk, W, N, kv_bits=0, rope_theta=0.0):
    w = W.workload(args.workload)
    L = args.layers
    # warm-up, the timed steps, then as many again timed one by one for the spread
    total_steps = args.warmup + 2 * args.steps
    n0 = w.context
    cap = n0 + total_steps
    mask = W.retrieval_mask(w)[0]
    dev = torch.device("cuda")
    cache = hsk.DuoCache(num_layers=L, batch=1, num_q_heads=w.hq, num_kv_heads=w.hkv,
                         head_dim=w.d, sink=w.sink, recent=w.recent, capacity=cap,
                         retrieval_mask=[mask] * L, dtype=torch.bfloat16,
                         out_dtype=torch.bfloat16, device=dev, max_splits=1024,
                         kv_bits=kv_bits, rope_theta=rope_theta)
    if args.splits:
        hsk.duo_set_decode_splits(cache, args.splits)
    t = time.time()
    chunk = 1 << 16
    for t0 in range(0, n0, chunk):
        t1 = min(n0, t0 + chunk)
        k = torch.from_numpy(W.tokens(w, "k", 0, 0, t0, t1)).to(dev).to(torch.bfloat16)
        v = torch.from_numpy(W.tokens(w, "v", 0, 0, t0, t1)).to(dev).to(torch.bfloat16)
        for layer in range(L):
            cache.kv_append(layer, k, v, seq=0)
        del k, v
    qs = torch.from_numpy(W.tokens(w, "q", 0, 0, n0, n0 + total_steps)).to(dev).to(torch.bfloat16)
    ks = torch.from_numpy(W.tokens(w, "k", 0, 0, n0, n0 + total_steps)).to(dev).to(torch.bfloat16)
    vs = torch.from_numpy(W.tokens(w, "v", 0, 0, n0, n0 + total_steps)).to(dev).to(torch.bfloat16)
    out = torch.empty((1, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    kind = (f" ({kv_bits}-bit full caches" + (", pre-RoPE keys)" if rope_theta else ")")
            if kv_bits in (4, 8) else "")
    log(f"decode leg{kind}: {w.name}, {L} replica "
        f"layers filled to {n0} tokens in {time.time() - t:.1f}s")

    lib = N.lib()
    h = cache.handle
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    qstride = w.hq * w.d * 2
    kstride = w.hkv * w.d * 2
    qp, kp, vp, op = qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), ctypes.c_void_p(out.data_ptr())
    decode, decode_step = lib.duo_attn_decode, lib.duo_decode_step

    def step(s):
        # one decoding step of every replica layer: append of the step's token fused with
        # the attention (duo_decode_step)
        kk = ctypes.c_void_p(kp + s * kstride)
        vv = ctypes.c_void_p(vp + s * kstride)
        qq = ctypes.c_void_p(qp + s * qstride)
        for layer in range(L):
            if args.unfused:
                st = lib.duo_kv_append(h, layer, -1, kk, vv, 1, stream)
                st |= decode(h, layer, qq, op, None, stream)
            else:
                st = decode_step(h, layer, qq, kk, vv, op, None, stream)
            if st:
                raise RuntimeError(f"libduo call failed: {N.status_string(st)}")

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for s in range(args.warmup, args.warmup + args.steps):
        step(s)
    total_ms = tm.stop_ms()
    torch.cuda.synchronize()
    ms_per_step = total_ms / args.steps

    # Second timed pass over the next `steps` steps: the library's kernel timers record a HIP
    # event pair on this stream around every split attention kernel (the split merge kernel
    # is outside the pair), and every step sits between its own pair of events for the
    # spread. Kept out of the pass above: the extra event records cost about 2 us per step.
    hsk.duo_timing_enable(cache, args.steps * L)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, s in enumerate(range(args.warmup + args.steps, total_steps)):
        evs[i][0].record()
        step(s)
        evs[i][1].record()
    torch.cuda.synchronize()
    kern_ms, kern_n = hsk.duo_timing_read(cache, "decode")
    hsk.duo_timing_enable(cache, 0)
    assert kern_n == args.steps * L, kern_n
    kern_us = kern_ms * 1e3 / kern_n
    import numpy as np
    per_step_us = np.array([a.elapsed_time(b) * 1e3 / L for a, b in evs])
    pct = {f"p{q}": float(np.percentile(per_step_us, q)) for q in (10, 50, 90)}

    # algorithmic bytes of one layer-step, averaged over the timed steps (the second pass,
    # 100 tokens longer, differs by less than 0.1 %)
    cfg1, _m = hsk.make_config(num_layers=1, batch=1, num_q_heads=w.hq, num_kv_heads=w.hkv,
                               head_dim=w.d, sink=w.sink, recent=w.recent, capacity=cap,
                               retrieval_mask=[mask], kv_bits=kv_bits)
    kv_bytes = []
    for s in range(args.warmup, args.warmup + args.steps):
        kv_bytes.append(hsk.duo_kv_bytes(cfg1, [n0 + s + 1], 0)[1])
    io_bytes = 2 * w.hq * w.d * 2 + 2 * 2 * w.hkv * w.d * 2  # q in, out, new K/V in + stored
    step_bytes = sum(kv_bytes) / len(kv_bytes) + io_bytes
    us_layer = ms_per_step * 1e3 / L
    gbs = step_bytes / (us_layer * 1e-6) / 1e9
    kern_gbs = step_bytes / (kern_us * 1e-6) / 1e9

    # one duo_attn_decode call (split kernel + merge kernel), back-to-back over the replica
    # layers at the final length
    reps = max(4, 64 // L)
    for layer in range(L):
        decode(h, layer, ctypes.c_void_p(qp), op, None, stream)
    torch.cuda.synchronize()
    tm.start()
    for _ in range(reps):
        for layer in range(L):
            decode(h, layer, ctypes.c_void_p(qp), op, None, stream)
    dec_ms = tm.stop_ms() / (reps * L)
    n_final = n0 + total_steps
    dec_bytes = hsk.duo_kv_bytes(cfg1, [n_final], 0)[1] + 2 * w.hq * w.d * 2
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    result = dict(
        workload=w, layers=L, ms_per_step=ms_per_step, us_layer=us_layer, gbs=gbs,
        step_bytes=step_bytes, dec_us=dec_ms * 1e3, dec_bytes=dec_bytes, dec_gbs=dec_gbs,
        kern_us=kern_us, kern_gbs=kern_gbs, kern_n=kern_n, step_pct=pct,
        n_final=n_final, history=(n0, total_steps))
    del cache, qs, ks, vs
    torch.cuda.empty_cache()
    return result


STAGED_PATH = ("duo_attn_prefill_staged on the bf16 cache: the values each chunk reads (retrieval "
               "prefix, chunk, streaming caches) converted to fp16 copies in caller staging by a "
               "separate kernel, whose time attn_ms includes; the kernel figures cover "
               "prefill_kernel alone. Outputs bit-identical to duo_attn_prefill (below).")


def prefill_leg(args, torch, hsk, W, N, mode="window", kv_bits=0, rope_theta=0.0, gqa=False,
                v16=False):
    """The 32K MHA prompt in 4K chunks; with v16 through duo_attn_prefill_staged on the bf16
    cache (the values the chunk reads converted to fp16 copies in staging first, which the
    calls' time includes; the kernel timers cover the prefill kernel alone); with kv_bits 4
    over a 4-bit cache (duo_attn_prefill_staged: the retrieval prefix read back into staging,
    keys in bf16 and values in fp16, the chunk's and streaming values in fp16 beside them,
    then the prefill kernel; the kernel timers cover it alone); with rope_theta the
    cache holds pre-RoPE keys, and every key the chunk reads is staged turned. With gqa the
    same 32K prompt in 4K chunks on the Llama-3-8B-shaped GQA layer (32 q / 8 KV heads, 4
    retrieval)."""
    w = W.workload("c2")
    if gqa:
        w = W.workload("c3").with_(prefill_len=w.prefill_len, prefill_chunk=w.prefill_chunk)
    mask = W.retrieval_mask(w)[0]
    dev = torch.device("cuda")
    P, C = w.prefill_len, w.prefill_chunk
    cache = hsk.DuoCache(num_layers=1, batch=1, num_q_heads=w.hq, num_kv_heads=w.hkv,
                         head_dim=w.d, sink=w.sink, recent=w.recent, capacity=P,
                         retrieval_mask=[mask], dtype=torch.bfloat16, out_dtype=torch.bfloat16,
                         streaming_prefill=mode, device=dev, kv_bits=kv_bits,
                         rope_theta=rope_theta)
    staged = kv_bits in (4, 8) or v16
    # the largest staging of the pass (the last chunk's), as duo_prefill_staging_bytes gives it
    up = lambda x: (x + 255) // 256 * 256
    row = w.d * 2
    chunk_b = C * w.hkv * row
    str_b = int((mask == 0).sum()) * (w.sink + w.recent) * row
    end = (1 if v16 else 2) * int(mask.sum()) * P * row  # read-backs (bf16 cache: fp16 values)
    if rope_theta:
        end = up(end) + up(chunk_b) + str_b
    need = up(end) + up(chunk_b) + str_b  # the chunk's and the streaming values in fp16
    staging = torch.empty(need if staged else 16, dtype=torch.uint8, device=dev)
    q = torch.from_numpy(W.tokens(w, "q", 0, 0, 0, P)).to(dev).to(torch.bfloat16)
    k = torch.from_numpy(W.tokens(w, "k", 0, 0, 0, P)).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(W.tokens(w, "v", 0, 0, 0, P)).to(dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    lib = N.lib()
    h = cache.handle
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rs = w.hq * w.d * 2
    ks = w.hkv * w.d * 2

    def run_pass(timer_attn=None):
        hsk.duo_cache_reset(cache)
        attn_ms = 0.0
        for c0 in range(0, P, C):
            if timer_attn is not None:
                timer_attn.start()
            qq = ctypes.c_void_p(q.data_ptr() + c0 * rs)
            kk = ctypes.c_void_p(k.data_ptr() + c0 * ks)
            vv = ctypes.c_void_p(v.data_ptr() + c0 * ks)
            oo = ctypes.c_void_p(out.data_ptr() + c0 * rs)
            if staged:
                st = lib.duo_attn_prefill_staged(h, 0, 0, qq, kk, vv, C, oo, None,
                                                 ctypes.c_void_p(staging.data_ptr()),
                                                 staging.numel(), stream)
            else:
                st = lib.duo_attn_prefill(h, 0, 0, qq, kk, vv, C, oo, None, stream)
            if timer_attn is not None:
                attn_ms += timer_attn.stop_ms()
            if st:
                raise RuntimeError(f"prefill failed: {N.status_string(st)}")
            st = lib.duo_kv_append(h, 0, 0, ctypes.c_void_p(k.data_ptr() + c0 * ks),
                                   ctypes.c_void_p(v.data_ptr() + c0 * ks), C, stream)
            if st:
                raise RuntimeError(f"append failed: {N.status_string(st)}")
        return attn_ms

    run_pass()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(args.prefill_passes):
        run_pass()
    pass_ms = tm.stop_ms() / args.prefill_passes
    # attention calls alone (events around each call), with the kernel timers around each
    # attention kernel launch
    hsk.duo_timing_enable(cache, args.prefill_passes * (P // C))
    attn = []
    for _ in range(args.prefill_passes):
        attn.append(run_pass(Timer(torch)))
    attn_ms = sum(attn) / len(attn)
    kern_ms, kern_n = hsk.duo_timing_read(cache, "prefill")
    hsk.duo_timing_enable(cache, 0)
    assert kern_n == args.prefill_passes * (P // C), kern_n
    kern_ms_pass = kern_ms / args.prefill_passes
    # algorithmic flops: 4 d per visible (query, key) pair; query p sees p + 1 keys on a
    # retrieval head and, on a streaming head, min(p + 1, S + R) (window mode) or the
    # min(c, S + R) held tokens plus p - c + 1 chunk tokens (chunk mode, chunk starting at c)
    S, R = w.sink, w.recent
    hr = int(mask.sum())
    hs = w.hkv - hr
    pairs_ret = P * (P + 1) // 2
    if mode == "chunk":
        pairs_str = sum(min(p - p % C, S + R) + p % C + 1 for p in range(P))
    else:
        pairs_str = sum(min(p + 1, S + R) for p in range(P))
    flops = 4 * w.d * (hr * pairs_ret + hs * pairs_str) * (w.hq // w.hkv)
    del cache, q, k, v, out, staging
    torch.cuda.empty_cache()
    return dict(workload=w, pass_ms=pass_ms, attn_ms=attn_ms, flops=flops,
                tflops=flops / (attn_ms * 1e-3) / 1e12, kern_ms=kern_ms_pass,
                kern_tflops=flops / (kern_ms_pass * 1e-3) / 1e12,
                tflops_incl_append=flops / (pass_ms * 1e-3) / 1e12)


def gate_mixed_leg(args, torch, hsk, W, N):
    """Identification-phase attention: a Llama-2-7B-shaped MHA layer (32 heads, d 128, sink 16
    + recent 512) over one 32,768-token sequence processed whole, every head blending its
    causal and sink + recent outputs by a gate drawn in [0, 1]."""
    import numpy as np
    w = W.workload("c2")
    T, H, d = w.prefill_len, w.hq, w.d
    dev = torch.device("cuda")
    cache = hsk.DuoCache(num_layers=1, batch=1, num_q_heads=H, num_kv_heads=H, head_dim=d,
                         sink=w.sink, recent=w.recent, capacity=T,
                         retrieval_mask=[np.ones(H, dtype=np.uint8)], dtype=torch.bfloat16,
                         out_dtype=torch.bfloat16, device=dev)
    q, k, v = (torch.from_numpy(W.tokens(w, t, 0, 0, 0, T)).to(dev).to(torch.bfloat16)
               for t in "qkv")
    out = torch.empty_like(q)
    alpha = np.random.default_rng(91).random(H).astype(np.float32)
    lib = N.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pa = alpha.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    args_ = (cache.handle, 0, 0, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
             ctypes.c_void_p(v.data_ptr()), T)

    def mixed():
        st = lib.duo_attn_gate_mixed(*args_, pa, ctypes.c_void_p(out.data_ptr()), stream)
        if st:
            raise RuntimeError(f"gate-mixed failed: {N.status_string(st)}")

    def full():
        st = lib.duo_attn_prefill(*args_, ctypes.c_void_p(out.data_ptr()), None, stream)
        if st:
            raise RuntimeError(f"prefill failed: {N.status_string(st)}")

    reps = max(2, args.prefill_passes)
    res = {}
    for name, fn in (("mixed", mixed), ("full", full)):
        fn()
        torch.cuda.synchronize()
        tm = Timer(torch)
        tm.start()
        for _ in range(reps):
            fn()
        res[name] = tm.stop_ms() / reps
    S, R = w.sink, w.recent
    pairs_full = T * (T + 1) // 2
    pairs_str = sum(min(p + 1, S + R) for p in range(T))
    flops = 4 * d * H * (pairs_full + pairs_str)
    del cache, q, k, v, out
    torch.cuda.empty_cache()
    return dict(workload=w, ms=res["mixed"], full_ms=res["full"], flops=flops,
                tflops=flops / (res["mixed"] * 1e-3) / 1e12,
                full_tflops=4 * d * H * pairs_full / (res["full"] * 1e-3) / 1e12)


def reorder_leg(args, torch, hsk, N):
    """One-time head reordering of a Llama-3-8B-shaped model's attention projections: gates
    of 32 layers x 8 KV heads binarized at 50 %, then every layer's Q, K, V rows and output
    projection columns permuted on the GPU (128 launches, 2.68 GB of bf16 weights, each byte
    read and written once)."""
    import numpy as np
    L, Hkv, G, d, hidden = 32, 8, 4, 128, 4096
    Hq = Hkv * G
    rng = np.random.default_rng(5)
    alpha = np.clip(rng.normal(0.3, 0.3, (L, Hkv)), 0, 1).astype(np.float32)
    mask, _, n_ret = hsk.duo_binarize_gates(alpha, 0.5)
    orders = [hsk.duo_head_order(mask[layer], G) for layer in range(L)]
    shapes = [(Hq * d, hidden), (Hkv * d, hidden), (Hkv * d, hidden), (hidden, Hq * d)]
    src = [[torch.randn(s, device="cuda", dtype=torch.bfloat16) for s in shapes] for _ in range(L)]
    dst = [[torch.empty_like(t) for t in layer] for layer in src]
    # the first pass goes through the binding (its checks), the timed ones through the C
    # calls with prepared arguments
    for layer in range(L):
        kv_o, q_o = orders[layer]
        for t, (o, nb, bb, order) in enumerate([(1, Hq, d * hidden * 2, q_o),
                                                (1, Hkv, d * hidden * 2, kv_o),
                                                (1, Hkv, d * hidden * 2, kv_o),
                                                (hidden, Hq, d * 2, q_o)]):
            hsk.duo_permute_blocks(src[layer][t], dst[layer][t], o, nb, bb, order)
    lib = hsk.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P32 = ctypes.POINTER(ctypes.c_int32)
    keep = [(np.ascontiguousarray(kv, dtype=np.int32), np.ascontiguousarray(q, dtype=np.int32))
            for kv, q in orders]
    calls = []
    for layer in range(L):
        kv_o, q_o = (a.ctypes.data_as(P32) for a in keep[layer])
        for t, (o, nb, bb, order) in enumerate([(1, Hq, d * hidden * 2, q_o),
                                                (1, Hkv, d * hidden * 2, kv_o),
                                                (1, Hkv, d * hidden * 2, kv_o),
                                                (hidden, Hq, d * 2, q_o)]):
            calls.append((ctypes.c_void_p(src[layer][t].data_ptr()),
                          ctypes.c_void_p(dst[layer][t].data_ptr()), o, nb, bb, order, t))

    def run(only=None):
        for s_, d_, o, nb, bb, order, t in calls:
            if only is None or t == only:
                st = lib.duo_permute_blocks(s_, d_, o, nb, bb, order, stream)
                if st:
                    raise RuntimeError(f"permute failed: {N.status_string(st)}")

    run()
    torch.cuda.synchronize()
    tm = Timer(torch)
    reps = 5
    tm.start()
    for _ in range(reps):
        run()
    ms = tm.stop_ms() / reps
    nbytes = sum(t.numel() * 2 for layer in src for t in layer)
    # the output projection alone (column blocks of 256 bytes), timed the same way
    tm.start()
    for _ in range(reps):
        run(only=3)
    ms_o = tm.stop_ms() / reps
    o_bytes = sum(layer[3].numel() * 2 for layer in src)
    del src, dst
    torch.cuda.empty_cache()
    return dict(ms=ms, bytes=nbytes, gbs=2 * nbytes / (ms * 1e-3) / 1e9, n_ret=n_ret,
                o_gbs=2 * o_bytes / (ms_o * 1e-3) / 1e9)


def c4_leg(args, torch, hsk, N):
    """Full-depth GQA decode: 32 layers of the Llama-3-8B-shaped head layout (32 q / 8 kv
    heads, d 128, bf16, sink 16 + recent 512, per-layer retrieval masks at 50 %), batch 8 with
    ragged contexts drawn in [16K, 32K]. One step is the fused append + decode
    (duo_decode_step) of every layer for all 8 sequences: one whole-model attention step.
    K/V/q come from a seeded device generator (torch.randn, seed 4000 + 64 layer + b for the
    fill; the step tokens from seed 4999), rounded once to bf16."""
    import numpy as np
    import workloads as W
    w = W.workload("c4")
    lens0 = [int(x) for x in W.initial_lengths(w)]
    masks = W.retrieval_mask(w)
    L, B = w.layers, w.batch
    total_steps = args.warmup + 2 * args.steps
    cap = max(lens0) + total_steps
    dev = torch.device("cuda")
    cache = hsk.DuoCache(num_layers=L, batch=B, num_q_heads=w.hq, num_kv_heads=w.hkv,
                         head_dim=w.d, sink=w.sink, recent=w.recent, capacity=cap,
                         retrieval_mask=masks, dtype=torch.bfloat16, out_dtype=torch.bfloat16,
                         device=dev, max_splits=1024)
    gen = torch.Generator(device=dev)
    t = time.time()
    for layer in range(L):
        for b, n in enumerate(lens0):
            gen.manual_seed(4000 + 64 * layer + b)
            k = torch.randn((n, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
            v = torch.randn((n, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
            cache.kv_append(layer, k, v, seq=b)
            del k, v
    gen.manual_seed(4999)
    qs = torch.randn((total_steps, B, w.hq, w.d), generator=gen, device=dev).to(torch.bfloat16)
    ks = torch.randn((total_steps, B, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    vs = torch.randn((total_steps, B, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"c4 leg: {L} layers x batch {B}, lengths {lens0}, filled in {time.time() - t:.1f}s")
    lib = N.lib()
    h = cache.handle
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    qstride, kstride = B * w.hq * w.d * 2, B * w.hkv * w.d * 2
    qp, kp, vp, op = qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), ctypes.c_void_p(out.data_ptr())
    decode_step = lib.duo_decode_step

    def step(s):
        qq = ctypes.c_void_p(qp + s * qstride)
        kk = ctypes.c_void_p(kp + s * kstride)
        vv = ctypes.c_void_p(vp + s * kstride)
        for layer in range(L):
            st = decode_step(h, layer, qq, kk, vv, op, None, stream)
            if st:
                raise RuntimeError(f"libduo call failed: {N.status_string(st)}")

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for s in range(args.warmup, args.warmup + args.steps):
        step(s)
    ms_per_step = tm.stop_ms() / args.steps
    # second pass: kernel timers around every split attention kernel, events around each step
    hsk.duo_timing_enable(cache, args.steps * L)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, s in enumerate(range(args.warmup + args.steps, total_steps)):
        evs[i][0].record()
        step(s)
        evs[i][1].record()
    torch.cuda.synchronize()
    kern_ms, kern_n = hsk.duo_timing_read(cache, "decode")
    hsk.duo_timing_enable(cache, 0)
    assert kern_n == args.steps * L, kern_n
    kern_ms_step = kern_ms / args.steps
    per_step = np.array([a.elapsed_time(b) for a, b in evs])
    pct = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    # algorithmic bytes of a whole-model step (every layer, every sequence), averaged over the
    # first pass's steps; the second pass is args.steps tokens longer (< 0.1 % more bytes)
    cfg, _m = hsk.make_config(num_layers=L, batch=B, num_q_heads=w.hq, num_kv_heads=w.hkv,
                              head_dim=w.d, sink=w.sink, recent=w.recent, capacity=cap,
                              retrieval_mask=masks)
    io_layer = 2 * B * w.hq * w.d * 2 + 2 * 2 * B * w.hkv * w.d * 2
    tot = []
    for s in range(args.warmup, args.warmup + args.steps):
        lens = [n + s + 1 for n in lens0]
        tot.append(sum(hsk.duo_kv_bytes(cfg, lens, layer)[1] for layer in range(L)) + L * io_layer)
    step_bytes = float(np.mean(tot))
    full_bytes = sum(hsk.duo_kv_bytes(cfg, [n + args.warmup + 1 for n in lens0], layer)[0]
                     for layer in range(L))
    del cache, qs, ks, vs
    torch.cuda.empty_cache()
    return dict(workload=w, lens0=lens0, ms_per_step=ms_per_step, step_bytes=step_bytes,
                gbs=step_bytes / (ms_per_step * 1e-3) / 1e9, kern_ms_step=kern_ms_step,
                kern_gbs=step_bytes / (kern_ms_step * 1e-3) / 1e9, step_pct=pct,
                full_bytes=full_bytes)


def read_probe(torch, hsk):
    """Read bandwidth of a plain streaming-read kernel (duo_read_probe): 8 buffers of the 128K
    decode layer's size (270 MB, 2.16 GB in all, so the Infinity Cache cannot hold them) read
    round-robin, and one 2 GiB buffer, at several grid sizes; the best rate of each."""
    res = {}
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, nbytes, nbuf in (("270MB", 269_573_120, 8), ("2GiB", 1 << 31, 1)):
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
        best = None
        for blocks in (512, 1024, 2048, 4096):
            for bf in bufs:
                hsk.duo_read_probe(bf, flag, blocks)
            torch.cuda.synchronize()
            tm = Timer(torch)
            reps = 4 * nbuf if nbuf > 1 else 6
            tm.start()
            for i in range(reps):
                hsk.duo_read_probe(bufs[i % nbuf], flag, blocks)
            us = tm.stop_ms() * 1e3 / reps
            gbs = nbytes / (us * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, us, blocks)
        res[name] = {"GBps": round(best[0], 1), "us": round(best[1], 3), "blocks": best[2]}
        del bufs
        torch.cuda.empty_cache()
    return res


def copy_probe(torch):
    """Achievable HBM bandwidth of a plain device copy (read + write bytes)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(10):
        b.copy_(a)
    ms = tm.stop_ms() / 10
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def blas_threads() -> int:
    """Threads numpy's BLAS runs with (the oracle's matrix products are its only parallel
    part)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def host_cores() -> dict:
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = None
    return {"cpu_count": os.cpu_count(), "affinity_cpus": aff, "blas_threads": blas_threads(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(args, W, w, n):
    """The float64 oracle decoding one step of the same layer on the host's cores."""
    import numpy as np
    from oracle import duo_oracle as O
    threads = blas_threads()
    mask = W.retrieval_mask(w)[0]
    k = W.tokens(w, "k", 0, 0, 0, n)
    v = W.tokens(w, "v", 0, 0, 0, n)
    q = W.tokens(w, "q", 0, 0, n - 1, n)[0]
    t = time.time()
    calls = 0
    while True:
        O.decode_step(q, k, v, mask, w.sink, w.recent)
        calls += 1
        if time.time() - t > args.cpu_seconds:
            break
    sec = (time.time() - t) / calls
    return dict(sec_per_step=sec, calls=calls, threads=threads)


def cpu_prefill_sample(args, W):
    """The float64 oracle pre-filling a sample of the 32K MHA prompt on the host's cores: the
    last 64 queries of the third 4K chunk (positions 12,224..12,287), all 32 heads."""
    from oracle import duo_oracle as O
    w = W.workload("c2")
    mask = W.retrieval_mask(w)[0]
    start, m = 12224, 64
    k = W.tokens(w, "k", 0, 0, 0, start + m)
    v = W.tokens(w, "v", 0, 0, 0, start + m)
    q = W.tokens(w, "q", 0, 0, start, start + m)
    t = time.time()
    O.prefill_chunk(q, k, v, start, mask, w.sink, w.recent)
    sec = time.time() - t
    S, R = w.sink, w.recent
    hr = int(mask.sum())
    pairs = sum(hr * (p + 1) + (w.hkv - hr) * min(p + 1, S + R) for p in range(start, start + m))
    flops = 4 * w.d * pairs * (w.hq // w.hkv)
    return dict(sec=sec, flops=flops, tflops=flops / sec / 1e12)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    import head_split_kv_amd as hsk
    from head_split_kv_amd import _native as N
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dec = decode_leg(args, torch, hsk, W, N)
    log(f"decode: {dec['us_layer']:.2f} us/layer-step, {dec['gbs']:.0f} GB/s; split kernel "
        f"{dec['kern_us']:.2f} us = {dec['kern_gbs']:.0f} GB/s ({dec['kern_n']} launches timed); "
        f"one duo_attn_decode call {dec['dec_us']:.2f} us = {dec['dec_gbs']:.0f} GB/s")
    dec4 = None
    if not args.no_kv4:
        dec4 = decode_leg(args, torch, hsk, W, N, kv_bits=4)
        log(f"decode, 4-bit full caches: {dec4['us_layer']:.2f} us/layer-step "
            f"({dec['us_layer'] / dec4['us_layer']:.2f}x the bf16 step), {dec4['gbs']:.0f} GB/s of "
            f"stored bytes; split kernel {dec4['kern_us']:.2f} us = {dec4['kern_gbs']:.0f} GB/s; "
            f"one duo_attn_decode call {dec4['dec_us']:.2f} us")
    dec8 = None
    if not args.no_kv8:
        dec8 = decode_leg(args, torch, hsk, W, N, kv_bits=8)
        log(f"decode, 8-bit full caches: {dec8['us_layer']:.2f} us/layer-step "
            f"({dec['us_layer'] / dec8['us_layer']:.2f}x the bf16 step), {dec8['gbs']:.0f} GB/s of "
            f"stored bytes; split kernel {dec8['kern_us']:.2f} us = {dec8['kern_gbs']:.0f} GB/s; "
            f"one duo_attn_decode call {dec8['dec_us']:.2f} us")
    dec4r = None
    if not args.no_kv4rope:
        dec4r = decode_leg(args, torch, hsk, W, N, kv_bits=4, rope_theta=ROPE_THETA)
        log(f"decode, 4-bit full caches with pre-RoPE keys: {dec4r['us_layer']:.2f} "
            f"us/layer-step, {dec4r['gbs']:.0f} GB/s of stored bytes; split kernel "
            f"{dec4r['kern_us']:.2f} us = {dec4r['kern_gbs']:.0f} GB/s; one duo_attn_decode "
            f"call {dec4r['dec_us']:.2f} us")
    modes = set(args.prefill_modes.split(","))
    # a failing leg ends the run with an error (no leg is dropped from the line silently)
    # the window, chunk and GQA legs time both paths of a bf16 cache: duo_attn_prefill_staged
    # with the values staged as fp16 copies (the line's figures, staging included) and
    # duo_attn_prefill (the V tiles converted in LDS)
    def both(label, **kw):
        r16 = prefill_leg(args, torch, hsk, W, N, v16=True, **kw)
        r = prefill_leg(args, torch, hsk, W, N, **kw)
        for tag, x in (("values staged as fp16", r16), ("duo_attn_prefill", r)):
            log(f"{label} ({tag}): {x['attn_ms']:.3f} ms attention for {x['flops'] / 1e12:.3f} "
                f"TFLOP = {x['tflops']:.1f} TFLOP/s; attention kernel {x['kern_ms']:.3f} ms = "
                f"{x['kern_tflops']:.1f} TFLOP/s")
        return r16, r

    pre = pre_plain = None
    if not args.no_prefill and "window" in modes:
        pre, pre_plain = both("prefill")
    pre_chunk = pre_chunk_plain = None
    if not args.no_prefill and "chunk" in modes:
        pre_chunk, pre_chunk_plain = both("prefill, chunk-granular streaming heads", mode="chunk")
    pre_gqa = pre_gqa_plain = None
    if not args.no_prefill and "gqa" in modes:
        pre_gqa, pre_gqa_plain = both("prefill, GQA layer", gqa=True)
    pre_kv4 = None
    if not args.no_prefill and "kv4" in modes:
        pre_kv4 = prefill_leg(args, torch, hsk, W, N, kv_bits=4)
        log(f"prefill over a 4-bit cache: {pre_kv4['attn_ms']:.3f} ms attention (read-back "
            f"included) = {pre_kv4['tflops']:.1f} TFLOP/s; attention kernel "
            f"{pre_kv4['kern_ms']:.3f} ms = {pre_kv4['kern_tflops']:.1f} TFLOP/s")
    pre_kv4r = None
    if not args.no_prefill and "kv4rope" in modes:
        pre_kv4r = prefill_leg(args, torch, hsk, W, N, kv_bits=4, rope_theta=PREFILL_ROPE_THETA)
        log(f"prefill over a 4-bit cache with pre-RoPE keys: {pre_kv4r['attn_ms']:.3f} ms "
            f"attention (staging included) = {pre_kv4r['tflops']:.1f} TFLOP/s; attention kernel "
            f"{pre_kv4r['kern_ms']:.3f} ms = {pre_kv4r['kern_tflops']:.1f} TFLOP/s")
    mix = None
    if not args.no_prefill and "mixed" in modes:
        mix = gate_mixed_leg(args, torch, hsk, W, N)
        log(f"gate-mixed: {mix['ms']:.3f} ms for {mix['flops'] / 1e12:.3f} TFLOP = "
            f"{mix['tflops']:.1f} TFLOP/s; the causal pass alone {mix['full_ms']:.3f} ms = "
            f"{mix['full_tflops']:.1f} TFLOP/s")
    c4 = None
    if not args.no_c4:
        c4 = c4_leg(args, torch, hsk, N)
        log(f"c4: {c4['ms_per_step'] * 1e3:.1f} us per whole-model step, {c4['gbs']:.0f} GB/s; "
            f"split kernels {c4['kern_ms_step'] * 1e3:.1f} us per step = {c4['kern_gbs']:.0f} GB/s")
    reo = None
    if not args.no_reorder:
        reo = reorder_leg(args, torch, hsk, N)
        log(f"reorder: {reo['ms']:.3f} ms for {reo['bytes'] / 1e9:.2f} GB of projections = "
            f"{reo['gbs']:.0f} GB/s (read + write); output projections alone {reo['o_gbs']:.0f} GB/s")
    probe = rprobe = None
    if not args.no_probe:
        probe = copy_probe(torch)
        rprobe = read_probe(torch, hsk)
        log(f"probes: device copy {probe:.0f} GB/s (read + write); streaming read {rprobe}")
    w = dec["workload"]
    cpu = cpu_pre = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, W, w, w.context)
        log(f"oracle: {cpu['sec_per_step']:.3f} s per decode step on {cpu['threads']} threads")
        cpu_pre = cpu_prefill_sample(args, W)
        log(f"oracle prefill sample: {cpu_pre['sec']:.2f} s, {cpu_pre['tflops'] * 1e3:.3f} GFLOP/s")
    cores = host_cores()
    traffic = committed_traffic("decode.hip", f"decode_{args.workload}")

    def plain_obj(x, traffic_key):
        """The same prompt through duo_attn_prefill (each V tile converted in LDS)."""
        o = {"attn_ms": round(x["attn_ms"], 3), "tflops": round(x["tflops"], 1),
             "kernel_ms_per_pass": round(x["kern_ms"], 3),
             "kernel_tflops": round(x["kern_tflops"], 1),
             "frac": round(x["kern_tflops"] / BF16_PEAK_TFLOPS, 4)}
        if traffic_key:
            o["traffic"] = committed_traffic("prefill.hip", traffic_key)
            o["mfma_counters"] = committed_mfma("prefill.hip", traffic_key + "_mfma")
        return o

    out = {
        "metric": METRIC,
        "value": round(dec["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16; no dataset)",
        "config": {
            "workload": f"{w.name}: decode, 1 sequence, {w.hq} q / {w.hkv} kv heads, d={w.d}, "
                        f"{w.n_retrieval} retrieval kv heads, sink {w.sink} + recent {w.recent}, "
                        f"context {w.context}; step = append+decode on {dec['layers']} replica "
                        f"layers",
            "context": w.context, "replica_layers": dec["layers"], "global_batch": 1,
        },
        "us_per_layer_step": round(dec["us_layer"], 3),
        "us_per_layer_step_spread": {k: round(v, 3) for k, v in dec["step_pct"].items()},
        "hbm_frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
        "decode_call_us": round(dec["dec_us"], 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(dec["kern_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["kern_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "decode_kernel<bf16, d128, G4> (split attention kernel of duo_decode_step)",
            "kernel_us": round(dec["kern_us"], 3),
            "algorithmic_bytes_per_launch": int(dec["step_bytes"]),
        },
        "hbm_copy_probe_GBps": None if probe is None else round(probe, 1),
        "hbm_read_probe": None if rprobe is None else dict(
            rprobe, what="duo_read_probe: non-temporal 16-byte loads and nothing else, best of "
                         "512..4096 blocks; 270MB = 8 buffers of the 128K layer's K/V size read "
                         "round-robin (2.16 GB, beyond the Infinity Cache), 2GiB = one buffer"),
        "c4": None if c4 is None else {
            "workload": f"{c4['workload'].name}: 32 layers x batch 8, ragged contexts "
                        f"{min(c4['lens0'])}..{max(c4['lens0'])} (seeded), 32 q / 8 kv heads, "
                        f"d=128, bf16, per-layer retrieval masks at 50 %, sink 16 + recent 512; "
                        f"step = append+decode of every layer (one whole-model attention step)",
            "initial_lengths": c4["lens0"],
            "us_per_model_step": round(c4["ms_per_step"] * 1e3, 2),
            "us_per_model_step_spread": {k: round(v * 1e3, 2) for k, v in c4["step_pct"].items()},
            "GBps": round(c4["gbs"], 1),
            "hbm_frac": round(c4["gbs"] / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_model_step": int(c4["step_bytes"]),
            "full_attention_kv_bytes": int(c4["full_bytes"]),
            "roofline": {"bound": "hbm", "achieved": round(c4["kern_gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(c4["kern_gbs"] / HBM_PEAK_GBS, 4),
                         "kernel": "decode_kernel<bf16, d128, G4>, 32 launches per step",
                         "kernel_us_per_model_step": round(c4["kern_ms_step"] * 1e3, 2)},
        },
        "decode_kv4": None if dec4 is None else {
            "workload": "the same 128K GQA decode with 4-bit full caches (keys per channel over "
                        "128-token groups, values per token, bf16 residual group)",
            "us_per_layer_step": round(dec4["us_layer"], 3),
            "speedup_vs_bf16_step": round(dec["us_layer"] / dec4["us_layer"], 3),
            "GBps": round(dec4["gbs"], 1),
            "stored_bytes_per_layer_step": int(dec4["step_bytes"]),
            "decode_call_us": round(dec4["dec_us"], 3),
            "roofline": {"bound": "hbm", "achieved": round(dec4["kern_gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dec4["kern_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": committed_traffic("decode.hip", f"decode_kv4_{args.workload}"),
                         "kernel": "decode_q4_kernel<d128, G4> (split attention kernel)",
                         "kernel_us": round(dec4["kern_us"], 3)},
        },
        "decode_kv8": None if dec8 is None else {
            "workload": "the same 128K GQA decode with 8-bit full caches (the 4-bit scheme with "
                        "255 levels)",
            "us_per_layer_step": round(dec8["us_layer"], 3),
            "speedup_vs_bf16_step": round(dec["us_layer"] / dec8["us_layer"], 3),
            "GBps": round(dec8["gbs"], 1),
            "stored_bytes_per_layer_step": int(dec8["step_bytes"]),
            "decode_call_us": round(dec8["dec_us"], 3),
            "roofline": {"bound": "hbm", "achieved": round(dec8["kern_gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dec8["kern_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": committed_traffic("decode.hip", f"decode_kv8_{args.workload}"),
                         "kernel": "decode_q4_kernel<d128, G4, 8-bit> (split attention kernel)",
                         "kernel_us": round(dec8["kern_us"], 3)},
        },
        "decode_kv4_rope": None if dec4r is None else {
            "workload": "the same 4-bit decode with pre-RoPE keys (base 500,000): every key "
                        "turned at its own position inside the kernel, after dequantization on "
                        "retrieval heads, as stored on streaming heads",
            "us_per_layer_step": round(dec4r["us_layer"], 3),
            "GBps": round(dec4r["gbs"], 1),
            "stored_bytes_per_layer_step": int(dec4r["step_bytes"]),
            "decode_call_us": round(dec4r["dec_us"], 3),
            "roofline": {"bound": "hbm", "achieved": round(dec4r["kern_gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dec4r["kern_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": None,
                         "kernel": "decode_q4_kernel<d128, G4, pre-RoPE> (split attention kernel)",
                         "kernel_us": round(dec4r["kern_us"], 3)},
        },
        "gate_mixed": None if mix is None else {
            "workload": "identification-phase attention: Llama-2-7B-shaped MHA layer, one "
                        "32,768-token sequence processed whole, every head blending causal and "
                        "sink 16 + recent 512 outputs by its gate",
            "ms": round(mix["ms"], 3), "tflops": round(mix["tflops"], 1),
            "frac": round(mix["tflops"] / BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": int(mix["flops"]),
            "causal_pass_alone_ms": round(mix["full_ms"], 3),
            "causal_pass_alone_tflops": round(mix["full_tflops"], 1),
        },
        "head_reorder": None if reo is None else {
            "workload": "Llama-3-8B-shaped attention projections, 32 layers (Q, K, V rows and "
                        "output-projection columns, bf16), heads ordered by gates binarized at "
                        f"50 % ({reo['n_ret']} of 256 KV heads retrieval)",
            "ms": round(reo["ms"], 3), "bytes": int(reo["bytes"]),
            "GBps": round(reo["gbs"], 1), "frac": round(reo["gbs"] / HBM_PEAK_GBS, 4),
            "output_projection_GBps": round(reo["o_gbs"], 1),
        },
        "prefill": None if pre is None else {
            "workload": f"{pre['workload'].name}: 32K prompt in 4K chunks",
            "path": STAGED_PATH,
            "attn_ms": round(pre["attn_ms"], 3),
            "ms_incl_append": round(pre["pass_ms"], 3),
            "tflops": round(pre["tflops"], 1),
            "roofline": {"bound": "mfma", "achieved": round(pre["kern_tflops"], 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre["kern_tflops"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": committed_traffic("prefill.hip", "prefill_c2_v16"),
                         "mfma_counters": committed_mfma("prefill.hip", "prefill_c2_v16_mfma"),
                         "kernel": "prefill_kernel<d128, G1, fp16 values> (8 launches per pass)",
                         "kernel_ms_per_pass": round(pre["kern_ms"], 3),
                         "algorithmic_flops": int(pre["flops"])},
            "duo_attn_prefill": plain_obj(pre_plain, "prefill_c2"),
        },
        "prefill_kv4": None if pre_kv4 is None else {
            "workload": f"{pre_kv4['workload'].name}: 32K prompt in 4K chunks over 4-bit full "
                        f"caches (retrieval prefix read back into staging per chunk, keys in "
                        f"bf16, values and the chunk's and streaming values in fp16)",
            "attn_ms": round(pre_kv4["attn_ms"], 3),
            "ms_incl_append": round(pre_kv4["pass_ms"], 3),
            "tflops": round(pre_kv4["tflops"], 1),
            "kernel_ms_per_pass": round(pre_kv4["kern_ms"], 3),
            "kernel_tflops": round(pre_kv4["kern_tflops"], 1),
            "frac": round(pre_kv4["kern_tflops"] / BF16_PEAK_TFLOPS, 4),
        },
        "prefill_kv4_rope": None if pre_kv4r is None else {
            "workload": f"{pre_kv4r['workload'].name}: 32K prompt in 4K chunks over 4-bit full "
                        f"caches holding pre-RoPE keys (base 10,000): values read back and "
                        f"every key the chunk reads turned, into staging per chunk (keys "
                        f"bf16, values fp16)",
            "attn_ms": round(pre_kv4r["attn_ms"], 3),
            "ms_incl_append": round(pre_kv4r["pass_ms"], 3),
            "tflops": round(pre_kv4r["tflops"], 1),
            "kernel_ms_per_pass": round(pre_kv4r["kern_ms"], 3),
            "kernel_tflops": round(pre_kv4r["kern_tflops"], 1),
            "frac": round(pre_kv4r["kern_tflops"] / BF16_PEAK_TFLOPS, 4),
        },
        "prefill_chunk_mode": None if pre_chunk is None else {
            "workload": f"{pre_chunk['workload'].name}: 32K prompt in 4K chunks, streaming heads "
                        f"over the pruned cache plus the chunk",
            "path": STAGED_PATH,
            "attn_ms": round(pre_chunk["attn_ms"], 3),
            "ms_incl_append": round(pre_chunk["pass_ms"], 3),
            "tflops": round(pre_chunk["tflops"], 1),
            "kernel_ms_per_pass": round(pre_chunk["kern_ms"], 3),
            "kernel_tflops": round(pre_chunk["kern_tflops"], 1),
            "frac": round(pre_chunk["kern_tflops"] / BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": int(pre_chunk["flops"]),
            "duo_attn_prefill": plain_obj(pre_chunk_plain, None),
        },
        "prefill_gqa": None if pre_gqa is None else {
            "workload": f"{pre_gqa['workload'].name}: the 32K prompt in 4K chunks on the GQA layer "
                        f"(32 q / 8 KV heads, 4 retrieval, sink 16 + recent 512)",
            "path": STAGED_PATH,
            "attn_ms": round(pre_gqa["attn_ms"], 3),
            "ms_incl_append": round(pre_gqa["pass_ms"], 3),
            "tflops": round(pre_gqa["tflops"], 1),
            "kernel_ms_per_pass": round(pre_gqa["kern_ms"], 3),
            "kernel_tflops": round(pre_gqa["kern_tflops"], 1),
            "frac": round(pre_gqa["kern_tflops"] / BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": int(pre_gqa["flops"]),
            "mfma_counters": committed_mfma("prefill.hip", "prefill_gqa_v16_mfma"),
            "duo_attn_prefill": plain_obj(pre_gqa_plain, None),
        },
        "cpu_prefill_baseline": None if cpu is None else {
            "value": round(cpu_pre["tflops"], 6), "unit": "TFLOP/s", "cores": cpu["threads"],
            "kind": "oracle", "host": cores,
            "sample": f"float64 oracle prefill of 64 queries (positions 12224..12287) x 32 heads "
                      f"of the 32K MHA prompt, {cpu_pre['sec']:.2f} s",
        },
        "cpu_baseline": None if cpu is None else {
            "value": round(dec["dec_bytes"] / cpu["sec_per_step"] / 1e9, 3),
            "unit": "GB/s",
            "cores": cpu["threads"],
            "host": cores,
            "kind": "oracle",
            "sample": f"{cpu['calls']} float64 oracle decode step(s) of one {w.name} layer at "
                      f"{w.context} tokens (all 32 query heads), {cpu['sec_per_step']:.2f} s each",
        },
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
