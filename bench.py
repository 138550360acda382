#!/usr/bin/env python3
"""Benchmark of the compressed-KV hot path on one MI355X.

Workload (1.3B-class video-DiT layer, 12 heads x d=128, bf16, centroid + INT2
group-32 codec with 256 centroids per head, 1560 tokens per latent frame):
one step =
  1. encode one 3-frame chunk of keys and of values (4680 tokens each) into the
     compressed history at its offset (nearest centroid, residual, group scale/zero,
     quantize, pack), and
  2. decode-fused attention of 4680 queries over all 32760 compressed keys/values.
The history (chunks before the timed one) is encoded once before timing; all
inputs are resident in HBM when the timed region starts.  The metric is query
tokens per second (each query token covers all 12 heads).

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.
`--workload dplr|temporal|mixed|chunk|rotated|jensen|fit` measures the other paths instead (the 30-layer
cross-layer chain, the temporal chain + attention over its reconstruction,
mixed-dimensional attention, attention over a compressed history plus an
uncompressed current chunk, the default workload with H64-rotated residuals, and the
current-chunk attention with the Jensen-bias correction, and online centroid fitting at
block fill); the default line is the one above.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def encode_bytes(n_tokens: int, heads: int, dim: int, bits: int, group: int, n_centroids: int,
                 x_bytes: int = 2) -> int:
    """Algorithmic bytes of one centroid-codec encode: read x once, read the centroid
    table once, write codes + scale/zero + uint8 index once."""
    per_th = dim * x_bytes + dim * bits // 8 + 4 * (dim // group) + (1 if n_centroids <= 256 else 2)
    return n_tokens * heads * per_th + heads * n_centroids * dim * x_bytes


def attention_flops(nq: int, nk: int, dim: int, heads: int) -> float:
    """QK^T and PV: 2 * 2 * Nq * Nk * d per head."""
    return 4.0 * nq * nk * dim * heads


def cpu_baseline(d: dict, sample_heads=(0, 1), enc_frames: int = 1, q_sample: int = 512) -> dict:
    """The oracle, as it stands, timed on this host on a bounded sample of one step.

    Sample: encode of `enc_frames` latent frame(s) of keys and values (all heads), decode of
    the full compressed history and attention of `q_sample` queries for `sample_heads`
    (the history of those heads is encoded by the oracle before timing).  Each part is
    scaled to the full step (4680-token chunk, 12 heads, 4680 queries)."""
    import numpy as np
    from oracle import attention as oatt, codec as ocodec, numerics as nm

    H, D, T = d["heads"], d["dim"], d["tokens_per_frame"]
    lo, hi = d["chunk"]
    nq = d["Q"].shape[0]
    hs = list(sample_heads)
    Kf, Vf = nm.bf16_to_f32(d["K"]), nm.bf16_to_f32(d["V"])
    Ck, Cv = nm.bf16_to_f32(d["Ck"]), nm.bf16_to_f32(d["Cv"])
    # setup (untimed): the oracle's own compressed history for the sampled heads
    hist_k = ocodec.encode_centroid(Kf[:, hs], Ck[hs], 2, 32)["store"]
    hist_v = ocodec.encode_centroid(Vf[:, hs], Cv[hs], 2, 32)["store"]
    t0 = time.perf_counter()
    for x, C in ((Kf, Ck), (Vf, Cv)):
        ocodec.encode_centroid(x[lo:lo + enc_frames * T], C, 2, 32)
    t_enc = time.perf_counter() - t0
    t0 = time.perf_counter()
    kh = oatt.cache_view(ocodec.decode_store(hist_k, 2, 32, D, C=Ck[hs]), "bf16")
    vh = oatt.cache_view(ocodec.decode_store(hist_v, 2, 32, D, C=Cv[hs]), "bf16")
    t_dec = time.perf_counter() - t0
    q = nm.bf16_to_f32(d["Q"][:q_sample][:, hs])
    t0 = time.perf_counter()
    oatt.attention(q, kh, vh, d["scale"])
    t_att = time.perf_counter() - t0
    step = t_enc * (hi - lo) / (enc_frames * T) + t_dec * H / len(hs) \
        + t_att * (nq / q_sample) * (H / len(hs))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    return {
        "value": nq / step, "unit": "query-tok/s", "cores": len(os.sched_getaffinity(0)),
        "blas_threads": int(blas_threads), "kind": "oracle",
        "single_threaded_parts": ["encode", "decode"],
        "sample": (f"oracle encode of {enc_frames} frame(s) x {H} heads (K and V, single-threaded "
                   f"numpy), decode of the {d['K'].shape[0]}-token history (single-threaded "
                   f"numpy) and fp64 attention of {q_sample} queries for {len(hs)} heads "
                   f"({blas_threads} BLAS threads); scaled to one full step"),
        "seconds": {"encode": t_enc, "decode": t_dec, "attention": t_att, "step_estimate": step},
    }


def recorded_traffic(profile: str, source):
    """HBM bytes per launch of a kernel, as measured by the FETCH_SIZE and WRITE_SIZE
    passes summarized in `profile` (scaled by the reference copy's readings), or None.
    The summary records the sha256 of the kernel source it measured (of the sources'
    concatenation when `source` is a tuple); once that source has changed the numbers no
    longer describe the kernel and None is returned."""
    import hashlib
    import re
    srcs = (source,) if isinstance(source, str) else tuple(source)
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        h = hashlib.sha256()
        for src in srcs:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        sha = h.hexdigest()
    except OSError:
        return None
    m = re.search(r"traffic_per_launch: read_bytes=(\d+) write_bytes=(\d+) source_sha256=([0-9a-f]+)", text)
    if not m or m.group(3) != sha:
        return None
    return int(m.group(1)) + int(m.group(2))


def copy_reference(torch, dev):
    """One plain 256 MiB device-to-device copy (its HBM counters calibrate the others)."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def log(msg: str):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _timed(torch, step, steps: int, warmup: int):
    """Warm up, then time `steps` calls of step(i) between device synchronizations;
    returns (seconds per step, per-step event pairs)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, ev


def percentiles_ms(times_s) -> dict:
    """p10 / p50 / p90 of per-step times (seconds in, milliseconds out)."""
    a = np.asarray(times_s, dtype=np.float64) * 1e3
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


def _line(metric, value, unit, args, t_step, dtype, config, roofline, **extra):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded, shapes of the video-DiT caches)", "config": config,
           "roofline": roofline}
    out.update(extra)
    return out


def bench_dplr(args, torch, kvc, synth, dev):
    """30-layer cross-layer chain (12 heads x 128, 32760 tokens, rank 64): per layer the
    keys are predicted from the reconstructed keys of the layer before and the values from
    [keys of this layer ; reconstructed values of the layer before] (block-diagonal + rank
    64), the residual is quantized INT2 g32; layer 0 is an INT4 g32 anchor.  One step =
    encoding all 30 layers of K and V.  Roofline: algorithmic HBM bytes (inputs read once,
    codes and scale/zero written once, predictor parameters read once)."""
    n, H, D, r, layers = 32760, 12, 128, 64, 30
    prm = synth.cfg2_params()

    def f(name, t=False):
        b = torch.from_numpy(prm[name].view("int16")).view(torch.bfloat16)
        return (b.t() if t else b).contiguous().to(dev)

    WK, UK, WV, UV, VKt, VVt = f("WK"), f("UK"), f("WV"), f("UV"), f("VK", True), f("VV", True)
    log("drawing 30 layers on the device")
    xs = [(k, v) for k, v in synth.cfg2_layers_device(dev, params=prm)]
    anchor = kvc.Codec(H, D, 4, 32, kvc.BASE_NONE)
    kcod = kvc.Codec(H, D, 2, 32, kvc.BASE_DPLR, rank=r, n_inputs=1)
    vcod = kvc.Codec(H, D, 2, 32, kvc.BASE_DPLR, rank=r, n_inputs=2)
    stores = [(kvc.Store.allocate(anchor if l == 0 else kcod, n, dev),
               kvc.Store.allocate(anchor if l == 0 else vcod, n, dev)) for l in range(layers)]
    rec = [[torch.empty((n, H, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
           for _ in range(2)]
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_ENCODE, vcod, n, dev)      # keys (current stream)
    ws_v = kvc.kvc.workspace_for(kvc.kvc.OP_ENCODE, vcod, n, dev)    # values (second stream)
    s_v = torch.cuda.Stream(device=dev)   # default priority

    def step(_):
        # keys on the current stream, values on s_v: layer l's values and layer l+1's keys
        # both need only K^_l, so they run concurrently.  Events order the rest: values
        # wait for their layer's keys; keys of layer l overwrite the buffer that the values
        # of layer l-2 read, so they wait for those.
        main = torch.cuda.current_stream()
        k_done, v_done = [], []
        for l in range(layers):
            k, v = xs[l]
            rk, rv = rec[l & 1]
            pk, pv = rec[(l + 1) & 1]
            if l >= 2:
                main.wait_event(v_done[l - 2])
            if l == 0:
                kvc.kvc_encode(anchor, k, stores[l][0], 0, None, recon_out=rk)
            else:
                kvc.kvc_encode(kcod, k, stores[l][0], 0,
                               kvc.BaseParams(prev0=pk, w_block=WK, u=UK, v_lr=VKt),
                               recon_out=rk, workspace=ws)
            k_done.append(torch.cuda.Event())
            k_done[l].record(main)
            with torch.cuda.stream(s_v):
                s_v.wait_event(k_done[l])
                if l == 0:
                    kvc.kvc_encode(anchor, v, stores[l][1], 0, None, recon_out=rv)
                else:
                    kvc.kvc_encode(vcod, v, stores[l][1], 0,
                                   kvc.BaseParams(prev0=rk, prev1=pv, w_block=WV, u=UV, v_lr=VVt),
                                   recon_out=rv, workspace=ws_v)
                v_done.append(torch.cuda.Event())
                v_done[l].record(s_v)
        main.wait_event(v_done[-1])

    log("timing")
    t_step, ev = _timed(torch, step, args.steps, args.warmup)
    t_ev = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    # algorithmic bytes: every tensor the closed-loop chain must move, once - the layer's
    # K and V read, the previous reconstructions read as predictor inputs (values also
    # read this layer's reconstructed keys), codes + scale/zero and the reconstructions
    # written, the predictor parameters read
    row = n * H * D * 2
    cz2 = n * H * (D * 2 // 8 + 4 * D // 32)
    cz4 = n * H * (D * 4 // 8 + 4 * D // 32)
    par_k = sum(int(np.prod(prm[k].shape)) * 2 for k in ("WK", "UK", "VK"))
    par_v = sum(int(np.prod(prm[k].shape)) * 2 for k in ("WV", "UV", "VV"))
    per_k, per_v = 2 * row + cz2 + row + par_k, 3 * row + cz2 + row + par_v
    alg = 2 * (row + cz4 + row) + (layers - 1) * (per_k + per_v)
    flops = (layers - 1) * n * 2 * (H * D * r + H * D * D + H * D * r          # keys
                                    + 2 * H * D * r + 2 * H * D * D + H * D * r)  # values
    gbs = alg / t_ev / 1e9
    # the dominant call: one layer's value encode (rank-r product + fused predictor and
    # quantizer), timed alone
    l = layers // 2
    k_in, v_in = rec[l & 1][0], rec[(l + 1) & 1][1]
    vcall = lambda _: kvc.kvc_encode(vcod, xs[l][1], stores[l][1], 0,
                                     kvc.BaseParams(prev0=k_in, prev1=v_in, w_block=WV, u=UV, v_lr=VVt),
                                     recon_out=rec[l & 1][1], workspace=ws)
    _, ev_v = _timed(torch, vcall, max(1, min(args.steps, 10)), 1)
    t_v = sum(a.elapsed_time(b) for a, b in ev_v) / len(ev_v) * 1e-3
    v_gbs = per_v / t_v / 1e9
    return _line("cross-layer block-DPLR chain encode GB/s (30 layers K+V)", gbs, "GB/s", args,
                 t_step, "bf16", {"workload": "block-DPLR cross-layer chain, 30 layers x 12 heads "
                                  "x 128, 32760 tokens, rank 64, INT2 g32 (INT4 g32 layer 0)",
                                  "layers": layers, "tokens": n, "heads": H, "rank": r},
                 {"bound": "hbm", "achieved": v_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": v_gbs / HBM_PEAK_GBS,
                  "traffic": recorded_traffic("pred_kernel_dplr_chain_30x12x128_32760tok.md",
                                              "kv_cache_compression_02_amd/csrc/predict_fused.hip"),
                  "kernel": "value encode call (rank_kernel + pred_kernel)", "ms": t_v * 1e3},
                 chain_ms=t_ev * 1e3, chain_frac_hbm=gbs / HBM_PEAK_GBS,
                 predictor_tflops=flops / t_ev / 1e12, algorithmic_bytes=alg, flops=flops)


def bench_temporal(args, torch, kvc, synth, dev):
    """Temporal chain (40 heads x 128, 16 frames x 1560 tokens, INT2 g64 after an INT4
    g64 anchor frame): keys predicted per channel from the two previous reconstructed
    frames, values from the aligned reconstructed keys and the previous values; then
    attention of the next 3 frames' 4680 queries over the 24960 reconstructed tokens.
    One step = the 16-frame encode of K and V + the attention."""
    log("drawing the temporal workload (numpy, about 1.5 minutes)")
    d = synth.cfg3()
    H, T, F, D = d["heads"], d["tokens_per_frame"], d["n_frames"], d["dim"]
    nk, nq = F * T, d["Q"].shape[0]

    def b16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    K, V, Q, M = b16(d["K"]), b16(d["V"]), b16(d["Q"]), b16(d["M"])
    a_d, b_d, be_d = (torch.from_numpy(x).to(dev) for x in (d["a"], d["b"], d["beta"]))
    kcod = kvc.Codec(H, D, d["bits"], d["group"], kvc.BASE_TEMPORAL)
    anchor = kvc.Codec(H, D, d["anchor_bits"], d["group"], kvc.BASE_NONE)
    dense = kvc.Codec(H, D, 16, 128, kvc.BASE_NONE)
    khat = torch.empty((nk, H, D), dtype=torch.bfloat16, device=dev)
    vhat = torch.empty_like(khat)
    ks = [kvc.Store.allocate(anchor if t == 0 else kcod, T, dev) for t in range(F)]
    vs = [kvc.Store.allocate(anchor if t == 0 else kcod, T, dev) for t in range(F)]
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_ENCODE, kcod, T, dev)
    out = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
    att_ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND, dense, nk, dev, n_queries=nq)
    ev_att = []

    def fr(x, t):
        return x[t * T:(t + 1) * T]

    s_v = torch.cuda.Stream(device=dev)   # default priority

    def step(i):
        # keys on the current stream, values on s_v: frame t's values and frame t+1's keys
        # both need only K^_t, so they run concurrently; values wait for their frame's keys
        main = torch.cuda.current_stream()
        for t in range(F):
            if t == 0:
                kvc.kvc_encode(anchor, fr(K, 0), ks[0], 0, None, recon_out=fr(khat, 0))
            else:
                p2 = fr(khat, t - 2) if t > 1 else fr(khat, t - 1)
                kvc.kvc_encode(kcod, fr(K, t), ks[t], 0,
                               kvc.BaseParams(prev0=fr(khat, t - 1), prev1=p2, coef_a=a_d, coef_b=b_d),
                               recon_out=fr(khat, t))
            k_done = torch.cuda.Event()
            k_done.record(main)
            with torch.cuda.stream(s_v):
                s_v.wait_event(k_done)
                if t == 0:
                    kvc.kvc_encode(anchor, fr(V, 0), vs[0], 0, None, recon_out=fr(vhat, 0))
                else:
                    kvc.kvc_encode(kcod, fr(V, t), vs[t], 0,
                                   kvc.BaseParams(aux=fr(khat, t), prev0=fr(vhat, t - 1), w_block=M,
                                                  coef_a=be_d), recon_out=fr(vhat, t), workspace=ws)
        v_end = torch.cuda.Event()
        v_end.record(s_v)
        main.wait_event(v_end)
        if i is not None:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record()
        kvc.kvc_attend_compressed(dense, kvc.Store.dense(khat), None, dense, kvc.Store.dense(vhat),
                                  None, nk, Q, d["scale"], out=out, workspace=att_ws)
        if i is not None:
            e[1].record()
            ev_att.append(e)

    log("timing")
    t_step, ev = _timed(torch, step, args.steps, args.warmup)
    t_ev = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    t_att = sum(a.elapsed_time(b) for a, b in ev_att) / len(ev_att) * 1e-3
    flops = attention_flops(nq, nk, D, H)
    achieved = flops / t_att / 1e12
    # encode bytes the closed-loop chain must move once: each frame's K and V read, the
    # reconstructions it predicts from read (keys: frames t-1 and t-2, the same frame at
    # t = 1; values: this frame's keys and the previous values), codes + scale/zero and
    # reconstructions written, the value map M and beta read per frame
    row = T * H * D * 2
    cz2, cz4 = T * H * (D * 2 // 8 + 4 * D // 64), T * H * (D * 4 // 8 + 4 * D // 64)
    par = H * D * D * 2 + H * D * 4
    enc_bytes = 2 * (row + cz4 + row) + sum(
        (row + (2 if t >= 2 else 1) * row + cz2 + row) + (3 * row + cz2 + row + par)
        for t in range(1, F))
    t_enc = t_ev - t_att
    return _line("temporal chain: attention query-tok/s (16-frame K+V encode + attention)",
                 nq / t_ev, "query-tok/s", args, t_step, "bf16",
                 {"workload": "temporal AR(2) keys + key->value cross predictor, 40 heads x 128, "
                              "16 frames x 1560 tokens, INT2 g64 (INT4 g64 frame 0); attention "
                              "4680 q x 24960 keys", "heads": H, "frames": F, "tokens": nk,
                  "queries": nq},
                 {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / BF16_PEAK_TFLOPS,
                  "traffic": recorded_traffic("attend_bf16_kernel_dense_temporal_40x128_4680q_24960k.md",
                                              "kv_cache_compression_02_amd/csrc/attend.hip"),
                  "kernel": "attend_bf16_kernel",
                  "ms": t_att * 1e3},
                 encode={"ms": t_enc * 1e3, "bytes": enc_bytes, "GB/s": enc_bytes / t_enc / 1e9,
                         "frac_hbm": enc_bytes / t_enc / 1e9 / HBM_PEAK_GBS})


def bench_chunk(args, torch, kvc, synth, dev, jensen: bool = False):
    """cfg1 with the most recent 3 frames kept uncompressed: 4680 queries attend to the
    28080 compressed history tokens (centroid + INT2 g32, 256 centroids/head) and the
    4680-token current chunk in bf16, one softmax over both (history key splits and the
    chunk as separate parts, merged by log-sum-exp).  One step = that attention; with
    `jensen` the history keys' logits carry the Jensen-bias correction."""
    d = synth.cfg1()
    H, D, C = d["heads"], d["dim"], d["centroids"]
    lo, hi = d["chunk"]
    nq = d["Q"].shape[0]

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).to(dev)

    codec = kvc.Codec(H, D, d["bits"], d["group"], kvc.BASE_CENTROID, C)
    ks, vs = kvc.Store.allocate(codec, lo, dev), kvc.Store.allocate(codec, lo, dev)
    kb = kvc.BaseParams(centroids=b16(d["Ck"]))
    vb = kvc.BaseParams(centroids=b16(d["Cv"]))
    kvc.kvc_encode(codec, b16(d["K"][:lo]), ks, 0, kb)
    kvc.kvc_encode(codec, b16(d["V"][:lo]), vs, 0, vb)
    kb.centroid_tables = kvc.kvc_centroid_tables(codec, kb.centroids)   # fp16 images (or None)
    vb.centroid_tables = kvc.kvc_centroid_tables(codec, vb.centroids)
    Kc, Vc, Q = b16(d["K"][lo:hi]), b16(d["V"][lo:hi]), b16(d["Q"])
    out = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND_CHUNK, codec, lo, dev, n_queries=nq)

    flags = kvc.ATTEND_JENSEN if jensen else 0

    def step(_):
        kvc.kvc_attend_compressed_chunk(codec, ks, kb, codec, vs, vb, lo, Kc, Vc, Q, d["scale"],
                                        ws, out=out, flags=flags)

    log("timing")
    t_step, ev = _timed(torch, step, args.steps, args.warmup)
    t_ev = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    achieved = attention_flops(nq, hi, D, H) / t_ev / 1e12
    jb = ", Jensen-corrected history logits" if jensen else ""
    return _line("compressed-history + current-chunk attention query-tok/s" + jb, nq / t_ev,
                 "query-tok/s", args, t_step, "bf16",
                 {"workload": "centroid+INT2 g32 history of 28080 tokens + uncompressed 4680-token "
                              "current chunk, 12 heads x 128, 256 centroids/head, 4680 queries" + jb,
                  "heads": H, "head_dim": D, "history_tokens": lo, "chunk_tokens": hi - lo,
                  "queries": nq, "jensen": jensen},
                 {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                  "traffic": recorded_traffic("attend_bf16_kernel_chunk_jensen_12x128_4680q_28080k_4680c.md"
                                              if jensen else
                                              "attend_bf16_kernel_chunk_12x128_4680q_28080k_4680c.md",
                                              "kv_cache_compression_02_amd/csrc/attend.hip"),
                  "kernel": "attend_bf16_kernel (history parts + chunk part + merge)",
                  "ms": t_ev * 1e3})


def bench_mixed(args, torch, kvc, synth, dev):
    """NanoKV-Fast style attention: 12 heads x 128, 65520 keys with 512 centroids per
    head, INT4 key coefficients on a 16-dim basis, INT2 g32 values; 4680 queries scored as
    q.C[a] + (B^T q).c without rebuilding keys.  One step = the attention.  Roofline: the
    method's algorithmic flops (Q C^T table + projection + scores + PV)."""
    log("drawing the mixed-dimensional workload")
    d = synth.cfg4()
    H, C, m, D = d["heads"], d["centroids"], d["coeff_dim"], d["dim"]
    nk, nq = d["K"].shape[0], d["Q"].shape[0]

    def b16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    kc = kvc.Codec(H, D, d["k_bits"], m, kvc.BASE_COEFF, C, coeff_dim=m)
    vc = kvc.Codec(H, D, d["v_bits"], d["v_group"], kvc.BASE_CENTROID, C)
    ks, vs = kvc.Store.allocate(kc, nk, dev), kvc.Store.allocate(vc, nk, dev)
    kb = kvc.BaseParams(centroids=b16(d["Ck"]), basis=b16(d["B"]))
    vb = kvc.BaseParams(centroids=b16(d["Cv"]))
    Kx, Vx = b16(d["K"]), b16(d["V"])
    kvc.kvc_encode(kc, Kx, ks, 0, kb)
    kvc.kvc_encode(vc, Vx, vs, 0, vb)
    vb.centroid_tables = kvc.kvc_centroid_tables(vc, vb.centroids)   # fp16 image (or None)
    # the encode of the whole 65520-token history (K: nearest of 512 centroids + INT4
    # coefficients of the residual on the basis; V: nearest centroid + INT2 g32), timed
    # with events apart from the attention steps
    log("timing the history encode")
    reps = max(1, min(args.steps, 5))
    _, ev_k = _timed(torch, lambda _: kvc.kvc_encode(kc, Kx, ks, 0, kb), reps, 1)
    _, ev_v = _timed(torch, lambda _: kvc.kvc_encode(vc, Vx, vs, 0, vb), reps, 1)
    t_k = sum(a.elapsed_time(b) for a, b in ev_k) / reps * 1e-3
    t_v = sum(a.elapsed_time(b) for a, b in ev_v) / reps * 1e-3
    x_b = nk * H * D * 2
    cen_b = H * C * D * 2
    enc_k = x_b + cen_b + D * m * 2 + nk * H * (m * d["k_bits"] // 8 + 4 + 2)
    enc_v = x_b + cen_b + nk * H * (D * d["v_bits"] // 8 + 4 * D // d["v_group"] + 2)
    Q = b16(d["Q"])
    out = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND_MIXED, kc, nk, dev, n_queries=nq)

    def step(_):
        kvc.kvc_attend_mixed_dim(kc, ks, kb, vc, vs, vb, nk, Q, d["scale"], out=out, workspace=ws)

    log("timing")
    t_step, ev = _timed(torch, step, args.steps, args.warmup)
    t_ev = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    flops = H * (2.0 * nq * C * D + 2.0 * nq * D * m + 2.0 * nq * nk * m + 2.0 * nq * nk * D)
    achieved = flops / t_ev / 1e12
    return _line("mixed-dimensional attention query-tok/s", nq / t_ev, "query-tok/s", args, t_step,
                 "bf16", {"workload": "NanoKV-Fast style mixed-dimensional attention, 12 heads x "
                                      "128, 65520 keys, 512 centroids/head, INT4 m=16 key "
                                      "coefficients, INT2 g32 values, 4680 queries",
                          "heads": H, "keys": nk, "queries": nq, "centroids": C, "coeff_dim": m},
                 {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / BF16_PEAK_TFLOPS,
                  "traffic": recorded_traffic("attend_mixed_cl_kernel_mixed_12x128_4680q_65520k.md",
                                              "kv_cache_compression_02_amd/csrc/attend.hip"),
                  "kernel": "attend_mixed_cl_kernel (+ the centroid-block sort of the history: "
                            "one kvc_attend_mixed_dim call)", "ms": t_ev * 1e3},
                 full_attention_equivalent_tflops=attention_flops(nq, nk, D, H) / t_ev / 1e12,
                 encode={"keys_ms": t_k * 1e3, "values_ms": t_v * 1e3, "bytes": enc_k + enc_v,
                         "GB/s": (enc_k + enc_v) / (t_k + t_v) / 1e9,
                         "frac_hbm": (enc_k + enc_v) / (t_k + t_v) / 1e9 / HBM_PEAK_GBS})


def bench_rotated(args, torch, kvc, synth, dev):
    """The default workload's shapes with the Hn residual transform: K and V residuals
    rotated by H64 / 8 per 64-channel group before INT2 g64 quantization (256
    centroids/head).  One step = encode of the 4680-token chunk (K, V) + attention of
    4680 queries over the 32760-token history, whose tile decode rotates back."""
    d = synth.cfg1()
    H, D, C = d["heads"], d["dim"], d["centroids"]
    bits, group, rot = 2, 64, 64
    lo, hi = d["chunk"]
    nk, nq = d["K"].shape[0], d["Q"].shape[0]

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).to(dev)

    K, V, Q = b16(d["K"]), b16(d["V"]), b16(d["Q"])
    codec = kvc.Codec(H, D, bits, group, kvc.BASE_CENTROID, C, rotation=rot)
    ks, vs = kvc.Store.allocate(codec, nk, dev), kvc.Store.allocate(codec, nk, dev)
    kb = kvc.BaseParams(centroids=b16(d["Ck"]))
    vb = kvc.BaseParams(centroids=b16(d["Cv"]))
    kvc.kvc_encode(codec, K[:lo], ks, 0, kb)
    kvc.kvc_encode(codec, V[:lo], vs, 0, vb)
    kb.centroid_tables = kvc.kvc_centroid_tables(codec, kb.centroids)   # fp16 images (or None)
    vb.centroid_tables = kvc.kvc_centroid_tables(codec, vb.centroids)
    Kc, Vc = K[lo:hi].contiguous(), V[lo:hi].contiguous()
    out = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND, codec, nk, dev, n_queries=nq)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record()
        kvc.kvc_encode_kv(codec, Kc, Vc, ks, vs, lo, kb, vb)
        if e: e[1].record()
        kvc.kvc_attend_compressed(codec, ks, kb, codec, vs, vb, nk, Q, d["scale"], out=out,
                                  workspace=ws)
        if e: e[2].record()

    log("timing")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_enc = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps * 1e-3
    t_att = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps * 1e-3
    achieved = attention_flops(nq, nk, D, H) / t_att / 1e12
    enc_b = 2 * encode_bytes(hi - lo, H, D, bits, group, C)
    line = _line("compressed-KV attention query-tok/s, H64-rotated residuals (encode 3-frame "
                 "chunk + attention over history)", nq * args.steps / elapsed, "query-tok/s",
                 args, elapsed / args.steps, "bf16",
                 {"workload": "centroid+H64-rotated INT2 g64 codec, 12 heads x 128, 256 "
                              "centroids/head; encode 4680-token chunk (K,V) + attention 4680 q "
                              "x 32760 keys",
                  "heads": H, "head_dim": D, "history_tokens": nk, "queries": nq,
                  "chunk_tokens": hi - lo, "bits": bits, "group": group, "rotation": rot,
                  "centroids": C},
                 {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                  "traffic": recorded_traffic("attend_bf16_kernel_rotated_h64_12x128_4680q_32760k.md",
                                              "kv_cache_compression_02_amd/csrc/attend.hip"),
                  "kernel": "attend_bf16_kernel (rotated)", "ms": t_att * 1e3})
    line["encode"] = {"ms": t_enc * 1e3, "bytes": enc_b, "GB/s": enc_b / t_enc / 1e9,
                      "frac_hbm": enc_b / t_enc / 1e9 / HBM_PEAK_GBS}
    return line


def bench_fit(args, torch, kvc, synth, dev):
    """Online centroid fitting at block fill on the cfg1 chunk: 10 Lloyd iterations on
    the 4680-token block of K and of V (12 heads x 128, 256 centroids/head, from every
    18th token).  One step = both fits.  Algorithmic bytes per iteration and tensor: the
    block read by the assignment and again by the update, the table read and written."""
    d = synth.cfg1()
    H, D, C = d["heads"], d["dim"], d["centroids"]
    lo, hi = d["chunk"]
    n = hi - lo
    iters = 10

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).to(dev)

    codec = kvc.Codec(H, D, d["bits"], d["group"], kvc.BASE_CENTROID, C)
    X = [b16(d["K"][lo:hi]), b16(d["V"][lo:hi])]
    init = [b16(np.ascontiguousarray(a[lo:hi][::18][:C].transpose(1, 0, 2))) for a in (d["K"], d["V"])]
    tabs = [t.clone() for t in init]
    ws = kvc.kvc.workspace_for(kvc.kvc.OP_FIT, codec, n, dev)

    def step(_):
        for x, t, t0 in zip(X, tabs, init):
            t.copy_(t0)
            kvc.kvc_fit_centroids(codec, x, t, iters, workspace=ws)

    log("timing")
    t_step, ev = _timed(torch, step, args.steps, args.warmup)
    t_ev = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    per_iter = 2 * (2 * n * H * D * 2 + 2 * H * C * D * 2 + n * H)
    gbs = per_iter * iters / t_ev / 1e9
    return _line("online centroid fit, token-iterations/s (Lloyd, K and V)",
                 2 * n * iters / t_ev, "token-iterations/s", args, t_step, "bf16",
                 {"workload": "Lloyd fit of 256 centroids/head on one 4680-token block of K and "
                              "of V, 12 heads x 128, 10 iterations from every 18th token",
                  "heads": H, "head_dim": D, "tokens": n, "centroids": C, "iterations": iters},
                 {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS,
                  # per timed step: both tensors' 10 iterations of the two kernels
                  "traffic": (lambda b: None if b is None else b * 2 * iters)(recorded_traffic(
                      "fit_update_kernel_cfg1_chunk_12x128_4680tok_256c.md",
                      ("kv_cache_compression_02_amd/csrc/encode.hip",
                       "kv_cache_compression_02_amd/csrc/fit.hip"))),
                  "kernel": "encode_c16_kernel (assignment) + fit_update_kernel", "ms": t_ev * 1e3})


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-ref", action="store_true",
                    help="run one plain 256 MiB device copy first (calibrates HBM counters)")
    ap.add_argument("--workload", default="centroid",
                    choices=("centroid", "dplr", "temporal", "mixed", "chunk", "rotated", "jensen",
                             "fit"),
                    help="centroid: the default line; the others measure the cross-layer "
                         "chain, the temporal chain + attention, mixed-dimensional attention, "
                         "attention over the compressed history plus an uncompressed chunk, "
                         "the default workload with H64-rotated residuals, the current-chunk "
                         "attention with the Jensen-bias correction, online centroid fitting")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              f"the multi-GPU sharding is described, not built", file=sys.stderr)
        return 2

    import torch

    import kv_cache_compression_02_amd as kvc
    import synth

    dev = torch.device("cuda:0")
    if args.copy_ref:
        copy_reference(torch, dev)
    if args.workload != "centroid":
        line = {"dplr": bench_dplr, "temporal": bench_temporal, "mixed": bench_mixed,
                "chunk": bench_chunk, "rotated": bench_rotated,
                "jensen": lambda *a: bench_chunk(*a, jensen=True),
                "fit": bench_fit}[args.workload](
            args, torch, kvc, synth, dev)
        print(json.dumps(line))
        return 0
    d = synth.cfg1()
    H, D, C = d["heads"], d["dim"], d["centroids"]
    bits, group = d["bits"], d["group"]
    lo, hi = d["chunk"]
    nk, nq = d["K"].shape[0], d["Q"].shape[0]

    def dev_bf16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    K, V, Q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["Q"])
    codec = kvc.Codec(H, D, bits, group, kvc.BASE_CENTROID, C)
    ks, vs = kvc.Store.allocate(codec, nk, dev), kvc.Store.allocate(codec, nk, dev)
    kb = kvc.BaseParams(centroids=dev_bf16(d["Ck"]))
    vb = kvc.BaseParams(centroids=dev_bf16(d["Cv"]))
    out = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
    # history before the timed chunk, encoded once, chunk by chunk as a cache fills
    # (every encode launch of the run then has the timed launch's shape)
    for c0 in range(0, lo, hi - lo):
        c1 = min(lo, c0 + (hi - lo))
        kvc.kvc_encode_kv(codec, K[c0:c1], V[c0:c1], ks, vs, c0, kb, vb)
    Kc, Vc = K[lo:hi].contiguous(), V[lo:hi].contiguous()
    att_ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND, codec, nk, dev, n_queries=nq)
    # fp16 images of the centroid tables for the tile decode, made once per table like the
    # tables themselves (None where a table has no exact image: the bf16 table is used)
    ka = kvc.BaseParams(centroids=kb.centroids,
                        centroid_tables=kvc.kvc_centroid_tables(codec, kb.centroids))
    va = kvc.BaseParams(centroids=vb.centroids,
                        centroid_tables=kvc.kvc_centroid_tables(codec, vb.centroids))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record()
        kvc.kvc_encode_kv(codec, Kc, Vc, ks, vs, lo, kb, vb)   # the chunk's K and V, one launch
        if e: e[1].record()
        kvc.kvc_attend_compressed(codec, ks, ka, codec, vs, va, nk, Q, d["scale"], out=out,
                                  workspace=att_ws)
        if e: e[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    enc_s = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    att_s = [e[1].elapsed_time(e[2]) * 1e-3 for e in ev]
    t_enc = sum(enc_s) / args.steps
    t_att = sum(att_s) / args.steps
    flops = attention_flops(nq, nk, D, H)
    enc_b = 2 * encode_bytes(hi - lo, H, D, bits, group, C)
    achieved = flops / t_att / 1e12
    line = {
        "metric": "compressed-KV attention query-tok/s (encode 3-frame chunk + attention over history)",
        "value": nq * args.steps / elapsed,
        "unit": "query-tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded clustered AR(1) video-DiT KV, 1560 tokens/frame)",
        "config": {"workload": "centroid+INT2 g32 codec, 12 heads x 128, 256 centroids/head; "
                               "encode 4680-token chunk (K,V) + attention 4680 q x 32760 keys",
                   "heads": H, "head_dim": D, "history_tokens": nk, "queries": nq,
                   "chunk_tokens": hi - lo, "bits": bits, "group": group, "centroids": C,
                   "centroid_tables": "fp16 images" if ka.centroid_tables is not None
                                      and va.centroid_tables is not None else "bf16"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic("attend_bf16_kernel_centroid_int2_12x128_4680q_32760k.md",
                                                 "kv_cache_compression_02_amd/csrc/attend.hip"),
                     "kernel": "attend_bf16_kernel", "ms": t_att * 1e3,
                     "ms_percentiles": percentiles_ms(att_s)},
        "encode": {"ms": t_enc * 1e3, "bytes": enc_b, "GB/s": enc_b / t_enc / 1e9,
                   "frac_hbm": enc_b / t_enc / 1e9 / HBM_PEAK_GBS,
                   "ms_percentiles": percentiles_ms(enc_s)},
    }
    # decode of the whole compressed history (K and V) to bf16, timed apart from the step
    kdec = torch.empty((nk, H, D), dtype=torch.bfloat16, device=dev)
    vdec = torch.empty_like(kdec)

    def dec(_):
        kvc.kvc_decode(codec, ks, 0, nk, kb, out=kdec, out_dtype=kvc.BF16)
        kvc.kvc_decode(codec, vs, 0, nk, vb, out=vdec, out_dtype=kvc.BF16)

    _, ev_d = _timed(torch, dec, max(1, min(args.steps, 10)), 1)
    t_dec = sum(a.elapsed_time(b) for a, b in ev_d) / len(ev_d) * 1e-3
    # per tensor: codes + scale/zero + index read, bf16 rows written, the table once
    dec_b = 2 * (nk * H * (D * bits // 8 + 4 * D // group + 1) + nk * H * D * 2 + H * C * D * 2)
    line["decode"] = {"ms": t_dec * 1e3, "bytes": dec_b, "GB/s": dec_b / t_dec / 1e9,
                      "frac_hbm": dec_b / t_dec / 1e9 / HBM_PEAK_GBS,
                      "what": "decode of the 32760-token history, K and V, to bf16"}
    # the unfused alternative at the same shape: decode the whole history to bf16, then
    # dense attention over the decoded caches (the same kernel family without the tile
    # decode), timed as one call sequence against the fused attention above
    dense = kvc.Codec(H, D, 16, 128, kvc.BASE_NONE)
    dense_ws = kvc.kvc.workspace_for(kvc.kvc.OP_ATTEND, dense, nk, dev, n_queries=nq)
    out_u = torch.empty_like(out)

    def unfused(_):
        dec(None)
        kvc.kvc_attend_compressed(dense, kvc.Store.dense(kdec), None, dense, kvc.Store.dense(vdec),
                                  None, nk, Q, d["scale"], out=out_u, workspace=dense_ws)

    _, ev_u = _timed(torch, unfused, max(1, min(args.steps, 10)), 1)
    u_s = [a.elapsed_time(b) * 1e-3 for a, b in ev_u]
    t_u = sum(u_s) / len(u_s)
    line["unfused_reference"] = {
        "what": "kvc_decode of K and V to bf16 + dense attention over the decoded caches",
        "ms": t_u * 1e3, "frac": flops / t_u / 1e12 / BF16_PEAK_TFLOPS,
        "ms_percentiles": percentiles_ms(u_s),
        "fused_over_unfused_speedup": t_u / t_att,
        "max_abs_diff_vs_fused": float((out_u - out).abs().max().item())}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
