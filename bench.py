"""Throughput of the packed-KV hot path on one MI355X.

One step = quantise the full K and V caches (write side) + decode attention
over the packed cache for every query (read side), on the isotropic decode
workload: B=16, 32 heads, d=128, context 32768, fp16 K/V ~ N(0, 1/d), one
fp16 query per head, scheme KQV at n=4 (KV and QKQV with --scheme).

Prints one JSON line.  `value` = decode GB/s of packed cache read
(algorithmic packed bytes / time of the decode entry point, HIP events on the
stream the kernels run on); quantize tok/s and the whole-step time ride
along.  `roofline` covers the decode chain, `quantize_roofline` the K + V
quantize of the step, beside `copy_floor_ms`: the same bytes moved in the
same access pattern with no arithmetic (tq_stream_rw); `quality` holds the measures of the packed cache at the
workload's full size (computed outside the timed region); `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload on the
host cores.  --workload heavy-tailed | low-rank | headq-gqa | structured prints
the line of another regime at its own full size instead (timings and quality;
structured compares SQU-KV with TQ-KV).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PACKED_BYTES = {  # per token-head (K + V) at d=128, n=4, fp32 norms / gamma
    "kv": 68 + 68, "kqv": 68 + 72, "qkqv": 72 + 72, "tq-kv": 68 + 68, "tq-qkv": 72 + 68,
}
# Arithmetic of the path: fp16 operands (value centroids, the fp16 sketch S,
# S q and the softmax weights in the value sums; the write side's matrix-core
# products) with fp32 accumulation; key scores against fp32 centroids.
ARITH = "f16xf16+f32acc"
QUALITY_KEYS = ("kl_mean", "kl_max", "top5_recall", "relmse_k", "relmse_v", "dir_err_k", "dir_err_v",
                "fisher_mean", "spearman_fisher_kl", "spearman_keymse_kl", "a2_value_mean", "n_queries")


def packed_bytes_total(kp, vp):
    """Bytes of all planes of both packed tensors (rounded to 16)."""
    n = 0
    for p in (kp, vp):
        for t in (p.codes, p.norms, p.qjl, p.gamma):
            if t is not None:
                n += t.numel()
    return n // 16 * 16


def _profile_fields(name):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        line = line.strip().lstrip("#").strip()
        if "=" in line:
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    return fields


def measured_traffic(scheme, chain="decode"):
    """HBM bytes per launch of the decode chain (or of the step's K + V
    quantize, chain="quantize") from the committed rocprofv3 counter summary,
    if it was taken on the current sources of that chain (else None)."""
    from compressed_decode_attention_kv_amd import profiling as pf
    f = _profile_fields("traffic_isotropic_%s.txt" % scheme)
    if not f:
        return None
    sha = pf.decode_sources_sha() if chain == "decode" else pf.quantize_sources_sha()
    if f.get("%s_sources_sha1" % chain) != sha or "%s_chain_bytes" % chain not in f:
        return None
    return float(f["%s_chain_bytes" % chain])


def measured_mfma_util(scheme):
    """MfmaUtil (%) of the quantize kernels from the committed SQ counter
    summary, if it was taken on the current quantize sources (else None)."""
    from compressed_decode_attention_kv_amd import profiling as pf
    path = os.path.join(ROOT, "profiles", "counters_isotropic_%s.txt" % scheme)
    f = _profile_fields("counters_isotropic_%s.txt" % scheme)
    if not f or f.get("quantize_sources_sha1") != pf.quantize_sources_sha():
        return None
    out = {}
    cols = None
    for line in open(path):
        if line.startswith("kernel"):
            cols = line.split()
        elif cols and line.startswith(pf.QCHAIN):
            name = line[:90].strip()
            vals = line[90:].split()
            try:  # columns counted from the right ("VALU insts" is two words in the header)
                out[name] = float(vals[cols.index("MfmaUtil%") - len(cols)])
            except (ValueError, IndexError):
                pass
    return out or None


def cpu_baseline(scheme, budget_s=12.0):
    """Oracle (float64 numpy) on whole (b, h) slices of the same workload:
    quantise K and V of one head (32768 tokens) and decode its query; repeat
    slices until the budget is spent.  Scaled to decode GB/s of packed bytes.
    Beside it, the oracle on the single-head workload (T=4096, d=128, 16
    queries, fp32 N(0,1), KQV n=4) with one BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from compressed_decode_attention_kv_amd import synth
    from oracle import attention as oat
    from oracle import quantizer as oqz
    from oracle import schemes as osc

    (km, kb), (vm, vb) = osc.modes(scheme, 4)
    sk = oqz.QState(128, km, kb, 0)
    sv = oqz.QState(128, vm, vb, 0)
    T = 32768
    done, t_quant, t_dec, slices = 0, 0.0, 0.0, 0
    t_start = time.time()
    while time.time() - t_start < budget_s and slices < 64:
        K, V, Q = synth.isotropic(1, 1, 1, T, 128, seed=100 + slices, dtype=np.float16)
        K, V, Q = K[0, 0].astype(np.float64), V[0, 0].astype(np.float64), Q[0].astype(np.float64)
        t0 = time.time()
        qk, qv = oqz.quantize(K, sk), oqz.quantize(V, sv)
        t1 = time.time()
        Kh, Vh = oqz.dequantize(qk, sk), oqz.dequantize(qv, sv)
        oat.attend(Q, Kh, Vh)
        t2 = time.time()
        t_quant += t1 - t0
        t_dec += t2 - t1
        slices += 1
        done += T
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    gbs = done * PACKED_BYTES[scheme] / t_dec / 1e9
    # Single head, T=4096, one thread.
    K1, V1, Q1 = synth.isotropic_small(seed=0)
    K1, V1, Q1 = K1[0, 0].astype(np.float64), V1[0, 0].astype(np.float64), Q1[0].astype(np.float64)
    s1k, s1v = oqz.QState(128, oqz.MSE, 4, 0), oqz.QState(128, oqz.PROD, 4, 0)
    with threadpool_limits(limits=1):
        t0 = time.time()
        q1k, q1v = oqz.quantize(K1, s1k), oqz.quantize(V1, s1v)
        t1 = time.time()
        oat.attend(Q1, oqz.dequantize(q1k, s1k), oqz.dequantize(q1v, s1v))
        t2 = time.time()
    return {"value": gbs, "unit": "GB/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": "%d whole (batch, head) slices x 32768 tokens, d=128, scheme %s n=4 "
                      "(decode = dense dequantise + attention); quantize %.3g tok/s"
                      % (slices, scheme, done / t_quant),
            "single_head_1thread": {"workload": "T=4096 d=128, 16 queries, fp32 N(0,1), kqv n=4", "threads": 1,
                                    "quantize_ms": round(1e3 * (t1 - t0), 2), "decode_ms": round(1e3 * (t2 - t1), 2),
                                    "decode_GBps": round(4096 * 140 / (t2 - t1) / 1e9, 5)}}


def _median_ms(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2]


def _quality(tq, q, k, v, kp, vp):
    """Quality measures of the packed cache against the raw tensors
    (tq_metrics on the GPU), rounded."""
    m = tq.metrics(q, k, v, kp, vp)
    out = {}
    for key in QUALITY_KEYS:
        x = m[key]
        if isinstance(x, float) and math.isnan(x):
            continue
        out[key] = int(x) if key == "n_queries" else float("%.6g" % x)
    return out


def _exact_attention(torch, Q, K, V, G):
    """Reference attention over the raw tensors in float32 (a quality
    reference outside the timed region): out [B, Hq, d]."""
    B, Hkv, T, d = K.shape
    out = torch.empty((B, Hkv * G, d), dtype=torch.float32, device=K.device)
    for b in range(B):
        q = Q[b].float().reshape(Hkv, G, d)
        kt = K[b].float().transpose(1, 2).contiguous()
        p = torch.softmax(torch.matmul(q, kt) / math.sqrt(d), dim=-1)
        out[b] = torch.matmul(p, V[b].float().contiguous()).reshape(Hkv * G, d)
    return out


def _a2_policy_rows(torch, tq, args, K, V, Q, C, basis, B, Hkv, G, T, d, packed_bytes):
    """HeadQ keys with 2-bit values: uniform widths against the A^2-weighted
    two-tier policy at the same 2-bit mean ([P3] section 5).  Output error
    against exact float32 attention; the plan's surrogate for both."""
    import numpy as np
    Np = 8
    probes = torch.from_numpy(np.ascontiguousarray(
        np.broadcast_to(C[:, :G * Np].reshape(1, Hkv * G, Np, d), (B, Hkv * G, Np, d)))).cuda().half()
    o_ref = _exact_attention(torch, Q, K, V, G)

    def out_err(o):
        e2 = float(torch.sum((o - o_ref) ** 2))
        s2 = float(torch.sum(o_ref ** 2))
        cos = torch.sum(o * o_ref, dim=-1) / (torch.linalg.norm(o, dim=-1) * torch.linalg.norm(o_ref, dim=-1))
        return {"snr_out_db": round(10 * math.log10(s2 / e2), 4),
                "phi_out": float("%.6g" % float(torch.mean(torch.arccos(torch.clamp(cos, -1, 1)))))}

    kp = tq.quantize(K, tq.KEYS, "headq", 2, 13, basis=basis)
    vp = tq.quantize(V, tq.VALUES, "headq", 2, 13)
    u_q_ms = _median_ms(torch, lambda: (tq.quantize(K, tq.KEYS, "headq", 2, 13, basis=basis),
                                        tq.quantize(V, tq.VALUES, "headq", 2, 13)), args.steps, args.warmup)
    out, lse = tq.decode_attention(Q, kp, vp)
    ws = torch.empty(tq.decode_workspace_size(kp, vp, Q.shape[1]), dtype=torch.uint8, device="cuda")
    u_d_ms = _median_ms(torch, lambda: tq.decode_attention(Q, kp, vp, out, lse, ws), args.steps, args.warmup)
    uniform = {"values": "uniform 2-bit TQ-MSE", "quantize_ms": round(u_q_ms, 4), "decode_ms": round(u_d_ms, 4),
               "packed_bytes": packed_bytes(kp) + packed_bytes(vp),
               "quality": dict(_quality(tq, Q, K, V, kp, vp), **out_err(out))}
    del kp, vp

    def policy_row(pr, label):
        cache = [None]

        def build():
            cache[0] = tq.TwoTierCache(pr, K, V, "headq", 2, seed=13, basis=basis)
        p_q_ms = _median_ms(torch, build, max(2, args.steps // 4), 1)
        c = cache[0]
        p_d_ms = _median_ms(torch, lambda: c.decode(Q), args.steps, args.warmup)
        o_pol, _ = c.decode(Q)
        plan = c.plan
        return {"probes": label,
                "values": "A^2 two-tier: %d tokens/head at %d bits, %d at %d bits" % (
                    plan["n_high"], plan["b_hi"], T - plan["n_high"], plan["b_lo"]),
                "quantize_ms": round(p_q_ms, 4), "decode_ms": round(p_d_ms, 4),
                "packed_bytes": sum(packed_bytes(kp) + packed_bytes(vp) for kp, vp in c.tiers),
                "quality": out_err(o_pol),
                "surrogate": {"%d/%d bits, %d high" % cand: float("%.6g" % sv)
                              for cand, sv in zip(plan["candidates"], plan["surrogate"])}}
    # Probes that do not know the step's queries (calibration queries at
    # random positions), and probes that do (the step's own queries, as when
    # the queries of the last window are known at write time).
    pol = [policy_row(probes, "8 calibration queries per query head"),
           policy_row(Q.reshape(B, Hkv * G, 1, d).contiguous(), "the step's own queries")]
    return {"scheme": "headq + A^2 value policy", "n_bits": 2, "uniform": uniform, "policy": pol}


def other_workload(args):
    """The pages' other regimes at full size (not the headline): one JSON
    line with the median quantize / decode time and the quality measures per
    scheme."""
    import numpy as np
    import torch
    from compressed_decode_attention_kv_amd import synth, tq

    torch.cuda.set_device(0)
    rows = []

    def packed_bytes(p):
        return sum(t.numel() for t in (p.codes, p.norms, p.qjl, p.gamma, p.side, p.side_scale) if t is not None)

    if args.workload == "heavy-tailed":
        B, H, T, d = 4, 8, 131072, 128
        K, V = synth.device_heavy_tailed(B, H, T, d, seed=33)
        in_bytes = 2 * K.numel() * 4
        for scheme in ("kv", "tq-kv", "tq-qkv"):
            for n in (2, 3):
                ps = []

                def quant():
                    ps[:] = [tq.quantize(K, tq.KEYS, scheme, n, 0), tq.quantize(V, tq.VALUES, scheme, n, 0)]
                q_ms = _median_ms(torch, quant, args.steps, args.warmup)
                moved = in_bytes + sum(packed_bytes(p) for p in ps)
                rows.append({"scheme": scheme, "n_bits": n, "quantize_ms": round(q_ms, 4),
                             "quantize_tok_per_s": round(B * T / (q_ms * 1e-3), 1),
                             "quantize_hbm_GBps": round(moved / (q_ms * 1e-3) / 1e9, 1),
                             "quality": _quality(tq, None, K, V, ps[0], ps[1])})
        cfg = "heavy-tailed: B=4 H=8 T=131072 d=128 fp32 Student-t(3) + 1% outlier tokens; quantize only"
    elif args.workload == "low-rank":
        G = 64   # queries per head: half inside the key subspace, half isotropic
        K, V, Q = synth.low_rank(4, 65536, 1024, G, seed=40)
        K, V, Q = (torch.from_numpy(x).cuda() for x in (K, V, Q))
        for scheme in ("kqv", "qkqv"):
            kp = tq.quantize(K, tq.KEYS, scheme, 4, 3)
            vp = tq.quantize(V, tq.VALUES, scheme, 4, 3)
            q_ms = _median_ms(torch, lambda: (tq.quantize(K, tq.KEYS, scheme, 4, 3),
                                              tq.quantize(V, tq.VALUES, scheme, 4, 3)), args.steps, args.warmup)
            out, lse = tq.decode_attention(Q, kp, vp)
            ws = torch.empty(tq.decode_workspace_size(kp, vp, Q.shape[1]), dtype=torch.uint8, device="cuda")
            d_ms = _median_ms(torch, lambda: tq.decode_attention(Q, kp, vp, out, lse, ws), args.steps, args.warmup)
            nb = packed_bytes(kp) + packed_bytes(vp)
            rows.append({"scheme": scheme, "n_bits": 4, "quantize_ms": round(q_ms, 4), "decode_ms": round(d_ms, 4),
                         "decode_GBps": round(nb / (d_ms * 1e-3) / 1e9, 1), "queries": int(Q.shape[1]),
                         "quality": _quality(tq, Q, K, V, kp, vp)})
        cfg = "low-rank: H=4 T=65536 d=1024 fp32, K rank 16 (0.7^i) + 0.01 noise, 64 queries per head"
    elif args.workload == "structured":
        # SQU-KV against TQ-KV at 2 and 3 bits ([P2] Recomendações Práticas 2:
        # structured data, low bit widths) at the headline decode shape.
        B, H, G, T, d = 16, 32, 1, 32768, 128
        K, V, Q, CK, CV = synth.device_structured(B, H, G, T, d, seed=66)
        fit_t0 = time.time()
        spec = {}
        for name, C in (("K", CK), ("V", CV)):
            fits = [tq.spectral_fit(C[h]) for h in range(H)]
            spec[name] = tuple(torch.from_numpy(np.ascontiguousarray(np.stack([f[i] for f in fits]))).cuda()
                               for i in range(3))
        fit_s = time.time() - fit_t0
        in_bytes = 2 * K.numel() * 2
        for scheme in ("squ-kv", "tq-kv"):
            for n in (2, 3):
                ks, vs = (spec["K"], spec["V"]) if scheme == "squ-kv" else (None, None)
                ps = []

                def quant():
                    ps[:] = [tq.quantize(K, tq.KEYS, scheme, n, 0, spectral=ks),
                             tq.quantize(V, tq.VALUES, scheme, n, 0, spectral=vs)]
                q_ms = _median_ms(torch, quant, args.steps, args.warmup)
                kp, vp = ps
                out, lse = tq.decode_attention(Q, kp, vp)
                ws = torch.empty(tq.decode_workspace_size(kp, vp, Q.shape[1]), dtype=torch.uint8, device="cuda")
                d_ms = _median_ms(torch, lambda: tq.decode_attention(Q, kp, vp, out, lse, ws), args.steps,
                                  args.warmup)
                nb = packed_bytes(kp) + packed_bytes(vp)
                row = {"scheme": scheme, "n_bits": n, "quantize_ms": round(q_ms, 4),
                       "quantize_tok_per_s": round(B * H * T / (q_ms * 1e-3), 1),
                       "quantize_hbm_GBps": round((in_bytes + nb) / (q_ms * 1e-3) / 1e9, 1),
                       "decode_ms": round(d_ms, 4), "decode_GBps": round(nb / (d_ms * 1e-3) / 1e9, 1),
                       "decode_pct_hbm_peak": round(100.0 * nb / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                       "quality": _quality(tq, Q, K, V, kp, vp)}
                if scheme == "squ-kv":
                    # The SQU-KV projection at d = 128 runs on the fp16 matrix cores as three
                    # products (hi hi, hi lo, lo hi) of 2 d^2 flops per token-head per tensor;
                    # the kernel is bound by its decision logic, not by these.
                    fl = 3 * 2.0 * 2 * d * d * B * H * T
                    row["quantize_mfma_TFLOPs"] = round(fl / (q_ms * 1e-3) / 1e12, 2)
                    row["quantize_pct_fp16_mfma_peak"] = round(100.0 * fl / (q_ms * 1e-3) / 1e12 / 2500.0, 2)
                rows.append(row)
        cfg = "structured: B=16 H=32 T=32768 d=128 fp16, K and V each a per-head mean + rank-16 (0.7^i) + 0.01 " \
              "noise, 1 query per head (those of the even heads in the key span); SQU-KV fitted by " \
              "tq_spectral_fit on 4096 separate calibration draws per head and tensor (%.1f s on the host)" % fit_s
    else:  # headq-gqa
        B, Hkv, G, T, d, r = 8, 8, 4, 131072, 128, 16
        K, V, Q, C = synth.device_rope_gqa(B, Hkv, G, T, d, seed=55)
        U = np.stack([tq.headq_fit(C[h], r) for h in range(Hkv)])
        basis = torch.from_numpy(np.ascontiguousarray(U)).cuda()
        for scheme in ("headq", "tq-kv"):
            bas = basis if scheme == "headq" else None
            kp = tq.quantize(K, tq.KEYS, scheme, 4, 13, basis=bas)
            vp = tq.quantize(V, tq.VALUES, scheme, 4, 13)
            q_ms = _median_ms(torch, lambda: (tq.quantize(K, tq.KEYS, scheme, 4, 13, basis=bas),
                                              tq.quantize(V, tq.VALUES, scheme, 4, 13)), args.steps, args.warmup)
            out, lse = tq.decode_attention(Q, kp, vp)
            ws = torch.empty(tq.decode_workspace_size(kp, vp, Q.shape[1]), dtype=torch.uint8, device="cuda")
            d_ms = _median_ms(torch, lambda: tq.decode_attention(Q, kp, vp, out, lse, ws), args.steps, args.warmup)
            nb = packed_bytes(kp) + packed_bytes(vp)
            rows.append({"scheme": scheme, "n_bits": 4, "quantize_ms": round(q_ms, 4), "decode_ms": round(d_ms, 4),
                         "decode_GBps": round(nb / (d_ms * 1e-3) / 1e9, 1),
                         "decode_pct_hbm_peak": round(100.0 * nb / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                         "quality": _quality(tq, Q, K, V, kp, vp)})
        rows.append(_a2_policy_rows(torch, tq, args, K, V, Q, C, basis, B, Hkv, G, T, d, packed_bytes))
        cfg = "headq-gqa: B=8, 8 KV heads x 4 query heads, T=131072, d=128, fp16 post-RoPE keys; rank-16 basis " \
              "fitted from 4096 calibration queries per KV head; the A^2 value policy at a 2-bit value budget " \
              "takes 8 of those calibration queries per query head as its probes"
    print(json.dumps({"workload": args.workload, "config": cfg, "data": "synthetic", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "dtype": ARITH, "results": rows}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--scheme", default="kqv", choices=sorted(PACKED_BYTES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--beside", default=None,
                    help="comma-separated schemes timed the same way and reported beside the headline "
                         "(default: the other two of kv, kqv, qkqv; '' for none)")
    ap.add_argument("--no-gen-step", action="store_true",
                    help="skip the append + decode generation-step timing (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="no quality pass and no MALL-flushed leg after the step loop (profiling runs: the step "
                         "loop's decode launches are then the last full-size ones before the streaming-read "
                         "reference)")
    ap.add_argument("--B", type=int, default=16)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--T", type=int, default=32768)
    ap.add_argument("--workload", default="isotropic", choices=["isotropic", "heavy-tailed", "low-rank", "headq-gqa", "structured"],
                    help="isotropic: the headline line; the others print their own line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.workload != "isotropic":
        other_workload(args)
        return

    import torch
    from compressed_decode_attention_kv_amd import synth, tq

    torch.cuda.set_device(0)
    B, H, T, d, n = args.B, args.H, args.T, 128, 4
    K, V, Q = synth.device_isotropic(B, H, 1, T, d, seed=1)
    torch.cuda.synchronize()

    kdesc, _ = tq.tensor_desc(K)
    vdesc, _ = tq.tensor_desc(V)
    qdesc, _ = tq.tensor_desc(Q)
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lib = tq.lib()
    import ctypes

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run_steps(scheme):
        """Quantize K and V, then decode, `warmup` untimed and `steps` timed
        times; returns the packed tensors, workspace, decode callable and
        the timings."""
        kp = tq.quantize(K, tq.KEYS, scheme, n, 0)
        vp = tq.quantize(V, tq.VALUES, scheme, n, 0)
        ws = torch.empty(tq.decode_workspace_size(kp, vp, H), dtype=torch.uint8, device="cuda")
        sid = tq.SCHEMES[scheme]

        def quant():
            tq._check(lib.tq_quantize(ctypes.byref(kdesc), tq.KEYS, sid, n, 0, None, None, ctypes.byref(kp.c), stream()))
            tq._check(lib.tq_quantize(ctypes.byref(vdesc), tq.VALUES, sid, n, 0, None, None, ctypes.byref(vp.c),
                                      stream()))

        def decode():
            tq._check(lib.tq_decode_attention(ctypes.byref(qdesc), ctypes.byref(kp.c), ctypes.byref(vp.c),
                                              out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), stream()))

        for _ in range(args.warmup):
            quant()
            decode()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.time()
        for e in ev:
            e[0].record()
            quant()
            e[1].record()
            decode()
            e[2].record()
        torch.cuda.synchronize()
        wall = time.time() - t0
        q_ms = [a.elapsed_time(b) for a, b, _ in ev]
        d_ms = [b.elapsed_time(c) for _, b, c in ev]
        assert torch.isfinite(out).all().item()
        return {"kp": kp, "vp": vp, "ws": ws, "sid": sid, "decode": decode, "step_ms": wall * 1000.0 / args.steps,
                "q_avg": sum(q_ms) / len(q_ms), "d_avg": sum(d_ms) / len(d_ms), "d_sorted": sorted(d_ms)}

    r = run_steps(args.scheme)
    kp, vp, ws, sid = r["kp"], r["vp"], r["ws"], r["sid"]
    packed = B * H * T * PACKED_BYTES[args.scheme]
    dec_gbs = packed / (r["d_avg"] * 1e-3) / 1e9
    tok_s = B * T / (r["q_avg"] * 1e-3)
    # Quantize: both fp16 inputs read, every packed plane written, per step.
    q_bytes = 2 * K.numel() * K.element_size() + packed
    q_gbs = q_bytes / (r["q_avg"] * 1e-3) / 1e9
    d_sorted = r["d_sorted"]

    res = {
        "metric": "packed-KV decode attention GB/s (% HBM peak) + quantize tok/s, d=128 n=4",
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ARITH, "data": "synthetic",
        "config": {"workload": "isotropic decode: B=%d H=%d T=%d d=%d fp16 K/V~N(0,1/d), 1 query/head, %s n=%d"
                               % (B, H, T, d, args.scheme, n),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": d, "scheme": args.scheme, "n_bits": n},
        "decode_ms": round(r["d_avg"], 4),
        "decode_ms_median": round(d_sorted[len(d_sorted) // 2], 4),
        "decode_ms_min": round(d_sorted[0], 4),
        "decode_pct_hbm_peak": round(100.0 * dec_gbs / HBM_PEAK_GBS, 2),
        "quantize_ms": round(r["q_avg"], 4),
        "quantize_tok_per_s": round(tok_s, 1),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.scheme),
                     "kernel": "decode chain (query prep + split decode + combine)",
                     "algorithmic_bytes_per_launch": packed},
        "quantize_roofline": {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic(args.scheme, "quantize"),
                              "kernel": "K + V quantize of one step",
                              "algorithmic_bytes_per_launch": q_bytes,
                              "mfma_util_pct": measured_mfma_util(args.scheme)},
    }

    # Streaming-read reference: the same non-temporal 128-bit loads over a
    # plain buffer of the packed cache's size (also the known-size reference
    # of the HBM byte counters).
    sbuf = torch.empty(packed_bytes_total(kp, vp), dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    tq.stream_read(sbuf, sink)
    torch.cuda.synchronize()
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in sev:
        a.record()
        tq.stream_read(sbuf, sink)
        b.record()
    torch.cuda.synchronize()
    s_ms = sum(a.elapsed_time(b) for a, b in sev) / len(sev)
    stream_gbs = sbuf.numel() / (s_ms * 1e-3) / 1e9
    res["stream_read_GBps"] = round(stream_gbs, 1)
    res["stream_read_bytes"] = int(packed_bytes_total(kp, vp))
    res["decode_pct_of_stream_read"] = round(100.0 * dec_gbs / stream_gbs, 2)
    del sbuf
    # Write-side floor: the step's quantize traffic (fp16 rows in; packed code
    # rows and per-token float planes out, in the quantiser's access pattern)
    # with no arithmetic, timed the same way.
    rows = B * H * T
    code_rows = [p.codes.numel() // rows for p in (kp, vp)]
    if all(c % 64 == 0 for c in code_rows):
        dst = torch.empty(rows * max(code_rows), dtype=torch.uint8, device="cuda")
        pl = torch.empty((2, rows), dtype=torch.float32, device="cuda")
        nplanes = [sum(1 for t in (p.norms, p.gamma, p.side_scale) if t is not None) for p in (kp, vp)]

        def floor_step():
            for c, npl in zip(code_rows, nplanes):
                tq.stream_rw(K, rows, d * K.element_size(), dst, c, pl, npl)
        floor_step()
        torch.cuda.synchronize()
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in fev:
            a.record()
            floor_step()
            b.record()
        torch.cuda.synchronize()
        fl_ms = sum(a.elapsed_time(b) for a, b in fev) / len(fev)
        res["quantize_roofline"]["copy_floor_ms"] = round(fl_ms, 4)
        res["quantize_roofline"]["pct_of_copy_floor"] = round(100.0 * fl_ms / r["q_avg"], 2)
        del dst, pl
    if not args.no_extras:
        # The decode alone, each repetition after a 1 GiB write that evicts
        # the 256 MB MALL (the step's quantize leaves the planes in no cache:
        # its stores are non-temporal).
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for i, (a, b) in enumerate(fev):
            flush.fill_(i & 0xFF)
            a.record()
            r["decode"]()
            b.record()
        torch.cuda.synchronize()
        f_ms = sorted(a.elapsed_time(b) for a, b in fev)
        res["decode_ms_mall_flushed_median"] = round(f_ms[len(f_ms) // 2], 4)
        del flush
        res["quality"] = {args.scheme: _quality(tq, Q, K, V, kp, vp)}

    # One generation step on the same cache: append one new token per
    # (batch, head) to K and V, then decode over per-sequence lengths.  The
    # token goes to the last slot (T - 1) and is that slot's own token, so the
    # cache is unchanged and the step can be repeated.
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    kn, vn = K[:, :, T - 1:T].contiguous(), V[:, :, T - 1:T].contiguous()
    kndesc, _ = tq.tensor_desc(kn)
    vndesc, _ = tq.tensor_desc(vn)

    def gen_step():
        tq._check(lib.tq_quantize_append(ctypes.byref(kndesc), tq.KEYS, sid, n, 0, None, None, pos.data_ptr(),
                                         ctypes.byref(kp.c), stream()))
        tq._check(lib.tq_quantize_append(ctypes.byref(vndesc), tq.VALUES, sid, n, 0, None, None, pos.data_ptr(),
                                         ctypes.byref(vp.c), stream()))
        tq._check(lib.tq_decode_attention_lens(ctypes.byref(qdesc), ctypes.byref(kp.c), ctypes.byref(vp.c),
                                               lens.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                               ws.numel(), stream()))

    if not args.no_gen_step:
        for _ in range(3):
            gen_step()
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in gev:
            a.record()
            gen_step()
            b.record()
        torch.cuda.synchronize()
        res["append_decode_step_ms"] = round(sorted(a.elapsed_time(b) for a, b in gev)[len(gev) // 2], 4)
        assert torch.isfinite(out).all().item()

    # The other schemes of the workload, timed the same way (not the headline).
    beside = [x for x in ("kv", "kqv", "qkqv") if x != args.scheme] if args.beside is None else \
        [x for x in args.beside.split(",") if x]
    del kp, vp, ws, r
    torch.cuda.empty_cache()
    res["beside"] = {}
    for scheme in beside:
        br = run_steps(scheme)
        nbytes = B * H * T * PACKED_BYTES[scheme]
        res["beside"][scheme] = {"decode_ms": round(br["d_avg"], 4),
                                 "decode_GBps": round(nbytes / (br["d_avg"] * 1e-3) / 1e9, 1),
                                 "decode_pct_hbm_peak": round(100.0 * nbytes / (br["d_avg"] * 1e-3) / 1e9
                                                              / HBM_PEAK_GBS, 2),
                                 "quantize_ms": round(br["q_avg"], 4)}
        if not args.no_extras:
            res["quality"][scheme] = _quality(tq, Q, K, V, br["kp"], br["vp"])
        del br
        torch.cuda.empty_cache()
    if "quality" in res and "kqv" in res["quality"] and "qkqv" in res["quality"]:
        # [P1] "Contribuciones Clave" 2 compares the KL of QKQV and KQV at n=4.
        res["quality"]["kl_ratio_qkqv_over_kqv"] = round(res["quality"]["qkqv"]["kl_mean"]
                                                         / res["quality"]["kqv"]["kl_mean"], 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.scheme)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
