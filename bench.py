#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = the whole prefill path over the Kimi K3 KDA layer workload (B=1, T=8192,
H=96, K=V=128, bf16 q/k/v, bf16 gate logits, fp32 beta/state): one chunk-prefill call
with the bounded gate evaluated in its kernels (zero initial state, fp32 final state,
bf16 output), in its two-kernel form -- a pre-pass over every (chunk, head) into a
workspace allocated once beforehand, then the chain kernel for the serial part, fed by
direct global-to-LDS copies of the packages.  Inputs are resident in HBM before timing
starts.  Reported:

* value: prefill tokens/s over K timed steps (ms_per_step = wall time per step);
* roofline: the call's algorithmic HBM traffic (1,284 B per token-head with the gate
  logits in bf16) and algorithmic flops (6KV + 64(3K+2V) per token-head) divided by its
  average time (HIP events on the launch stream around the call's 2 launches), against
  8 TB/s and 2.5 PFLOP/s bf16; the single-kernel form is timed beside it;
* decode: 256 successive single-token steps over a kept [64,96,128,128] fp32 state
  (one fused step kernel per step, the gate evaluated inside it; with --gate separate
  the gate kernel before each step), with the step kernel's algorithmic bytes (state
  read + write plus the token vectors) per launch over its launch time;
* cpu_baseline: the fp64 oracle (gate + token scan) on half the heads of the same
  prefill workload, timed on the host cores and scaled to the whole workload.

Prints ONE JSON line.  Only N=1 is meaningful: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix cores


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash(name) -> str:
    """Hash of a kernel source file, or of several (a list) taken in order."""
    h = hashlib.sha256()
    for n in ([name] if isinstance(name, str) else name):
        h.update(open(os.path.join(ROOT, "gated_delta_rule_31_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file: str, workload: str):
    """Counter-measured HBM bytes per launch (profiles/traffic.json), if they were taken
    on the kernel source as it is now; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(workload)
        if not e or e.get("source_sha256_16") != kernel_source_hash(kernel_file):
            return None
        return float(e["bytes_per_launch"])
    except Exception:
        return None


COPY_BYTES = 1 << 30
TWO_PASS_SOURCES = ["kda_chunk_pack.h", "kda_chunk_kernel.h", "kda_chunk_chain.hip", "kda_chunk_chain2.h"]


def _counter_means(path, counter):
    """Mean counter value per kernel (rocprofv3 counter_collection.csv, KiB per dispatch)."""
    import csv
    import collections
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, gate="fused"):
    """HBM bytes per launch of the chunk and step kernels: FETCH_SIZE and WRITE_SIZE (KiB)
    each scaled by what the same counter reads for a plain copy of known size (a copy of
    N bytes reads N and writes N)."""
    def copy_kib(path, counter):
        m = _counter_means(path, counter)
        big = max(m.items(), key=lambda kv: kv[1])  # the 1 GiB copy kernel
        return big[1], big[0]
    cf, cname = copy_kib(copy_fetch_csv, "FETCH_SIZE")
    cw, _ = copy_kib(copy_write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / cf
    w_scale = COPY_BYTES / cw
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    out = {"_calibration": {"copy_kernel": cname[:120], "copy_bytes": COPY_BYTES, "fetch_kib": cf,
                            "write_kib": cw, "bytes_per_fetch_kib": f_scale, "bytes_per_write_kib": w_scale}}
    zg = gate == "fused"
    # the exact instantiations the benchmark times (K = V = 128, bf16, chunk 32)
    chunk_pat = "PrecMixed, 128, 128, 32, 64, %d>" % (1 if zg else 0)
    flag = "Lb1E" if zg else "Lb0E"  # (these two appear under their mangled names)
    # the two-kernel form per call: the pre-pass over every (chunk, head) item (packages in
    # the paired column order), then the DMA-fed chain kernel
    two_pass = [(("chunk_pack_kernel<", "PrecMixed, 128, 32, %d, true>" % (1 if zg else 0)), 1),
                (("chunk_chain2_kernel<128, 128, 32, 4>",), 1)]
    entries = [("k3_prefill_chunk_fwd_" + gate, [("chunk_fwd_kernel<", chunk_pat)], "kda_chunk_kernel.h"),
               ("decode_recurrent_step_" + gate, [("recurrent_step_kernelIDF16bLi128ELi128E" + flag,)], "kda_step.hip"),
               ("short_recurrent_fwd_" + gate, [("recurrent_fwd_kernelIDF16bLi128ELi128E" + flag,)],
                "kda_recurrent.hip")]
    # the backward's kernels at the K3 shape (bf16 inputs); a name may appear mangled or not
    for kern in ("prep", "vgrads", "kgrads"):
        entries.append(("k3_bwd_" + kern, [("bwd_%s_kernelIDF16bLi128ELi128E" % kern,)], "kda_bwd.hip"))
    for kern in ("states", "dstates"):
        entries.append(("k3_bwd_" + kern, [("bwd_%s_kernel<128, 128>" % kern,), ("bwd_%s_kernelILi128ELi128E" % kern,)],
                        "kda_bwd.hip"))
    # the two-kernel form: the bytes of all its launches per call
    fk = [sum(v for k, v in fetch.items() if all(p_ in k for p_ in pats)) for pats, _ in two_pass]
    wk = [sum(v for k, v in write.items() if all(p_ in k for p_ in pats)) for pats, _ in two_pass]
    if all(fk) and all(wk):
        names = ("pack", "chain")
        out["k3_prefill_two_pass_" + gate] = {
            "fetch_kib_per_launch": dict(zip(names, fk)), "write_kib_per_launch": dict(zip(names, wk)),
            "launches_per_call": dict(zip(names, [n for _, n in two_pass])),
            "bytes_per_launch": sum(n * (f * f_scale + w * w_scale) for (_, n), f, w in zip(two_pass, fk, wk)),
            "source_sha256_16": kernel_source_hash(TWO_PASS_SOURCES)}
    for key, alts, src in entries:
        match = lambda k: any(all(p_ in k for p_ in pats) for pats in alts)
        fk = [v for k, v in fetch.items() if match(k)]
        wk = [v for k, v in write.items() if match(k)]
        if not fk or not wk:
            continue
        out[key] = {"fetch_kib": fk[0], "write_kib": wk[0],
                    "bytes_per_launch": fk[0] * f_scale + wk[0] * w_scale,
                    "source_sha256_16": kernel_source_hash(src)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=32)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--gate", choices=("fused", "separate"), default="fused",
                    help="fused: the kernels take the gate logits; separate: bounded_decay writes a "
                         "float32 gate that the kernels read")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward (training) block")
    ap.add_argument("--no-short", action="store_true", help="skip the short-continuation (token-recurrent) block")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed-sequence (8 sequences) prefill block")
    ap.add_argument("--only", choices=("prefill", "varlen", "gate", "bwd", "decode", "short"),
                    help="run one workload block alone (for per-workload kernel traces); the JSON line then "
                         "holds that block only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=48)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                                "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE results into profiles/traffic.json")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, gate=args.gate)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_31_amd as kda
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes 4 times" % n)
        return

    run = lambda name: args.only is None or args.only == name
    run_prefill = run("prefill")

    # ---------------- prefill ---------------------------------------------------------
    B, T, H, K, V = 1, 8192, 96, 128, 128
    log("generating prefill inputs")
    inp = synth.k3_prefill(device="cuda")
    q, k, v, z, ls, beta = inp.q, inp.k, inp.v, inp.z, inp.log_scale, inp.beta
    g = torch.empty(B, T, H, K, dtype=torch.float32, device=dev)
    out = torch.empty(B, T, H, V, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    fused = args.gate == "fused"
    nws = kda.chunk_fwd_workspace_size(q.dtype, B, T, H, K, V, args.chunk)
    if nws == 0:
        log("chunk size %d has no two-kernel form at this shape: timing the single-kernel form" % args.chunk)
    wsp = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)  # allocated once, outside the timed steps

    def step(ev_pair=None, two_pass=nws > 0):
        if not fused:
            kda.bounded_decay(z, ls, lower_bound=-5.0, out_log=False, out=g)
        if ev_pair is not None:
            ev_pair[0].record(stream)
        w = dict(workspace=wsp) if two_pass else dict(two_pass=False)
        if fused:
            kda.chunk_fwd_fused_gate(q, k, v, z, ls, beta, lower_bound=-5.0, initial_state=None,
                                     chunk_size=args.chunk, out=out, final_state=fin, **w)
        else:
            kda.chunk_fwd(q, k, v, g, beta, initial_state=None, chunk_size=args.chunk, gate_is_log=False,
                          out=out, final_state=fin, **w)
        if ev_pair is not None:
            ev_pair[1].record(stream)

    th = B * T * H
    gate_bytes = 2 * K if fused else 4 * K                  # bf16 logits, or the fp32 gate tensor
    if run_prefill:
        log("warmup %d" % args.warmup)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        log("timing %d steps" % args.steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        chunk_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        ms_per_step = wall * 1e3 / args.steps
        tokens_per_s = B * T / (wall / args.steps)

        alg_bytes = th * (3 * 2 * K + gate_bytes + 4 + 2 * V)   # q,k,v bf16 + gate + beta + out bf16
        alg_flops = th * (6 * K * V + 64 * (3 * K + 2 * V))
        achieved_gbs = alg_bytes / (chunk_ms * 1e-3) / 1e9
        achieved_tflops = alg_flops / (chunk_ms * 1e-3) / 1e12
        traffic = load_traffic(TWO_PASS_SOURCES, "k3_prefill_two_pass_" + args.gate)
        log("prefill: %.3f ms/step, prefill call %.3f ms, %.1f GB/s, %.1f TFLOP/s" %
            (ms_per_step, chunk_ms, achieved_gbs, achieved_tflops))
        # the single-kernel form of the same call, beside it (not part of the timed steps)
        full = args.only is None
        for _ in range(2 if full else 0):
            step(two_pass=False)
        oev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10 if full else 1)]
        for e_ in (oev if full else []):
            step(e_, two_pass=False)
        torch.cuda.synchronize()
        one_ms = sum(a_.elapsed_time(b_) for a_, b_ in oev) / len(oev) if full else float("nan")
        one_gbs = alg_bytes / (one_ms * 1e-3) / 1e9
        log("prefill, single-kernel form: %.3f ms" % one_ms)

        result = {
            "metric": "KDA prefill tokens/s (H=96,D=128) + % MFMA peak; decode state HBM GB/s",
            "value": tokens_per_s,
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "k3_prefill_B1_T8192_H96_K128_V128", "global_batch": B, "seq_len": T,
                       "heads": H, "key_dim": K, "value_dim": V, "chunk_size": args.chunk,
                       "step": "chunk_fwd_fused_gate" if fused else "bounded_decay + chunk_fwd",
                       "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved_gbs / HBM_PEAK_GBS,
                         "traffic": traffic if nws > 0 else None,
                         "kernel": "one prefill call: chunk_pack_kernel (pre-pass over all chunks), then "
                         "chunk_chain2_kernel (the serial chain)" if nws > 0 else "chunk_fwd_kernel",
                         "launch_ms": chunk_ms, "algorithmic_bytes_per_launch": alg_bytes},
            "mfma": {"achieved": achieved_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_tflops / BF16_PEAK_TFLOPS, "algorithmic_flops_per_launch": alg_flops},
            "prefill_single_kernel": {"kernel": "chunk_fwd_kernel", "launch_ms": one_ms,
                                      "tokens_per_s": B * T / (one_ms * 1e-3),
                                      "hbm": {"achieved": one_gbs, "frac": one_gbs / HBM_PEAK_GBS,
                                              "traffic": load_traffic("kda_chunk_kernel.h",
                                                                      "k3_prefill_chunk_fwd_" + args.gate)}},
        }
        if fused and full:
            # the same layer with the model's in-kernel input preparation: q/k unit norm, beta
            # from its logits, state stored [V,K]
            bl = torch.logit(beta)
            fin_vk = torch.empty(B, H, V, K, dtype=torch.float32, device=dev)

            def pstep():
                kda.chunk_fwd_fused_gate(q, k, v, z, ls, bl, lower_bound=-5.0, chunk_size=args.chunk, out=out,
                                         final_state=fin_vk, qk_l2norm=True, beta_logits=True, state_vk=True,
                                         **(dict(workspace=wsp) if nws > 0 else dict(two_pass=False)))
            for _ in range(3):  # warm-up: the [V,K] final state and the variant's kernels
                pstep()
            torch.cuda.synchronize()
            pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
            for a_, b_ in pev:
                a_.record(stream)
                pstep()
                b_.record(stream)
            torch.cuda.synchronize()
            p_ms = sum(a_.elapsed_time(b_) for a_, b_ in pev) / len(pev)
            p_gbs = alg_bytes / (p_ms * 1e-3) / 1e9
            log("prefill with in-kernel preparation: %.3f ms" % p_ms)
            result["prefill_prepared_in_kernel"] = {
                "workload": "k3_prefill_B1_T8192_H96_K128_V128", "call": "chunk_fwd_fused_gate(qk_l2norm, beta_logits, "
                "state_vk)", "tokens_per_s": B * T / (p_ms * 1e-3), "launch_ms": p_ms,
                "roofline": {"bound": "hbm", "achieved": p_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": p_gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg_bytes}}
            del bl, fin_vk
        n64 = kda.chunk_fwd_workspace_size(q.dtype, B, T, H, K, V, 64)
        if fused and full and n64 > 0 and args.chunk != 64:
            # the same call at chunk size 64 (half the serial chunk steps, twice the A-matrix
            # work per chunk), beside the default
            w64 = torch.empty(n64, dtype=torch.uint8, device=dev)

            def cstep():
                kda.chunk_fwd_fused_gate(q, k, v, z, ls, beta, lower_bound=-5.0, initial_state=None, chunk_size=64,
                                         out=out, final_state=fin, workspace=w64)
            for _ in range(3):
                cstep()
            torch.cuda.synchronize()
            cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
            for a_, b_ in cev:
                a_.record(stream)
                cstep()
                b_.record(stream)
            torch.cuda.synchronize()
            c_ms = sum(a_.elapsed_time(b_) for a_, b_ in cev) / len(cev)
            c_gbs = alg_bytes / (c_ms * 1e-3) / 1e9
            log("prefill at chunk size 64: %.3f ms" % c_ms)
            result["prefill_chunk64"] = {
                "workload": "k3_prefill_B1_T8192_H96_K128_V128", "chunk_size": 64, "launch_ms": c_ms,
                "tokens_per_s": B * T / (c_ms * 1e-3),
                "roofline": {"bound": "hbm", "achieved": c_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": c_gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg_bytes}}
            del w64
    else:
        result = {"metric": "KDA prefill tokens/s (H=96,D=128) + % MFMA peak; decode state HBM GB/s",
                  "only": args.only, "n_gpus": 1, "dtype": "bf16", "data": "synthetic"}
    del g, out, wsp

    # ---------------- packed sequences: 8 sequences of 1,024-32,768 tokens --------------
    if not args.no_varlen and run("varlen"):
        log("generating packed-sequence inputs")
        vl = synth.varlen_stress(device="cuda")
        Tv = vl.q.shape[1]
        Nv = vl.num_seqs
        vo = torch.empty(1, Tv, H, V, dtype=torch.bfloat16, device=dev)
        vf = torch.empty(Nv, H, K, V, dtype=torch.float32, device=dev)
        vws_n = kda.chunk_fwd_workspace_size(vl.q.dtype, 1, Tv, H, K, V, args.chunk, num_seqs=Nv, varlen=True)
        vws = torch.empty(max(vws_n, 1), dtype=torch.uint8, device=dev)

        def vcall():
            kda.chunk_fwd_fused_gate(vl.q, vl.k, vl.v, vl.z, vl.log_scale, vl.beta, lower_bound=-5.0,
                                     cu_seqlens=vl.cu_seqlens, chunk_size=args.chunk, out=vo, final_state=vf,
                                     **(dict(workspace=vws) if vws_n > 0 else dict(two_pass=False)))
        vcall()
        torch.cuda.synchronize()
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        t0 = time.perf_counter()
        for a_, b_ in vev:
            a_.record(stream)
            vcall()
            b_.record(stream)
        torch.cuda.synchronize()
        vwall = (time.perf_counter() - t0) / len(vev)
        v_ms = sum(a_.elapsed_time(b_) for a_, b_ in vev) / len(vev)
        vth = Tv * H
        v_bytes = vth * (3 * 2 * K + 2 * K + 4 + 2 * V)   # the same 1,284 B per token-head as above
        v_gbs = v_bytes / (v_ms * 1e-3) / 1e9
        log("packed sequences (%d tokens): %.3f ms per call, %.0f GB/s" % (Tv, v_ms, v_gbs))
        result["varlen"] = {
            "workload": vl.name, "tokens": Tv, "sequences": Nv,
            "lengths": [int(x) for x in (vl.cu_seqlens[1:] - vl.cu_seqlens[:-1]).tolist()],
            "call": "chunk_fwd_fused_gate(cu_seqlens)", "tokens_per_s": Tv / (v_ms * 1e-3), "launch_ms": v_ms,
            "ms_per_call_wall": vwall * 1e3,
            "roofline": {"bound": "hbm", "achieved": v_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": v_gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": v_bytes}}
        if not args.no_cpu_baseline and args.only is None:
            import oracle
            from tests.helpers import f64
            hs = list(range(0, H, 4))  # 24 of the 96 heads, every sequence
            cu = vl.cu_seqlens.cpu().tolist()
            sl = lambda x: f64(x[:, :, hs])
            threads = oracle.max_threads()
            t0 = time.perf_counter()
            al = oracle.bounded_decay(sl(vl.z), f64(vl.log_scale)[hs], g_min=-5.0)
            qs, ks, vs, bs = sl(vl.q), sl(vl.k), sl(vl.v), sl(vl.beta)
            oracle.scan(qs, ks, vs, al, bs, cu_seqlens=cu)
            vcpu = (time.perf_counter() - t0) * H / len(hs)
            result["varlen"]["cpu_baseline"] = {
                "value": Tv / vcpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": "fp64 gate + token scan of %d of the %d heads over all %d sequences, scaled by %d/%d"
                          % (len(hs), H, Nv, H, len(hs))}
            del al, qs, ks, vs, bs
        del vl, vo, vf, vws

    # ---------------- the gate alone: bounded_decay over the same logits ----------------
    # (the separate elementwise kernel of the unfused path: bf16 logits in, float32
    # retention out, 6 B per element)
    if run("gate"):
        ga = torch.empty(B, T, H, K, dtype=torch.float32, device=dev)
        for _ in range(3):
            kda.bounded_decay(z, ls, lower_bound=-5.0, out=ga)
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a_, b_ in gev:
            a_.record(stream)
            kda.bounded_decay(z, ls, lower_bound=-5.0, out=ga)
            b_.record(stream)
        torch.cuda.synchronize()
        g_us = sum(a_.elapsed_time(b_) for a_, b_ in gev) / len(gev) * 1e3
        g_bytes = th * K * (2 + 4)
        g_gbs = g_bytes / (g_us * 1e-6) / 1e9
        log("bounded_decay: %.1f us per call, %.0f GB/s" % (g_us, g_gbs))
        result["bounded_decay"] = {
            "workload": "k3_prefill_B1_T8192_H96_K128 logits (bf16) -> alpha (fp32)", "calls": len(gev),
            "launch_us_avg": g_us,
            "roofline": {"bound": "hbm", "achieved": g_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": g_gbs / HBM_PEAK_GBS, "kernel": "bounded_decay_kernel",
                         "algorithmic_bytes_per_launch": g_bytes}}
        del ga

    # ---------------- backward ----------------------------------------------------------
    if not args.no_bwd and run("bwd"):
        # gradients of the same K3 prefill: bf16 q, k, v and d_out, float32 retention (the
        # gate tensor the backward takes), bf16 dq, dk, dv, float32 dgate and dbeta
        alpha_b = kda.bounded_decay(z, ls, lower_bound=-5.0)
        d_out_b, d_fin_b = synth.cotangents(B, T, H, V, K, 1, seed=7, device="cuda")
        d_out_b = d_out_b.to(torch.bfloat16)
        ws = torch.empty(kda.chunk_bwd_workspace_size(B, T, H, K, V), dtype=torch.uint8, device=dev)

        def bstep():
            return kda.chunk_bwd(q, k, v, alpha_b, beta, d_out_b, d_final_state=d_fin_b,
                                 grad_dtype=torch.bfloat16, workspace=ws)
        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a_, b_ in bev:
            a_.record(stream)
            bstep()
            b_.record(stream)
        torch.cuda.synchronize()
        b_ms = sum(a_.elapsed_time(b_) for a_, b_ in bev) / len(bev)
        # per token-head: q, k, v, d_out bf16 + alpha fp32 + beta in; dq, dk, dv bf16 + dgate fp32 + dbeta out
        b_bytes = th * (2 * (2 * K + V) + 4 * K + 4 + 2 * V + 2 * (2 * K + V) + 4 * K + 4)
        # dense products per 64-token chunk and head (C = 64): recomputed forward (A matrices, W, U,
        # states) and the reverse (state gradients, the V contractions, dT, dA, adjoints)
        C_, ckv, cck, ccv = 64, 2 * 64 * K * V, 64 * 64 * K, 64 * 64 * V   # flops of one full / triangular product
        per_chunk = (2 * cck + cck + ccv                    # prep: Abar, A_qk, W = T(.), U = T(.) (triangular)
                     + 2 * ckv                              # states: W S, Kd^T Vt
                     + 3 * ckv + ccv                        # dstates: Kd dS', Qg^T dO, W^T dVt, A_qk^T dO
                     + 3 * ckv + 4 * ccv + ccv              # vgrads: dO S^T, dVt S^T, Vt dS'^T, dO Vt^T, dVt V^T, T^T dVt
                     + 2 * cck + 4 * C_ ** 3 + cck + 4 * cck)  # kgrads: dT, T products, T^T dW, adjoints
        b_flops = (T // C_) * B * H * per_chunk
        b_tf = b_flops / (b_ms * 1e-3) / 1e12
        b_gbs = b_bytes / (b_ms * 1e-3) / 1e9
        log("backward: %.3f ms, %.1f TFLOP/s fp32 matrix, %.1f GB/s" % (b_ms, b_tf, b_gbs))
        result["prefill_backward"] = {
            "workload": "k3_prefill_B1_T8192_H96_K128_V128", "call": "chunk_bwd (5 kernels, float32)",
            "tokens_per_s": B * T / (b_ms * 1e-3), "launch_ms": b_ms,
            "roofline": {"bound": "mfma", "achieved": b_tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": b_tf / FP32_PEAK_TFLOPS, "algorithmic_flops_per_call": b_flops},
            "hbm": {"achieved": b_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": b_gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes_per_call": b_bytes}}
        del ws, alpha_b, d_out_b, d_fin_b

    # ---------------- decode ------------------------------------------------------------
    if not args.no_decode and run("decode"):
        nd = args.decode_steps
        log("generating decode inputs (%d steps)" % nd)
        dec = synth.decode(device="cuda", steps=nd)
        Bd, Hd = dec.q.shape[1], dec.q.shape[2]
        state = dec.state.clone()
        al = torch.empty(Bd, Hd, K, dtype=torch.float32, device=dev)
        od = torch.empty(Bd, Hd, V, dtype=torch.bfloat16, device=dev)

        def dstep(t, ev_pair=None):
            if not fused:
                kda.bounded_decay(dec.z[t], dec.log_scale, out=al)
            if ev_pair is not None:
                ev_pair[0].record(stream)
            if fused:
                kda.recurrent_step_fused_gate(dec.q[t], dec.k[t], dec.v[t], dec.z[t], dec.log_scale, dec.beta[t],
                                              state, out=od)
            else:
                kda.recurrent_step(dec.q[t], dec.k[t], dec.v[t], al, dec.beta[t], state, out=od)
            if ev_pair is not None:
                ev_pair[1].record(stream)

        for t in range(min(8, nd)):
            dstep(t)
        state.copy_(dec.state)
        torch.cuda.synchronize()
        devs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nd)]
        t0 = time.perf_counter()
        for t in range(nd):
            dstep(t, devs[t])
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        step_ms = sorted(a.elapsed_time(b) for a, b in devs)
        step_med = step_ms[len(step_ms) // 2]
        step_avg = sum(step_ms) / len(step_ms)
        # state read + write, q, k, v bf16, gate (bf16 logits or fp32), beta, out bf16
        pair_bytes = 2 * K * V * 4 + 2 * 2 * K + 2 * V + gate_bytes + 4 + 2 * V
        d_bytes = Bd * Hd * pair_bytes
        d_gbs = d_bytes / (step_avg * 1e-3) / 1e9
        dtraffic = load_traffic("kda_step.hip", "decode_recurrent_step_" + args.gate)
        log("decode: %.3f ms/step wall, step kernel avg %.1f us (median %.1f), %.0f GB/s" %
            (dwall * 1e3 / nd, step_avg * 1e3, step_med * 1e3, d_gbs))
        result["decode"] = {
            "workload": "decode_B64_H96_K128_V128_steps%d" % nd,
            "tokens_per_s": Bd * nd / dwall,
            "ms_per_step": dwall * 1e3 / nd,
            "step": "recurrent_step_fused_gate" if fused else "bounded_decay + recurrent_step",
            "roofline": {"bound": "hbm", "achieved": d_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_gbs / HBM_PEAK_GBS, "traffic": dtraffic, "kernel": "recurrent_step_kernel",
                         "launch_us_avg": step_avg * 1e3, "launch_us_median": step_med * 1e3,
                         "algorithmic_bytes_per_launch": d_bytes},
        }
        # a plain device copy of the same byte count, timed the same way, as a practical
        # reference for what read+write streaming reaches on this GPU (context only)
        half = d_bytes // 2
        src = torch.empty(half, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a_, b_ in cev:
            a_.record(stream)
            dst.copy_(src)
            b_.record(stream)
        torch.cuda.synchronize()
        copy_ms = sum(a_.elapsed_time(b_) for a_, b_ in cev) / len(cev)
        result["decode"]["device_copy_GBps_same_bytes"] = 2 * half / (copy_ms * 1e-3) / 1e9
        if fused:
            # the step with the model's in-kernel preparation and the state stored [V,K]
            st_vk = state.transpose(-1, -2).contiguous()
            blog = torch.logit(dec.beta)
            vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min(64, nd))]
            for t, (a_, b_) in enumerate(vev):
                a_.record(stream)
                kda.recurrent_step_fused_gate(dec.q[t], dec.k[t], dec.v[t], dec.z[t], dec.log_scale, blog[t], st_vk,
                                              out=od, qk_l2norm=True, beta_logits=True, state_vk=True)
                b_.record(stream)
            torch.cuda.synchronize()
            skip = 4 if len(vev) > 8 else 0  # the first steps after the layout change warm up
            v_us = sum(a_.elapsed_time(b_) for a_, b_ in vev[skip:]) / (len(vev) - skip) * 1e3
            v_gbs = d_bytes / (v_us * 1e-6) / 1e9
            log("decode with in-kernel preparation, [V,K] state: %.1f us per step" % v_us)
            result["decode_prepared_in_kernel"] = {
                "workload": "decode_B64_H96_K128_V128", "call": "recurrent_step_fused_gate(qk_l2norm, beta_logits, "
                "state_vk)", "launch_us_avg": v_us,
                "roofline": {"bound": "hbm", "achieved": v_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": v_gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": d_bytes}}
            del st_vk, blog
        if not args.no_cpu_baseline and args.only is None:
            # the oracle on a sample of the (sequence, head) pairs: the same 256 steps from the
            # same kept state, one token scan per pair
            import oracle
            from tests.helpers import f64
            npairs = 192
            threads = oracle.max_threads()
            t0 = time.perf_counter()
            for i in range(npairs):
                b_i, h_i = (i * 37) % Bd, (i * 53) % Hd
                slx = lambda x: f64(x[:, b_i:b_i + 1, h_i:h_i + 1]).swapaxes(0, 1)  # [1, steps, 1, ...]
                al_ = oracle.bounded_decay(slx(dec.z), f64(dec.log_scale[h_i:h_i + 1]), g_min=-5.0)
                oracle.scan(slx(dec.q), slx(dec.k), slx(dec.v), al_, slx(dec.beta), f64(dec.state[b_i:b_i + 1, h_i:h_i + 1]))
            d_cpu = (time.perf_counter() - t0) * (Bd * Hd) / npairs
            result["decode"]["cpu_baseline"] = {
                "value": Bd * nd / d_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": "%d of the %d (sequence, head) pairs over all %d steps, scaled" % (npairs, Bd * Hd, nd)}
        del dec, state, src, dst

    # ---------------- short continuations: the token-recurrent prefill ------------------
    if not args.no_short and run("short"):
        log("generating short-continuation inputs")
        sp = synth.short_prompts(device="cuda")
        Bs, Ts, Hs = sp.q.shape[0], sp.q.shape[1], sp.q.shape[2]
        so = torch.empty(Bs, Ts, Hs, V, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(Bs, Hs, K, V, dtype=torch.float32, device=dev)

        def rcall():
            if fused:
                kda.recurrent_fwd_fused_gate(sp.q, sp.k, sp.v, sp.z, sp.log_scale, sp.beta, lower_bound=-5.0,
                                             initial_state=sp.initial_state, out=so, final_state=sf)
            else:
                kda.recurrent_fwd(sp.q, sp.k, sp.v, sg, sp.beta, initial_state=sp.initial_state, out=so,
                                  final_state=sf)

        if not fused:
            sg = kda.bounded_decay(sp.z, sp.log_scale, lower_bound=-5.0)
        for _ in range(3):
            rcall()
        torch.cuda.synchronize()
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        t0 = time.perf_counter()
        for a_, b_ in rev:
            a_.record(stream)
            rcall()
            b_.record(stream)
        torch.cuda.synchronize()
        rwall = time.perf_counter() - t0
        r_ms = sum(a_.elapsed_time(b_) for a_, b_ in rev) / len(rev)
        # per (sequence, head): state read + write, and per token q, k, v, gate, beta, out
        r_bytes = Bs * Hs * (2 * K * V * 4 + Ts * (3 * 2 * K + gate_bytes + 4 + 2 * V))
        r_gbs = r_bytes / (r_ms * 1e-3) / 1e9
        log("short continuations: %.1f us per call, %.0f GB/s" % (r_ms * 1e3, r_gbs))
        result["short_continuations"] = {
            "workload": sp.name, "call": "recurrent_fwd_fused_gate" if fused else "recurrent_fwd",
            "tokens_per_s": Bs * Ts / (r_ms * 1e-3), "us_per_call": r_ms * 1e3,
            "roofline": {"bound": "hbm", "achieved": r_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": r_gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("kda_recurrent.hip", "short_recurrent_fwd_" + args.gate),
                         "kernel": "recurrent_fwd_kernel",
                         "algorithmic_bytes_per_launch": r_bytes},
        }
        del so, sf

    # ---------------- CPU baseline: the oracle on a head sample -------------------------
    if not args.no_cpu_baseline and args.only is None:
        import oracle
        from tests.helpers import f64
        hs = list(range(0, H, max(1, H // args.cpu_heads)))[:args.cpu_heads]
        log("cpu baseline: oracle on %d of %d heads" % (len(hs), H))
        qs, ks, vs, zs = (f64(x[:, :, hs]) for x in (q, k, v, z))
        bs = f64(beta[:, :, hs])
        lss = f64(ls)[hs]
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        alpha = oracle.bounded_decay(zs, lss, g_min=-5.0)
        oracle.scan(qs, ks, vs, alpha, bs)
        cpu_s = time.perf_counter() - t0
        cpu_tps = B * T / (cpu_s * H / len(hs))
        result["cpu_baseline"] = {"value": cpu_tps, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "sample": "fp64 gate + token scan of %d of the %d heads (T=8192), %.1f s wall, "
                                            "scaled by %d/%d" % (len(hs), H, cpu_s, H, len(hs))}
        if not args.no_short and run("short"):
            # the same oracle on a sample of the short-continuation (sequence, head) pairs
            npairs = 48
            t0 = time.perf_counter()
            for i in range(npairs):
                b_i, h_i = (i * 37) % Bs, (i * 53) % Hs
                sl = lambda x: f64(x[b_i:b_i + 1, :, h_i:h_i + 1])
                al = oracle.bounded_decay(sl(sp.z), f64(sp.log_scale[h_i:h_i + 1]), g_min=-5.0)
                oracle.scan(sl(sp.q), sl(sp.k), sl(sp.v), al, sl(sp.beta),
                            f64(sp.initial_state[b_i:b_i + 1, h_i:h_i + 1]))
            r_cpu = (time.perf_counter() - t0) * (Bs * Hs) / npairs
            result["short_continuations"]["cpu_baseline"] = {
                "value": Bs * Ts / r_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": "%d of the %d (sequence, head) pairs, scaled" % (npairs, Bs * Hs)}
        log("cpu baseline %.1f tokens/s (%.1f s on %d threads)" % (cpu_tps, cpu_s, threads))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
