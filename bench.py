"""Benchmark of the draft-then-verify attention hot path on one MI355X.

One step = one round of the path over one batch: k draft decode-attention
calls over the lossy cache (rotating over 4 identical copies of that cache, as
consecutive layers would, so the 256 MB Infinity Cache cannot serve them), one
causal verify-attention call over the full bf16 cache and one accept call.
The vocab projection that turns attention outputs into logits is not part of
the path; it runs once before timing to produce the draft ids and the verify
logits that accept consumes.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE = 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="llama3_8b_layer_b8_l32k_int2_k32")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-units", type=int, default=8, help="(b, kv-head) units in the CPU oracle sample")
    return p.parse_args()


def cpu_baseline(w, dw, n_accept_sum, units):
    """Time the fp64 oracle on a bounded sample of the same workload: for `units`
    (b, kv-head) slices, every draft step of the round and the verify pass (the
    compressor is not timed on either side).  Scaled to the whole batch."""
    import numpy as np
    from oracle import round as R
    import oracle.vc_oracle as O
    np_ = dw.np
    g = w.g
    picks = [(u // w.Hkv, u % w.Hkv) for u in range(min(units, w.B * w.Hkv))]
    comps = {}
    for (b, h) in picks:
        if w.kind == "quant":
            comps[(b, h)] = R.unit_compressed(w, np_["K"][b, h], np_["V"][b, h])
    t0 = time.perf_counter()
    for (b, h) in picks:
        keep = dw.keep_np[b, h] if w.kind == "token_drop" else None
        R.unit_draft(w, np_["K"][b, h], np_["V"][b, h], np_["Kn"][b, h], np_["Vn"][b, h],
                     np_["Q"][b, h * g:(h + 1) * g], keep=keep, comp=comps.get((b, h)))
        R.unit_verify(w, np_["K"][b, h], np_["V"][b, h], np_["Kn"][b, h], np_["Vn"][b, h],
                      np_["Q"][b, h * g:(h + 1) * g])
    dt = time.perf_counter() - t0
    full = dt * (w.B * w.Hkv) / len(picks)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": (n_accept_sum + w.B) / full, "unit": "verified tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(picks)} of {w.B * w.Hkv} (batch, kv-head) units, {w.k} draft steps + verify, "
                      f"fp64 numpy, {dt:.1f} s measured, scaled x{(w.B * w.Hkv) / len(picks):.0f}"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the hot path is per-GPU data parallel with no exchange; "
              f"--gpus {a.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import compressed_kv_draft_amd as vc
    from compressed_kv_draft_amd import workload as WL
    from synth import configs as C

    w = C.ALL[a.config]
    torch.cuda.set_device(0)
    dw = WL.DeviceWorkload(w, device="cuda:0")
    comps = [dw.comp] + [WL.clone_compressed(dw.comp) for _ in range(ROTATE - 1)]

    # untimed: draft ids and verify logits through the harness vocab projection
    for j in range(w.k):
        dw.draft_step(j)
    d_ids = vc.argmax(dw.draft_logits().contiguous()).reshape(w.B, w.k)
    dw.verify()
    vlog = dw.verify_logits()
    out_ids = torch.empty((w.B, w.n_q), dtype=torch.int32, device="cuda:0")
    n_acc = torch.empty(w.B, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = []

    def step(record):
        for j in range(w.k):
            c = comps[j % ROTATE]
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            vc.draft_attn(c, dw.tails[j], dw.q_steps[j], dw.scale, out=dw.draft_out[j], ws=dw.draft_ws,
                          Hkv=w.Hkv)
            if record:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record(stream)
                ev.append(("draft", j, e0, e1))
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        dw.verify()
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            ev.append(("verify", 0, e0, e1))
        vc.accept(d_ids, vlog, out_ids=out_ids, n_accept=n_acc)

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    n = n_acc.cpu().numpy().astype(np.int64)
    tokens_per_step = int((n + 1).sum())
    wall = t1 - t0
    ms = 1e3 * wall / a.steps
    value = tokens_per_step * a.steps / wall
    d_ms = [e0.elapsed_time(e1) for (k_, j, e0, e1) in ev if k_ == "draft"]
    v_ms = [e0.elapsed_time(e1) for (k_, j, e0, e1) in ev if k_ == "verify"]
    d_avg = float(np.mean(d_ms)) * 1e-3
    v_avg = float(np.mean(v_ms)) * 1e-3
    d_bytes = float(np.mean([WL.draft_step_bytes(w, j) for j in range(w.k)]))
    v_bytes = float(WL.verify_bytes(w))
    d_gbs = d_bytes / d_avg / 1e9
    v_gbs = v_bytes / v_avg / 1e9
    draft_total = sum(d_ms) / a.steps
    verify_total = sum(v_ms) / a.steps
    dominant = "draft" if draft_total >= verify_total else "verify"
    roof = {"bound": "hbm", "kernel": "vc_draft_attn (draft_mfma_kernel + draft_combine_kernel)"
            if dominant == "draft" else "vc_verify_attn (verify_mfma_kernel + verify_combine_kernel)",
            "achieved": round(d_gbs if dominant == "draft" else v_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round((d_gbs if dominant == "draft" else v_gbs) / HBM_PEAK_GBS, 4), "traffic": None,
            "bytes_per_launch": int(d_bytes if dominant == "draft" else v_bytes),
            "avg_launch_us": round(1e6 * (d_avg if dominant == "draft" else v_avg), 2)}
    step_s = wall / a.steps
    line = {
        "metric": "verified tokens/sec per GPU; draft/verify attention HBM TB/s vs peak",
        "value": round(value, 1), "unit": "verified tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "context": w.L, "draft_len": w.k, "draft_cache": f"{w.kind}{w.bits if w.kind == 'quant' else ''}",
                   "residual": w.residual, "vocab": w.vocab, "layers_rotated": ROTATE,
                   "step": "k x vc_draft_attn + vc_verify_attn + vc_accept (one layer; vocab projection outside)",
                   "arithmetic": "draft: int2 codes as exact f16 MFMA operands, q*s and p*s as f16 hi+lo; "
                                 "verify: bf16 q.k, f16 p.v MFMA; fp32 accumulate and softmax"},
        "accept": {"n_accept": n.tolist(), "tokens_per_step": tokens_per_step,
                   "tokens_per_s_at_n_eq_k": round(w.B * w.n_q / step_s, 1),
                   "tokens_per_s_at_n_eq_25": round(w.B * 26 / step_s, 1)},
        "draft": {"avg_us": round(1e6 * d_avg, 2), "GBps": round(d_gbs, 1), "frac_hbm": round(d_gbs / HBM_PEAK_GBS, 4),
                  "bytes": int(d_bytes), "ms_per_step": round(draft_total, 4)},
        "verify": {"avg_us": round(1e6 * v_avg, 2), "GBps": round(v_gbs, 1), "frac_hbm": round(v_gbs / HBM_PEAK_GBS, 4),
                   "bytes": int(v_bytes), "TFLOPs": round(WL.verify_flops(w) / v_avg / 1e12, 1),
                   "ms_per_step": round(verify_total, 4)},
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, dw, int(n.sum()), a.cpu_units)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
