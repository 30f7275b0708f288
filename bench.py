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
    p.add_argument("--warmup", type=int, default=25, help="untimed rounds; the clocks settle within ~50 ms of load")
    p.add_argument("--config", default=None,
                   help="time one round of this single-layer workload instead of the default headline (the "
                        "staggered two-group cycle of the Llama-70B-shaped layer plus the other long-context rounds)")
    p.add_argument("--legs", default="llama3_8b_layer_b8_l32k_int2_k32,qwen_32b_layer_b4_l128k_drop10_k32",
                   help="single-layer rounds reported beside the headline cycle (comma-separated; empty for none)")
    p.add_argument("--leg-steps", type=int, default=10)
    p.add_argument("--leg-warmup", type=int, default=15)
    p.add_argument("--leg-cpu-units", type=int, default=2)
    p.add_argument("--pace", type=int, default=8,
                   help="staggered cycle: draft calls issued before each chunk's verify (0: all k in one burst); "
                        "bursts longer than ~1.5 ms set off the GPU's power management (per-call time 134 -> 184 us)")
    p.add_argument("--no-e2e-leg", action="store_true",
                   help="leave out the tiny decoder's end-to-end rate from the default line")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="replay each phase of the round (k draft calls, verify, accept) as a recorded HIP graph "
                        "instead of issuing every call from the host (measured about 2 %% slower: with no gaps "
                        "between kernels the clocks settle lower)")
    p.add_argument("--no-full-kv-decode", action="store_true",
                   help="skip the full-KV decode baseline (keeps per-kernel profiles to the path's own calls)")
    p.add_argument("--cpu-units", type=int, default=None,
                   help="(b, kv-head) units in the CPU oracle sample (default 8 for a round, 24 for the cycle: "
                        "about 10-15 s of oracle work)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy, 3 times (the reference kernel for "
                        "scaling the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    p.add_argument("--steps-e2e", type=int, default=3)
    p.add_argument("--warmup-e2e", type=int, default=1)
    p.add_argument("--e2e", action="store_true",
                   help="end-to-end draft-then-verify generation with the tiny decoder (256 tokens, int4 draft, "
                        "k = 32): verified tokens/s and the acceptance histogram instead of the per-layer line")
    p.add_argument("--e2e-groups", action="store_true",
                   help="two request groups of the tiny decoder: lock-step vs staggered on two streams, fixed vs "
                        "adaptive draft length (vc_sched_choose_k); prints that JSON line instead")
    p.add_argument("--stagger", action="store_true",
                   help="measure the full-KV prefetch of one request group against the other group's drafting "
                        "(Llama-70B-shaped paged workload) and print that JSON line instead")
    return p.parse_args()


def stagger(a):
    """Cross-resource staggering on one GPU: group B's full KV (shuffled 16-token
    pages, pinned host pool) streams to the device pool on a copy stream while
    group A runs its k draft steps on the compute stream.  Times draft alone,
    copy alone and both together; overlap = 1 - (t_both - t_copy) / min(t_d, t_c), the
    difference taken over paired runs.
    Then group B's verify: once after all its chunks have landed, and chunk by
    chunk (vc_verify_attn_range on each 4096-key chunk as soon as it lands, the
    new rows as one more range, then vc_verify_merge).  The verify's tail is the
    GPU time from the last chunk landing to the verified output: after the whole
    copy it is the whole verify; chunk by chunk it is one chunk's share plus the
    new rows and the merge.  Hidden share = 1 - tail / t_verify."""
    import numpy as np
    import torch

    import compressed_kv_draft_amd as vc
    from compressed_kv_draft_amd import workload as WL
    from synth import configs as C
    from synth import inputs as I

    w = C.LLAMA70B
    bg = w.B // w.groups
    torch.cuda.set_device(0)
    # group A: its int4 draft cache (contiguous) and tail
    wa = w.with_(B=bg, paged=False)
    dw = WL.DeviceWorkload(wa, device="cuda:0", with_vocab=False)
    # group B: the paged full KV of sequences bg .. 2bg-1 in a pinned host pool
    table, n_slots = I.page_table(w)
    page_bytes = w.Hkv * 2 * w.page_tokens * w.D * 2
    host = torch.empty(n_slots * page_bytes, dtype=torch.uint8)
    host.fill_(0x3C)
    seqs = list(range(bg, 2 * bg))
    chunks = [(t, min(t + w.chunk_tokens, w.L)) for t in range(0, w.L, w.chunk_tokens)]
    pages_per_chunk = len(seqs) * (w.chunk_tokens // w.page_tokens)
    n_pages = pages_per_chunk * len(chunks)
    copy_bytes = n_pages * page_bytes
    chunk_bytes = pages_per_chunk * page_bytes
    # group B's device pool: its chunks one after the other, then the pages of
    # the new rows (device-only); a device page table points the paged verify here
    ctx_pages = w.L // w.page_tokens
    pps = table.shape[1]
    extra = pps - ctx_pages
    seq_chunk_pages = w.chunk_tokens // w.page_tokens
    pool_b = torch.empty((n_pages + bg * extra) * page_bytes, dtype=torch.uint8, device="cuda:0")
    pool_b[copy_bytes:].fill_(0x3C)
    dev_region = pool_b[:copy_bytes]
    tab_b = np.empty((bg, pps), dtype=np.int32)
    for i in range(bg):
        p = np.arange(ctx_pages)
        tab_b[i, :ctx_pages] = (p // seq_chunk_pages) * pages_per_chunk + i * seq_chunk_pages + p % seq_chunk_pages
        tab_b[i, ctx_pages:] = n_pages + i * extra + np.arange(extra)
    full_b = vc.FullKV(pool_b, None, 0, torch.from_numpy(tab_b).to("cuda:0"), w.page_tokens, pps,
                       n_pages + bg * extra)
    q_b = torch.randn((bg, w.Hq, w.n_q, w.D), device="cuda:0").to(torch.bfloat16)
    ctx_b = torch.full((bg,), w.L, dtype=torch.int32, device="cuda:0")
    scale = float(np.float32(1.0 / np.sqrt(w.D)))
    # three staging buffers: the gather of chunk c waits only for the copy of c - 3
    n_stage = 3
    staging = [torch.empty(chunk_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(n_stage)]
    landed = [torch.cuda.Event() for _ in chunks]     # chunk c is on the device
    comp = torch.cuda.current_stream()
    cps = torch.cuda.Stream()

    def drafts():
        for j in range(w.k):
            dw.draft_step(j)

    def copy_chunk(c):
        t0, t1 = chunks[c]
        vc.prefetch_full_kv(host, page_bytes, table, seqs, t0, t1, w.page_tokens, staging[c % n_stage],
                            dev_region[c * chunk_bytes:(c + 1) * chunk_bytes], stream=cps, done_event=landed[c],
                            staging_free=landed[c - n_stage] if c >= n_stage else None)

    def copies():
        for c in range(len(chunks)):
            copy_chunk(c)

    def timed(fn, stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), 1e3 * (time.perf_counter() - t0)

    drafts()
    copies()
    torch.cuda.synchronize()
    # the k draft steps as one HIP graph: one submission from the host
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        drafts()
    torch.cuda.synchronize()
    drafts_eager = drafts

    def drafts():
        graph.replay()

    graph.replay()
    torch.cuda.synchronize()
    ref = dw.draft_out.clone()
    drafts_eager()
    torch.cuda.synchronize()
    if not torch.equal(ref, dw.draft_out):
        raise RuntimeError("graph replay of the draft steps differs from eager execution")
    reps = max(1, a.steps)
    td = float(np.median([timed(drafts, comp)[0] for _ in range(reps)]))
    tc = float(np.median([timed(copies, cps)[1] for _ in range(reps)]))   # wall: includes the host gather
    big = staging[0]
    tref = float(np.median([timed(lambda: dev_region[:chunk_bytes].copy_(big, non_blocking=True), comp)[0]
                            for _ in range(reps)]))
    import threading
    # copy alone and copy + drafts alternate, so that the slow drift of the PCIe
    # rate (a few ms over a 40 ms copy) cancels in the paired differences
    both, d_in, alone = [], [], []
    for _ in range(reps):
        alone.append(timed(copies, cps)[1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        # the prefetch runs on its own host thread (its gathers and copy submissions
        # release the GIL), as a serving runtime's prefetcher would
        th = threading.Thread(target=copies)
        th.start()
        dA0, dA1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dA0.record(comp)
        drafts()
        dA1.record(comp)
        th.join()
        torch.cuda.synchronize()
        both.append(1e3 * (time.perf_counter() - t0))
        d_in.append(dA0.elapsed_time(dA1))
    tb = float(np.median(both))
    tdi = float(np.median(d_in))
    extra = float(np.median(np.array(both) - np.array(alone)))   # what the drafts added to the copy
    overlap = (min(td, tc) - extra) / min(td, tc)

    # group B's verify: whole, after all chunks; and chunk by chunk as they land
    ranges = chunks + [(w.L, w.L + w.n_q)]
    slots = [vc.verify_range_parts(bg, w.Hq, w.Hkv, w.D, w.n_q, t0, t1) for t0, t1 in ranges]
    row_f = bg * w.Hq * w.n_q * (w.D + 2)
    parts = torch.empty(sum(slots) * row_f, dtype=torch.float32, device="cuda:0")
    out_whole = torch.empty((bg, w.Hq, w.n_q, w.D), dtype=torch.float32, device="cuda:0")
    out_pipe = torch.empty_like(out_whole)
    last_landed = torch.cuda.Event(enable_timing=True)
    merged = torch.cuda.Event(enable_timing=True)

    def verify_whole():
        vc.verify_attn(q_b, full_b, ctx_b, w.L, w.Hkv, scale, out=out_whole)

    def copies_flagged(flags):
        for c in range(len(chunks)):
            copy_chunk(c)
            if c == len(chunks) - 1:
                last_landed.record(cps)
            flags[c].set()

    def pipelined():
        flags = [threading.Event() for _ in chunks]
        th = threading.Thread(target=copies_flagged, args=(flags,))
        th.start()
        off = 0
        for c, ((t0, t1), n) in enumerate(zip(ranges, slots)):
            if c < len(chunks):
                flags[c].wait()             # the chunk's copy (and its event) is enqueued
                comp.wait_event(landed[c])  # ... and the verify of its keys waits for it to land
            vc.verify_attn_range(q_b, full_b, ctx_b, w.L, w.Hkv, scale, t0, t1, parts[off * row_f:])
            off += n
        vc.verify_merge(parts, sum(slots), bg, w.Hq, w.n_q, w.D, out=out_pipe)
        merged.record(comp)
        th.join()

    copies()
    torch.cuda.synchronize()
    verify_whole()
    pipelined()
    torch.cuda.synchronize()
    rel = float(torch.linalg.norm(out_pipe - out_whole) / torch.linalg.norm(out_whole))
    if not rel < 1e-5:
        raise RuntimeError(f"chunked verify differs from the whole verify: rel L2 {rel:.2e}")
    tv = float(np.median([timed(verify_whole, comp)[0] for _ in range(reps)]))
    serial, pipe, tails = [], [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        copies()
        comp.wait_stream(cps)
        verify_whole()
        torch.cuda.synchronize()
        serial.append(1e3 * (time.perf_counter() - t0))
        t0 = time.perf_counter()
        pipelined()
        torch.cuda.synchronize()
        pipe.append(1e3 * (time.perf_counter() - t0))
        tails.append(last_landed.elapsed_time(merged))
    ts, tp, tt = float(np.median(serial)), float(np.median(pipe)), float(np.median(tails))
    line = {"metric": "full-KV prefetch overlap with draft compute (cross-resource staggering, one GPU)",
            "value": round(overlap, 4), "unit": "fraction of the shorter activity hidden", "n_gpus": 1,
            "steps": reps, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": w.name + "_stagger", "draft_group": f"seqs 0..{bg - 1}, int4, k={w.k}",
                       "prefetch_group": f"seqs {bg}..{2 * bg - 1}, {len(chunks)} chunks of {w.chunk_tokens} "
                                         f"tokens, {n_pages} shuffled pages of {page_bytes} B"},
            "t_draft_ms": round(td, 3), "t_copy_ms": round(tc, 3), "t_both_ms": round(tb, 3),
            "verify_ms": round(tv, 3), "copy_then_verify_ms": round(ts, 3), "chunked_verify_ms": round(tp, 3),
            "chunked_verify_tail_ms": round(tt, 3), "verify_hidden_fraction": round(1.0 - tt / tv, 4),
            "chunked_vs_whole_rel_l2": rel,
            "chunked_verify": f"{len(chunks)} ranges of {w.chunk_tokens} keys as they land + new rows + merge, "
                              f"{sum(slots)} partial slots",
            "draft_under_copy_ms": round(tdi, 3), "draft_slowdown": round(tdi / td, 4),
            "prefetch_GBps": round(copy_bytes / tc / 1e6, 2),
            "pcie_GBps_one_chunk_copy": round(chunk_bytes / tref / 1e6, 2),
            "copy_bytes": int(copy_bytes)}
    print(json.dumps(line), flush=True)


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 3}),
          flush=True)


TRAFFIC_SOURCES = {"draft": ("draft.hip", "lds_dma.h", "mfma.h", "vc_common.h"),
                   "verify": ("verify.hip", "lds_dma.h", "mfma.h", "vc_common.h")}


def kernel_source_digest(kind="draft"):
    """sha256 of a kernel's sources and of the compiler flags of its file: ties a
    stored counter reading to the code it was taken on."""
    import hashlib
    from compressed_kv_draft_amd import build as B
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, "compressed_kv_draft_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(B.FLAGS + B.FILE_FLAGS.get(TRAFFIC_SOURCES[kind][0], [])).encode())
    return h.hexdigest()


def stored_traffic(workload: str, kind: str = "draft"):
    """HBM bytes per vc_draft_attn (kind "draft") or vc_verify_attn ("verify") call
    from the committed counter summary profiles/hbm_traffic_<kind>_<workload>.txt,
    or None when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kind}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_digest(kind):
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


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
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import compressed_kv_draft_amd.workload as WL
    round_bytes = sum(WL.draft_step_bytes(w, j) for j in range(w.k)) + WL.verify_bytes(w)
    return {"value": (n_accept_sum + w.B) / full, "unit": "verified tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": model,
            "effective_GBps": round(round_bytes / full / 1e9, 3),
            "sample": f"{len(picks)} of {w.B * w.Hkv} (batch, kv-head) units, {w.k} draft steps + verify, "
                      f"fp64 numpy, {dt:.1f} s measured, scaled x{(w.B * w.Hkv) / len(picks):.0f}"}


def e2e_record(steps: int, warmup: int, with_eager: bool = True):
    """Tiny decoder end to end: prefill, then 256 greedy tokens by the loop.
    Every attention and token decision runs in libvc; the dense layers are
    torch fp32.  Drafting replays one recorded HIP graph per position (the
    eager rate is reported beside it when with_eager).  Returns decode
    tokens/s (prefill excluded), the accepted-count histogram, and whether the
    tokens equal the stored oracle sequence."""
    import numpy as np
    import torch

    from compressed_kv_draft_amd.tinylm import TinyLM
    from synth import configs as C
    from synth import model as M
    cfg = C.LM_E2E
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    prompt = M.prompt(cfg)

    def timed(graph):
        runs = []
        for i in range(warmup + steps):
            lm = TinyLM(cfg, W, cos, sin)
            toks, acc, st = lm.generate(prompt, cfg.n_gen, graph=graph)
            if i >= warmup:
                runs.append((toks, acc, st))
            del lm
            torch.cuda.empty_cache()
        return runs
    eager = timed(False) if with_eager else []
    runs = timed(True)
    gold = None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", f"e2e_{cfg.name}.txt")
    if os.path.exists(path):
        for line in open(path):
            if line.startswith("tokens="):
                gold = [int(x) for x in line.split("=", 1)[1].split()]
    dec = [r[2]["decode_s"] for r in runs]
    toks, acc, st = runs[int(np.argmin(dec))]
    hist = {str(k): int(v) for k, v in zip(*np.unique(acc, return_counts=True))}
    rec = {"metric": "end-to-end verified tokens/s (tiny decoder, draft-then-verify, greedy)",
           "value": round((cfg.n_gen - 1) / min(dec), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "higher_is_better": True, "data": "synthetic",
           "config": {"workload": cfg.name, "layers": cfg.n_layers, "d_model": cfg.d_model, "q_heads": cfg.Hq,
                      "kv_heads": cfg.Hkv, "head_dim": cfg.D, "ffn": cfg.ffn, "vocab": cfg.vocab,
                      "prompt": cfg.prompt, "draft_len": cfg.k, "generated": cfg.n_gen, "draft_cache": "int4",
                      "dense_layers": "torch fp32 (outside the measured path)"},
           "rounds": st["rounds"], "accepted_per_round": acc, "accepted_histogram": hist,
           "mean_tokens_per_round": round(float(np.mean(np.array(acc) + 1)), 2),
           "decode_s": [round(x, 4) for x in dec], "prefill_s": round(st["prefill_s"], 4),
           "drafting": "one HIP graph per draft position, replayed k times per round",
           "equals_oracle_greedy": (toks == gold) if gold is not None else None}
    if with_eager:
        rec["eager_value"] = round((cfg.n_gen - 1) / min(r[2]["decode_s"] for r in eager), 1)
        rec["graph_equals_eager"] = all(r[0] == toks and r[1] == acc for r in eager)
    return rec


def e2e(a):
    print(json.dumps(e2e_record(a.steps_e2e, a.warmup_e2e)), flush=True)


def e2e_groups(a):
    """Two request groups of the tiny decoder (prompts 0 and 1, 256 tokens
    each), decode only: lock-step on one stream with k = 32, staggered on two
    streams with k = 32, and staggered with the draft length chosen per round
    by vc_sched_choose_k from each group's acceptance history and event-timed
    phases; then lock-step and staggered-adaptive again with the full caches
    in pinned host memory, copied into one shared device region before each
    verification (the copy beside the other group's drafting when staggered).  Reports summed tokens/s, the draft lengths used, and whether every
    run emitted the same tokens (group 0 also against the stored oracle
    sequence)."""
    import numpy as np
    import torch

    from compressed_kv_draft_amd.groups import StaggeredGroups
    from compressed_kv_draft_amd.tinylm import FullStaging, TinyLM
    from synth import configs as C
    from synth import model as M
    cfg = C.LM_E2E
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    prompts = [M.prompt(cfg, r) for r in (0, 1)]
    gold = None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", f"e2e_{cfg.name}.txt")
    if os.path.exists(path):
        for line in open(path):
            if line.startswith("tokens="):
                gold = [int(x) for x in line.split("=", 1)[1].split()]
    modes = {"lockstep_k32": (False, cfg.k, cfg.k, False), "staggered_k32": (True, cfg.k, cfg.k, False),
             "staggered_adaptive": (True, 1, cfg.k, False),
             "lockstep_k32_host_full_kv": (False, cfg.k, cfg.k, True),
             "staggered_adaptive_host_full_kv": (True, 1, cfg.k, True)}
    out, toks_ref = {}, None
    same = True
    for name, (stag, kmin, kmax, host) in modes.items():
        best = None
        for i in range(a.warmup_e2e + a.steps_e2e):
            st = FullStaging(cfg) if host else None
            base = TinyLM(cfg, W, cos, sin, staging=st)
            lms = [base, TinyLM(cfg, None, None, None, shared=base, staging=st)]
            res = StaggeredGroups(lms, k_min=kmin, k_max=kmax, stagger=stag).run(prompts, cfg.n_gen)
            toks = [[int(x) for x in t] for t in res["tokens"]]
            toks_ref = toks if toks_ref is None else toks_ref
            same = same and toks == toks_ref
            if i >= a.warmup_e2e and (best is None or res["wall_s"] < best["wall_s"]):
                best = res
            del lms, base, st
            torch.cuda.empty_cache()
        out[name] = {"tokens_per_s": round(best["tokens_per_s"], 1), "decode_s": round(best["wall_s"], 4),
                     "rounds": [len(r) for r in best["rounds"]],
                     "k_per_round": [[r["k"] for r in g] for g in best["rounds"]],
                     "mean_tokens_per_round": [round(float(np.mean([r["n"] + 1 for r in g])), 2)
                                               for g in best["rounds"]]}
        print(f"[e2e-groups] {name}: {out[name]['tokens_per_s']} tokens/s", flush=True)
    line = {"metric": "end-to-end verified tokens/s, two request groups (tiny decoder, greedy)",
            "value": out["staggered_adaptive"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": a.steps_e2e, "warmup": a.warmup_e2e, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": cfg.name + "_x2_groups", "groups": 2, "prompt": cfg.prompt,
                       "generated_per_group": cfg.n_gen, "k_max": cfg.k,
                       "dense_layers": "torch fp32 (outside the measured path)"},
            "modes": out, "all_runs_same_tokens": same,
            "group0_equals_oracle_greedy": (toks_ref[0] == gold) if gold is not None else None}
    print(json.dumps(line), flush=True)


def full_kv_decode(w, dw, value, step_s, launches=20, graph=False):
    """Baseline without drafting: one decode step reads the whole bf16 cache
    (vc_draft_attn with the identity compressor over the L context rows plus the
    current row) and yields one token per sequence.  Returns its timing and
    tokens/s, and the speed-up of the draft-then-verify step over it."""
    import torch

    import compressed_kv_draft_amd as vc
    dev = dw.full_k.device
    ident = vc.identity_cache(dw.full_k, dw.full_v, w.L + 1)
    no_tail = vc.Tail()
    ws = torch.zeros(vc.draft_ws_bytes(w.B, w.Hq, w.Hkv, w.D, w.L + 1), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    q = dw.q_steps[0]
    stream = torch.cuda.current_stream()
    def run():
        for _ in range(launches):
            vc.draft_attn(ident, no_tail, q, dw.scale, out=out, ws=ws, Hkv=w.Hkv)
    run()
    if graph:   # launched the same way as the path's own phases
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        run = g.replay
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    nbytes = w.B * w.Hkv * (w.L + 1) * w.D * 2 * 2
    tps = w.B / t
    return {"avg_us": round(1e6 * t, 2), "bytes": nbytes, "GBps": round(nbytes / t / 1e9, 1),
            "tokens_per_s": round(tps, 1), "speedup_at_measured_n": round(value / tps, 3),
            "speedup_at_n_eq_k": round(w.B * w.n_q / step_s / tps, 3),
            "speedup_at_n_eq_25": round(w.B * 26 / step_s / tps, 3)}


def cycle(a):
    """The default step: one staggered cycle of the Llama-70B-shaped layer.

    Sixteen sequences form two request groups of eight.  Every sequence's full
    bf16 context KV sits in pinned host memory as shuffled 16-token pages; the
    device keeps each group's int4 draft cache and one region for the full KV
    of the group being verified.  A cycle has two halves.  In each, one group
    runs its k = 32 draft steps while the other group's full KV streams into
    the region in 4096-token chunks on a copy stream (vc_prefetch_full_kv on a
    host thread); as each chunk lands, the verifying group's verify runs over
    it (vc_verify_attn_range), then over the new rows, then vc_verify_merge and
    vc_accept.  The drafting group's calls are issued `--pace` at a time before
    each chunk's verify, spread over the transfer.  The copy of chunk c into the region waits only for the previous
    group's verify of chunk c.  Inputs are resident (host pool, device caches)
    before timing; the vocabulary projection that makes draft ids and verify
    logits runs once, untimed.  `value` = verified tokens of both groups per
    cycle over the cycle's wall time."""
    import threading

    import numpy as np
    import torch

    import compressed_kv_draft_amd as vc
    from compressed_kv_draft_amd import workload as WL
    from synth import configs as C

    w = C.LLAMA70B
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    cw = WL.CycleWorkload(w, device="cuda:0", rotate=2)
    G, bg = w.groups, cw.bg
    wg = w.with_(B=bg)                                   # one group's shape
    print(f"[cycle] setup {time.perf_counter() - t_setup:.1f} s", flush=True)
    comp = torch.cuda.current_stream()
    cps = torch.cuda.Stream()
    n_chunks = len(cw.chunks)
    n_stage = 3
    staging = [torch.empty(cw.chunk_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(n_stage)]
    landed = [torch.cuda.Event() for _ in range(n_chunks)]      # chunk c of the copying group is on the device
    verified = [torch.cuda.Event() for _ in range(n_chunks)]    # the region's chunk c has been read by verify
    for e in verified:
        e.record(comp)
    ranges = cw.chunks + [(w.L, w.L + w.n_q)]
    slots = [vc.verify_range_parts(bg, w.Hq, w.Hkv, w.D, w.n_q, t0, t1) for t0, t1 in ranges]
    row_f = bg * w.Hq * w.n_q * (w.D + 2)
    parts = torch.empty(sum(slots) * row_f, dtype=torch.float32, device="cuda:0")
    out_ids = [torch.empty((bg, w.n_q), dtype=torch.int32, device="cuda:0") for _ in range(G)]
    n_acc = [torch.empty(bg, dtype=torch.int32, device="cuda:0") for _ in range(G)]
    d_ids, vlog = [None] * G, [None] * G
    copies_done = [0]
    errors = []

    def copy_group(gi, flags, last=None):
        try:
            for c, (t0, t1) in enumerate(cw.chunks):
                cps.wait_event(verified[c])
                free = landed[(c - n_stage) % n_chunks] if (copies_done[0] or c >= n_stage) else None
                vc.prefetch_full_kv(cw.host, cw.page_bytes, cw.table, cw.seqs[gi], t0, t1, w.page_tokens,
                                    staging[c % n_stage], cw.region[c * cw.chunk_bytes:(c + 1) * cw.chunk_bytes],
                                    stream=cps, done_event=landed[c], staging_free=free)
                if flags is not None:
                    flags[c].set()
            if last is not None:
                last.record(cps)
            copies_done[0] += 1
        except Exception as e:          # surfaced by the main thread, which would otherwise wait forever
            errors.append(e)
            if flags is not None:
                for f in flags:
                    f.set()

    def drafts(gi):
        for j in range(w.k):
            cw.draft_step(gi, j)

    def verify_chunks(gi, flags):
        off = 0
        for c, ((t0, t1), n) in enumerate(zip(ranges, slots)):
            if c < n_chunks:
                if flags is not None and not flags[c].wait(120):
                    raise RuntimeError("prefetch thread stalled")
                if errors:
                    raise errors[0]
                comp.wait_event(landed[c])
            vc.verify_attn_range(cw.q_verify[gi], cw.full[gi], cw.ctx_len, w.L, w.Hkv, cw.scale, t0, t1,
                                 parts[off * row_f:])
            if c < n_chunks:
                verified[c].record(comp)
            off += n
        vc.verify_merge(parts, sum(slots), bg, w.Hq, w.n_q, w.D, out=cw.verify_out[gi])

    pace = a.pace if a.pace > 0 else w.k

    def half(gx, gy, rec=None):
        """Group gx drafts while group gy's full KV streams in and is verified:
        `pace` draft calls of gx, then the verify of gy's next chunk once it has
        landed, and so on, so that drafting is spread over the transfer."""
        flags = [threading.Event() for _ in range(n_chunks)]
        th = threading.Thread(target=copy_group, args=(gy, flags, rec["landed"] if rec else None))
        th.start()
        off, j = 0, 0
        spans = []
        for c, ((t0, t1), n) in enumerate(zip(ranges, slots)):
            if j < w.k:
                e0, e1 = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if rec \
                    else (None, None)
                if rec:
                    e0.record(comp)
                for _ in range(min(pace, w.k - j) if c < n_chunks else w.k - j):
                    cw.draft_step(gx, j)
                    j += 1
                if rec:
                    e1.record(comp)
                    spans.append((e0, e1))
            if c < n_chunks:
                if not flags[c].wait(120):
                    raise RuntimeError("prefetch thread stalled")
                if errors:
                    raise errors[0]
                comp.wait_event(landed[c])
            vc.verify_attn_range(cw.q_verify[gy], cw.full[gy], cw.ctx_len, w.L, w.Hkv, cw.scale, t0, t1,
                                 parts[off * row_f:])
            if c < n_chunks:
                verified[c].record(comp)
            off += n
        vc.verify_merge(parts, sum(slots), bg, w.Hq, w.n_q, w.D, out=cw.verify_out[gy])
        vc.accept(d_ids[gy], vlog[gy], out_ids=out_ids[gy], n_accept=n_acc[gy])
        if rec:
            rec["end"].record(comp)
            rec["spans"] = spans
        th.join()
        if errors:
            raise errors[0]

    # untimed: each group's drafts and verify once, the vocabulary projection for
    # draft ids and verify logits, and the chunked verify against a whole verify
    # of the same resident pages
    rel = []
    for gi in range(G):
        drafts(gi)
        d_ids[gi] = vc.argmax(cw.draft_logits(gi).contiguous()).reshape(bg, w.k)
        copy_group(gi, None)
        verify_chunks(gi, None)
        vlog[gi] = cw.verify_logits(gi)
        whole = vc.verify_attn(cw.q_verify[gi], cw.full[gi], cw.ctx_len, w.L, w.Hkv, cw.scale, ws=cw.verify_ws)
        torch.cuda.synchronize()
        rel.append(float(torch.linalg.norm(whole - cw.verify_out[gi]) / torch.linalg.norm(whole)))
    # the two partition the keys differently, so P's f16 rounding (relative to
    # each partition's running max) differs: each is ~2e-4 from the oracle
    if not max(rel) < 1e-3:
        raise RuntimeError(f"chunked verify differs from the whole verify: rel L2 {rel}")
    for _ in range(max(1, a.warmup // 8)):
        half(0, 1)
        half(1, 0)
    torch.cuda.synchronize()

    recs = []
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for gx, gy in ((0, 1), (1, 0)):
            rec = {k: torch.cuda.Event(enable_timing=True) for k in ("end", "landed")}
            half(gx, gy, rec)
            recs.append(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cycle_s = wall / a.steps
    n = [x.cpu().numpy().astype(np.int64) for x in n_acc]
    tokens = int(sum((x + 1).sum() for x in n))
    value = tokens / cycle_s
    d_call = float(np.mean([sum(e0.elapsed_time(e1) for e0, e1 in r["spans"]) for r in recs])) * 1e-3 / w.k
    tail = float(np.median([r["landed"].elapsed_time(r["end"]) for r in recs])) * 1e-3

    # untimed references on the same buffers: the copy alone, the drafts alone,
    # verify of resident pages (whole, and chunk by chunk with nothing to wait for)
    def wall_of(fn, reps=3):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t)
        return float(np.median(ts))

    def gpu_of(fn, reps=5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(comp)
        for _ in range(reps):
            fn()
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = wall_of(lambda: copy_group(1, None))
    t_end = time.perf_counter() + 0.3       # continuous drafting, clocks settled
    while time.perf_counter() < t_end:
        drafts(0)
        torch.cuda.synchronize()
    d_alone = gpu_of(lambda: drafts(0), reps=5) / w.k
    t_vwhole = gpu_of(lambda: vc.verify_attn(cw.q_verify[1], cw.full[1], cw.ctx_len, w.L, w.Hkv, cw.scale,
                                             out=cw.verify_out[1], ws=cw.verify_ws))
    t_vchunk = gpu_of(lambda: verify_chunks(1, None))
    d_bytes = float(np.mean([WL.draft_step_bytes(wg, j) for j in range(w.k)]))
    v_bytes = float(WL.verify_bytes(wg))
    copy_bytes = n_chunks * cw.chunk_bytes
    d_gbs = d_bytes / d_call / 1e9
    v_gbs = v_bytes / t_vwhole / 1e9
    pcie_only = G * t_copy
    base_tps = w.B / pcie_only       # full-KV decode with the full KV in host memory: every token streams it
    roof = {"bound": "hbm", "kernel": "vc_draft_attn (draft_mfma_kernel<128,4,2> + draft_combine_kernel), int4, "
                                      "one group of 8 sequences",
            "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(d_gbs / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(w.name + "_cycle", "draft"), "bytes_per_launch": int(d_bytes),
            "avg_launch_us": round(1e6 * d_call, 2),
            "how": "each run of draft calls timed with HIP events on the launch stream, summed over the k calls "
                   "of a half-cycle"}
    line = {
        "metric": "verified tokens/sec per GPU; draft/verify attention HBM TB/s vs peak",
        "value": round(value, 1), "unit": "verified tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": 2 * max(1, a.warmup // 8), "ms_per_step": round(1e3 * cycle_s, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": path_dtype(w),
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, shuffled page table); inputs resident before timing",
        "config": {"workload": w.name + "_staggered_cycle", "batch": w.B, "groups": G, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "context": w.L, "draft_len": w.k, "draft_cache": "quant4",
                   "residual": w.residual, "page_tokens": w.page_tokens, "chunk_tokens": w.chunk_tokens,
                   "full_kv": "pinned host pool, streamed over PCIe every verify",
                   "step": "one cycle = 2 halves; each: one group's k draft calls beside the other group's "
                           "full-KV prefetch (16 chunks) + chunked verify + merge + accept",
                   "draft_pace": f"{pace} draft calls before each chunk's verify",
                   "arithmetic": path_arithmetic(w)},
        "accept": {"n_accept": [x.tolist() for x in n], "tokens_per_cycle": tokens,
                   "tokens_per_s_at_n_eq_k": round(w.B * w.n_q / cycle_s, 1),
                   "tokens_per_s_at_n_eq_25": round(w.B * 26 / cycle_s, 1),
                   "note": "synthetic single-layer queries are drawn independently per position, so the measured "
                           "acceptance is low; the n = k and n = 25 rates use the same measured cycle time"},
        "cycle": {"cycle_ms": round(1e3 * cycle_s, 3), "pcie_only_ms": round(1e3 * pcie_only, 3),
                  "cycle_over_pcie_only": round(cycle_s / pcie_only, 4),
                  "copy_ms_per_group_alone": round(1e3 * t_copy, 3),
                  "prefetch_GBps_alone": round(copy_bytes / t_copy / 1e9, 2),
                  "prefetch_GBps_in_cycle": round(G * copy_bytes / cycle_s / 1e9, 2),
                  "draft_ms_per_half": round(1e3 * d_call * w.k, 3),
                  "verify_tail_after_last_chunk_ms": round(1e3 * tail, 3),
                  "compute_per_half_ms": round(1e3 * (d_alone * w.k + t_vchunk), 3),
                  "compute_hidden_under_transfer": round(min(1.0, max(0.0, (
                      G * (d_alone * w.k + t_vchunk) + pcie_only - cycle_s) / (G * (d_alone * w.k + t_vchunk)))), 4),
                  "compute_hidden_how": "share of the cycle's GPU work (each half's k draft calls alone plus its "
                                        "chunked verify alone) that adds no time over the copy-only transfers: "
                                        "(compute + copy-only - cycle) / compute, clipped to [0, 1]",
                  "draft_in_cycle_over_continuous": round(d_call / d_alone, 4),
                  "chunked_vs_whole_verify_rel_l2": max(rel)},
        "draft": {"avg_us": round(1e6 * d_call, 2), "GBps": round(d_gbs, 1), "frac_hbm": round(d_gbs / HBM_PEAK_GBS, 4),
                  "bytes": int(d_bytes), "continuous_avg_us": round(1e6 * d_alone, 2),
                  "continuous_frac_hbm": round(d_bytes / d_alone / 1e9 / HBM_PEAK_GBS, 4),
                  "how": "avg_us: the calls inside the timed cycles; continuous: 0.3 s of back-to-back drafting "
                         "first, then 5 x k calls with nothing else running"},
        "verify": {"avg_us": round(1e6 * t_vwhole, 2), "GBps": round(v_gbs, 1), "frac_hbm": round(v_gbs / HBM_PEAK_GBS, 4),
                   "bytes": int(v_bytes), "TFLOPs": round(WL.verify_flops(wg) / t_vwhole / 1e12, 1),
                   "chunked_17_ranges_plus_merge_us": round(1e6 * t_vchunk, 2),
                   "traffic": stored_traffic(w.name + "_cycle", "verify"),
                   "how": "one group, all pages resident, HIP events"},
        "roofline": roof,
        "full_kv_decode_host_resident": {
            "tokens_per_s": round(base_tps, 1),
            "how": "upper bound: one token per sequence per full-KV transfer of every group at the measured copy "
                   "rate, decode compute hidden under the copy",
            "speedup_at_measured_n": round(value / base_tps, 3),
            "speedup_at_n_eq_k": round(w.B * w.n_q / cycle_s / base_tps, 3),
            "speedup_at_n_eq_25": round(w.B * 26 / cycle_s / base_tps, 3)},
    }
    print(f"[cycle] {value:.1f} verified tok/s, cycle {1e3 * cycle_s:.2f} ms (PCIe only {1e3 * pcie_only:.2f}), "
          f"draft {1e6 * d_call:.1f} us/call ({d_gbs / HBM_PEAK_GBS:.3f} of HBM), verify {1e6 * t_vwhole:.1f} us",
          flush=True)
    units = 0 if a.no_cpu_baseline else (24 if a.cpu_units is None else a.cpu_units)
    if units:
        line["cpu_baseline"] = cycle_cpu_baseline(w, cw, tokens, units)
    del cw, staging, parts
    torch.cuda.empty_cache()
    from synth import configs as C2
    legs = {}
    for name in [x for x in a.legs.split(",") if x]:
        t = time.perf_counter()
        r = round_line(C2.ALL[name], a, a.leg_steps, a.leg_warmup, 0 if a.no_cpu_baseline else a.leg_cpu_units,
                       False)
        legs[name] = {"value": r["value"], "ms_per_step": r["ms_per_step"], "dtype": r["dtype"],
                      "draft": r["draft"], "verify": r["verify"], "accept": r["accept"],
                      "cpu_baseline": r.get("cpu_baseline")}
        print(f"[leg] {name}: draft {r['draft']['avg_us']} us ({r['draft']['frac_hbm']}), verify "
              f"{r['verify']['avg_us']} us ({r['verify']['frac_hbm']}), {time.perf_counter() - t:.1f} s", flush=True)
    line["other_workloads"] = legs
    if not a.no_e2e_leg:
        t = time.perf_counter()
        r = e2e_record(1, 1, with_eager=False)
        line["end_to_end"] = {k: r[k] for k in ("value", "unit", "config", "rounds", "accepted_histogram",
                                                "mean_tokens_per_round", "decode_s", "prefill_s", "drafting",
                                                "equals_oracle_greedy")}
        print(f"[e2e] {r['value']} tokens/s, equals oracle greedy: {r['equals_oracle_greedy']}, "
              f"{time.perf_counter() - t:.1f} s", flush=True)
    print(json.dumps(line), flush=True)


def cycle_cpu_baseline(w, cw, tokens_per_cycle, units):
    """The fp64 oracle on `units` (batch, kv-head) units of group 0 (its first
    sequences): the k draft steps and the verify of one round each, scaled to
    all B * Hkv units, giving verified tokens per cycle over the oracle's time
    (no transfer is modelled on the CPU side)."""
    import numpy as np
    from oracle import round as R
    import compressed_kv_draft_amd.workload as WL
    wg = w.with_(B=cw.bg)
    g = w.g
    picks = [(u // w.Hkv, u % w.Hkv) for u in range(min(units, WL.CPU_SAMPLE_SEQS * w.Hkv))]
    comps = {}
    for (b, h) in picks:
        comps[(b, h)] = R.unit_compressed(wg, cw.np_ctx["K"][b, h], cw.np_ctx["V"][b, h])
    t0 = time.perf_counter()
    for (b, h) in picks:
        args = (cw.np_ctx["K"][b, h], cw.np_ctx["V"][b, h], cw.np_kn[b, h], cw.np_vn[b, h],
                cw.np_q[b, h * g:(h + 1) * g])
        R.unit_draft(wg, *args, comp=comps[(b, h)])
        R.unit_verify(wg, *args)
    dt = time.perf_counter() - t0
    full = dt * (w.B * w.Hkv) / len(picks)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cyc_bytes = w.groups * (sum(WL.draft_step_bytes(wg, j) for j in range(w.k)) + WL.verify_bytes(wg))
    return {"value": tokens_per_cycle / full, "unit": "verified tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "effective_GBps": round(cyc_bytes / full / 1e9, 3),
            "sample": f"{len(picks)} of {w.B * w.Hkv} (batch, kv-head) units, {w.k} draft steps + verify each, "
                      f"fp64 numpy, {dt:.1f} s measured, scaled x{(w.B * w.Hkv) / len(picks):.0f}"}


def path_dtype(w) -> str:
    """Arithmetic types of a round: the draft's matrix operands, then the verify's."""
    return ("f16" if w.kind == "quant" else "bf16") + "+bf16/f16"


def path_arithmetic(w) -> str:
    if w.kind == "quant":
        d = (f"draft: int{w.bits} codes as exact f16 MFMA operands, q*s and p*s as f16 hi+lo, "
             f"bf16 MFMA for the exact tail rows")
    else:
        d = ("draft: gathered bf16 rows" if w.kind == "token_drop" else "draft: bf16 rows") + \
            ", bf16 MFMA for q.k, P as bf16 hi+lo for P.V"
    return d + "; verify: bf16 q.k and f16 P.V MFMA; fp32 accumulate and softmax"


def round_line(w, a, steps, warmup, cpu_units, full_kv):
    """Time `steps` rounds of one single-layer workload (k draft calls rotating
    over ROTATE copies of the lossy cache, one verify, one accept) and return
    its JSON record."""
    import numpy as np
    import torch

    import compressed_kv_draft_amd as vc
    from compressed_kv_draft_amd import workload as WL

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

    def drafts():
        for j in range(w.k):
            vc.draft_attn(comps[j % ROTATE], dw.tails[j], dw.q_steps[j], dw.scale, out=dw.draft_out[j],
                          ws=dw.draft_ws, Hkv=w.Hkv)

    def accept():
        vc.accept(d_ids, vlog, out_ids=out_ids, n_accept=n_acc)

    phases = [drafts, dw.verify, accept]

    def step(record):
        marks = []
        for ph in phases:
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
            ph()
        if record:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append(e)
            ev.append(("draft", marks[0], marks[1]))
            ev.append(("verify", marks[1], marks[2]))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    if a.graph:
        # each phase recorded once (after the warm-up, so the library's per-device
        # plans exist) and replayed on the stream: the same calls without their
        # host launch gaps; nothing in them allocates or sets memory
        graphs = []
        for ph in phases:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                ph()
            graphs.append(g)
        phases = [g.replay for g in graphs]
        for _ in range(3):
            step(False)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    n = n_acc.cpu().numpy().astype(np.int64)
    tokens_per_step = int((n + 1).sum())
    wall = t1 - t0
    ms = 1e3 * wall / steps
    value = tokens_per_step * steps / wall
    d_ms = [e0.elapsed_time(e1) / w.k for (k_, e0, e1) in ev if k_ == "draft"]   # per draft call
    v_ms = [e0.elapsed_time(e1) for (k_, e0, e1) in ev if k_ == "verify"]
    d_avg = float(np.mean(d_ms)) * 1e-3
    v_avg = float(np.mean(v_ms)) * 1e-3
    d_bytes = float(np.mean([WL.draft_step_bytes(w, j) for j in range(w.k)]))
    v_bytes = float(WL.verify_bytes(w))
    d_gbs = d_bytes / d_avg / 1e9
    v_gbs = v_bytes / v_avg / 1e9
    draft_total = sum(d_ms) * w.k / steps
    verify_total = sum(v_ms) / steps
    dominant = "draft" if draft_total >= verify_total else "verify"
    roof = {"bound": "hbm", "kernel": "vc_draft_attn (draft_mfma_kernel + draft_combine_kernel)"
            if dominant == "draft" else "vc_verify_attn (verify_mfma_kernel + verify_combine_kernel)",
            "achieved": round(d_gbs if dominant == "draft" else v_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round((d_gbs if dominant == "draft" else v_gbs) / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(w.name, dominant),
            "bytes_per_launch": int(d_bytes if dominant == "draft" else v_bytes),
            "avg_launch_us": round(1e6 * (d_avg if dominant == "draft" else v_avg), 2)}
    step_s = wall / steps
    line = {
        "metric": "verified tokens/sec per GPU; draft/verify attention HBM TB/s vs peak",
        "value": round(value, 1), "unit": "verified tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": path_dtype(w), "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "context": w.L, "draft_len": w.k, "draft_cache": f"{w.kind}{w.bits if w.kind == 'quant' else ''}",
                   "residual": w.residual, "vocab": w.vocab, "layers_rotated": ROTATE,
                   "step": "k x vc_draft_attn + vc_verify_attn + vc_accept (one layer; vocab projection outside)",
                   "arithmetic": path_arithmetic(w)},
        "accept": {"n_accept": n.tolist(), "tokens_per_step": tokens_per_step,
                   "tokens_per_s_at_n_eq_k": round(w.B * w.n_q / step_s, 1),
                   "tokens_per_s_at_n_eq_25": round(w.B * 26 / step_s, 1)},
        "draft": {"avg_us": round(1e6 * d_avg, 2), "GBps": round(d_gbs, 1), "frac_hbm": round(d_gbs / HBM_PEAK_GBS, 4),
                  "bytes": int(d_bytes), "ms_per_step": round(draft_total, 4),
                  "traffic": stored_traffic(w.name, "draft")},
        "verify": {"avg_us": round(1e6 * v_avg, 2), "GBps": round(v_gbs, 1), "frac_hbm": round(v_gbs / HBM_PEAK_GBS, 4),
                   "bytes": int(v_bytes), "TFLOPs": round(WL.verify_flops(w) / v_avg / 1e12, 1),
                   "ms_per_step": round(verify_total, 4), "traffic": stored_traffic(w.name, "verify")},
        "roofline": roof,
        "launch": "each phase (k draft calls | verify | accept) replayed as one recorded HIP graph" if a.graph
                  else "host launches",
        "timing": "HIP events around each phase on the launch stream; draft avg_us = draft phase / k",
    }
    if full_kv:
        line["full_kv_decode"] = full_kv_decode(w, dw, value, step_s, graph=a.graph)
        sr = line["full_kv_decode"]["GBps"]
        line["stream_read"] = {"GBps": sr, "how": "the full-KV decode above: vc_draft_attn streaming the whole "
                                                  "bf16 cache once, the read rate reached in practice",
                               "draft_frac": round(d_gbs / sr, 4), "verify_frac": round(v_gbs / sr, 4)}
    if cpu_units:
        line["cpu_baseline"] = cpu_baseline(w, dw, int(n.sum()), cpu_units)
    del dw, comps
    torch.cuda.empty_cache()
    return line




def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the hot path is per-GPU data parallel with no exchange; "
              f"--gpus {a.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if a.stagger:
        stagger(a)
        return
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.e2e:
        e2e(a)
        return
    if a.e2e_groups:
        e2e_groups(a)
        return
    from synth import configs as C
    if a.config is None:
        cycle(a)
        return
    units = 0 if a.no_cpu_baseline else (8 if a.cpu_units is None else a.cpu_units)
    line = round_line(C.ALL[a.config], a, a.steps, a.warmup, units, not a.no_full_kv_decode)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
