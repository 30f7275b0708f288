"""Request groups staggered on one GPU, each with an adaptive draft length.

[VC Key System Innovations P1] drafting and verification stress different
resources, so the runtime staggers request groups: while one group drafts,
another verifies.  [P2] high acceptance lets a group verify less often.

Each group is a TinyLM (its own caches, shared weights) on a stream of its
own.  The host loop walks the groups in turn: it enqueues a group's
verification, waits for its accept result, books the outcome, asks the
library's policy (vc_sched_choose_k) for that group's next draft length and
enqueues its next draft round.  While the host waits on one group, the other
group's drafting already sits on its own stream, so verification of one group
runs beside drafting of the next: with two groups the phases alternate
(A verifies while B drafts, then B verifies while A drafts).  With stagger off
all groups share one stream, so the same calls run one after another (the
lock-step order).

Groups built with a shared FullStaging keep their full caches in pinned host
memory.  The next group's full cache is then copied into the staging region on
a copy stream as soon as the current group's verification has released it, so
the transfer runs beside the drafting.  This is the single-GPU form of P1:
drafting streams HBM while the other group's full KV crosses PCIe.

The policy sees, per group, the accepted drafts and the rounds that ended at a
mismatch and the mean time of one draft step and of one verification so far
(HIP events on the group's stream, or a fixed clock for reproducible
decisions).  Staggered, a two-phase cycle of groups g and h lasts
max(D_g, V_h) + max(D_h, V_g) (D drafting, V verification), so g's drafting
runs beside t_overlap = V_h and the rest of its cycle is
t_rest = max(V_g, D_h), with h's draft length as last chosen; lock-step, g's
cycle is D_g + V_g.  Output tokens do not depend on the draft lengths chosen: every
emitted token is the verifier's.
"""
from __future__ import annotations

import time

import torch

from . import _lib as vc


class StaggeredGroups:
    def __init__(self, lms, k_min: int = 1, k_max: int | None = None, stagger: bool = True, clock=None):
        """lms: TinyLM instances, one per request group.  clock: None (measure
        with HIP events) or a function group -> (t_draft_step, t_verify) used
        instead of measurements."""
        self.lms = list(lms)
        self.k_min = k_min
        self.k_max = min(lm.cfg.k for lm in self.lms) if k_max is None else k_max
        self.stagger = stagger
        self.clock = clock

    def run(self, prompts, n_gen: int, graph: bool = True) -> dict:
        G = len(self.lms)
        if self.stagger:
            streams = [torch.cuda.Stream() for _ in range(G)]
            copy_stream = torch.cuda.Stream()
        else:
            streams = [torch.cuda.current_stream()] * G
            copy_stream = streams[0]
        host_kv = self.lms[0].staging is not None
        fetched = [False] * G
        for lm, p, s in zip(self.lms, prompts, streams):
            with torch.cuda.stream(s):
                lm.start(p, graph=graph)
        torch.cuda.synchronize()
        hist = [[0, 0] for _ in range(G)]           # accepted drafts, rounds ended at a mismatch
        t_d = [None] * G                            # mean time of one draft step
        t_v = [None] * G                            # mean time of one verification (with accept and bookkeeping)
        sums = [[0.0, 0, 0.0, 0] for _ in range(G)]  # draft ms, draft steps, verify ms, verifications
        ks = [self.k_max] * G
        log = [[] for _ in range(G)]                # per round: k, n and the policy's inputs and answer
        ev = [None] * G

        def draft(g):
            with torch.cuda.stream(streams[g]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                self.lms[g].draft_round(ks[g])
                e1.record()
            ev[g] = (e0, e1)

        t0 = time.perf_counter()
        for g in range(G):
            draft(g)
        active = [True] * G
        while any(active):
            for g in range(G):
                if not active[g]:
                    continue
                lm = self.lms[g]
                if host_kv and not fetched[g]:
                    lm.fetch(copy_stream)
                with torch.cuda.stream(streams[g]):
                    v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    v0.record()
                    n = lm.verify_round(ks[g])
                    v1.record()
                fetched[g] = False
                if host_kv:   # the next verifying group's full cache, beside this group's drafting
                    for d in range(1, G):
                        h = (g + d) % G
                        if active[h]:
                            if not fetched[h]:
                                self.lms[h].fetch(copy_stream)
                                fetched[h] = True
                            break
                v1.synchronize()
                k = ks[g]
                rec = dict(k=k, n=n)
                log[g].append(rec)
                hist[g][0] += n
                hist[g][1] += int(n < k)
                if self.clock is not None:
                    t_d[g], t_v[g] = self.clock(g)
                else:
                    sm = sums[g]
                    sm[0] += ev[g][0].elapsed_time(ev[g][1])
                    sm[1] += k
                    sm[2] += v0.elapsed_time(v1)
                    sm[3] += 1
                    t_d[g], t_v[g] = sm[0] / sm[1], sm[2] / sm[3]
                if lm.done(n_gen):
                    active[g] = False
                    continue
                nxt = (g + 1) % G
                overlap, rest = 0.0, t_v[g]
                if self.stagger and G > 1 and active[nxt] and t_v[nxt] is not None:
                    overlap = t_v[nxt]
                    rest = max(t_v[g], ks[nxt] * t_d[nxt])
                args = (hist[g][0], hist[g][1], t_d[g], overlap, rest, self.k_min, self.k_max)
                ks[g] = vc.sched_choose_k(*args)
                rec.update(policy_args=args, next_k=ks[g])
                draft(g)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        toks = [lm.out[:n_gen] for lm in self.lms]
        return dict(tokens=toks, rounds=log, wall_s=wall,
                    tokens_per_s=sum(len(t) - 1 for t in toks) / wall if wall > 0 else 0.0)
