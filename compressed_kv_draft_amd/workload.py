"""Device state of one single-layer draft/verify workload (harness glue).

Lays the seeded synthetic inputs out in device memory in the layouts the C ABI
expects and runs the GPU compressor (vc_quantize_kv) for the draft cache.  Used
by the benchmark and the GPU tests; holds no attention arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import inputs as I
from synth.configs import Workload

from . import _lib as vc


# sequences of the cycle workload kept on the host for the CPU baseline sample
CPU_SAMPLE_SEQS = 3


def bf16_dev(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def paged_pool(w: Workload, k_all: np.ndarray, v_all: np.ndarray, table: np.ndarray, n_slots: int) -> np.ndarray:
    """Pool [n_slots, Hkv, 2, page, D] (bf16 bits) holding rows [0, L + n_q) of every sequence."""
    pt = w.page_tokens
    P = table.shape[1]
    n = w.L + w.n_q
    pool = np.zeros((n_slots, w.Hkv, 2, pt, w.D), dtype=np.uint16)
    pad = P * pt - n
    for b in range(w.B):
        kb = np.pad(k_all[b], ((0, 0), (0, pad), (0, 0))).reshape(w.Hkv, P, pt, w.D)
        vb = np.pad(v_all[b], ((0, 0), (0, pad), (0, 0))).reshape(w.Hkv, P, pt, w.D)
        pool[table[b], :, 0] = kb.transpose(1, 0, 2, 3)
        pool[table[b], :, 1] = vb.transpose(1, 0, 2, 3)
    return pool


class DeviceWorkload:
    """All inputs of one round on the device.

    full_k/full_v  bf16 [B, Hkv, L + n_q, D]: context then the n_q new rows
    comp           the draft cache (quant / token_drop / identity)
    tail           exact rows of the draft: recent window then new rows
    tail_lens[j]   int32 [B] tail length of draft step j (window + j + 1)
    q_steps[j]     bf16 [B, Hq, D] query of draft step j; q_verify [B, Hq, n_q, D]
    """

    def __init__(self, w: Workload, device="cuda", Q: np.ndarray | None = None, with_vocab: bool = True,
                 ctx=None):
        self.w = w
        self.device = device
        g = w.g
        if ctx is None:
            K = I.context_kv(w, "k")
            V = I.context_kv(w, "v")
        else:
            K, V = ctx
        Kn = I.new_rows(w, "k")
        Vn = I.new_rows(w, "v")
        if Q is None:
            Q = I.queries(w)
        self.np = dict(K=K, V=V, Kn=Kn, Vn=Vn, Q=Q)
        k_all = np.concatenate([K, Kn], axis=2)
        v_all = np.concatenate([V, Vn], axis=2)
        self.L_cap = w.L + w.n_q
        self.paged = w.paged
        if w.paged:
            table, n_slots = I.page_table(w)
            self.page_table_np = table
            self.n_slots = n_slots
            pool = paged_pool(w, k_all, v_all, table, n_slots)
            self.pool_np = pool
            self.pool = torch.from_numpy(pool.view(np.int16)).to(device).view(torch.bfloat16)
            self.page_table = torch.from_numpy(table).to(device)
            self.full = vc.FullKV(self.pool, None, 0, self.page_table, w.page_tokens, table.shape[1], n_slots)
        self.full_k = bf16_dev(k_all, device)
        self.full_v = bf16_dev(v_all, device)
        if not w.paged:
            self.full = vc.FullKV(self.full_k, self.full_v, L_cap=self.L_cap)
        del k_all, v_all
        self.ctx_len = torch.full((w.B,), w.L, dtype=torch.int32, device=device)
        # draft cache
        if w.kind == "quant":
            self.comp = vc.quantize_kv(self.full_k, self.full_v, w.bits, w.n_quant)
            R = w.residual
            tk = np.concatenate([K[:, :, w.L - R:w.L], Kn], axis=2)
            tv = np.concatenate([V[:, :, w.L - R:w.L], Vn], axis=2)
        elif w.kind == "token_drop":
            self.keep_np = I.keep_indices(w)
            self.keep = torch.from_numpy(self.keep_np).to(device)
            self.comp = vc.token_drop_cache(self.full_k, self.full_v, self.keep)
            R = 0
            tk, tv = Kn, Vn
        else:
            self.comp = vc.identity_cache(self.full_k, self.full_v, w.L)
            R = 0
            tk, tv = Kn, Vn
        self.tail_k = bf16_dev(tk, device)
        self.tail_v = bf16_dev(tv, device)
        self.tail_lens = [torch.full((w.B,), R + j + 1, dtype=torch.int32, device=device) for j in range(w.k)]
        self.tails = [vc.Tail(self.tail_k, self.tail_v, tl) for tl in self.tail_lens]
        self.q_verify = bf16_dev(Q, device)
        self.q_steps = [self.q_verify[:, :, j, :].contiguous() for j in range(w.k)]
        self.scale = float(np.float32(1.0 / np.sqrt(w.D)))
        self.n_main = {"quant": w.n_quant, "token_drop": w.n_keep, "identity": w.L}[w.kind]
        self.draft_ws = torch.zeros(vc.draft_ws_bytes(w.B, w.Hq, w.Hkv, w.D, self.n_main + R + w.n_q),
                                    dtype=torch.uint8, device=device)
        self.verify_ws = torch.empty(vc.verify_ws_bytes(w.B, w.Hq, w.Hkv, w.D, w.n_q, w.L),
                                     dtype=torch.uint8, device=device)
        self.draft_out = torch.empty((w.k, w.B, w.Hq, w.D), dtype=torch.float32, device=device)
        self.verify_out = torch.empty((w.B, w.Hq, w.n_q, w.D), dtype=torch.float32, device=device)
        self.W = None
        if with_vocab:
            self.W = torch.from_numpy(I.vocab_matrix(w)).to(device)

    # one round of the path -------------------------------------------------
    def draft_step(self, j: int, stream=None):
        w = self.w
        return vc.draft_attn(self.comp, self.tails[j], self.q_steps[j], self.scale, out=self.draft_out[j],
                             ws=self.draft_ws, Hkv=w.Hkv, stream=stream)

    def verify(self, stream=None):
        w = self.w
        return vc.verify_attn(self.q_verify, self.full, self.ctx_len, w.L, w.Hkv, self.scale,
                              out=self.verify_out, ws=self.verify_ws, stream=stream)

    def draft_logits(self):
        """[B, k, V] logits of the drafts (harness glue: fp32 GEMM in torch)."""
        w = self.w
        o = self.draft_out.permute(1, 0, 2, 3).reshape(w.B, w.k, w.Hq * w.D)
        return torch.matmul(o, self.W)

    def verify_logits(self):
        w = self.w
        o = self.verify_out.permute(0, 2, 1, 3).reshape(w.B, w.n_q, w.Hq * w.D)
        return torch.matmul(o, self.W).contiguous()


def clone_compressed(comp: vc.Compressed) -> vc.Compressed:
    """Same cache contents in fresh device buffers (another 'layer' for rotation)."""
    t = dict(comp.t)
    for f in ("k_codes", "v_codes", "k_meta", "v_meta", "keep_idx"):
        if t.get(f) is not None:
            t[f] = t[f].clone()
    for f in ("k_full", "v_full"):
        if t.get(f) is not None:
            t[f] = t[f].clone()
    t.pop("src_keepalive", None)
    return vc.Compressed(comp.kind, **t)


def draft_step_bytes(w: Workload, j: int) -> int:
    """Algorithmic HBM bytes of draft step j: everything the method must read
    (compressed codes + scales/zeros, or gathered rows + indices, plus the exact
    tail rows and the queries) and write (outputs)."""
    units = w.B * w.Hkv
    D = w.D
    if w.kind == "quant":
        nq = w.n_quant
        per = 2 * nq * D * w.bits // 8 + (nq // 32) * D * 4 + nq * (D // 32) * 4
        tail = w.residual + j + 1
    elif w.kind == "token_drop":
        per = w.n_keep * (2 * D * 2 + 4)
        tail = j + 1
    else:
        per = w.L * 2 * D * 2
        tail = j + 1
    per += tail * 2 * D * 2
    return units * per + w.B * w.Hq * D * (2 + 4)


def verify_bytes(w: Workload) -> int:
    """Algorithmic HBM bytes of one verify: the full K/V rows [0, L + n_q) once,
    the queries and the fp32 outputs."""
    n = w.L + w.n_q
    return w.B * w.Hkv * n * 2 * w.D * 2 + w.B * w.Hq * w.n_q * w.D * (2 + 4)


def verify_flops(w: Workload) -> int:
    """q.k and p.v MACs x 2 over the causal key ranges."""
    keys = sum(w.L + j + 1 for j in range(w.n_q))
    return 2 * 2 * w.B * w.Hq * keys * w.D


class CycleWorkload:
    """Device and host state of the staggered two-group cycle (harness glue).

    The batch is split into request groups of B / groups sequences.  Each group
    has its own QUANT draft cache (device, `rotate` copies so that consecutive
    draft steps read different buffers, as consecutive layers would), exact
    tail (recent window + the round's drafted rows) and queries.  The full
    context KV of every sequence lives in one pinned host pool of shuffled
    pages (the layout of include/vc.h's paged cache).  The device holds one
    region for the full KV of the group being verified (chunk c of all its
    sequences after chunk c - 1, as the prefetch lands them) followed by the
    pages of every group's new rows, which exist only on the device; each
    group has a device page table into that pool.
    """

    def __init__(self, w: Workload, device="cuda", rotate: int = 2, with_vocab: bool = True):
        assert w.kind == "quant" and w.paged and w.L % w.chunk_tokens == 0 and w.chunk_tokens % w.page_tokens == 0
        self.w = w
        G = w.groups
        bg = w.B // G
        self.bg = bg
        pt = w.page_tokens
        table, _ = I.page_table(w)
        self.table = table                                   # host int32 [B, pages_per_seq]
        ctx_pages = w.L // pt
        pps = table.shape[1]
        extra = pps - ctx_pages
        self.page_bytes = w.Hkv * 2 * pt * w.D * 2
        n_ctx_slots = w.B * ctx_pages
        assert int(table[:, :ctx_pages].max()) < n_ctx_slots
        self.chunks = [(t, t + w.chunk_tokens) for t in range(0, w.L, w.chunk_tokens)]
        scp = w.chunk_tokens // pt                           # pages of one sequence in one chunk
        self.pages_per_chunk = bg * scp
        self.chunk_bytes = self.pages_per_chunk * self.page_bytes
        n_region = self.pages_per_chunk * len(self.chunks)
        self.region_bytes = n_region * self.page_bytes
        self.host = torch.empty(n_ctx_slots * self.page_bytes, dtype=torch.uint8, pin_memory=True)
        host_pages = self.host.numpy().view(np.uint16).reshape(n_ctx_slots, w.Hkv, 2, pt, w.D)
        n_dev_pages = n_region + w.B * extra
        self.pool = torch.empty(n_dev_pages * self.page_bytes, dtype=torch.uint8, device=device)
        self.region = self.pool[:self.region_bytes]
        dev_pages = self.pool.view(torch.int16).view(n_dev_pages, w.Hkv, 2, pt, w.D)
        Kn, Vn = I.new_rows(w, "k"), I.new_rows(w, "v")
        Q = I.queries(w)
        R = w.residual
        self.seqs, self.comps, self.tails, self.q_steps, self.q_verify, self.full = [], [], [], [], [], []
        self.np_ctx = {}
        for gi in range(G):
            seqs = list(range(gi * bg, (gi + 1) * bg))
            self.seqs.append(seqs)
            K = I.context_kv_seqs(w, "k", seqs)
            V = I.context_kv_seqs(w, "v", seqs)
            tab = np.empty((bg, pps), dtype=np.int32)
            for i, b in enumerate(seqs):
                slots = table[b, :ctx_pages]
                host_pages[slots, :, 0] = K[i].reshape(w.Hkv, ctx_pages, pt, w.D).transpose(1, 0, 2, 3)
                host_pages[slots, :, 1] = V[i].reshape(w.Hkv, ctx_pages, pt, w.D).transpose(1, 0, 2, 3)
                p = np.arange(ctx_pages)
                tab[i, :ctx_pages] = (p // scp) * self.pages_per_chunk + i * scp + p % scp
                new_slots = n_region + b * extra + np.arange(extra)
                tab[i, ctx_pages:] = new_slots
                pad = extra * pt - w.n_q
                for which, src in ((0, Kn), (1, Vn)):
                    rows = np.pad(src[b], ((0, 0), (0, pad), (0, 0))).reshape(w.Hkv, extra, pt, w.D)
                    dev_pages[torch.from_numpy(new_slots).long().to(device), :, which] = \
                        torch.from_numpy(np.ascontiguousarray(rows.transpose(1, 0, 2, 3)).view(np.int16)).to(device)
            # the draft cache: quantise the group's context on the device
            kd = bf16_dev(K, device)
            vd = bf16_dev(V, device)
            comp = vc.quantize_kv(kd, vd, w.bits, w.n_quant)
            torch.cuda.synchronize()
            comp.t.pop("src_keepalive", None)
            self.comps.append([comp] + [clone_compressed(comp) for _ in range(rotate - 1)])
            del kd, vd
            tk = np.concatenate([K[:, :, w.L - R:], Kn[seqs]], axis=2)
            tv = np.concatenate([V[:, :, w.L - R:], Vn[seqs]], axis=2)
            tkd, tvd = bf16_dev(tk, device), bf16_dev(tv, device)
            lens = [torch.full((bg,), R + j + 1, dtype=torch.int32, device=device) for j in range(w.k)]
            self.tails.append([vc.Tail(tkd, tvd, tl) for tl in lens])
            qv = bf16_dev(Q[seqs], device)
            self.q_verify.append(qv)
            self.q_steps.append([qv[:, :, j, :].contiguous() for j in range(w.k)])
            self.full.append(vc.FullKV(self.pool, None, 0, torch.from_numpy(tab).to(device), pt, pps, n_dev_pages))
            if gi == 0:
                # the first sequences of group 0, for the CPU baseline sample
                self.np_ctx = {"K": K[:CPU_SAMPLE_SEQS].copy(), "V": V[:CPU_SAMPLE_SEQS].copy()}
            del K, V
        self.np_q, self.np_kn, self.np_vn = Q, Kn, Vn
        self.ctx_len = torch.full((bg,), w.L, dtype=torch.int32, device=device)
        self.scale = float(np.float32(1.0 / np.sqrt(w.D)))
        self.draft_ws = torch.zeros(vc.draft_ws_bytes(bg, w.Hq, w.Hkv, w.D, w.n_quant + R + w.n_q),
                                    dtype=torch.uint8, device=device)
        self.verify_ws = torch.empty(vc.verify_ws_bytes(bg, w.Hq, w.Hkv, w.D, w.n_q, w.L), dtype=torch.uint8,
                                     device=device)
        self.draft_out = [torch.empty((w.k, bg, w.Hq, w.D), dtype=torch.float32, device=device) for _ in range(G)]
        self.verify_out = [torch.empty((bg, w.Hq, w.n_q, w.D), dtype=torch.float32, device=device)
                           for _ in range(G)]
        self.W = torch.from_numpy(I.vocab_matrix(w)).to(device) if with_vocab else None

    def draft_step(self, gi: int, j: int, stream=None):
        w = self.w
        comps = self.comps[gi]
        return vc.draft_attn(comps[j % len(comps)], self.tails[gi][j], self.q_steps[gi][j], self.scale,
                             out=self.draft_out[gi][j], ws=self.draft_ws, Hkv=w.Hkv, stream=stream)

    def draft_logits(self, gi: int):
        w = self.w
        o = self.draft_out[gi].permute(1, 0, 2, 3).reshape(self.bg, w.k, w.Hq * w.D)
        return torch.matmul(o, self.W)

    def verify_logits(self, gi: int):
        w = self.w
        o = self.verify_out[gi].permute(0, 2, 1, 3).reshape(self.bg, w.n_q, w.Hq * w.D)
        return torch.matmul(o, self.W).contiguous()
