"""Greedy generation by the draft-then-verify loop on a small Llama-style decoder.

[VC Core Algorithm] the target model drafts k tokens reading the compressed
cache, verifies them in one causal pass over the full cache, keeps the
matching prefix plus one verifier token and repeats from there.

Every attention and every token decision runs in libvc: vc_verify_attn (the
prefill and each verification pass), vc_quantize_kv (the int4 draft cache of
the prompt), vc_draft_attn (each draft position), vc_argmax (draft tokens and
the first token) and vc_accept.  The dense layers, norms and rotary positions
around them are torch fp32 operations (harness glue, not the measured path).

Model: pre-norm blocks x += O(attn(RMSNorm(x))); x += SwiGLU(RMSNorm(x)); a
final RMSNorm and the vocabulary head.  q, and the k/v rows written to the
caches, are rounded to bf16 after the rotary step; attention outputs are fp32.
Cache bookkeeping per round, with the pending token at position ctx:
  * draft position j (token x_j at ctx + j) writes its k/v into the draft tail
    at row (ctx - P) + j and attends to the int4 prompt plus tail rows
    [0, ctx - P + j]; the tail's first ctx - P rows are the verified rows of
    earlier rounds;
  * verification writes the k/v of positions ctx .. ctx + k into the full cache
    and attends causally; after acceptance of n drafts, rows ctx .. ctx + n
    are copied into the tail (the draft's own rows there are overwritten) and
    the rows after them are left to be rewritten by the next round.
"""
from __future__ import annotations

import time

import numpy as np
import torch
import torch.nn.functional as F

from . import _lib as vc


class FullStaging:
    """One device region for the full cache of whichever request group is
    verifying: bf16 [1, Hkv, L_cap, D] K and V per layer.  [VC Key System
    Innovations P1; Architecture Support: full KV kept in CPU memory]  Groups
    that share it keep their own full caches in pinned host memory, copy them
    in before each verification (TinyLM.fetch) and write the rows it adds back
    out; `free` marks the end of the last use."""

    def __init__(self, cfg, device="cuda"):
        bf = dict(dtype=torch.bfloat16, device=device)
        self.K = [torch.zeros((1, cfg.Hkv, cfg.L_cap, cfg.D), **bf) for _ in range(cfg.n_layers)]
        self.V = [torch.zeros((1, cfg.Hkv, cfg.L_cap, cfg.D), **bf) for _ in range(cfg.n_layers)]
        self.full = [vc.FullKV(self.K[l], self.V[l], L_cap=cfg.L_cap) for l in range(cfg.n_layers)]
        self.free = torch.cuda.Event()


def _bf16_to_f32(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16).float()


class TinyLM:
    def __init__(self, cfg, W: dict | None, cos: np.ndarray | None, sin: np.ndarray | None, device="cuda",
                 shared: "TinyLM | None" = None, staging: FullStaging | None = None):
        """shared: another instance whose weights and rotary tables this one
        reuses (a second request group of the same model); W, cos, sin are
        then ignored.  Every instance has its own draft caches.  staging: keep
        the full cache in pinned host memory and verify in this shared device
        region (fetch() before each verification); None keeps it on the
        device."""
        torch.backends.cuda.matmul.allow_tf32 = False
        self.cfg, self.dev = cfg, device
        c = cfg
        if shared is not None:
            for n in ("embed", "layers", "final_norm", "head", "cos", "sin"):
                setattr(self, n, getattr(shared, n))
        else:
            f = lambda b: _bf16_to_f32(b, device)  # noqa: E731
            self.embed = f(W["embed"])
            self.layers = [{n: f(W[n][l]) for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
                                                       "attn_norm", "ffn_norm")} for l in range(c.n_layers)]
            self.final_norm = f(W["final_norm"])
            self.head = f(W["lm_head"])
            self.cos = torch.from_numpy(np.ascontiguousarray(cos)).to(device)
            self.sin = torch.from_numpy(np.ascontiguousarray(sin)).to(device)
        self.scale = float(np.float32(1.0 / np.sqrt(c.D)))
        bf = dict(dtype=torch.bfloat16, device=device)
        self.staging = staging
        if staging is not None:
            self.K, self.V, self.full = staging.K, staging.V, staging.full
            pin = dict(dtype=torch.bfloat16, pin_memory=True)
            self.K_h = [torch.zeros((1, c.Hkv, c.L_cap, c.D), **pin) for _ in range(c.n_layers)]
            self.V_h = [torch.zeros((1, c.Hkv, c.L_cap, c.D), **pin) for _ in range(c.n_layers)]
            self.landed = torch.cuda.Event()
        else:
            self.K = [torch.zeros((1, c.Hkv, c.L_cap, c.D), **bf) for _ in range(c.n_layers)]
            self.V = [torch.zeros((1, c.Hkv, c.L_cap, c.D), **bf) for _ in range(c.n_layers)]
            self.full = [vc.FullKV(self.K[l], self.V[l], L_cap=c.L_cap) for l in range(c.n_layers)]
        self.TK = [torch.zeros((1, c.Hkv, c.T_cap, c.D), **bf) for _ in range(c.n_layers)]
        self.TV = [torch.zeros((1, c.Hkv, c.T_cap, c.D), **bf) for _ in range(c.n_layers)]
        self.tail_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.tails = [vc.Tail(self.TK[l], self.TV[l], self.tail_len) for l in range(c.n_layers)]
        self.ctx_t = torch.zeros(1, dtype=torch.int32, device=device)
        self.comp = None
        self.draft_ws = None
        self.verify_ws = torch.empty(
            vc.verify_ws_bytes(1, c.Hq, c.Hkv, c.D, c.k + 1, c.L_cap - (c.k + 1)), dtype=torch.uint8, device=device)
        self.q_out = torch.empty((1, c.Hq, c.D), dtype=torch.float32, device=device)

    # ------------------------------------------------------------ dense glue

    def _rms(self, x, gain):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.cfg.eps) * gain

    def _rope(self, x, pos):
        """x [n, H, D] fp32, pos int64 [n]: rotate channel pairs (i, i + D/2)."""
        half = self.cfg.D // 2
        cs, sn = self.cos[pos][:, None, :], self.sin[pos][:, None, :]
        a, b = x[..., :half], x[..., half:]
        return torch.cat([a * cs - b * sn, b * cs + a * sn], dim=-1)

    def _project(self, l, x, pos):
        """x [n, d] -> q bf16 [1, Hq, n, D]; k, v bf16 [Hkv, n, D]."""
        c, P = self.cfg, self.layers[l]
        n = x.shape[0]
        a = self._rms(x, P["attn_norm"])
        q = self._rope((a @ P["wq"]).view(n, c.Hq, c.D), pos)
        k = self._rope((a @ P["wk"]).view(n, c.Hkv, c.D), pos)
        v = (a @ P["wv"]).view(n, c.Hkv, c.D)
        q = q.to(torch.bfloat16).transpose(0, 1).contiguous().unsqueeze(0)
        return q, k.to(torch.bfloat16).transpose(0, 1), v.to(torch.bfloat16).transpose(0, 1)

    def _finish(self, l, x, o):
        """x [n, d]; o fp32 [Hq, n, D]."""
        c, P = self.cfg, self.layers[l]
        n = x.shape[0]
        x = x + o.transpose(0, 1).reshape(n, c.Hq * c.D) @ P["wo"]
        a = self._rms(x, P["ffn_norm"])
        return x + (F.silu(a @ P["w_gate"]) * (a @ P["w_up"])) @ P["w_down"]

    def _logits(self, x):
        return self._rms(x, self.final_norm) @ self.head

    # ------------------------------------------------------------ passes

    def causal_pass(self, ids: torch.Tensor, start: int) -> torch.Tensor:
        """Positions start .. start + n - 1 through every layer in one causal
        pass over the full cache (vc_verify_attn); returns final hidden [n, d]."""
        c = self.cfg
        n = ids.shape[0]
        pos = torch.arange(start, start + n, device=self.dev)
        x = self.embed[ids.long()]
        self.ctx_t.fill_(start)
        ws = self.verify_ws
        need = vc.verify_ws_bytes(1, c.Hq, c.Hkv, c.D, n, start)
        if need > ws.numel():
            ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
        for l in range(c.n_layers):
            q, k, v = self._project(l, x, pos)
            self.K[l][0, :, start:start + n] = k
            self.V[l][0, :, start:start + n] = v
            o = vc.verify_attn(q, self.full[l], self.ctx_t, start, c.Hkv, self.scale, ws=ws)
            x = self._finish(l, x, o[0])
        return x

    def prefill(self, prompt: torch.Tensor) -> torch.Tensor:
        """Full-cache prefill, then the int4 draft cache of every layer.  Returns
        the last prompt position's logits [V]."""
        c = self.cfg
        P = prompt.shape[0]
        if self.staging is not None:
            torch.cuda.current_stream().wait_event(self.staging.free)
        x = self.causal_pass(prompt, 0)
        self.comp = [vc.quantize_kv(self.K[l], self.V[l], c.bits, P) for l in range(c.n_layers)]
        if self.staging is not None:
            self._write_back(0, P)
        self.draft_ws = torch.zeros(vc.draft_ws_bytes(1, c.Hq, c.Hkv, c.D, P + c.T_cap), dtype=torch.uint8,
                                    device=self.dev)
        return self._logits(x[-1:])[0]

    def draft_step(self, tok: torch.Tensor, pos: int, row: int) -> torch.Tensor:
        """One draft position (token tok, int32 [1] on the device) at position
        pos, writing its tail row `row`; returns its logits [1, V]."""
        c = self.cfg
        x = self.embed[tok.long()]
        p = self._pos(pos)
        self.tail_len.fill_(row + 1)
        for l in range(c.n_layers):
            q, k, v = self._project(l, x, p)
            self.TK[l][0, :, row] = k[:, 0]
            self.TV[l][0, :, row] = v[:, 0]
            o = vc.draft_attn(self.comp[l], self.tails[l], q[:, :, 0].contiguous(), self.scale, out=self.q_out,
                              ws=self.draft_ws, Hkv=c.Hkv)
            x = self._finish(l, x, o[0][:, None, :])
        return self._logits(x)

    # ------------------------------------------------------------ host-resident full cache

    def _write_back(self, r0: int, n: int):
        """Rows [r0, r0 + n) of the staging region -> this group's host cache,
        then mark the region free (on the current stream)."""
        for l in range(self.cfg.n_layers):
            self.K_h[l][0, :, r0:r0 + n].copy_(self.K[l][0, :, r0:r0 + n], non_blocking=True)
            self.V_h[l][0, :, r0:r0 + n].copy_(self.V[l][0, :, r0:r0 + n], non_blocking=True)
        self.staging.free.record(torch.cuda.current_stream())

    def fetch(self, copy_stream):
        """Copy this group's full cache into the staging region on copy_stream,
        once the region's last user is done with it; verify_round waits for
        the copy."""
        copy_stream.wait_event(self.staging.free)
        with torch.cuda.stream(copy_stream):
            for l in range(self.cfg.n_layers):
                self.K[l].copy_(self.K_h[l], non_blocking=True)
                self.V[l].copy_(self.V_h[l], non_blocking=True)
            self.landed.record(copy_stream)

    def _pos(self, pos: int) -> torch.Tensor:
        return torch.full((1,), pos, dtype=torch.int64, device=self.dev)

    # ------------------------------------------------------------ graph-captured drafting

    def _draft_step_dev(self):
        """One draft position with all of its state on the device: token g_tok,
        position g_pos, tail row g_row, draft slot g_j.  Writes the drafted
        token into g_tok and g_drafts[g_j] and advances the counters, so the
        same recorded work can be replayed for every position of a round."""
        c = self.cfg
        x = self.embed[self.g_tok.long()]
        self.tail_len.copy_(self.g_row + 1)
        for l in range(c.n_layers):
            q, k, v = self._project(l, x, self.g_pos)
            self.TK[l].index_copy_(2, self.g_row, k.unsqueeze(0))
            self.TV[l].index_copy_(2, self.g_row, v.unsqueeze(0))
            o = vc.draft_attn(self.comp[l], self.tails[l], q[:, :, 0].contiguous(), self.scale, out=self.q_out,
                              ws=self.draft_ws, Hkv=c.Hkv)
            x = self._finish(l, x, o[0][:, None, :])
        vc.argmax(self._logits(x), ids=self.g_tok)
        self.g_drafts.index_copy_(0, self.g_j, self.g_tok)
        self.g_pos += 1
        self.g_row += 1
        self.g_j += 1

    def _capture_draft_step(self):
        """Record _draft_step_dev as a HIP graph (after one eager run, which sets
        up library handles and the kernels' occupancy caches).  The recorded work
        allocates nothing and sets no memory with hipMemset."""
        dev = self.dev
        self.g_tok = torch.zeros(1, dtype=torch.int32, device=dev)
        self.g_pos = torch.zeros(1, dtype=torch.int64, device=dev)
        self.g_row = torch.zeros(1, dtype=torch.int64, device=dev)
        self.g_j = torch.zeros(1, dtype=torch.int64, device=dev)
        self.g_drafts = torch.zeros(self.cfg.k, dtype=torch.int32, device=dev)
        saved = [(t.clone(), u.clone()) for t, u in zip(self.TK, self.TV)]
        self.g_pos.fill_(self.cfg.prompt)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self._draft_step_dev()
        torch.cuda.current_stream().wait_stream(s)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._draft_step_dev()
        for (t, u), T, V in zip(saved, self.TK, self.TV):   # undo the eager run's tail writes
            T.copy_(t)
            V.copy_(u)

    # ------------------------------------------------------------ the loop

    def start(self, prompt: np.ndarray, graph: bool = False):
        """Prefill, the first token and (graph) the recorded draft position, on
        the current stream.  Then draft_round / verify_round advance the loop."""
        c = self.cfg
        self.P = len(prompt)
        ids = torch.from_numpy(np.asarray(prompt, dtype=np.int32)).to(self.dev)
        lg = self.prefill(ids)
        self.pending = vc.argmax(lg[None])                  # int32 [1]
        self.use_graph = graph
        if graph:
            self._capture_draft_step()
        self.out = [int(self.pending.item())]
        self.top1 = [float(lg.max().item())]
        self.ctx = self.P
        self.accepted = []
        self.drafts = torch.empty((1, c.k), dtype=torch.int32, device=self.dev)

    def done(self, n_gen: int) -> bool:
        return len(self.out) >= n_gen

    def draft_round(self, k: int):
        """Enqueue k draft positions (k <= cfg.k) on the current stream."""
        c = self.cfg
        if not 1 <= k <= c.k:
            raise ValueError(f"draft length {k} outside [1, {c.k}]")
        ctx, P = self.ctx, self.P
        if self.use_graph:
            self.g_tok.copy_(self.pending)
            self.g_pos.fill_(ctx)
            self.g_row.fill_(ctx - P)
            self.g_j.zero_()
            for _ in range(k):
                self.graph.replay()
            self.drafts[0, :k].copy_(self.g_drafts[:k])
        else:
            tok = self.pending
            for j in range(k):
                lgd = self.draft_step(tok, ctx + j, ctx - P + j)
                tok = vc.argmax(lgd, ids=self.drafts[0, j:j + 1])

    def verify_round(self, k: int) -> int:
        """Verify the pending token and the k drafts of the last draft_round in
        one causal pass, accept, and move the verified rows into the draft
        tail.  Waits for the accept result; returns the accepted count."""
        c = self.cfg
        ctx, P = self.ctx, self.P
        if self.staging is not None:
            torch.cuda.current_stream().wait_event(self.landed)
        seq = torch.cat([self.pending, self.drafts[0, :k]])
        x = self.causal_pass(seq, ctx)
        vlog = self._logits(x)
        emitted, n_acc = vc.accept(self.drafts[:, :k].contiguous(), vlog[None])
        n = int(n_acc.item())
        self.out.extend(emitted[0, :n + 1].tolist())
        self.top1.extend(vlog[:n + 1].max(dim=-1).values.tolist())
        self.accepted.append(n)
        r0 = ctx - P
        for l in range(c.n_layers):
            self.TK[l][0, :, r0:r0 + n + 1] = self.K[l][0, :, ctx:ctx + n + 1]
            self.TV[l][0, :, r0:r0 + n + 1] = self.V[l][0, :, ctx:ctx + n + 1]
        if self.staging is not None:
            self._write_back(ctx, n + 1)
        self.ctx = ctx + n + 1
        self.pending = emitted[0, n:n + 1].clone()
        return n

    def generate(self, prompt: np.ndarray, n_gen: int, graph: bool = False):
        """Returns (tokens [n_gen] list, per-round accepted counts, stats dict
        with timings and the logit of every emitted token).  graph: replay a
        HIP graph of one draft position k times per round instead of issuing
        its ~200 launches from the host each time (recorded after the
        prefill, outside the timed decode)."""
        c = self.cfg
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.start(prompt, graph=False)
        torch.cuda.synchronize()
        t_pre = time.perf_counter()
        if graph:
            self.use_graph = True
            self._capture_draft_step()
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        while not self.done(n_gen):
            self.draft_round(c.k)
            self.verify_round(c.k)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        out = self.out[:n_gen]
        stats = dict(prefill_s=t_pre - t0, decode_s=t2 - t1, rounds=len(self.accepted), top1=self.top1[:n_gen],
                     graph=graph, tokens_per_s=(len(out) - 1) / (t2 - t1) if t2 > t1 else 0.0)
        return out, self.accepted, stats
