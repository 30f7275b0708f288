"""Workload shapes (sizes only; no arithmetic of the method).

Single-layer attention workloads shaped like the models the VeriCache pages
evaluate, plus a tiny case small enough for exhaustive oracle checks.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int            # context tokens already in the cache
    k: int            # draft length; verify runs n_q = k + 1 positions
    kind: str         # draft compressor: 'quant' | 'token_drop' | 'identity'
    bits: int = 4     # quant only
    residual: int = 0  # trailing context tokens kept exact (bf16) in the draft cache
    keep_frac: float = 0.0  # token_drop only
    vocab: int = 1024
    paged: bool = False
    page_tokens: int = 16
    groups: int = 1   # request groups for staggering
    chunk_tokens: int = 4096
    seed: int = 1

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_q(self) -> int:
        return self.k + 1

    @property
    def n_quant(self) -> int:
        return self.L - self.residual if self.kind == "quant" else 0

    @property
    def n_keep(self) -> int:
        return int(self.keep_frac * self.L) if self.kind == "token_drop" else 0

    @property
    def w_std(self) -> float:
        return (1.0 / (self.Hq * self.D)) ** 0.5

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny_b1_h4x1_d64_l512_int4_k8", B=1, Hq=4, Hkv=1, D=64, L=512, k=8,
                kind="quant", bits=4, residual=0, vocab=1024, seed=1)
LLAMA8B = Workload("llama3_8b_layer_b8_l32k_int2_k32", B=8, Hq=32, Hkv=8, D=128, L=32768, k=32,
                   kind="quant", bits=2, residual=128, vocab=32000, seed=2)
QWEN32B = Workload("qwen_32b_layer_b4_l128k_drop10_k32", B=4, Hq=64, Hkv=8, D=128, L=131072, k=32,
                   kind="token_drop", keep_frac=0.1, vocab=32000, seed=3)
LLAMA70B = Workload("llama_70b_layer_b16_l64k_int4_paged_k32", B=16, Hq=64, Hkv=8, D=128, L=65536, k=32,
                    kind="quant", bits=4, residual=128, vocab=32000, paged=True, page_tokens=16,
                    groups=2, chunk_tokens=4096, seed=4)

ALL = {w.name: w for w in (TINY, LLAMA8B, QWEN32B, LLAMA70B)}


@dataclass(frozen=True)
class TinyLM:
    """A small Llama-style decoder run end to end through the draft-then-verify loop.

    Architecture (the pages name none): pre-norm blocks of RMSNorm -> Q/K/V
    projections -> rotary positions -> GQA attention -> output projection ->
    residual, then RMSNorm -> SwiGLU feed-forward -> residual; a final RMSNorm
    and an untied vocabulary head.  Weight matrices are stored [in, out]."""
    name: str
    n_layers: int
    d_model: int
    Hq: int
    Hkv: int
    D: int
    ffn: int
    vocab: int
    prompt: int       # prompt tokens (all quantised for the draft cache)
    k: int            # draft length
    n_gen: int        # generated tokens
    bits: int = 4
    q_gain: float = 1.0   # W_q std multiplier: sharpens attention so that the lossy draft matters
    plant: float = 0.0    # successor-plant strength (logit units) added to the vocabulary head
    rope_theta: float = 10000.0
    eps: float = 1e-5
    seed: int = 5

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def L_cap(self) -> int:
        """Rows of the full cache: prompt + generated + one round of drafts, rounded up to 64."""
        n = self.prompt + self.n_gen + self.k + 1
        return (n + 63) // 64 * 64

    @property
    def T_cap(self) -> int:
        """Rows of the draft's exact tail: generated rows plus one round of drafts, rounded up to 32."""
        n = self.n_gen + self.k + 1
        return (n + 31) // 32 * 32

    def with_(self, **kw) -> "TinyLM":
        return replace(self, **kw)


LM_E2E = TinyLM("tiny_lm_4l_d1024_p16k_int4_k32_g256", n_layers=4, d_model=1024, Hq=16, Hkv=4, D=64,
                ffn=2816, vocab=32000, prompt=16384, k=32, n_gen=256, bits=4, q_gain=3.0, plant=12.0, seed=5)
LM_SMALL = TinyLM("small_lm_2l_d256_p256_int4_k8_g40", n_layers=2, d_model=256, Hq=4, Hkv=2, D=64,
                  ffn=512, vocab=2048, prompt=256, k=8, n_gen=40, bits=4, q_gain=1.0, plant=6.0, seed=15)
