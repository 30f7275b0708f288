"""The staggering scheduler's draft-length rule, written from its definition.

TEST INFRASTRUCTURE ONLY: imported by tests/ alone; the library's policy
(vc_sched_* in libvc) is separate code.

[VC Key System Innovations P2] high acceptance of same-model compressed
drafting lets the system verify less often; [P1] one request group drafts while
another loads its full KV and verifies.  The pages give no formula; the rule
is: each draft of a round matches with probability a until the first mismatch;
a is estimated from the group's history with one prior match and one prior
mismatch; the next draft length k in [k_min, k_max] maximises expected emitted
tokens over the round time max(k t_draft, t_overlap) + t_rest, ties to the
smaller k.  fp64 throughout.
"""
from __future__ import annotations


def accept_rate(accepted: int, rejections: int) -> float:
    """(accepted + 1) / (accepted + rejections + 2)."""
    return (accepted + 1.0) / (accepted + rejections + 2.0)


def expected_tokens(a: float, k: int) -> float:
    """1 + a + a^2 + ... + a^k, summed in that order: the accepted drafts plus
    the verifier's token of one round."""
    s, p = 1.0, 1.0
    for _ in range(k):
        p = p * a
        s = s + p
    return s


def round_time(k: int, t_draft: float, t_overlap: float, t_rest: float) -> float:
    return max(k * t_draft, t_overlap) + t_rest


def choose_k(accepted: int, rejections: int, t_draft: float, t_overlap: float, t_rest: float, k_min: int,
             k_max: int) -> int:
    a = accept_rate(accepted, rejections)
    rate = {k: expected_tokens(a, k) / round_time(k, t_draft, t_overlap, t_rest) for k in range(k_min, k_max + 1)}
    best = max(rate.values())
    return min(k for k, r in rate.items() if r == best)
