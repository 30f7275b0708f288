"""End-to-end draft-then-verify generation on the GPU against the oracle.

[VC Experimental Results] under greedy decoding the loop's output is the one
the model produces with its full cache.  The tiny decoder at full size (4
layers, d_model 1024, 16 query / 4 KV heads, head dim 64, 16384-token prompt,
int4 draft cache, k = 32, 256 tokens) must reproduce the oracle's full-cache
greedy tokens stored in tests/golden (written by make_e2e_golden.py, which
calls only oracle/); a smaller decoder is compared with the oracle run live.
Both runs must also reject at least one draft, so the rollback path runs.
"""
import os

import numpy as np
import pytest

from synth import configs as C
from synth import model as M

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(cfg):
    kv = {}
    with open(os.path.join(GOLD, f"e2e_{cfg.name}.txt")) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            if line.startswith("n_layers="):
                for item in line.split():
                    a, b = item.split("=")
                    kv[a] = b
                continue
            a, b = line.rstrip("\n").split("=", 1)
            kv[a] = b
    return kv


def _run(cfg, graph=False, W=None):
    from compressed_kv_draft_amd.tinylm import TinyLM
    W = M.weights(cfg) if W is None else W
    cos, sin = M.rope_tables(cfg)
    lm = TinyLM(cfg, W, cos, sin)
    return lm.generate(M.prompt(cfg), cfg.n_gen, graph=graph)


def _compare(cfg, toks, acc, stats, want, want_top1, margins):
    print(f"  rounds {stats['rounds']} accepted {acc} decode {stats['decode_s']:.3f} s "
          f"({stats['tokens_per_s']:.0f} tok/s) prefill {stats['prefill_s']:.3f} s", flush=True)
    n = min(len(toks), len(want))
    diff = [i for i in range(n) if toks[i] != want[i]]
    if diff:
        i = diff[0]
        pytest.fail(f"{cfg.name}: first mismatch at token {i}: got {toks[i]}, oracle {want[i]} "
                    f"(oracle margin there {margins[i]:.5f})")
    assert len(toks) == cfg.n_gen
    err = np.abs(np.array(stats["top1"]) - np.array(want_top1))
    print(f"  emitted-token logit |gpu - oracle| max {err.max():.2e}; min oracle margin {min(margins):.4f}",
          flush=True)
    assert err.max() < 0.25 * min(margins)
    assert min(acc) < cfg.k, "no draft rejected: rollback path untested"


def test_e2e_tiny_lm_equals_oracle_greedy():
    """Both ways of drafting (eager launches, and one recorded HIP graph per
    draft position replayed k times a round) reproduce the oracle's tokens and
    take identical drafts (equal accepted counts)."""
    cfg = C.LM_E2E
    g = _golden(cfg)
    assert g["config"] == cfg.name
    assert float(g["q_gain"]) == cfg.q_gain and float(g["plant"]) == cfg.plant and int(g["seed"]) == cfg.seed
    want = [int(x) for x in g["tokens"].split()]
    W = M.weights(cfg)
    runs = {}
    for graph in (False, True):
        print(f"[case] e2e {cfg.name} graph={graph}", flush=True)
        toks, acc, stats = _run(cfg, graph=graph, W=W)
        _compare(cfg, toks, acc, stats, want, [float(x) for x in g["top1"].split()],
                 [float(x) for x in g["margin"].split()])
        runs[graph] = (toks, acc)
    assert runs[True] == runs[False]


def test_e2e_small_lm_equals_oracle_greedy():
    from oracle import e2e as E
    cfg = C.LM_SMALL
    print(f"[case] e2e {cfg.name}", flush=True)
    cos, sin = M.rope_tables(cfg)
    m = E.Model(cfg, M.weights(cfg), cos, sin)
    want, top, marg = E.greedy_decode(m, M.prompt(cfg), cfg.n_gen)
    runs = {}
    for graph in (False, True):
        print(f"[case] e2e {cfg.name} graph={graph}", flush=True)
        toks, acc, stats = _run(cfg, graph=graph)
        _compare(cfg, toks, acc, stats, [int(x) for x in want], list(top), list(marg))
        runs[graph] = (toks, acc)
    assert runs[True] == runs[False]


def test_staggered_groups_adaptive_k_equal_oracle_greedy():
    """Two request groups on two streams (one verifies while the other
    drafts), each choosing its draft length per round with the library's
    policy, emit the oracle's greedy tokens for their prompts; so does the
    lock-step order on one stream.  With a fixed clock the decisions are
    reproducible and each equals the oracle's rule on the inputs the scheduler
    passed, whose acceptance counts must be the running sums of the rounds'
    outcomes.  One group's clock makes drafting dear, so it runs short rounds
    (draft lengths below the maximum take the variable-length path)."""
    from compressed_kv_draft_amd.groups import StaggeredGroups
    from compressed_kv_draft_amd.tinylm import TinyLM
    from oracle import e2e as E
    from oracle import sched as S
    cfg = C.LM_SMALL
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    m = E.Model(cfg, W, cos, sin)
    prompts = [M.prompt(cfg, r) for r in (0, 1)]
    want = [[int(x) for x in E.greedy_decode(m, p, cfg.n_gen)[0]] for p in prompts]
    fixed = {0: (0.1, 0.5), 1: (1.0, 0.5)}
    for stagger, clock in ((True, fixed.get), (True, None), (False, fixed.get)):
        print(f"[case] groups stagger={stagger} clock={'fixed' if clock else 'events'}", flush=True)
        base = TinyLM(cfg, W, cos, sin)
        lms = [base, TinyLM(cfg, None, None, None, shared=base)]
        res = StaggeredGroups(lms, k_min=1, k_max=cfg.k, stagger=stagger, clock=clock).run(prompts, cfg.n_gen)
        for g in range(2):
            ks = [r["k"] for r in res["rounds"][g]]
            print(f"  group {g}: k per round {ks}, accepted {[r['n'] for r in res['rounds'][g]]}", flush=True)
            assert [int(x) for x in res["tokens"][g]] == want[g], (stagger, g)
            acc = rej = 0
            for i, r in enumerate(res["rounds"][g]):
                assert 0 <= r["n"] <= r["k"] <= cfg.k
                acc += r["n"]
                rej += r["n"] < r["k"]
                if "next_k" in r:
                    a = r["policy_args"]
                    assert (a[0], a[1]) == (acc, rej)
                    assert r["next_k"] == S.choose_k(*a)
                    assert res["rounds"][g][i + 1]["k"] == r["next_k"]
        if clock is not None:
            assert min(r["k"] for r in res["rounds"][1]) < cfg.k
        del lms, base


def test_staggered_groups_host_full_kv_equal_oracle_greedy():
    """Full caches in pinned host memory and one shared device staging region
    (each group's full KV is copied in before its verification while the
    other group drafts, and the rows it adds are written back): both groups
    still emit the oracle's greedy tokens, staggered and lock-step."""
    from compressed_kv_draft_amd.groups import StaggeredGroups
    from compressed_kv_draft_amd.tinylm import FullStaging, TinyLM
    from oracle import e2e as E
    cfg = C.LM_SMALL
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    m = E.Model(cfg, W, cos, sin)
    prompts = [M.prompt(cfg, r) for r in (0, 1)]
    want = [[int(x) for x in E.greedy_decode(m, p, cfg.n_gen)[0]] for p in prompts]
    for stagger, clock in ((True, None), (False, {0: (1.0, 6.0), 1: (1.0, 0.5)}.get)):
        print(f"[case] groups host full KV stagger={stagger}", flush=True)
        st = FullStaging(cfg)
        base = TinyLM(cfg, W, cos, sin, staging=st)
        lms = [base, TinyLM(cfg, None, None, None, shared=base, staging=st)]
        res = StaggeredGroups(lms, k_min=1, k_max=cfg.k, stagger=stagger, clock=clock).run(prompts, cfg.n_gen)
        for g in range(2):
            print(f"  group {g}: k per round {[r['k'] for r in res['rounds'][g]]}", flush=True)
            assert [int(x) for x in res["tokens"][g]] == want[g], (stagger, g)
        del lms, base, st
