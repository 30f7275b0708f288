"""Write the expected output of the end-to-end tiny-decoder run (calls only oracle/ and synth/).

    python tests/golden/make_e2e_golden.py [--loop]

Runs the fp64 oracle: prefill of the 16384-token prompt, then plain greedy
decoding with the full cache for 256 tokens, recording per step the token, its
logit and the gap to the runner-up.  With --loop it also runs the oracle's own
draft-then-verify loop (int4 draft cache, k = 32) and records its per-round
accepted counts and whether its output equals the greedy one.  The prefill in
float64 takes several minutes on 8 cores.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import e2e as E  # noqa: E402
from synth import configs as C  # noqa: E402
from synth import model as M  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e2e_" + C.LM_E2E.name + ".txt")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--loop", action="store_true")
    args = ap.parse_args()
    cfg = C.LM_E2E
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    m = E.Model(cfg, W, cos, sin)
    p = M.prompt(cfg)
    t = time.time()
    cache = E.Cache(cfg)
    first = E.prefill(m, cache, p)
    print(f"prefill {time.time() - t:.0f} s", flush=True)
    saved = ([k[:, :cfg.prompt].copy() for k in cache.K], [v[:, :cfg.prompt].copy() for v in cache.V])
    toks, top, marg = E.greedy_decode(m, p, cfg.n_gen, cache=cache, first_logits=first)
    print(f"greedy done; min margin {marg.min():.4f}", flush=True)
    lines = [
        "# Expected output of the end-to-end tiny-decoder run, written by make_e2e_golden.py",
        "# from the fp64 oracle (greedy decoding with the full cache).",
        f"config={cfg.name}",
        f"n_layers={cfg.n_layers} d_model={cfg.d_model} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} ffn={cfg.ffn} "
        f"vocab={cfg.vocab} prompt={cfg.prompt} k={cfg.k} n_gen={cfg.n_gen} bits={cfg.bits} "
        f"q_gain={cfg.q_gain} plant={cfg.plant} seed={cfg.seed}",
        "tokens=" + " ".join(str(int(x)) for x in toks),
        "top1=" + " ".join(f"{x:.6f}" for x in top),
        "margin=" + " ".join(f"{x:.6f}" for x in marg),
        f"min_margin={marg.min():.6f}",
    ]
    if args.loop:
        c2 = E.Cache(cfg)
        for l in range(cfg.n_layers):
            c2.K[l][:, :cfg.prompt] = saved[0][l]
            c2.V[l][:, :cfg.prompt] = saved[1][l]
        t = time.time()
        tv, acc, _ = E.vericache_decode(m, p, cfg.n_gen, cache=c2, first_logits=first)
        print(f"loop {time.time() - t:.0f} s; equal {np.array_equal(tv, toks)}; accepted {acc}", flush=True)
        lines += ["oracle_loop_accepted=" + " ".join(str(a) for a in acc),
                  f"oracle_loop_equal={int(np.array_equal(tv, toks))}"]
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
