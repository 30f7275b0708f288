"""Parity at the full long-context shapes, in the launch configuration the
benchmark times (same workload builder, same entry points, same grids).

The GPU computes every (batch, kv-head) unit; the fp64 oracle recomputes every
unit too (first and last draft step, the whole verify pass), one unit per
worker thread, and each unit must meet the attention tolerance.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import round as R
from synth import configs as C

from test_parity_gpu import assert_close

# The draft kernel's own accuracy is far inside the acceptance bar; a rel-L2
# above this flags a numerical regression (e.g. a biased operand split).
DRAFT_DESIGN_REL = 1e-4

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

FULL = [C.LLAMA8B, C.QWEN32B, C.LLAMA70B]
CHUNK = 8   # units per test case: each case reports within seconds


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(8, n))


_RUN = {}   # the GPU outputs and inputs of one workload, computed once for its chunks


def _gpu_run(w):
    if w.name not in _RUN:
        import torch
        from compressed_kv_draft_amd.workload import DeviceWorkload
        _RUN.clear()    # one workload's inputs in memory at a time
        print(f"[case] full-size {w.name}: building inputs and running the GPU path", flush=True)
        dw = DeviceWorkload(w, device="cuda:0", with_vocab=False)
        steps = [0, w.k - 1]
        for j in steps:
            dw.draft_step(j)
        dw.verify()
        torch.cuda.synchronize()
        _RUN[w.name] = dict(steps=steps, dout=dw.draft_out.cpu().numpy(), vout=dw.verify_out.cpu().numpy(),
                            npd=dw.np, keep=dw.keep_np if w.kind == "token_drop" else None)
        del dw
        torch.cuda.empty_cache()
    return _RUN[w.name]


def _cases():
    out = []
    for w in FULL:
        units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
        for i in range(0, len(units), CHUNK):
            out.append((w, units[i:i + CHUNK]))
    return out


@pytest.mark.parametrize("w,units", _cases(), ids=lambda x: getattr(x, "name", None) or f"units{x[0][0]}_{x[0][1]}")
def test_full_shape_every_unit(w, units):
    """Every (batch, kv-head) unit of the full-size workload, CHUNK units per case:
    the first and last draft step and the whole verify against the oracle."""
    r = _gpu_run(w)
    steps, dout, vout, npd, keep_np = r["steps"], r["dout"], r["vout"], r["npd"], r["keep"]
    g = w.g

    def oracle_unit(bh):
        b, h = bh
        keep = keep_np[b, h] if keep_np is not None else None
        args = (npd["K"][b, h], npd["V"][b, h], npd["Kn"][b, h], npd["Vn"][b, h], npd["Q"][b, h * g:(h + 1) * g])
        return bh, R.unit_draft(w, *args, keep=keep, positions=steps), R.unit_verify(w, *args)

    worst = 0.0
    with ThreadPoolExecutor(_workers()) as ex:
        for (b, h), ref, refv in ex.map(oracle_unit, units):
            for j in steps:
                got = dout[j, b, h * g:(h + 1) * g]
                assert_close(got, ref[:, j], f"{w.name} draft step {j} b{b} h{h}")
                rel = np.linalg.norm(got - ref[:, j]) / np.linalg.norm(ref[:, j])
                worst = max(worst, rel)
                assert rel <= DRAFT_DESIGN_REL, (w.name, j, b, h, rel)
            assert_close(vout[b, h * g:(h + 1) * g], refv, f"{w.name} verify b{b} h{h}")
    print(f"[result] {w.name} units {units[0]}..{units[-1]}: worst draft rel-L2 {worst:.2e}", flush=True)
