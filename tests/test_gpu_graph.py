"""A step captured in a HIP graph (through torch.cuda.graph) replays to the same
bits as the step run eagerly: the library records only kernel launches on the
stream it is given (no memsets, no allocations, no host synchronisation).

Each replay follows eager work of the program's own (poisoning the output and
the appended slots, then a synchronisation), and every replay is compared with
the eager result, output and pools, bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from paged_kv_cache_286_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small(Hq, Hkv, D, kv, qd, lens, qlens, seed):
    nb = sum(-(-int(L) // 16) for L in lens) + 17
    cfg = W.Config("small", "small", Hq, Hkv, D, 16, nb, kv, qd, seed)
    return W.generate(W.custom_plan(cfg, lens, qlens, seed))


CASES = {
    "tiny_decode": lambda: W.generate(W.make_plan("tiny_decode")),
    # split partitions and the merge launch
    "decode_split_bf16": lambda: _small(8, 8, 128, W.BF16, W.BF16, [1, 700, 3000, 4096], [1, 1, 1, 1], 21),
    # the prologue, prefill items, verify rows and decode items in one step (fp8, GQA)
    "mixed_fp8_gqa": lambda: _small(16, 2, 128, W.FP8, W.BF16, [90, 1000, 2500, 40], [90, 64, 1, 4], 22),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay_matches_eager(name):
    from paged_kv_cache_286_amd.device import DeviceStep
    wl = CASES[name]()
    _say(f"[gpu] graph replay {name}: seqs={wl.plan.num_seqs} rows={wl.plan.total_q_tokens}")
    ds = DeviceStep(wl)
    ds.step()
    torch.cuda.synchronize()
    out_ref = ds.out.clone()
    k_ref, v_ref = ds.k_pool.clone(), ds.v_pool.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm the capture stream once, eagerly
        ds.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.step()
    torch.cuda.synchronize()
    for r in range(3):
        ds.out.fill_(-1)                     # eager work between replays
        ds.poison_appended_slots()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ds.out, out_ref), f"replay {r}: output differs from the eager step"
        assert torch.equal(ds.k_pool, k_ref) and torch.equal(ds.v_pool, v_ref), \
            f"replay {r}: pools differ from the eager step"
    _say(f"    3 replays bit-identical to the eager step")
