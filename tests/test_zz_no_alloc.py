"""The allocation-free attention entry point (``wf_wave_attention_noalloc``)
against ``wf_wave_attention``: same kernels, the split groups' partial
results in the library's static device array instead of the handle's table
buffer.  Two requests in a row, the second smaller, each compared bit for
bit with the table-buffer path under a forced split (every round splits its
two longest groups, so the static array is written and read every round);
a split that needs more than the array holds is rejected before any launch.
"""

import gc

import pytest
import torch

from chunk_causal_dit_round_amd import wf
from chunk_causal_dit_round_amd.workloads import WAN14B_4STEP, Workload
from wfcheck import Rollout

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _outputs(w, noalloc, split=wf.WF_SPLIT_FORCE):
    """out of every round of request ``w`` (publish + attention per layer)."""
    ro = Rollout(w, split=split)
    s = ro.sess
    outs = []
    try:
        for k in range(w.n_chunk + w.S):
            ro.fill(k)
            plan = s.plan(k)
            for layer in range(w.n_layers):
                s.publish(plan, layer)
                if noalloc:
                    wf.wf_wave_attention_noalloc(s.h, plan, layer, s.bufs["q_rot"][layer],
                                                 s.bufs["out"][layer])
                else:
                    s.attention(plan, layer)
            s.commit(plan)
            torch.cuda.synchronize()
            outs.append(s.bufs["out"].clone())
    finally:
        ro.close()
    return outs


CASES = [
    # larger first: 360 tokens, 3 heads, two layers, five stages
    Workload("noalloc_n360", S=4, W=4, n_chunk=10, F=3, Hh=10, Ww=12, n_heads=3,
             head_dim=128, n_layers=2),
    # then a smaller request: the array still holds the first one's partials
    Workload("noalloc_n72", S=2, W=2, n_chunk=6, F=3, Hh=4, Ww=6, n_heads=2,
             head_dim=128, n_layers=1),
]


def test_noalloc_matches_table_buffer_path_two_requests():
    for w in CASES:
        print(f"{w.name}: {w.n_chunk + w.S} rounds", flush=True)
        ref = _outputs(w, noalloc=False)
        got = _outputs(w, noalloc=True)
        for k, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"{w.name} round {k}: outputs differ"


def test_noalloc_rejects_a_split_beyond_the_static_array():
    """14B-class shape, one layer: in round 1 the stage-0 group (two pages)
    is split under WF_SPLIT_FORCE, which needs 2 x (N H D + 2 N H) x 4 bytes
    = 195 MB of scratch, more than the 128 MiB array: WF_ESMALL and no
    launch.  With the split off the same call runs and equals the table-
    buffer path."""
    w = WAN14B_4STEP.with_(name="noalloc_14b", n_layers=1, n_chunk=3)
    nh = w.n_tokens * w.n_heads
    assert 2 * (nh * w.head_dim + 2 * nh) * 4 > wf.WF_STATIC_SCRATCH_BYTES
    ro = Rollout(w, split=wf.WF_SPLIT_FORCE)
    s = ro.sess
    try:
        ro.fill(0)
        plan = s.plan(0)
        s.publish(plan, 0)
        s.attention(plan, 0)
        s.commit(plan)
        ro.fill(1)
        plan = s.plan(1)
        s.publish(plan, 0)
        before = s.bufs["out"].clone()
        st = wf.status_of(wf.wf_wave_attention_noalloc, s.h, plan, 0, s.bufs["q_rot"][0],
                          s.bufs["out"][0])
        assert st == wf.WF_ESMALL, st
        assert "split scratch" in wf.wf_last_error()
        torch.cuda.synchronize()
        assert torch.equal(before, s.bufs["out"])
        wf.wf_set_attention_split(s.h, wf.WF_SPLIT_OFF)
        wf.wf_wave_attention_noalloc(s.h, plan, 0, s.bufs["q_rot"][0], s.bufs["out"][0])
        torch.cuda.synchronize()
        got = s.bufs["out"].clone()
        s.attention(plan, 0)
        torch.cuda.synchronize()
        assert torch.equal(got, s.bufs["out"])
    finally:
        ro.close()
