"""Facts the pages print (tests/golden/pages_facts.json), checked against this library."""
import json
import os

import pytest
import torch

import synth

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def test_uneven_split_and_shard_width():
    f = FACTS["uneven_split"]
    assert synth.default_split(f["V"], f["ranks"]) == f["widths"]
    g = FACTS["tp8_shard_width"]
    assert synth.default_split(g["V"], g["tp"]) == [g["v_local"]] * g["tp"]
    assert synth.WORKLOADS["tp8_shard"].V == g["v_local"]


def test_jsd_peak_memory_accounting_on_host():
    """The printed peaks are exactly 3 bf16 [N, V_local] tensors: two resident inputs
    and one student gradient."""
    f = FACTS["jsd_peak_memory"]
    N = f["workload"]["N"]
    for tp, gib in f["peak_allocated_gib_per_rank"].items():
        v = f["v_local"][tp]
        assert v * int(tp) == f["workload"]["V"]
        assert abs(3 * N * v * 2 / 2**30 - gib) < 0.0005


@pytest.mark.gpu
@pytest.mark.parametrize("tp", ["2", "4"])
def test_jsd_peak_memory_matches_the_pages(tp):
    import vocab_sharded_softmax_amd as vj

    f = FACTS["jsd_peak_memory"]
    N, v = f["workload"]["N"], f["v_local"][tp]
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    b = synth.draw("full_vocab", device="cuda", N=N, V=v)
    s = b.s.requires_grad_()
    t = b.t  # frozen teacher
    del b
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    loss = vj.jsd(s, t, f["workload"]["beta"])
    loss.sum().backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    assert s.grad is not None and s.grad.dtype == torch.bfloat16
    three = 3 * N * v * 2  # two resident input shards + one student gradient
    # beyond those, only O(N) statistics and a workspace whose size does not depend on V
    extra = peak - three
    assert 0 <= extra <= vj.vjsd_workspace_bytes(N, 1) + 64 * N + (1 << 20), extra
    assert extra < 4 << 20
    # so the peak is the pages' figure up to that V-independent allowance
    assert abs(three / 2**30 - f["peak_allocated_gib_per_rank"][tp]) < 0.0005
