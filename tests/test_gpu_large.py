"""Tensors of more than 2^31 elements: every index past that point must be formed in 64
bits.  The one call and the two calls on 16391 x 151936 (two-sweep rows) and 140003 x
16032 (register-held rows) bf16 pairs, both gradients, bit for bit against each other,
with rows at both ends and past the 2^31st element against the fp64 oracle; entropy
forward and backward on the larger of them."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_values
from test_gpu_fwd_bwd import check_oracle, check_two_calls
from test_gpu_siblings import run_entropy

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31


@pytest.fixture(autouse=True)
def _release_memory():
    """These tests hold tens of GB; hand them back to the device afterwards."""
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,V", [(16391, 151936), (140003, 16032)])
def test_jsd_beyond_2_31_elements(N, V):
    assert N * V > LIMIT
    b = synth.draw("full_vocab", device="cuda", N=N, V=V, seed=77)
    res, gout = check_two_calls(b.s, b.t, 0.4)
    first_past = LIMIT // V + 1  # the first row that starts past element 2^31
    rows = np.array([0, N // 2, first_past - 1, first_past, N - 1])
    check_oracle(b.s, b.t, 0.4, gout, res, rows=rows)


def test_entropy_beyond_2_31_elements():
    N, V = 16391, 151936
    b = synth.draw("full_vocab", device="cuda", N=N, V=V, seed=78)
    x = b.s
    del b
    gout = torch.rand(N, generator=torch.Generator(device="cuda").manual_seed(3),
                      device="cuda") + 0.5
    g = run_entropy(x, None, gout)
    rows = np.array([0, LIMIT // V, LIMIT // V + 1, N - 1])
    xc = x[rows].cpu()
    ref = oracle.entropy(xc, gout=gout[rows].cpu().double().numpy())
    assert_values(g["ent"][rows], ref["ent"], x.dtype, "entropy")
    assert_grads(g["gx"][rows], ref["gx"], x.dtype, "d/dx")
