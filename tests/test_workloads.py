"""The seeded input generators (CPU)."""
import numpy as np
import torch

import workloads as W


def test_seeded_and_shaped():
    a = W.make("a", 2, 70, 3, 5, init="fp32")
    b = W.make("a", 2, 70, 3, 5, init="fp32")
    for x, y in ((a.q, b.q), (a.g, b.g), (a.beta, b.beta), (a.initial_state, b.initial_state)):
        assert torch.equal(x, y)
    assert a.q.shape == (2, 70, 3, 128) and a.beta.shape == (2, 70, 3) and a.q.dtype == torch.bfloat16
    assert a.A_log.dtype == torch.float32 and a.dt_bias.shape == (3, 128)
    assert ((a.A_log >= 0) & (a.A_log <= np.log(16) + 1e-6)).all()


def test_varlen_lengths_procedure():
    lens = W.varlen_lengths(32768, 37, 8192, 1103)
    assert sum(lens) == 32768
    assert all(L % 64 != 0 for L in lens) and min(lens) >= 37
    assert lens == W.varlen_lengths(32768, 37, 8192, 1103)


def test_config_shapes():
    for i in range(5):
        s = W.config_shape(i)
        assert s["K"] == 128 and s["V"] == 128
    w = W.config(3)
    assert w.cu_seqlens[-1].item() == 32768 and w.initial_state.shape[0] == w.N
