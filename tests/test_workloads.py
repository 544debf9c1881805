"""The seeded generators are deterministic and shaped as the workloads say."""

import numpy as np
import torch

import workloads as W


def test_five_workloads():
    assert [w.index for w in W.WORKLOADS] == [0, 1, 2, 3, 4]
    w2 = W.get(2)
    assert (w2.batch, w2.n_q_heads, w2.n_kv_heads, w2.head_dim) == (4, 32, 8, 128)
    assert w2.capacity == 2048 + 128 and w2.group == 4
    assert W.get("tiny").capacity == 64 + 8


def test_draws_are_seeded_bf16():
    a = W.normal_bf16((4, 8), 1, 0, 0, "q")
    b = W.normal_bf16((4, 8), 1, 0, 0, "q")
    c = W.normal_bf16((4, 8), 1, 0, 1, "q")
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    assert not torch.equal(a, c)
    w = W.normal_bf16((20000,), 0, 0, 0, "w_q", std=0.02).float()
    assert abs(w.std().item() - 0.02) < 1e-3


def test_ragged_lengths():
    lens = W.ragged_lengths(3, 4, (512, 1024, 1536, 2048))
    assert len(lens) == 4 and len(set(lens)) >= 2
    assert set(lens) <= {512, 1024, 1536, 2048}
    assert lens == W.ragged_lengths(3, 4, (512, 1024, 1536, 2048))
    cu, pos = W.packed_layout([3, 2], start=[0, 5])
    assert cu.tolist() == [0, 3, 5] and pos.tolist() == [0, 1, 2, 5, 6]
