"""CPU checks of the trainer around the optimizer (no GPU needed)."""
import numpy as np
import pytest
import torch

import workloads
from trainer.gpt import GPT, count_params, lr_at
from trainer.loop import Tape


def test_gpt_matches_the_gpt11m_tensor_list():
    m = GPT()
    sizes = sorted(p.numel() for p in m.parameters())
    assert count_params(m) == workloads.total(2) == 11256832
    assert sizes == sorted(workloads.sizes(2))


def test_init_rule():
    m = GPT(layers=1)
    for name, p in m.named_parameters():
        if name.endswith("bias"):
            assert torch.all(p == 0), name
        elif ".ln" in name or name.startswith("lnf"):
            assert torch.all(p == 1), name
        else:
            assert abs(float(p.std()) - 0.02) < 0.003, name


def test_forward_shapes_and_loss_on_cpu():
    m = GPT(layers=1, ctx=64)
    x = torch.randint(0, 12096, (2, 16))
    loss = m(x, x)
    assert loss.ndim == 0 and np.isfinite(float(loss))
    assert m(x).shape == (2, 16, 12096)


def test_tape_is_sequential_and_never_wraps():
    t = Tape(np.arange(21, dtype=np.int64), 2, 5)
    x, y = t.next("cpu")
    assert x.tolist() == [[0, 1, 2, 3, 4], [5, 6, 7, 8, 9]] and y[0, 0] == 1
    t.next("cpu")
    with pytest.raises(RuntimeError, match="exhausted"):
        t.next("cpu")


def test_schedule():
    assert lr_at(1, 1.0, 4, 10) == 0.25 and lr_at(4, 1.0, 4, 10) == 1.0
    assert lr_at(10, 1.0, 4, 10) == 0.0 and lr_at(7, 1.0, 4, 10) == 0.5
