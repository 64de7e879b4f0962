"""Helpers for GPU tests: device copies of seeded host inputs (test code)."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev_u16(a):
    """uint16 bf16 bits (numpy) -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print(*a, flush=True)
