"""Helpers for the GPU parity tests (import only from tests)."""
import sys

import numpy as np
import pytest

COEF_ATOL = 1e-5  # float32 coefficients vs the oracle (absolute)


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    import normalized_cross_correlation_amd as ncc
    ncc.lib()  # raises when libncc.so is missing: the HIP path must run
    return torch.device("cuda:0")


def dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


class route:
    """Context manager selecting the library's correlation route (None: the
    default choice) through ncc_set_option; restores the previous route."""

    def __init__(self, name):
        self.name = name or "auto"

    def __enter__(self):
        import normalized_cross_correlation_amd as ncc
        self.ctx = ncc.options(route=self.name)
        self.ctx.__enter__()

    def __exit__(self, *a):
        self.ctx.__exit__(*a)
