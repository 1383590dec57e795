"""Helpers for the GPU parity tests (inputs from `synth`, expectations from
`oracle`; nothing here computes any part of the method)."""
import sys

import numpy as np

TOL = 2e-5  # normwise relative error bound for fp32 outputs


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def guarded(torch_mod, n, dtype, pad=256, fill=0x5A):
    """A device buffer with `pad` canary elements on both sides. Returns (full, inner)."""
    full = torch_mod.empty(n + 2 * pad, dtype=dtype, device="cuda")
    full.view(torch_mod.uint8).fill_(fill)
    return full, full[pad:pad + n]


def canary_ok(torch_mod, full, n, pad=256, fill=0x5A):
    b = full.view(torch_mod.uint8)
    isz = full.element_size()
    head = b[: pad * isz]
    tail = b[(pad + n) * isz:]
    return bool((head == fill).all()) and bool((tail == fill).all())
