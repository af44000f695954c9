"""Small helpers for the GPU parity tests (device copies, workspace)."""
import numpy as np


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def workspace(q4k, m, hidden, inter, top_k=0, regime=0):
    import torch
    nbytes = q4k.ffn_swiglu_q4k_workspace_bytes(m, hidden, inter, top_k, regime)
    assert nbytes > 0
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


def say(*args):
    print(*args, flush=True)
