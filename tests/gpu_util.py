"""Helpers of the GPU tests: device buffers from host arrays, the stream
handle, and the comparison metric.  Marshalling only."""
import sys

import numpy as np


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def dev(arr, torch):
    """Host array (uint16 = bf16 bits, float32, int32) -> device tensor."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.cpu().numpy()


def stream(torch):
    return torch.cuda.current_stream().cuda_stream


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    """max |got - ref| / max |ref| (the per-tensor metric of the parity tests)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
