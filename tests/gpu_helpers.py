"""Shared helpers of the GPU parity tests: metrics and host<->device moves.
The metrics are the ones the parity bar is stated in."""
import json
import os

import numpy as np


def rel_frobenius(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want.ravel())
    return float(np.linalg.norm((got - want).ravel()) / (den if den > 0 else 1.0))


def rel_inf(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def to_dev_bf16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).ravel()).view(
        torch.bfloat16).cuda()


def to_dev_f32(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32).ravel()).cuda()


def bf16_bits(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_host(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def to_dev_f16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).ravel()).view(
        torch.float16).cuda()


def record(test: str, **values):
    """Append one JSON line of measured parity figures to the file named by
    JA_PARITY_RECORD (nothing when it is unset), so that a GPU run keeps the
    errors it measured and not only whether they passed."""
    path = os.environ.get("JA_PARITY_RECORD")
    if not path:
        return
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(dict(test=test, **values), sort_keys=True) + "\n")
