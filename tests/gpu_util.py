"""Helpers for the GPU parity tests (device transfer and the tolerance check)."""
import numpy as np
import torch

# bf16 outputs and gradients: |gpu - oracle| <= ATOL + RTOL * |oracle|, element by element
ATOL, RTOL = 1e-2, 2e-2


def dev_bf16(a):
    """float32 array of exact bf16 values -> cuda bf16 tensor (lossless)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t16 = t.to(torch.bfloat16)
    assert torch.equal(t16.float(), t), "input is not exactly representable in bf16"
    return t16.cuda()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, name="", atol=ATOL, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    msg = (f"{name}: {int(bad.sum())}/{bad.size} outside tolerance, max abs err {err.max():.3g}, "
           f"rel Frobenius err {fro:.3g}")
    print(msg)
    assert not bad.any(), msg
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    return fro
