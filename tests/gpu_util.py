"""Helpers for the GPU parity tests (device buffers, guard bands, tolerances)."""

import sys

import numpy as np
import torch

# Relative Frobenius tolerance for the bf16 contractions, per output tensor.
REL_FRO_TOL = 5e-3

GUARD = 4096          # guard-band bytes on each side of an output buffer
GUARD_BYTE = 0xA5


def say(msg):
    """Name the case before a GPU step, flushed, so a failing run says what it was doing."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")


def guarded(nbytes, dtype):
    """A device buffer of nbytes bytes viewed as dtype, with guard bands of GUARD_BYTE.

    Returns (full uint8 buffer, view).  The view starts GUARD bytes in (keeps
    16-byte alignment)."""
    full = torch.full((nbytes + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=dev())
    view = full[GUARD:GUARD + nbytes].view(dtype)
    return full, view


def guards_intact(full, nbytes):
    torch.cuda.synchronize()
    h = full.cpu().numpy()
    return bool(np.all(h[:GUARD] == GUARD_BYTE) and np.all(h[GUARD + nbytes:] == GUARD_BYTE))


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()
