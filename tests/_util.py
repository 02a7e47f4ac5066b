"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

# Layer-output tolerance: relative L2 <= 5e-3 and max |err| <= 3e-2 against
# the oracle's float64 values (fp32 accumulation on the GPU).
REL_L2 = 5e-3
MAX_ABS = 3e-2


def dev(a):
    """numpy -> torch on cuda:0 (fp16 stays fp16, uint8 stays uint8)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.detach().cpu().numpy()


def empty_packed(rows, cols):
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda:0")
    meta = torch.empty((rows, cols // 64, 2), dtype=torch.float16, device="cuda:0")
    return codes, meta


def bits16(a):
    return np.asarray(a).view(np.uint16)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, rel=REL_L2, abs_=MAX_ABS, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(got, ref)
    m = float(np.abs(got - ref).max()) if got.size else 0.0
    assert r <= rel and m <= abs_, f"{what}: rel_l2={r:.3e} (<= {rel}), max_abs={m:.3e} (<= {abs_})"
    return r, m


def log(msg):
    print(msg, flush=True)
