"""Shared test plumbing: moving seeded inputs to the GPU and back."""
import numpy as np


def to_dev(a: np.ndarray, dtype: str = "f32", device="cuda"):
    """numpy -> torch on device; bf16 arrays arrive as uint16 bits."""
    import torch
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.uint64:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_np64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def attn_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Attention parity bar: bf16 max-abs <= 2e-2 and rel-L2 <= 1e-2;
    fp32 both <= 1e-5."""
    tol_abs, tol_rel = (2e-2, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if err.size else 0.0
    assert mx <= tol_abs and rel <= tol_rel, f"{what}: max-abs {mx:.3g}, rel-L2 {rel:.3g}"
    return mx, rel
