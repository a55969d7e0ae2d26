"""Independent helpers for the tests: library conversions (numpy / torch), not the oracle's code."""
import numpy as np
import torch


def f32_of(bits: np.ndarray, dt: str) -> np.ndarray:
    """16-bit patterns -> float32 via numpy (fp16) or torch (bf16)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dt == "fp16":
        return b.view(np.float16).astype(np.float32)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()


def bits_of(f: np.ndarray, dt: str) -> np.ndarray:
    """float32/float64 -> 16-bit patterns, round to nearest even, via numpy (fp16) or torch (bf16)."""
    if dt == "fp16":
        return np.ascontiguousarray(np.asarray(f).astype(np.float16)).view(np.uint16)
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(f, dtype=np.float32))).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def ulp16(v: np.ndarray, dt: str) -> np.ndarray:
    """Spacing of the 16-bit format at |v| (float64)."""
    mant = 10 if dt == "fp16" else 7
    emin = -14 if dt == "fp16" else -126
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - mant)
