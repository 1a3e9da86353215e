"""Small array helpers shared by the tests (no method arithmetic here)."""

import numpy as np
import torch


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns as a numpy array."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32)


def f32_to_bf16_torch(f: np.ndarray) -> np.ndarray:
    """torch's own fp32 -> bf16 cast (round to nearest even), as bit patterns."""
    return bf16_bits(torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to(torch.bfloat16))


def bf16_ulp_distance(a_u16: np.ndarray, b_u16: np.ndarray) -> np.ndarray:
    """Distance in units of last place between two bf16 arrays (+0 == -0)."""
    def ordered(u):
        u = np.asarray(u, dtype=np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(ordered(a_u16) - ordered(b_u16))


def load_golden(name: str) -> dict:
    """A text fixture under tests/golden/: "key: values" lines, '#' comments,
    matrix rows separated by '|'.  Integers stay integers; any value with a
    '.' makes its array float."""
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            rows = [r.split() for r in val.split("|")]
            is_float = any("." in v for r in rows for v in r)
            arr = np.array([[float(v) if is_float else int(v) for v in r] for r in rows])
            out[key] = arr[0] if len(rows) == 1 else arr
            if arr.size == 1 and len(rows) == 1:
                out[key] = arr.reshape(-1)[0].item()
    return out
