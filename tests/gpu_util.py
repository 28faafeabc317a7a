"""Helpers for the GPU parity tests: move the generators' numpy arrays to the
device as exactly the same bytes, and read results back."""
import sys

import numpy as np
import torch


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Encoded host array (fp32, or bf16 as uint16 bits) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to("cuda")


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def f16_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float16))).to("cuda")


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
