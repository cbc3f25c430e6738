"""Shared test helpers: moving seeded numpy inputs to the GPU and results back."""
import numpy as np
import torch


def have_gpu() -> bool:
    return torch.cuda.is_available()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def dev_codes(codes: np.ndarray, q: str) -> torch.Tensor:
    """Oracle codes (int8 / E4M3 bytes / bf16 bits) as a device tensor of the matching dtype."""
    if q == "i8":
        return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.int8)).cuda()
    if q == "fp8":
        return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda().view(torch.float8_e4m3fn)
    if q == "bf16":
        return dev_bf16(codes)
    raise ValueError(q)


def host(t: torch.Tensor) -> np.ndarray:
    """Raw host copy: int8 / uint8 bytes / uint16 bf16 bits / float32 / int32."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
