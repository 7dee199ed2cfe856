"""Host <-> device helpers for the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import weight_only_int4_group_amd as q4


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an AMD GPU (torch.cuda.is_available() is False)")
    q4.library()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(arr: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def log(msg: str):
    print(msg, flush=True)
