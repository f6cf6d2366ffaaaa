"""Device-side helpers for the GPU parity tests (marshalling only)."""
import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import gemm_tile_granular_bf16_amd as pk
    pk.library()  # raises if the HIP library is missing: no silent fallback
    return pk


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bfloat16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def sample_rows(M: int, n: int, seed: int, must=()):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(int(r) for r in must if 0 <= r < M)
    rows.update(int(r) for r in rng.integers(0, M, size=n))
    return sorted(rows)


def log(msg: str):
    print(msg, flush=True)
