"""Helpers for the GPU tests: numpy <-> device tensors and bitwise comparison."""
import numpy as np
import torch


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 (bf16 bits) / float32 / uint8 -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str, block_bytes: int = 0):
    g = np.ascontiguousarray(got).view(np.uint8).reshape(-1)
    w = np.ascontiguousarray(want).view(np.uint8).reshape(-1)
    assert g.size == w.size, f"{what}: size {g.size} != {w.size}"
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = int(bad[0])
        msg = f"{what}: {bad.size} bytes differ; first at byte {i}: got {g[i]:#04x} want {w[i]:#04x}"
        if block_bytes:
            b = i // block_bytes
            msg += (f" (block {b}: got {g[b*block_bytes:(b+1)*block_bytes].tobytes().hex()} "
                    f"want {w[b*block_bytes:(b+1)*block_bytes].tobytes().hex()})")
        raise AssertionError(msg)
