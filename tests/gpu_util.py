"""Helpers for the GPU parity tests: move seeded numpy inputs to cuda:0 and back,
and read the error word that the library's bounded waits leave in its workspace."""
import numpy as np
import torch

import prefix_scan_stream_amd as ps

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ws_error_word() -> int:
    """Error bits of the current stream's cached workspace, read through the C ABI
    (ls_workspace_check): 0 when no call on it gave up a bounded wait."""
    return ps.workspace_error_flags(DEV)


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)
