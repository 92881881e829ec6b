"""Helpers for the GPU parity tests: move seeded numpy inputs to cuda:0 and back,
and read the error word that the library's look-back leaves in its workspace."""
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
    """Error bits of the last call that used the current stream's workspace
    (0 = clean; 1 = a look-back gave up waiting)."""
    torch.cuda.synchronize()
    ws = ps.workspace_for(DEV, torch.cuda.current_stream(DEV), 0)
    return int(ws[4:8].cpu().numpy().view(np.uint32)[0])


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)
