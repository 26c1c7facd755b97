"""Helpers for the GPU parity tests: upload seeded host arrays, build table handles."""
import sys

import numpy as np
import torch

import embedding_table_gather_amd as etg


def note(msg: str) -> None:
    """Name the case before a GPU step (so a failing run says which one)."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def table(host: np.ndarray, dtype: int, V: int, d: int) -> etg.Table:
    return etg.Table(to_dev(host), dtype, V, d)


def ids_dev(ids: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


def bits(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
