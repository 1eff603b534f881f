"""Helpers for the GPU tests: numpy <-> torch device buffers (BF16 carried as
uint16 bit patterns on the host), guarded allocations."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_like_np(count: int, np_dtype) -> torch.Tensor:
    if np_dtype == np.uint16:
        return torch.empty(count, dtype=torch.bfloat16, device=DEV)
    if np_dtype == np.uint8:
        return torch.empty(count, dtype=torch.uint8, device=DEV)
    return torch.empty(count, dtype=torch.float32, device=DEV)


class Guarded:
    """A device buffer of `count` elements with `pad` sentinel elements on
    both sides (pad keeps the 16-byte alignment)."""

    def __init__(self, count: int, torch_dtype, pad: int = 64, sentinel=None):
        self.count, self.pad = count, pad
        self.full = torch.empty(count + 2 * pad, dtype=torch_dtype, device=DEV)
        if torch_dtype == torch.bfloat16:
            self.full.view(torch.int16).fill_(0x7FA5)       # a NaN pattern
        elif torch_dtype == torch.uint8:
            self.full.fill_(0xA5 if sentinel is None else sentinel)
        else:
            self.full.view(torch.int32).fill_(0x7FA5A5A5)   # a NaN pattern
        self.before = self.full[:pad].clone()
        self.after = self.full[pad + count:].clone()
        self.t = self.full[pad:pad + count]

    def guards_intact(self) -> bool:
        def same(a, b):
            if a.dtype == torch.bfloat16:
                return torch.equal(a.view(torch.int16), b.view(torch.int16))
            if a.dtype == torch.float32:
                return torch.equal(a.view(torch.int32), b.view(torch.int32))
            return torch.equal(a, b)
        return same(self.full[:self.pad], self.before) and \
            same(self.full[self.pad + self.count:], self.after)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    if a.dtype == np.float32:
        a = a.view(np.uint32)
    if b.dtype == np.float32:
        b = b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    av = a.view(np.uint32) if a.dtype == np.float32 else a
    bv = b.view(np.uint32) if b.dtype == np.float32 else b
    idx = np.nonzero(av != bv)[0]
    if idx.size == 0:
        return "no mismatch"
    i = idx[0]
    return f"{idx.size} mismatches, first at {i}: got {a[i]!r} want {b[i]!r}"
