"""Helpers for GPU parity tests: host <-> device transfer of bit patterns and
hand-built scaling records. No method arithmetic here."""
import struct

import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def scale_record(bias: int, flags: int = 0, amax: float = 1.0) -> torch.Tensor:
    """A record with the given bias (scale = 2^bias), built on the host."""
    raw = struct.pack("<fiffIIII", amax, bias, 2.0 ** bias, 2.0 ** -bias, flags, 0, 0, 0) + bytes(32)
    return torch.from_numpy(np.frombuffer(raw, dtype=np.int32).copy()).cuda()


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]
