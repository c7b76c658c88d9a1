"""The layer's persistent state on disk: the expert bias b [N_r] (fp32) and the step counter.

The bias is the only state the auxiliary-loss-free balancing carries from step to step ("DeepSeek_V3_Report:
Annotation", section on auxiliary-loss-free load balancing: b_i moves by the update speed after every step
and is used for the routing only); the step counter says how many updates produced it. File layout, little
endian: 8-byte magic b"MOEBIAS\\0", uint32 format version (1), uint32 N_r, uint64 step, then N_r float32
values as the device holds them (raw bits, so a reload is bit-exact).
"""
from __future__ import annotations

import struct

import numpy as np

MAGIC = b"MOEBIAS\0"
VERSION = 1
_HEADER = struct.Struct("<8sIIQ")


def save_bias_state(path: str, bias: np.ndarray, step: int) -> None:
    """Write b (any float32 array of N_r values) and the step counter to path."""
    b = np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
    if step < 0:
        raise ValueError("step must be >= 0")
    with open(path, "wb") as f:
        f.write(_HEADER.pack(MAGIC, VERSION, b.size, int(step)))
        f.write(b.astype("<f4").tobytes())


def load_bias_state(path: str, n_routed: int | None = None):
    """(b as float32 [N_r], step) from path; raises ValueError on a foreign, truncated or mismatched file."""
    with open(path, "rb") as f:
        head = f.read(_HEADER.size)
        if len(head) != _HEADER.size:
            raise ValueError(f"{path}: truncated header")
        magic, version, n, step = _HEADER.unpack(head)
        if magic != MAGIC:
            raise ValueError(f"{path}: not a bias state file")
        if version != VERSION:
            raise ValueError(f"{path}: format version {version}, expected {VERSION}")
        if n_routed is not None and n != n_routed:
            raise ValueError(f"{path}: holds {n} expert biases, the layer has {n_routed}")
        body = f.read()
    if len(body) != 4 * n:
        raise ValueError(f"{path}: {len(body)} bytes of bias, expected {4 * n}")
    return np.frombuffer(body, dtype="<f4").astype(np.float32), int(step)
