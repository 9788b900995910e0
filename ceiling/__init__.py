"""Empirical streaming ceilings for the SwiGLU access patterns (measurement only).

bench.py runs these zero-arithmetic kernels beside the SwiGLU kernels:
 * `launch`: the row-packed patterns, same grid and lane mapping as the wide
   SwiGLU kernels (how much time the arithmetic adds);
 * `probe`: kernels of other structures over separate flat streams (one-shot
   grids of 256 or 1024 lanes, a persistent grid-stride loop with four
   vectors per lane in flight, block-contiguous chunks), for the forward and
   backward mixes and for read-only, write-only and copy traffic. The best of
   them is a ceiling that the SwiGLU kernels' own design does not set.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_ceiling.hip")
LIB = os.path.join(HERE, "libstream_ceiling.so")

STRUCTURES = {0: "one-shot, 256 lanes", 1: "one-shot, 1024 lanes",
              2: "grid-stride, 4 vectors in flight, 8 blocks per CU",
              3: "block-contiguous chunks, 4 blocks per CU"}
MIXES = {"fwd": 0, "bwd": 1, "read": 2, "write": 3, "copy": 4}
# streams each mix reads and writes (vectors of 16 bytes, nvec each)
MIX_STREAMS = {"fwd": (2, 1), "bwd": (3, 2), "read": (1, 0), "write": (0, 1), "copy": (1, 1)}
# Offset between consecutive flat streams carved from one allocation: 4 KiB,
# so that the streams do not start on the same memory channel.
SKEW_BYTES = 4096

_lib = None


def build(verbose: bool = False) -> str:
    from swiglu_activation_amd.build import hipcc
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed: {res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        lib.stream_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p]
        lib.stream_ceiling_launch.restype = ctypes.c_int
        lib.stream_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p]
        lib.stream_probe_launch.restype = ctypes.c_int
        _lib = lib
    return _lib


def launch(pattern: int, x, dy, out, rows: int, nv16: int, stream) -> None:
    """pattern 0: x -> out (forward mix); 1: x, dy -> out (backward mix).
    nv16 = 16-byte vectors per half row. Tensors are torch device tensors."""
    need_x = rows * 2 * nv16 * 16
    need_o = rows * (nv16 if pattern == 0 else 2 * nv16) * 16
    if x.numel() * x.element_size() < need_x or out.numel() * out.element_size() < need_o:
        raise ValueError("buffers too small for the ceiling pattern")
    if pattern == 1 and dy.numel() * dy.element_size() < rows * nv16 * 16:
        raise ValueError("dy too small for the ceiling pattern")
    rc = load().stream_ceiling_launch(pattern, x.data_ptr(), dy.data_ptr() if dy is not None else None,
                                      out.data_ptr(), rows, nv16, ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"stream_ceiling_launch returned {rc}")


class FlatStreams:
    """Five flat streams (three read, two written) of nvec 16-byte vectors,
    carved from one device allocation, SKEW_BYTES apart beyond their length."""

    def __init__(self, nvec: int, device):
        import torch
        self.nvec = nvec
        step = nvec * 16 + SKEW_BYTES
        self.buf = torch.ones(5 * step // 4, dtype=torch.int32, device=device)
        base = self.buf.data_ptr()
        self.ptrs = [base + i * step for i in range(5)]


def probe(structure: int, mix: str, fs: FlatStreams, stream=None, cached: bool = False) -> None:
    """Launch one independent-structure kernel on the flat streams, on
    `stream` (default: torch's current stream at the time of the call, which
    is the capturing stream inside a graph capture)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    r0, r1, r2, w0, w1 = fs.ptrs
    rc = load().stream_probe_launch(structure, MIXES[mix], int(cached), r0, r1, r2, w0, w1,
                                    fs.nvec, ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"stream_probe_launch returned {rc}")


def mix_bytes(mix: str, nvec: int) -> int:
    r, w = MIX_STREAMS[mix]
    return (r + w) * nvec * 16
