"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side callers.

This module holds no attention arithmetic: it only draws N(0, 1) numbers from a
seed and stores them as fp32 or as bf16 bit patterns (round-to-nearest-even),
so that both the CPU oracle and the HIP path read the *same stored values*.

Seeding rule: ``numpy.random.default_rng([workload_id, tensor_id, part_id])``
draws ``standard_normal(shape, dtype=float32)``.  Partitions are keyed by their
*global* partition id, so the partition mapper decides which data a GPU uses.
"""
from __future__ import annotations

import numpy as np

# tensor ids used in the seed triple
T_Q, T_K, T_V, T_DO, T_O_IN, T_LSE_IN = 0, 1, 2, 3, 4, 5


def normal_f32(workload_id: int, tensor_id: int, part_id: int, shape) -> np.ndarray:
    """Seeded N(0,1) draw in float32 (C-contiguous)."""
    rng = np.random.default_rng([int(workload_id), int(tensor_id), int(part_id)])
    return rng.standard_normal(tuple(shape), dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(workload_id: int, tensor_id: int, part_id: int, shape):
    """Seeded N(0,1) draw stored as bf16.  Returns (bits uint16, exact values float32)."""
    bits = f32_to_bf16_bits(normal_f32(workload_id, tensor_id, part_id, shape))
    return bits, bf16_bits_to_f32(bits)
