"""Exact upcasts of the stored input formats to float64 (oracle; test infrastructure).

The oracle reads the same stored bits the GPU reads and converts them to float64
exactly, so a comparison measures the kernel's arithmetic, not input rounding.

* bfloat16 is the upper 16 bits of an IEEE binary32; widening is a shift.
* float16 is IEEE binary16, which numpy represents natively.
* fp8 "e4m3" (named as a KV-cache precision in "Ask, Don't Equip", section
  研究动机) is read as the OCP E4M3 format: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448 and exponent field 0 encodes the
  subnormals m/8 * 2^-6. The table below is built from that definition.
"""
from __future__ import annotations

import math

import numpy as np


def default_scale(head_dim: int) -> float:
    """1/sqrt(D) rounded once to binary32, as the library's default scale."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_code_table() -> np.ndarray:
    return _E4M3.copy()


def e4m3_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes).astype(np.uint8)]


def tensor_to_f64(t, dtype: str) -> np.ndarray:
    """Widen a CPU torch tensor (or numpy array) holding ``dtype`` values to float64.

    The tensor's bits are reinterpreted as unsigned integers before widening, so
    no torch arithmetic is involved.
    """
    import torch  # local: the oracle's arithmetic is numpy; torch only exposes the bits
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if dtype == "f32":
            return t.numpy().astype(np.float64)
        if dtype == "f64":
            return t.numpy().copy()
        if dtype in ("bf16", "f16"):
            bits = t.view(torch.int16).numpy().view(np.uint16)
        elif dtype == "fp8_e4m3":
            bits = t.view(torch.uint8).numpy()
        else:
            raise ValueError(dtype)
    else:
        bits = np.asarray(t)
        if dtype in ("f32", "f64"):
            return bits.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "fp8_e4m3":
        return e4m3_codes_to_f64(bits)
    raise ValueError(dtype)
