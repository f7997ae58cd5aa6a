"""The decode-packed NVFP4 weight layout of include/nvfp4.h, written out with
numpy for the tests: for 16-row group g and 128-wide K chunk c, a block of
1152 bytes at (g * K / 128 + c) * 1152 holding 1024 code bytes (byte
16 l + b = code byte 64 c + 16 (l // 16) + b of row 16 g + l % 16) and then
128 scale bytes (byte 8 r + t = scale byte 8 c + t of row 16 g + r); rows
past N are zeros.  ``pack_loops`` spells the definition out element by
element; ``pack`` is the same layout by reshapes, for full-size weights."""
from __future__ import annotations

import numpy as np

BLOCK = 1152


def pack_loops(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    N, K = codes.shape[0], codes.shape[1] * 2
    G, C = (N + 15) // 16, K // 128
    out = np.zeros(G * C * BLOCK, dtype=np.uint8)
    for g in range(G):
        for c in range(C):
            base = (g * C + c) * BLOCK
            for lane in range(64):
                row = 16 * g + lane % 16
                if row < N:
                    src = 64 * c + 16 * (lane // 16)
                    out[base + 16 * lane: base + 16 * lane + 16] = codes[row, src: src + 16]
            for r in range(16):
                row = 16 * g + r
                if row < N:
                    out[base + 1024 + 8 * r: base + 1024 + 8 * r + 8] = scales[row, 8 * c: 8 * c + 8]
    return out


def pack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    N, K = codes.shape[0], codes.shape[1] * 2
    G, C = (N + 15) // 16, K // 128
    cp = np.zeros((G * 16, K // 2), dtype=np.uint8)
    cp[:N] = codes
    sp = np.zeros((G * 16, K // 16), dtype=np.uint8)
    sp[:N] = scales
    # codes: [g, row r, chunk c, quarter q, byte b] -> [g, c, q, r, b] (lane = 16 q + r)
    cb = cp.reshape(G, 16, C, 4, 16).transpose(0, 2, 3, 1, 4).reshape(G, C, 1024)
    # scales: [g, r, c, t] -> [g, c, r, t]
    sb = sp.reshape(G, 16, C, 8).transpose(0, 2, 1, 3).reshape(G, C, 128)
    return np.concatenate([cb, sb], axis=2).reshape(-1)


BF16_BLOCK = 1024


def pack_bf16_loops(w_bits: np.ndarray) -> np.ndarray:
    """BF16 decode-packed layout, element by element: for 16-row group g and
    32-wide K step t, 1 KB at (g * K / 32 + t) * 1024 whose byte 16 l + b is
    byte 16 (l // 16) + b of step t (64 bytes) of row 16 g + l % 16."""
    N, K = w_bits.shape
    rows = w_bits.astype(np.uint16).view(np.uint8).reshape(N, 2 * K)
    G, T = (N + 15) // 16, K // 32
    out = np.zeros(G * T * BF16_BLOCK, dtype=np.uint8)
    for g in range(G):
        for t in range(T):
            base = (g * T + t) * BF16_BLOCK
            for lane in range(64):
                row = 16 * g + lane % 16
                if row < N:
                    src = 64 * t + 16 * (lane // 16)
                    out[base + 16 * lane: base + 16 * lane + 16] = rows[row, src: src + 16]
    return out


def pack_bf16(w_bits: np.ndarray) -> np.ndarray:
    N, K = w_bits.shape
    G, T = (N + 15) // 16, K // 32
    rows = np.zeros((G * 16, 2 * K), dtype=np.uint8)
    rows[:N] = np.ascontiguousarray(w_bits.astype(np.uint16)).view(np.uint8).reshape(N, 2 * K)
    # [g, row r, step t, quarter q, byte b] -> [g, t, q, r, b]
    return rows.reshape(G, 16, T, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
