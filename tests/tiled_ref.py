"""numpy statement of the tiled NVFP4 layout documented in include/wq.h
(used only to check the GPU conversion kernels byte for byte)."""
import numpy as np


def tile_ref(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    M, half = codes.shape
    K = 2 * half
    T, S = -(-M // 16), -(-K // 256)
    cp = np.zeros((16 * T, 128 * S), np.uint8)
    cp[:M, :half] = codes
    sp = np.zeros((16 * T, 16 * S), np.uint8)
    sp[:M, :K // 16] = scales
    c4 = cp.reshape(T, 16, S, 128)          # [t][c][s][byte]
    s4 = sp.reshape(T, 16, S, 16)           # [t][c][s][block]
    out = np.zeros((T, S, 2304), np.uint8)
    for h in range(2):
        for g in range(4):
            for j in range(4):
                src = 64 * h + 16 * j + 4 * g
                for c in range(16):
                    dst = 1024 * h + 16 * (c + 16 * g) + 4 * j
                    out[:, :, dst:dst + 4] = c4[:, c, :, src:src + 4]
    for p in range(2):
        for c in range(16):
            for h in range(2):
                for j in range(4):
                    out[:, :, 2048 + 8 * (16 * p + c) + 4 * h + j] = s4[:, c, :, 8 * h + 2 * j + p]
    return out.reshape(-1)


def untile_ref(tiled: np.ndarray, M: int, K: int):
    T, S = -(-M // 16), -(-K // 256)
    b = tiled.reshape(T, S, 2304)
    cp = np.zeros((T, 16, S, 128), np.uint8)
    sp = np.zeros((T, 16, S, 16), np.uint8)
    for h in range(2):
        for g in range(4):
            for j in range(4):
                src = 64 * h + 16 * j + 4 * g
                for c in range(16):
                    dst = 1024 * h + 16 * (c + 16 * g) + 4 * j
                    cp[:, c, :, src:src + 4] = b[:, :, dst:dst + 4]
    for p in range(2):
        for c in range(16):
            for h in range(2):
                for j in range(4):
                    sp[:, c, :, 8 * h + 2 * j + p] = b[:, :, 2048 + 8 * (16 * p + c) + 4 * h + j]
    codes = cp.reshape(16 * T, 128 * S)[:M, :K // 2]
    scales = sp.reshape(16 * T, 16 * S)[:M, :K // 16]
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def fp8_tile_ref(w: np.ndarray) -> np.ndarray:
    """numpy statement of the tiled FP8-row layout documented in include/wq.h."""
    M, K = w.shape
    T, S = -(-M // 16), -(-K // 128)
    wp = np.zeros((16 * T, 128 * S), np.uint8)
    wp[:M, :K] = w
    w4 = wp.reshape(T, 16, S, 128)          # [t][c][s][byte]
    out = np.zeros((T, S, 2048), np.uint8)
    for h in range(2):
        for g in range(4):
            src = 64 * h + 16 * g
            for c in range(16):
                dst = 1024 * h + 16 * (c + 16 * g)
                out[:, :, dst:dst + 16] = w4[:, c, :, src:src + 16]
    return out.reshape(-1)


def fp8_untile_ref(tiled: np.ndarray, M: int, K: int) -> np.ndarray:
    T, S = -(-M // 16), -(-K // 128)
    b = tiled.reshape(T, S, 2048)
    wp = np.zeros((T, 16, S, 128), np.uint8)
    for h in range(2):
        for g in range(4):
            src = 64 * h + 16 * g
            for c in range(16):
                dst = 1024 * h + 16 * (c + 16 * g)
                wp[:, c, :, src:src + 16] = b[:, :, dst:dst + 16]
    return np.ascontiguousarray(wp.reshape(16 * T, 128 * S)[:M, :K])
