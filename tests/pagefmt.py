"""Page reader for tests, written from the page format's description (sections
of 16-byte lane chunks), as reshapes rather than per-element offsets."""
import numpy as np


def _rows(sec: np.ndarray, D: int) -> np.ndarray:
    """Row section (2-byte elements) -> [16][D]: byte chunks [c][lane][half][e]
    with lane = t + 16 q holding dims 16 b + 4 q + e of block b = 2 c + half."""
    a = sec.view(np.uint16).reshape(D // 32, 4, 16, 2, 4)     # [c][q][t][half][e]
    return a.transpose(2, 0, 3, 1, 4).reshape(16, D)           # [t][c][half][q][e]


def _cols(sec: np.ndarray, D: int) -> np.ndarray:
    """Column section (2-byte elements) -> [16][D]: lane = n + 16 r holds slots
    4 r + e of dim 16 b + n."""
    a = sec.view(np.uint16).reshape(D // 32, 4, 16, 2, 4)     # [c][r][n][half][e]
    return a.transpose(1, 4, 0, 3, 2).reshape(16, D)           # [r][e][c][half][n]


def _cols8(sec: np.ndarray, D: int) -> np.ndarray:
    """int8 column section -> [16][D]: 4 bytes per lane and block, 4 blocks
    per 16-byte chunk."""
    a = sec.view(np.int8).reshape(D // 64, 4, 16, 4, 4)       # [c][r][n][b4][e]
    return a.transpose(1, 4, 0, 3, 2).reshape(16, D)           # [r][e][c][b4][n]


def read_page(page: np.ndarray, D: int, tier: int) -> dict:
    G = D // 8
    out = {}
    if tier in (0, 3):
        out["K"] = _rows(page[: 32 * D], D)
        out["V"] = _cols(page[32 * D: 64 * D], D)
        used = 64 * D
    elif tier == 1:
        out["V"] = _cols(page[: 32 * D], D)
        o = 32 * D
        out["codes"] = page[o: o + 16 * G].reshape(16, G)
        out["radius"] = page[o + 16 * G: o + 16 * G + 32].view(np.uint16)
        used = o + 16 * G + 32
    else:
        out["Vq"] = _cols8(page[: 16 * D], D)
        o = 16 * D
        out["codes4"] = page[o: o + 8 * G].reshape(16, G // 2)
        out["radius"] = page[o + 8 * G: o + 8 * G + 32].view(np.uint16)
        out["vscale"] = page[o + 8 * G + 32: o + 8 * G + 64].view(np.uint16)
        used = o + 8 * G + 64
    out["pad"] = page[used:]
    return out
