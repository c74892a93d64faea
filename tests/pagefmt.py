"""Page reader for tests, written from the page format's description (sections
of 16-byte chunks), as reshapes rather than per-element offsets."""
import numpy as np


def _wide(sec: np.ndarray, D: int) -> np.ndarray:
    """32*D bytes -> [16][D] uint16 (chunk index = i*64 + quarter*16 + token)."""
    L = D // 4
    a = sec.view(np.uint16).reshape(L // 8, 4, 16, 8)
    return a.transpose(2, 1, 0, 3).reshape(16, D)


def _narrow(sec: np.ndarray, D: int) -> np.ndarray:
    L = D // 4
    a = sec.view(np.int8).reshape(L // 16, 4, 16, 16)
    return a.transpose(2, 1, 0, 3).reshape(16, D)


def read_page(page: np.ndarray, D: int, tier: int) -> dict:
    G = D // 8
    out = {}
    if tier in (0, 3):
        out["K"] = _wide(page[: 32 * D], D)
        out["V"] = _wide(page[32 * D: 64 * D], D)
        used = 64 * D
    elif tier == 1:
        out["V"] = _wide(page[: 32 * D], D)
        o = 32 * D
        out["codes"] = page[o: o + 16 * G].reshape(16, G)
        out["radius"] = page[o + 16 * G: o + 16 * G + 32].view(np.uint16)
        used = o + 16 * G + 32
    else:
        out["Vq"] = _narrow(page[: 16 * D], D)
        o = 16 * D
        out["codes4"] = page[o: o + 8 * G].reshape(16, G // 2)
        out["radius"] = page[o + 8 * G: o + 8 * G + 32].view(np.uint16)
        out["vscale"] = page[o + 8 * G + 32: o + 8 * G + 64].view(np.uint16)
        used = o + 8 * G + 64
    out["pad"] = page[used:]
    return out
