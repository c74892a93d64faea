"""Page reader for tests, written from the page format's description (sections
of 16-byte lane chunks), as reshapes rather than per-element offsets."""
import numpy as np


def _lanes(sec: np.ndarray, per_chunk: int, D: int) -> np.ndarray:
    """Section bytes as elements -> [16][D].  The section is a run of 1 KiB
    blocks; block c holds chunk c of each of 64 lanes; lane (tl * 8 + db)
    holds slots tl and tl + 8, dims [db * B, (db + 1) * B), B = D / 8, slot
    tl first."""
    B = D // 8
    a = sec.reshape(-1, 64, per_chunk)                # [c][lane][e]
    lanes = a.transpose(1, 0, 2).reshape(64, 2 * B)   # [lane][w]
    x = lanes.reshape(8, 8, 2, B)                     # [tl][db][th][dl]
    return x.transpose(2, 0, 1, 3).reshape(16, D)     # [th*8+tl][db*B+dl]


def _wide(sec: np.ndarray, D: int) -> np.ndarray:
    """32*D bytes -> [16][D] uint16."""
    return _lanes(sec.view(np.uint16), 8, D)


def _narrow(sec: np.ndarray, D: int) -> np.ndarray:
    """16*D bytes -> [16][D] int8."""
    return _lanes(sec.view(np.int8), 16, D)


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
