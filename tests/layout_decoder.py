"""Pure-Python reader of the packed layer blob, written from the layout as the
header documents it (include/nq.h, csrc/nq_common.h).  Used to check that what
the pack kernels write is exactly the documented format."""
from __future__ import annotations

import struct

import numpy as np


def _up(v, a=256):
    return (v + a - 1) // a * a


def _tiles(R, C):
    return (R + 15) // 16, (C + 127) // 128


def decode_header(blob: bytes) -> dict:
    magic, version, m, n, r, sdt, bad, _ = struct.unpack_from("<IIiiiiii", blob, 0)
    offs = struct.unpack_from("<6Q", blob, 32)
    return dict(magic=magic, version=version, m=m, n=n, r=r, scale_dtype=sdt, bad=bad,
                off_u=offs[0], off_vt=offs[1], off_s1=offs[2], off_g=offs[3], off_s2=offs[4], total=offs[5])


def decode_signs(words: np.ndarray, R: int, C: int) -> np.ndarray:
    """int8 +-1 matrix (R x C) from the tile-layout words of one sign matrix."""
    RT, KT = _tiles(R, C)
    out = np.zeros((RT * 16, KT * 128), np.int8)
    lane = np.arange(64)
    for rt in range(RT):
        for kt in range(KT):
            q = kt // 4
            f = min(4, KT - 4 * q)
            idx = rt * KT * 64 + q * 256 + lane * f + (kt % 4)
            w = words[idx].astype(np.uint64)
            for b in range(32):
                col = kt * 128 + 32 * (lane >> 4) + 8 * (b % 4) + (b // 4)
                row = rt * 16 + (lane & 15)
                out[row, col] = np.where((w >> np.uint64(b)) & np.uint64(1), 1, -1)
    return out[:R, :C]


def decode_blob(blob: bytes):
    h = decode_header(blob)
    m, n, r = h["m"], h["n"], h["r"]
    sb = 4 if h["scale_dtype"] == 0 else 2
    sdt = np.float32 if sb == 4 else np.float16
    assert h["off_u"] == 256
    RT, KT = _tiles(m, r)
    assert h["off_vt"] == _up(256 + RT * KT * 256)
    RT2, KT2 = _tiles(r, n)
    assert h["off_s1"] == _up(h["off_vt"] + RT2 * KT2 * 256)
    words = np.frombuffer(blob, np.uint32)
    U = decode_signs(words[h["off_u"] // 4:h["off_vt"] // 4], m, r)
    Vt = decode_signs(words[h["off_vt"] // 4:h["off_s1"] // 4], r, n)
    s1 = np.frombuffer(blob, sdt, m, h["off_s1"])
    g = np.frombuffer(blob, sdt, r, h["off_g"])
    s2 = np.frombuffer(blob, sdt, n, h["off_s2"])
    return h, U, Vt.T.copy(), s1, g, s2
