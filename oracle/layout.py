"""Reference packer / unpacker for the library's packed layout, version 1.

Oracle; test infrastructure.  Written from the layout text only (the C header
states the same layout in prose); it shares no code with the HIP packer.
The pages name the formats but give no bit layout; the layout is the
library's own.  Packing is integer bit-placement only: values are unchanged.

One packed matrix is a sequence of planes.  Each plane starts at an offset
that is a multiple of 256 bytes (plane sizes are rounded up to 256), and a
stack of `batch` matrices places matrix i at i * (packed bytes of one).
All multi-byte fields are little-endian.

  q8_0       plane qs    N*K bytes      byte n*K + k = q[n][k] (two's complement)
             plane scale N*(K/32) f16   element n*(K/32) + b = scale[n][b]
  w4a16_g64  plane qs    N*K/2 bytes    byte n*K/2 + j = q[n][2j] | q[n][2j+1] << 4
             plane sz    N*(K/64) u32   word n*K/64 + g = scale[n][g] | zero[n][g] << 16
  q4k        plane qs    as w4a16_g64
             plane meta  N*(K/256) 16-byte records, record (n, t):
                         bytes 0-1 d[n][t], bytes 2-3 dmin[n][t], bytes 4..15 a 96-bit
                         little-endian integer V with sc[n][8t+j] at bits 6j..6j+5 and
                         m[n][8t+j] at bits 48+6j..48+6j+5 (j = 0..7)
  q6k        plane ql    N*K/2 bytes    low 4 bits of q, nibble order as w4a16_g64
             plane qh    N*(K/16) u32   word (n, t) covers k = 16t..16t+15; its bits
                         8c+2f..8c+2f+1 (c, f = 0..3) hold bits 4-5 of
                         q[n][16t + 8*(f >> 1) + 2c + (f & 1)]
             plane s     N*(K/16) int8  s[n][j]
             plane d     N*(K/256) f16  d[n][t]
  q4_0       plane qs    as w4a16_g64
             plane d     N*(K/32) f16   element n*(K/32) + b = d[n][b]
  q5_0       plane qs    as w4a16_g64 (low 4 bits of q)
             plane qh    N*(K/32) u32   word (n, u) covers k = 32u..32u+31; its bit
                         8c + 2i + e (c, i = 0..3, e = 0..1) holds bit 4 of
                         q[n][32u + 8i + 2c + e]
             plane d     as q4_0
  q5k        plane qs    as w4a16_g64 (low 4 bits of q)
             plane qh    as q5_0
             plane meta  as q4k
  bf16       plane w     N*K bf16       element n*K + k = q[n][k]
  i8row      plane qs    N*K bytes      byte n*K + k = q[n][k] (two's complement)
             plane scale N f32          element n = scale[n]

Fields are masked to their width (4 bits for nibbles, 5 bits for q5 codes,
6 bits for sc/m/q6).
"""
from __future__ import annotations

import numpy as np

BLOCK = {"q8_0": 32, "w4a16_g64": 64, "q4k": 256, "q6k": 256, "q4_0": 32, "q5_0": 32, "q5k": 256,
         "bf16": 32, "i8row": 32}
ALIGN = 256


def _planes(fmt: str, N: int, K: int):
    """(name, bytes) of each plane of one matrix, in order."""
    if fmt == "q8_0":
        return [("qs", N * K), ("scale", N * (K // 32) * 2)]
    if fmt == "w4a16_g64":
        return [("qs", N * K // 2), ("sz", N * (K // 64) * 4)]
    if fmt == "q4k":
        return [("qs", N * K // 2), ("meta", N * (K // 256) * 16)]
    if fmt == "q6k":
        return [("ql", N * K // 2), ("qh", N * (K // 16) * 4), ("s", N * (K // 16)),
                ("d", N * (K // 256) * 2)]
    if fmt == "q4_0":
        return [("qs", N * K // 2), ("d", N * (K // 32) * 2)]
    if fmt == "q5_0":
        return [("qs", N * K // 2), ("qh", N * (K // 32) * 4), ("d", N * (K // 32) * 2)]
    if fmt == "q5k":
        return [("qs", N * K // 2), ("qh", N * (K // 32) * 4), ("meta", N * (K // 256) * 16)]
    if fmt == "bf16":
        return [("w", N * K * 2)]
    if fmt == "i8row":
        return [("qs", N * K), ("scale", N * 4)]
    raise ValueError(f"unknown format {fmt!r}")


def _round_up(v: int, a: int = ALIGN) -> int:
    return (v + a - 1) // a * a


def plane_offsets(fmt: str, N: int, K: int) -> dict:
    off, out = 0, {}
    for name, nb in _planes(fmt, N, K):
        out[name] = (off, nb)
        off += _round_up(nb)
    return out


def packed_bytes_ref(fmt: str, N: int, K: int, batch: int = 1) -> int:
    if K % BLOCK[fmt]:
        raise ValueError("K must be a multiple of the block size")
    return batch * sum(_round_up(nb) for _, nb in _planes(fmt, N, K))


def _nibbles(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8) & 0xF
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _unnibbles(b: np.ndarray, N: int, K: int) -> np.ndarray:
    b = b.reshape(N, K // 2)
    q = np.empty((N, K), dtype=np.uint8)
    q[:, 0::2] = b & 0xF
    q[:, 1::2] = b >> 4
    return q


def _f16_bytes(bits) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.uint8).ravel()


def _qh_words(q: np.ndarray) -> np.ndarray:
    """The qh plane of q6k: [N][K/16] uint32 from 6-bit q [N][K]."""
    N, K = q.shape
    hi = ((np.asarray(q, dtype=np.uint8) >> 4) & 3).astype(np.uint32).reshape(N, K // 16, 16)
    w = np.zeros((N, K // 16), dtype=np.uint32)
    for c in range(4):
        for f in range(4):
            k = 8 * (f >> 1) + 2 * c + (f & 1)
            w |= hi[:, :, k] << np.uint32(8 * c + 2 * f)
    return w


def _qh_unwords(w: np.ndarray, N: int, K: int) -> np.ndarray:
    w = w.reshape(N, K // 16).astype(np.uint32)
    hi = np.zeros((N, K // 16, 16), dtype=np.uint8)
    for c in range(4):
        for f in range(4):
            k = 8 * (f >> 1) + 2 * c + (f & 1)
            hi[:, :, k] = (w >> np.uint32(8 * c + 2 * f)) & 3
    return hi.reshape(N, K)


def _q5_hwords(q: np.ndarray) -> np.ndarray:
    """The qh plane of q5_0 / q5k: [N][K/32] uint32 from 5-bit q [N][K]."""
    N, K = q.shape
    hi = ((np.asarray(q, dtype=np.uint8) >> 4) & 1).astype(np.uint32).reshape(N, K // 32, 32)
    w = np.zeros((N, K // 32), dtype=np.uint32)
    for i in range(4):
        for c in range(4):
            for e in range(2):
                w |= hi[:, :, 8 * i + 2 * c + e] << np.uint32(8 * c + 2 * i + e)
    return w


def _q5_unhwords(w: np.ndarray, N: int, K: int) -> np.ndarray:
    w = w.reshape(N, K // 32).astype(np.uint32)
    hi = np.zeros((N, K // 32, 32), dtype=np.uint8)
    for i in range(4):
        for c in range(4):
            for e in range(2):
                hi[:, :, 8 * i + 2 * c + e] = (w >> np.uint32(8 * c + 2 * i + e)) & 1
    return hi.reshape(N, K)


def _q4k_meta(sc, m, d, dmin) -> np.ndarray:
    """[N][K/256][16] bytes of q4k meta records."""
    N, nsb = np.asarray(d).shape
    sc = (np.asarray(sc, dtype=np.uint8) & 0x3F).reshape(N, nsb, 8)
    m = (np.asarray(m, dtype=np.uint8) & 0x3F).reshape(N, nsb, 8)
    rec = np.zeros((N, nsb, 16), dtype=np.uint8)
    rec[:, :, 0:2] = np.asarray(d, dtype=np.uint16).reshape(N, nsb, 1).view(np.uint8)
    rec[:, :, 2:4] = np.asarray(dmin, dtype=np.uint16).reshape(N, nsb, 1).view(np.uint8)
    # build V bit by bit: 16 six-bit fields -> 96 bits -> 12 bytes
    fields = np.concatenate([sc, m], axis=2).astype(np.uint64)  # field i at bit 6i
    for i in range(16):
        for bit in range(6):
            pos = 6 * i + bit
            rec[:, :, 4 + pos // 8] |= (((fields[:, :, i] >> np.uint64(bit)) & 1) << np.uint64(pos % 8)).astype(np.uint8)
    return rec


def _q4k_unmeta(rec: np.ndarray):
    N, nsb, _ = rec.shape
    d = np.ascontiguousarray(rec[:, :, 0:2]).view(np.uint16).reshape(N, nsb)
    dmin = np.ascontiguousarray(rec[:, :, 2:4]).view(np.uint16).reshape(N, nsb)
    fields = np.zeros((N, nsb, 16), dtype=np.uint8)
    for i in range(16):
        for bit in range(6):
            pos = 6 * i + bit
            fields[:, :, i] |= ((rec[:, :, 4 + pos // 8] >> (pos % 8)) & 1) << bit
    sc = fields[:, :, :8].reshape(N, nsb * 8)
    m = fields[:, :, 8:].reshape(N, nsb * 8)
    return sc, m, d, dmin


def pack_ref(fmt: str, w: dict) -> np.ndarray:
    """Packed bytes (uint8 array of packed_bytes_ref) of one matrix."""
    q = np.asarray(w["q"])
    N, K = q.shape
    out = np.zeros(packed_bytes_ref(fmt, N, K), dtype=np.uint8)
    po = plane_offsets(fmt, N, K)

    def put(name, data):
        off, nb = po[name]
        data = np.ascontiguousarray(data).view(np.uint8).ravel()
        assert data.size == nb, (name, data.size, nb)
        out[off:off + nb] = data

    if fmt == "q8_0":
        put("qs", np.asarray(q, dtype=np.int8))
        put("scale", _f16_bytes(w["scale"]))
    elif fmt == "w4a16_g64":
        put("qs", _nibbles(q))
        sz = np.asarray(w["scale"], dtype=np.uint32) | (np.asarray(w["zero"], dtype=np.uint32) << 16)
        put("sz", sz.astype(np.uint32))
    elif fmt == "q4k":
        put("qs", _nibbles(q))
        put("meta", _q4k_meta(w["sc"], w["m"], w["d"], w["dmin"]))
    elif fmt == "q6k":
        q6 = np.asarray(q, dtype=np.uint8) & 0x3F
        put("ql", _nibbles(q6 & 0xF))
        put("qh", _qh_words(q6))
        put("s", np.asarray(w["s"], dtype=np.int8))
        put("d", _f16_bytes(w["d"]))
    elif fmt == "q4_0":
        put("qs", _nibbles(q))
        put("d", _f16_bytes(w["d"]))
    elif fmt in ("q5_0", "q5k"):
        q5 = np.asarray(q, dtype=np.uint8) & 0x1F
        put("qs", _nibbles(q5 & 0xF))
        put("qh", _q5_hwords(q5))
        if fmt == "q5_0":
            put("d", _f16_bytes(w["d"]))
        else:
            put("meta", _q4k_meta(w["sc"], w["m"], w["d"], w["dmin"]))
    elif fmt == "bf16":
        put("w", _f16_bytes(q))
    elif fmt == "i8row":
        put("qs", np.asarray(q, dtype=np.int8))
        put("scale", np.asarray(w["scale"], dtype=np.float32))
    else:
        raise ValueError(fmt)
    return out


def unpack_ref(fmt: str, N: int, K: int, buf) -> dict:
    """Logical arrays of one packed matrix (inverse of pack_ref up to field masking)."""
    buf = np.asarray(buf, dtype=np.uint8).ravel()
    po = plane_offsets(fmt, N, K)

    def get(name):
        off, nb = po[name]
        return buf[off:off + nb]

    if fmt == "q8_0":
        return {"q": get("qs").view(np.int8).reshape(N, K).copy(),
                "scale": get("scale").view(np.uint16).reshape(N, K // 32).copy()}
    if fmt == "w4a16_g64":
        sz = get("sz").view(np.uint32).reshape(N, K // 64)
        return {"q": _unnibbles(get("qs"), N, K),
                "scale": (sz & 0xFFFF).astype(np.uint16), "zero": (sz >> 16).astype(np.uint16)}
    if fmt == "q4k":
        sc, m, d, dmin = _q4k_unmeta(get("meta").reshape(N, K // 256, 16))
        return {"q": _unnibbles(get("qs"), N, K), "sc": sc, "m": m, "d": d, "dmin": dmin}
    if fmt == "q6k":
        lo = _unnibbles(get("ql"), N, K)
        hi = _qh_unwords(get("qh").view(np.uint32), N, K)
        return {"q": (lo | (hi << 4)).astype(np.uint8),
                "s": get("s").view(np.int8).reshape(N, K // 16).copy(),
                "d": get("d").view(np.uint16).reshape(N, K // 256).copy()}
    if fmt == "q4_0":
        return {"q": _unnibbles(get("qs"), N, K), "d": get("d").view(np.uint16).reshape(N, K // 32).copy()}
    if fmt in ("q5_0", "q5k"):
        q = (_unnibbles(get("qs"), N, K) | (_q5_unhwords(get("qh").view(np.uint32), N, K) << 4)).astype(np.uint8)
        if fmt == "q5_0":
            return {"q": q, "d": get("d").view(np.uint16).reshape(N, K // 32).copy()}
        sc, m, d, dmin = _q4k_unmeta(get("meta").reshape(N, K // 256, 16))
        return {"q": q, "sc": sc, "m": m, "d": d, "dmin": dmin}
    if fmt == "bf16":
        return {"q": get("w").view(np.uint16).reshape(N, K).copy()}
    if fmt == "i8row":
        return {"q": get("qs").view(np.int8).reshape(N, K).copy(),
                "scale": get("scale").view(np.float32).reshape(N).copy()}
    raise ValueError(fmt)
