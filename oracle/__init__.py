"""CPU oracle for block-scaled FP8 quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference the GPU
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; the product path
(``fp8_precision_quant_amd``) never does, and the two share no code.

The arithmetic lives in ``fp8q_oracle.c`` (plain C, fp32 rounding exactly as
written, no FMA contraction).  This module only marshals numpy arrays and
maps the scale-grid layouts onto one scale per (row, chunk), which is plain
indexing:

* 1x128 row tiles: tile (r, j) covers ``X[r, 128j:128j+128]``, scale ``S[r, j]``.
* 128x128 blocks: block (i, j) covers ``X[128i:+128, 128j:+128]``, ``S[i, j]``.
* per-tensor: one tile, ``S[0, 0]``.

Tile shapes come from the pages: one scale per 128x128 weight block
("FP8-RL" article, section 一) and fine-grained per-tile scales for
activations and gradients (Ling 2.0 FP8 blog, "fine-grained quantization");
the 1x128 activation tile is the reading used for the pages' unstated tile
size.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

TILE = 128

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            i64, p = ctypes.c_int64, ctypes.c_void_p
            L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.orc_e4m3_decode.restype = ctypes.c_float
            L.orc_e4m3_encode.argtypes = [ctypes.c_float]
            L.orc_e4m3_encode.restype = ctypes.c_uint8
            L.orc_decode_array.argtypes = [p, i64, p]
            L.orc_encode_array.argtypes = [p, i64, p]
            L.orc_quant_tiles.argtypes = [p, i64, i64, i64, i64, p, p]
            L.orc_quant_tiles_pow2.argtypes = [p, i64, i64, i64, i64, p, p]
            L.orc_pow2_exponent.argtypes = [ctypes.c_float]
            L.orc_pow2_exponent.restype = ctypes.c_int
            L.orc_e8m0_decode_array.argtypes = [p, i64, p]
            f64 = ctypes.c_double
            L.orc_adamw_step.argtypes = [i64, p, p, p, p, f64, f64, f64, f64, f64, i64]
            L.orc_adamw_fp8_step.argtypes = [i64, p, p, p, p, p, p, f64, f64, f64, f64, f64, i64]
            L.orc_gemm_f32.argtypes = [i64, i64, i64, p, p, p, p, p, i64, p]
            L.orc_gemm_f64.argtypes = [i64, i64, i64, p, p, p, p, p, i64, p, p]
            L.orc_f32_to_bf16.argtypes = [p, i64, p]
            L.orc_underflow_count.argtypes = [p, p, i64, p, p]
            L.orc_num_threads.restype = ctypes.c_int
            L.orc_set_num_threads.argtypes = [ctypes.c_int]
            _lib = L
    return _lib


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops (timing only)."""
    lib().orc_set_num_threads(int(n))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# codec
# ---------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN code bytes -> fp32 values (NaN for 0x7F / 0xFF)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().orc_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    """fp32 values -> E4M3FN codes: nearest, ties to even, saturating at 448."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_encode_array(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def quant_tiles(x, tile_rows: int, tile_cols: int):
    """Quantize fp32 ``x[R, C]`` with tiles of ``tile_rows x tile_cols``.

    Returns ``(q uint8[R, C], s float32[ceil(R/tr), ceil(C/tc)])``.
    """
    x = _c(x, np.float32)
    assert x.ndim == 2
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty((-(-R // tile_rows), -(-C // tile_cols)), np.float32)
    if R and C:
        lib().orc_quant_tiles(_ptr(x), R, C, tile_rows, tile_cols, _ptr(q), _ptr(s))
    return q, s


def quant_1x128(x):
    """1x128 row tiles along the last axis (activations and gradients)."""
    return quant_tiles(x, 1, TILE)


def quant_128x128(x):
    """128x128 blocks (weights)."""
    return quant_tiles(x, TILE, TILE)


def quant_tensor(x):
    """One scale for the whole tensor; returns ``(q, s)`` with ``s.shape == (1, 1)``."""
    x = _c(x, np.float32)
    R, C = x.shape
    return quant_tiles(x, max(R, 1), max(C, 1))


def quant_transpose(x):
    """Row tiles of X and row tiles of X^T (column tiles of X, stored transposed).

    Returns ``(q_row[R, C], s_row[R, ceil(C/128)], q_colT[C, R], s_colT[C, ceil(R/128)])``.
    """
    x = _c(x, np.float32)
    q_row, s_row = quant_1x128(x)
    q_colT, s_colT = quant_1x128(np.ascontiguousarray(x.T))
    return q_row, s_row, q_colT, s_colT


def quantize(x, kind: str):
    return {"row": quant_1x128, "block": quant_128x128, "tensor": quant_tensor}[kind](x)


# ---------------------------------------------------------------------------
# power-of-two (E8M0) scales: the micro-scaling variant of block scaling
# (Introl FP8 infrastructure guide, scaling strategies and the Blackwell
# section: MXFP8 block scales applied by the hardware).  Reading: the same
# tiles, s = 2^e with e the smallest integer >= -126 such that amax <= 448 2^e,
# stored as the byte e + 127.
# ---------------------------------------------------------------------------

def pow2_exponent(amax: float) -> int:
    """e of one tile from its fp32 amax."""
    return int(lib().orc_pow2_exponent(float(np.float32(amax))))


def e8m0_decode(b) -> np.ndarray:
    """E8M0 bytes -> fp32 2^(b-127) (NaN for 255)."""
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    lib().orc_e8m0_decode_array(_ptr(b), b.size, _ptr(out))
    return out


def quant_tiles_pow2(x, tile_rows: int, tile_cols: int):
    """Like ``quant_tiles`` with power-of-two scales.

    Returns ``(q uint8[R, C], e uint8[ceil(R/tr), ceil(C/tc)])``, ``e`` the
    E8M0 scale bytes.
    """
    x = _c(x, np.float32)
    assert x.ndim == 2
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    e = np.empty((-(-R // tile_rows), -(-C // tile_cols)), np.uint8)
    if R and C:
        lib().orc_quant_tiles_pow2(_ptr(x), R, C, tile_rows, tile_cols, _ptr(q), _ptr(e))
    return q, e


def quant_1x128_pow2(x):
    return quant_tiles_pow2(x, 1, TILE)


def quant_128x128_pow2(x):
    return quant_tiles_pow2(x, TILE, TILE)


def quant_transpose_pow2(x):
    """Row tiles of X and of X^T with power-of-two scales:
    ``(q_row, e_row, q_colT, e_colT)``."""
    x = _c(x, np.float32)
    q_row, e_row = quant_1x128_pow2(x)
    q_colT, e_colT = quant_1x128_pow2(np.ascontiguousarray(x.T))
    return q_row, e_row, q_colT, e_colT


# ---------------------------------------------------------------------------
# scale expansion: one scale per (row of A, chunk) and (column of C, chunk)
# ---------------------------------------------------------------------------

def expand_a_scales(sa, kind: str, M: int, KB: int) -> np.ndarray:
    sa = np.asarray(sa, np.float32)
    if kind == "row":        # SA(m, kb) = sa[m, kb]
        return _c(sa[:M, :KB], np.float32)
    if kind == "tensor":     # SA(m, kb) = sa[0, 0]
        return np.full((M, KB), sa.reshape(-1)[0], np.float32)
    raise ValueError(kind)


def expand_b_scales(sb, kind: str, layout: str, N: int, KB: int) -> np.ndarray:
    """SB(n, kb) for output column n and chunk kb.

    ``layout == "NK"``: B stored [N][K], its scale grid indexed [n-tile][k-tile].
    ``layout == "KN"``: B stored [K][N] (the contraction axis is B's row axis),
    its scale grid follows the storage: [k-block][n-block].
    """
    sb = np.asarray(sb, np.float32)
    n = np.arange(N)
    kb = np.arange(KB)
    if kind == "tensor":
        return np.full((N, KB), sb.reshape(-1)[0], np.float32)
    if layout == "NK":
        if kind == "block":
            return _c(sb[n[:, None] // TILE, kb[None, :]], np.float32)
        if kind == "row":
            return _c(sb[:N, :KB], np.float32)
    if layout == "KN" and kind == "block":
        return _c(sb[kb[None, :], n[:, None] // TILE], np.float32)
    raise ValueError((kind, layout))


def b_as_nk(b, layout: str) -> np.ndarray:
    """B codes with the contraction axis contiguous: [N][K]."""
    b = np.asarray(b, np.uint8)
    return _c(b if layout == "NK" else b.T, np.uint8)


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = _c(rows, np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < M))
    return r, r.size


def gemm_f32(a, sa_full, b_nk, sb_full, rows=None) -> np.ndarray:
    """fp32 block-scaled GEMM on expanded scales; returns C[len(rows) or M, N]."""
    a = _c(a, np.uint8)
    b = _c(b_nk, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    KB = -(-K // TILE)
    sa = _c(sa_full, np.float32)
    sb = _c(sb_full, np.float32)
    assert sa.shape == (M, KB) and sb.shape == (N, KB)
    r, nr = _rows_arg(rows, M)
    out = np.zeros((nr, N), np.float32)
    if nr and N:
        lib().orc_gemm_f32(M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                           None if r is None else _ptr(r), nr, _ptr(out))
    return out


def gemm_f64(a, sa_full, b_nk, sb_full, rows=None):
    """fp64 evaluation of the same sum, plus the absolute-product sum R."""
    a = _c(a, np.uint8)
    b = _c(b_nk, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    KB = -(-K // TILE)
    sa = _c(sa_full, np.float32)
    sb = _c(sb_full, np.float32)
    assert sa.shape == (M, KB) and sb.shape == (N, KB)
    r, nr = _rows_arg(rows, M)
    C = np.zeros((nr, N), np.float64)
    R = np.zeros((nr, N), np.float64)
    if nr and N:
        lib().orc_gemm_f64(M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                           None if r is None else _ptr(r), nr, _ptr(C), _ptr(R))
    return C, R


def gemm_blockscaled(a, sa, sa_kind, b, sb, sb_kind, b_layout="NK", rows=None,
                     f64=False):
    """C = sum_kb SA(m,kb) SB(n,kb) sum_{k in kb} dec(A[m,k]) dec(B^[n,k]).

    ``a``: codes [M][K]; ``b``: codes [N][K] ("NK") or [K][N] ("KN");
    scale grids as produced by the quantizers.  Returns fp32 C (or
    ``(C64, R)`` when ``f64``).
    """
    a = np.asarray(a, np.uint8)
    M, K = a.shape
    b_nk = b_as_nk(b, b_layout)
    N = b_nk.shape[0]
    KB = -(-K // TILE)
    sa_full = expand_a_scales(sa, sa_kind, M, KB)
    sb_full = expand_b_scales(sb, sb_kind, b_layout, N, KB)
    if f64:
        return gemm_f64(a, sa_full, b_nk, sb_full, rows)
    return gemm_f32(a, sa_full, b_nk, sb_full, rows)


def grouped_gemm(a, sa, offsets, b, sb, rows=None, f64=False):
    """Per group e, rows [off[e], off[e+1]) of A times expert weights B[e] (NK).

    ``a`` [M_pad][K] codes with 1x128 scales ``sa``; ``b`` [G][N][K] codes with
    128x128 block scales ``sb`` [G][ceil(N/128)][ceil(K/128)].  Rows outside
    every group produce zeros.  ``rows`` optionally selects output rows.
    """
    a = np.asarray(a, np.uint8)
    off = np.asarray(offsets, np.int64)
    G = off.size - 1
    M, K = a.shape
    N = b.shape[1]
    want = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((want.size, N), np.float64 if f64 else np.float32)
    R = np.zeros((want.size, N), np.float64) if f64 else None
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        if sel.size == 0:
            continue
        local = want[sel] - lo
        res = gemm_blockscaled(a[lo:hi], np.asarray(sa)[lo:hi], "row", b[e], sb[e],
                               "block", "NK", rows=local, f64=f64)
        if f64:
            out[sel], R[sel] = res
        else:
            out[sel] = res
    return (out, R) if f64 else out


def grouped_gemm_dgrad(a, sa, offsets, w, sw, rows=None, f64=False):
    """MoE dgrad per group: rows [off[e], off[e+1]) of dY times expert weight
    W[e] read as stored (Ling 2.0 FP8 blog, "FP8 on-demand transpose weight";
    groups padded per "FP8 padding routing map").

    ``a`` dY codes [M_pad][N] with 1x128 scales ``sa`` along N; ``w`` [G][N][K]
    codes with 128x128 block scales ``sw`` [G][ceil(N/128)][ceil(K/128)].  The
    contraction runs over W's rows, i.e. W[e] is the [K][N] ("KN") operand of
    the definition with its block grid as stored.  Rows outside every group
    produce zeros.
    """
    a = np.asarray(a, np.uint8)
    off = np.asarray(offsets, np.int64)
    G = off.size - 1
    M = a.shape[0]
    K = w.shape[2]
    want = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((want.size, K), np.float64 if f64 else np.float32)
    R = np.zeros((want.size, K), np.float64) if f64 else None
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        if sel.size == 0:
            continue
        res = gemm_blockscaled(a[lo:hi], np.asarray(sa)[lo:hi], "row", w[e], sw[e],
                               "block", "KN", rows=want[sel] - lo, f64=f64)
        if f64:
            out[sel], R[sel] = res
        else:
            out[sel] = res
    return (out, R) if f64 else out


def grouped_gemm_wgrad(at, sat, bt, sbt, offsets, rows=None, f64=False):
    """MoE weight gradient per group: dW[e] = sum over the group's tokens only
    of dY^T times X (the transposed re-quantization of Ling 2.0 FP8 blog,
    "grad (transpose)"; groups per "FP8 padding routing map").

    ``at`` dY^T codes [N][M_pad] and ``bt`` X^T codes [K][M_pad], both with
    1x128 scales along tokens (``sat`` [N][M_pad/128], ``sbt`` [K][M_pad/128]);
    every offset is a multiple of 128, so group e's chunks are the token
    chunks [off[e], off[e+1]) / 128.  Returns [G][len(rows) or N][K]; a group
    with no tokens gives zeros.
    """
    at = np.asarray(at, np.uint8)
    bt = np.asarray(bt, np.uint8)
    off = np.asarray(offsets, np.int64)
    G = off.size - 1
    N, K = at.shape[0], bt.shape[0]
    nr = N if rows is None else len(rows)
    out = np.zeros((G, nr, K), np.float64 if f64 else np.float32)
    R = np.zeros((G, nr, K), np.float64) if f64 else None
    for e in range(G):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        assert lo % TILE == 0 and hi % TILE == 0
        cl, ch = lo // TILE, hi // TILE
        res = gemm_blockscaled(at[:, lo:hi], np.asarray(sat)[:, cl:ch], "row",
                               bt[:, lo:hi], np.asarray(sbt)[:, cl:ch], "row", "NK",
                               rows=rows, f64=f64)
        if f64:
            out[e], R[e] = res
        else:
            out[e] = res
    return (out, R) if f64 else out


# ---------------------------------------------------------------------------
# Adam with FP8 moments (Ling 2.0 FP8 blog, "FP8 Optimizer")
# ---------------------------------------------------------------------------

def adamw_step(p, g, m, v, lr, beta1, beta2, eps, wd, t):
    """One fp32 AdamW step (see ``orc_adamw_step``); returns new ``(p, m, v)``."""
    p = _c(p, np.float32).copy()
    g = _c(g, np.float32)
    m = _c(m, np.float32).copy()
    v = _c(v, np.float32).copy()
    lib().orc_adamw_step(p.size, _ptr(p), _ptr(g), _ptr(m), _ptr(v), lr, beta1, beta2, eps, wd, t)
    return p, m, v


def adamw_fp8_step(p, g, mq, ms, vq, vs, lr, beta1, beta2, eps, wd, t):
    """One AdamW step with E4M3 moments and one fp32 scale per 128 elements:
    returns new ``(p, mq, ms, vq, vs)`` (flat arrays)."""
    p = _c(p, np.float32).reshape(-1).copy()
    g = _c(g, np.float32).reshape(-1)
    mq, vq = _c(mq, np.uint8).reshape(-1).copy(), _c(vq, np.uint8).reshape(-1).copy()
    ms, vs = _c(ms, np.float32).reshape(-1).copy(), _c(vs, np.float32).reshape(-1).copy()
    n = p.size
    assert g.size == n and mq.size == n and vq.size == n and ms.size == vs.size == -(-n // TILE)
    lib().orc_adamw_fp8_step(n, _ptr(p), _ptr(g), _ptr(mq), _ptr(ms), _ptr(vq), _ptr(vs),
                             lr, beta1, beta2, eps, wd, t)
    return p, mq, ms, vq, vs


# ---------------------------------------------------------------------------
# output rounding and statistics
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns the uint16 bit patterns."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def underflow_fraction(x, q) -> float:
    """Fraction of non-zero inputs whose code decodes to zero."""
    x = _c(x, np.float32)
    q = _c(q, np.uint8)
    assert x.shape == q.shape
    u = ctypes.c_int64()
    nz = ctypes.c_int64()
    lib().orc_underflow_count(_ptr(x), _ptr(q), x.size, ctypes.byref(u), ctypes.byref(nz))
    return u.value / nz.value if nz.value else 0.0


def exact_gemm_f64(x, w, rows=None) -> np.ndarray:
    """y = x w^T in fp64 from the unquantized inputs (quality reference)."""
    x = np.asarray(x, np.float64)
    if rows is not None:
        x = x[np.asarray(rows)]
    return x @ np.asarray(w, np.float64).T
