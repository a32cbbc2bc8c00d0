"""ORACLE -- test infrastructure, not product code.

ctypes wrapper over ``dsa_oracle.c``, the plain CPU statement of the DSA
sparse-attention layer (see that file's header for the pages it follows and
for the readings taken where they are silent).  Only ``tests/``, the smoke
check and the benchmark's CPU-baseline leg may import this package; the HIP
library never does, and the two share no code.

All arrays are numpy, in the oracle's logical layouts (one sequence):
  index_k, K, V : [T][G][C] uint16 (bf16 bits);  index_q : [Hi][P] uint16;  z : [Hi] float32
  q : [Hq][D] uint16;  codes : [R][G][P] uint8;  scales : [R][G] float32
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "lib", "liboracle.so")

# Geometry of the DSA layer (pages: regions of 8, 256-d summaries, 16 indexer heads,
# top-512; 64 query heads in 4 KV groups of head_dim 192; window 512).
REGION, PROXY, GROUPS, IDX_HEADS, Q_HEADS, HEAD_DIM, TOPK, WINDOW = 8, 256, 4, 16, 64, 192, 512, 512
TAU = 1.0 / math.sqrt(HEAD_DIM)

_lib = None


def build(verbose=False):
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           os.path.join(_HERE, "dsa_oracle.c"), "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stderr}")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i64, i32, f64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
        L.or_num_threads.restype = ctypes.c_int
        L.or_e4m3_value.argtypes = [ctypes.c_uint8]
        L.or_e4m3_value.restype = f64
        L.or_e4m3_encode.argtypes = [f32]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_compress_regions.argtypes = [vp, i64, i32, i32, i64, i64, vp, vp]
        L.or_scores.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, vp]
        L.or_select.argtypes = [vp, i64, i32, vp]
        L.or_select.restype = i32
        L.or_attend.argtypes = [vp, vp, vp, i32, i32, i32, i64, vp, vp, i32, f64, vp]
        L.or_swa.argtypes = [vp, vp, vp, i32, i32, i32, i64, i64, f64, vp]
        L.or_quantize_rows.argtypes = [vp, i64, i32, vp, vp]
        L.or_attend_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp, vp, i32, f64, vp]
        L.or_dsa_query.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, i64,
                                   vp, vp, vp, vp]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().or_num_threads())


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous arrays"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3_value(code: int) -> float:
    return lib().or_e4m3_value(int(code))


def e4m3_encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32).ravel()
    f = lib().or_e4m3_encode
    return np.array([f(float(v)) for v in x], dtype=np.uint8)


def compress_regions(index_k, r0, r1, codes=None, scales=None):
    """Summaries of regions [r0, r1) of one sequence from index_k [T][G][P]."""
    ik = _c(index_k, np.uint16)
    T, G, P = ik.shape
    assert 0 <= r0 <= r1 and 8 * r1 <= T, "only complete regions are summarised"
    R = max(r1, 1)
    if codes is None:
        codes = np.zeros((R, G, P), dtype=np.uint8)
        scales = np.zeros((R, G), dtype=np.float32)
    lib().or_compress_regions(_p(ik), T, G, P, r0, r1, _p(codes), _p(scales))
    return codes, scales


def scores(index_q, z, codes, scales, n_regions):
    """Scores [G][n_regions] of regions [0, n_regions) for one query."""
    iq, zz = _c(index_q, np.uint16), _c(z, np.float32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.float32)
    Hi, P = iq.shape
    G = codes.shape[1]
    out = np.zeros((G, max(n_regions, 0)), dtype=np.float64)
    if n_regions > 0:
        lib().or_scores(_p(iq), _p(zz), _p(codes), _p(scales), G, P, Hi // G, n_regions, _p(out))
    return out


def select(scores_g, c, k=TOPK):
    """Top-k of candidate regions 0..c-1 (scores_g[0..c)) plus the forced current region c."""
    s = _c(scores_g[:c], np.float64)
    if s.size == 0:
        s = np.zeros(1)
    sel = np.zeros(max(k, 1), dtype=np.int32)
    n = lib().or_select(_p(s), int(c), int(k), _p(sel))
    return sel[:n].copy()


def attend(q, K, V, p, sel_lists, k=TOPK, tau=TAU):
    """Sparse GQA for one query at position p over the selected regions of each group."""
    q, K, V = _c(q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    Hq, D = q.shape
    G = K.shape[1]
    sel = np.full((G, k), -1, dtype=np.int32)
    nsel = np.zeros(G, dtype=np.int32)
    for g, lst in enumerate(sel_lists):
        lst = np.asarray(lst, dtype=np.int32)
        sel[g, :lst.size] = lst
        nsel[g] = lst.size
    out = np.zeros((Hq, D), dtype=np.float64)
    lib().or_attend(_p(q), _p(K), _p(V), G, D, Hq, int(p), _p(sel), _p(nsel), k, float(tau), _p(out))
    return out


def quantize_rows(X):
    """FP8 cache rows: X [..][C] bf16 bits -> (E4M3 codes, same shape; fp32 scales [..])."""
    X = _c(X, np.uint16)
    C = X.shape[-1]
    rows = X.reshape(-1, C)
    codes = np.zeros(rows.shape, dtype=np.uint8)
    scales = np.zeros(rows.shape[0], dtype=np.float32)
    lib().or_quantize_rows(_p(rows), rows.shape[0], C, _p(codes), _p(scales))
    return codes.reshape(X.shape), scales.reshape(X.shape[:-1])


def attend_fp8(q, Kc, Ks, Vc, Vs, p, sel_lists, k=TOPK, tau=TAU):
    """attend() over an FP8 cache: Kc/Vc [T][G][D] codes, Ks/Vs [T][G] row scales."""
    q = _c(q, np.uint16)
    Kc, Vc = _c(Kc, np.uint8), _c(Vc, np.uint8)
    Ks, Vs = _c(Ks, np.float32), _c(Vs, np.float32)
    Hq, D = q.shape
    G = Kc.shape[1]
    sel = np.full((G, k), -1, dtype=np.int32)
    nsel = np.zeros(G, dtype=np.int32)
    for g, lst in enumerate(sel_lists):
        lst = np.asarray(lst, dtype=np.int32)
        sel[g, :lst.size] = lst
        nsel[g] = lst.size
    out = np.zeros((Hq, D), dtype=np.float64)
    lib().or_attend_fp8(_p(q), _p(Kc), _p(Ks), _p(Vc), _p(Vs), G, D, Hq, int(p), _p(sel), _p(nsel), k, float(tau),
                        _p(out))
    return out


def swa(q, K, V, p, window=WINDOW, tau=TAU):
    """Sliding-window attention of one query at p over positions max(0,p-W+1)..p of K/V [T][G][D]."""
    q, K, V = _c(q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    Hq, D = q.shape
    G = K.shape[1]
    out = np.zeros((Hq, D), dtype=np.float64)
    lib().or_swa(_p(q), _p(K), _p(V), G, D, Hq, int(p), int(window), float(tau), _p(out))
    return out


def dsa_query(index_q, z, codes, scales, q, K, V, p, k=TOPK, tau=TAU, want_scores=False):
    """One query end to end: scores -> top-k (+ forced current region) -> sparse GQA.

    ``codes``/``scales`` must hold the summaries of every region before p // 8.
    Returns (sel [G][k] padded with -1, nsel [G], out [Hq][D] fp64, scores [G][c] or None)."""
    iq, zz = _c(index_q, np.uint16), _c(z, np.float32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.float32)
    q, K, V = _c(q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    Hi, P = iq.shape
    Hq, D = q.shape
    G = K.shape[1]
    c = p // 8
    sel = np.full((G, k), -1, dtype=np.int32)
    nsel = np.zeros(G, dtype=np.int32)
    out = np.zeros((Hq, D), dtype=np.float64)
    sc = np.zeros((G, max(c, 1)), dtype=np.float64) if want_scores else None
    lib().or_dsa_query(_p(iq), _p(zz), _p(codes), _p(scales), _p(q), _p(K), _p(V), G, P, Hi, D, Hq, k,
                       float(tau), int(p), _p(sel), _p(nsel), _p(out),
                       _p(sc) if sc is not None else None)
    return sel, nsel, out, (sc[:, :c] if sc is not None else None)
