"""Seeded, counter-based synthetic inputs shared by the CPU oracle harness and the GPU harness.

Holds no arithmetic of the attention method. Every value is a pure function of
(seed, tensor id, logical flat index); see ``csrc/gen_core.h`` for the exact
definition (SplitMix64 mixing, Irwin-Hall(12) normals, bf16 round-to-nearest-even).

Three implementations of that one definition live here:
  * ``ref_*``     -- plain numpy, the readable definition (slow, small slices);
  * ``host_*``    -- the C library (``csrc/gen_host.c``), fast, host buffers;
  * ``dev_*``     -- the HIP library (``csrc/gen_device.hip``), writes GPU buffers
                     in the physical layouts of the attention library.
Tests pin the C and HIP versions to the numpy one bit for bit.

Workload recipe (tensor ids; the seed of workload i is ``SEED_BASE + i``):
  Q=1, K=2, V=3 ~ N(0,1) bf16; index_k=4, index_q=5 ~ N(0,1)/16 bf16;
  z=6 ~ U(0,1) fp32; planted-region mask=7, planted coefficients=9;
  sliding-window layer l (0-based) uses ids + 16*(l+1).
Indexer front-end: hidden states x (id 12) ~ N(0,1) bf16, projection weights (id 13) ~ N(0,1)/sqrt(H)
  bf16, RMSNorm gains (id 14) 0.75 + 0.5 U(0,1) fp32 (gamma_q first, then gamma_k).
Correlated prefill chunk (neighbouring queries select overlapping regions):
  anchors of index_q (id 10, N(0,1)/16) and of z (id 11, U(0,1)) every ``every``
  queries; query i blends anchors a = i // every and a + 1 with t = (i mod every)
  / every (norm-preserving weights for index_q, linear for z) and mixes in
  ``noise`` of its own i.i.d. index_q (id 5).  See ``host_correlated_index_queries``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

SEED_BASE = 0xD5A00000
TID_Q, TID_K, TID_V, TID_IK, TID_IQ, TID_Z, TID_MASK, TID_COEF = 1, 2, 3, 4, 5, 6, 7, 9
TID_IQ_ANCHOR, TID_Z_ANCHOR = 10, 11
TID_X, TID_W, TID_GAMMA = 12, 13, 14
IK_SCALE = 1.0 / 16.0

LAYOUT_GROUP_MAJOR, LAYOUT_REGION_T, LAYOUT_TOKEN_MAJOR, LAYOUT_KTILED = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBDIR = os.path.join(_HERE, "lib")
HOST_LIB = os.path.join(_LIBDIR, "libdsa_inputs_host.so")
DEV_LIB = os.path.join(_LIBDIR, "libdsa_inputs_dev.so")

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
P002_THRESH = 85899346


def tid_swa(tid: int, layer: int) -> int:
    """Tensor id of tensor ``tid`` for sliding-window layer ``layer`` (0-based)."""
    return tid + 16 * (layer + 1)


# ----------------------------------------------------------------------------------------------
# numpy reference (the readable definition)
# ----------------------------------------------------------------------------------------------
def ref_mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def ref_stream_key(seed: int, tid: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return ref_mix64(np.uint64(seed) + GAMMA * np.uint64(tid + 1))


def ref_word(key, idx, j):
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return ref_mix64(np.uint64(key) + GAMMA * (np.uint64(4) * idx + np.uint64(j + 1)))


def _sum4x16(w):
    m = np.uint64(0xFFFF)
    return ((w & m) + ((w >> np.uint64(16)) & m) + ((w >> np.uint64(32)) & m)
            + (w >> np.uint64(48))).astype(np.int64)


def ref_normal_f32(seed, tid, idx):
    key = ref_stream_key(seed, tid)
    s = _sum4x16(ref_word(key, idx, 0)) + _sum4x16(ref_word(key, idx, 1)) + _sum4x16(ref_word(key, idx, 2))
    return ((s - 393210).astype(np.float32) * np.float32(1.0 / 65536.0)).astype(np.float32)


def ref_uniform_f32(seed, tid, idx):
    key = ref_stream_key(seed, tid)
    return ((ref_word(key, idx, 0) >> np.uint64(40)).astype(np.float32)
            * np.float32(1.0 / 16777216.0)).astype(np.float32)


def ref_bernoulli(seed, tid, idx, thresh=P002_THRESH):
    key = ref_stream_key(seed, tid)
    return (ref_word(key, idx, 0) >> np.uint64(32)) < np.uint64(thresh)


def bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (NaN stays NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def ref_hadamard16(row, col):
    x = np.bitwise_and(np.asarray(row, dtype=np.uint32), np.asarray(col, dtype=np.uint32))
    par = np.zeros_like(x)
    for bit in range(8):
        par ^= (x >> np.uint32(bit)) & np.uint32(1)
    return np.where(par == 1, np.float32(-0.0625), np.float32(0.0625)).astype(np.float32)


def ref_planted_beta(seed, breg, g, G, d):
    """fp32 bias for planted (sequence-region breg, group g) at channels d (see gen_core.h)."""
    base = (np.uint64(breg) * np.uint64(G) + np.uint64(g)) * np.uint64(4)
    c = [np.float32(0.5) * ref_normal_f32(seed, TID_COEF, base + np.uint64(k)) for k in range(4)]
    beta = (c[0] * ref_hadamard16(1 + 4 * g, d)).astype(np.float32)
    for k in range(1, 4):
        beta = (beta + (c[k] * ref_hadamard16(1 + 4 * g + k, d)).astype(np.float32)).astype(np.float32)
    return beta


def ref_tokens_bf16(seed, tid, T, G, C, b, t0, nt, scale=1.0):
    """Tokens [t0, t0+nt) of sequence b of logical [B][T][G][C]; returns [nt][G][C] bf16 bits."""
    idx = ((np.uint64(b) * np.uint64(T) + np.uint64(t0)) * np.uint64(G * C)
           + np.arange(nt * G * C, dtype=np.uint64))
    return bf16_rne(ref_normal_f32(seed, tid, idx) * np.float32(scale)).reshape(nt, G, C)


def ref_index_k(seed, T, G, P, b, t0, nt, planted=False):
    x = (ref_normal_f32(seed, TID_IK, ((np.uint64(b) * np.uint64(T) + np.uint64(t0)) * np.uint64(G * P)
                                       + np.arange(nt * G * P, dtype=np.uint64)))
         * np.float32(IK_SCALE)).astype(np.float32).reshape(nt, G, P)
    if planted:
        R = T // 8
        d = np.arange(P, dtype=np.uint32)
        for tl in range(nt):
            t = t0 + tl
            breg = b * R + t // 8
            if ref_bernoulli(seed, TID_MASK, np.uint64(breg)):
                for g in range(G):
                    x[tl, g] = (x[tl, g] + ref_planted_beta(seed, breg, g, G, d)).astype(np.float32)
    return bf16_rne(x)


# ----------------------------------------------------------------------------------------------
# C host library
# ----------------------------------------------------------------------------------------------
_host = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, u32, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_float, ctypes.c_void_p)
        lib.dsagen_normal_bf16.argtypes = [u64, u32, u64, u64, f32, vp]
        lib.dsagen_normal_f32.argtypes = [u64, u32, u64, u64, f32, vp]
        lib.dsagen_uniform_f32.argtypes = [u64, u32, u64, u64, vp]
        lib.dsagen_bernoulli_u8.argtypes = [u64, u32, u64, u64, u32, vp]
        lib.dsagen_tokens_bf16.argtypes = [u64, u32, i64, i32, i32, i32, i64, i64, f32, vp]
        lib.dsagen_index_k.argtypes = [u64, u32, u32, u32, ctypes.c_int, i64, i32, i32, i32, i64, i64, vp]
        _host = lib
    return _host


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def host_normal_bf16(seed, tid, n, scale=1.0, start=0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _host_lib().dsagen_normal_bf16(seed, tid, start, n, scale, _ptr(out))
    return out


def host_uniform_f32(seed, tid, n, start=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host_lib().dsagen_uniform_f32(seed, tid, start, n, _ptr(out))
    return out


def host_bernoulli(seed, tid, n, start=0, thresh=P002_THRESH) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _host_lib().dsagen_bernoulli_u8(seed, tid, start, n, thresh, _ptr(out))
    return out.astype(bool)


def host_tokens_bf16(seed, tid, T, G, C, b, t0, nt, scale=1.0) -> np.ndarray:
    out = np.empty((nt, G, C), dtype=np.uint16)
    _host_lib().dsagen_tokens_bf16(seed, tid, T, G, C, b, t0, nt, scale, _ptr(out))
    return out


def host_index_k(seed, T, G, P, b, t0, nt, planted=False) -> np.ndarray:
    out = np.empty((nt, G, P), dtype=np.uint16)
    _host_lib().dsagen_index_k(seed, TID_IK, TID_MASK, TID_COEF, int(planted), T, G, P, b, t0, nt, _ptr(out))
    return out


def host_correlated_index_queries(seed, nq, heads=16, P=256, every=64, noise=0.1):
    """index_q [nq][heads][P] (bf16 bits) and z [nq][heads] (fp32) of a prefill chunk whose neighbouring
    queries are correlated: a smooth path between anchor queries every ``every`` queries, plus ``noise``
    of each query's own i.i.d. index_q (noise = 1 gives the i.i.d. workload back).  float32 arithmetic,
    one bf16 rounding at the end."""
    na = nq // every + 2
    A = bf16_to_f32(host_normal_bf16(seed, TID_IQ_ANCHOR, na * heads * P, IK_SCALE)).reshape(na, heads, P)
    Z = host_uniform_f32(seed, TID_Z_ANCHOR, na * heads).reshape(na, heads)
    own = bf16_to_f32(host_normal_bf16(seed, TID_IQ, nq * heads * P, IK_SCALE)).reshape(nq, heads, P)
    i = np.arange(nq)
    a = i // every
    t = ((i % every) / np.float32(every)).astype(np.float32)
    nrm = np.sqrt((np.float32(1) - t) * (np.float32(1) - t) + t * t).astype(np.float32)
    w0 = ((np.float32(1) - t) / nrm).astype(np.float32)[:, None, None]
    w1 = (t / nrm).astype(np.float32)[:, None, None]
    path = w0 * A[a] + w1 * A[a + 1]
    c_path = np.float32(np.sqrt(np.float32(1) - np.float32(noise) * np.float32(noise)))
    iq = c_path * path + np.float32(noise) * own
    z = ((np.float32(1) - t)[:, None] * Z[a] + t[:, None] * Z[a + 1]).astype(np.float32)
    return bf16_rne(iq.astype(np.float32)), z


def host_frontend_inputs(seed, T, H, n_rows):
    """x [T][H] and W [n_rows][H] (bf16 bits), gamma_q and gamma_k [256] (fp32) of the indexer front-end."""
    x = host_normal_bf16(seed, TID_X, T * H).reshape(T, H)
    w = host_normal_bf16(seed, TID_W, n_rows * H, 1.0 / float(np.sqrt(H))).reshape(n_rows, H)
    u = host_uniform_f32(seed, TID_GAMMA, 512)
    g = (np.float32(0.75) + np.float32(0.5) * u).astype(np.float32)
    return x, w, g[:256].copy(), g[256:].copy()


# ----------------------------------------------------------------------------------------------
# HIP device library (takes raw device pointers and a hipStream_t as integers)
# ----------------------------------------------------------------------------------------------
_dev = None


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        u64, u32, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_float, ctypes.c_void_p)
        lib.dsagen_dev_tokens.argtypes = [u64, u32, u32, u32, ctypes.c_int, i32, i64, i32, i32, i64, i64,
                                          i64, i64, i32, f32, vp, vp]
        lib.dsagen_dev_tokens.restype = ctypes.c_int
        lib.dsagen_dev_flat.argtypes = [u64, u32, u64, u64, f32, ctypes.c_int, vp, vp]
        lib.dsagen_dev_flat.restype = ctypes.c_int
        _dev = lib
    return _dev


def dev_tokens(ptr, stream, seed, tid, B, T, G, C, t0, nt, tcap, tmod, layout, scale=1.0,
               planted=False):
    """Fill tokens [t0, t0+nt) of all B sequences of logical [B][T][G][C] into a device buffer."""
    rc = _dev_lib().dsagen_dev_tokens(seed, tid, TID_MASK, TID_COEF, int(planted), B, T, G, C, t0, nt,
                                      tcap, tmod, layout, scale, ctypes.c_void_p(ptr), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"dsagen_dev_tokens failed: {rc}")


def dev_flat(ptr, stream, seed, tid, n, kind, scale=1.0, start=0):
    """kind 0: bf16 normal*scale, 1: fp32 uniform, 2: fp32 normal*scale; flat indices [start, start+n)."""
    rc = _dev_lib().dsagen_dev_flat(seed, tid, start, n, scale, kind, ctypes.c_void_p(ptr), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"dsagen_dev_flat failed: {rc}")


# ----------------------------------------------------------------------------------------------
# build
# ----------------------------------------------------------------------------------------------
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    os.makedirs(_LIBDIR, exist_ok=True)
    src = os.path.join(_HERE, "csrc")
    cmds = [
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         os.path.join(src, "gen_host.c"), "-o", HOST_LIB],
        [HIPCC, *HIP_FLAGS, os.path.join(src, "gen_device.hip"), "-o", DEV_LIB],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c), flush=True)
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(c)}\n{r.stdout}\n{r.stderr}")
