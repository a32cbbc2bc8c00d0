"""Python binding of the gfx950 DSA sparse-attention C ABI (``include/dsa.h``).

Argument marshalling only: every step runs in the HIP library
``lib/libdsa_mi355x.so``; nothing here computes.  Functions take torch tensors
on the GPU (PyTorch provides device memory and streams), check dtypes, devices,
contiguity and sizes, and call the entry point of the same name on the current
torch stream (or ``stream=`` a torch.cuda.Stream).  A missing library raises.

Layouts are those of the header: caches are group-major, V is
region-transposed ([B][G][tcap/8][D][8]); bf16 tensors are torch.bfloat16.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libdsa_mi355x.so")

REGION, PROXY, GROUPS, IDX_HEADS, Q_HEADS, HEAD_DIM, MAX_TOPK, WINDOW = 8, 256, 4, 16, 64, 192, 512, 512

ENTRY_POINTS = [
    "dsa_geometry_default", "dsa_status_string", "dsa_last_error", "dsa_cache_write",
    "dsa_compress_regions", "dsa_score_topk_workspace_size", "dsa_score_topk",
    "dsa_sparse_gqa_workspace_size", "dsa_sparse_gqa_decode",
    "dsa_sparse_gqa_prefill_workspace_size", "dsa_sparse_gqa_prefill",
    "dsa_decode_step_workspace_size", "dsa_decode_step",
    "swa_attention_workspace_size", "swa_attention", "swa_ring_append",
    "dsa_profile_enable", "dsa_profile_kernel_stats",
    "dsa_cache_write_paged", "dsa_compress_regions_paged", "dsa_score_topk_paged", "dsa_sparse_gqa_decode_paged",
    "dsa_sparse_gqa_prefill_paged", "dsa_decode_step_paged",
    "dsa_cache_write_fp8", "dsa_sparse_gqa_decode_fp8", "dsa_sparse_gqa_prefill_fp8", "dsa_decode_step_fp8",
    "dsa_cache_write_fp8_paged", "dsa_sparse_gqa_decode_fp8_paged", "dsa_sparse_gqa_prefill_fp8_paged",
    "dsa_decode_step_fp8_paged", "dsa_sparse_gqa_prefill_merged", "dsa_sparse_gqa_prefill_merged_paged",
    "dsa_rope_config_default", "dsa_indexer_workspace_size", "dsa_indexer_project", "dsa_rope_qk",
    "dsa_decode_step_noalloc", "swa_decode_step",
]


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class Geometry(ctypes.Structure):
    _fields_ = [("region_size", ctypes.c_int32), ("proxy_dim", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class RopeConfig(ctypes.Structure):
    _fields_ = [("rot_dims", ctypes.c_int32), ("theta", ctypes.c_float), ("factor", ctypes.c_float),
                ("low_freq_factor", ctypes.c_float), ("high_freq_factor", ctypes.c_float),
                ("original_max_pos", ctypes.c_int32)]


class PageTable(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


PAGE_POSITIONS = 128  # positions per page of the paged caches (16 regions, one summary tile)


class Pages:
    """A block table [n_seqs][max_pages] int32 on the device plus the pool size; keeps the tensor alive
    for as long as the C struct that points at it."""

    def __init__(self, block_table: torch.Tensor, n_pages: int):
        if block_table.dim() != 2 or block_table.dtype != torch.int32:
            raise TypeError("block_table must be a 2-D int32 tensor [n_seqs][max_pages]")
        self.table = block_table.contiguous()
        self.n_seqs, self.max_pages = self.table.shape
        self.n_pages = int(n_pages)
        self.struct = PageTable(ctypes.c_void_p(self.table.data_ptr()), self.max_pages, self.n_pages)

    @property
    def tcap(self) -> int:
        return self.max_pages * PAGE_POSITIONS


def paged_pools(n_pages: int, device="cuda", index_k: bool = True):
    """Zero-filled pools of n_pages pages in the documented paged layouts."""
    z = lambda n, dt: torch.zeros(n, dtype=dt, device=device)
    per = PAGE_POSITIONS * GROUPS
    return {"k": z(n_pages * per * HEAD_DIM, torch.bfloat16), "v": z(n_pages * per * HEAD_DIM, torch.bfloat16),
            "ik": z(n_pages * per * PROXY, torch.bfloat16) if index_k else None,
            "summ": z(n_pages * GROUPS * 4096, torch.uint8),
            "scale": z(n_pages * GROUPS * (PAGE_POSITIONS // REGION), torch.float32)}


_lib = None


def load() -> ctypes.CDLL:
    """Loads the HIP library; raises if it is not built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library {LIB_PATH} is missing; build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    G = ctypes.POINTER(Geometry)
    L.dsa_geometry_default.argtypes = [G]
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_cache_write.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, vp]
    L.dsa_compress_regions.argtypes = [G, i32, vp, i64, vp, vp, i32, vp, vp, vp]
    L.dsa_score_topk_workspace_size.argtypes = [G, i32, i32]
    L.dsa_score_topk_workspace_size.restype = sz
    L.dsa_score_topk.argtypes = [G, i32, vp, vp, vp, vp, i32, vp, vp, i64, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_workspace_size.argtypes = [G, i32]
    L.dsa_sparse_gqa_workspace_size.restype = sz
    L.dsa_sparse_gqa_decode.argtypes = [G, i32, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_workspace_size.argtypes = [G, i32]
    L.dsa_sparse_gqa_prefill_workspace_size.restype = sz
    L.dsa_sparse_gqa_prefill.argtypes = [G, i32, vp, vp, vp, i32, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.dsa_decode_step_workspace_size.argtypes = [G, i32, i32]
    L.dsa_decode_step_workspace_size.restype = sz
    L.dsa_decode_step.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_decode_step_noalloc.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp]
    L.swa_attention_workspace_size.argtypes = [G, i32, i32, i32]
    L.swa_attention_workspace_size.restype = sz
    L.swa_attention.argtypes = [G, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.swa_ring_append.argtypes = [G, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.swa_decode_step.argtypes = [G, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    P = ctypes.POINTER(PageTable)
    L.dsa_cache_write_paged.argtypes = [G, i32, vp, vp, vp, vp, vp, P, i32, vp, vp, vp, vp]
    L.dsa_compress_regions_paged.argtypes = [G, i32, P, vp, vp, vp, i32, vp, vp, vp]
    L.dsa_score_topk_paged.argtypes = [G, i32, vp, vp, vp, vp, i32, P, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_decode_paged.argtypes = [G, i32, vp, P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_paged.argtypes = [G, i32, vp, vp, vp, i32, P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_decode_step_paged.argtypes = [G, i32, vp, vp, vp, P, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_cache_write_fp8.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, vp, i32, i64, vp]
    L.dsa_sparse_gqa_decode_fp8.argtypes = [G, i32, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_fp8.argtypes = [G, i32, vp, vp, vp, i32, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.dsa_decode_step_fp8.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp, sz,
                                      vp]
    R = ctypes.POINTER(RopeConfig)
    L.dsa_rope_config_default.argtypes = [R]
    L.dsa_indexer_workspace_size.argtypes = [i32, i32]
    L.dsa_indexer_workspace_size.restype = sz
    L.dsa_indexer_project.argtypes = [R, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_rope_qk.argtypes = [R, i32, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_merged.argtypes = [G, i32, vp, vp, vp, i32, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_merged_paged.argtypes = [G, i32, vp, vp, vp, i32, P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_cache_write_fp8_paged.argtypes = [G, i32, vp, vp, vp, vp, P, i32, vp, vp, vp, vp]
    L.dsa_sparse_gqa_decode_fp8_paged.argtypes = [G, i32, vp, P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_gqa_prefill_fp8_paged.argtypes = [G, i32, vp, vp, vp, i32, P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_decode_step_fp8_paged.argtypes = [G, i32, vp, vp, vp, P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                            sz, vp]
    L.dsa_profile_enable.argtypes = [ctypes.c_int]
    L.dsa_profile_kernel_stats.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int32)]
    for name in ENTRY_POINTS:
        f = getattr(L, name)
        if f.restype is ctypes.c_int:  # default
            f.restype = ctypes.c_int
    _lib = L
    return L


def geometry(topk: int = MAX_TOPK, softmax_scale: float | None = None) -> Geometry:
    g = Geometry()
    load().dsa_geometry_default(ctypes.byref(g))
    g.topk = topk
    if softmax_scale is not None:
        g.softmax_scale = softmax_scale
    return g


def _check(status: int):
    if status != 0:
        L = load()
        raise DsaError(status, f"{L.dsa_status_string(status).decode()}: {L.dsa_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _numel_at_least(t, n, name):
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {n}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled, 256-byte aligned device buffer (uint8) of at least nbytes (no entry point
    depends on the contents of its workspace on entry)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------------------------------------
def dsa_cache_write(geom, tok_seq, tok_pos, k_new, v_new, ik_new, k_cache, v_cache, ik_cache, n_seqs, tcap,
                    stream=None):
    n = tok_seq.numel()
    for t, nm in ((tok_seq, "tok_seq"), (tok_pos, "tok_pos")):
        _dt(t, torch.int32, nm)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (ik_new, "ik_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache"), (ik_cache, "ik_cache")):
        _dt(t, torch.bfloat16, nm)
    _numel_at_least(k_new, n * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, n * GROUPS * HEAD_DIM, "v_new")
    _numel_at_least(k_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "k_cache")
    _numel_at_least(v_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "v_cache")
    if ik_new is not None:
        _numel_at_least(ik_new, n * GROUPS * PROXY, "ik_new")
        _numel_at_least(ik_cache, n_seqs * GROUPS * tcap * PROXY, "ik_cache")
    _check(load().dsa_cache_write(ctypes.byref(geom), n, _ptr(tok_seq), _ptr(tok_pos), _ptr(k_new), _ptr(v_new),
                                  _ptr(ik_new), _ptr(k_cache), _ptr(v_cache), _ptr(ik_cache), n_seqs, tcap,
                                  _stream(stream)))


def dsa_compress_regions(geom, index_k, tcap, region_begin, region_end, max_span, summ, scale, stream=None):
    batch = region_begin.numel()
    _dt(index_k, torch.bfloat16, "index_k")
    _dt(region_begin, torch.int32, "region_begin")
    _dt(region_end, torch.int32, "region_end")
    _dt(summ, torch.uint8, "summ")
    _dt(scale, torch.float32, "scale")
    _numel_at_least(index_k, batch * GROUPS * tcap * PROXY, "index_k")
    _numel_at_least(summ, batch * GROUPS * (tcap // REGION) * PROXY, "summ")
    _numel_at_least(scale, batch * GROUPS * (tcap // REGION), "scale")
    _check(load().dsa_compress_regions(ctypes.byref(geom), batch, _ptr(index_k), tcap, _ptr(region_begin),
                                       _ptr(region_end), max_span, _ptr(summ), _ptr(scale), _stream(stream)))


def dsa_score_topk_workspace_size(geom, n_queries, max_regions) -> int:
    return int(load().dsa_score_topk_workspace_size(ctypes.byref(geom), n_queries, max_regions))


def dsa_score_topk(geom, index_q, z, q_seq, q_pos, n_seqs, summ, scale, tcap, max_regions, sel, n_sel,
                   scores_out=None, workspace=None, stream=None):
    nq = q_seq.numel()
    _dt(index_q, torch.bfloat16, "index_q")
    _dt(z, torch.float32, "z")
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(summ, torch.uint8, "summ")
    _dt(scale, torch.float32, "scale")
    _dt(scores_out, torch.float32, "scores_out")
    _numel_at_least(index_q, nq * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, nq * IDX_HEADS, "z")
    _numel_at_least(summ, n_seqs * GROUPS * (tcap // REGION) * PROXY, "summ")
    _numel_at_least(scale, n_seqs * GROUPS * (tcap // REGION), "scale")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _numel_at_least(scores_out, nq * GROUPS * max_regions, "scores_out")
    need = dsa_score_topk_workspace_size(geom, nq, max_regions)
    if workspace is None:
        workspace = globals()["workspace"](need, q_seq.device)
    _check(load().dsa_score_topk(ctypes.byref(geom), nq, _ptr(index_q), _ptr(z), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                 _ptr(summ), _ptr(scale), tcap, max_regions, _ptr(sel), _ptr(n_sel),
                                 _ptr(scores_out), _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_sparse_gqa_workspace_size(geom, batch) -> int:
    return int(load().dsa_sparse_gqa_workspace_size(ctypes.byref(geom), batch))


def dsa_sparse_gqa_decode(geom, q, k_cache, v_cache, tcap, seq_len, sel, n_sel, out, workspace=None, stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(k_cache, batch * GROUPS * tcap * HEAD_DIM, "k_cache")
    _numel_at_least(v_cache, batch * GROUPS * tcap * HEAD_DIM, "v_cache")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_workspace_size(geom, batch), q.device)
    _check(load().dsa_sparse_gqa_decode(ctypes.byref(geom), batch, _ptr(q), _ptr(k_cache), _ptr(v_cache), tcap,
                                        _ptr(seq_len), _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))


def dsa_decode_step_workspace_size(geom, batch, max_regions) -> int:
    return int(load().dsa_decode_step_workspace_size(ctypes.byref(geom), batch, max_regions))


def _decode_step_checks(geom, q, index_q, z, index_k, k_cache, v_cache, tcap, seq_len, summ, scale, sel, n_sel,
                        out):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (index_q, "index_q"), (index_k, "index_k"), (k_cache, "k_cache"),
                  (v_cache, "v_cache"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(z, torch.float32, "z")
    _dt(summ, torch.uint8, "summ")
    _dt(scale, torch.float32, "scale")
    R = tcap // REGION
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(index_q, batch * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, batch * IDX_HEADS, "z")
    _numel_at_least(index_k, batch * GROUPS * tcap * PROXY, "index_k")
    _numel_at_least(k_cache, batch * GROUPS * tcap * HEAD_DIM, "k_cache")
    _numel_at_least(v_cache, batch * GROUPS * tcap * HEAD_DIM, "v_cache")
    _numel_at_least(summ, batch * GROUPS * R * PROXY, "summ")
    _numel_at_least(scale, batch * GROUPS * R, "scale")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    return batch


def dsa_decode_step(geom, q, index_q, z, index_k, k_cache, v_cache, tcap, seq_len, summ, scale, max_regions, sel,
                    n_sel, out, workspace=None, stream=None):
    batch = _decode_step_checks(geom, q, index_q, z, index_k, k_cache, v_cache, tcap, seq_len, summ, scale, sel,
                                n_sel, out)
    if workspace is None:
        workspace = globals()["workspace"](dsa_decode_step_workspace_size(geom, batch, max_regions), q.device)
    _check(load().dsa_decode_step(ctypes.byref(geom), batch, _ptr(q), _ptr(index_q), _ptr(z), _ptr(index_k),
                                  _ptr(k_cache), _ptr(v_cache), tcap, _ptr(seq_len), _ptr(summ), _ptr(scale),
                                  max_regions, _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))


def dsa_decode_step_noalloc(geom, q, index_q, z, index_k, k_cache, v_cache, tcap, seq_len, summ, scale, max_regions,
                            sel, n_sel, out, stream=None):
    """dsa_decode_step with the library's static scratch area as its workspace (nothing allocated)."""
    batch = _decode_step_checks(geom, q, index_q, z, index_k, k_cache, v_cache, tcap, seq_len, summ, scale, sel,
                                n_sel, out)
    _check(load().dsa_decode_step_noalloc(ctypes.byref(geom), batch, _ptr(q), _ptr(index_q), _ptr(z), _ptr(index_k),
                                          _ptr(k_cache), _ptr(v_cache), tcap, _ptr(seq_len), _ptr(summ), _ptr(scale),
                                          max_regions, _ptr(sel), _ptr(n_sel), _ptr(out), _stream(stream)))


def dsa_sparse_gqa_prefill_workspace_size(geom, n_queries) -> int:
    return int(load().dsa_sparse_gqa_prefill_workspace_size(ctypes.byref(geom), n_queries))


def dsa_sparse_gqa_prefill(geom, q, q_seq, q_pos, n_seqs, k_cache, v_cache, tcap, sel, n_sel, out, workspace=None,
                           stream=None):
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(k_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "k_cache")
    _numel_at_least(v_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "v_cache")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                         _ptr(k_cache), _ptr(v_cache), tcap, _ptr(sel), _ptr(n_sel), _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_sparse_gqa_prefill_merged(geom, q, q_seq, q_pos, n_seqs, k_cache, v_cache, tcap, sel, n_sel, out,
                                  workspace=None, stream=None):
    """Neighbour-merged prefill: the result of dsa_sparse_gqa_prefill, 2 consecutive queries sharing each
    region of their selections' union."""
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (out, "out"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _numel_at_least(k_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "k_cache")
    _numel_at_least(v_cache, n_seqs * GROUPS * tcap * HEAD_DIM, "v_cache")
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill_merged(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                                _ptr(k_cache), _ptr(v_cache), tcap, _ptr(sel), _ptr(n_sel),
                                                _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))


def swa_attention_workspace_size(geom, window, n_seqs, max_new_per_seq) -> int:
    return int(load().swa_attention_workspace_size(ctypes.byref(geom), window, n_seqs, max_new_per_seq))


def _swa_common(n_seqs, max_new, seq_pos0, seq_row0, k_new, v_new, k_ring, v_ring, window):
    _dt(seq_pos0, torch.int32, "seq_pos0")
    _dt(seq_row0, torch.int32, "seq_row0")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_ring, "k_ring"), (v_ring, "v_ring")):
        _dt(t, torch.bfloat16, nm)
    _numel_at_least(seq_pos0, n_seqs, "seq_pos0")
    _numel_at_least(seq_row0, n_seqs + 1, "seq_row0")
    _numel_at_least(k_ring, n_seqs * GROUPS * window * HEAD_DIM, "k_ring")
    _numel_at_least(v_ring, n_seqs * GROUPS * window * HEAD_DIM, "v_ring")
    rows = n_seqs * max_new
    _numel_at_least(k_new, rows * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, rows * GROUPS * HEAD_DIM, "v_new")


def swa_attention(geom, window, max_new_per_seq, seq_pos0, seq_row0, q, k_new, v_new, k_ring, v_ring, out,
                  workspace=None, stream=None):
    n_seqs = seq_pos0.numel()
    _swa_common(n_seqs, max_new_per_seq, seq_pos0, seq_row0, k_new, v_new, k_ring, v_ring, window)
    _dt(q, torch.bfloat16, "q")
    _dt(out, torch.bfloat16, "out")
    _numel_at_least(q, n_seqs * max_new_per_seq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, n_seqs * max_new_per_seq * Q_HEADS * HEAD_DIM, "out")
    if workspace is None:
        workspace = globals()["workspace"](swa_attention_workspace_size(geom, window, n_seqs, max_new_per_seq),
                                           q.device)
    _check(load().swa_attention(ctypes.byref(geom), window, n_seqs, max_new_per_seq, _ptr(seq_pos0),
                                _ptr(seq_row0), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring),
                                _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))


def swa_ring_append(geom, window, max_new_per_seq, seq_pos0, seq_row0, k_new, v_new, k_ring, v_ring, stream=None):
    n_seqs = seq_pos0.numel()
    _swa_common(n_seqs, max_new_per_seq, seq_pos0, seq_row0, k_new, v_new, k_ring, v_ring, window)
    _check(load().swa_ring_append(ctypes.byref(geom), window, n_seqs, max_new_per_seq, _ptr(seq_pos0),
                                  _ptr(seq_row0), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring),
                                  _stream(stream)))


def swa_decode_step(geom, window, seq_pos, q, k_new, v_new, k_ring, v_ring, out, stream=None):
    """Sliding-window decode (one new token per sequence, row s) followed by the ring append."""
    n_seqs = seq_pos.numel()
    _dt(seq_pos, torch.int32, "seq_pos")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_ring, "k_ring"), (v_ring, "v_ring"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    _numel_at_least(k_ring, n_seqs * GROUPS * window * HEAD_DIM, "k_ring")
    _numel_at_least(v_ring, n_seqs * GROUPS * window * HEAD_DIM, "v_ring")
    _numel_at_least(k_new, n_seqs * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, n_seqs * GROUPS * HEAD_DIM, "v_new")
    _numel_at_least(q, n_seqs * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, n_seqs * Q_HEADS * HEAD_DIM, "out")
    _check(load().swa_decode_step(ctypes.byref(geom), window, n_seqs, _ptr(seq_pos), _ptr(q), _ptr(k_new),
                                  _ptr(v_new), _ptr(k_ring), _ptr(v_ring), _ptr(out), _stream(stream)))


# ---- paged caches ----------------------------------------------------------------------------
def _pools_check(pages: Pages, k_pool, v_pool, ik_pool=None, summ_pool=None, scale_pool=None):
    per = pages.n_pages * PAGE_POSITIONS * GROUPS
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool"), (ik_pool, "ik_pool")):
        _dt(t, torch.bfloat16, nm)
    _numel_at_least(k_pool, per * HEAD_DIM, "k_pool")
    _numel_at_least(v_pool, per * HEAD_DIM, "v_pool")
    _numel_at_least(ik_pool, per * PROXY, "ik_pool")
    _dt(summ_pool, torch.uint8, "summ_pool")
    _dt(scale_pool, torch.float32, "scale_pool")
    _numel_at_least(summ_pool, pages.n_pages * GROUPS * 4096, "summ_pool")
    _numel_at_least(scale_pool, pages.n_pages * GROUPS * (PAGE_POSITIONS // REGION), "scale_pool")


def _pages(pages: Pages, n_seqs: int):
    if pages.n_seqs < n_seqs:
        raise ValueError(f"block table has {pages.n_seqs} rows, needs {n_seqs}")
    if not pages.table.is_cuda:
        raise ValueError("the block table must live on the GPU")
    return ctypes.byref(pages.struct)


def dsa_cache_write_paged(geom, tok_seq, tok_pos, k_new, v_new, ik_new, pages: Pages, n_seqs, k_pool, v_pool,
                          ik_pool=None, stream=None):
    n = tok_seq.numel()
    for t, nm in ((tok_seq, "tok_seq"), (tok_pos, "tok_pos")):
        _dt(t, torch.int32, nm)
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (ik_new, "ik_new")):
        _dt(t, torch.bfloat16, nm)
    _numel_at_least(k_new, n * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, n * GROUPS * HEAD_DIM, "v_new")
    _numel_at_least(ik_new, n * GROUPS * PROXY, "ik_new")
    _pools_check(pages, k_pool, v_pool, ik_pool)
    _check(load().dsa_cache_write_paged(ctypes.byref(geom), n, _ptr(tok_seq), _ptr(tok_pos), _ptr(k_new),
                                        _ptr(v_new), _ptr(ik_new), _pages(pages, n_seqs), n_seqs, _ptr(k_pool),
                                        _ptr(v_pool), _ptr(ik_pool), _stream(stream)))


def dsa_compress_regions_paged(geom, pages: Pages, ik_pool, region_begin, region_end, max_span, summ_pool,
                               scale_pool, stream=None):
    batch = region_begin.numel()
    _dt(region_begin, torch.int32, "region_begin")
    _dt(region_end, torch.int32, "region_end")
    _dt(ik_pool, torch.bfloat16, "ik_pool")
    _numel_at_least(ik_pool, pages.n_pages * PAGE_POSITIONS * GROUPS * PROXY, "ik_pool")
    _pools_check(pages, None, None, None, summ_pool, scale_pool)
    _check(load().dsa_compress_regions_paged(ctypes.byref(geom), batch, _pages(pages, batch), _ptr(ik_pool),
                                             _ptr(region_begin), _ptr(region_end), max_span, _ptr(summ_pool),
                                             _ptr(scale_pool), _stream(stream)))


def dsa_score_topk_paged(geom, index_q, z, q_seq, q_pos, n_seqs, pages: Pages, summ_pool, scale_pool, max_regions,
                         sel, n_sel, scores_out=None, workspace=None, stream=None):
    nq = q_seq.numel()
    _dt(index_q, torch.bfloat16, "index_q")
    _dt(z, torch.float32, "z")
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(scores_out, torch.float32, "scores_out")
    _numel_at_least(index_q, nq * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, nq * IDX_HEADS, "z")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _numel_at_least(scores_out, nq * GROUPS * max_regions, "scores_out")
    _pools_check(pages, None, None, None, summ_pool, scale_pool)
    if workspace is None:
        workspace = globals()["workspace"](dsa_score_topk_workspace_size(geom, nq, max_regions), q_seq.device)
    _check(load().dsa_score_topk_paged(ctypes.byref(geom), nq, _ptr(index_q), _ptr(z), _ptr(q_seq), _ptr(q_pos),
                                       n_seqs, _pages(pages, n_seqs), _ptr(summ_pool), _ptr(scale_pool), max_regions,
                                       _ptr(sel), _ptr(n_sel), _ptr(scores_out), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))


def dsa_sparse_gqa_decode_paged(geom, q, pages: Pages, k_pool, v_pool, seq_len, sel, n_sel, out, workspace=None,
                                stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _pools_check(pages, k_pool, v_pool)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_workspace_size(geom, batch), q.device)
    _check(load().dsa_sparse_gqa_decode_paged(ctypes.byref(geom), batch, _ptr(q), _pages(pages, batch),
                                              _ptr(k_pool), _ptr(v_pool), _ptr(seq_len), _ptr(sel), _ptr(n_sel),
                                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_sparse_gqa_prefill_paged(geom, q, q_seq, q_pos, n_seqs, pages: Pages, k_pool, v_pool, sel, n_sel, out,
                                 workspace=None, stream=None):
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _pools_check(pages, k_pool, v_pool)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill_paged(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                               _pages(pages, n_seqs), _ptr(k_pool), _ptr(v_pool), _ptr(sel),
                                               _ptr(n_sel), _ptr(out), _ptr(workspace), workspace.numel(),
                                               _stream(stream)))


def dsa_sparse_gqa_prefill_merged_paged(geom, q, q_seq, q_pos, n_seqs, pages: Pages, k_pool, v_pool, sel, n_sel,
                                        out, workspace=None, stream=None):
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _pools_check(pages, k_pool, v_pool)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill_merged_paged(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos),
                                                      n_seqs, _pages(pages, n_seqs), _ptr(k_pool), _ptr(v_pool),
                                                      _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(workspace),
                                                      workspace.numel(), _stream(stream)))


def dsa_decode_step_paged(geom, q, index_q, z, pages: Pages, ik_pool, k_pool, v_pool, seq_len, summ_pool,
                          scale_pool, max_regions, sel, n_sel, out, workspace=None, stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (index_q, "index_q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(z, torch.float32, "z")
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(index_q, batch * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, batch * IDX_HEADS, "z")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _pools_check(pages, k_pool, v_pool, ik_pool, summ_pool, scale_pool)
    if workspace is None:
        workspace = globals()["workspace"](dsa_decode_step_workspace_size(geom, batch, max_regions), q.device)
    _check(load().dsa_decode_step_paged(ctypes.byref(geom), batch, _ptr(q), _ptr(index_q), _ptr(z),
                                        _pages(pages, batch), _ptr(ik_pool), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(seq_len), _ptr(summ_pool), _ptr(scale_pool), max_regions, _ptr(sel),
                                        _ptr(n_sel), _ptr(out), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))


# ---- FP8 K/V caches ---------------------------------------------------------------------------
def fp8_caches(n_seqs: int, tcap: int, device="cuda"):
    """Zero-filled FP8 K/V caches (k8, v8 uint8 and kv_scale fp32) of n_seqs sequences, capacity tcap."""
    R = tcap // REGION
    return (torch.zeros(n_seqs * GROUPS * tcap * HEAD_DIM, dtype=torch.uint8, device=device),
            torch.zeros(n_seqs * GROUPS * tcap * HEAD_DIM, dtype=torch.uint8, device=device),
            torch.zeros(n_seqs * GROUPS * R * 16, dtype=torch.float32, device=device))


def _fp8_check(k8, v8, kvs, n_seqs, tcap):
    _dt(k8, torch.uint8, "k8_cache")
    _dt(v8, torch.uint8, "v8_cache")
    _dt(kvs, torch.float32, "kv_scale")
    _numel_at_least(k8, n_seqs * GROUPS * tcap * HEAD_DIM, "k8_cache")
    _numel_at_least(v8, n_seqs * GROUPS * tcap * HEAD_DIM, "v8_cache")
    _numel_at_least(kvs, n_seqs * GROUPS * (tcap // REGION) * 16, "kv_scale")


def dsa_cache_write_fp8(geom, tok_seq, tok_pos, k_new, v_new, k8, v8, kvs, n_seqs, tcap, stream=None):
    n = tok_seq.numel()
    for t, nm in ((tok_seq, "tok_seq"), (tok_pos, "tok_pos")):
        _dt(t, torch.int32, nm)
    _dt(k_new, torch.bfloat16, "k_new")
    _dt(v_new, torch.bfloat16, "v_new")
    _numel_at_least(k_new, n * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, n * GROUPS * HEAD_DIM, "v_new")
    _fp8_check(k8, v8, kvs, n_seqs, tcap)
    _check(load().dsa_cache_write_fp8(ctypes.byref(geom), n, _ptr(tok_seq), _ptr(tok_pos), _ptr(k_new), _ptr(v_new),
                                      _ptr(k8), _ptr(v8), _ptr(kvs), n_seqs, tcap, _stream(stream)))


def dsa_sparse_gqa_decode_fp8(geom, q, k8, v8, kvs, tcap, seq_len, sel, n_sel, out, workspace=None, stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _fp8_check(k8, v8, kvs, batch, tcap)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_workspace_size(geom, batch), q.device)
    _check(load().dsa_sparse_gqa_decode_fp8(ctypes.byref(geom), batch, _ptr(q), _ptr(k8), _ptr(v8), _ptr(kvs), tcap,
                                            _ptr(seq_len), _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(workspace),
                                            workspace.numel(), _stream(stream)))


def dsa_sparse_gqa_prefill_fp8(geom, q, q_seq, q_pos, n_seqs, k8, v8, kvs, tcap, sel, n_sel, out, workspace=None,
                               stream=None):
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _fp8_check(k8, v8, kvs, n_seqs, tcap)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill_fp8(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                             _ptr(k8), _ptr(v8), _ptr(kvs), tcap, _ptr(sel), _ptr(n_sel), _ptr(out),
                                             _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_decode_step_fp8(geom, q, index_q, z, index_k, k8, v8, kvs, tcap, seq_len, summ, scale, max_regions, sel,
                        n_sel, out, workspace=None, stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (index_q, "index_q"), (index_k, "index_k"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(z, torch.float32, "z")
    _dt(summ, torch.uint8, "summ")
    _dt(scale, torch.float32, "scale")
    R = tcap // REGION
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(index_q, batch * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, batch * IDX_HEADS, "z")
    _numel_at_least(index_k, batch * GROUPS * tcap * PROXY, "index_k")
    _numel_at_least(summ, batch * GROUPS * R * PROXY, "summ")
    _numel_at_least(scale, batch * GROUPS * R, "scale")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _fp8_check(k8, v8, kvs, batch, tcap)
    if workspace is None:
        workspace = globals()["workspace"](dsa_decode_step_workspace_size(geom, batch, max_regions), q.device)
    _check(load().dsa_decode_step_fp8(ctypes.byref(geom), batch, _ptr(q), _ptr(index_q), _ptr(z), _ptr(index_k),
                                      _ptr(k8), _ptr(v8), _ptr(kvs), tcap, _ptr(seq_len), _ptr(summ), _ptr(scale),
                                      max_regions, _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(stream)))


# ---- FP8 K/V caches in pages ------------------------------------------------------------------
def fp8_pools(n_pages: int, device="cuda"):
    """Zero-filled paged FP8 pools (k8, v8 uint8 and kv_scale fp32) of n_pages pages."""
    per = n_pages * GROUPS * PAGE_POSITIONS
    return (torch.zeros(per * HEAD_DIM, dtype=torch.uint8, device=device),
            torch.zeros(per * HEAD_DIM, dtype=torch.uint8, device=device),
            torch.zeros(per // REGION * 16, dtype=torch.float32, device=device))


def _fp8_pools_check(pages: Pages, k8, v8, kvs):
    _fp8_check(k8, v8, kvs, 1, pages.n_pages * PAGE_POSITIONS)


def dsa_cache_write_fp8_paged(geom, tok_seq, tok_pos, k_new, v_new, pages: Pages, n_seqs, k8, v8, kvs, stream=None):
    n = tok_seq.numel()
    for t, nm in ((tok_seq, "tok_seq"), (tok_pos, "tok_pos")):
        _dt(t, torch.int32, nm)
    _dt(k_new, torch.bfloat16, "k_new")
    _dt(v_new, torch.bfloat16, "v_new")
    _numel_at_least(k_new, n * GROUPS * HEAD_DIM, "k_new")
    _numel_at_least(v_new, n * GROUPS * HEAD_DIM, "v_new")
    _fp8_pools_check(pages, k8, v8, kvs)
    _check(load().dsa_cache_write_fp8_paged(ctypes.byref(geom), n, _ptr(tok_seq), _ptr(tok_pos), _ptr(k_new),
                                            _ptr(v_new), _pages(pages, n_seqs), n_seqs, _ptr(k8), _ptr(v8), _ptr(kvs),
                                            _stream(stream)))


def dsa_sparse_gqa_decode_fp8_paged(geom, q, pages: Pages, k8, v8, kvs, seq_len, sel, n_sel, out, workspace=None,
                                    stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _fp8_pools_check(pages, k8, v8, kvs)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_workspace_size(geom, batch), q.device)
    _check(load().dsa_sparse_gqa_decode_fp8_paged(ctypes.byref(geom), batch, _ptr(q), _pages(pages, batch), _ptr(k8),
                                                  _ptr(v8), _ptr(kvs), _ptr(seq_len), _ptr(sel), _ptr(n_sel),
                                                  _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_sparse_gqa_prefill_fp8_paged(geom, q, q_seq, q_pos, n_seqs, pages: Pages, k8, v8, kvs, sel, n_sel, out,
                                     workspace=None, stream=None):
    nq = q_seq.numel()
    for t, nm in ((q, "q"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((q_seq, "q_seq"), (q_pos, "q_pos"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _numel_at_least(q, nq * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, nq * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(sel, nq * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, nq * GROUPS, "n_sel")
    _fp8_pools_check(pages, k8, v8, kvs)
    if workspace is None:
        workspace = globals()["workspace"](dsa_sparse_gqa_prefill_workspace_size(geom, nq), q.device)
    _check(load().dsa_sparse_gqa_prefill_fp8_paged(ctypes.byref(geom), nq, _ptr(q), _ptr(q_seq), _ptr(q_pos), n_seqs,
                                                   _pages(pages, n_seqs), _ptr(k8), _ptr(v8), _ptr(kvs), _ptr(sel),
                                                   _ptr(n_sel), _ptr(out), _ptr(workspace), workspace.numel(),
                                                   _stream(stream)))


def dsa_decode_step_fp8_paged(geom, q, index_q, z, pages: Pages, ik_pool, k8, v8, kvs, seq_len, summ_pool,
                              scale_pool, max_regions, sel, n_sel, out, workspace=None, stream=None):
    batch = seq_len.numel()
    for t, nm in ((q, "q"), (index_q, "index_q"), (ik_pool, "ik_pool"), (out, "out")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((seq_len, "seq_len"), (sel, "sel"), (n_sel, "n_sel")):
        _dt(t, torch.int32, nm)
    _dt(z, torch.float32, "z")
    _numel_at_least(q, batch * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(out, batch * Q_HEADS * HEAD_DIM, "out")
    _numel_at_least(index_q, batch * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(z, batch * IDX_HEADS, "z")
    _numel_at_least(ik_pool, pages.n_pages * PAGE_POSITIONS * GROUPS * PROXY, "ik_pool")
    _numel_at_least(sel, batch * GROUPS * geom.topk, "sel")
    _numel_at_least(n_sel, batch * GROUPS, "n_sel")
    _pools_check(pages, None, None, None, summ_pool, scale_pool)
    _fp8_pools_check(pages, k8, v8, kvs)
    if workspace is None:
        workspace = globals()["workspace"](dsa_decode_step_workspace_size(geom, batch, max_regions), q.device)
    _check(load().dsa_decode_step_fp8_paged(ctypes.byref(geom), batch, _ptr(q), _ptr(index_q), _ptr(z),
                                            _pages(pages, batch), _ptr(ik_pool), _ptr(k8), _ptr(v8), _ptr(kvs),
                                            _ptr(seq_len), _ptr(summ_pool), _ptr(scale_pool), max_regions, _ptr(sel),
                                            _ptr(n_sel), _ptr(out), _ptr(workspace), workspace.numel(),
                                            _stream(stream)))


# ---- indexer front-end and the attention's partial RoPE ---------------------------------------
IDX_PROJ_ROWS = (IDX_HEADS + GROUPS) * PROXY + IDX_HEADS  # weight rows: index_q heads, index_k groups, z


def rope_config(**override) -> RopeConfig:
    """The library's default rotation settings (pages' llama3 values; theta 10000 and factor 8 as
    stand-ins), with fields overridden by keyword."""
    c = RopeConfig()
    _check(load().dsa_rope_config_default(ctypes.byref(c)))
    for k, v in override.items():
        setattr(c, k, v)
    return c


def dsa_indexer_workspace_size(n_tokens, hidden=0) -> int:
    return int(load().dsa_indexer_workspace_size(n_tokens, hidden))


def dsa_indexer_project(rope, x, w, gamma_q, gamma_k, pos, index_q, index_k, z, hidden, workspace=None,
                        stream=None):
    n = pos.numel()
    for t, nm in ((x, "x"), (w, "w"), (index_q, "index_q"), (index_k, "index_k")):
        _dt(t, torch.bfloat16, nm)
    for t, nm in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k"), (z, "z")):
        _dt(t, torch.float32, nm)
    _dt(pos, torch.int32, "pos")
    _numel_at_least(x, n * hidden, "x")
    _numel_at_least(w, IDX_PROJ_ROWS * hidden, "w")
    _numel_at_least(gamma_q, PROXY, "gamma_q")
    _numel_at_least(gamma_k, PROXY, "gamma_k")
    _numel_at_least(index_q, n * IDX_HEADS * PROXY, "index_q")
    _numel_at_least(index_k, n * GROUPS * PROXY, "index_k")
    _numel_at_least(z, n * IDX_HEADS, "z")
    if workspace is None:
        workspace = globals()["workspace"](dsa_indexer_workspace_size(n, hidden), pos.device)
    _check(load().dsa_indexer_project(ctypes.byref(rope), n, hidden, _ptr(x), _ptr(w), _ptr(gamma_q),
                                      _ptr(gamma_k), _ptr(pos), _ptr(index_q), _ptr(index_k), _ptr(z),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_rope_qk(rope, pos, q, k, workspace=None, stream=None):
    n = pos.numel()
    _dt(pos, torch.int32, "pos")
    _dt(q, torch.bfloat16, "q")
    _dt(k, torch.bfloat16, "k")
    _numel_at_least(q, n * Q_HEADS * HEAD_DIM, "q")
    _numel_at_least(k, n * GROUPS * HEAD_DIM, "k")
    if workspace is None:
        workspace = globals()["workspace"](dsa_indexer_workspace_size(n), pos.device)
    _check(load().dsa_rope_qk(ctypes.byref(rope), n, _ptr(pos), _ptr(q), _ptr(k), _ptr(workspace),
                              workspace.numel(), _stream(stream)))


def profile_enable(on: bool = True):
    """Starts (clearing earlier records) or stops per-kernel hipEvent timing inside the library."""
    _check(load().dsa_profile_enable(1 if on else 0))


def profile_kernel_stats(kernel: str):
    """(total milliseconds, launches) of one kernel since profile_enable(True); waits for its events."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    _check(load().dsa_profile_kernel_stats(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)
