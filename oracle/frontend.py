"""ORACLE -- test infrastructure, not product code.

Plain fp64 numpy statement of the indexer front-end and of the partial rotary
embedding of the attention's Q/K.  Only ``tests/``, the smoke check and the
benchmark's CPU-baseline leg may use it; it shares nothing with the HIP path.

What it follows:
  * [P2] "Step-5-Preview 如何实现1M长上下文？..." (yfxerp.com/news/376439), section
    索引器打分 + Top-K 选择: the indexer projects the hidden state into index_q /
    index_k / index_z, then normalises them and applies RoPE to part of the
    dimensions; its closing paragraph: llama3-type rope_scaling on the
    full-attention layers only;
  * [P1] (kwkr.cn/news/601179), DSA 稀疏注意力 section, the paragraph after ④:
    llama3-style interpolation with low_freq_factor 1.0 and high_freq_factor
    32.0; partial rotary factor 1/3 on the full-attention layers;
  * [P3] "100 万 token 上下文实测..." (kwkr.cn/news/593658), section 一:
    original_max_position_embeddings 1048576; of the 192-d head about 64
    dimensions rotate.
Readings where the pages are silent (each a parameter here):
  * normalisation = RMSNorm over each 256-d vector, eps 1e-6, one learned gain
    vector for the 16 query heads and one for the 4 key groups;
  * the index vectors rotate their first 64 dimensions (the count the pages
    give for the attention head), pairs (i, i + 32) ("rotate half");
  * base frequencies theta^(-2i/64) with theta = 10000 and llama3 factor 8
    (neither value is on the pages);
  * index_k is one 256-d key per KV group (the summaries are per group); z is
    the plain projection (no activation is named).
Arrays: x [T][H] and weights [N][H] as bf16 bits (uint16), positions int.
"""
from __future__ import annotations

import math

import numpy as np

IDX_HEADS, GROUPS, PROXY, Q_HEADS, HEAD_DIM = 16, 4, 256, 64, 192
ROT_DIMS = 64
THETA = 10000.0
LLAMA3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=32.0, original_max_pos=1048576)
EPS = 1e-6


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def llama3_scale_freq(freq, factor, low_freq_factor, high_freq_factor, original_max_pos):
    """llama3 frequency scaling of one base frequency: wavelengths shorter than
    original_max_pos / high_freq_factor keep their frequency, those longer than
    original_max_pos / low_freq_factor are slowed by `factor`, and in between the
    frequency moves linearly in original_max_pos / wavelength from one to the other."""
    wavelen = 2.0 * math.pi / freq
    high_wavelen = original_max_pos / high_freq_factor
    low_wavelen = original_max_pos / low_freq_factor
    if wavelen < high_wavelen:
        return freq
    if wavelen > low_wavelen:
        return freq / factor
    s = (original_max_pos / wavelen - low_freq_factor) / (high_freq_factor - low_freq_factor)
    return (1.0 - s) * freq / factor + s * freq


def inv_freq(rot_dims=ROT_DIMS, theta=THETA, **llama3) -> np.ndarray:
    """The rot_dims/2 rotation frequencies: theta^(-2i/rot_dims), llama3-scaled."""
    cfg = dict(LLAMA3)
    cfg.update(llama3)
    return np.array([llama3_scale_freq(theta ** (-2.0 * i / rot_dims), **cfg) for i in range(rot_dims // 2)])


def rope(x, pos, freqs, rot_dims=ROT_DIMS):
    """Rotates the first rot_dims of the last axis of x [T][..][C] (fp64) by position pos[t]:
    pair (i, i + rot_dims/2) turns by the angle pos * freqs[i]."""
    x = np.array(x, dtype=np.float64)
    h = rot_dims // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * np.asarray(freqs, dtype=np.float64)[None, :]  # [T][h]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    a, b = x[..., :h].copy(), x[..., h:rot_dims].copy()
    x[..., :h] = a * c - b * s
    x[..., h:rot_dims] = b * c + a * s
    return x


def rms_norm(x, gamma, eps=EPS):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


def indexer_frontend(x_bits, w_bits, gamma_q, gamma_k, pos, rot_dims=ROT_DIMS, theta=THETA, **llama3):
    """Hidden states -> (index_q [T][16][256], index_k [T][4][256], z [T][16]), fp64.
    w rows: 16*256 index_q columns, then 4*256 index_k columns, then 16 z columns."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    y = x @ w.T  # [T][N]
    T = x.shape[0]
    nq, nk = IDX_HEADS * PROXY, GROUPS * PROXY
    fr = inv_freq(rot_dims, theta, **llama3)
    iq = rope(rms_norm(y[:, :nq].reshape(T, IDX_HEADS, PROXY), gamma_q), pos, fr, rot_dims)
    ik = rope(rms_norm(y[:, nq:nq + nk].reshape(T, GROUPS, PROXY), gamma_k), pos, fr, rot_dims)
    z = y[:, nq + nk:nq + nk + IDX_HEADS]
    return iq, ik, z


def rope_qk(q_bits, k_bits, pos, rot_dims=ROT_DIMS, theta=THETA, **llama3):
    """Partial RoPE of the attention's q [T][64][192] and k [T][4][192] (bf16 bits) -> fp64."""
    fr = inv_freq(rot_dims, theta, **llama3)
    return rope(bf16_to_f64(q_bits), pos, fr, rot_dims), rope(bf16_to_f64(k_bits), pos, fr, rot_dims)
