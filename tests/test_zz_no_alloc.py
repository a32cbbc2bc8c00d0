"""dsa_decode_step_noalloc (the decode step over the library's static scratch area) against
dsa_decode_step with a caller workspace: identical selections and outputs, bit for bit, on two calls
in a row (the second with a smaller batch and context, over the scratch the first call left), and
argument checks that reject shapes beyond the static area before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa

import _harness as H

pytestmark = pytest.mark.gpu

G, P, HQ, D = H.G, H.P, H.HQ, H.D


def _inputs(seed, lens, planted):
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, planted)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    return dict(B=B, tcap=tcap, R=R, ik=ik, K=K, V=V, q=q, iq=iq, z=z, lens=H.i32(lens_np), lens_np=lens_np)


def _run(a, noalloc):
    B, tcap, R = a["B"], a["tcap"], a["R"]
    geom = dsa.geometry()
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, a["ik"], tcap, H.i32(np.zeros(B)), H.i32((a["lens_np"] - 1) // 8), R, summ,
                             scale)
    sel = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
    nsel = torch.empty(B * G, dtype=torch.int32, device="cuda")
    out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    f = dsa.dsa_decode_step_noalloc if noalloc else dsa.dsa_decode_step
    f(geom, a["q"], a["iq"], a["z"], a["ik"], a["K"], a["V"], tcap, a["lens"], summ, scale, R, sel, nsel, out)
    return summ, scale, sel, nsel, out


def _same(x, y):
    for u, v, what in zip(x, y, ("summ", "scale", "sel", "nsel", "out")):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), what


def test_noalloc_decode_step_matches_the_workspace_call_twice_in_a_row():
    # first call: the 1M-token batch-4 shape (15 MiB of scratch, decode tile selection)
    big = _inputs(0x0A1, [1 << 20] * 4, planted=True)
    ref1 = _run(big, noalloc=False)
    got1 = _run(big, noalloc=True)
    torch.cuda.synchronize()
    _same(ref1, got1)
    del big, ref1, got1
    # second call, smaller: ragged contexts (partial current regions, p = 0) over the scratch the first
    # call left behind
    small = _inputs(0x0A2, [70001, 9000, 8192, 17, 1], planted=False)
    ref2 = _run(small, noalloc=False)
    got2 = _run(small, noalloc=True)
    torch.cuda.synchronize()
    _same(ref2, got2)


def test_noalloc_decode_step_rejects_shapes_beyond_the_static_area():
    geom = dsa.geometry()
    B, tcap = 64, 1 << 20  # the workspace of this shape exceeds the 64 MiB area
    assert dsa.dsa_decode_step_workspace_size(geom, B, tcap // 8) > 64 << 20
    L = dsa.load()
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    p = dummy.data_ptr()
    rc = L.dsa_decode_step_noalloc(ctypes.byref(geom), B, p, p, p, p, p, p, tcap, p, p, p, tcap // 8, p, p, p,
                                   None)
    assert rc == 2, rc  # DSA_ERR_UNSUPPORTED, before any launch
    assert "static area" in L.dsa_last_error().decode()
