"""The Python binding checks shapes, dtypes and row contiguity before it
hands device pointers to the C ABI (the C side sees only pointers and sizes,
so a transposed or mistyped tensor would otherwise be read out of bounds).
Runs without a GPU: tensors here live on the CPU, so a call whose arguments
pass every check still stops at the device check, before any pointer is
marshalled."""
import pytest
import torch

import transformer_depth_wise_amd as tdw

T, d, S, n = 8, 64, 3, 2
bf, f32 = torch.bfloat16, torch.float32


def rows(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def not_on_gpu(fn, *a, **k):
    with pytest.raises(ValueError, match="not on a GPU"):
        fn(*a, **k)


def test_phase1_arguments():
    src, w, lse, out = rows(n, T, d), rows(S, d, dtype=f32), rows(S, T, dtype=f32), rows(S, T, d)
    not_on_gpu(tdw.attnres_phase1, src, n, w, None, 1e-6, out, None, lse)
    with pytest.raises(ValueError, match="src: shape"):
        tdw.attnres_phase1(rows(1, T, d), n, w, None, 1e-6, out, None, lse)       # fewer slabs than sources
    with pytest.raises(ValueError, match="contiguous"):
        tdw.attnres_phase1(rows(n, d, T).transpose(1, 2), n, w, None, 1e-6, out, None, lse)
    with pytest.raises(TypeError, match="w: dtype"):
        tdw.attnres_phase1(src, n, w.to(bf), None, 1e-6, out, None, lse)
    with pytest.raises(ValueError, match="w: shape"):
        tdw.attnres_phase1(src, n, rows(d, S, dtype=f32).t(), None, 1e-6, out, None, lse)
    with pytest.raises(ValueError, match="out"):
        tdw.attnres_phase1(src, n, w, None, 1e-6, rows(S, T, d, dtype=f32), None, lse)  # dtype differs from src
    with pytest.raises(ValueError, match="out"):
        tdw.attnres_phase1(src, n, w, None, 1e-6, rows(S - 1, T, d), None, lse)
    with pytest.raises(ValueError, match="key_gain"):
        tdw.attnres_phase1(src, n, w, rows(S, d + 8, dtype=f32), 1e-6, out, None, lse)
    with pytest.raises(TypeError, match="src: rows"):
        tdw.attnres_phase1(src.to(torch.float16), n, w, None, 1e-6, out, None, lse)
    # slabs sliced along tokens keep contiguous rows: accepted up to the device check
    big = rows(n, 2 * T, d)
    not_on_gpu(tdw.attnres_phase1, big[:, 3:3 + T], n, w, None, 1e-6, out, None, lse)


def test_first_prenorm_arguments():
    src, w, lse, out = rows(n, T, d), rows(S, d, dtype=f32), rows(S, T, dtype=f32), rows(S, T, d)
    not_on_gpu(tdw.attnres_phase1_first_prenorm, src, n, w, None, 1e-6, out, None, lse, None, rows(T, d))
    with pytest.raises(ValueError, match="x_out is required"):
        tdw.attnres_phase1_first_prenorm(src, n, w, None, 1e-6, out, None, lse, None, None)
    with pytest.raises(ValueError, match="h_out: shape"):
        tdw.attnres_phase1_first_prenorm(src, n, w, None, 1e-6, out, None, lse, None, rows(T, d), rows(T + 1, d))
    with pytest.raises(ValueError, match="prenorm_gain"):
        tdw.attnres_phase1_first_prenorm(src, n, w, None, 1e-6, out, None, lse, rows(2 * d, dtype=f32),
                                         rows(T, d))


def test_merge_arguments():
    o, lse, v, w = rows(T, d), rows(T, dtype=f32), rows(T, d), rows(d, dtype=f32)
    p24 = torch.zeros(3 * T * d, dtype=torch.uint8)
    not_on_gpu(tdw.attnres_phase2_merge, o, lse, p24, v, p24, w, None, None, 1e-6, None, rows(T, d))
    not_on_gpu(tdw.attnres_phase2_merge, o, lse, rows(T, d, dtype=f32), v, None, w, None, None, 1e-6, None,
               rows(T, d))
    with pytest.raises(ValueError, match="P24"):
        tdw.attnres_phase2_merge(o, lse, p24[:-1], v, None, w, None, None, 1e-6, None, rows(T, d))
    q16 = torch.zeros(T * d + 2 * T, dtype=torch.int16)
    not_on_gpu(tdw.attnres_phase2_merge, o, lse, q16, v, q16, w, None, None, 1e-6, None, rows(T, d))
    with pytest.raises(ValueError, match="Q16"):      # the row exponents are missing
        tdw.attnres_phase2_merge(o, lse, q16[:T * d], v, None, w, None, None, 1e-6, None, rows(T, d))
    with pytest.raises(TypeError, match="partial_out"):
        tdw.attnres_phase2_merge(o, lse, None, v, rows(T, d), w, None, None, 1e-6, None, rows(T, d))  # bf16 out
    with pytest.raises(TypeError, match="sublayer_prev"):
        tdw.attnres_phase2_merge(o, lse, None, rows(T, d, dtype=f32), None, w, None, None, 1e-6, None, rows(T, d))
    with pytest.raises(ValueError, match="p1_lse"):
        tdw.attnres_phase2_merge(o, rows(T, 2, dtype=f32), None, v, None, w, None, None, 1e-6, None, rows(T, d))
    with pytest.raises(ValueError, match="x_out: rows must be contiguous"):
        tdw.attnres_phase2_merge(o, lse, None, v, None, w, None, None, 1e-6, None, rows(T, 2 * d)[:, ::2])


def test_full_multi_and_accumulate_arguments():
    src, w = rows(n, T, d), rows(d, dtype=f32)
    not_on_gpu(tdw.attnres_full, src, n, w, None, None, 1e-6, rows(T, d), None, rows(T, dtype=f32))
    with pytest.raises(ValueError, match="lse_out"):
        tdw.attnres_full(src, n, w, None, None, 1e-6, rows(T, d), None, rows(T + 1, dtype=f32))
    with pytest.raises(ValueError, match="w is required"):
        tdw.attnres_full(src, n, None, None, None, 1e-6, rows(T, d), None, None)
    o, lse = rows(T, d), rows(T, dtype=f32)
    not_on_gpu(tdw.attnres_phase2_merge_multi, o, lse, None, 0, None, None, None, 1e-6, None, rows(T, d))
    with pytest.raises(ValueError, match="src is required"):
        tdw.attnres_phase2_merge_multi(o, lse, None, 2, w, None, None, 1e-6, None, rows(T, d))
    not_on_gpu(tdw.attnres_block_accumulate, torch.zeros(3 * T * d, dtype=torch.uint8), rows(T, d), rows(T, d))
    with pytest.raises(ValueError, match="out: shape"):
        tdw.attnres_block_accumulate(None, rows(T, d), rows(d, T))
    with pytest.raises(TypeError, match="v2"):
        tdw.attnres_block_accumulate(None, rows(T, d), rows(T, d), v2=rows(T, d, dtype=f32))


def test_backward_arguments():
    src, dx, w, ws = rows(n, T, d), rows(T, d), rows(d, dtype=f32), rows(64, dtype=f32)
    not_on_gpu(tdw.attnres_site_backward, src, n, w, None, None, False, 1e-6, dx, rows(n, T, d),
               rows(d, dtype=f32), None, None, ws)
    with pytest.raises(ValueError, match="dw is required"):
        tdw.attnres_site_backward(src, n, w, None, None, False, 1e-6, dx, rows(n, T, d), None, None, None, ws)
    not_on_gpu(tdw.attnres_site_backward_accumulate, src, n, w, None, None, True, 1e-6, dx,
               rows(n, T, d, dtype=f32), rows(d, dtype=f32), None, rows(d, dtype=f32), ws)
    with pytest.raises(TypeError, match="dsrc"):    # the accumulated gradients are fp32 rows
        tdw.attnres_site_backward_accumulate(src, n, w, None, None, True, 1e-6, dx, rows(n, T, d),
                                             rows(d, dtype=f32), None, None, ws)
    o, lse, G = rows(T, d), rows(T, dtype=f32), rows(T, d)
    c, gp, R = rows(T, dtype=f32), rows(T, dtype=f32), rows(T, d, dtype=f32)
    not_on_gpu(tdw.attnres_phase2_backward, o, lse, None, rows(T, d), w, None, None, 1e-6, dx, R, G, c, gp,
               rows(d, dtype=f32), None, None, ws)
    with pytest.raises(TypeError, match="dpartial"):
        tdw.attnres_phase2_backward(o, lse, None, rows(T, d), w, None, None, 1e-6, dx, rows(T, d), G, c, gp,
                                    None, None, None, ws)
    with pytest.raises(ValueError, match="c_out is required"):
        tdw.attnres_phase2_backward(o, lse, None, None, w, None, None, 1e-6, dx, None, G, None, gp,
                                    None, None, None, ws)
    wS = rows(S, d, dtype=f32)
    gin, dsrc = rows(S, T, d), rows(n, T, d, dtype=f32)
    cS = rows(S, T, dtype=f32)
    not_on_gpu(tdw.attnres_phase1_backward, src, n, wS, None, 1e-6, gin, cS, cS, dsrc, rows(S, d, dtype=f32),
               None, ws, accumulate=True)
    with pytest.raises(ValueError, match="g_in: shape"):
        tdw.attnres_phase1_backward(src, n, wS, None, 1e-6, rows(S - 1, T, d), cS, cS, dsrc,
                                    rows(S, d, dtype=f32), None, ws)
    with pytest.raises(TypeError, match="dsrc"):
        tdw.attnres_phase1_backward(src, n, wS, None, 1e-6, gin, cS, cS, rows(n, T, d),
                                    rows(S, d, dtype=f32), None, ws)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        tdw.attnres_phase1_backward(src, n, wS, None, 1e-6, gin, cS, cS, dsrc, rows(S, d, dtype=f32), None,
                                    rows(64, 2, dtype=f32)[:, 0])
