"""The Python binding rejects tensors whose shapes do not match what the
kernels index, before anything reaches the library (the C ABI takes bare
pointers, so a short tensor would be read or written past its end).  CPU
tensors: with a mismatched shape the call must raise ValueError from the
shape check; with matching shapes it gets past that check and stops at the
device check (TypeError), so no kernel is ever launched here."""
import pytest
import torch

import slot_memory_sequence_amd as gsa

B, H, T, D, M = 2, 3, 70, 64, 32


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def f32(*shape):
    return t(*shape, dtype=torch.float32)


def fwd_args():
    return dict(q=t(B, H, T, D), k=t(B, H, T, D), v=t(B, H, T, D), g=t(B, H, T, M))


def test_gsa_fwd_shapes():
    a = fwd_args()
    with pytest.raises(TypeError):  # shapes fine: stops at the device check
        gsa.gsa_fwd(**a)
    for name, bad in (("k", t(B, H, T - 1, D)), ("v", t(B, H + 1, T, D)), ("g", t(B, H, T + 1, M)),
                      ("k", t(B, H, T, D + 8))):
        b = dict(a)
        b[name] = bad
        with pytest.raises(ValueError, match=name):
            gsa.gsa_fwd(**b)
    for kw, bad in (("k0", f32(B, H, M + 1, D)), ("v0", f32(B, H, M, D - 1)), ("out", t(B, H, T, D - 8)),
                    ("k_final", f32(B, H, M, D + 1)), ("v_final", f32(B, 1, M, D))):
        with pytest.raises(ValueError, match=kw):
            gsa.gsa_fwd(**a, **{kw: bad})
    with pytest.raises(ValueError, match="dimensions"):
        gsa.gsa_fwd(t(B, H, T), a["k"], a["v"], a["g"])


def test_gsa_fwd_varlen_shapes():
    cu = [0, 30, 30, 70]
    q, v, g = t(H, 70, D), t(H, 70, D), t(H, 70, M)
    with pytest.raises(TypeError):
        gsa.gsa_fwd_varlen(q, q, v, g, cu)
    with pytest.raises(ValueError, match="cu_seqlens"):
        gsa.gsa_fwd_varlen(q, q, v, g, [0, 30, 60])
    with pytest.raises(ValueError, match="k"):
        gsa.gsa_fwd_varlen(q, t(H, 69, D), v, g, cu)
    with pytest.raises(ValueError, match="k0"):
        gsa.gsa_fwd_varlen(q, q, v, g, cu, k0=f32(2, H, M, D))
    with pytest.raises(ValueError, match="v_final"):
        gsa.gsa_fwd_varlen(q, q, v, g, cu, v_final=f32(3, H, M, D + 1))


def test_gla_fwd_shapes():
    q = t(B, H, T, D)
    with pytest.raises(TypeError):
        gsa.gla_fwd(q, q, q, q)
    with pytest.raises(ValueError, match="g"):
        gsa.gla_fwd(q, q, q, t(B, H, T, M))
    with pytest.raises(ValueError, match="s0"):
        gsa.gla_fwd(q, q, q, q, f32(B, H, D, D + 1))
    with pytest.raises(ValueError, match="s_final"):
        gsa.gla_fwd(q, q, q, q, s_final=f32(B, H, D, 1))


def test_decode_shapes():
    q, g = t(5, H, D), t(5, H, M)
    ks, vs = f32(5, H, M, D), f32(5, H, M, D)
    with pytest.raises(TypeError):
        gsa.gsa_decode_step(q, q, q, g, ks, vs)
    with pytest.raises(ValueError, match="k_state"):
        gsa.gsa_decode_step(q, q, q, g, f32(4, H, M, D), vs)
    with pytest.raises(ValueError, match="v_state"):
        gsa.gsa_decode_step(q, q, q, g, ks, f32(5, H, M + 1, D))
    with pytest.raises(ValueError, match="g"):
        gsa.gsa_decode_step(q, q, q, t(5, H, M + 2), ks, vs)
    with pytest.raises(ValueError, match="out"):
        gsa.gsa_decode_step(q, q, q, g, ks, vs, out=t(5, H, D + 1))
    s = f32(5, H, D, D)
    with pytest.raises(TypeError):
        gsa.gla_decode_step(q, q, q, q, s)
    with pytest.raises(ValueError, match="s_state"):
        gsa.gla_decode_step(q, q, q, q, f32(5, H, D, D - 1))


def test_bwd_shapes():
    a = fwd_args()
    do = t(B, H, T, D)
    with pytest.raises(TypeError):
        gsa.gsa_bwd(a["q"], a["k"], a["v"], a["g"], do)
    with pytest.raises(ValueError, match="d_o"):
        gsa.gsa_bwd(a["q"], a["k"], a["v"], a["g"], t(B, H, T - 1, D))
    with pytest.raises(ValueError, match="d_kf"):
        gsa.gsa_bwd(a["q"], a["k"], a["v"], a["g"], do, d_kf=f32(B, H, M, D + 4))
    with pytest.raises(ValueError, match="v0"):
        gsa.gsa_bwd(a["q"], a["k"], a["v"], a["g"], do, v0=f32(B, H, 1, D))
    cu = [0, 20, 70]
    q, g = t(H, 70, D), t(H, 70, M)
    with pytest.raises(TypeError):
        gsa.gsa_bwd_varlen(q, q, q, g, q, cu)
    with pytest.raises(ValueError, match="d_o"):
        gsa.gsa_bwd_varlen(q, q, q, g, t(H, 71, D), cu)
    with pytest.raises(ValueError, match="cu_seqlens"):
        gsa.gsa_bwd_varlen(q, q, q, g, q, [0, 20, 69])
    with pytest.raises(ValueError, match="k0"):
        gsa.gsa_bwd_varlen(q, q, q, g, q, cu, k0=f32(3, H, M, D))


def test_training_pair_shapes():
    a = fwd_args()
    with pytest.raises(TypeError):  # shapes fine: stops at the device check
        gsa.gsa_fwd_train(**a)
    with pytest.raises(ValueError, match="g"):
        gsa.gsa_fwd_train(a["q"], a["k"], a["v"], t(B, H, T - 1, M))
    with pytest.raises(ValueError, match="v_final"):
        gsa.gsa_fwd_train(**a, v_final=f32(B, H, M, D + 1))
    st = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(TypeError):
        gsa.gsa_bwd_train(a["q"], a["k"], a["v"], a["g"], t(B, H, T, D), st)
    with pytest.raises(ValueError, match="d_o"):
        gsa.gsa_bwd_train(a["q"], a["k"], a["v"], a["g"], t(B, H, T + 1, D), st)
    with pytest.raises(ValueError, match="d_kf"):
        gsa.gsa_bwd_train(a["q"], a["k"], a["v"], a["g"], t(B, H, T, D), st, d_kf=f32(B, H, M + 1, D))
