"""Pins for the oracle's cache write (O6): the new token's indexer key
(LayerNorm with bias, interleaved RoPE on its trailing span, fp8 cast) and its
latent row (latent entries as given, interleaved RoPE on the trailing span).

Independent checks: torch's float64 layer_norm (library), numpy complex
multiplication for the rotation of each (2i, 2i+1) pair (library), the
relative-position property of a rotary table built from angles, torch's fp8
cast and every code and midpoint of the format (exhaustive)."""
import numpy as np
import pytest
import torch


def bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def decode(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def angle_table(n_pos, D_rope, base=10000.0):
    """cos(p*theta_i) at [p, i], sin at [p, D_rope/2 + i]; theta_i = base^(-2i/D_rope)."""
    th = base ** (-np.arange(0, D_rope, 2, dtype=np.float64) / D_rope)
    a = np.arange(n_pos, dtype=np.float64)[:, None] * th[None, :]
    return np.concatenate([np.cos(a), np.sin(a)], axis=1).astype(np.float32)


def rotate_complex(x, table, pos):
    """Pairs (2i, 2i+1) as complex numbers times cos + j sin."""
    D = x.shape[1]
    z = x[:, 0::2] + 1j * x[:, 1::2]
    tb = table[pos].astype(np.float64)
    r = z * (tb[:, :D // 2] + 1j * tb[:, D // 2:])
    out = np.empty_like(x)
    out[:, 0::2] = r.real
    out[:, 1::2] = r.imag
    return out


# ---------------------------------------------------------------- fp8 cast --
def fp8_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_fp8_every_code_round_trips(orc):
    v = fp8_values()
    codes = np.arange(256)
    finite = (codes & 0x7F) != 0x7F
    got = orc.encode_fp8(v[finite])
    assert np.array_equal(got, codes[finite].astype(np.uint8))


def test_fp8_midpoints_tie_to_even(orc):
    """Halfway between neighbouring codes goes to the even code; a nudge either
    way goes to the nearer one."""
    v = fp8_values()[:0x7F]                             # 0 .. 448, increasing
    mid = (v[:-1] + v[1:]) / 2
    lo, hi = np.arange(0x7E), np.arange(1, 0x7F)
    want = np.where(lo % 2 == 0, lo, hi).astype(np.uint8)
    assert np.array_equal(orc.encode_fp8(mid), want)
    assert np.array_equal(orc.encode_fp8(-mid), want | 0x80)
    eps = (v[1:] - v[:-1]) * 1e-3
    assert np.array_equal(orc.encode_fp8(mid - eps), lo.astype(np.uint8))
    assert np.array_equal(orc.encode_fp8(mid + eps), hi.astype(np.uint8))


def test_fp8_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (0.01, 1.0, 30.0)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.encode_fp8(x.astype(np.float64)), want)


def test_fp8_saturates(orc):
    """The format has no infinity: the cast saturates at +-448 (code 0x7E)."""
    got = orc.encode_fp8([448.0, 449.0, 464.0, 500.0, 1e30, np.inf, -449.0, -1e30, -np.inf])
    assert list(got) == [0x7E] * 6 + [0xFE] * 3


# ------------------------------------------------------------- LayerNorm ----
@pytest.mark.parametrize("D_I", [32, 64, 128])
def test_layer_norm_matches_torch(orc, D_I):
    rng = np.random.default_rng(D_I)
    T = 7
    x = bf16(rng.standard_normal((T, D_I)) * 3 + 0.5)
    w = (1 + 0.2 * rng.standard_normal(D_I)).astype(np.float32)
    b = (0.3 * rng.standard_normal(D_I)).astype(np.float32)
    eps = 1e-6
    y, code = orc.index_key(x, w, b, eps, np.zeros((1, 0), np.float32), np.zeros(T, np.int32), 0)
    want = torch.nn.functional.layer_norm(torch.from_numpy(decode(x)), (D_I,), torch.from_numpy(w.astype(np.float64)),
                                          torch.from_numpy(b.astype(np.float64)), eps).numpy()
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(code, torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn)
                          .view(torch.uint8).numpy())


def test_layer_norm_constant_row_gives_bias(orc):
    D_I, T = 64, 3
    x = bf16(np.full((T, D_I), 1.75))
    w = np.linspace(0.5, 2, D_I).astype(np.float32)
    b = np.linspace(-1, 1, D_I).astype(np.float32)
    y, _ = orc.index_key(x, w, b, 1e-6, np.zeros((1, 0), np.float32), np.zeros(T, np.int32), 0)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), (T, D_I)))


# ------------------------------------------------------------------ RoPE ----
def test_latent_row_rotates_trailing_pairs(orc):
    rng = np.random.default_rng(7)
    T, D_qk, D_rope = 6, 576, 64
    x = bf16(rng.standard_normal((T, D_qk)))
    tab = angle_table(5000, D_rope)
    pos = np.array([0, 1, 2, 17, 1000, 4999], np.int32)
    out = orc.latent_row(x, tab, pos, D_rope)
    xd = decode(x)
    assert np.array_equal(out[:, :D_qk - D_rope], xd[:, :D_qk - D_rope])
    assert np.allclose(out[:, D_qk - D_rope:], rotate_complex(xd[:, D_qk - D_rope:], tab, pos), rtol=0, atol=1e-12)
    assert np.array_equal(out[0], xd[0])                       # position 0: cos 1, sin 0


def test_rope_relative_position(orc):
    """Rotary tables built from angles make the dot product of two rotated
    spans depend on the difference of the positions only."""
    rng = np.random.default_rng(8)
    D_qk, D_rope = 80, 16
    tab = angle_table(300, D_rope)
    a = bf16(rng.standard_normal((1, D_qk)))
    c = bf16(rng.standard_normal((1, D_qk)))

    def dot(p, q):
        ra = orc.latent_row(a, tab, np.array([p], np.int32), D_rope)[0, -D_rope:]
        rc = orc.latent_row(c, tab, np.array([q], np.int32), D_rope)[0, -D_rope:]
        return ra @ rc

    ref = dot(40, 3)
    for d in (1, 10, 200):
        assert abs(dot(40 + d, 3 + d) - ref) < 1e-4 * (1 + abs(ref))
    assert abs(dot(41, 3) - ref) > 1e-3                         # and it does change with the difference


def test_index_key_rotates_trailing_span(orc):
    rng = np.random.default_rng(9)
    T, D_I, D_rope = 5, 128, 64
    x = bf16(rng.standard_normal((T, D_I)))
    w = (1 + 0.1 * rng.standard_normal(D_I)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D_I)).astype(np.float32)
    tab = angle_table(70000, D_rope)
    pos = np.array([0, 5, 4096, 65535, 69999], np.int32)
    y0, _ = orc.index_key(x, w, b, 1e-6, tab, pos, 0)
    y, code = orc.index_key(x, w, b, 1e-6, tab, pos, D_rope)
    assert np.array_equal(y[:, :D_I - D_rope], y0[:, :D_I - D_rope])
    assert np.allclose(y[:, D_I - D_rope:], rotate_complex(y0[:, D_I - D_rope:], tab, pos), rtol=0, atol=1e-12)
    assert np.array_equal(code, torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn)
                          .view(torch.uint8).numpy())
