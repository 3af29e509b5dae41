"""Pins for the oracle's gated head output (O5):
out[t,h,e] = sigmoid(gate[t,h,e]) * sum_c wv_b[h,e,c] * o[t,h,c].

Independent checks: closed forms with an identity and a rank-1 up-projection
(integer-valued bf16 inputs, so every product and sum is exact), the gate's
limits, and invariance under a permutation of the heads."""
import numpy as np
import torch


def bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def decode(b):
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def test_identity_upprojection(orc):
    """wv_b = [I | 0]: out is the gated leading D_o latent entries; gate 0
    halves them exactly, a large gate keeps them, a very negative one zeroes."""
    rng = np.random.default_rng(1)
    T, H, D_v, D_o = 3, 2, 64, 32
    o = bf16(rng.integers(-64, 64, size=(T, H, D_v)) / 8.0)
    w = np.zeros((H, D_o, D_v), np.float32)
    for h in range(H):
        w[h, :, :D_o] = np.eye(D_o)
    wv = bf16(w)
    od = decode(o)
    out = orc.gated_output(o, wv, bf16(np.zeros((T, H, D_o))))
    assert np.array_equal(out, 0.5 * od[:, :, :D_o])
    out = orc.gated_output(o, wv, bf16(np.full((T, H, D_o), 60.0)))
    assert np.allclose(out, od[:, :, :D_o], rtol=1e-20, atol=1e-24)
    out = orc.gated_output(o, wv, bf16(np.full((T, H, D_o), -60.0)))
    assert np.all(np.abs(out) <= np.abs(od[:, :, :D_o]) * 1e-25)


def test_rank1_closed_form(orc):
    """wv_b[h,e,c] = u[h,e] * v[h,c]: out = sigmoid(g) * u[h,e] * (v[h] . o[t,h]);
    a gate that varies along e, never along c, fixes which space it acts in."""
    rng = np.random.default_rng(2)
    T, H, D_v, D_o = 2, 3, 64, 48
    u = rng.integers(-3, 4, size=(H, D_o)).astype(np.float64)
    v = rng.integers(-2, 3, size=(H, D_v)).astype(np.float64)
    o = rng.integers(-16, 17, size=(T, H, D_v)).astype(np.float64) / 4.0
    g = np.where(np.arange(D_o) % 3 == 0, 0.0, 60.0)[None, None, :].repeat(T, 0).repeat(H, 1)
    out = orc.gated_output(bf16(o), bf16(u[:, :, None] * v[:, None, :]), bf16(g))
    dot = np.einsum("hc,thc->th", v, o)                    # integers / 4: exact
    want = u[None, :, :] * dot[:, :, None] * np.where(g == 0.0, 0.5, 1.0)
    assert np.allclose(out, want, rtol=1e-20, atol=1e-24)


def test_gate_is_logistic(orc):
    """One latent entry and a unit up-projection: out = o * 1/(1 + e^-g) at
    gate values whose logistic is known (0 -> 1/2, ln 3 -> 3/4 up to bf16)."""
    T, H, D_v, D_o = 1, 1, 64, 64
    o = np.zeros((T, H, D_v))
    o[0, 0, 0] = 2.0
    w = np.zeros((H, D_o, D_v))
    w[0, :, 0] = 1.0
    gv = np.linspace(-8, 8, D_o)
    gb = bf16(gv[None, None, :])
    out = orc.gated_output(bf16(o), bf16(w), gb)
    g = decode(gb)[0, 0]
    assert np.allclose(out[0, 0], 2.0 / (1.0 + np.exp(-g)), rtol=1e-15)
    assert np.all(np.diff(out[0, 0]) > 0) and out[0, 0, 0] > 0 and out[0, 0, -1] < 2.0


def test_heads_permute(orc):
    """Permuting the heads of o, wv_b and gate permutes the output's heads."""
    rng = np.random.default_rng(3)
    T, H, D_v, D_o = 2, 5, 64, 64
    o = bf16(rng.standard_normal((T, H, D_v)))
    wv = bf16(rng.standard_normal((H, D_o, D_v)) / 8)
    g = bf16(rng.standard_normal((T, H, D_o)))
    base = orc.gated_output(o, wv, g)
    p = rng.permutation(H)
    perm = orc.gated_output(np.ascontiguousarray(o[:, p]), np.ascontiguousarray(wv[p]), np.ascontiguousarray(g[:, p]))
    assert np.array_equal(perm, base[:, p])
