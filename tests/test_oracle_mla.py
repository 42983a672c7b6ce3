"""Pins of the oracle's MLA modes (GLM5.3 sparse-attention page, MLA-modes paragraph).

The page states the cost trade-off of the two modes (MQA mode: 3.4 times the FLOPs of the MHA
mode) but not their equations.  Pins: the FLOP ratio of the modes at the latent shape of the
workloads equals the page's 3.4, and both modes give the same attention output on random inputs,
in float64, through the same SDPA routine the decode oracle uses (so a dropped rotary term, a
transposed up-projection or a wrong scale in either mode fails).
"""
import numpy as np
import pytest

from oracle import mla, sdpa


def test_flop_ratio_is_the_pages():
    c = mla.mode_costs(H=64, d_c=512, r=64, d_nope=128, d_v=128)
    assert c["mqa_macs"] / c["mha_macs"] == pytest.approx(3.4, abs=1e-12)
    # memory read per token: 35.6x at these dims (the page quotes 42x for its model's dims)
    assert c["mha_values"] / c["mqa_values"] == pytest.approx(64 * 320 / 576)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_modes_agree(seed):
    rng = np.random.default_rng(seed)
    H, d_c, r, d_nope, d_v, n = 4, 16, 4, 8, 6, 23
    c = rng.standard_normal((n, d_c))
    rk = rng.standard_normal((n, r))
    w_uk = rng.standard_normal((H, d_nope, d_c)) / 4
    w_uv = rng.standard_normal((H, d_v, d_c)) / 4
    q_nope = rng.standard_normal((H, d_nope))
    q_rope = rng.standard_normal((H, r))
    scale = 1.0 / np.sqrt(d_nope + r)
    # MHA mode: one KV head per query head
    k, v = mla.mha_kv(c, rk, w_uk, w_uv)
    o_mha = sdpa.attend(np.concatenate([q_nope, q_rope], axis=1), k, v, scale)
    # MQA mode: every head reads the latent row, whose first d_c values are the value
    lat = np.concatenate([c, rk], axis=1)[:, None, :]
    o_lat = sdpa.attend(mla.absorb_query(q_nope, q_rope, w_uk), lat, lat[:, :, :d_c], scale)
    o_mqa = mla.unabsorb_output(o_lat, w_uv)
    assert np.allclose(o_mha, o_mqa, rtol=1e-12, atol=1e-12)
    # and the modes are not trivially equal: dropping the rotary part of the keys changes o
    k2 = k.copy()
    k2[:, :, d_nope:] = 0
    assert not np.allclose(sdpa.attend(np.concatenate([q_nope, q_rope], axis=1), k2, v, scale), o_mha)
