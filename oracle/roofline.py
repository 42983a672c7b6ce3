"""Arithmetic intensity of MLA decode in MQA mode (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page, roofline paragraph.  It defines L
(sequence length), d (head dim), r (RoPE dim), H (heads) and b (bytes per
value), then gives the FLOPs, bytes loaded and their ratio, but the three
equations did not survive extraction.  Reconstruction (stated reading):

* FLOPs: every one of the H heads takes a dot product with each of the L
  latent rows over d + r dims and accumulates d value dims: 2 H L (2d + r);
* bytes: the L latent rows of d + r values, b bytes each: L (d + r) b;
* intensity: 2 H (2d + r) / ((d + r) b), independent of L.

The page's surviving numbers pin it: d=512, r=64, b=2, H=64 gives 120.8 FLOP/B,
and 258.2 FLOP/B solved for H gives roughly 128 heads.
"""


def mqa_flops(L: int, d: int, r: int, H: int) -> float:
    return 2.0 * H * L * (2 * d + r)


def mqa_bytes(L: int, d: int, r: int, b: int) -> float:
    return float(L) * (d + r) * b


def mqa_intensity(d: int, r: int, H: int, b: int) -> float:
    return 2.0 * H * (2 * d + r) / ((d + r) * b)


def heads_for_intensity(ai: float, d: int, r: int, b: int) -> float:
    return ai * (d + r) * b / (2.0 * (2 * d + r))
