"""fa_bwd (the attention backward pass) against the fp64 oracle, through the
C ABI (needs a gfx950 GPU). Every case prints its name, shape and seed before
touching the GPU.

Rule: each gradient element g with oracle value r and oracle magnitude sum m
(the sum of the absolute values of the terms r adds up, the P_ij A_i terms
included, each rounded operand counted at no less than the type's smallest
normal, see oracle_attention_bwd) satisfies |g - r| <= 2 u m + ulp(r),
u = 2^-11 for fp16 and 2^-8 for bf16 (the unit roundoff). Each term carries
one rounding of P or dS to the element type (at most u relative, or half
the subnormal spacing below the smallest normal) and a recomputed P whose
LSE comes from the forward (within about u of the exact one: the fp16
forward sums rounded probabilities); the fp32 products and sums add far
less. The output itself is rounded once, within half an ulp."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import decode, to_bits, to_device, ulp_bf16

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def ulp(r, dtype):
    if dtype == "bf16":
        return ulp_bf16(r)
    ax = np.maximum(np.abs(r), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - 10)


def inputs(B, H, S, D, dtype, seed):
    q, k, v = synth.make_qkv(B, H, S, D, dtype, seed)
    do, _, _ = synth.make_qkv(B, H, S, D, dtype, seed + 1)
    return q, k, v, do


def gpu_grads(q, k, v, do, dtype, scale, mask, window):
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, scale=scale, mask=mask, window=window)
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, scale=scale, mask=mask, window=window)
    torch.cuda.synchronize()
    return [decode(to_bits(g), dtype).reshape(q.shape) for g in (dq, dk, dv)]


def check(orc, q, k, v, do, dtype, scale, mask, window=(-1, -1)):
    got = gpu_grads(q, k, v, do, dtype, scale, mask, window)
    refs, mags = orc.attention_bwd(q, k, v, do, dtype, scale, mask, window)
    for name, g, r, m in zip(("dq", "dk", "dv"), got, refs, mags):
        assert np.all(np.isfinite(g)), name
        bound = 2 * U[dtype] * m + ulp(r, dtype)
        worst = np.abs(g - r) / bound
        assert worst.max() <= 1.0, (name, float(worst.max()),
                                    np.unravel_index(worst.argmax(), worst.shape))


SHAPES = [(1, 2, 300, 64), (2, 2, 320, 128), (1, 3, 777, 128), (1, 2, 129, 64), (1, 1, 1, 128),
          (1, 2, 64, 128)]
MASKS = [("full", (-1, -1)), ("causal", (-1, -1)), ("window", (100, 0)), ("window", (37, 50)),
         ("window", (-1, 20)), ("window", (0, 0))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", MASKS, ids=str)
def test_bwd_parity(orc, dtype, shape, mask, window):
    B, H, S, D = shape
    seed = 800 + S + D
    say("bwd", dtype, shape, mask, window, "seed", seed)
    q, k, v, do = inputs(B, H, S, D, dtype, seed)
    check(orc, q, k, v, do, dtype, 1.0 / math.sqrt(D), mask, window)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.5])
def test_bwd_scales(orc, scale):
    say("bwd scale", scale)
    q, k, v, do = inputs(1, 2, 200, 64, "f16", seed=811)
    check(orc, q, k, v, do, "f16", scale, "causal")


def test_bwd_is_deterministic():
    say("bwd determinism")
    q, k, v, do = inputs(2, 2, 500, 128, "bf16", seed=812)
    a = gpu_grads(q, k, v, do, "bf16", 0.1, "causal", (-1, -1))
    b = gpu_grads(q, k, v, do, "bf16", 0.1, "causal", (-1, -1))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_headline_shape_two_heads(orc):
    """B4 H32 S4096 D128 fp16 causal at full size, checked on two heads."""
    w = synth.WORKLOADS["b4h32s4096_causal"]
    say("bwd b4h32s4096 causal (two heads)")
    q, k, v = synth.workload_inputs("b4h32s4096_causal")
    do, _, _ = synth.make_qkv(w["B"], w["H"], w["S"], w["D"], "f16", seed=813)
    got = gpu_grads(q, k, v, do, "f16", w["scale"], "causal", (-1, -1))
    for b, h in ((0, 0), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        refs, mags = orc.attention_bwd(q[sl], k[sl], v[sl], do[sl], "f16", w["scale"], "causal")
        for name, g, r, m in zip(("dq", "dk", "dv"), got, refs, mags):
            bound = 2 * U["f16"] * m + ulp(r, "f16")
            worst = np.abs(g[sl] - r) / bound
            assert worst.max() <= 1.0, (b, h, name, float(worst.max()))


@pytest.mark.parametrize("case", [(4, 16, 2048, 64, "f16", "window", (300, 0)),
                                  (5, 13, 1300, 64, "bf16", "causal", (-1, -1))],
                         ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{c[4]}{c[5]}")
def test_bwd_persistent_schedule(orc, case):
    """Both kernels run persistent workgroups over work lists (XCD lists and,
    under a window, the equal-cost tiles first; a single list when B*H is not
    a multiple of 8), several items per workgroup here. Every head's
    gradients equal that head's gradients computed alone (a launch with a
    different schedule) bit for bit, so every item ran exactly once; a few
    heads are also checked against the oracle."""
    B, H, S, D, dtype, mask, window = case
    seed = 820 + S
    say("bwd persistent schedule", case, "seed", seed)
    q, k, v, do = inputs(B, H, S, D, dtype, seed)
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, do))
    # one forward for the batch: a head's forward alone may take another
    # layout, whose O and LSE differ in the last bits
    o, lse = fa.forward(tq, tk, tv, scale=scale, mask=mask, window=window)

    def grads(bsl, hsl):
        parts = [t[bsl, hsl].contiguous() for t in (tq, tk, tv, o, lse, tdo)]
        out = fa.backward(*parts, scale=scale, mask=mask, window=window)
        torch.cuda.synchronize()
        return [decode(to_bits(gr), dtype).reshape(gr.shape) for gr in out]

    got = grads(slice(None), slice(None))
    for b in range(B):
        for h in range(H):
            alone = grads(slice(b, b + 1), slice(h, h + 1))
            for name, g, a in zip(("dq", "dk", "dv"), got, alone):
                assert np.array_equal(g[b:b + 1, h:h + 1], a, equal_nan=True), (b, h, name)
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, H // 3)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        refs, mags = orc.attention_bwd(q[sl], k[sl], v[sl], do[sl], dtype, scale, mask, window)
        for name, g, r, m in zip(("dq", "dk", "dv"), got, refs, mags):
            bound = 2 * U[dtype] * m + ulp(r, dtype)
            worst = np.abs(g[sl] - r) / bound
            assert worst.max() <= 1.0, (b, h, name, float(worst.max()))
