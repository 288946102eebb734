"""fa_rope and fa_fwd_rope (rotary position embedding) against the fp64
oracle, through the C ABI (needs a gfx950 GPU). Every case prints its name,
shape and seed before touching the GPU.

Rule for the rotated tensors themselves: each output element y of a pair
(a, b) turned by (c, s) lies within ulp(r) + 2^-22 (|a c| + |b s|) of the
oracle's fp64 value r, ulp taken in the element type at r. The kernel forms
a c - b s (or b c + a s) in fp32, within 2 * 2^-24 (|a c| + |b s|) of r (two
products and a sum, each rounded once), then rounds once to the element
type, within half a unit; the rule doubles both terms. The second term
matters only where the two products nearly cancel."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import compare, decode, to_bits, to_device, ulp_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def ulp(r, dtype):
    if dtype == "bf16":
        return ulp_bf16(r)
    ax = np.maximum(np.abs(r), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - 10)


def tables(n_pos, D, base=10000.0):
    cos, sin = synth.rope_tables(n_pos, D, base)
    return cos, sin, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()


def product_sizes(xd, cos, sin, mode, S):
    """|a c| + |b s| for every element of [B,H,S,D] rows at positions 0..S-1."""
    D = xd.shape[-1]
    c = np.abs(cos[:S].astype(np.float64))
    s = np.abs(sin[:S].astype(np.float64))
    if mode == "halves":
        a, b = np.abs(xd[..., : D // 2]), np.abs(xd[..., D // 2:])
    else:
        a, b = np.abs(xd[..., 0::2]), np.abs(xd[..., 1::2])
    m = np.maximum(a * c + b * s, b * c + a * s)
    out = np.empty_like(xd)
    if mode == "halves":
        out[..., : D // 2], out[..., D // 2:] = m, m
    else:
        out[..., 0::2], out[..., 1::2] = m, m
    return out


def check_rotated(orc, bits, x_bits, cos, sin, mode, dtype, S):
    """``bits``: GPU output [B,H,S,D] of rotating ``x_bits`` at positions 0..S-1."""
    pos = np.tile(np.arange(S), x_bits.shape[0] * x_bits.shape[1])
    ref = orc.rope(x_bits, pos, cos, sin, mode, dtype).reshape(x_bits.shape)
    got = decode(bits, dtype).reshape(x_bits.shape)
    xd = decode(x_bits, dtype).reshape(x_bits.shape)
    bound = ulp(ref, dtype) + 2.0 ** -22 * product_sizes(xd, cos, sin, mode, S)
    err = np.abs(got - ref) / bound
    assert err.max() <= 1.0, (err.max(), np.unravel_index(err.argmax(), err.shape))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["halves", "interleaved"])
def test_rope_kernel(orc, dtype, D, mode):
    B, H, S = 2, 3, 333
    say("rope", dtype, D, mode, (B, H, S))
    x, _, _ = synth.make_qkv(B, H, S, D, dtype, seed=600 + D)
    cos, sin, tc, ts = tables(S + 17, D)
    y = fa.rope(to_device(x, dtype), tc, ts, mode=mode)
    torch.cuda.synchronize()
    check_rotated(orc, to_bits(y), x, cos, sin, mode, dtype, S)


def test_rope_in_place_equals_out_of_place():
    say("rope in place")
    x, _, _ = synth.make_qkv(1, 4, 100, 128, "bf16", seed=601)
    _, _, tc, ts = tables(100, 128)
    tx = to_device(x, "bf16")
    y = fa.rope(tx, tc, ts, mode="interleaved")
    fa.rope(tx, tc, ts, mode="interleaved", out=tx)
    torch.cuda.synchronize()
    assert torch.equal(tx.view(torch.int16), y.view(torch.int16))


SHAPES = [(2, 3, 1000, 128), (1, 4, 777, 64), (1, 2, 300, 64)]
MASKS = [("causal", (-1, -1)), ("full", (-1, -1)), ("window", (100, 0)), ("window", (37, 50))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["halves", "interleaved"])
@pytest.mark.parametrize("mask,window", MASKS, ids=str)
def test_fwd_rope_parity(orc, dtype, shape, mode, mask, window):
    B, H, S, D = shape
    seed = 700 + S + D
    say("fwd_rope", dtype, shape, mode, mask, window, "seed", seed)
    q, k, v = synth.make_qkv(B, H, S, D, dtype, seed)
    cos, sin, tc, ts = tables(S, D)
    scale = 1.0 / math.sqrt(D)
    o, lse, k_rot = fa.forward_rope(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                                    tc, ts, mode=mode, scale=scale, mask=mask, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_rope(q, k, v, dtype, scale, mask, window, cos, sin, mode)
    st = compare(to_bits(o), lse.cpu().numpy(), o_ref, lse_ref, dtype)
    assert st["pass"], st
    check_rotated(orc, to_bits(k_rot), k, cos, sin, mode, dtype, S)


def test_fwd_rope_in_place_and_tables_longer_than_s(orc):
    """k rotated in place; tables with more rows than positions used."""
    B, H, S, D = 1, 2, 500, 128
    say("fwd_rope in place", (B, H, S, D))
    q, k, v = synth.make_qkv(B, H, S, D, "f16", seed=702)
    cos, sin, tc, ts = tables(4 * S, D, base=500000.0)
    tk = to_device(k, "f16")
    o, lse, k_rot = fa.forward_rope(to_device(q, "f16"), tk, to_device(v, "f16"), tc, ts,
                                    k_rot=tk, mask="causal")
    torch.cuda.synchronize()
    assert k_rot.data_ptr() == tk.data_ptr()
    o_ref, lse_ref = orc.attention_rope(q, k, v, "f16", 1.0 / math.sqrt(D), "causal", (-1, -1),
                                        cos, sin, "halves")
    st = compare(to_bits(o), lse.cpu().numpy(), o_ref, lse_ref, "f16")
    assert st["pass"], st


def test_fwd_rope_zero_angles_is_the_plain_forward():
    """cos 1, sin 0: the output equals fa_fwd's bit for bit (rotating by zero
    leaves every fp16 value as it was)."""
    B, H, S, D = 2, 2, 400, 64
    say("fwd_rope zero angles")
    q, k, v = synth.make_qkv(B, H, S, D, "f16", seed=703)
    tc = torch.ones((S, D // 2), dtype=torch.float32, device="cuda")
    ts = torch.zeros((S, D // 2), dtype=torch.float32, device="cuda")
    tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
    o, lse, _ = fa.forward_rope(tq, tk, tv, tc, ts, mask="causal")
    o0, lse0 = fa.forward(tq, tk, tv, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))


def test_named_workload_sampled_rows(orc):
    """The headline shape with RoPE at full size, in the launch the benchmark
    times, on sampled rows."""
    w = synth.WORKLOADS["b4h32s4096_causal"]
    B, H, S, D = w["B"], w["H"], w["S"], w["D"]
    say("fwd_rope b4h32s4096 causal sampled")
    q, k, v = synth.workload_inputs("b4h32s4096_causal")
    cos, sin, tc, ts = tables(S, D)
    o, lse, _ = fa.forward_rope(to_device(q, "f16"), to_device(k, "f16"), to_device(v, "f16"),
                                tc, ts, scale=w["scale"], mask="causal")
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(B * H * S, 200, replace=False),
                                     [0, S - 1, S, B * H * S - 1]]))
    o_ref, lse_ref = orc.attention_rope_rows(q, k, v, "f16", w["scale"], "causal", (-1, -1),
                                             cos, sin, "halves", rows=rows)
    st = compare(to_bits(o).reshape(-1, D)[rows], lse.cpu().numpy().reshape(-1)[rows], o_ref,
                 lse_ref, "f16")
    assert st["pass"], st


# ---------------------------------------------------------------------------
# new rows against a cache of rotated keys

DEC_SHAPES = [(2, 3, 1, 777, 128), (1, 2, 16, 2000, 64), (2, 2, 5, 129, 128), (1, 4, 32, 32, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", DEC_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["halves", "interleaved"])
@pytest.mark.parametrize("mask,window", [("causal", (-1, -1)), ("window", (100, 0))], ids=str)
def test_decode_rope_parity(orc, dtype, shape, mode, mask, window):
    B, H, Sq, Sk, D = shape
    seed = 720 + Sq + Sk + D
    say("decode_rope", dtype, shape, mode, mask, window, "seed", seed)
    q, _, _ = synth.make_qkv(B, H, Sq, D, dtype, seed)
    _, k, v = synth.make_qkv(B, H, Sk, D, dtype, seed + 1)
    cos, sin, tc, ts = tables(Sk + 9, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.decode(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), scale=scale,
                       mask=mask, window=window, rope=(tc, ts, mode))
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_kv_rope(q, k, v, dtype, scale, mask, window, cos, sin, mode)
    st = compare(to_bits(o), lse.cpu().numpy(), o_ref, lse_ref, dtype)
    assert st["pass"], st


def test_decode_rope_continues_the_prefill(orc):
    """A prefill with fa_fwd_rope fills the cache (k_rot); the cache call with
    the new rows rotated at the end positions reproduces the prefill's last
    rows (fp16, causal)."""
    B, H, S, D, Sq = 1, 3, 600, 128, 8
    say("decode_rope after prefill", (B, H, S, D, Sq))
    q, k, v = synth.make_qkv(B, H, S, D, "f16", seed=730)
    cos, sin, tc, ts = tables(S, D)
    tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
    o_full, lse_full, k_rot = fa.forward_rope(tq, tk, tv, tc, ts, mask="causal")
    o_dec, lse_dec = fa.decode(tq[:, :, S - Sq:].contiguous(), k_rot, tv, mask="causal",
                               rope=(tc, ts, "halves"))
    torch.cuda.synchronize()
    # both are within tolerance of the same oracle rows; compare them directly
    a = decode(to_bits(o_dec), "f16")
    b = decode(to_bits(o_full[:, :, S - Sq:]), "f16")
    assert np.max(np.abs(a - b)) <= 2e-3
    assert np.max(np.abs(lse_dec.cpu().numpy() - lse_full[:, :, S - Sq:].cpu().numpy())) <= 1e-3


def test_decode_paged_rope_parity(orc):
    """The paged cache with rotated new rows, against the oracle on the same
    (contiguous) cache."""
    B, H, Sq, Sk, D, ps = 2, 4, 3, 1024, 128, 64
    say("decode_paged_rope", (B, H, Sq, Sk, D, ps))
    q, _, _ = synth.make_qkv(B, H, Sq, D, "f16", seed=731)
    _, k, v = synth.make_qkv(B, H, Sk, D, "f16", seed=732)
    kp, vp, table = synth.paged_cache(k, v, ps, seed=733)
    cos, sin, tc, ts = tables(Sk, D)
    lens = torch.full((B,), Sk, dtype=torch.int32, device="cuda")
    o, lse = fa.decode_paged(to_device(q, "f16"), to_device(kp, "f16"), to_device(vp, "f16"),
                             torch.from_numpy(table).cuda(), lens, Sk, mask="causal",
                             rope=(tc, ts, "interleaved"))
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_kv_rope(q, k, v, "f16", 1.0 / math.sqrt(D), "causal",
                                           (-1, -1), cos, sin, "interleaved")
    st = compare(to_bits(o), lse.cpu().numpy(), o_ref, lse_ref, "f16")
    assert st["pass"], st
