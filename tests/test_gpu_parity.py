"""The HIP path against the fp64 oracle, through the C ABI (needs a gfx950 GPU).

Every case prints its name, shape and seed before touching the GPU."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import compare, decode, sample_rows, to_bits, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def gpu_run(q, k, v, dtype, scale, mask, window=(-1, -1), with_lse=True):
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = fa.forward(tq, tk, tv, scale=scale, mask=mask, window=window,
                        return_lse=with_lse)
    torch.cuda.synchronize()
    return to_bits(o), (lse.cpu().numpy() if lse is not None else None)


def check_full(orc, q, k, v, dtype, scale, mask, window=(-1, -1)):
    o_bits, lse = gpu_run(q, k, v, dtype, scale, mask, window)
    o_ref, lse_ref = orc.attention(q, k, v, dtype, scale, mask, window)
    st = compare(o_bits, lse, o_ref, lse_ref, dtype)
    assert st["pass"], st
    return st


# ---------------------------------------------------------------------------
# whole-tensor parity at sizes spanning several tiles and a ragged tail

SHAPES = [(2, 3, 1000, 128), (1, 4, 777, 64), (2, 2, 320, 128), (1, 2, 300, 64)]
MASKS = [("full", (-1, -1)), ("causal", (-1, -1)), ("window", (100, 0)),
         ("window", (37, 50)), ("window", (-1, 20)), ("window", (300, -1)),
         ("window", (64, 64))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", MASKS, ids=lambda m: str(m))
def test_parity_whole_tensor(orc, dtype, shape, mask, window):
    B, H, S, D = shape
    seed = 100 + S + D
    say("whole", dtype, shape, mask, window, "seed", seed)
    q, k, v = synth.make_qkv(B, H, S, D, dtype, seed)
    check_full(orc, q, k, v, dtype, 1.0 / math.sqrt(D), mask, window)


# Work layouts: grids of fewer than two 256-row items per CU run the key-split
# variant (128-row items, the two wave groups on alternate key tiles, merged at
# the end); many heads at a short length keep the 256-row items. Both layouts
# meet every mask and both head dimensions here (the small whole-tensor shapes
# above and the tail cases are key-split launches).
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(8, 64, 300, 128), (4, 128, 200, 64)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", [("full", (-1, -1)), ("causal", (-1, -1)),
                                         ("window", (-1, 20)), ("window", (299, 3))], ids=str)
def test_parity_unsplit_layout(orc, dtype, shape, mask, window):
    B, H, S, D = shape
    say("unsplit layout", dtype, shape, mask, window)
    q, k, v = synth.make_qkv(B, H, S, D, dtype, seed=200 + S + D)
    check_full(orc, q, k, v, dtype, 1.0 / math.sqrt(D), mask, window)


# The key-split layout at item counts that exercise its edges: one key tile per
# item (the odd group has none), odd tile counts, an item whose last rows lie
# past the sequence, several items per workgroup, windows that leave a group
# without visible tiles for some waves.
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 40, 128), (1, 3, 64, 64), (2, 3, 129, 128),
                                   (1, 2, 448, 64), (2, 64, 700, 128)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", [("causal", (-1, -1)), ("window", (0, 0)),
                                         ("window", (63, 0)), ("window", (130, 70)),
                                         ("full", (-1, -1))], ids=str)
def test_parity_split_layout_edges(orc, dtype, shape, mask, window):
    B, H, S, D = shape
    say("split layout", dtype, shape, mask, window)
    q, k, v = synth.make_qkv(B, H, S, D, dtype, seed=300 + S + D)
    check_full(orc, q, k, v, dtype, 1.0 / math.sqrt(D), mask, window)


@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,window", [("causal", (-1, -1)), ("full", (-1, -1)),
                                         ("window", (40, 3))], ids=str)
def test_parity_tails(orc, S, D, mask, window):
    say("tail", S, D, mask, window)
    q, k, v = synth.make_qkv(1, 2, S, D, "f16", seed=7 + S)
    check_full(orc, q, k, v, "f16", 1.0 / math.sqrt(D), mask, window)


# ---------------------------------------------------------------------------
# the named workloads at full size, on sampled rows

_CACHE = {}


def _inputs(name):
    w = synth.WORKLOADS[name]
    key = (w["B"], w["H"], w["S"], w["D"], w["dtype"], w["seed"], w.get("outlier_frac", 0.0))
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = synth.workload_inputs(name)
    return _CACHE[key]


# More query tiles than workgroups: each workgroup runs several items back to
# back, so the next item's Q and K(0) prefetch, the per-wave skipped leading
# and trailing steps and the early output stores all meet whole-tensor parity.
@pytest.mark.parametrize("shape", [(4, 64, 512, 128), (2, 64, 640, 64)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", [("causal", (-1, -1)), ("window", (100, 0)),
                                         ("window", (37, 50))], ids=str)
def test_parity_many_items_per_workgroup(orc, shape, mask, window):
    B, H, S, D = shape
    say("many items", shape, mask, window)
    q, k, v = synth.make_qkv(B, H, S, D, "f16", 93)
    check_full(orc, q, k, v, "f16", 1.0 / math.sqrt(D), mask, window)


# Named workloads checked over the whole tensor, head chunk by head chunk (a
# chunk's oracle rows take about 15 s on 16 host cores at the B4 H32 S4096
# D128 causal shape), and those checked on at least 32k rows that include
# every head's query-tile, key-tile and window edges.
WHOLE = ("tiny_full", "tiny_causal", "d64_causal", "b4h32s4096_causal",
         "b4h32s4096_win1024", "b4h32s4096_win1000", "b4h4s4096_causal",
         "b4h32s4096_causal_rope")
SAMPLED = ("b4h32s4096_full", "long_bf16_outliers")
HEADS_PER_CHUNK = 16
# The sampled workloads over the whole tensor as well: about 3 (full mask) and
# 4.5 (B1 H64 S16384) minutes of oracle time on 16 host cores, which would
# double the GPU suite, so they run only when FA_WHOLE_SLOW=1 is set.
WHOLE_SLOW = {"b4h32s4096_full": 16, "long_bf16_outliers": 4}
_OUT = {}


def _workload_output(name):
    """The GPU result of a named workload, in the launch the benchmark times
    (computed once per workload; RoPE workloads through forward_rope)."""
    if name not in _OUT:
        _OUT.clear()
        w = synth.WORKLOADS[name]
        q, k, v = _inputs(name)
        if w.get("rope"):
            cos, sin = synth.rope_tables(w["S"], w["D"], w["rope_base"])
            tq, tk, tv = (to_device(x, w["dtype"]) for x in (q, k, v))
            o, lse, _ = fa.forward_rope(tq, tk, tv, torch.from_numpy(cos).cuda(),
                                        torch.from_numpy(sin).cuda(), mode=w["rope"],
                                        scale=w["scale"], mask=w["mask"], window=w["window"])
            torch.cuda.synchronize()
            _OUT[name] = (to_bits(o), lse.cpu().numpy(), (cos, sin))
        else:
            o_bits, lse = gpu_run(q, k, v, w["dtype"], w["scale"], w["mask"], w["window"])
            _OUT[name] = (o_bits, lse, None)
    return _OUT[name]


def _oracle_rows(orc, name, rows):
    w = synth.WORKLOADS[name]
    q, k, v = _inputs(name)
    if w.get("rope"):
        cos, sin = _workload_output(name)[2]
        return orc.attention_rope_rows(q, k, v, w["dtype"], w["scale"], w["mask"], w["window"],
                                       cos, sin, w["rope"], rows=rows)
    return orc.attention_rows(q, k, v, w["dtype"], w["scale"], w["mask"], w["window"], rows)


def _chunks():
    out = []
    for name in WHOLE:
        w = synth.WORKLOADS[name]
        bh = w["B"] * w["H"]
        for c0 in range(0, bh, HEADS_PER_CHUNK):
            out.append((name, c0, min(bh, c0 + HEADS_PER_CHUNK)))
    return out


def _slow_chunks():
    out = []
    for name, per in WHOLE_SLOW.items():
        w = synth.WORKLOADS[name]
        bh = w["B"] * w["H"]
        for c0 in range(0, bh, per):
            out.append((name, c0, min(bh, c0 + per)))
    return out


@pytest.mark.parametrize("name,h0,h1", _slow_chunks(), ids=lambda x: str(x))
def test_parity_workload_whole_slow(orc, name, h0, h1):
    """Every row of heads h0 .. h1-1 of a sampled workload (opt-in: FA_WHOLE_SLOW=1)."""
    if os.environ.get("FA_WHOLE_SLOW") != "1":
        pytest.skip("whole-tensor check of a sampled workload: set FA_WHOLE_SLOW=1 "
                    "(minutes of host oracle time)")
    test_parity_workload_whole(orc, name, h0, h1)


@pytest.mark.parametrize("name,h0,h1", _chunks(), ids=lambda x: str(x))
def test_parity_workload_whole(orc, name, h0, h1):
    """Every row of heads h0 .. h1-1 of a named workload at full size."""
    w = synth.WORKLOADS[name]
    B, H, S, D, dtype = w["B"], w["H"], w["S"], w["D"], w["dtype"]
    say("workload whole", name, (B, H, S, D), dtype, w["mask"], w["window"], "seed", w["seed"],
        "heads", h0, h1)
    o_bits, lse, _ = _workload_output(name)
    rows = np.arange(h0 * S, h1 * S, dtype=np.int64)
    o_ref, lse_ref = _oracle_rows(orc, name, rows)
    st = compare(o_bits.reshape(-1, D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype)
    say("stats", st)
    assert st["pass"], st


def edge_rows(B, H, S, n_min, seed, extra_i=()):
    """Flat row indices: for every head the rows at query-tile (256), key-tile
    (64) and wave (32) edges near both ends and the middle of the sequence,
    plus the ``extra_i`` positions (window edges), topped up with random rows
    to at least ``n_min``."""
    edges = set()
    for c in (0, 256, S // 2, S - 256):
        for o in (0, 1, 31, 32, 63, 64, 65, 127, 128, 255):
            edges.add(c + o)
            edges.add(c - 1 - o)
    edges.update((S - 1, S - 2, *extra_i))
    edges = np.array(sorted(i for i in edges if 0 <= i < S), dtype=np.int64)
    rows = (np.arange(B * H, dtype=np.int64)[:, None] * S + edges[None, :]).ravel()
    rng = np.random.default_rng(seed)
    need = max(0, n_min - rows.size)
    if need:
        rows = np.concatenate([rows, rng.choice(B * H * S, size=need + rows.size, replace=False)])
    rows = np.unique(rows)
    return rows


@pytest.mark.parametrize("name", SAMPLED)
def test_parity_workload_sampled(orc, name):
    """A named workload at full size on >= 32k rows including every head's edges."""
    w = synth.WORKLOADS[name]
    B, H, S, D, dtype = w["B"], w["H"], w["S"], w["D"], w["dtype"]
    say("workload sampled", name, (B, H, S, D), dtype, w["mask"], w["window"], "seed", w["seed"])
    o_bits, lse, _ = _workload_output(name)
    wl = w["window"][0]
    extra = (wl - 1, wl, wl + 1, wl + 63, wl + 64) if wl > 0 else ()
    rows = edge_rows(B, H, S, 32768, seed=w["seed"], extra_i=extra)
    assert rows.size >= 32768
    o_ref, lse_ref = _oracle_rows(orc, name, rows)
    st = compare(o_bits.reshape(-1, D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype)
    say("stats", st)
    assert st["pass"], st


def test_named_workloads_are_all_covered():
    assert set(WHOLE) | set(SAMPLED) == set(synth.WORKLOADS)


# ---------------------------------------------------------------------------
# closed forms through the GPU path

def test_zero_q_gives_prefix_means(orc):
    S, D = 333, 128
    _, k, v = synth.make_qkv(1, 1, S, D, "f16", seed=31)
    q = np.zeros_like(k)
    say("zero-q prefix means", S, D)
    o_bits, lse = gpu_run(q, k, v, "f16", 0.088, "causal")
    vd = decode(v, "f16")[0, 0]
    prefix = np.cumsum(vd, axis=0) / np.arange(1, S + 1)[:, None]
    o = decode(o_bits, "f16")[0, 0]
    assert np.max(np.abs(o - prefix)) < 2e-3
    assert np.max(np.abs(lse[0, 0] - np.log(np.arange(1, S + 1)))) < 1e-5


def test_constant_v_is_reproduced():
    S, D = 257, 64
    q, k, _ = synth.make_qkv(2, 2, S, D, "bf16", seed=32)
    c = (np.arange(D) % 7 - 3).astype(np.float32) * 0.5
    v = synth.f32_to_bits(np.broadcast_to(c, (2, 2, S, D)), "bf16")
    for mask, window in MASKS:
        say("constant v", mask, window)
        o_bits, _ = gpu_run(q, k, v, "bf16", 0.125, mask, window)
        o = decode(o_bits, "bf16")
        assert np.max(np.abs(o - c)) <= 2 ** -7, (mask, window)


def test_one_hot_dominant_key_copies_v_row():
    S, D = 128, 128
    target = np.array([max(0, i - (i * 7) % 11) for i in range(S)])   # target <= i
    Q = np.zeros((1, 1, S, D), np.float32)
    K = np.zeros((1, 1, S, D), np.float32)
    for j in range(S):
        K[0, 0, j, j % D] = 8.0
    for i in range(S):
        Q[0, 0, i, target[i] % D] = 8.0
    _, _, v = synth.make_qkv(1, 1, S, D, "f16", seed=33)
    say("one-hot dominant key")
    o_bits, _ = gpu_run(synth.f32_to_bits(Q, "f16"), synth.f32_to_bits(K, "f16"), v, "f16", 1.0,
                        "causal")
    o = decode(o_bits, "f16")[0, 0]
    vd = decode(v, "f16")[0, 0]
    assert np.max(np.abs(o - vd[target])) <= 2e-3


# ---------------------------------------------------------------------------
# properties of the launch

def test_deterministic_bitwise():
    q, k, v = synth.make_qkv(2, 8, 1500, 128, "f16", seed=41)
    say("determinism")
    a = gpu_run(q, k, v, "f16", 0.09, "causal")
    b = gpu_run(q, k, v, "f16", 0.09, "causal")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_heads_are_independent():
    B, H, S, D = 2, 8, 600, 64
    q, k, v = synth.make_qkv(B, H, S, D, "bf16", seed=42)
    say("slice independence")
    o_all, l_all = gpu_run(q, k, v, "bf16", 0.125, "window", (200, 10))
    for b, h in ((0, 0), (1, 5), (1, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o1, l1 = gpu_run(q[sl], k[sl], v[sl], "bf16", 0.125, "window", (200, 10))
        assert np.array_equal(o1[0, 0], o_all[b, h]) and np.array_equal(l1[0, 0], l_all[b, h])


def test_lse_pointer_may_be_null(orc):
    q, k, v = synth.make_qkv(1, 2, 300, 128, "f16", seed=43)
    say("null lse")
    o_bits, lse = gpu_run(q, k, v, "f16", 0.1, "causal", with_lse=False)
    assert lse is None
    o_ref, _ = orc.attention(q, k, v, "f16", 0.1, "causal")
    st = compare(o_bits, None, o_ref, None, "f16")
    assert st["pass"], st


@pytest.mark.parametrize("scale", [0.0, -0.1, 0.5])
def test_scale_sign_and_zero(orc, scale):
    q, k, v = synth.make_qkv(1, 2, 200, 64, "f16", seed=44)
    say("scale", scale)
    check_full(orc, q, k, v, "f16", scale, "window", (50, 5))


def test_empty_problems_do_nothing():
    say("empty")
    for shape in ((0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 0, 64)):
        t = torch.zeros(shape, dtype=torch.float16, device="cuda")
        o, lse = fa.forward(t, t, t, mask="causal")
        torch.cuda.synchronize()
        assert o.shape == shape and lse.shape == shape[:3]


def test_runs_on_a_side_stream(orc):
    q, k, v = synth.make_qkv(1, 2, 500, 128, "bf16", seed=45)
    say("side stream")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.forward(tq, tk, tv, scale=0.1, mask="causal")
    s.synchronize()
    o_ref, lse_ref = orc.attention(q, k, v, "bf16", 0.1, "causal")
    st = compare(to_bits(o), lse.cpu().numpy(), o_ref, lse_ref, "bf16")
    assert st["pass"], st
