"""Pins for the fp64 CPU oracle: checks against things other than itself.

Each ``pin_*`` function takes a loaded oracle and raises AssertionError when
the oracle disagrees with a closed form, an invariant, a special case that
reduces to a library routine, or the pages' printed numbers. They are plain
functions (not tests) so that the suite can also run them against copies of
the oracle with a deliberate mistake built in and show that one of them fails.
"""
import json
import math
import os

import numpy as np
import torch

from synth import f32_to_bits, make_qkv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASK_CASES = [
    ("full", (-1, -1)),
    ("causal", (-1, -1)),
    ("window", (3, 0)),
    ("window", (0, 2)),
    ("window", (5, 7)),
    ("window", (-1, 4)),
    ("window", (6, -1)),
]


def _bits(x, dtype="f16"):
    return f32_to_bits(np.asarray(x, dtype=np.float32), dtype)


def _decode_ref(bits, dtype):
    """Decode with library routines (numpy's float16, torch's bfloat16)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.double().numpy()


def _bool_mask(S, mask, window):
    """Visibility as a boolean [S, S] matrix, built with numpy index arithmetic."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    if mask == "full":
        return np.ones((S, S), dtype=bool)
    if mask == "causal":
        return j <= i
    wl, wr = window
    ok = np.ones((S, S), dtype=bool)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


# --------------------------------------------------------------------------
# encodings


def pin_decoders(orc):
    """Every fp16 and bf16 bit pattern decodes as numpy / torch decode it."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        got = orc.decode(allbits, dtype)
        ref = _decode_ref(allbits, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dtype
        assert np.array_equal(got[~nan], ref[~nan]), dtype
        # signed zeros keep their sign
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), dtype


# --------------------------------------------------------------------------
# mask predicate and pair counts


def _window_count_closed(S, wl, wr):
    """Per-row count of an inclusive window, summed (no pair enumeration)."""
    total = 0
    for i in range(S):
        lo = 0 if wl < 0 else max(0, i - wl)
        hi = S - 1 if wr < 0 else min(S - 1, i + wr)
        total += max(0, hi - lo + 1)
    return total


def pin_pair_counts(orc):
    """Pair counts: S^2, S(S+1)/2, the causal-window closed form, mirror symmetry."""
    for S in (1, 2, 3, 63, 64, 65, 127, 128, 129, 300):
        assert orc.pair_count(S, "full") == S * S
        assert orc.pair_count(S, "causal") == S * (S + 1) // 2
        assert orc.pair_count(S, "window", (-1, -1)) == S * S
        assert orc.pair_count(S, "window", (-1, 0)) == S * (S + 1) // 2
        for wl in (0, 1, 63, 64, 65, S - 1):
            if 0 <= wl < S:
                closed = wl * (wl + 1) // 2 + (S - wl) * (wl + 1)
                assert orc.pair_count(S, "window", (wl, 0)) == closed, (S, wl)
        for wl in (-1, 0, 1, 5, 64, S, S + 5):
            for wr in (-1, 0, 2, 65, S + 1):
                c = orc.pair_count(S, "window", (wl, wr))
                assert c == _window_count_closed(S, wl, wr), (S, wl, wr)
                # reversing the sequence swaps the two window sides
                assert c == orc.pair_count(S, "window", (wr, wl)), (S, wl, wr)


def pin_page_numbers(orc):
    """Numbers the pages print (tests/golden/page_numbers.json)."""
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        items = json.load(f)
    by_key = {it["key"]: it for it in items}
    n = orc.pair_count(4096, "full")
    assert n == by_key["full_scores_s4096"]["value"]
    assert n * 4 == by_key["fp32_score_bytes_s4096"]["value"]
    assert 1.0 / math.sqrt(64) == by_key["scale_d64"]["value"]


# --------------------------------------------------------------------------
# attention values


def pin_sdpa(orc):
    """Matches torch's CPU fp64 scaled_dot_product_attention with a boolean mask,
    and torch.logsumexp of the masked scaled scores for the LSE."""
    rng = np.random.default_rng(11)
    for dtype in ("f16", "bf16"):
        for (S, D) in ((1, 8), (5, 8), (37, 16), (64, 64), (100, 32)):
            q, k, v = make_qkv(2, 2, S, D, dtype, seed=int(rng.integers(1 << 30)))
            qd = torch.from_numpy(_decode_ref(q, dtype))
            kd = torch.from_numpy(_decode_ref(k, dtype))
            vd = torch.from_numpy(_decode_ref(v, dtype))
            for mask, window in MASK_CASES:
                scale = 1.0 / math.sqrt(D) if mask != "window" else 0.3
                bm = torch.from_numpy(_bool_mask(S, mask, window))
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qd, kd, vd, attn_mask=bm, scale=scale).numpy()
                scores = torch.matmul(qd, kd.transpose(-1, -2)) * scale
                scores = scores.masked_fill(~bm, float("-inf"))
                lse_ref = torch.logsumexp(scores, dim=-1).numpy()
                o, lse = orc.attention(q, k, v, dtype, scale, mask, window)
                assert np.max(np.abs(o - ref)) < 1e-12, (dtype, S, D, mask, window)
                assert np.max(np.abs(lse - lse_ref)) < 1e-12, (dtype, S, D, mask, window)


def pin_uniform_weights(orc):
    """Q = 0 makes every visible key weigh the same: O_i is the mean of the
    visible V rows (prefix means for causal) and LSE_i = ln(count_i)."""
    S, D = 50, 16
    _, _, v = make_qkv(1, 1, S, D, "f16", seed=5)
    q = np.zeros_like(v)
    _, k, _ = make_qkv(1, 1, S, D, "f16", seed=6)
    vd = _decode_ref(v, "f16")[0, 0]
    for mask, window in MASK_CASES + [("window", (10, 0))]:
        vis = _bool_mask(S, mask, window)
        cnt = vis.sum(axis=1)
        means = (vis.astype(np.float64) @ vd) / cnt[:, None]
        if mask == "causal":
            prefix = np.cumsum(vd, axis=0) / np.arange(1, S + 1)[:, None]
            assert np.max(np.abs(means - prefix)) < 1e-12
        o, lse = orc.attention(q, k, v, "f16", 0.7, mask, window)
        assert np.max(np.abs(o[0, 0] - means)) < 1e-12, (mask, window)
        assert np.max(np.abs(lse[0, 0] - np.log(cnt))) < 1e-12, (mask, window)
    # scale = 0 with nonzero Q is the same case
    qn, _, _ = make_qkv(1, 1, S, D, "f16", seed=7)
    o0, lse0 = orc.attention(qn, k, v, "f16", 0.0, "causal")
    prefix = np.cumsum(vd, axis=0) / np.arange(1, S + 1)[:, None]
    assert np.max(np.abs(o0[0, 0] - prefix)) < 1e-12
    assert np.max(np.abs(lse0[0, 0] - np.log(np.arange(1, S + 1)))) < 1e-12


def pin_constant_v(orc):
    """V rows all equal to one vector c give O_i = c for every row and mask."""
    S, D = 40, 8
    q, k, _ = make_qkv(1, 2, S, D, "f16", seed=8)
    c = np.array([1.5, -2.0, 0.25, 3.0, 0.0, -0.5, 7.0, 1.0], dtype=np.float32)
    v = _bits(np.broadcast_to(c, (1, 2, S, D)))
    for mask, window in MASK_CASES:
        o, _ = orc.attention(q, k, v, "f16", 0.35, mask, window)
        assert np.max(np.abs(o - c.astype(np.float64))) < 1e-14, (mask, window)


def pin_single_visible_key(orc):
    """Causal row 0 sees only key 0: O_0 = V_0 exactly, LSE_0 = scale*q_0.k_0."""
    S, D = 9, 16
    q, k, v = make_qkv(1, 1, S, D, "f16", seed=9)
    scale = 0.25
    o, lse = orc.attention(q, k, v, "f16", scale, "causal")
    qd, kd, vd = (_decode_ref(x, "f16")[0, 0] for x in (q, k, v))
    assert np.array_equal(o[0, 0, 0], vd[0])
    assert abs(lse[0, 0, 0] - scale * float(np.dot(qd[0], kd[0]))) < 1e-12
    # window (0, 0) sees only the key at the same position: O_i = V_i
    o, _ = orc.attention(q, k, v, "f16", scale, "window", (0, 0))
    assert np.array_equal(o[0, 0], vd)


def pin_one_hot_dominant(orc):
    """One visible key scoring 64 above every other copies that key's V row."""
    S, D = 12, 16
    target = [0, 0, 1, 3, 2, 5, 6, 0, 8, 4, 10, 11]   # target[i] <= i: causal-visible
    K = np.zeros((S, D), np.float32)
    Q = np.zeros((S, D), np.float32)
    for j in range(S):
        K[j, j] = 8.0
    for i in range(S):
        Q[i, target[i]] = 8.0
    _, _, v = make_qkv(1, 1, S, D, "f16", seed=10)
    q = _bits(Q[None, None])
    k = _bits(K[None, None])
    vd = _decode_ref(v, "f16")[0, 0]
    for mask in ("causal", "full"):
        o, lse = orc.attention(q, k, v, "f16", 1.0, mask)
        for i in range(S):
            nvis = (i + 1) if mask == "causal" else S
            assert np.max(np.abs(o[0, 0, i] - vd[target[i]])) <= 1e-15, (mask, i)
            expect = 64.0 + math.log1p((nvis - 1) * math.exp(-64.0))
            assert abs(lse[0, 0, i] - expect) < 1e-12, (mask, i)


def pin_two_keys(orc):
    """S = 2, full mask: O_0 = sigmoid(s00 - s01) V_0 + sigmoid(s01 - s00) V_1."""
    D = 8
    q, k, v = make_qkv(1, 1, 2, D, "f16", seed=12)
    qd, kd, vd = (_decode_ref(x, "f16")[0, 0] for x in (q, k, v))
    scale = 0.9
    o, lse = orc.attention(q, k, v, "f16", scale, "full")
    for i in range(2):
        s0 = scale * float(np.dot(qd[i], kd[0]))
        s1 = scale * float(np.dot(qd[i], kd[1]))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.max(np.abs(o[0, 0, i] - (w0 * vd[0] + w1 * vd[1]))) < 1e-14
        assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) < 1e-13


def pin_shift_invariance(orc):
    """Adding one vector u to every key row leaves O unchanged and shifts
    LSE_i by scale*q_i.u (exactly representable integer-valued inputs)."""
    rng = np.random.default_rng(13)
    S, D = 30, 8
    Q = rng.integers(-3, 4, size=(1, 1, S, D)).astype(np.float32)
    K = rng.integers(-3, 4, size=(1, 1, S, D)).astype(np.float32)
    u = rng.integers(-2, 3, size=D).astype(np.float32)
    _, _, v = make_qkv(1, 1, S, D, "f16", seed=14)
    scale = 0.125
    for mask, window in MASK_CASES:
        o1, l1 = orc.attention(_bits(Q), _bits(K), v, "f16", scale, mask, window)
        o2, l2 = orc.attention(_bits(Q), _bits(K + u), v, "f16", scale, mask, window)
        shift = scale * (Q[0, 0].astype(np.float64) @ u.astype(np.float64))
        assert np.max(np.abs(o1 - o2)) < 1e-12, (mask, window)
        assert np.max(np.abs((l2 - l1)[0, 0] - shift)) < 1e-12, (mask, window)


def pin_permutation(orc):
    """Full mask: permuting the (K, V) rows together changes nothing."""
    S, D = 33, 16
    q, k, v = make_qkv(1, 2, S, D, "bf16", seed=15)
    perm = np.random.default_rng(16).permutation(S)
    o1, l1 = orc.attention(q, k, v, "bf16", 0.2, "full")
    o2, l2 = orc.attention(q, k[:, :, perm], v[:, :, perm], "bf16", 0.2, "full")
    assert np.max(np.abs(o1 - o2)) < 1e-13
    assert np.max(np.abs(l1 - l2)) < 1e-13


def pin_linearity_in_v(orc):
    """O(2 V1 - V2) = 2 O(V1) - O(V2) (integer-valued V, exact in fp16)."""
    rng = np.random.default_rng(17)
    S, D = 26, 8
    q, k, _ = make_qkv(1, 1, S, D, "f16", seed=18)
    V1 = rng.integers(-8, 9, size=(1, 1, S, D)).astype(np.float32)
    V2 = rng.integers(-8, 9, size=(1, 1, S, D)).astype(np.float32)
    for mask, window in MASK_CASES:
        a, _ = orc.attention(q, k, _bits(V1), "f16", 0.3, mask, window)
        b, _ = orc.attention(q, k, _bits(V2), "f16", 0.3, mask, window)
        c, _ = orc.attention(q, k, _bits(2 * V1 - V2), "f16", 0.3, mask, window)
        assert np.max(np.abs(c - (2 * a - b))) < 1e-12, (mask, window)


def pin_mask_equivalences(orc):
    """window(-1,-1) = full, window(-1,0) = causal, window(S-1,0) = causal,
    window(S-1,S-1) = full, bit for bit."""
    S, D = 45, 16
    q, k, v = make_qkv(2, 1, S, D, "f16", seed=19)
    full = orc.attention(q, k, v, "f16", 0.25, "full")
    causal = orc.attention(q, k, v, "f16", 0.25, "causal")
    for window, ref in (((-1, -1), full), ((-1, 0), causal), ((S - 1, 0), causal),
                        ((S - 1, S - 1), full), ((S + 3, -1), full)):
        got = orc.attention(q, k, v, "f16", 0.25, "window", window)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), window


def pin_probabilities(orc):
    """The materialised probability rows sum to 1, vanish where masked, and
    P @ V (numpy) reproduces O."""
    S, D = 24, 8
    q, k, v = make_qkv(1, 1, S, D, "f16", seed=20)
    vd = _decode_ref(v, "f16")[0, 0]
    for mask, window in MASK_CASES:
        p, o, _ = orc.attention_probs(q[0, 0], k[0, 0], v[0, 0], "f16", 0.5, mask, window)
        vis = _bool_mask(S, mask, window)
        assert np.all(p[~vis] == 0.0), (mask, window)
        assert np.all(p[vis] > 0.0), (mask, window)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14, (mask, window)
        assert np.max(np.abs(p @ vd - o)) < 1e-13, (mask, window)


def pin_scale_is_a_multiplier(orc):
    """Doubling the scale equals doubling Q (exact in fp16)."""
    S, D = 20, 8
    rng = np.random.default_rng(21)
    Q = rng.integers(-4, 5, size=(1, 1, S, D)).astype(np.float32)
    _, k, v = make_qkv(1, 1, S, D, "f16", seed=22)
    a = orc.attention(_bits(Q), k, v, "f16", 0.25, "causal")
    b = orc.attention(_bits(2 * Q), k, v, "f16", 0.125, "causal")
    assert np.max(np.abs(a[0] - b[0])) < 1e-12 and np.max(np.abs(a[1] - b[1])) < 1e-12


# --------------------------------------------------------------------------
# new rows against a key/value cache (incremental decoding)

KV_SHAPES = [(1, 1), (1, 37), (3, 3), (5, 64), (16, 100), (16, 16), (32, 70)]


def _bool_mask_kv(Sq, Sk, mask, window):
    """Visibility of Sk cached keys from Sq new rows placed at the end of the
    sequence (row i at position Sk - Sq + i), with numpy index arithmetic."""
    i = (Sk - Sq) + np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    if mask == "full":
        return np.ones((Sq, Sk), dtype=bool)
    if mask == "causal":
        return j <= i
    wl, wr = window
    ok = np.ones((Sq, Sk), dtype=bool)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


def pin_kv_sdpa(orc):
    """Cache attention matches torch's CPU fp64 scaled_dot_product_attention
    with a rectangular bottom-right boolean mask, and torch.logsumexp."""
    rng = np.random.default_rng(31)
    for dtype in ("f16", "bf16"):
        for (Sq, Sk) in KV_SHAPES:
            D = 16
            q, _, _ = make_qkv(2, 2, Sq, D, dtype, seed=int(rng.integers(1 << 30)))
            _, k, v = make_qkv(2, 2, Sk, D, dtype, seed=int(rng.integers(1 << 30)))
            qd = torch.from_numpy(_decode_ref(q, dtype))
            kd = torch.from_numpy(_decode_ref(k, dtype))
            vd = torch.from_numpy(_decode_ref(v, dtype))
            for mask, window in MASK_CASES:
                bm = _bool_mask_kv(Sq, Sk, mask, window)
                if not bm.any(axis=1).all():
                    continue  # a row with no visible key: covered by the definition only
                scale = 0.35
                bmt = torch.from_numpy(bm)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qd, kd, vd, attn_mask=bmt, scale=scale).numpy()
                scores = torch.matmul(qd, kd.transpose(-1, -2)) * scale
                lse_ref = torch.logsumexp(scores.masked_fill(~bmt, float("-inf")), dim=-1).numpy()
                o, lse = orc.attention_kv(q, k, v, dtype, scale, mask, window)
                assert np.max(np.abs(o - ref)) < 1e-12, (dtype, Sq, Sk, mask, window)
                assert np.max(np.abs(lse - lse_ref)) < 1e-12, (dtype, Sq, Sk, mask, window)


def pin_varlen_block_diagonal_sdpa(orc):
    """Packed sequences match torch's CPU fp64 scaled_dot_product_attention
    over the whole packed batch, per head, with a block-diagonal boolean mask
    (the mask rule applied to each block's own row numbers), and
    torch.logsumexp; tokens in no sequence stay NaN."""
    from synth import cu_seqlens_of, make_varlen_qkv
    for dtype in ("f16", "bf16"):
        for lengths, extra in (([5, 1, 9, 0, 12], 0), ([17], 3), ([3, 3, 3, 3], 2)):
            cu = cu_seqlens_of(lengths)
            T = int(cu[-1]) + extra
            q, k, v = make_varlen_qkv(T, 2, 8, dtype, seed=40 + T)
            seq = np.full(T, -1)
            row = np.zeros(T, dtype=np.int64)
            for b, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
                seq[a:e] = b
                row[a:e] = np.arange(e - a)
            qd, kd, vd = (torch.from_numpy(_decode_ref(x, dtype)).transpose(0, 1) for x in (q, k, v))
            for mask, window in MASK_CASES:
                same = (seq[:, None] == seq[None, :]) & (seq[:, None] >= 0)
                bm = same & _bool_mask_kv(T, T, mask, window)  # row i vs key j, positions
                # _bool_mask_kv at Sq == Sk compares token indices; within one
                # block those differ from the row numbers by the same offset.
                if not bm[seq >= 0].any(axis=1).all():
                    continue  # a row with no visible key: covered by the definition only
                bmt = torch.from_numpy(bm)
                keep = torch.from_numpy(seq >= 0)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qd[:, keep], kd, vd, attn_mask=bmt[keep], scale=0.4).numpy()
                scores = torch.matmul(qd, kd.transpose(-1, -2)) * 0.4
                lse_ref = torch.logsumexp(scores.masked_fill(~bmt, float("-inf")), dim=-1)
                o, lse = orc.attention_varlen(q, k, v, cu, dtype, 0.4, mask, window)
                got = np.ascontiguousarray(o[seq >= 0].transpose(1, 0, 2))
                assert np.max(np.abs(got - ref)) < 1e-12, (dtype, lengths, mask, window)
                assert np.max(np.abs(lse[seq >= 0] - lse_ref.numpy().T[seq >= 0])) < 1e-12
                assert np.isnan(o[seq < 0]).all() and np.isnan(lse[seq < 0]).all()


def _rope_complex(xd, pos, cos, sin, mode):
    """RoPE through complex multiplication: pair t of a row (halves: dims t and
    t + D/2; interleaved: dims 2t and 2t + 1) read as the complex number
    x_a + i x_b, times c + i s from the tables at the row's position."""
    D = xd.shape[-1]
    if mode == "halves":
        z = xd[..., : D // 2] + 1j * xd[..., D // 2:]
    else:
        z = xd[..., 0::2] + 1j * xd[..., 1::2]
    w = cos.astype(np.float64)[pos] + 1j * sin.astype(np.float64)[pos]
    z = z * w
    out = np.empty_like(xd)
    if mode == "halves":
        out[..., : D // 2], out[..., D // 2:] = z.real, z.imag
    else:
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def pin_pure_python(orc):
    """The oracle against a per-element pure-Python evaluation of the
    definition (math.fsum for every sum, math.exp, Python floats decoded by
    numpy) on tiny shapes, every mask: within 1e-12."""
    rng = np.random.default_rng(44)
    for dtype in ("f16", "bf16"):
        for S, D in ((1, 4), (5, 8), (12, 3)):
            q, k, v = make_qkv(1, 2, S, D, dtype, seed=int(rng.integers(1 << 30)))
            qd, kd, vd = (_decode_ref(x, dtype) for x in (q, k, v))
            for mask, window in MASK_CASES:
                vis = _bool_mask_kv(S, S, mask, window)
                o, lse = orc.attention(q, k, v, dtype, 0.3, mask, window)
                for h in range(2):
                    for i in range(S):
                        js = [j for j in range(S) if vis[i, j]]
                        sc = {j: 0.3 * math.fsum(float(qd[0, h, i, d]) * float(kd[0, h, j, d])
                                                 for d in range(D)) for j in js}
                        m = max(sc.values())
                        e = {j: math.exp(sc[j] - m) for j in js}
                        den = math.fsum(e.values())
                        for d in range(D):
                            ref = math.fsum(e[j] * float(vd[0, h, j, d]) for j in js) / den
                            assert abs(o[0, h, i, d] - ref) <= 1e-12 * max(1.0, abs(ref))
                        assert abs(lse[0, h, i] - (m + math.log(den))) <= 1e-12 * max(1.0, abs(m))


def pin_rope_is_complex_rotation(orc):
    """RoPE of a row equals multiplying each of its pairs, read as a complex
    number, by cos + i sin of the row's position (random angles), in both
    pairings; it keeps every pair's length."""
    rng = np.random.default_rng(33)
    for dtype in ("f16", "bf16"):
        for D in (8, 64, 128):
            ang = rng.uniform(-7.0, 7.0, (11, D // 2))
            cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
            x, _, _ = make_qkv(1, 1, 20, D, dtype, seed=int(rng.integers(1 << 30)))
            x = x[0, 0]
            pos = rng.integers(0, 11, 20)
            xd = _decode_ref(x, dtype)
            for mode in ("halves", "interleaved"):
                got = orc.rope(x, pos, cos, sin, mode, dtype)
                ref = _rope_complex(xd, pos, cos, sin, mode)
                assert np.max(np.abs(got - ref)) < 1e-12, (dtype, D, mode)
                assert abs(np.sum(got ** 2) - np.sum(xd ** 2)) < 1e-6 * np.sum(xd ** 2) + 1e-9


def pin_round_to_element_type(orc):
    """Rounding to fp16 matches numpy's float64 -> float16 conversion (round to
    nearest even, subnormals, overflow); rounding to bf16 matches torch's
    float32 -> bfloat16 conversion on float32 values, and exact halfway cases
    and their neighbours 2^-40 away round to even / to the nearer value."""
    rng = np.random.default_rng(36)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
                        [0.0, -0.0, 65504.0, 65519.9, 65520.0, -7e4, 2.0 ** -25, 3 * 2.0 ** -26,
                         2.0 ** -24 * 1.5, 1e-9]])
    got = orc.round_to(x, "f16")
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    x32 = (rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000)).astype(np.float32)
    got = orc.round_to(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref)
    # bf16 values 1 + k/128 are spaced 2^-7 apart near 1: halfway cases round to even
    for k in range(0, 10):
        lo = 1.0 + k / 128.0
        mid = lo + 2.0 ** -8
        even = lo if k % 2 == 0 else lo + 2.0 ** -7
        assert orc.round_to([mid], "bf16")[0] == even
        assert orc.round_to([mid + 2.0 ** -40], "bf16")[0] == lo + 2.0 ** -7
        assert orc.round_to([mid - 2.0 ** -40], "bf16")[0] == lo


def pin_rope_attention_sdpa(orc):
    """RoPE attention equals torch's CPU fp64 scaled_dot_product_attention of
    the q and k rows rotated (by complex multiplication) at their positions and
    rounded to the element type (numpy for fp16, the oracle's pinned rounding
    for bf16), with the mask, and torch.logsumexp; tables from the usual
    frequency ladder."""
    from synth import rope_tables
    for dtype in ("f16", "bf16"):
        for mode in ("halves", "interleaved"):
            S, D = 37, 16
            q, k, v = make_qkv(1, 2, S, D, dtype, seed=34)
            cos, sin = rope_tables(S + 5, D, base=100.0)
            pos = np.arange(S)

            def rounded(x):
                if dtype == "f16":
                    return x.astype(np.float16).astype(np.float64)
                return orc.round_to(x, "bf16")

            qd = torch.from_numpy(rounded(_rope_complex(_decode_ref(q, dtype), pos, cos, sin,
                                                        mode)))
            kd = torch.from_numpy(rounded(_rope_complex(_decode_ref(k, dtype), pos, cos, sin,
                                                        mode)))
            vd = torch.from_numpy(_decode_ref(v, dtype))
            for mask, window in MASK_CASES:
                bm = torch.from_numpy(_bool_mask_kv(S, S, mask, window))
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qd, kd, vd, attn_mask=bm, scale=0.3).numpy()
                sc = torch.matmul(qd, kd.transpose(-1, -2)) * 0.3
                lse_ref = torch.logsumexp(sc.masked_fill(~bm, float("-inf")), dim=-1).numpy()
                o, lse = orc.attention_rope(q, k, v, dtype, 0.3, mask, window, cos, sin, mode)
                assert np.max(np.abs(o - ref)) < 1e-12, (dtype, mode, mask, window)
                assert np.max(np.abs(lse - lse_ref)) < 1e-12, (dtype, mode, mask, window)


def pin_rope_zero_angle_is_plain_attention(orc):
    """Tables of angle 0 (cos 1, sin 0) give the plain attention exactly."""
    q, k, v = make_qkv(2, 2, 50, 32, "f16", seed=35)
    cos, sin = np.ones((50, 16), np.float32), np.zeros((50, 16), np.float32)
    for mode in ("halves", "interleaved"):
        o, lse = orc.attention_rope(q, k, v, "f16", 0.2, "causal", (-1, -1), cos, sin, mode)
        o0, lse0 = orc.attention(q, k, v, "f16", 0.2, "causal")
        assert np.array_equal(o, o0) and np.array_equal(lse, lse0)


def pin_bwd_autograd(orc):
    """The gradients equal torch autograd through fp64 scaled_dot_product_attention
    (CPU) with the mask; every magnitude sum bounds its gradient."""
    rng = np.random.default_rng(37)
    for dtype in ("f16", "bf16"):
        for S in (1, 9, 37):
            q, k, v = make_qkv(2, 2, S, 16, dtype, seed=int(rng.integers(1 << 30)))
            do, _, _ = make_qkv(2, 2, S, 16, dtype, seed=int(rng.integers(1 << 30)))
            for mask, window in MASK_CASES:
                bm = torch.from_numpy(_bool_mask_kv(S, S, mask, window))
                t = [torch.from_numpy(_decode_ref(x, dtype)).requires_grad_(True)
                     for x in (q, k, v)]
                o = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=bm,
                                                                     scale=0.45)
                o.backward(torch.from_numpy(_decode_ref(do, dtype)))
                (dq, dk, dv), mags = orc.attention_bwd(q, k, v, do, dtype, 0.45, mask, window)
                for got, ref in zip((dq, dk, dv), t):
                    assert np.max(np.abs(got - ref.grad.numpy())) < 1e-11, (dtype, S, mask, window)
                for g, m in zip((dq, dk, dv), mags):
                    assert np.all(np.abs(g) <= m * (1 + 1e-12) + 1e-300)


def pin_bwd_magnitude_sums(orc):
    """The magnitude sums that set the backward comparison rule, evaluated
    independently: P from torch's softmax of the masked fp64 scores, dS as
    torch autograd's gradient of the loss sum(O * dO) with respect to the
    scaled-score matrix, A_i = sum_d |dO_id O_id| with O = P V, and the three
    sums as numpy matrix products over the visible pairs, each operand of a
    rounded product (P, dS) floored at the element type's smallest normal:
      mag_dV = (max(P, t) on visible pairs)^T |dO|,
      mag_dQ = |scale| (max(|dS|, t) + P A) |K|,   mag_dK = |scale| (...)^T |Q|."""
    rng = np.random.default_rng(44)
    for dtype, tiny in (("f16", 2.0 ** -14), ("bf16", 2.0 ** -126)):
        for S, scale in ((1, 0.45), (11, 0.45), (29, -0.8)):
            q, k, v = make_qkv(1, 2, S, 8, dtype, seed=int(rng.integers(1 << 30)))
            do, _, _ = make_qkv(1, 2, S, 8, dtype, seed=int(rng.integers(1 << 30)))
            Q, K, V, dO = (_decode_ref(x, dtype) for x in (q, k, v, do))
            for mask, window in MASK_CASES:
                vis = _bool_mask_kv(S, S, mask, window)
                _, mags = orc.attention_bwd(q, k, v, do, dtype, scale, mask, window)
                for h in range(2):
                    s = torch.from_numpy(Q[0, h] @ K[0, h].T * scale).requires_grad_(True)
                    P = torch.softmax(s.masked_fill(~torch.from_numpy(vis), -math.inf), dim=1)
                    O = P @ torch.from_numpy(V[0, h])
                    (O * torch.from_numpy(dO[0, h])).sum().backward()
                    Pn = P.detach().numpy()
                    dS = s.grad.numpy()
                    A = np.abs(dO[0, h] * O.detach().numpy()).sum(axis=1)
                    wv = np.where(vis, np.maximum(Pn, tiny), 0.0)
                    wqk = np.where(vis, np.maximum(np.abs(dS), tiny) + Pn * A[:, None], 0.0)
                    ref_dv = wv.T @ np.abs(dO[0, h])
                    ref_dq = abs(scale) * (wqk @ np.abs(K[0, h]))
                    ref_dk = abs(scale) * (wqk.T @ np.abs(Q[0, h]))
                    for got, ref in zip(mags, (ref_dq, ref_dk, ref_dv)):
                        assert np.allclose(got[0, h], ref, rtol=1e-10, atol=1e-300), \
                            (dtype, S, mask, window, h)


def pin_bwd_closed_forms(orc):
    """Q = 0 (uniform weights): dV_j is the sum over the rows that see key j of
    dO_i divided by their visible-key count, and dK = 0 when V rows are all
    equal (dP is constant along each row, so dS = 0); constant K rows give
    dQ = 0 (each row of dS sums to zero); and sum(dQ * Q) = sum(dK * K)."""
    S, D = 23, 8
    _, k, v = make_qkv(1, 2, S, D, "f16", seed=38)
    do, _, _ = make_qkv(1, 2, S, D, "f16", seed=39)
    q0 = np.zeros_like(k)
    dod = _decode_ref(do, "f16")
    for mask, window in MASK_CASES:
        vis = _bool_mask_kv(S, S, mask, window)
        (dq, dk, dv), _ = orc.attention_bwd(q0, k, v, do, "f16", 0.7, mask, window)
        w = vis / vis.sum(axis=1, keepdims=True)          # uniform weights per row
        ref = np.einsum("ij,bhid->bhjd", w, dod)
        assert np.max(np.abs(dv - ref)) < 1e-12, (mask, window)
    vconst = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
    (dq, dk, dv), _ = orc.attention_bwd(k, k, vconst, do, "f16", 0.7, "causal")
    assert np.max(np.abs(dk)) < 1e-12 and np.max(np.abs(dq)) < 1e-12
    kconst = np.broadcast_to(k[:, :, :1, :], k.shape).copy()
    q, _, _ = make_qkv(1, 2, S, D, "f16", seed=40)
    (dq, dk, dv), _ = orc.attention_bwd(q, kconst, v, do, "f16", 0.7, "full")
    assert np.max(np.abs(dq)) < 1e-12
    (dq, dk, dv), _ = orc.attention_bwd(q, k, v, do, "f16", 0.7, "window", (5, 2))
    lhs = np.sum(dq * _decode_ref(q, "f16"))
    rhs = np.sum(dk * _decode_ref(k, "f16"))
    assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


def pin_kv_rope_is_the_tail_of_the_square_case(orc):
    """New rows against a cache of rotated keys give the last rows of the square
    RoPE attention when the cache holds the square case's keys rotated and
    rounded (numpy complex rotation, numpy float16 rounding); zero angles give
    the plain cache attention."""
    from synth import rope_tables
    Sk, D = 40, 16
    for mode in ("halves", "interleaved"):
        Q, K, V = make_qkv(1, 2, Sk, D, "f16", seed=41)
        cos, sin = rope_tables(Sk + 3, D, base=50.0)
        krot = _rope_complex(_decode_ref(K, "f16"), np.arange(Sk), cos, sin, mode)
        kbits = f32_to_bits(krot.astype(np.float16).astype(np.float32), "f16")
        o_sq, lse_sq = orc.attention_rope(Q, K, V, "f16", 0.3, "causal", (-1, -1), cos, sin, mode)
        for Sq in (1, 5, Sk):
            q = np.ascontiguousarray(Q[:, :, Sk - Sq:, :])
            o, lse = orc.attention_kv_rope(q, kbits, V, "f16", 0.3, "causal", (-1, -1), cos, sin,
                                           mode)
            assert np.max(np.abs(o - o_sq[:, :, Sk - Sq:, :])) < 1e-12, (mode, Sq)
            assert np.max(np.abs(lse - lse_sq[:, :, Sk - Sq:])) < 1e-12, (mode, Sq)
    q, k, v = make_qkv(1, 2, 7, D, "bf16", seed=42)
    _, k2, v2 = make_qkv(1, 2, 30, D, "bf16", seed=43)
    one, zero = np.ones((30, D // 2), np.float32), np.zeros((30, D // 2), np.float32)
    o, lse = orc.attention_kv_rope(q, k2, v2, "bf16", 0.5, "window", (9, 0), one, zero, "halves")
    o0, lse0 = orc.attention_kv(q, k2, v2, "bf16", 0.5, "window", (9, 0))
    assert np.array_equal(o, o0) and np.array_equal(lse, lse0)


def pin_kv_is_the_tail_of_the_square_case(orc):
    """New rows at the end of a sequence give the last rows of the square
    problem whose query rows end with them (any earlier query rows)."""
    rng = np.random.default_rng(32)
    for (Sq, Sk) in ((1, 50), (7, 40), (16, 16)):
        Q, k, v = make_qkv(1, 3, Sk, 8, "f16", seed=int(rng.integers(1 << 30)))
        q = np.ascontiguousarray(Q[:, :, Sk - Sq:, :])
        for mask, window in (("causal", (-1, -1)), ("window", (4, 0)), ("full", (-1, -1))):
            o_sq, lse_sq = orc.attention(Q, k, v, "f16", 0.5, mask, window)
            o, lse = orc.attention_kv(q, k, v, "f16", 0.5, mask, window)
            assert np.max(np.abs(o - o_sq[:, :, Sk - Sq:, :])) < 1e-13, (Sq, Sk, mask)
            assert np.max(np.abs(lse - lse_sq[:, :, Sk - Sq:])) < 1e-13, (Sq, Sk, mask)


def pin_kv_uniform_weights(orc):
    """Q = 0: each new row's output is the plain mean of the V rows it can see,
    and its LSE is the log of how many there are (closed form, numpy)."""
    Sq, Sk, D = 6, 29, 8
    q = _bits(np.zeros((1, 1, Sq, D)))
    _, k, v = make_qkv(1, 1, Sk, D, "f16", seed=33)
    vd = _decode_ref(v, "f16")[0, 0]
    for mask, window in MASK_CASES:
        vis = _bool_mask_kv(Sq, Sk, mask, window)
        o, lse = orc.attention_kv(q, k, v, "f16", 0.7, mask, window)
        for i in range(Sq):
            n = int(vis[i].sum())
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-12, (mask, window, i)
            assert np.max(np.abs(o[0, 0, i] - vd[vis[i]].mean(axis=0))) < 1e-12, (mask, i)


ALL_PINS = [
    pin_decoders,
    pin_pair_counts,
    pin_page_numbers,
    pin_sdpa,
    pin_uniform_weights,
    pin_constant_v,
    pin_single_visible_key,
    pin_one_hot_dominant,
    pin_two_keys,
    pin_shift_invariance,
    pin_permutation,
    pin_linearity_in_v,
    pin_mask_equivalences,
    pin_probabilities,
    pin_scale_is_a_multiplier,
    pin_kv_sdpa,
    pin_kv_is_the_tail_of_the_square_case,
    pin_kv_uniform_weights,
    pin_varlen_block_diagonal_sdpa,
    pin_pure_python,
    pin_round_to_element_type,
    pin_rope_is_complex_rotation,
    pin_rope_attention_sdpa,
    pin_rope_zero_angle_is_plain_attention,
    pin_bwd_autograd,
    pin_bwd_closed_forms,
    pin_bwd_magnitude_sums,
    pin_kv_rope_is_the_tail_of_the_square_case,
]
