"""fa_decode (new query rows against a key/value cache) against the fp64 oracle,
through the C ABI (needs a gfx950 GPU). Every case prints its name, shape and
seed before touching the GPU."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import compare, to_bits, to_device

pytestmark = pytest.mark.gpu

_MCODE = {"full": 0, "causal": 1, "window": 2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make(B, H, Sq, Sk, D, dtype, seed):
    q, _, _ = synth.make_qkv(B, H, Sq, D, dtype, seed)
    _, k, v = synth.make_qkv(B, H, Sk, D, dtype, seed + 1)
    return q, k, v


def run(q, k, v, dtype, scale, mask, window=(-1, -1), workspace=None):
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = fa.decode(tq, tk, tv, scale=scale, mask=mask, window=window, workspace=workspace)
    torch.cuda.synchronize()
    return to_bits(o), lse.cpu().numpy()


def check(orc, q, k, v, dtype, scale, mask, window=(-1, -1), workspace=None):
    o_bits, lse = run(q, k, v, dtype, scale, mask, window, workspace)
    o_ref, lse_ref = orc.attention_kv(q, k, v, dtype, scale, mask, window)
    st = compare(o_bits, lse, o_ref, lse_ref, dtype)
    assert st["pass"], st
    return o_bits, lse


def n_splits_used(B, H, Sq, Sk, D, mask, window):
    return fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, _MCODE[mask], *window) > 0


SHAPES = [  # B, H, Sq, Sk, D
    (1, 2, 1, 37, 64), (2, 3, 1, 1000, 128), (2, 2, 4, 4096, 128), (1, 4, 16, 777, 64),
    (1, 2, 32, 2000, 128), (2, 1, 7, 7, 128), (1, 3, 32, 32, 64), (3, 2, 5, 129, 128),
]
MASKS = [("causal", (-1, -1)), ("full", (-1, -1)), ("window", (100, 0)), ("window", (20, 3)),
         ("window", (-1, 2)), ("window", (0, 0))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask,window", MASKS, ids=str)
def test_decode_parity(orc, dtype, shape, mask, window):
    B, H, Sq, Sk, D = shape
    seed = 500 + Sq + Sk + D
    say("decode", dtype, shape, mask, window, "seed", seed,
        "split" if n_splits_used(B, H, Sq, Sk, D, mask, window) else "single")
    q, k, v = make(B, H, Sq, Sk, D, dtype, seed)
    check(orc, q, k, v, dtype, 1.0 / math.sqrt(D), mask, window)


def test_both_paths_are_exercised():
    assert n_splits_used(2, 2, 4, 4096, 128, "causal", (-1, -1))
    assert not n_splits_used(2, 1, 7, 7, 128, "causal", (-1, -1))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_decode_scales(orc, scale):
    say("decode scale", scale)
    q, k, v = make(1, 2, 3, 300, 128, "f16", seed=71)
    check(orc, q, k, v, "f16", scale, "causal")


def test_workspace_contents_do_not_matter(orc):
    B, H, Sq, Sk, D = 1, 4, 8, 3000, 128
    say("decode workspace reuse", B, H, Sq, Sk, D)
    need = fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, 1)
    assert need > 0
    ws = torch.full((need + 64,), 0x7F, dtype=torch.uint8, device="cuda")  # NaN-ish bytes
    q, k, v = make(B, H, Sq, Sk, D, "bf16", seed=72)
    a = check(orc, q, k, v, "bf16", 0.1, "causal", workspace=ws)
    b = check(orc, q, k, v, "bf16", 0.1, "causal", workspace=ws)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])  # deterministic


def test_short_workspace_is_rejected():
    B, H, Sq, Sk, D = 1, 4, 8, 3000, 128
    say("decode short workspace")
    need = fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, 1)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    q = torch.zeros(B, H, Sq, D, dtype=torch.float16, device="cuda")
    kv = torch.zeros(B, H, Sk, D, dtype=torch.float16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.decode(q, kv, kv.clone(), mask="causal", workspace=ws)
    assert e.value.status == -1


def test_square_case_matches_the_forward_rows(orc):
    """Sq == Sk: both entry points compute the same attention (different
    kernels; both within tolerance of the oracle)."""
    B, H, S, D = 1, 2, 24, 64
    say("decode square", B, H, S, D)
    q, k, v = synth.make_qkv(B, H, S, D, "f16", seed=73)
    o_d, lse_d = check(orc, q, k, v, "f16", 0.125, "causal")
    tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
    o_f, lse_f = fa.forward(tq, tk, tv, scale=0.125, mask="causal")
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention(q, k, v, "f16", 0.125, "causal")
    assert compare(to_bits(o_f), lse_f.cpu().numpy(), o_ref, lse_ref, "f16")["pass"]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_long_cache_sampled_heads(orc, dtype):
    """A serving-sized cache (Sk = 16384); the oracle runs on two of the heads."""
    B, H, Sq, Sk, D = 2, 8, 16, 16384, 128
    say("decode long", dtype, B, H, Sq, Sk, D)
    q, k, v = make(B, H, Sq, Sk, D, dtype, seed=74)
    o_bits, lse = run(q, k, v, dtype, 1.0 / math.sqrt(D), "causal")
    for (b, h) in ((0, 3), (1, 7)):
        o_ref, lse_ref = orc.attention_kv(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                          v[b:b + 1, h:h + 1], dtype, 1.0 / math.sqrt(D),
                                          "causal")
        st = compare(o_bits[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, lse_ref, dtype)
        assert st["pass"], (b, h, st)


# ---------------------------------------------------------------------------
# paged cache: pools [num_pages, page_size, H, D], a block table per sequence,
# per-sequence lengths; the oracle sees each sequence's contiguous cache

def build_pages(k, v, seq_lens, page_size, rng, extra_pages=3):
    """Scatter contiguous caches k, v [B, H, Sk, D] into randomly placed pages;
    unused table entries hold -1."""
    B, H, Sk, D = k.shape
    need = [(L + page_size - 1) // page_size for L in seq_lens]
    max_pages = max(max(need), 1) + 1
    num_pages = sum(need) + extra_pages
    order = rng.permutation(num_pages)
    kp = np.zeros((num_pages, page_size, H, D), np.uint16)
    vp = np.zeros_like(kp)
    table = np.full((B, max_pages), -1, np.int32)
    nxt = 0
    for b, L in enumerate(seq_lens):
        for j in range(need[b]):
            pg = int(order[nxt])
            nxt += 1
            table[b, j] = pg
            lo, hi = j * page_size, min(L, (j + 1) * page_size)
            kp[pg, :hi - lo] = k[b, :, lo:hi, :].transpose(1, 0, 2)
            vp[pg, :hi - lo] = v[b, :, lo:hi, :].transpose(1, 0, 2)
    return kp, vp, table


def run_paged(q, kp, vp, table, seq_lens, max_seq, dtype, scale, mask, window=(-1, -1)):
    tq, tkp, tvp = (to_device(x, dtype) for x in (q, kp, vp))
    tt = torch.from_numpy(table).cuda()
    tl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    o, lse = fa.decode_paged(tq, tkp, tvp, tt, tl, max_seq, scale=scale, mask=mask,
                             window=window)
    torch.cuda.synchronize()
    return to_bits(o), lse.cpu().numpy()


PAGED = [  # B, H, Sq, seq_lens, D, page_size
    (3, 2, 1, [37, 300, 1000], 128, 32),
    (2, 4, 4, [4, 2049], 128, 64),
    (4, 1, 16, [16, 100, 513, 4096], 64, 256),
    (2, 2, 32, [700, 33], 128, 128),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", PAGED, ids=lambda c: f"B{c[0]}H{c[1]}q{c[2]}d{c[4]}p{c[5]}")
@pytest.mark.parametrize("mask,window", [("causal", (-1, -1)), ("full", (-1, -1)),
                                         ("window", (200, 0)), ("window", (40, 5))], ids=str)
def test_paged_parity(orc, dtype, case, mask, window):
    B, H, Sq, seq_lens, D, ps = case
    max_seq = max(seq_lens)
    seed = 900 + Sq + D + ps
    say("paged", dtype, case, mask, window, "seed", seed)
    rng = np.random.default_rng(seed)
    q, k, v = make(B, H, Sq, max_seq, D, dtype, seed)
    kp, vp, table = build_pages(k, v, seq_lens, ps, rng)
    o_bits, lse = run_paged(q, kp, vp, table, seq_lens, max_seq, dtype, 0.1, mask, window)
    for b, L in enumerate(seq_lens):
        o_ref, lse_ref = orc.attention_kv(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                          dtype, 0.1, mask, window)
        st = compare(o_bits[b:b + 1], lse[b:b + 1], o_ref, lse_ref, dtype)
        assert st["pass"], (b, L, st)


def test_paged_short_sequence_rows_see_nothing(orc):
    """seq_len < Sq: rows at negative positions get O = 0 and LSE = -inf; the
    others attend over the keys they can see."""
    B, H, Sq, D, ps = 1, 2, 8, 64, 32
    seq_lens = [5]
    say("paged short", B, H, Sq, seq_lens)
    q, k, v = make(B, H, Sq, 40, D, "f16", seed=77)
    kp, vp, table = build_pages(k, v, seq_lens, ps, np.random.default_rng(1))
    o_bits, lse = run_paged(q, kp, vp, table, seq_lens, 40, "f16", 0.2, "causal")
    n_dead = Sq - seq_lens[0]
    assert np.all(o_bits[:, :, :n_dead] == 0) and np.all(lse[:, :, :n_dead] == -np.inf)
    o_ref, lse_ref = orc.attention_kv(q[:, :, n_dead:], k[:, :, :5], v[:, :, :5], "f16", 0.2,
                                      "causal")
    assert compare(o_bits[:, :, n_dead:], lse[:, :, n_dead:], o_ref, lse_ref, "f16")["pass"]


def test_paged_bad_page_index_reads_zero_keys(orc):
    """A table entry outside the pool makes that page's keys and values zero."""
    B, H, Sq, D, ps = 1, 2, 2, 128, 32
    seq_lens = [96]
    say("paged bad page", B, H, Sq, seq_lens)
    q, k, v = make(B, H, Sq, 96, D, "f16", seed=78)
    kp, vp, table = build_pages(k, v, seq_lens, ps, np.random.default_rng(2))
    table[0, 1] = kp.shape[0] + 5  # the second page: keys 32 .. 63
    o_bits, lse = run_paged(q, kp, vp, table, seq_lens, 96, "f16", 0.1, "full")
    k0, v0 = k.copy(), v.copy()
    k0[:, :, 32:64] = 0
    v0[:, :, 32:64] = 0
    o_ref, lse_ref = orc.attention_kv(q, k0, v0, "f16", 0.1, "full")
    assert compare(o_bits, lse, o_ref, lse_ref, "f16")["pass"]


def test_paged_equals_contiguous_bitwise():
    """One sequence whose pages are in order is the contiguous cache: same
    kernel, same tiles, so the same bits."""
    B, H, Sq, Sk, D, ps = 1, 1, 3, 512, 128, 64
    say("paged vs contiguous", B, H, Sq, Sk)
    q, k, v = make(B, H, Sq, Sk, D, "bf16", seed=79)
    kp = k[0].transpose(1, 0, 2).reshape(Sk // ps, ps, H, D).copy()
    vp = v[0].transpose(1, 0, 2).reshape(Sk // ps, ps, H, D).copy()
    table = np.arange(Sk // ps, dtype=np.int32)[None, :]
    a = run_paged(q, kp, vp, table, [Sk], Sk, "bf16", 0.1, "causal")
    b = run(q, k, v, "bf16", 0.1, "causal")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
