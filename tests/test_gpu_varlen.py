"""fa_fwd_varlen (packed variable-length sequences) against the fp64 oracle,
through the C ABI (needs a gfx950 GPU). Every case prints its name, lengths
and seed before touching the GPU."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import compare, to_bits, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0xFFFF  # a NaN in both fp16 and bf16


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run(q, k, v, cu, max_seqlen, dtype, scale, mask, window=(-1, -1)):
    """GPU output bits [T,H,D] and LSE [T,H], with o and lse pre-filled with NaN."""
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    out = to_device(np.full(q.shape, SENTINEL, np.uint16), dtype)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    tcu = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    fa.forward_varlen(tq, tk, tv, tcu, max_seqlen, scale=scale, mask=mask, window=window,
                      out=out, lse=lse)
    torch.cuda.synchronize()
    return to_bits(out), lse.cpu().numpy()


def covered(cu, T):
    m = np.zeros(T, dtype=bool)
    for a, b in zip(cu[:-1], cu[1:]):
        m[a:b] = True
    return m


def check(orc, lengths, extra, H, D, dtype, mask, window, seed, scale=None):
    cu = synth.cu_seqlens_of(lengths)
    T = int(cu[-1]) + extra
    q, k, v = synth.make_varlen_qkv(T, H, D, dtype, seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o_bits, lse = run(q, k, v, cu, max(lengths), dtype, scale, mask, window)
    o_ref, lse_ref = orc.attention_varlen(q, k, v, cu, dtype, scale, mask, window)
    m = covered(cu, T)
    st = compare(o_bits[m], lse[m], o_ref[m], lse_ref[m], dtype)
    assert st["pass"], st
    assert (o_bits[~m] == SENTINEL).all(), "a token outside every sequence was written"
    assert np.isnan(lse[~m]).all(), "an LSE outside every sequence was written"
    return q, k, v, cu, o_bits, lse


LENGTHS = [
    ([1000, 1, 257, 0, 256, 63], 37),   # one token, an empty sequence, tile edges, a tail
    ([300, 300, 300], 0),
    ([2048, 5], 3),                     # several query tiles next to a tiny sequence
    ([777], 0),
]
MASKS = [("full", (-1, -1)), ("causal", (-1, -1)), ("window", (100, 0)),
         ("window", (37, 50)), ("window", (-1, 20))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lengths,extra", LENGTHS, ids=lambda x: str(x))
@pytest.mark.parametrize("mask,window", MASKS, ids=str)
def test_varlen_parity(orc, dtype, D, lengths, extra, mask, window):
    seed = 900 + sum(lengths) + D
    say("varlen", dtype, D, lengths, "+", extra, mask, window, "seed", seed)
    check(orc, lengths, extra, 3, D, dtype, mask, window, seed)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_each_sequence_is_bitwise_the_dense_call(dtype):
    """Sequence b of a packed call gives, bit for bit, what fa_fwd gives for
    that sequence in [1, H', L, D] layout when fa_fwd also runs 256-row items
    (the packed layout always does): the sequence's H heads are repeated to
    H' = 512 heads, enough items that the dense call keeps that layout, and
    every repeat must equal the packed result. (Bounded-left windows, and
    dense calls with fewer than two 256-row items per CU, run the key-split
    layout, whose merge orders the additions differently; those meet the
    oracle instead, in the parity tests.)"""
    lengths = [513, 1, 256, 90, 1200]
    cu = synth.cu_seqlens_of(lengths)
    T, H, D = int(cu[-1]), 4, 128
    reps = 128
    say("varlen vs dense", dtype, lengths)
    q, k, v = synth.make_varlen_qkv(T, H, D, dtype, seed=77)
    for mask, window in (("causal", (-1, -1)), ("full", (-1, -1)), ("window", (-1, 10))):
        o_bits, lse = run(q, k, v, cu, max(lengths), dtype, 0.09, mask, window)
        for a, b in zip(cu[:-1], cu[1:]):
            def head_major(x):
                hm = np.ascontiguousarray(x[a:b].transpose(1, 0, 2))       # [H, L, D]
                return to_device(np.ascontiguousarray(np.tile(hm, (reps, 1, 1)))[None], dtype)
            od, ld = fa.forward(head_major(q), head_major(k), head_major(v), scale=0.09,
                                mask=mask, window=window)
            torch.cuda.synchronize()
            dense = to_bits(od)[0].reshape(reps, H, b - a, D)
            ldn = ld.cpu().numpy()[0].reshape(reps, H, b - a)
            for r in (0, reps - 1):
                assert np.array_equal(o_bits[a:b], dense[r].transpose(1, 0, 2)), (a, b, mask, r)
                assert np.array_equal(lse[a:b].view(np.uint32),
                                      ldn[r].T.copy().view(np.uint32)), (a, b, mask, r)


def test_max_seqlen_bounds_every_sequence(orc):
    """A sequence longer than max_seqlen is attended over its first max_seqlen
    tokens only; its later tokens are not written."""
    lengths, max_seqlen = [700, 100], 500
    cu = synth.cu_seqlens_of(lengths)
    T, H, D = int(cu[-1]), 2, 64
    say("varlen max_seqlen", lengths, max_seqlen)
    q, k, v = synth.make_varlen_qkv(T, H, D, "f16", seed=78)
    o_bits, lse = run(q, k, v, cu, max_seqlen, "f16", 0.125, "causal")
    # sequence 0 cut to tokens 0..499; tokens 500..699 then form a piece of
    # their own in the reference, only to keep its indexing plain
    o_ref, lse_ref = orc.attention_varlen(q, k, v, [0, 500, 700, 800], "f16", 0.125, "causal")
    m = covered([0, 500], T) | covered([700, 800], T)
    st = compare(o_bits[m], lse[m], o_ref[m], lse_ref[m], "f16")
    assert st["pass"], st
    assert (o_bits[500:700] == SENTINEL).all() and np.isnan(lse[500:700]).all()


def test_offsets_past_the_tensors_are_clamped(orc):
    """cu_seqlens entries beyond total_tokens are clamped to it on the GPU."""
    T, H, D = 300, 2, 128
    cu = [0, 100, 1 << 20]
    say("varlen clamped offsets", cu, T)
    q, k, v = synth.make_varlen_qkv(T, H, D, "f16", seed=79)
    o_bits, lse = run(q, k, v, cu, 4096, "f16", 0.1, "causal")
    o_ref, lse_ref = orc.attention_varlen(q, k, v, [0, 100, 300], "f16", 0.1, "causal")
    st = compare(o_bits, lse, o_ref, lse_ref, "f16")
    assert st["pass"], st


def test_named_workload_sampled_rows(orc):
    """The packed 16384-token workload at full size, in the launch the
    benchmark times, on rows sampled from every sequence and head."""
    name = "varlen_h32_t16384_causal"
    w = synth.VARLEN_WORKLOADS[name]
    q, k, v, cu = synth.varlen_inputs(name)
    lengths = np.diff(cu)
    say(name, "lengths", list(lengths))
    o_bits, lse = run(q, k, v, cu, int(lengths.max()), w["dtype"], w["scale"], w["mask"],
                      w["window"])
    rng = np.random.default_rng(123)
    H, D = w["H"], w["D"]
    for a, b in zip(cu[:-1], cu[1:]):
        L = int(b - a)
        rows_i = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 6)]))
        heads = rng.integers(0, H, rows_i.size)
        flat = heads * L + rows_i  # [1, H, L, D] flat row index

        def head_major(x):
            return np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]

        o_ref, lse_ref = orc.attention_rows(head_major(q), head_major(k), head_major(v),
                                            w["dtype"], w["scale"], w["mask"], w["window"],
                                            rows=flat)
        got = o_bits[a + rows_i, heads]
        st = compare(got, lse[a + rows_i, heads], o_ref, lse_ref, w["dtype"])
        assert st["pass"], (a, b, st)


def test_more_sequences_than_one_launch_holds(orc):
    """Batches above the per-launch sequence table (1024) run as several
    launches; every sequence still gets its own attention."""
    rng = np.random.default_rng(80)
    lengths = [int(x) for x in rng.integers(0, 9, 2500)]
    say("varlen many sequences", len(lengths), "tokens", sum(lengths))
    check(orc, lengths, 5, 2, 64, "f16", "causal", (-1, -1), seed=81)
