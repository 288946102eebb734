"""fa_fwd_varlen on the host: argument checks that return before any HIP call
and the FLOP count against the oracle's visibility rule (no GPU needed)."""
import pytest

import tiled_attention_11_amd as fa

OK, INVALID, UNSUPPORTED, ALIGN, TOO_LARGE = 0, -1, -2, -3, -4
Q, K, V, O, L, C = (i << 40 for i in range(1, 7))


def call(q=Q, k=K, v=V, o=O, lse=L, cu=C, nseq=3, max_seqlen=100, T=250, H=4, D=128,
         scale=0.1, mask=1, wl=-1, wr=-1, dtype=0):
    return fa.fa_fwd_varlen(q, k, v, o, lse, cu, nseq, max_seqlen, T, H, D, scale, mask, wl,
                            wr, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nseq=-1), INVALID), (dict(max_seqlen=-1), INVALID), (dict(T=-5), INVALID),
    (dict(H=-1), INVALID), (dict(dtype=2), INVALID), (dict(mask=3), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("-inf")), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(D=0), UNSUPPORTED),
    (dict(cu=None), INVALID), (dict(q=None), INVALID), (dict(o=None), INVALID),
    (dict(q=Q + 8), ALIGN), (dict(o=O + 4), ALIGN), (dict(lse=L + 2), ALIGN),
    (dict(cu=C + 2), ALIGN),
    (dict(cu=O + 64), INVALID),  # cu_seqlens inside o
    (dict(lse=Q + 16), INVALID),  # lse inside q
    (dict(o=K), INVALID),
    # one head of one sequence: max_seqlen * H * D * 2 must stay under 2^31
    (dict(max_seqlen=1 << 17, H=64, D=128, T=1 << 17), TOO_LARGE),
])
def test_rejected_before_launch(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(nseq=0), dict(max_seqlen=0), dict(T=0), dict(H=0),
                                dict(nseq=0, q=None, k=None, v=None, o=None, cu=None)])
def test_empty_problem_is_a_no_op(kw):
    assert call(**kw) == OK


CASES = [([5, 0, 17, 1], "causal", (-1, -1)), ([300], "full", (-1, -1)),
         ([64, 65, 1], "window", (10, 0)), ([40, 7], "window", (3, 5)),
         ([0], "causal", (-1, -1)), ([33, 12], "window", (-1, 2))]


@pytest.mark.parametrize("lengths,mask,window", CASES)
def test_flops_sum_the_sequences_visible_pairs(orc, lengths, mask, window):
    pairs = sum(orc.pair_count(n, mask, window) for n in lengths)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    m = {"full": 0, "causal": 1, "window": 2}[mask]
    for D in (64, 128):
        assert fa.fa_fwd_varlen_flops(cu, 3, D, m, *window) == 4 * D * 3 * pairs


def test_flops_rejects_bad_offsets():
    assert fa.fa_fwd_varlen_flops([0, 5, 3], 2, 64, 1) == INVALID
    assert fa.fa_fwd_varlen_flops([-1, 5], 2, 64, 1) == INVALID
    assert fa.fa_fwd_varlen_flops([0, 5], 2, 64, 9) == INVALID
    assert fa.fa_fwd_varlen_flops([0], 2, 64, 1) == 0
