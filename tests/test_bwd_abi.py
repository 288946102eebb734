"""fa_bwd on the host: argument checks that return before any HIP call, the
workspace size and the FLOP count (no GPU needed)."""
import pytest

import tiled_attention_11_amd as fa

OK, INVALID, UNSUPPORTED, ALIGN, TOO_LARGE = 0, -1, -2, -3, -4
GB = 1 << 30
Q, K, V, O, L, DO, DQ, DK, DV, W = ((i + 1) * 4 * GB for i in range(10))


def call(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=2, H=3, S=100, D=128,
         scale=0.1, mask=1, dtype=0, ws=W, ws_bytes=2 * 3 * 100 * 4):
    return fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, S, D, scale, mask, -1, -1, dtype, ws,
                     ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INVALID), (dict(S=-1), INVALID), (dict(dtype=2), INVALID), (dict(mask=3), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(D=96), UNSUPPORTED), (dict(lse=None), INVALID),
    (dict(do=None), INVALID), (dict(ws=None), INVALID), (dict(ws_bytes=2399), INVALID),
    (dict(q=Q + 8), ALIGN), (dict(dk=DK + 4), ALIGN), (dict(lse=L + 2), ALIGN),
    (dict(ws=W + 2), ALIGN),
    (dict(dq=K), INVALID),            # an output over an input
    (dict(dv=DK + 1024), INVALID),    # two outputs overlapping
    (dict(ws=DQ + 64), INVALID),      # workspace over an output
    (dict(ws=L), INVALID),            # workspace over the lse input
    (dict(S=1 << 23), TOO_LARGE),     # a head's [S, D] block of 2^31 bytes
])
def test_rejected_before_launch(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0, ws=None), dict(H=0, q=None)])
def test_empty_problem_is_a_no_op(kw):
    assert call(**kw) == OK


def test_workspace_and_flops():
    assert fa.fa_bwd_workspace_bytes(2, 3, 100) == 2400
    assert fa.fa_bwd_workspace_bytes(-1, 3, 100) == INVALID
    for S, mask in ((100, 1), (77, 0), (300, 2)):
        assert fa.fa_bwd_flops(2, 3, S, 64, mask, 20, 5) == \
            fa.fa_fwd_flops(2, 3, S, 64, mask, 20, 5) // 4 * 10
