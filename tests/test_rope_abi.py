"""fa_rope and fa_fwd_rope on the host: argument checks that return before any
HIP call (no GPU needed)."""
import pytest

import tiled_attention_11_amd as fa

OK, INVALID, UNSUPPORTED, ALIGN, TOO_LARGE = 0, -1, -2, -3, -4
GB = 1 << 30
X, Y, C, S_, Q, K, V, O, L, KR = ((i + 1) * 4 * GB for i in range(10))


def rope(x=X, y=Y, c=C, s=S_, n_pos=100, mode=0, B=2, H=3, S=100, D=128, dtype=0):
    return fa.fa_rope(x, y, c, s, n_pos, mode, B, H, S, D, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INVALID), (dict(S=-2), INVALID), (dict(dtype=3), INVALID),
    (dict(mode=2), INVALID), (dict(mode=-1), INVALID), (dict(D=96), UNSUPPORTED),
    (dict(n_pos=99), INVALID), (dict(x=None), INVALID), (dict(c=None), INVALID),
    (dict(y=Y + 8), ALIGN), (dict(s=S_ + 4), ALIGN),
    (dict(y=X + 256), INVALID),             # partial overlap of x and y
    (dict(c=Y + 1024), INVALID),            # table inside the output
    (dict(B=1 << 12, H=1 << 12, S=1 << 10, n_pos=1 << 10), TOO_LARGE),
])
def test_rope_rejected_before_launch(kw, code):
    assert rope(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0, n_pos=0), dict(H=0, x=None, y=None)])
def test_rope_empty_problem_is_a_no_op(kw):
    assert rope(**kw) == OK


def fwd(q=Q, k=K, v=V, o=O, lse=L, kr=KR, c=C, s=S_, n_pos=100, mode=0, B=2, H=3, S=100, D=128,
        scale=0.1, mask=1, dtype=0):
    return fa.fa_fwd_rope(q, k, v, o, lse, kr, c, s, n_pos, mode, B, H, S, D, scale, mask, -1,
                          -1, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=5), INVALID), (dict(n_pos=50), INVALID), (dict(kr=None), INVALID),
    (dict(c=None), INVALID), (dict(c=C + 4), ALIGN), (dict(kr=KR + 2), ALIGN),
    (dict(kr=Q), INVALID),                  # k_rot on q
    (dict(kr=V + 64), INVALID),             # k_rot inside v
    (dict(kr=K + 64), INVALID),             # k_rot partly over k
    (dict(c=O + 128), INVALID),             # table inside o
    (dict(o=K), INVALID),                   # o over the unrotated k
    (dict(lse=C), INVALID),                 # lse over a table
    (dict(D=80), UNSUPPORTED), (dict(scale=float("nan")), INVALID), (dict(mask=4), INVALID),
])
def test_fwd_rope_rejected_before_launch(kw, code):
    assert fwd(**kw) == code


def test_fwd_rope_in_place_and_empty_are_accepted_on_the_host():
    # B*H*S == 0 returns before any launch; an in-place k_rot passes the checks
    assert fwd(B=0, kr=K) == OK
    assert fwd(S=0, n_pos=0) == OK


def dec(rope_mode=0, n_pos=100, c=C, Sq=4, Sk=100, o=O):
    return fa.fa_decode_rope(Q, K, V, o, L, c, S_, n_pos, rope_mode, 2, 3, Sq, Sk, 128, 0.1, 1,
                             -1, -1, 0, DQ_WS, 1 << 30, None)


DQ_WS = 11 * 4 * GB


@pytest.mark.parametrize("kw,code", [
    (dict(rope_mode=3), INVALID), (dict(n_pos=99), INVALID), (dict(c=None), INVALID),
    (dict(c=C + 4), ALIGN), (dict(c=O + 64), INVALID), (dict(Sq=40), UNSUPPORTED),
])
def test_decode_rope_rejected_before_launch(kw, code):
    assert dec(**kw) == code


def test_decode_paged_rope_rejects_page_size_zero():
    assert fa.fa_decode_paged_rope(Q, K, V, O, L, X, Y, C, S_, 100, 0, 2, 3, 1, 100, 128, 8, 0, 2,
                                   0.1, 1, -1, -1, 0, DQ_WS, 1 << 30, None) == UNSUPPORTED
