"""fa_decode on the host: argument checks that return before any HIP call and
the FLOP count, against the oracle's visibility rule (no GPU needed)."""
import pytest

import tiled_attention_11_amd as fa

OK, INVALID, UNSUPPORTED = 0, -1, -2
Q, K, V, O, L, W = (i << 40 for i in range(1, 7))


def call(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Sq=4, Sk=100, D=128, scale=0.1, mask=1, wl=-1,
         wr=-1, dtype=0, ws=W, ws_bytes=1 << 30):
    return fa.fa_decode(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask, wl, wr, dtype, ws,
                        ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INVALID), (dict(H=-1), INVALID), (dict(Sq=-1), INVALID), (dict(Sk=-3), INVALID),
    (dict(Sq=5, Sk=4), INVALID), (dict(Sq=33, Sk=100), UNSUPPORTED),
    (dict(dtype=2), INVALID), (dict(mask=3), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(D=96), UNSUPPORTED), (dict(D=0), UNSUPPORTED),
])
def test_rejected_before_launch(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0), dict(Sq=0, Sk=0),
                                dict(B=0, q=None, k=None, v=None, o=None, ws=None)])
def test_empty_problem_is_a_no_op(kw):
    assert call(**kw) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(Sq=5, Sk=4), INVALID), (dict(Sq=40), UNSUPPORTED), (dict(D=80), UNSUPPORTED),
    (dict(mask=7), INVALID), (dict(B=-2), INVALID),
])
def test_workspace_query_rejects_what_decode_rejects(kw, code):
    a = dict(B=2, H=3, Sq=4, Sk=100, D=128, mask=1, wl=-1, wr=-1)
    a.update(kw)
    got = fa.fa_decode_workspace_bytes(a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["mask"],
                                       a["wl"], a["wr"])
    assert got == code


def test_workspace_query_of_an_empty_problem_is_zero():
    assert fa.fa_decode_workspace_bytes(0, 4, 3, 50, 64, 1) == 0
    assert fa.fa_decode_workspace_bytes(2, 4, 0, 50, 64, 1) == 0


CASES = [(1, 1, "causal", (-1, -1)), (1, 37, "causal", (-1, -1)), (5, 64, "full", (-1, -1)),
         (16, 100, "causal", (-1, -1)), (32, 70, "window", (10, 0)), (7, 40, "window", (3, 5)),
         (4, 4, "window", (-1, 2)), (9, 300, "window", (50, -1))]


@pytest.mark.parametrize("Sq,Sk,mask,window", CASES)
def test_flops_count_visible_pairs_at_the_rows_positions(orc, Sq, Sk, mask, window):
    pairs = sum(orc.visible(Sk - Sq + i, j, mask, window) for i in range(Sq) for j in range(Sk))
    m = {"full": 0, "causal": 1, "window": 2}[mask]
    for D in (64, 128):
        assert fa.fa_decode_flops(2, 3, Sq, Sk, D, m, *window) == 4 * D * 6 * pairs


def test_flops_rejects_bad_arguments():
    assert fa.fa_decode_flops(1, 1, 5, 4, 64, 1, -1, -1) == INVALID
    assert fa.fa_decode_flops(1, 1, 2, 4, 64, 9, -1, -1) == INVALID


def call_paged(B=2, H=3, Sq=4, max_seq=100, D=128, num_pages=8, page_size=64, max_pages=2,
               mask=1, dtype=0):
    return fa.fa_decode_paged(Q, K, V, O, L, W, W + 4096, B, H, Sq, max_seq, D, num_pages,
                              page_size, max_pages, 0.1, mask, -1, -1, dtype, W + 8192, 1 << 30,
                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=0), UNSUPPORTED), (dict(page_size=16), UNSUPPORTED),
    (dict(page_size=48), UNSUPPORTED), (dict(page_size=-32), UNSUPPORTED),
    (dict(num_pages=0), INVALID), (dict(max_pages=0), INVALID),
    (dict(max_pages=1, page_size=64, max_seq=100), INVALID),
    (dict(Sq=5, max_seq=4), INVALID), (dict(Sq=33), UNSUPPORTED), (dict(D=96), UNSUPPORTED),
    (dict(dtype=3), INVALID), (dict(mask=5), INVALID),
])
def test_paged_rejected_before_launch(kw, code):
    assert call_paged(**kw) == code


def test_paged_empty_problem_is_a_no_op():
    assert call_paged(B=0) == OK and call_paged(Sq=0) == OK
