// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation, the
// visible-pair and FLOP counts, and the hand-off to the gfx950 kernels.
//
// Validation is plain host code and runs before any HIP call, so every error
// except FA_ERR_HIP leaves nothing enqueued and nothing written.

#include "fa.h"
#include "fa_internal.h"

#include <cmath>
#include <cstdint>

namespace {

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Visible key range [lo, hi] of query row i (an empty range has lo > hi), from
// the window form of the mask that fa_internal.h describes.
inline void key_range(int64_t i, int64_t S, int64_t win_lo, int64_t win_hi,
                      int64_t *lo, int64_t *hi) {
    int64_t a = i - win_lo, b = i + win_hi;
    *lo = a > 0 ? a : 0;
    *hi = b < S - 1 ? b : S - 1;
}

// Mask mode and window arguments -> (win_lo, win_hi); false on a bad mode.
bool window_of(int mask_mode, int win_l, int win_r, int *win_lo, int *win_hi) {
    switch (mask_mode) {
    case FA_MASK_FULL:
        *win_lo = fa::kUnbounded;
        *win_hi = fa::kUnbounded;
        return true;
    case FA_MASK_CAUSAL:
        *win_lo = fa::kUnbounded;
        *win_hi = 0;
        return true;
    case FA_MASK_WINDOW:
        *win_lo = (win_l < 0 || win_l > fa::kUnbounded) ? fa::kUnbounded : win_l;
        *win_hi = (win_r < 0 || win_r > fa::kUnbounded) ? fa::kUnbounded : win_r;
        return true;
    default:
        return false;
    }
}

bool overlaps(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb) {
    return a < b + nb && b < a + na;
}

}  // namespace

extern "C" int64_t fa_visible_pairs(int S, int mask_mode, int win_l, int win_r) {
    int win_lo, win_hi;
    if (S < 0 || !window_of(mask_mode, win_l, win_r, &win_lo, &win_hi))
        return FA_ERR_INVALID_ARG;
    int64_t total = 0;
    for (int64_t i = 0; i < S; ++i) {
        int64_t lo, hi;
        key_range(i, S, win_lo, win_hi, &lo, &hi);
        if (hi >= lo) total += hi - lo + 1;
    }
    return total;
}

extern "C" int64_t fa_fwd_flops(int B, int H, int S, int D, int mask_mode, int win_l,
                                int win_r) {
    if (B < 0 || H < 0 || D <= 0) return FA_ERR_INVALID_ARG;
    int64_t pairs = fa_visible_pairs(S, mask_mode, win_l, win_r);
    if (pairs < 0) return pairs;
    // 4 * D * B * H * pairs, refusing anything that does not fit in int64.
    __int128 f = (__int128)4 * D * B * H * pairs;
    if (f > (__int128)INT64_MAX) return FA_ERR_TOO_LARGE;
    return (int64_t)f;
}

extern "C" const char *fa_strerror(int status) {
    switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128 only)";
    case FA_ERR_ALIGNMENT: return "misaligned pointer (q/k/v/o need 16 bytes, lse 4)";
    case FA_ERR_TOO_LARGE: return "problem too large for the kernel's index ranges";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
    }
}

extern "C" int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int S, int D, float scale, int mask_mode, int win_l,
                      int win_r, int dtype, hipStream_t stream) {
    // ---- scalar arguments -------------------------------------------------
    if (B < 0 || H < 0 || S < 0) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    int win_lo, win_hi;
    if (!window_of(mask_mode, win_l, win_r, &win_lo, &win_hi)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S == 0) return FA_OK;  // nothing to compute, nothing read

    // ---- sizes ------------------------------------------------------------
    const uint64_t head_bytes = (uint64_t)S * D * 2;
    if (head_bytes >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t n_qtiles = ((uint64_t)S + fa::kBlockM - 1) / fa::kBlockM;
    if (bh * n_qtiles > (uint64_t)INT32_MAX) return FA_ERR_TOO_LARGE;
    const __int128 tensor_bytes = (__int128)bh * head_bytes;
    if (tensor_bytes > (__int128)INT64_MAX / 4) return FA_ERR_TOO_LARGE;

    // ---- pointers ---------------------------------------------------------
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v,
                    po = (uintptr_t)o, pl = (uintptr_t)lse;
    if ((pq | pk | pv | po) & 15u) return FA_ERR_ALIGNMENT;
    if (lse && (pl & 3u)) return FA_ERR_ALIGNMENT;
    const uint64_t nbytes = (uint64_t)tensor_bytes;
    const uint64_t lbytes = bh * (uint64_t)S * 4;
    if (overlaps(po, nbytes, pq, nbytes) || overlaps(po, nbytes, pk, nbytes) ||
        overlaps(po, nbytes, pv, nbytes))
        return FA_ERR_INVALID_ARG;
    if (lse && (overlaps(pl, lbytes, pq, nbytes) || overlaps(pl, lbytes, pk, nbytes) ||
                overlaps(pl, lbytes, pv, nbytes) || overlaps(pl, lbytes, po, nbytes)))
        return FA_ERR_INVALID_ARG;

    // ---- launch -----------------------------------------------------------
    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.S = S;
    p.n_qtiles = (int)n_qtiles;
    p.win_lo = win_lo;
    p.win_hi = win_hi;
    // Scores go to base 2 in one multiply by c2 = |scale| * log2(e). c2 is
    // floored at 2^-100: below that every visible score under 2^76 in
    // magnitude (any fp16 input gives |q.k| < 2^40) maps to under 2^-24, so
    // exp2 of it is exactly 1.0f, the same fp32 result as a zero scale, while
    // c2 stays positive and hidden scores (-inf) keep probability exactly 0.
    p.c2 = std::fmax(std::fabs(scale) * 1.4426950408889634f, 0x1p-100f);
    p.negate_q = scale < 0.0f;

    // One workgroup per CU (each takes a whole CU), each running its share of
    // the bh * n_qtiles query tiles; see FwdParams.
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n_cu <= 0)
        return FA_ERR_HIP;
    const uint64_t n_items = bh * n_qtiles;
    uint64_t grid = n_items < (uint64_t)n_cu ? n_items : (uint64_t)n_cu;
    const bool xcd = bh % kNumXcd == 0 && grid >= (uint64_t)kNumXcd;
    if (xcd) grid -= grid % kNumXcd;
    const uint64_t list_heads = xcd ? bh / kNumXcd : bh;
    const uint64_t nj = xcd ? grid / kNumXcd : grid;  // workgroups per list
    // Heads per group: enough that a round of nj positions covers about one
    // group, so the workgroups of a list share few heads at a time.
    uint64_t gh = 1;
    while (2 * gh * n_qtiles <= nj && list_heads % (2 * gh) == 0) gh *= 2;
    p.grid = (int)grid;
    p.xcd_lists = xcd;
    p.list_len = (int)(list_heads * n_qtiles);
    p.group_heads = (int)gh;
    hipError_t err = fa::launch_fwd(p, D, dtype, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---- new query rows against a key/value cache ---------------------------------

namespace {

// Everything fa_decode decides before launching: the visible tile range and
// the split of it into per-workgroup ranges. Shared with the workspace query
// so both agree on the number of splits.
struct DecodePlan {
    int win_lo, win_hi;
    int t_first, t_last;
    int tiles_per_split, nsplit;
    int64_t ws_bytes;  // 0 when nsplit == 1
    bool empty;        // B*H*Sq == 0: nothing to do
};

int plan_decode(int B, int H, int Sq, int Sk, int D, int mask_mode, int win_l, int win_r,
                DecodePlan *pl) {
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || Sq > Sk) return FA_ERR_INVALID_ARG;
    if (!window_of(mask_mode, win_l, win_r, &pl->win_lo, &pl->win_hi)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if (Sq > fa::kDecodeMaxRows) return FA_ERR_UNSUPPORTED;
    pl->empty = (int64_t)B * H * Sq == 0;
    pl->t_first = pl->t_last = 0;
    pl->tiles_per_split = pl->nsplit = 1;
    pl->ws_bytes = 0;
    if (pl->empty) return FA_OK;
    if ((uint64_t)Sk * D * 2 >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    // Keys visible from some row: row i sits at position Sk - Sq + i.
    const int64_t pos0 = (int64_t)Sk - Sq;
    int64_t lo, hi, lo2, hi2;
    key_range(pos0, Sk, pl->win_lo, pl->win_hi, &lo, &hi);
    key_range(pos0 + Sq - 1, Sk, pl->win_lo, pl->win_hi, &lo2, &hi2);
    (void)hi;
    (void)lo2;
    pl->t_first = (int)(lo / fa::kDecodeBN);
    pl->t_last = (int)(hi2 / fa::kDecodeBN);
    const int nt = pl->t_last - pl->t_first + 1;
    // Splits: about two workgroups (one wave each) per CU over all heads,
    // never more than one per tile.
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n_cu <= 0)
        return FA_ERR_HIP;
    const int64_t bh = (int64_t)B * H;
    int64_t want = (2 * (int64_t)n_cu + bh - 1) / bh;
    if (want > nt) want = nt;
    if (want < 1) want = 1;
    pl->tiles_per_split = (int)((nt + want - 1) / want);
    pl->nsplit = (nt + pl->tiles_per_split - 1) / pl->tiles_per_split;
    if (bh * pl->nsplit > (int64_t)INT32_MAX || bh * Sq > (int64_t)INT32_MAX)
        return FA_ERR_TOO_LARGE;
    if (pl->nsplit > 1) {
        const __int128 ws = (__int128)bh * pl->nsplit * Sq * (D + 1) * 4;
        if (ws > (__int128)INT64_MAX / 4) return FA_ERR_TOO_LARGE;
        pl->ws_bytes = (int64_t)ws;
    }
    return FA_OK;
}

}  // namespace

extern "C" int64_t fa_decode_workspace_bytes(int B, int H, int Sq, int Sk, int D, int mask_mode,
                                             int win_l, int win_r) {
    DecodePlan pl;
    const int rc = plan_decode(B, H, Sq, Sk, D, mask_mode, win_l, win_r, &pl);
    return rc == FA_OK ? pl.ws_bytes : rc;
}

extern "C" int64_t fa_decode_flops(int B, int H, int Sq, int Sk, int D, int mask_mode, int win_l,
                                   int win_r) {
    int win_lo, win_hi;
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || Sq > Sk || D <= 0 ||
        !window_of(mask_mode, win_l, win_r, &win_lo, &win_hi))
        return FA_ERR_INVALID_ARG;
    int64_t pairs = 0;
    for (int64_t i = 0; i < Sq; ++i) {
        int64_t lo, hi;
        key_range((int64_t)Sk - Sq + i, Sk, win_lo, win_hi, &lo, &hi);
        if (hi >= lo) pairs += hi - lo + 1;
    }
    __int128 f = (__int128)4 * D * B * H * pairs;
    if (f > (__int128)INT64_MAX) return FA_ERR_TOO_LARGE;
    return (int64_t)f;
}

extern "C" int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int H, int Sq, int Sk, int D, float scale, int mask_mode,
                         int win_l, int win_r, int dtype, void *workspace,
                         int64_t workspace_bytes, hipStream_t stream) {
    // ---- scalar arguments and the plan (no HIP work queued before success) ----
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    DecodePlan pl;
    const int rc = plan_decode(B, H, Sq, Sk, D, mask_mode, win_l, win_r, &pl);
    if (rc != FA_OK) return rc;
    if (pl.empty) return FA_OK;
    if (workspace_bytes < 0) return FA_ERR_INVALID_ARG;

    // ---- pointers ---------------------------------------------------------------
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return FA_ERR_INVALID_ARG;
    const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v, po = (uintptr_t)o,
                    pl_ = (uintptr_t)lse, pw = (uintptr_t)workspace;
    if ((pq | pk | pv | po) & 15u) return FA_ERR_ALIGNMENT;
    if (lse && (pl_ & 3u)) return FA_ERR_ALIGNMENT;
    if (pl.ws_bytes > 0 && (pw & 15u)) return FA_ERR_ALIGNMENT;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t qbytes = bh * Sq * D * 2, kvbytes = bh * Sk * D * 2, lbytes = bh * Sq * 4;
    const uint64_t wbytes = (uint64_t)pl.ws_bytes;
    // outputs and workspace must not overlap the inputs or each other
    const uintptr_t outs[3] = {po, pl_, pw};
    const uint64_t outn[3] = {qbytes, lse ? lbytes : 0, wbytes};
    const uintptr_t ins[3] = {pq, pk, pv};
    const uint64_t inn[3] = {qbytes, kvbytes, kvbytes};
    for (int a = 0; a < 3; ++a) {
        if (!outn[a]) continue;
        for (int b = 0; b < 3; ++b)
            if (overlaps(outs[a], outn[a], ins[b], inn[b])) return FA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 3; ++b)
            if (outn[b] && overlaps(outs[a], outn[a], outs[b], outn[b])) return FA_ERR_INVALID_ARG;
    }

    // ---- launch -------------------------------------------------------------------
    fa::DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.ws_o = pl.nsplit > 1 ? static_cast<float *>(workspace) : nullptr;
    p.ws_lse = pl.nsplit > 1 ? static_cast<float *>(workspace) + bh * pl.nsplit * Sq * D : nullptr;
    p.B = B;
    p.H = H;
    p.Sq = Sq;
    p.Sk = Sk;
    p.pos0 = Sk - Sq;
    p.win_lo = pl.win_lo;
    p.win_hi = pl.win_hi;
    p.c2 = std::fmax(std::fabs(scale) * 1.4426950408889634f, 0x1p-100f);  // as in fa_fwd
    p.negate_q = scale < 0.0f;
    p.t_first = pl.t_first;
    p.t_last = pl.t_last;
    p.tiles_per_split = pl.tiles_per_split;
    p.nsplit = pl.nsplit;
    hipError_t err = fa::launch_decode(p, D, dtype, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

