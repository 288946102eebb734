// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation, the
// visible-pair and FLOP counts, and the hand-off to the gfx950 kernels.
//
// Validation is plain host code and runs before any HIP call, so every error
// except FA_ERR_HIP leaves nothing enqueued and nothing written.

#include "fa.h"
#include "fa_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <functional>

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

// Scores go to base 2 in one multiply by c2 = |scale| * log2(e). c2 is
// floored at 2^-100: below that every visible score under 2^76 in magnitude
// (any fp16 input gives |q.k| < 2^40) maps to under 2^-24, so exp2 of it is
// exactly 1.0f, the same fp32 result as a zero scale, while c2 stays positive
// and hidden scores (-inf) keep probability exactly 0.
float base2_scale(float scale) {
    return std::fmax(std::fabs(scale) * 1.4426950408889634f, 0x1p-100f);
}

// Work distribution and launch of the forward kernel, for p with everything
// but the fields set here filled in: one workgroup per CU (each takes a whole
// CU), each running its share of the bh * n_qtiles query tiles; see FwdParams.
// The current device's CU count, queried once per device and cached (a
// relaxed atomic per device: concurrent first calls store the same value).
int device_cus(int *n_cu) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *n_cu = c;
            return FA_OK;
        }
    }
    if (hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        *n_cu <= 0)
        return FA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(*n_cu, std::memory_order_relaxed);
    return FA_OK;
}

// Work lists for a persistent grid over bh heads of `levels` items each
// (fa::ListPlan). xcd_ok: the heads split evenly over the 8 XCD lists. cost
// (may be empty): an item's relative cost by level, which selects the flat
// part: the last levels of a head that cost the most, all alike (a sliding
// window's tiles past the window's length), taken first when there are at
// least two of them (a causal mask has one costliest tile per head: the
// grouped order pairs its tiles best), they fill at least one round of the
// list and they are not the whole head (a full mask keeps the grouped order).
fa::ListPlan plan_lists(uint64_t bh, uint64_t levels, bool xcd_ok, int n_cu,
                        const std::function<int64_t(uint64_t)> &cost) {
    const uint64_t n_items = bh * levels;
    uint64_t grid = n_items < (uint64_t)n_cu ? n_items : (uint64_t)n_cu;
    const bool xcd = xcd_ok && grid >= (uint64_t)kNumXcd;
    if (xcd) grid -= grid % kNumXcd;
    const uint64_t list_heads = xcd ? bh / kNumXcd : bh;
    const uint64_t nj = xcd ? grid / kNumXcd : grid;  // workgroups per list
    uint64_t n_flat = 0;
    if (cost) {
        int64_t most = 0;
        for (uint64_t l = 0; l < levels; ++l) most = std::max(most, cost(l));
        while (n_flat < levels && cost(levels - 1 - n_flat) == most) ++n_flat;
        bool suffix = true;  // every level below the flat part costs less
        for (uint64_t l = 0; l + n_flat < levels && suffix; ++l) suffix = cost(l) < most;
        if (!suffix || n_flat < 2 || n_flat == levels || list_heads * n_flat < nj) n_flat = 0;
    }
    // Heads per group (of the levels below the flat part): enough that a
    // round of nj positions covers about one group, so the workgroups of a
    // list share few heads at a time.
    const uint64_t n_rest = levels - n_flat;
    uint64_t gh = 1;
    while (2 * gh * n_rest <= nj && list_heads % (2 * gh) == 0) gh *= 2;
    fa::ListPlan pl;
    pl.grid = (int)grid;
    pl.xcd_lists = xcd;
    pl.list_len = (int)(list_heads * levels);
    pl.levels = (int)levels;
    pl.group_heads = (int)gh;
    pl.n_flat = (int)n_flat;
    pl.flat_items = (int)(list_heads * n_flat);
    pl.group_shift = 0;
    while ((1ull << pl.group_shift) < gh) ++pl.group_shift;
    fa::div_magic(n_flat ? (uint32_t)n_flat : 1u, &pl.flat_m, &pl.flat_s);
    fa::div_magic((uint32_t)(gh * n_rest), &pl.group_m, &pl.group_s);
    return pl;
}

// Tiles of `tile` keys (or queries) that rows r0 .. r1 see under the window
// [i - lo, i + hi] (clipped to 0 .. S - 1): the key tiles of a query tile,
// or, with lo and hi swapped, the query tiles of a key tile.
int64_t tiles_seen(int64_t r0, int64_t r1, int64_t S, int64_t lo, int64_t hi, int64_t tile) {
    const int64_t first = std::max<int64_t>(0, r0 - lo) / tile;
    const int64_t last = std::min<int64_t>(S - 1, r1 + hi) / tile;
    return last - first + 1;
}

// rows: the sequence length that sets the item count (the longest sequence
// when packed). allow_split: the layout may use the key-split variant.
void plan_fwd(fa::FwdParams &p, uint64_t bh, uint64_t rows, int D, int n_cu, bool allow_split) {
    // The key split (128-row items, the two wave groups of a workgroup on
    // alternate key tiles, merged at the end) for grids with fewer than two
    // 256-row items per CU: the heaviest causal item then sets the time, and
    // half-height items pair up evenly (B1 H32 S2048 D64 causal: 34.0 against
    // 40.9 us). Not for sliding windows, where it measured 8% slower (each
    // half-height item still pays a first and a last half-step, and the merge).
    const uint64_t items256 = bh * ((rows + fa::kBlockM - 1) / fa::kBlockM);
    const bool split = allow_split && items256 < 2 * (uint64_t)n_cu;
    const int block_m = split ? fa::kBlockMSplit : fa::kBlockM;
    const uint64_t n_qtiles = (rows + block_m - 1) / block_m;
    p.key_split = split;
    p.n_qtiles = (int)n_qtiles;
    // Packed sequences split heads over the lists by h % 8 within every
    // sequence, and order items by their own walk (no costs here).
    const bool xcd_ok = p.cu_seqlens ? p.H % kNumXcd == 0 : bh % kNumXcd == 0;
    std::function<int64_t(uint64_t)> cost;
    if (!p.cu_seqlens) {
        const int64_t bn = fa::fwd_key_tile(D), S = (int64_t)rows;
        const int64_t lo = p.win_lo, hi = p.win_hi;
        cost = [=](uint64_t qt) {
            const int64_t q0 = (int64_t)qt * block_m;
            return tiles_seen(q0, std::min<int64_t>(q0 + block_m - 1, S - 1), S, lo, hi, bn);
        };
    }
    p.plan = plan_lists(bh, n_qtiles, xcd_ok, n_cu, cost);
}

int plan_and_launch_fwd(fa::FwdParams &p, uint64_t bh, uint64_t rows, int D, int dtype,
                        hipStream_t stream, bool allow_split) {
    int n_cu = 0;
    if (device_cus(&n_cu) != FA_OK) return FA_ERR_HIP;
    plan_fwd(p, bh, rows, D, n_cu, allow_split);
    hipError_t err = fa::launch_fwd(p, D, dtype, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
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
    case FA_ERR_ALIGNMENT:
        return "misaligned pointer (q/k/v/o need 16 bytes, lse and index arrays 4)";
    case FA_ERR_TOO_LARGE: return "problem too large for the kernel's index ranges";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
    }
}

namespace {

// Rotary-embedding arguments of fa_fwd_rope (checked by fwd_core before
// anything is enqueued).
struct RopeArgs {
    const void *k_in;  // k before rotation; the forward reads k_rot
    void *k_rot;
    const float *cos, *sin;
    int n_pos, mode;
};

// fa_fwd, and fa_fwd_rope when rope != nullptr (k is then the rotated buffer).
int fwd_core(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
             int S, int D, float scale, int mask_mode, int win_l, int win_r, int dtype,
             hipStream_t stream, const RopeArgs *rope) {
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
    const uint64_t n_qtiles = ((uint64_t)S + fa::kBlockMSplit - 1) / fa::kBlockMSplit;
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
    if (rope) {
        // tables: [n_pos >= S, D/2] fp32, 16-byte aligned; k_rot (= k here) is
        // either the input k itself (rotated in place) or clear of every other
        // buffer, and no output overlaps the tables
        if (rope->mode != FA_ROPE_HALVES && rope->mode != FA_ROPE_INTERLEAVED)
            return FA_ERR_INVALID_ARG;
        if (!rope->k_in || !rope->cos || !rope->sin || rope->n_pos < S)
            return FA_ERR_INVALID_ARG;
        const uintptr_t pki = (uintptr_t)rope->k_in, pc = (uintptr_t)rope->cos,
                        ps = (uintptr_t)rope->sin;
        if ((pki | pc | ps) & 15u) return FA_ERR_ALIGNMENT;
        const uint64_t tbytes = (uint64_t)rope->n_pos * (D / 2) * 4;
        if ((pki != pk && overlaps(pk, nbytes, pki, nbytes)) || overlaps(pk, nbytes, pq, nbytes) ||
            overlaps(pk, nbytes, pv, nbytes))
            return FA_ERR_INVALID_ARG;
        if (overlaps(pk, nbytes, pc, tbytes) || overlaps(pk, nbytes, ps, tbytes) ||
            overlaps(po, nbytes, pc, tbytes) || overlaps(po, nbytes, ps, tbytes) ||
            overlaps(po, nbytes, pki, nbytes))
            return FA_ERR_INVALID_ARG;
        if (lse && (overlaps(pl, lbytes, pc, tbytes) || overlaps(pl, lbytes, ps, tbytes) ||
                    overlaps(pl, lbytes, pki, nbytes)))
            return FA_ERR_INVALID_ARG;
        if ((uint64_t)bh * S * (D / 16) >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    }

    // ---- launch -----------------------------------------------------------
    if (rope) {
        fa::RopeParams rp;
        rp.x = rope->k_in;
        rp.y = rope->k_rot;
        rp.cos = rope->cos;
        rp.sin = rope->sin;
        rp.rows = (int64_t)bh * S;
        rp.S = S;
        rp.interleaved = rope->mode == FA_ROPE_INTERLEAVED;
        if (fa::launch_rope(rp, D, dtype, stream) != hipSuccess) return FA_ERR_HIP;
    }
    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.S = S;
    p.win_lo = win_lo;
    p.win_hi = win_hi;
    p.c2 = base2_scale(scale);
    p.negate_q = scale < 0.0f;
    p.row_stride = D;
    p.cu_seqlens = nullptr;
    p.total_tokens = 0;
    p.rope_cos = rope ? rope->cos : nullptr;
    p.rope_sin = rope ? rope->sin : nullptr;
    p.rope_interleaved = rope ? rope->mode == FA_ROPE_INTERLEAVED : 0;
    return plan_and_launch_fwd(p, bh, (uint64_t)S, D, dtype, stream, true);
}

}  // namespace

extern "C" int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int S, int D, float scale, int mask_mode, int win_l,
                      int win_r, int dtype, hipStream_t stream) {
    return fwd_core(q, k, v, o, lse, B, H, S, D, scale, mask_mode, win_l, win_r, dtype, stream,
                    nullptr);
}

extern "C" int64_t fa_fwd_schedule(int B, int H, int S, int D, int mask_mode, int win_l,
                                   int win_r, int n_cu, int32_t *items, int64_t max_items) {
    if (B < 0 || H < 0 || S < 0 || n_cu < 1 || max_items < 0) return FA_ERR_INVALID_ARG;
    int win_lo, win_hi;
    if (!window_of(mask_mode, win_l, win_r, &win_lo, &win_hi)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S == 0) return 0;
    const uint64_t bh = (uint64_t)B * H;
    if ((uint64_t)S * D * 2 >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    if (bh * (((uint64_t)S + fa::kBlockMSplit - 1) / fa::kBlockMSplit) > (uint64_t)INT32_MAX)
        return FA_ERR_TOO_LARGE;
    if (max_items > 0 && !items) return FA_ERR_INVALID_ARG;
    fa::FwdParams p{};
    p.B = B;
    p.H = H;
    p.S = S;
    p.win_lo = win_lo;
    p.win_hi = win_hi;
    p.cu_seqlens = nullptr;
    plan_fwd(p, bh, (uint64_t)S, D, n_cu, true);
    const int rows = p.key_split ? fa::kBlockMSplit : fa::kBlockM;
    const int64_t bn = fa::fwd_key_tile(D);
    int64_t n = 0;
    for (int w = 0; w < p.plan.grid; ++w)
        for (int r = 0;; ++r) {
            int x, head, level;
            const int pos = fa::list_pos_at(p.plan, w, p.plan.grid, r, x);
            if (!fa::list_item(p.plan, x, pos, head, level)) break;
            if (n < max_items) {
                const int64_t q0 = (int64_t)level * rows;
                int32_t *e = items + 6 * n;
                e[0] = w;
                e[1] = r;
                e[2] = head;
                e[3] = (int32_t)q0;
                e[4] = rows;
                e[5] = (int32_t)tiles_seen(q0, std::min<int64_t>(q0 + rows - 1, S - 1), S,
                                           win_lo, win_hi, bn);
            }
            ++n;
        }
    return n;
}

extern "C" int fa_fwd_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                           void *k_rot, const float *cos_table, const float *sin_table,
                           int n_pos, int rope_mode, int B, int H, int S, int D, float scale,
                           int mask_mode, int win_l, int win_r, int dtype,
                           hipStream_t stream) {
    if (!k_rot) return FA_ERR_INVALID_ARG;
    RopeArgs r{k, k_rot, cos_table, sin_table, n_pos, rope_mode};
    return fwd_core(q, k_rot, v, o, lse, B, H, S, D, scale, mask_mode, win_l, win_r, dtype,
                    stream, &r);
}

extern "C" int fa_rope(const void *x, void *y, const float *cos_table, const float *sin_table,
                       int n_pos, int rope_mode, int B, int H, int S, int D, int dtype,
                       hipStream_t stream) {
    if (B < 0 || H < 0 || S < 0) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (rope_mode != FA_ROPE_HALVES && rope_mode != FA_ROPE_INTERLEAVED) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S == 0) return FA_OK;
    if (n_pos < S) return FA_ERR_INVALID_ARG;
    const uint64_t rows = (uint64_t)B * H * S;
    if (rows * (D / 16) >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    if (!x || !y || !cos_table || !sin_table) return FA_ERR_INVALID_ARG;
    const uintptr_t px = (uintptr_t)x, py = (uintptr_t)y, pc = (uintptr_t)cos_table,
                    ps = (uintptr_t)sin_table;
    if ((px | py | pc | ps) & 15u) return FA_ERR_ALIGNMENT;
    const uint64_t nbytes = rows * D * 2, tbytes = (uint64_t)n_pos * (D / 2) * 4;
    if (px != py && overlaps(px, nbytes, py, nbytes)) return FA_ERR_INVALID_ARG;
    if (overlaps(py, nbytes, pc, tbytes) || overlaps(py, nbytes, ps, tbytes))
        return FA_ERR_INVALID_ARG;
    fa::RopeParams rp;
    rp.x = x;
    rp.y = y;
    rp.cos = cos_table;
    rp.sin = sin_table;
    rp.rows = (int64_t)rows;
    rp.S = S;
    rp.interleaved = rope_mode == FA_ROPE_INTERLEAVED;
    return fa::launch_rope(rp, D, dtype, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                             const int32_t *cu_seqlens, int nseq, int max_seqlen,
                             int total_tokens, int H, int D, float scale, int mask_mode,
                             int win_l, int win_r, int dtype, hipStream_t stream) {
    // ---- scalar arguments -------------------------------------------------
    if (nseq < 0 || max_seqlen < 0 || total_tokens < 0 || H < 0) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    int win_lo, win_hi;
    if (!window_of(mask_mode, win_l, win_r, &win_lo, &win_hi)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)nseq * H * max_seqlen == 0 || total_tokens == 0) return FA_OK;

    // ---- sizes ------------------------------------------------------------
    // One head of one sequence spans (max_seqlen - 1) token rows of H * D
    // elements plus one row: the kernel's 32-bit buffer ranges must hold it.
    const uint64_t row_bytes = (uint64_t)H * D * 2;
    if ((uint64_t)max_seqlen * row_bytes >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    const uint64_t bh = (uint64_t)nseq * H;
    const uint64_t n_qtiles = ((uint64_t)max_seqlen + fa::kBlockM - 1) / fa::kBlockM;
    if (bh * n_qtiles > (uint64_t)INT32_MAX) return FA_ERR_TOO_LARGE;
    const __int128 tensor_bytes = (__int128)total_tokens * row_bytes;
    if (tensor_bytes > (__int128)INT64_MAX / 4) return FA_ERR_TOO_LARGE;

    // ---- pointers ---------------------------------------------------------
    if (!q || !k || !v || !o || !cu_seqlens) return FA_ERR_INVALID_ARG;
    const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v,
                    po = (uintptr_t)o, pl = (uintptr_t)lse, pc = (uintptr_t)cu_seqlens;
    if ((pq | pk | pv | po) & 15u) return FA_ERR_ALIGNMENT;
    if ((lse && (pl & 3u)) || (pc & 3u)) return FA_ERR_ALIGNMENT;
    const uint64_t nbytes = (uint64_t)tensor_bytes;
    const uint64_t lbytes = (uint64_t)total_tokens * H * 4;
    const uint64_t cbytes = ((uint64_t)nseq + 1) * 4;
    if (overlaps(po, nbytes, pq, nbytes) || overlaps(po, nbytes, pk, nbytes) ||
        overlaps(po, nbytes, pv, nbytes) || overlaps(po, nbytes, pc, cbytes))
        return FA_ERR_INVALID_ARG;
    if (lse && (overlaps(pl, lbytes, pq, nbytes) || overlaps(pl, lbytes, pk, nbytes) ||
                overlaps(pl, lbytes, pv, nbytes) || overlaps(pl, lbytes, po, nbytes) ||
                overlaps(pl, lbytes, pc, cbytes)))
        return FA_ERR_INVALID_ARG;

    // ---- launch -----------------------------------------------------------
    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.H = H;
    p.S = max_seqlen;
    p.win_lo = win_lo;
    p.win_hi = win_hi;
    p.c2 = base2_scale(scale);
    p.negate_q = scale < 0.0f;
    p.row_stride = H * D;
    p.total_tokens = total_tokens;
    p.rope_cos = p.rope_sin = nullptr;
    p.rope_interleaved = 0;
    // At most kMaxPackedSeqs sequences per launch (the kernel's LDS table).
    for (int first = 0; first < nseq; first += fa::kMaxPackedSeqs) {
        const int n = std::min(nseq - first, fa::kMaxPackedSeqs);
        p.B = n;
        p.cu_seqlens = cu_seqlens + first;
        const int rc =
            plan_and_launch_fwd(p, (uint64_t)n * H, (uint64_t)max_seqlen, D, dtype, stream, false);
        if (rc != FA_OK) return rc;
    }
    return FA_OK;
}

extern "C" int64_t fa_fwd_varlen_flops(const int32_t *cu_seqlens, int nseq, int H, int D,
                                       int mask_mode, int win_l, int win_r) {
    if (nseq < 0 || H < 0 || D <= 0 || (nseq > 0 && !cu_seqlens)) return FA_ERR_INVALID_ARG;
    __int128 f = 0;
    for (int b = 0; b < nseq; ++b) {
        if (cu_seqlens[b] < 0 || cu_seqlens[b + 1] < cu_seqlens[b]) return FA_ERR_INVALID_ARG;
        const int64_t pairs = fa_visible_pairs(cu_seqlens[b + 1] - cu_seqlens[b], mask_mode,
                                               win_l, win_r);
        if (pairs < 0) return pairs;
        f += (__int128)4 * D * H * pairs;
        if (f > (__int128)INT64_MAX) return FA_ERR_TOO_LARGE;
    }
    return (int64_t)f;
}

// ---- backward ---------------------------------------------------------------------

extern "C" int64_t fa_bwd_workspace_bytes(int B, int H, int S) {
    if (B < 0 || H < 0 || S < 0) return FA_ERR_INVALID_ARG;
    const __int128 n = (__int128)B * H * S * 4;
    if (n > (__int128)INT64_MAX) return FA_ERR_TOO_LARGE;
    return (int64_t)n;
}

extern "C" int fa_bwd(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                      int H, int S, int D, float scale, int mask_mode, int win_l, int win_r,
                      int dtype, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    // ---- scalar arguments -------------------------------------------------
    if (B < 0 || H < 0 || S < 0) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    int win_lo, win_hi;
    if (!window_of(mask_mode, win_l, win_r, &win_lo, &win_hi)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S == 0) return FA_OK;

    // ---- sizes ------------------------------------------------------------
    const uint64_t head_bytes = (uint64_t)S * D * 2;
    if (head_bytes >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t tiles = bh * (((uint64_t)S + 127) / 128);
    if (tiles > (uint64_t)INT32_MAX) return FA_ERR_TOO_LARGE;
    if (bh * S * (D / 8) >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    const uint64_t nbytes = bh * head_bytes;
    const uint64_t lbytes = bh * (uint64_t)S * 4;
    if (nbytes > (uint64_t)INT64_MAX / 4) return FA_ERR_TOO_LARGE;

    // ---- pointers ---------------------------------------------------------
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
        return FA_ERR_INVALID_ARG;
    if (workspace_bytes < (int64_t)lbytes) return FA_ERR_INVALID_ARG;
    const uintptr_t in[6] = {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o,
                             (uintptr_t)dout, (uintptr_t)lse};
    const uint64_t in_n[6] = {nbytes, nbytes, nbytes, nbytes, nbytes, lbytes};
    const uintptr_t out[4] = {(uintptr_t)dq, (uintptr_t)dk, (uintptr_t)dv, (uintptr_t)workspace};
    const uint64_t out_n[4] = {nbytes, nbytes, nbytes, lbytes};
    for (int t = 0; t < 5; ++t)
        if (in[t] & 15u) return FA_ERR_ALIGNMENT;
    for (int t = 0; t < 3; ++t)
        if (out[t] & 15u) return FA_ERR_ALIGNMENT;
    if ((in[5] | out[3]) & 3u) return FA_ERR_ALIGNMENT;
    for (int a = 0; a < 4; ++a) {
        for (int t = 0; t < 6; ++t)
            if (overlaps(out[a], out_n[a], in[t], in_n[t])) return FA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(out[a], out_n[a], out[b], out_n[b])) return FA_ERR_INVALID_ARG;
    }

    // ---- launch -----------------------------------------------------------
    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.rowdot = static_cast<float *>(workspace);
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.B = B;
    p.H = H;
    p.S = S;
    p.win_lo = win_lo;
    p.win_hi = win_hi;
    p.scale = scale;
    // Persistent grids over 256-row tiles: dQ items are query tiles (cost:
    // the 64-key tiles they see), dK/dV items key tiles, the level counting
    // down from the last tile (cost: the 32-query tiles that see them).
    int n_cu = 0;
    if (device_cus(&n_cu) != FA_OK) return FA_ERR_HIP;
    const int64_t rows = fa::kBwdRows, SS = S, lo = win_lo, hi = win_hi;
    const uint64_t ntiles = ((uint64_t)S + rows - 1) / rows;
    const bool xcd_ok = bh % kNumXcd == 0;
    p.dq_plan = plan_lists(bh, ntiles, xcd_ok, n_cu, [=](uint64_t qt) {
        const int64_t q0 = (int64_t)qt * rows;
        return tiles_seen(q0, std::min<int64_t>(q0 + rows - 1, SS - 1), SS, lo, hi, 64);
    });
    p.kv_plan = plan_lists(bh, ntiles, xcd_ok, n_cu, [=](uint64_t l) {
        const int64_t k0 = (int64_t)(ntiles - 1 - l) * rows;
        return tiles_seen(k0, std::min<int64_t>(k0 + rows - 1, SS - 1), SS, hi, lo, 32);
    });
    return fa::launch_bwd(p, D, dtype, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int64_t fa_bwd_flops(int B, int H, int S, int D, int mask_mode, int win_l,
                                int win_r) {
    // five products over the visible pairs (S, dP, dV, dK, dQ), 2 FLOPs per
    // multiply-add each: 10 * D per pair, 2.5 times the forward's count
    const int64_t f = fa_fwd_flops(B, H, S, D, mask_mode, win_l, win_r);
    if (f < 0) return f;
    if (f > INT64_MAX / 10 * 4) return FA_ERR_TOO_LARGE;
    return f / 4 * 10;
}

// ---- new query rows against a key/value cache ---------------------------------

namespace {

// Everything fa_decode decides before launching: the split of the visible
// tile range into per-workgroup ranges. Shared with the workspace queries so
// both agree on the number of splits.
struct DecodePlan {
    int win_lo, win_hi;
    int tiles_per_split, nsplit;
    int64_t ws_bytes;  // 0 when nsplit == 1
    bool empty;        // B*H*Sq == 0: nothing to do
};

// Sk is the cache length (paged: the largest any sequence may have). With
// `paged` the sequences' lengths are unknown here, so the split is planned
// over the most tiles any sequence's rows can see.
int plan_decode(int B, int H, int Sq, int Sk, int D, int mask_mode, int win_l, int win_r,
                bool paged, DecodePlan *pl) {
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || Sq > Sk) return FA_ERR_INVALID_ARG;
    if (!window_of(mask_mode, win_l, win_r, &pl->win_lo, &pl->win_hi)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if (Sq > fa::kDecodeMaxRows) return FA_ERR_UNSUPPORTED;
    pl->empty = (int64_t)B * H * Sq == 0;
    pl->tiles_per_split = pl->nsplit = 1;
    pl->ws_bytes = 0;
    if (pl->empty) return FA_OK;
    if ((uint64_t)Sk * D * 2 >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    int64_t nt;  // tiles the rows of one sequence can see
    if (!paged) {
        // rows at positions Sk - Sq .. Sk - 1
        int64_t lo, hi, lo2, hi2;
        key_range((int64_t)Sk - Sq, Sk, pl->win_lo, pl->win_hi, &lo, &hi);
        key_range((int64_t)Sk - 1, Sk, pl->win_lo, pl->win_hi, &lo2, &hi2);
        (void)hi;
        (void)lo2;
        nt = hi2 / fa::kDecodeBN - lo / fa::kDecodeBN + 1;
    } else {
        // a window spans at most Sq - 1 + win_lo + win_hi + 1 keys, plus one
        // partial tile at each end
        const int64_t span = (int64_t)Sq + pl->win_lo + pl->win_hi;
        const int64_t all = ((int64_t)Sk + fa::kDecodeBN - 1) / fa::kDecodeBN;
        nt = std::min<int64_t>(all, span / fa::kDecodeBN + 2);
    }
    // Splits: about two workgroups (one wave each) per CU over all heads,
    // never more than one per tile.
    int n_cu = 0;
    if (device_cus(&n_cu) != FA_OK) return FA_ERR_HIP;
    const int64_t bh = (int64_t)B * H;
    int64_t want = (2 * (int64_t)n_cu + bh - 1) / bh;
    if (want > nt) want = nt;
    if (want < 1) want = 1;
    pl->tiles_per_split = (int)((nt + want - 1) / want);
    pl->nsplit = (int)((nt + pl->tiles_per_split - 1) / pl->tiles_per_split);
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
    const int rc = plan_decode(B, H, Sq, Sk, D, mask_mode, win_l, win_r, false, &pl);
    return rc == FA_OK ? pl.ws_bytes : rc;
}

extern "C" int64_t fa_decode_paged_workspace_bytes(int B, int H, int Sq, int max_seq_len, int D,
                                                   int mask_mode, int win_l, int win_r) {
    DecodePlan pl;
    const int rc = plan_decode(B, H, Sq, max_seq_len, D, mask_mode, win_l, win_r, true, &pl);
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

namespace {

// Checks and launch shared by the contiguous and the paged cache entry points.
// kv_bytes: bytes of one of k, v (the pool when paged).
int decode_common(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                  int Sq, int Sk, int D, float scale, int mask_mode, int win_l, int win_r,
                  int dtype, void *workspace, int64_t workspace_bytes, hipStream_t stream,
                  const int32_t *block_table, const int32_t *seq_lens, int num_pages,
                  int page_size, int max_pages, const RopeArgs *rope = nullptr) {
    // ---- scalar arguments and the plan (no HIP work queued before success) ----
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    const bool paged = block_table != nullptr || seq_lens != nullptr || page_size != 0;
    if (paged) {
        if (page_size <= 0 || page_size % fa::kDecodeBN != 0) return FA_ERR_UNSUPPORTED;
        if (num_pages < 1 || max_pages < 1) return FA_ERR_INVALID_ARG;
        if ((int64_t)max_pages * page_size < Sk) return FA_ERR_INVALID_ARG;
        if ((int64_t)B * max_pages > (int64_t)INT32_MAX) return FA_ERR_TOO_LARGE;
        // one page's rows of one head must stay inside a 32-bit buffer range
        if ((uint64_t)page_size * H * D * 2 >= (1ull << 31)) return FA_ERR_TOO_LARGE;
    }
    if (rope) {
        // tables [n_pos >= Sk, D/2] fp32, 16-byte aligned, clear of o and lse
        // (checked before the plan, which queries the device)
        if (rope->mode != FA_ROPE_HALVES && rope->mode != FA_ROPE_INTERLEAVED)
            return FA_ERR_INVALID_ARG;
        if (!rope->cos || !rope->sin || rope->n_pos < Sk) return FA_ERR_INVALID_ARG;
        if (((uintptr_t)rope->cos | (uintptr_t)rope->sin) & 15u) return FA_ERR_ALIGNMENT;
        if (B >= 0 && H >= 0 && Sq >= 0 && (D == 64 || D == 128)) {
            const uint64_t tbytes = (uint64_t)rope->n_pos * (D / 2) * 4;
            const uint64_t ob = (uint64_t)B * H * Sq * D * 2, lb = (uint64_t)B * H * Sq * 4;
            for (const void *t : {(const void *)rope->cos, (const void *)rope->sin})
                if (overlaps((uintptr_t)o, ob, (uintptr_t)t, tbytes) ||
                    (lse && overlaps((uintptr_t)lse, lb, (uintptr_t)t, tbytes)))
                    return FA_ERR_INVALID_ARG;
        }
    }
    DecodePlan pl;
    const int rc = plan_decode(B, H, Sq, Sk, D, mask_mode, win_l, win_r, paged, &pl);
    if (rc != FA_OK) return rc;
    if (pl.empty) return FA_OK;
    if (workspace_bytes < 0) return FA_ERR_INVALID_ARG;

    // ---- pointers ---------------------------------------------------------------
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    if (paged && (!block_table || !seq_lens)) return FA_ERR_INVALID_ARG;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return FA_ERR_INVALID_ARG;
    const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v, po = (uintptr_t)o,
                    pl_ = (uintptr_t)lse, pw = (uintptr_t)workspace;
    if ((pq | pk | pv | po) & 15u) return FA_ERR_ALIGNMENT;
    if (lse && (pl_ & 3u)) return FA_ERR_ALIGNMENT;
    if (pl.ws_bytes > 0 && (pw & 15u)) return FA_ERR_ALIGNMENT;
    if (paged && (((uintptr_t)block_table | (uintptr_t)seq_lens) & 3u)) return FA_ERR_ALIGNMENT;
    const uint64_t bh = (uint64_t)B * H;
    const uint64_t qbytes = bh * Sq * D * 2, lbytes = bh * Sq * 4;
    const uint64_t kvbytes = paged ? (uint64_t)num_pages * page_size * H * D * 2 : bh * Sk * D * 2;
    const uint64_t wbytes = (uint64_t)pl.ws_bytes;
    // outputs and workspace must not overlap the inputs or each other
    const uintptr_t outs[3] = {po, pl_, pw};
    const uint64_t outn[3] = {qbytes, lse ? lbytes : 0, wbytes};
    const uintptr_t ins[5] = {pq, pk, pv, (uintptr_t)block_table, (uintptr_t)seq_lens};
    const uint64_t inn[5] = {qbytes, kvbytes, kvbytes, paged ? (uint64_t)B * max_pages * 4 : 0,
                             paged ? (uint64_t)B * 4 : 0};
    for (int a = 0; a < 3; ++a) {
        if (!outn[a]) continue;
        for (int b = 0; b < 5; ++b)
            if (inn[b] && overlaps(outs[a], outn[a], ins[b], inn[b])) return FA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 3; ++b)
            if (outn[b] && overlaps(outs[a], outn[a], outs[b], outn[b])) return FA_ERR_INVALID_ARG;
    }
    if (rope) {  // the workspace must not overlap the tables either
        const uint64_t tbytes = (uint64_t)rope->n_pos * (D / 2) * 4;
        if (wbytes && (overlaps(pw, wbytes, (uintptr_t)rope->cos, tbytes) ||
                       overlaps(pw, wbytes, (uintptr_t)rope->sin, tbytes)))
            return FA_ERR_INVALID_ARG;
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
    p.win_lo = pl.win_lo;
    p.win_hi = pl.win_hi;
    p.c2 = base2_scale(scale);
    p.negate_q = scale < 0.0f;
    p.tiles_per_split = pl.tiles_per_split;
    p.nsplit = pl.nsplit;
    p.block_table = paged ? block_table : nullptr;
    p.seq_lens = paged ? seq_lens : nullptr;
    p.page_size = paged ? page_size : 0;
    p.max_pages = paged ? max_pages : 0;
    p.num_pages = paged ? num_pages : 0;
    p.rope_cos = rope ? rope->cos : nullptr;
    p.rope_sin = rope ? rope->sin : nullptr;
    p.rope_interleaved = rope ? rope->mode == FA_ROPE_INTERLEAVED : 0;
    hipError_t err = fa::launch_decode(p, D, dtype, stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int H, int Sq, int Sk, int D, float scale, int mask_mode,
                         int win_l, int win_r, int dtype, void *workspace,
                         int64_t workspace_bytes, hipStream_t stream) {
    return decode_common(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r, dtype,
                         workspace, workspace_bytes, stream, nullptr, nullptr, 0, 0, 0);
}

extern "C" int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o,
                                 float *lse, int B, int H, int Sq, int Sk, int D, float scale,
                                 int mask_mode, int win_l, int win_r, int dtype,
                                 hipStream_t stream) {
    DecodePlan pl;
    const int rc = plan_decode(B, H, Sq, Sk, D, mask_mode, win_l, win_r, false, &pl);
    if (rc != FA_OK) return rc;
    if (pl.empty) return FA_OK;
    if (pl.ws_bytes > fa::kDecodeScratchBytes) return FA_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (pl.ws_bytes > 0 && fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
    return decode_common(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r, dtype,
                         ws, pl.ws_bytes, stream, nullptr, nullptr, 0, 0, 0);
}

extern "C" int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                               float *lse, const int32_t *block_table, const int32_t *seq_lens,
                               int B, int H, int Sq, int max_seq_len, int D, int num_pages,
                               int page_size, int max_pages, float scale, int mask_mode,
                               int win_l, int win_r, int dtype, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
    if (page_size == 0) return FA_ERR_UNSUPPORTED;  // 0 would mean "not paged" below
    return decode_common(q, k_pages, v_pages, o, lse, B, H, Sq, max_seq_len, D, scale, mask_mode,
                         win_l, win_r, dtype, workspace, workspace_bytes, stream, block_table,
                         seq_lens, num_pages, page_size, max_pages);
}

extern "C" int fa_decode_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                              const float *cos_table, const float *sin_table, int n_pos,
                              int rope_mode, int B, int H, int Sq, int Sk, int D, float scale,
                              int mask_mode, int win_l, int win_r, int dtype, void *workspace,
                              int64_t workspace_bytes, hipStream_t stream) {
    RopeArgs r{nullptr, nullptr, cos_table, sin_table, n_pos, rope_mode};
    return decode_common(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r, dtype,
                         workspace, workspace_bytes, stream, nullptr, nullptr, 0, 0, 0, &r);
}

extern "C" int fa_decode_paged_rope(const void *q, const void *k_pages, const void *v_pages,
                                    void *o, float *lse, const int32_t *block_table,
                                    const int32_t *seq_lens, const float *cos_table,
                                    const float *sin_table, int n_pos, int rope_mode, int B,
                                    int H, int Sq, int max_seq_len, int D, int num_pages,
                                    int page_size, int max_pages, float scale, int mask_mode,
                                    int win_l, int win_r, int dtype, void *workspace,
                                    int64_t workspace_bytes, hipStream_t stream) {
    if (page_size == 0) return FA_ERR_UNSUPPORTED;  // 0 would mean "not paged"
    RopeArgs r{nullptr, nullptr, cos_table, sin_table, n_pos, rope_mode};
    return decode_common(q, k_pages, v_pages, o, lse, B, H, Sq, max_seq_len, D, scale, mask_mode,
                         win_l, win_r, dtype, workspace, workspace_bytes, stream, block_table,
                         seq_lens, num_pages, page_size, max_pages, &r);
}
