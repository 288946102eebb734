// fa_internal.h -- launch parameters shared by the C-ABI host code and the
// gfx950 kernels of the attention forward. Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace fa {

// "Unbounded" window side: larger than any sequence index the ABI accepts,
// small enough that i + kUnbounded does not overflow a 32-bit int.
constexpr int kUnbounded = 1 << 30;

// Persistent-grid work lists, shared by the forward and backward kernels.
// `grid` workgroups (at most one per CU) each run a stream of items r = 0, 1,
// ...; an item is one tile (a level: 0 .. levels - 1) of one head, and a
// head's item costs are expected to grow with the level. xcd_lists: B*H % 8
// == 0 (packed: H % 8 == 0) and grid % 8 == 0, so list x (heads x, x + 8, ...)
// is served by workgroups w = x mod 8, which the dispatcher places on XCD x;
// otherwise one list holds every head. list_len: items per list. Round r
// hands list positions r*nj .. r*nj + nj - 1 to the list's nj workgroups,
// reversed on odd rounds (a snake). Positions: first the flat part (n_flat >
// 0: the last n_flat levels of every head cost the same, the most), head
// after head, each head's from the last level down (flat_items = heads in
// the list * n_flat); then the other levels in groups of group_heads heads
// (dividing the list's heads), each group's levels from the last to the
// first, the group's heads interleaved, so that a round of the snake pairs a
// group's costliest item with its cheapest and the workgroups of a list
// share few heads (and their L2) at a time.
struct ListPlan {
    int grid;
    int xcd_lists;
    int list_len;
    int levels;
    int group_heads;  // a power of two: log2 in group_shift
    int n_flat;
    int flat_items;
    int group_shift;
    // Division by n_flat and by group_heads * (levels - n_flat) as a
    // multiply and a shift (fast_div; the host sets them with div_magic).
    uint32_t flat_m, group_m;
    int flat_s, group_s;
};

// floor(n / d) for 0 <= n < 2^31 as (n * m) >> s, with m, s from
// div_magic(d) (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994: with l = ceil(log2 d) and m = floor(2^(31+l)
// / d) + 1, 2^(31+l) < m d <= 2^(31+l) + 2^l, which makes the quotient exact
// for every 31-bit n; m < 2^32).
inline void div_magic(uint32_t d, uint32_t *m, int *s) {
    int l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    *s = 31 + l;
    *m = (uint32_t)((1ull << *s) / d + 1);
}
__host__ __device__ inline int fast_div(int n, uint32_t m, int s) {
    return (int)(((uint64_t)(uint32_t)n * m) >> s);
}

// Workgroup w of `grid`: the list position of its item in round r (the
// snake), and its list x.
__host__ __device__ inline int list_pos_at(const ListPlan &pl, int w, int grid, int r, int &x) {
    int j = w, nj = grid;
    x = 0;
    if (pl.xcd_lists) {
        x = w & 7;
        j = w >> 3;
        nj = grid >> 3;
    }
    return r * nj + ((r & 1) ? nj - 1 - j : j);
}
// Position pos of list x -> head bh and level; false past the list's end.
// (The divisions are multiplies and shifts: a runtime integer division
// costs a few hundred cycles on the GPU, at every item start.)
__host__ __device__ inline bool list_item(const ListPlan &pl, int x, int pos, int &bh,
                                          int &level) {
    if (pos >= pl.list_len) return false;
    int hl;
    if (pos < pl.flat_items) {
        const int nf = pl.n_flat;
        hl = fast_div(pos, pl.flat_m, pl.flat_s);
        level = pl.levels - 1 - (pos - hl * nf);
    } else {
        const int rp = pos - pl.flat_items;
        const int nq = pl.levels - pl.n_flat;  // levels below the flat part
        const int per_group = nq << pl.group_shift;
        const int grp = fast_div(rp, pl.group_m, pl.group_s), within = rp - grp * per_group;
        level = nq - 1 - (within >> pl.group_shift);
        hl = (grp << pl.group_shift) + (within & (pl.group_heads - 1));
    }
    bh = pl.xcd_lists ? hl * 8 + x : hl;
    return true;
}

// Everything a kernel needs, computed and validated on the host.
struct FwdParams {
    const void *q, *k, *v;  // [B, H, S, D], or packed [T, H, D] (see row addressing)
    void *o;                // as q
    float *lse;             // [B, H, S] or [T, H], or nullptr
    int B, H, S;
    int n_qtiles;           // ceil(S / query rows per workgroup)
    // Key j is visible from query i iff i - win_lo <= j <= i + win_hi and j < S
    // (win_lo, win_hi in [0, kUnbounded]); covers all three mask modes.
    int win_lo, win_hi;
    float c2;               // max(|scale| * log2(e), 2^-100): scores go to base 2 in one multiply
    int negate_q;           // scale < 0: Q's sign is flipped on load instead
    // Work distribution: items are query tiles (levels = n_qtiles). Packed
    // sequences order their lists by query tile (the kernel's walk) and use
    // only grid and xcd_lists of the plan.
    ListPlan plan;
    // Row addressing. Row r of head h of sequence b starts at element
    // base + r * row_stride; its LSE at index lse_base + r * lse_stride.
    //   [B, H, S, D]:      base = (b*H + h)*S*D, row_stride = D;
    //                      lse [B, H, S]: lse_base = (b*H + h)*S, lse_stride = 1.
    //   packed [T, H, D]:  base = (start_b*H + h)*D, row_stride = H*D;
    //                      lse [T, H]: lse_base = start_b*H + h, lse_stride = H.
    // cu_seqlens != nullptr selects the packed layout: sequence b holds tokens
    // cu_seqlens[b] .. cu_seqlens[b+1]-1 (clamped to [0, total_tokens] and to at
    // most S rows, S then being the longest length allowed); B counts sequences.
    int row_stride;
    const int32_t *cu_seqlens;
    int total_tokens;
    // Rotary embedding of the query rows (rope_cos == nullptr: none): row i of
    // a sequence turns by the angles of row i of the [>= S, D/2] fp32 tables,
    // pairs of halves or (rope_interleaved) of neighbours. k is read as given.
    const float *rope_cos, *rope_sin;
    int rope_interleaved;
    // Key split ([B, H, S, D] only): work items of kBlockMSplit rows whose two
    // wave groups take alternate key tiles and merge at the end (n_qtiles then
    // counts items of that height).
    int key_split;
};

// Rotary embedding of x [rows / S, S, D] into y (may be x): row r at position r % S.
struct RopeParams {
    const void *x;
    void *y;
    const float *cos, *sin;  // [>= S, D/2]
    int64_t rows;
    int S;
    int interleaved;
};

hipError_t launch_rope(const RopeParams &p, int D, int dtype, hipStream_t stream);

// Query rows per work item of the forward kernel, and of its key-split variant.
constexpr int kBlockM = 256;
constexpr int kBlockMSplit = 128;
// Keys per tile of the forward kernel (16 KiB of K or V either way).
constexpr int fwd_key_tile(int D) { return D == 128 ? 64 : 128; }
// Sequences of one packed launch (the kernel keeps a table of them in LDS);
// the host splits larger batches over several launches.
constexpr int kMaxPackedSeqs = 1024;

// Enqueue the kernel for head dimension D and dtype (0 fp16, 1 bf16).
hipError_t launch_fwd(const FwdParams &p, int D, int dtype, hipStream_t stream);

// ---- backward -------------------------------------------------------------------
struct BwdParams {
    const void *q, *k, *v, *o, *dout;  // [B, H, S, D]
    const float *lse;                  // [B, H, S], natural log (the forward's)
    float *rowdot;                     // workspace [B, H, S]: D_i = dO_i . O_i
    void *dq, *dk, *dv;                // [B, H, S, D]
    int B, H, S;
    int win_lo, win_hi;                // as in FwdParams
    float scale;                       // signed
    // Work lists: dQ items are 256-row query tiles (level = tile index), dK/dV
    // items 256-key tiles (level = tiles - 1 - tile index: under causal masks
    // the first keys are seen by the most rows).
    ListPlan dq_plan, kv_plan;
};

// Rows (queries for dQ, keys for dK/dV) of a backward work item.
constexpr int kBwdRows = 256;

// Enqueue the two backward kernels (dQ with the row dots, then dK/dV).
hipError_t launch_bwd(const BwdParams &p, int D, int dtype, hipStream_t stream);

// ---- new query rows against a key/value cache ---------------------------------
// Keys per tile of the cache kernel.
constexpr int kDecodeBN = 32;
// Query rows of one call: one wave's MFMA block.
constexpr int kDecodeMaxRows = 32;

struct DecodeParams {
    const void *q;          // [B, H, Sq, D]
    const void *k, *v;      // [B, H, Sk, D], or page pools (below)
    void *o;                // [B, H, Sq, D]
    float *lse;             // [B, H, Sq] or nullptr
    float *ws_o;            // nsplit > 1: partial outputs [B*H, nsplit, Sq, D]
    float *ws_lse;          // nsplit > 1: partial LSEs [B*H, nsplit, Sq]
    int B, H, Sq;
    int Sk;                 // cached keys per sequence (paged: the largest seq_lens allows)
    int win_lo, win_hi;     // as in FwdParams, relative to each row's position
    float c2;
    int negate_q;
    // Splits: split s of a head covers tiles t0 + s*tiles_per_split .. +tiles_per_split-1,
    // clipped to the tiles visible from its sequence's rows; t0 is the first such tile.
    int tiles_per_split;
    int nsplit;             // splits per head; 1 writes o and lse directly
    // Paged cache (block_table != nullptr): k and v are pools [num_pages, page_size,
    // H, D]; key j of sequence b is row j % page_size of page
    // block_table[b * max_pages + j / page_size] (page_size a multiple of the tile),
    // and sequence b caches min(seq_lens[b], Sk) keys.
    const int32_t *block_table;
    const int32_t *seq_lens;
    int page_size, max_pages, num_pages;
    // Rotary embedding of the query rows (rope_cos == nullptr: none): row i
    // turns by the angles of its position (table row, clamped into [0, Sk - 1]);
    // the cache holds keys already rotated.
    const float *rope_cos, *rope_sin;
    int rope_interleaved;
};

// Enqueue the cache kernel (and, for nsplit > 1, the merge kernel).
hipError_t launch_decode(const DecodeParams &p, int D, int dtype, hipStream_t stream);

// Bytes of the device-resident scratch array that the allocation-free cache
// entry point uses for its split partials (one copy per GPU, alive until the
// process ends). A plan on a 256-CU device needs at most about 17 MB
// (B*H*nsplit < 2 * 512 splits of 32 rows of D + 1 floats).
constexpr int64_t kDecodeScratchBytes = 24ll << 20;

// Device address of the current device's scratch array, looked up
// (hipGetSymbolAddress) on the first call made with that device current and
// cached per device afterwards. No allocation.
hipError_t decode_scratch(void **ptr);

}  // namespace fa
