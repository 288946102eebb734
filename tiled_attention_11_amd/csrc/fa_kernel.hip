// fa_kernel.hip -- fused attention forward for gfx950 (MI355X), fp16/bf16 in,
// fp32 accumulate, D in {64, 128}.
//
// What it computes: O = softmax(scale * Q K^T + mask) V and the row LSE, with
// the online-softmax recurrence of the Ascend C FlashAttention-2 tile-fusion
// page (ascendai.csdn.net), section 1.2: a running row maximum m and row sum l,
// an unnormalised accumulator rescaled by exp(m_old - m_new) when m grows, and
// one division by l at the end. Tiling Q into row blocks and streaming K/V
// column blocks follows section 3 of that page and the ops-transformer
// walkthrough (hwcomputing.csdn.net, 6a0ef689), "core idea: tiling + online
// softmax"; skipping key blocks that the mask hides entirely follows section 6
// of the tile-fusion page; the window mask follows the catlass article
// (lnwmold.com/news/1200460), section "usage".
//
// gfx950 design (not the pages' Ascend design):
//  * A workgroup is 8 waves of 64 lanes, one per CU, persistent: it runs a
//    stream of work items from a precomputed list (ListPlan). The lists keep
//    a head's items on one XCD, put the costliest equal-cost items first
//    where a mask makes many (windows) and pair costly with cheap ones in a
//    snake order. An item is 256 query rows of one
//    (b, h), each wave owning 32 rows for the whole key loop. Small grids use
//    128-row items (key split): waves w and w + 4 share rows, take alternate
//    key tiles and merge their softmax states at the end.
//  * The waves form two groups (0-3 and 4-7, one wave of each per SIMD). The
//    groups alternate between an MFMA phase (P V of the previous key tile,
//    then the scores of the next) and a VALU phase (mask and online
//    softmax), in opposite order within each step of the key loop (one
//    workgroup barrier per step). On every SIMD one wave keeps the matrix
//    core busy while the other computes exponentials: a single wave cannot
//    issue VALU work fast enough to hide it under its own MFMAs, but two
//    waves of a SIMD co-issue.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16
//    (A = 32 keys x 16 dims, B = 16 dims x 32 queries). In the accumulator
//    layout lane l holds query l % 32 and 16 keys, so the row max and row sum
//    are in-lane reductions plus one v_permlane32_swap with lane l ^ 32, and
//    the per-row rescale of the output is a per-lane scalar.
//  * The output is accumulated transposed too, O^T += V^T P^T. P^T comes
//    straight out of the score accumulator as the B operand: rounded to fp16,
//    or for bf16 as two bf16 terms (value and remainder, two products). The
//    V^T A operand is read from the row-major V tile with the transposing
//    LDS load ds_read_b64_tr_b16 (a 16-lane group reads a 4 x 16 block and
//    each lane receives one column), so V is never transposed in registers.
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds,
//    16 bytes per lane, hardware zero-fill past the end of the sequence),
//    double-buffered. The blocks of a tile are spread over the phase that
//    issues them. The next item's Q and first K tile stream in during the
//    current item. No staging registers, no staging VALU.
//  * LDS tiles are unpadded and XOR-swizzled per row in 16-byte chunks so that
//    both the 16-byte K reads and the transposing V reads are free of bank
//    conflicts on the 64-bank gfx950 LDS.
//  * Key tiles that the mask hides from all of an item's rows are never
//    loaded. A wave skips the phases of tiles hidden from its own rows.
//    Fully visible tiles run without mask arithmetic; only boundary tiles
//    evaluate the predicate.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kWaves = 8;            // two groups of four, one wave of each per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = 32;        // query rows per wave
static_assert(kWaves * kWaveRows == kBlockM, "workgroup covers kBlockM rows");

// ---- tile geometry per head dimension ---------------------------------------
// D = 128: 64-key tiles; D = 64: 128-key tiles. Either way a K or V tile is
// 16 KiB, a wave issues 32 MFMAs per tile, and a stage (K + V) is 32 KiB.
template <int D> struct Geom {
    static constexpr int BN = fwd_key_tile(D);   // keys per tile
    static constexpr int RB = 2 * D;                   // bytes per K/V row
    static constexpr int CPR = RB / 16;                // 16-byte chunks per row
    static constexpr int TILE_BYTES = BN * RB;         // one K or V tile
    static constexpr int ROWS_PER_KB = 1024 / RB;      // rows per 1 KiB DMA block
    // A tile is 16 DMA blocks of 1 KiB; the four waves of one group issue them,
    // four blocks each.
    static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / 4;
    static_assert(TILE_BYTES == 16384, "tile geometry");
    static_assert(DMA_PER_WAVE * 4 * 1024 == TILE_BYTES, "DMA split");

    static __device__ __forceinline__ int kchunk(int q, int r) { return dev::kchunk<D>(q, r); }
    static __device__ __forceinline__ int vchunk(int q, int r) { return dev::vchunk<D>(q, r); }
};

// PACKED: rows of a head lie H * D elements apart in packed [T, H, D] tensors
// of variable-length sequences (FwdParams row addressing); otherwise [B, H, S, D].
// ROPE: query rows get their rotary embedding as they are read (FwdParams).
// KS (key split): a work item is kBlockMSplit = 128 query rows; waves w and
// w + 4 own the same 32 rows and take alternate key tiles (group 0 the even
// tiles of the item's range, group 1 the odd ones), each with its own online
// softmax state, merged through LDS at the end of the item. Items are half as
// tall, so a window (or a short causal row block) wastes fewer masked pairs and
// a small grid has twice as many items to balance; the price is the merge and
// twice the K/V tile traffic into LDS per step. Not combined with PACKED (the
// layout fills all 160 KiB of LDS).
template <typename T, int D, bool PACKED, bool ROPE, bool KS>
struct Kernel {
    typedef Geom<D> G;
    typedef typename Elem<T>::vec8 vec8;
    static_assert(!(KS && PACKED), "the key-split layout leaves no LDS for the sequence table");
    static constexpr int BM = KS ? kBlockMSplit : kBlockM;  // query rows per item
    static constexpr int BN = G::BN;
    static constexpr int NKB = BN / 32;   // 32-key score blocks per tile
    static constexpr int NDC = D / 16;    // 16-dim chunks of the QK^T contraction
    static constexpr int NDB = D / 32;    // 32-dim output blocks
    static constexpr int NPC = BN / 16;   // 16-key chunks of the PV contraction
    // The probabilities as MFMA operands: per 32-key block, 8 dwords of pairs
    // rounded to the element type, and for bf16 (8 significant bits) 8 more
    // holding the rounding remainders p - bf16(p), themselves rounded, which a
    // second product with the same V^T operand adds: 16 bits of each
    // probability reach the output. (One bf16 product alone leaves errors of
    // up to 2^-9 of sum_j p_j |v_j| / l, several output ulps where two large
    // terms cancel.)
    static constexpr bool kSplitP = Elem<T>::kCoarse;
    static constexpr int NPW = kSplitP ? 16 : 8;
    typedef uint32_t PBuf[NKB][NPW];

    // Per-wave state carried across key tiles.
    struct State {
        vec8 qf[NDC];       // Q^T fragments (B operand): row r0 + l32, dims 16c + 8g .. +7
        f32x16 oacc[NDB];   // O^T accumulator: lane holds query l32, dims of its C layout
        float m_run;        // reference maximum of the base-2 scaled scores
        float l_run;        // this lane's share of the row sum, relative to m_run
    };

    // Per-lane byte offsets, fixed for the whole key loop.
    struct Addr {
        uint32_t kdma[G::DMA_PER_WAVE];  // global offset of this lane's K chunk, per DMA block
        uint32_t vdma[G::DMA_PER_WAVE];  // same for V (different swizzle)
        uint32_t k[NDC];                 // LDS offset of the K fragment of chunk c, block 0
        uint32_t v[NDB];                 // LDS offset of the V^T fragment of block db, chunk 0
    };

    // Largest growth of the row maximum absorbed without rescaling: while a
    // row's new maximum stays within 2^8 of m_run, probabilities are taken
    // relative to the stale m_run (values up to 256, exact in fp32 and normal
    // in fp16/bf16), so O and l keep a common reference and the final O / l is
    // unchanged. Only a larger jump (or the first tile) rescales.
    static constexpr float kRescaleSlack = 8.0f;
    // A lane's probability sum over a tile up to which no single probability
    // can exceed 2^kRescaleSlack.
    static constexpr float kSlackSum = 256.0f;

    // MFMAs between an LDS operand read and its use in the MFMA phase.
    static constexpr int kDist = 8;

    static __device__ __forceinline__ void make_addr(Addr &ad, int wave, int lane, uint32_t rs) {
        const int l32 = lane & 31, g = lane >> 5;
        // DMA block b = DMA_PER_WAVE * (wave % 4) + i fills tile rows
        // [b * ROWS_PER_KB, +ROWS_PER_KB); lane L lands in physical chunk
        // L % CPR of row L / CPR, so it fetches the logical chunk stored there.
        const int pc = lane % G::CPR;
#pragma unroll
        for (int i = 0; i < G::DMA_PER_WAVE; ++i) {
            const int row = (G::DMA_PER_WAVE * (wave & 3) + i) * G::ROWS_PER_KB + lane / G::CPR;
            ad.kdma[i] = row * rs + G::kchunk(pc, row) * 16;  // XOR swizzle is its own inverse
            ad.vdma[i] = row * rs + G::vchunk(pc, row) * 16;
        }
        // K A operand, score block 0: row l32, logical chunk 2c + g.
#pragma unroll
        for (int c = 0; c < NDC; ++c)
            ad.k[c] = l32 * G::RB + G::kchunk(2 * c + g, l32) * 16;
        // V^T A operand (transposing read), key chunk 0, first half: lane in
        // 16-lane group G16 = lane / 16 (g = G16 / 2, h = G16 % 2), q = lane % 16
        // addresses row 4g + q / 4 and columns 32db + 16h + 4(q % 4) .. +3.
        const int q = lane & 15, h = (lane >> 4) & 1;
        const int vrow = 4 * g + (q >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * h + 4 * (q & 3);
            ad.v[db] = vrow * G::RB + G::vchunk(col >> 3, vrow) * 16 + (col & 7) * 2;
        }
    }

    // The source of one K or V tile: rows k0 .. k0 + BN - 1 of the head whose
    // row 0 is at `h`, rows `rse` elements apart, bound for the LDS slot at byte
    // address `slot`. The buffer resource starts at row k0 and ends with row
    // S - 1, so rows past the sequence read as zero (an empty resource, nrec 0,
    // fills the slot with zeros and reads nothing).
    struct TileSrc {
        i32x4 rsrc;
        uint32_t slot;
    };
    static __device__ __forceinline__ TileSrc tile_src(const uint16_t *h, int k0, int S, int rse,
                                                       uint32_t slot, bool valid = true) {
        const uint32_t nrec = !valid ? 0u
                              : PACKED ? (uint32_t)(S - k0 - 1) * (uint32_t)rse * 2u + G::RB
                                       : (uint32_t)(S - k0) * G::RB;
        return TileSrc{buffer_rsrc(h + (int64_t)k0 * rse, nrec), slot};
    }
    // DMA block i (of DMA_PER_WAVE) of this wave's share of a tile; `off`
    // holds the lane's source offset for it (which carries the matrix's swizzle).
    static __device__ __forceinline__ void dma_block(const TileSrc &s, uint32_t off, int wave,
                                                     int i) {
        dma16(s.rsrc, s.slot + (uint32_t)(G::DMA_PER_WAVE * (wave & 3) + i) * 1024u, off);
    }
    static __device__ __forceinline__ void load_tile(const TileSrc &s,
                                                     const uint32_t (&off)[G::DMA_PER_WAVE],
                                                     int wave) {
#pragma unroll
        for (int i = 0; i < G::DMA_PER_WAVE; ++i) dma_block(s, off[i], wave, i);
    }

    // ---- work items -------------------------------------------------------------
    // A work item is one query tile (BM rows) of one (b, h), taken from the
    // work lists of FwdParams::plan (ListPlan: persistent workgroups, XCD
    // lists, the snake; under a window the equal-cost tiles first). The grid
    // has at most one workgroup per CU and workgroup w runs its items r = 0,
    // 1, ... back to back as one stream of key tiles.
    struct Item {
        int bh, q0;     // head (b*H + h) and first query row
        int t_first;    // first key tile the workgroup's rows can see
        int nt;         // number of key tiles; 0 marks "no more items", -1 "skip this one"
        int t_in_lo, t_in_hi;  // [t_in_lo, t_in_hi): tiles visible in full from every row
        int S;          // PACKED: rows (queries and keys) of the item's sequence
        int64_t base;   // PACKED: element offset of row 0 of the item's head
    };
    // Rows of the item's sequence, and the element offset of row 0 of its head
    // in q, k, v and o (in both layouts, offset / D indexes row 0's LSE).
    // S_all is FwdParams::S, kept in a register by the caller.
    static __device__ __forceinline__ int seq_len(int S_all, const Item &it) {
        return PACKED ? it.S : S_all;
    }
    static __device__ __forceinline__ int64_t head_base(int S_all, const Item &it) {
        return PACKED ? it.base : (int64_t)it.bh * S_all * D;
    }

    static __device__ __forceinline__ Item item_of(const FwdParams &p, int r) {
        Item it;
        it.bh = it.q0 = it.t_first = it.nt = it.t_in_lo = it.t_in_hi = 0;
        int x, bh, qt;
        const int pos = list_pos(p.plan, r, x);
        if (!list_item(p.plan, x, pos, bh, qt)) return it;
        it.bh = bh;
        it.q0 = qt * BM;
        finish_item(p, it, p.S);
        return it;
    }

    // Packed sequences: the table of the launch's sequences (clamped start
    // token and length) that every workgroup builds in LDS, and the list
    // order. A list holds every sequence's heads h with h % 8 == x (all
    // heads without XCD lists) and runs its items level by level: first the
    // query tile of index n_qtiles - 1 of every (sequence, head) that has one,
    // then tile n_qtiles - 2, ..., down to tile 0. Item costs thus fall along
    // the list (each tile sees more keys than the one below it under causal
    // and full masks, and the same number under a window), and the snake
    // deals them out evenly however the lengths are mixed.
    struct Walk {
        int lvl;    // query tile index of the current level
        int begin;  // list position of the level's first item
        int count;  // items of the level
    };
    // Sequences with more than `lvl` query tiles (uniform).
    static __device__ __forceinline__ int active_count(const LDS i32x2 *tab, int n, int lvl) {
        const int lane = threadIdx.x & 63;
        int total = 0;
        for (int c = 0; c < n; c += 64) {
            const bool a = c + lane < n && tab[c + lane].y > lvl * BM;
            total += __builtin_popcountll(__builtin_amdgcn_ballot_w64(a));
        }
        return total;
    }
    // Index of the k-th (from 0) sequence with more than `lvl` query tiles.
    static __device__ __forceinline__ int active_select(const LDS i32x2 *tab, int n, int lvl,
                                                        int k) {
        const int lane = threadIdx.x & 63;
        for (int c = 0; c < n; c += 64) {
            const bool a = c + lane < n && tab[c + lane].y > lvl * BM;
            const uint64_t m = __builtin_amdgcn_ballot_w64(a);
            const int cnt = __builtin_popcountll(m);
            if (k < cnt) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                const uint64_t sel = __builtin_amdgcn_ballot_w64(a && (int)below == k);
                return c + (int)__builtin_ctzll(sel);
            }
            k -= cnt;
        }
        return 0;  // not reached for k < active_count(tab, n, lvl)
    }
    static __device__ __forceinline__ Item packed_item(const FwdParams &p, const LDS i32x2 *tab,
                                                       Walk &wk, int r) {
        Item it;
        it.bh = it.q0 = it.t_first = it.nt = it.t_in_lo = it.t_in_hi = it.S = 0;
        it.base = 0;
        int x;
        const int pos = list_pos(p.plan, r, x);
        const int hpl = p.plan.xcd_lists ? p.H >> 3 : p.H;  // heads per sequence in a list
        while (pos >= wk.begin + wk.count) {
            if (wk.lvl == 0) return it;  // past the last level: no more items
            wk.begin += wk.count;
            --wk.lvl;
            wk.count = hpl * active_count(tab, p.B, wk.lvl);
        }
        const int within = pos - wk.begin;
        const int k = within / hpl, i = within - k * hpl;
        const int b = active_select(tab, p.B, wk.lvl, k);
        const int start = __builtin_amdgcn_readfirstlane(tab[b].x);
        const int S = __builtin_amdgcn_readfirstlane(tab[b].y);
        const int h = p.plan.xcd_lists ? i * 8 + x : i;
        it.bh = b * p.H + h;
        it.q0 = wk.lvl * BM;
        it.S = S;
        it.base = ((int64_t)start * p.H + h) * D;
        finish_item(p, it, S);
        return it;
    }

    // Fill in the key-tile range of an item whose bh, q0 (< S) are set.
    static __device__ __forceinline__ void finish_item(const FwdParams &p, Item &it, int S) {
        const int qlast = min(it.q0 + BM - 1, S - 1);
        // Keys visible from any row of the item, in whole tiles; tiles outside
        // are never loaded. Every wave walks all of them: a tile hidden from a
        // wave's rows is simply fully masked for that wave.
        it.t_first = max(0, it.q0 - p.win_lo) / BN;
        const int t_last = min(S - 1, qlast + p.win_hi) / BN;
        it.nt = t_last - it.t_first + 1;
        // Tiles visible in full from every valid row of the item:
        // k0 >= qlast - win_lo and k0 + BN - 1 <= min(S - 1, q0 + win_hi).
        it.t_in_lo = max(it.t_first, (max(0, qlast - p.win_lo) + BN - 1) / BN);
        it.t_in_hi = (min(S - 1, it.q0 + p.win_hi) + 1) / BN;  // one past the last
        // Uniform across the workgroup: keep it in scalar registers.
        it.bh = __builtin_amdgcn_readfirstlane(it.bh);
        it.q0 = __builtin_amdgcn_readfirstlane(it.q0);
        it.t_first = __builtin_amdgcn_readfirstlane(it.t_first);
        it.nt = __builtin_amdgcn_readfirstlane(it.nt);
        it.t_in_lo = __builtin_amdgcn_readfirstlane(it.t_in_lo);
        it.t_in_hi = __builtin_amdgcn_readfirstlane(it.t_in_hi);
    }

    // The workgroup's item of round r (nt == 0: none left).
    static __device__ __forceinline__ Item next_item(const FwdParams &p, const LDS i32x2 *tab,
                                                     Walk &wk, int r) {
        if constexpr (PACKED)
            return packed_item(p, tab, wk, r);
        else
            return item_of(p, r);
    }

    // ---- phases -----------------------------------------------------------------
    // The workgroup's eight waves form two groups (waves 0-3 and 4-7; one wave
    // of each group per SIMD) that alternate between two kinds of work, so
    // that on every SIMD one wave keeps the matrix core busy while the other
    // runs the softmax on the VALU:
    //   M_m: O^T += V^T P^T of tile m - 1, then S^T = K Q^T of tile m (MFMA);
    //   V_m: mask, online softmax and P of tile m (VALU).
    // A group runs M_0, V_0, M_1, V_1, ..., M_T; group 1 runs each one phase
    // after group 0. Step i (one workgroup barrier at its end) holds M_i, V_i
    // of group 0 and V_(i-1), M_i of group 1. K(t) and V(t - 1) are read in
    // step t; both stream in (DMA) a step ahead and are double-buffered.

    // The probabilities of a tile's scores relative to reference mu: rounded
    // into pk (and, for bf16, their remainders), summed unrounded into psum;
    // dma(b), b = 0 .. NDMA - 1, spread over the exponentials.
    template <int NDMA, typename Dma>
    static __device__ __forceinline__ void probs(const f32x16 (&sacc)[NKB], PBuf &pk, float c2,
                                                 float mu, float &psum, const Dma &dma) {
        float psum0 = 0.0f, psum1 = 0.0f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, -mu));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], c2, -mu));
                const uint32_t hi = Elem<T>::pack(p0, p1);
                pk[kb][r >> 1] = hi;
                if constexpr (kSplitP) {
                    const float h0 = __builtin_bit_cast(float, hi << 16);
                    const float h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
                    pk[kb][8 + (r >> 1)] = Elem<T>::pack(p0 - h0, p1 - h1);
                }
                psum0 += p0;
                psum1 += p1;
                if constexpr (NDMA > 0) {
                    constexpr int kIters = NKB * 8;  // exponential pairs per lane
                    constexpr int kEvery = kIters / NDMA;
                    static_assert(kEvery * NDMA == kIters, "DMA calls spread evenly");
                    const int it = kb * 8 + (r >> 1);
                    if (it % kEvery == kEvery - 1) dma(it / kEvery);
                }
            }
        psum = psum0 + psum1;
    }

    // Softmax of one tile: mask (boundary tiles), tile maximum, rescale of O
    // and l when some row's maximum outgrows the slack (always on the first
    // visible tile, where m_run is -inf), and the probabilities: rounded once
    // to the MFMA operand type into pk, summed unrounded into l.
    // dma(b), b = 0 .. NDMA - 1, issues one DMA block of the caller's; the
    // calls are spread over the exponentials (all of them, in order, on every
    // path).
    template <int NDMA = 4, typename Dma>
    static __device__ __forceinline__ void softmax(State &st, f32x16 (&sacc)[NKB],
                                                   PBuf &pk, bool masked, int k0,
                                                   int qi, int S, int win_lo, int win_hi,
                                                   float c2, int g, const Dma &dma) {
        // Accumulator element r of block kb holds key k0 + 4g + off for query qi,
        // off = 32kb + 8(r/4) + r%4 (a compile-time constant). The key is
        // visible iff lo <= off <= hi, with lo = qi - win_lo - (k0 + 4g) and
        // hi = min(qi + win_hi, S - 1) - (k0 + 4g); a hidden score becomes -inf
        // (with c2 > 0 its probability exp2(-inf) is exactly 0). Per element
        // that is a compare against a constant and a select, plus, when some
        // lane's lower bound cuts into the tile (windows), a subtraction and an
        // unsigned range compare. A tile that hides every key from the wave's
        // rows leaves the softmax state as it is and gives P = 0.
        if (masked) {
            const int base = k0 + 4 * g;
            const int hi = min(qi + win_hi, S - 1) - base;
            const int lo = qi - win_lo - base;
            constexpr int kMaxOff = 32 * (NKB - 1) + 8 * 3 + 3;
            if (!__builtin_amdgcn_ballot_w64(hi >= 0 && lo <= kMaxOff && hi >= lo)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < NPW; ++r) pk[kb][r] = 0u;
#pragma unroll
                for (int b = 0; b < NDMA; ++b) dma(b);
                return;
            }
            if (!__builtin_amdgcn_ballot_w64(lo > 0)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                        sacc[kb][r] = off <= hi ? sacc[kb][r] : -INFINITY;
                    }
            } else {
                const uint32_t w = (uint32_t)(hi - lo);  // > w unsigned: outside [lo, hi]
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                        sacc[kb][r] = (uint32_t)(off - lo) <= w ? sacc[kb][r] : -INFINITY;
                    }
            }
        }
        // Fast path (fp16), once every row of the wave has a reference: take
        // the probabilities against the current m_run without forming the
        // tile's maximum. If no lane's probabilities add up to more than 2^8,
        // none exceeds the slack and the reference stands (the condition the
        // tile maximum would have checked, m_tile <= m_run + 8, for each
        // value); otherwise the tile goes the slow way below (DMA already
        // issued). Measured 2% faster on the causal and full B4 H32 S4096 D128
        // workloads; for bf16, whose probabilities take twice the work, a
        // redone tile costs more than the maximum saves (6% slower with the
        // x20 key outliers), so bf16 always forms the maximum.
        bool issued = false;
        if (!kSplitP && !__builtin_amdgcn_ballot_w64(st.m_run == -INFINITY)) {
            float psum;
            probs<NDMA>(sacc, pk, c2, st.m_run, psum, dma);
            if (!__builtin_amdgcn_ballot_w64(!(psum <= kSlackSum))) {
                st.l_run += psum;
                return;
            }
            issued = true;
        }
        // c2 > 0, so the maximum of the scaled scores is c2 times the maximum score.
        float smax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
        smax = max_with_partner(smax);
        const float m_tile = (smax == -INFINITY) ? -INFINITY : smax * c2;
        // O (which holds the tiles before this one) and l move to the new
        // reference here, in the softmax phase, so the MFMA phase carries no
        // rescale check.
        if (__builtin_amdgcn_ballot_w64(m_tile > st.m_run + kRescaleSlack)) {
            const float m_new = fmaxf(st.m_run, m_tile);
            const float alpha =
                (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m_run - m_new);
            st.m_run = m_new;
            st.l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) st.oacc[db] *= alpha;
        }
        const float mu = (st.m_run == -INFINITY) ? 0.0f : st.m_run;
        float psum;
        if (issued) probs<0>(sacc, pk, c2, mu, psum, dma);
        else probs<NDMA>(sacc, pk, c2, mu, psum, dma);
        st.l_run += psum;
    }

    // LDS: the K slots then the V slots. Without the key split: two of each,
    // relative tile i in slot i & 1. With it: four of each, group g's tile of
    // step i in slot 2 (i & 1) + g.
    static constexpr int NSLOT = KS ? 4 : 2;
    static __device__ __forceinline__ uint32_t kslot(int i, int grp = 0) {
        return (KS ? 2 * (i & 1) + grp : (i & 1)) * G::TILE_BYTES;
    }
    static __device__ __forceinline__ uint32_t vslot(int i, int grp = 0) {
        return (NSLOT + (KS ? 2 * (i & 1) + grp : (i & 1))) * G::TILE_BYTES;
    }
    // After the tile slots: Q of the workgroup's next item, BM rows in the K
    // swizzle, 32-row block b read by the wave(s) owning those rows: wave b
    // (b = w & 3 for both w and w + 4 under the key split, each of which
    // DMAs half of the block's 1 KiB pieces).
    static constexpr uint32_t kQRegion = 2 * NSLOT * G::TILE_BYTES;
    // LDS byte offset of the packed-sequence table (after the Q region).
    static constexpr uint32_t kTabOffset = kQRegion + BM * G::RB;
    static constexpr int kQBlocks = kWaveRows * G::RB / 1024;  // 1 KiB DMA blocks per 32 rows
    static_assert(kTabOffset <= 160 * 1024, "LDS budget");
    // The 32-row block of the item (and of the Q region) this wave owns.
    static __device__ __forceinline__ int row_block(int wave) { return KS ? (wave & 3) : wave; }
    // The wave's share [lo, hi) of its row block's Q pieces.
    static __device__ __forceinline__ int qpiece_lo(int wave) {
        return KS ? (wave >> 2) * (kQBlocks / 2) : 0;
    }
    static __device__ __forceinline__ int qpiece_hi(int wave) {
        return KS ? ((wave >> 2) + 1) * (kQBlocks / 2) : kQBlocks;
    }

    // DMA this wave's 32 rows of the item's Q (rows past S read as zero) into
    // its part of the Q region. Lane L of 1 KiB block b lands in physical
    // chunk L % CPR of region row b * ROWS_PER_KB + L / CPR, so it fetches the
    // logical chunk that the K swizzle stores there.
    // Blocks [b0, b1) of the wave's kQBlocks.
    static __device__ __forceinline__ void dma_q(const uint16_t *qh, int q0, int S, int rse,
                                                 uint32_t smem_addr, int wave, int lane,
                                                 int b0, int b1) {
        const int rb = row_block(wave);
        const int r0 = q0 + rb * kWaveRows;
        // A wave whose rows all lie past S gets an empty resource: every read
        // returns zero and nothing past the tensor is touched.
        const uint32_t nrec = r0 >= S ? 0u
                              : PACKED ? (uint32_t)(S - r0 - 1) * (uint32_t)rse * 2u + G::RB
                                       : (uint32_t)(S - r0) * G::RB;
        const i32x4 rsrc = buffer_rsrc(qh + (int64_t)r0 * rse, nrec);
        const uint32_t base = smem_addr + kQRegion + (uint32_t)(rb * kWaveRows) * G::RB;
        const int pc = lane % G::CPR;
#pragma unroll
        for (int b = 0; b < kQBlocks; ++b) {
            const int row = b * G::ROWS_PER_KB + lane / G::CPR;
            if (b >= b0 && b < b1)
                dma16(rsrc, base + (uint32_t)b * 1024u,
                      (uint32_t)row * (uint32_t)rse * 2u + (uint32_t)(G::kchunk(pc, row) * 16));
        }
    }

    // The epilogue of an item for one wave: O = O_acc / l (rounded to the
    // element type), LSE = ln 2 * (m + log2 l).
    // Blocks [DB0, DB1) of the D / 32 output blocks (all of them unless the key
    // split divides the row between a pair of waves); the LSE with write_lse.
    template <int DB0 = 0, int DB1 = NDB>
    static __device__ __forceinline__ void store_output(const FwdParams &p, const State &st,
                                                        int64_t head, int bh, int qi, int S,
                                                        int rse, int g, bool write_lse = true) {
        const float l_tot = sum_with_partner(st.l_run);
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        // Elements 4a .. 4a + 3 of block db hold dims 32db + 8a + 4g + 0..3 of
        // the row, which lanes l and l ^ 32 share. For each pair of 8-dim
        // chunks (2c, 2c + 1) the two lanes trade halves (v_permlane32_swap
        // trades lanes 32-63 of its first operand with lanes 0-31 of its
        // second), so that lane half g holds chunk 2c + g whole and stores it
        // with one 16-byte write: 32 contiguous bytes of a row per pair of
        // lanes instead of 16 (the O stores otherwise stall the epilogue).
        u32x4 ow[NDB][2];
#pragma unroll
        for (int db = DB0; db < DB1; ++db)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const f32x16 &a = st.oacc[db];
                const int e0 = 8 * c, e1 = 8 * c + 4;  // chunks 2c and 2c + 1
                const uint32_t x00 = Elem<T>::pack(a[e0 + 0] * inv, a[e0 + 1] * inv);
                const uint32_t x01 = Elem<T>::pack(a[e0 + 2] * inv, a[e0 + 3] * inv);
                const uint32_t x10 = Elem<T>::pack(a[e1 + 0] * inv, a[e1 + 1] * inv);
                const uint32_t x11 = Elem<T>::pack(a[e1 + 2] * inv, a[e1 + 3] * inv);
                const auto r0 = __builtin_amdgcn_permlane32_swap(x00, x10, false, false);
                const auto r1 = __builtin_amdgcn_permlane32_swap(x01, x11, false, false);
                ow[db][c] = u32x4{(uint32_t)r0[0], (uint32_t)r1[0], (uint32_t)r0[1],
                                  (uint32_t)r1[1]};
            }
        if (qi < S) {
            uint16_t *orow = static_cast<uint16_t *>(p.o) + head + (int64_t)qi * rse;
#pragma unroll
            for (int db = DB0; db < DB1; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    *reinterpret_cast<u32x4 *>(orow + 32 * db + 16 * c + 8 * g) = ow[db][c];
            if (p.lse && g == 0 && write_lse) {
                const float lse = l_tot > 0.0f
                                      ? 0.69314718055994531f * (st.m_run + __log2f(l_tot))
                                      : -INFINITY;
                if (PACKED)
                    p.lse[head / D + (int64_t)qi * p.H] = lse;
                else
                    p.lse[(int64_t)bh * S + qi] = lse;
            }
        }
    }

    // The key loop of one wave: steps 0 .. T (T tiles), each ended by a
    // workgroup barrier. In step i group 0 runs M_i then V_i, group 1 runs
    // V_(i-1) then M_i, so on each SIMD the two waves' MFMA and softmax phases
    // interleave with no barrier between them. In step i the waves of group 0
    // issue the DMA of K(i + 1) between their MFMAs and those of group 1 the
    // DMA of V(i) between their exponentials; at the end of the step every wave
    // waits for its own DMA, so after that barrier both tiles are in LDS.
    // Step i reads K(i) and V(i - 1) and writes K(i + 1) and V(i) into the
    // slots of K(i - 1) and V(i - 2), which step i - 1 read: the barrier
    // between the steps orders every refill after the reads it replaces.
    struct Loop {
        const FwdParams &p;
        const LDS char *smem;
        uint32_t smem_addr;
        const uint16_t *kh, *vh;
        int S, S_all, rse, t_first, ntiles, t_in_lo, t_in_hi, r0, rlast, qi, win_lo, win_hi;
        float c2;
        int g, wave, lane;
        const Addr &ad;
        int kbase;             // slot parity of this item's tile 0
        const Item &nx;        // the workgroup's next item (nx.nt == 0: none)
        int64_t head;          // element offset of row 0 of the item's head
        int bh;
        int nsteps;            // steps of the key loop before the final one (T)

        __device__ __forceinline__ bool tile_full(int t) const {
            const int k0 = t * BN;
            return (t >= t_in_lo && t < t_in_hi) ||
                   (k0 + BN - 1 <= S - 1 && k0 + BN - 1 <= r0 + win_hi && k0 >= rlast - win_lo);
        }
        // The tiles streamed in step i: K(i + 1) (after the last tile, the next
        // item's K(0), in the slot its parity continues into; with no next item
        // an empty source zero-fills the free slot) and V(i).
        __device__ __forceinline__ TileSrc ksrc(int i) const {
            if (i + 1 < ntiles)
                return tile_src(kh, (t_first + i + 1) * BN, S, rse, smem_addr + kslot(kbase + i + 1));
            return tile_src(static_cast<const uint16_t *>(p.k) + head_base(S_all, nx),
                            nx.t_first * BN, seq_len(S_all, nx), rse,
                            smem_addr + kslot(kbase + i + 1), nx.nt > 0);
        }
        __device__ __forceinline__ TileSrc vsrc(int i) const {
            return tile_src(vh, (t_first + i) * BN, S, rse, smem_addr + vslot(kbase + i));
        }
        // At steps i = 1 .. T: each wave's rows of the next item's Q, two 1 KiB
        // blocks per step (the rest at step T), so that no step stalls on a
        // burst of DMA. This item's Q has left the Q region (for registers)
        // before step 0 ends.
        __device__ __forceinline__ void dma_q_next(int i) const {
            constexpr int kPerPhase = 2;
            const int lo = qpiece_lo(wave), hi = qpiece_hi(wave);
            const int b0 = lo + kPerPhase * (i - 1);
            const int b1 = i == nsteps ? hi : min(hi, lo + kPerPhase * i);
            if (nx.nt > 0 && b0 < hi)
                dma_q(static_cast<const uint16_t *>(p.q) + head_base(S_all, nx), nx.q0,
                      seq_len(S_all, nx), rse, smem_addr, wave, lane, b0, b1);
        }
        // M_i: O^T += V^T P^T of tile i - 1 and S^T = K Q^T of tile i, as one stream
        // of MFMAs whose LDS operands are read kDist MFMAs ahead. P V chunk c's
        // B operand is P^T elements 8(c%2) .. +7 of score block c/2 (keys
        // 16c + 8a + 4g + b for element 4a + b); its A operand comes from two
        // transposing reads, rows 16c + 4g + (0..3) and 16c + 8 + 4g + (0..3),
        // offsets that keep the V swizzle of the lane's base row.
        // With DMA (group 0, step i < T) the wave also issues its
        // share of K(i + 1), one 1 KiB block after every NS / 4 MFMAs (group 1
        // streams V(i) from its softmax phase): issued all at once by every
        // wave, the 32 KiB of a phase queue up behind each other and stall the
        // issuing waves.
        template <bool QK, bool PV, bool DMA>
        __device__ __forceinline__ void mphase(State &st, f32x16 (&sacc)[NKB], const PBuf &pk,
                                               int i) const {
            TileSrc kt{};
            if constexpr (DMA) kt = ksrc(i);
            mcore<QK, PV, DMA ? G::DMA_PER_WAVE : 0>(
                st, sacc, pk, smem + kslot(kbase + i), smem + vslot(kbase + i - 1),
                [&](int b) { dma_block(kt, ad.kdma[b], wave, b); });
        }
        // The MFMA stream of a phase: P V of the tile whose V^T sits at `vs`
        // (PV) and the scores of the tile whose K sits at `ks` (QK), one after
        // the other or (fp16) alternating; with NDMA > 0, dma(b) for b = 0 ..
        // NDMA - 1 is called once every NS / NDMA MFMAs.
        template <bool QK, bool PV, int NDMA, typename Dma>
        __device__ __forceinline__ void mcore(State &st, f32x16 (&sacc)[NKB], const PBuf &pk,
                                              const LDS char *ks,
                                              const LDS char *vs, const Dma &dma) const {
            __builtin_amdgcn_s_setprio(1);
            // MFMA slot s < NPV: P V chunk c, block db; with the split P, chunk
            // c's slots are its NDB products of the rounded P, then its NDB of
            // the remainders, which reuse the V^T operands of the first NDB
            // (each accumulator's two products stay NDB slots apart).
            constexpr int NPP = kSplitP ? 2 : 1;
            constexpr int NPV = PV ? NPC * NDB * NPP : 0;
            constexpr int NQK = QK ? NDC * NKB : 0;  // then S^T chunk q / NKB, block q % NKB
            constexpr int NS = NPV + NQK;
            auto pv_slot = [](int s, int &c, int &db, int &half) {
                c = s / (NDB * NPP);
                half = (s / NDB) % NPP;
                db = s % NDB;
            };
            // LDS reads of slot s (the remainder slots read nothing)
            auto nreads = [&](int s) { return s < NPV ? ((s / NDB) % NPP == 0 ? 2 : 0) : 1; };
            vec8 a[NS];
            auto load = [&](int s) {
                if (s < NPV) {
                    int c, db, half;
                    pv_slot(s, c, db, half);
                    if (half) return;
                    const LDS char *base = vs + ad.v[db] + 16 * c * G::RB;
                    const fp16x4_t lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS fp16x4_t *)(base));
                    const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                        (LDS fp16x4_t *)(base + 8 * G::RB));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    a[s] = __builtin_bit_cast(vec8, u32x4{l2[0], l2[1], h2[0], h2[1]});
                } else {
                    const int q = s - NPV, c = q / NKB, kb = q % NKB;
                    a[s] = *reinterpret_cast<const LDS vec8 *>(ks + ad.k[c] + kb * 32 * G::RB);
                }
            };
            auto mma = [&](int s) {
                if (s < NPV) {
                    int c, db, half;
                    pv_slot(s, c, db, half);
                    // pairs 4 (c & 1) .. + 3 of block c / 2: words 4 (c & 1) + j
                    // (rounded) or 8 + 4 (c & 1) + j (remainders)
                    const int kb = c >> 1, w0 = 8 * half + 4 * (c & 1);
                    const u32x4 pw = {pk[kb][w0 + 0], pk[kb][w0 + 1], pk[kb][w0 + 2],
                                      pk[kb][w0 + 3]};
                    st.oacc[db] = Elem<T>::mma(a[half ? s - NDB : s], __builtin_bit_cast(vec8, pw),
                                               st.oacc[db]);
                } else {
                    const int q = s - NPV, c = q / NKB, kb = q % NKB;
                    sacc[kb] = Elem<T>::mma(a[s], st.qf[c], c == 0 ? f32x16{} : sacc[kb]);
                }
            };
            // Issue order u -> slot. With both products and a single P term
            // (fp16), P V and score slots alternate. The scores form only NKB
            // accumulator chains (two at D = 128). An MFMA waits for the
            // previous one of its chain for about two MFMA times, so with the
            // other wave of the SIMD in its softmax, two chains alone leave
            // the matrix core idle a third of the time; between the P V
            // products (NDB more chains) they do not.
            constexpr bool kMix = PV && QK && !kSplitP && NPV == NQK;
            auto at = [](int u) { return kMix ? ((u & 1) ? NPV + (u >> 1) : (u >> 1)) : u; };
#pragma unroll
            for (int u = 0; u < kDist && u < NS; ++u) load(at(u));
            constexpr int kPer = NS / (NDMA > 0 ? NDMA : 1);  // MFMAs per DMA block
            static_assert(NDMA == 0 || kPer * NDMA == NS, "DMA blocks spread evenly");
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                if (u + kDist < NS) load(at(u + kDist));
                mma(at(u));
                if constexpr (NDMA > 0)
                    if (u % kPer == kPer - 1) dma(u / kPer);
            }
            // Issue order: the first kDist reads, then per slot its look-ahead
            // read(s) and its MFMA.
            auto read_group = [&](int s) {
                if (nreads(s) == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                else if (nreads(s) == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            };
#pragma unroll
            for (int u = 0; u < kDist && u < NS; ++u) read_group(at(u));
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                if (u + kDist < NS) read_group(at(u + kDist));
                __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
            }
            if (QK) pin(sacc);
            if (PV) pin(st.oacc);
            __builtin_amdgcn_s_setprio(0);
            conservative_lds_wait();
        }
        // With DMA (group 1 in step i + 1, i + 1 < T) the wave issues its
        // share of V(i + 1), one block after each quarter of the exponentials.
        template <bool DMA>
        __device__ __forceinline__ void vphase(State &st, f32x16 (&sacc)[NKB], PBuf &pk,
                                               int i) const {
            const int t = t_first + i;
            TileSrc vt{};
            if constexpr (DMA) vt = vsrc(i + 1);
            const auto dma = [&](int b) {
                if constexpr (DMA) dma_block(vt, ad.vdma[b], wave, b);
            };
            softmax(st, sacc, pk, !tile_full(t), t * BN, qi, S, win_lo, win_hi, c2, g, dma);
            pin(pk);
            pin(st.l_run);
            pin(st.m_run);
            conservative_lds_wait();
        }
        // The end of a step: this wave's DMA has landed, then a bare barrier
        // (the kernel orders its own LDS traffic: every LDS read of a step has
        // returned before the step ends, the pinned MFMA results consumed
        // them, so a slot may be refilled after the barrier).
        static __device__ __forceinline__ void end_step() {
            __builtin_amdgcn_s_waitcnt(0);
            fence_barrier();
        }

        // Group 0's share of the K DMA of step i without MFMAs.
        __device__ __forceinline__ void dma_k(int i) const {
            const TileSrc kt = ksrc(i);
#pragma unroll
            for (int b = 0; b < G::DMA_PER_WAVE; ++b) dma_block(kt, ad.kdma[b], wave, b);
        }
        // Returns true when the wave has already stored its output (group 0
        // does so in the first step whose tiles its rows cannot see, where it
        // has no other work, instead of at the item boundary).
        // At D = 64 (128-key tiles: a softmax phase of 64 scores per lane
        // against 32 MFMAs) a second barrier between the halves of a step keeps
        // the two groups' phases aligned: 6% faster there, while at D = 128
        // the halves balance without it (1% faster without).
        static __device__ __forceinline__ void mid_step() {
            if constexpr (D == 64 || kConservativeSync) {
                conservative_lds_wait();
                fence_barrier();
            }
        }
        // ---- key split (KS) --------------------------------------------------------
        // Group g's step i works on the item's relative tile 2i + g (a tile past
        // the item's range is an empty source: zero-filled, never read from HBM,
        // and skipped by every wave). The K tiles of step i + 1 (both groups')
        // stream in from group 0's MFMA phase of step i, the V tiles of step i
        // from group 1's softmax phase of step i. Slots: group g's tiles of step
        // i in K / V slot 2 (i & 1) + g, so step i + 1's refills land in the
        // slots step i - 1 read, as without the split.
        static constexpr int DPW = G::DMA_PER_WAVE;
        __device__ __forceinline__ TileSrc ks_ksrc(int i, int grp) const {
            const int rel = 2 * (i + 1) + grp;
            if (i + 1 < nsteps)
                return tile_src(kh, (t_first + rel) * BN, S, rse,
                                smem_addr + kslot(kbase + i + 1, grp), rel < ntiles);
            return tile_src(static_cast<const uint16_t *>(p.k) + head_base(S_all, nx),
                            (nx.t_first + grp) * BN, seq_len(S_all, nx), rse,
                            smem_addr + kslot(kbase + i + 1, grp), nx.nt > grp);
        }
        __device__ __forceinline__ TileSrc ks_vsrc(int i, int grp) const {
            const int rel = 2 * i + grp;
            return tile_src(vh, (t_first + rel) * BN, S, rse, smem_addr + vslot(kbase + i, grp),
                            rel < ntiles);
        }
        // Group 0's K DMA of step i (for step i + 1) without MFMAs; group 1's V
        // DMA of step i without a softmax.
        __device__ __forceinline__ void ks_dma_k(int i) const {
            const TileSrc a = ks_ksrc(i, 0), b = ks_ksrc(i, 1);
#pragma unroll
            for (int x = 0; x < DPW; ++x) dma_block(a, ad.kdma[x], wave, x);
#pragma unroll
            for (int x = 0; x < DPW; ++x) dma_block(b, ad.kdma[x], wave, x);
        }
        __device__ __forceinline__ void ks_dma_v(int i) const {
            const TileSrc a = ks_vsrc(i, 0), b = ks_vsrc(i, 1);
#pragma unroll
            for (int x = 0; x < DPW; ++x) dma_block(a, ad.vdma[x], wave, x);
#pragma unroll
            for (int x = 0; x < DPW; ++x) dma_block(b, ad.vdma[x], wave, x);
        }
        // M phase of group GRP in step i: P V of its tile of step i - 1 (PV),
        // the scores of its tile of step i (QK); with DMA (group 0) the K tiles
        // of step i + 1, one block every NS / (2 DPW) MFMAs.
        template <int GRP, bool QK, bool PV, bool DMA>
        __device__ __forceinline__ void ks_mphase(State &st, f32x16 (&sacc)[NKB], const PBuf &pk,
                                                  int i) const {
            TileSrc a{}, b{};
            if constexpr (DMA) {
                a = ks_ksrc(i, 0);
                b = ks_ksrc(i, 1);
            }
            mcore<QK, PV, DMA ? 2 * DPW : 0>(
                st, sacc, pk, smem + kslot(kbase + i, GRP), smem + vslot(kbase + i - 1, GRP),
                [&](int x) { dma_block(x < DPW ? a : b, ad.kdma[x % DPW], wave, x % DPW); });
        }
        // Softmax of group GRP's tile of step j; with DMA (group 1) the V tiles
        // of step j + 1 spread over the exponentials.
        template <int GRP, bool DMA>
        __device__ __forceinline__ void ks_vphase(State &st, f32x16 (&sacc)[NKB], PBuf &pk,
                                                  int j) const {
            const int t = t_first + 2 * j + GRP;
            TileSrc a{}, b{};
            if constexpr (DMA) {
                a = ks_vsrc(j + 1, 0);
                b = ks_vsrc(j + 1, 1);
            }
            const auto dma = [&](int x) {
                if constexpr (DMA) dma_block(x < DPW ? a : b, ad.vdma[x % DPW], wave, x % DPW);
            };
            softmax<DMA ? 2 * DPW : 4>(st, sacc, pk, !tile_full(t), t * BN, qi, S, win_lo,
                                       win_hi, c2, g, dma);
            pin(pk);
            pin(st.l_run);
            pin(st.m_run);
            conservative_lds_wait();
        }
        // The key loop of a wave under the key split: steps 0 .. T (T = nsteps),
        // one barrier each (two at D = 64), like go(). Group 0 runs M_i, V_i,
        // group 1 V_(i-1), M_i; group 0's steps whose tiles hide every key from
        // the wave's rows keep only their DMA.
        template <int GRP>
        __device__ __forceinline__ void go_ks(State &st) const {
            f32x16 sacc[NKB];
            PBuf pk;
            const int NT = nsteps;
            // This group's steps whose tile shows the wave's rows a key: [f, l].
            const int ng = (ntiles - GRP + 1) >> 1;  // this group's tiles
            int f = 0, l = -1;
            if (r0 < S) {
                const int relo = max(0, r0 - win_lo) / BN - t_first;
                const int rehi = min(S - 1, rlast + win_hi) / BN - t_first;
                f = max(0, (relo - GRP + 1) >> 1);
                l = min(ng - 1, (rehi - GRP) >> 1);  // (an arithmetic shift keeps -1)
            }
            const bool any = f <= l;
            if (GRP == 0) {
                int i = 0;
                const int fs = any ? f : NT;
                for (; i < fs; ++i) {
                    if (i) dma_q_next(i);
                    ks_dma_k(i);
                    mid_step();
                    end_step();
                }
                if (any) {
                    if (i) dma_q_next(i);
                    ks_mphase<0, true, false, true>(st, sacc, pk, i);
                    mid_step();
                    ks_vphase<0, false>(st, sacc, pk, i);
                    end_step();
                    for (++i; i <= l; ++i) {
                        dma_q_next(i);
                        ks_mphase<0, true, true, true>(st, sacc, pk, i);
                        mid_step();
                        ks_vphase<0, false>(st, sacc, pk, i);
                        end_step();
                    }
                    dma_q_next(i);
                    if (i < NT) ks_mphase<0, false, true, true>(st, sacc, pk, i);
                    else ks_mphase<0, false, true, false>(st, sacc, pk, i);
                    mid_step();
                    end_step();
                    ++i;
                }
                for (; i <= NT; ++i) {
                    if (i) dma_q_next(i);
                    if (i < NT) ks_dma_k(i);
                    mid_step();
                    end_step();
                }
            } else {
                // Group 1 walks all of its steps: a tile hidden from the wave's
                // rows (at most one at either end of an item) takes the masked
                // softmax's all-hidden path, P = 0. (Skipping those steps, as
                // group 0 does, made the compiler spill registers here.)
                ks_dma_v(0);
                mid_step();
                ks_mphase<1, true, false, false>(st, sacc, pk, 0);
                end_step();
                for (int i = 1; i < NT; ++i) {
                    dma_q_next(i);
                    ks_vphase<1, true>(st, sacc, pk, i - 1);
                    mid_step();
                    ks_mphase<1, true, true, false>(st, sacc, pk, i);
                    end_step();
                }
                dma_q_next(NT);
                ks_vphase<1, false>(st, sacc, pk, NT - 1);
                mid_step();
                ks_mphase<1, false, true, false>(st, sacc, pk, NT);
                end_step();
            }
        }
        // End of an item under the key split: waves w and w ^ 4 hold the same
        // rows' (O, m, l) over complementary key tiles. Each keeps half of the
        // output blocks (group 0 the first half) and hands the other half, with
        // its m and l, to its partner through LDS: the V slots (free once the
        // last step's P V has read them) take the O halves, the K slots of the
        // last step's parity (the next item's first K tiles went to the other
        // parity) take m and l. Merged: m = max(m_a, m_b), O = 2^(m_a - m) O_a +
        // 2^(m_b - m) O_b, likewise l. The second barrier keeps the next item's
        // DMA into these slots behind every read.
        template <int GRP>
        __device__ __forceinline__ void ks_merge(State &st) const {
            constexpr int NH = NDB / 2;
            constexpr int GIVE = GRP == 0 ? NH : 0, KEEP = GRP == 0 ? 0 : NH;
            LDS float *xo = (LDS float *)(smem + vslot(0, 0));
            LDS float *xm = (LDS float *)(smem + kslot(kbase + nsteps - 1, 0));
#pragma unroll
            for (int k = 0; k < NH; ++k)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    xo[((wave * NH + k) * 16 + e) * 64 + lane] = st.oacc[GIVE + k][e];
            xm[wave * 128 + lane] = st.m_run;
            xm[wave * 128 + 64 + lane] = st.l_run;
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            fence_barrier();
            const int pw = wave ^ 4;
            const float mp = xm[pw * 128 + lane], lp = xm[pw * 128 + 64 + lane];
            const float m = fmaxf(st.m_run, mp);
            const float as = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.m_run - m);
            const float ap = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mp - m);
#pragma unroll
            for (int k = 0; k < NH; ++k)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    st.oacc[KEEP + k][e] =
                        as * st.oacc[KEEP + k][e] + ap * xo[((pw * NH + k) * 16 + e) * 64 + lane];
            st.l_run = as * st.l_run + ap * lp;
            st.m_run = m;
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            fence_barrier();
        }

        template <int GRP>
        __device__ __forceinline__ bool go(State &st) const {
            f32x16 sacc[NKB];
            PBuf pk;
            const int nt = ntiles;  // >= 1
            // The last tile (relative) with a key visible to this wave's rows:
            // past it, M_i and V_i have nothing to do for the wave.
            const int last = min(S - 1, rlast + win_hi) / BN - t_first;
            if (GRP == 0) {
                mphase<true, false, true>(st, sacc, pk, 0);
                mid_step();
                vphase<false>(st, sacc, pk, 0);
                end_step();
                const int i_end = min(nt, last + 2);
                int i = 1;
                for (; i < i_end; ++i) {
                    dma_q_next(i);
                    mphase<true, true, true>(st, sacc, pk, i);
                    mid_step();
                    vphase<false>(st, sacc, pk, i);
                    end_step();
                }
                bool stored = false;
                for (; i < nt; ++i) {  // tiles hidden from the wave: its DMA only
                    if (D == 128 && !stored) {  // (D = 64 has no registers to spare here)
                        store_output(p, st, head, bh, qi, S, rse, g);
                        stored = true;
                    }
                    dma_q_next(i);
                    dma_k(i);
                    mid_step();
                    end_step();
                }
                dma_q_next(nt);
                if (nt - 1 <= last) mphase<false, true, false>(st, sacc, pk, nt);
                mid_step();
                end_step();
                return stored;
            } else {
                // The first tile (relative) with a key visible to this wave's
                // rows: before it, M_i has nothing to do for the wave (V_i takes
                // its fast path for a hidden tile and still streams its DMA).
                const int first = min(nt, max(0, r0 - win_lo) / BN - t_first);
                load_tile(vsrc(0), ad.vdma, wave);
                mid_step();
                if (first == 0) mphase<true, false, false>(st, sacc, pk, 0);
                end_step();
                int i = 1;
                for (; i < first; ++i) {
                    dma_q_next(i);
                    vphase<true>(st, sacc, pk, i - 1);
                    mid_step();
                    end_step();
                }
                for (; i < nt; ++i) {
                    dma_q_next(i);
                    vphase<true>(st, sacc, pk, i - 1);
                    mid_step();
                    mphase<true, true, false>(st, sacc, pk, i);
                    end_step();
                }
                dma_q_next(nt);
                vphase<false>(st, sacc, pk, nt - 1);
                mid_step();
                if (nt - 1 <= last) mphase<false, true, false>(st, sacc, pk, nt);
                end_step();
                return false;
            }
        }
    };

    static __device__ void run(const FwdParams &p, LDS char *smem) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7
        const int l32 = lane & 31;
        const int g = lane >> 5;
        const int rse = PACKED ? p.row_stride : D;  // elements between consecutive rows of a head
        const int S_all = p.S;  // [B, H, S, D]: every sequence's length
        const int win_lo = p.win_lo, win_hi = p.win_hi;
        const float c2 = p.c2;
        const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
        Addr ad;
        make_addr(ad, wave, lane, (uint32_t)rse * 2u);

        // Packed sequences: the sequence table, with each offset clamped into
        // [0, total_tokens] (an end below its start moved up to it) and each
        // length to S, so that no value of cu_seqlens moves a row out of the
        // tensors.
        LDS i32x2 *tab = reinterpret_cast<LDS i32x2 *>(smem + kTabOffset);
        Walk wk{p.n_qtiles, 0, 0};
        if constexpr (PACKED) {
            const int ntok = p.total_tokens;
            for (int b = threadIdx.x; b < p.B; b += kThreads) {
                const int start = min(max(p.cu_seqlens[b], 0), ntok);
                const int end = min(max(p.cu_seqlens[b + 1], start), ntok);
                tab[b] = i32x2{start, min(end - start, S_all)};
            }
            __syncthreads();
        }

        // The workgroup's items, one after the other. Every item ends with a
        // workgroup barrier after its last LDS read and its wait for its DMA,
        // which includes the next item's K(0) and Q: the next item starts
        // with them in LDS.
        int r = 0;
        Item it = next_item(p, tab, wk, r);
        if (PACKED && it.nt == 0) return;  // every sequence is shorter than the workgroup's share
        {
            // K of the first step: tile 0 (and, under the key split, tile 1 from group 1)
            if (grp == 0 || KS)
                load_tile(tile_src(static_cast<const uint16_t *>(p.k) + head_base(S_all, it),
                                   (it.t_first + grp) * BN, seq_len(S_all, it), rse,
                                   smem_addr + kslot(0, grp), it.nt > grp),
                          ad.kdma, wave);
            dma_q(static_cast<const uint16_t *>(p.q) + head_base(S_all, it), it.q0,
                  seq_len(S_all, it), rse, smem_addr, wave, lane, qpiece_lo(wave),
                  qpiece_hi(wave));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        int kbase = 0;
        while (it.nt > 0) {
            ++r;
            const Item nx = next_item(p, tab, wk, r);
            const int S = seq_len(S_all, it);
            const int64_t head = head_base(S_all, it);
            const uint16_t *kh = static_cast<const uint16_t *>(p.k) + head;
            const uint16_t *vh = static_cast<const uint16_t *>(p.v) + head;

            // This wave's rows.
            const int r0 = it.q0 + row_block(wave) * kWaveRows;
            const int rlast = min(r0 + kWaveRows - 1, S - 1);
            const int qi = r0 + l32;  // this lane's query row

            // Q^T fragments from the Q region: the B-operand fragment of chunk c
            // is row l32, logical chunk 2c + g, the K read pattern.
            State st;
            {
                const LDS char *qs = smem + kQRegion + row_block(wave) * kWaveRows * G::RB;
                const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    u32x4 x = *reinterpret_cast<const LDS u32x4 *>(qs + ad.k[c]);
                    x ^= flip;
                    st.qf[c] = __builtin_bit_cast(vec8, x);
                }
                if constexpr (ROPE) {  // rotary embedding of the row at its position
                    const int64_t at = (int64_t)min(qi, S - 1) * (D / 2);
                    rope_fragments<T, D>(st.qf, g, p.rope_cos + at, p.rope_sin + at,
                                         p.rope_interleaved != 0);
                }
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) st.oacc[db] = f32x16{};
            st.m_run = -INFINITY;
            st.l_run = 0.0f;

            const int nsteps = KS ? (it.nt + 1) >> 1 : it.nt;
            Loop loop{p,     smem,   smem_addr, kh, vh,   S,  S_all,  rse, it.t_first, it.nt,
                      it.t_in_lo, it.t_in_hi, r0, rlast, qi, win_lo, win_hi, c2,  g, wave,
                      lane,  ad,     kbase,     nx,   head, it.bh, nsteps};
            if constexpr (KS) {
                if (grp == 0) {
                    loop.template go_ks<0>(st);
                    loop.template ks_merge<0>(st);
                    store_output<0, NDB / 2>(p, st, head, it.bh, qi, S, rse, g, true);
                } else {
                    loop.template go_ks<1>(st);
                    loop.template ks_merge<1>(st);
                    store_output<NDB / 2, NDB>(p, st, head, it.bh, qi, S, rse, g, false);
                }
            } else {
                const bool stored = grp == 0 ? loop.template go<0>(st) : loop.template go<1>(st);
                if (!stored) store_output(p, st, head, it.bh, qi, S, rse, g);
            }
            kbase += nsteps;
            it = nx;
        }
    }
};

template <typename T, int D, bool PACKED, bool ROPE, bool KS>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_kernel(FwdParams p) {
    typedef Kernel<T, D, PACKED, ROPE, KS> K;
    __shared__ __attribute__((aligned(1024)))
    char smem[K::kTabOffset + (PACKED ? kMaxPackedSeqs * 8 : 0)];
    K::run(p, (LDS char *)smem);
}

template <typename T, int D>
hipError_t launch_t(const FwdParams &p, hipStream_t stream) {
    void *args[] = {const_cast<FwdParams *>(&p)};
    // packed sequences take no rotary embedding
    const void *fn =
        p.cu_seqlens  ? reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, true, false, false>)
        : p.rope_cos  ? (p.key_split
                             ? reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, false, true, true>)
                             : reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, false, true, false>))
        : p.key_split ? reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, false, false, true>)
                      : reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, false, false, false>);
    return hipLaunchKernel(fn, dim3(p.plan.grid), dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int D, int dtype, hipStream_t stream) {
    if (D == 128) return dtype == 0 ? launch_t<_Float16, 128>(p, stream)
                                    : launch_t<__bf16, 128>(p, stream);
    if (D == 64) return dtype == 0 ? launch_t<_Float16, 64>(p, stream)
                                   : launch_t<__bf16, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
