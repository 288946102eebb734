// fa_bwd.hip -- the attention backward pass for gfx950 (MI355X): gradients
// dQ, dK, dV of O = softmax(scale * Q K^T + mask) V for fp16/bf16 [B, H, S, D]
// tensors, D in {64, 128}, with the forward's LSE as the saved state.
//
// What it computes: with P_ij = exp(scale * q_i . k_j - LSE_i) on visible
// pairs (0 elsewhere) and D_i = dO_i . O_i,
//   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . V_j - D_i),
//   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i:
// the gradients of the forward's definition (D_i is the softmax Jacobian's
// row term sum_k P_ik dP_ik). The ops-transformer FlashAttention walkthrough
// (hwcomputing.csdn.net, 6a0ef689), closing remark, notes that the backward
// needs state kept from the forward; the LSE is that state, so P is
// recomputed tile by tile and, as in the forward, no S x S matrix reaches
// memory.
//
// gfx950 design: two kernels, dQ then dK/dV.
//  * fa_bwd_dq: first D_i = dO_i . O_i (fp32) for its rows, into the caller's
//    workspace. A workgroup of 8 waves owns 256 query rows (32 per wave, a
//    row per lane as in the forward) and streams the visible 64-key tiles of
//    K and V through LDS (direct HBM -> LDS DMA, two stages). Per 32-key
//    block: S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16 (Q^T, dO^T
//    fragments held in registers), then P^T, dS^T in fp32 in the accumulator
//    layout (one query per lane: its LSE and D_i are scalars), and
//    dQ^T += K^T dS^T with K^T from transposing LDS reads
//    (ds_read_b64_tr_b16) and dS^T straight from the accumulator.
//  * fa_bwd_dkdv: the mirror image: a workgroup of 8 waves owns 256 keys (32
//    per wave, a key per lane; K^T fragments in registers, the workgroup's V
//    rows in LDS) and streams the 32-query tiles of Q and dO that see them,
//    with their LSE and -D_i staged in LDS. Per tile: S = Q K^T and
//    dP = dO V^T, then P and dS (a query per accumulator row),
//    dV^T += dO^T P and dK^T += Q^T dS.
//  Each streamed tile is read both row-wise (MFMA A operand) and transposed
//  (the A operand of the accumulating product), so it is stored twice, once
//  per LDS swizzle, which keeps both read patterns free of bank conflicts.
//  Hidden pairs get the exponent -inf by a select, never a branch. Both
//  kernels run persistent workgroups over the forward's work lists (a
//  head's tiles on one XCD's L2, costly and cheap tiles paired). dQ and dK/dV
//  each own their outputs, so there are no atomics and the results are
//  deterministic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

// Waves per workgroup (each owns 32 fixed rows: queries or keys). Both
// kernels fit two waves per SIMD (under 256 registers each), which lets one
// wave's VALU work run beside the other's MFMAs.
constexpr int kDqWaves = 8;
constexpr int kKvWaves = 8;
static_assert(32 * kDqWaves == kBwdRows && 32 * kKvWaves == kBwdRows, "work item rows");
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int BN_> struct BGeom {
    static constexpr int BN = BN_;                 // streamed rows per tile
    static constexpr int RB = 2 * D;               // bytes per row
    static constexpr int CPR = RB / 16;            // 16-byte chunks per row
    static constexpr int TILE_BYTES = BN * RB;
    static constexpr int ROWS_PER_KB = 1024 / RB;  // rows per 1 KiB DMA block
    static constexpr int NBLK = TILE_BYTES / 1024; // DMA blocks per tile
};

// Swizzles of a tile: row-read (MFMA A operand of rows) or transposed-read.
enum { kRowSwz = 0, kTrSwz = 1 };

template <typename T, int D>
struct Bwd {
    typedef BGeom<D, 64> G;     // dQ kernel: 64-key tiles
    typedef BGeom<D, 32> GQ;    // dK/dV kernel: 32-query tiles
    typedef typename Elem<T>::vec8 vec8;
    static constexpr int BN = G::BN;
    static constexpr int NDC = D / 16;   // 16-dim chunks of a dims contraction
    static constexpr int NDB = D / 32;   // 32-dim output blocks
    static constexpr int NSB = BN / 32;  // 32-row blocks of a streamed tile

    // Element e of a lane's 32 x 32 accumulator block sits at index
    // base + 8(e/4) + e%4 along the streamed dimension; the pair is visible iff
    // that index lies in [first, last]. The offsets are compile-time constants,
    // so a hidden exponent becomes -inf by one compare and select per element
    // (plus a subtraction and an unsigned range compare when some lane's lower
    // bound cuts into the block).
    static __device__ __forceinline__ void mask_block(float (&x)[16], int base, int first,
                                                      int last) {
        const int lo = first - base, hi = last - base;
        if (!__builtin_amdgcn_ballot_w64(lo > 0)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int off = 8 * (e >> 2) + (e & 3);
                x[e] = off <= hi ? x[e] : -INFINITY;
            }
        } else {
            const uint32_t w = (uint32_t)(hi - lo);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int off = 8 * (e >> 2) + (e & 3);
                x[e] = (hi >= lo && (uint32_t)(off - lo) <= w) ? x[e] : -INFINITY;
            }
        }
    }

    // Stream rows r0 .. r0 + NR - 1 of the [S, D] head at h into the LDS
    // tile at byte address slot, with the given swizzle (blocks wave,
    // wave + NW, ... of its 1 KiB DMA blocks are this wave's). Rows past S
    // read as zero.
    template <int SW, int NW, int NR>
    static __device__ __forceinline__ void load_tile(const uint16_t *h, int r0, int S,
                                                     uint32_t slot, int wave, int lane) {
        constexpr int RB = 2 * D, CPR = RB / 16, RPK = 1024 / RB, NBLK = NR * RB / 1024;
        const i32x4 rsrc = buffer_rsrc(h + (int64_t)r0 * D, r0 < S ? (uint32_t)(S - r0) * RB : 0u);
        const int pc = lane % CPR;
#pragma unroll
        for (int i = 0; i < (NBLK + NW - 1) / NW; ++i) {
            const int b = i * NW + wave;
            if (NBLK % NW == 0 || b < NBLK) {
                const int row = b * RPK + lane / CPR;
                const int lc = SW == kRowSwz ? kchunk<D>(pc, row) : vchunk<D>(pc, row);
                dma16(rsrc, slot + (uint32_t)b * 1024u, (uint32_t)(row * RB + lc * 16));
            }
        }
    }

    // MFMA B-operand fragments of one row (registers): fragment c holds dims
    // 16c + 8g .. + 7 of row r of the [S, D] head at h; zero past S.
    static __device__ __forceinline__ void load_frags(const uint16_t *h, int r, int S, int g,
                                                      vec8 (&f)[NDC]) {
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (r < S) x = *reinterpret_cast<const u32x4 *>(h + (int64_t)r * D + 16 * c + 8 * g);
            f[c] = __builtin_bit_cast(vec8, x);
        }
    }

    // Per-lane LDS offsets. Row read (A operand of 32 rows x 16 dims): row l32,
    // logical chunk 2c + g. Transposed read (A operand of 32 dims x 16 rows,
    // dims block db): as the forward's V^T read.
    struct Offs {
        uint32_t row[NDC];
        uint32_t tr[NDB];
    };
    static __device__ __forceinline__ void make_offs(Offs &o, int lane) {
        const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
        for (int c = 0; c < NDC; ++c) o.row[c] = l32 * G::RB + kchunk<D>(2 * c + g, l32) * 16;
        const int q = lane & 15, h = (lane >> 4) & 1;
        const int trow = 4 * g + (q >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * h + 4 * (q & 3);
            o.tr[db] = trow * G::RB + vchunk<D>(col >> 3, trow) * 16 + (col & 7) * 2;
        }
    }

    // A operand of 32 rows (block sb of the tile) x dims chunk c.
    static __device__ __forceinline__ vec8 read_rows(const LDS char *tile, const Offs &o, int sb,
                                                     int c) {
        return *reinterpret_cast<const LDS vec8 *>(tile + o.row[c] + sb * 32 * G::RB);
    }
    // A operand of 32 dims (block db) x 16 rows (chunk c16 of the tile), from
    // a tile stored with the transposed-read swizzle. Elements 0-3 are rows
    // 16 c16 + 4g + 0..3, elements 4-7 the same + 8: the rows an accumulator's
    // elements 8hh .. 8hh + 7 hold for the chunk's half hh.
    static __device__ __forceinline__ vec8 read_tr(const LDS char *tile, const Offs &o, int db,
                                                   int c16) {
        const LDS char *base = tile + o.tr[db] + 16 * c16 * G::RB;
        const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS fp16x4_t *)(base));
        const fp16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS fp16x4_t *)(base + 8 * G::RB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(vec8, u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
    static __device__ __forceinline__ vec8 half_of(const uint32_t (&pk)[8], int hh) {
        return __builtin_bit_cast(
            vec8, u32x4{pk[4 * hh + 0], pk[4 * hh + 1], pk[4 * hh + 2], pk[4 * hh + 3]});
    }

    // Store a D^T accumulator (lane = row r of the output, accumulator rows =
    // dims) times mul into row r of the [S, D] head at out.
    static __device__ __forceinline__ void store_rows(uint16_t *out, int r, int g,
                                                      const f32x16 (&acc)[NDB], float mul) {
        uint16_t *orow = out + (int64_t)r * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2 w;
                w[0] = Elem<T>::pack(acc[db][4 * a + 0] * mul, acc[db][4 * a + 1] * mul);
                w[1] = Elem<T>::pack(acc[db][4 * a + 2] * mul, acc[db][4 * a + 3] * mul);
                *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * a + 4 * g) = w;
            }
    }

    // ---- dQ -------------------------------------------------------------------
    // LDS per stage: K rows (row swizzle), K (transposed swizzle), V rows.
    static constexpr uint32_t kDqStage = 3 * G::TILE_BYTES;

    // The workgroup's items from its work list (persistent grid; see
    // ListPlan): a head's query tiles on one XCD, few heads per XCD at a
    // time, costly and cheap tiles paired. An item's LDS stages are free for
    // the next one after a barrier.
    static __device__ void dq(const BwdParams &p, LDS char *smem) {
        for (int r = 0;; ++r) {
            int x, bh, qt;
            const int pos = list_pos(p.dq_plan, r, x);
            if (!list_item(p.dq_plan, x, pos, bh, qt)) break;
            if (r) __syncthreads();
            dq_item(p, smem, __builtin_amdgcn_readfirstlane(bh), __builtin_amdgcn_readfirstlane(qt));
        }
    }
    static __device__ __forceinline__ void dq_item(const BwdParams &p, LDS char *smem, int bh,
                                                   int qt) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int l32 = lane & 31, g = lane >> 5;
        const int S = p.S;
        constexpr int ROWS = 32 * kDqWaves;
        const int q0 = qt * ROWS, qi = q0 + 32 * wave + l32;
        const int64_t head = (int64_t)bh * S * D;
        const uint16_t *qh = static_cast<const uint16_t *>(p.q) + head;
        const uint16_t *kh = static_cast<const uint16_t *>(p.k) + head;
        const uint16_t *vh = static_cast<const uint16_t *>(p.v) + head;
        const uint16_t *doh = static_cast<const uint16_t *>(p.dout) + head;

        vec8 qf[NDC], df[NDC];
        load_frags(qh, qi, S, g, qf);
        load_frags(doh, qi, S, g, df);
        const float lse2 = qi < S ? p.lse[(int64_t)bh * S + qi] * kLog2e : 0.0f;
        // D_i = dO_i . O_i in fp32: this lane's half of the row's dims (the
        // dO fragments it holds), then its partner's (lane ^ 32); written to
        // the workspace for the dK/dV kernel, which runs after this one.
        float drow;
        {
            vec8 of[NDC];
            load_frags(static_cast<const uint16_t *>(p.o) + head, qi, S, g, of);
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NDC; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)df[c][e], (float)of[c][e], acc);
            drow = acc + __shfl_xor(acc, 32);
            if (qi < S && g == 0) p.rowdot[(int64_t)bh * S + qi] = drow;
        }
        const float c2 = p.scale * kLog2e;

        const int qlast = min(q0 + ROWS - 1, S - 1);
        const int t_first = max(0, q0 - p.win_lo) / BN;
        const int t_last = min(S - 1, qlast + p.win_hi) / BN;
        // the wave's rows (uniform): 32-key blocks are classified per wave
        const int qw0 = q0 + 32 * wave, qw1 = min(qw0 + 31, S - 1);

        Offs o;
        make_offs(o, lane);
        const uint32_t sbase = (uint32_t)(uintptr_t)smem;
        auto issue = [&](int t, int s) {
            const uint32_t st = sbase + s * kDqStage;
            load_tile<kRowSwz, kDqWaves, BN>(kh, t * BN, S, st, wave, lane);
            load_tile<kTrSwz, kDqWaves, BN>(kh, t * BN, S, st + G::TILE_BYTES, wave, lane);
            load_tile<kRowSwz, kDqWaves, BN>(vh, t * BN, S, st + 2 * G::TILE_BYTES, wave, lane);
        };
        // Within a step the next tile's DMA goes in two parts, K and V rows
        // after the barrier and K transposed half-way through the key blocks,
        // so that no wave stalls behind a 48 KiB burst.
        auto issue_k = [&](int t, int s) {
            const uint32_t st = sbase + s * kDqStage;
            load_tile<kRowSwz, kDqWaves, BN>(kh, t * BN, S, st, wave, lane);
            load_tile<kRowSwz, kDqWaves, BN>(vh, t * BN, S, st + 2 * G::TILE_BYTES, wave, lane);
        };
        auto issue_kt = [&](int t, int s) {
            const uint32_t st = sbase + s * kDqStage;
            load_tile<kTrSwz, kDqWaves, BN>(kh, t * BN, S, st + G::TILE_BYTES, wave, lane);
        };

        f32x16 acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
        issue(t_first, 0);
        for (int t = t_first; t <= t_last; ++t) {
            const int s = (t - t_first) & 1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // tile t is in LDS; every wave is done with stage s ^ 1
            if (t < t_last) issue_k(t + 1, s ^ 1);
            const LDS char *kr = smem + s * kDqStage;
            const LDS char *kt = kr + G::TILE_BYTES;
            const LDS char *vr = kr + 2 * G::TILE_BYTES;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                if (sb == NSB / 2 && t < t_last) issue_kt(t + 1, s ^ 1);
                // Per wave (uniform): a key block that none of the wave's rows
                // sees is skipped; one that all of them see in full is not masked.
                const int kb0 = t * BN + 32 * sb, kb1 = min(kb0 + 31, S - 1);
                const bool empty =
                    qw0 >= S || kb0 >= S || kb0 > qw1 + p.win_hi || kb1 < qw0 - p.win_lo;
                if (empty) continue;
                const bool full = qw0 + 32 <= S && kb0 + 32 <= S && kb0 >= qw0 + 31 - p.win_lo &&
                                  kb0 + 31 <= qw0 + p.win_hi;
                f32x16 sa = f32x16{}, da = f32x16{};
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    sa = Elem<T>::mma(read_rows(kr, o, sb, c), qf[c], sa);
                    da = Elem<T>::mma(read_rows(vr, o, sb, c), df[c], da);
                }
                // element e: key t*BN + 32sb + 8(e/4) + 4g + e%4, query qi. A hidden
                // pair's exponent becomes -inf (exp2 gives exactly 0), by selects
                // under one uniform branch, so no exponential sits behind a branch.
                float x[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) x[e] = fmaf(sa[e], c2, -lse2);
                if (!full) mask_block(x, t * BN + 32 * sb + 4 * g, qi - p.win_lo,
                                      min(qi + p.win_hi, S - 1));
                uint32_t dsp[8];
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float d0 = __builtin_amdgcn_exp2f(x[e]) * (da[e] - drow);
                    const float d1 = __builtin_amdgcn_exp2f(x[e + 1]) * (da[e + 1] - drow);
                    dsp[e >> 1] = Elem<T>::pack(d0, d1);
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        acc[db] = Elem<T>::mma(read_tr(kt, o, db, 2 * sb + hh), half_of(dsp, hh),
                                               acc[db]);
            }
        }
        if (qi < S)
            store_rows(static_cast<uint16_t *>(p.dq) + head, qi, g, acc, p.scale);
    }

    // ---- dK, dV -----------------------------------------------------------------
    // LDS: the V rows of the workgroup's keys (row swizzle; the B operand of
    // dP = dO V^T is read from there, which keeps the wave under 256
    // registers), then per stage: Q rows, Q (transposed), dO rows, dO
    // (transposed), and the tile's LSE * log2(e) and D_i (32 floats each).
    static constexpr int QB = GQ::BN;  // query rows per streamed tile
    static constexpr uint32_t kKvV = 32 * kKvWaves * GQ::RB;
    static constexpr uint32_t kKvStage = 4 * GQ::TILE_BYTES + 2 * QB * 4;

    // The workgroup's items from its work list, as in dq; level l is key
    // tile ntk - 1 - l (under causal masks the first keys see the most rows).
    static __device__ void dkdv(const BwdParams &p, LDS char *smem) {
        const int ntk = (p.S + kBwdRows - 1) / kBwdRows;
        for (int r = 0;; ++r) {
            int x, bh, l;
            const int pos = list_pos(p.kv_plan, r, x);
            if (!list_item(p.kv_plan, x, pos, bh, l)) break;
            if (r) __syncthreads();
            dkdv_item(p, smem, __builtin_amdgcn_readfirstlane(bh),
                      __builtin_amdgcn_readfirstlane(ntk - 1 - l));
        }
    }
    static __device__ __forceinline__ void dkdv_item(const BwdParams &p, LDS char *smem, int bh,
                                                     int kt) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int l32 = lane & 31, g = lane >> 5;
        const int S = p.S;
        constexpr int ROWS = 32 * kKvWaves;
        const int k0 = kt * ROWS, kj = k0 + 32 * wave + l32;
        const int64_t head = (int64_t)bh * S * D;
        const uint16_t *qh = static_cast<const uint16_t *>(p.q) + head;
        const uint16_t *kh = static_cast<const uint16_t *>(p.k) + head;
        const uint16_t *vh = static_cast<const uint16_t *>(p.v) + head;
        const uint16_t *doh = static_cast<const uint16_t *>(p.dout) + head;
        const float *lse_h = p.lse + (int64_t)bh * S;
        const float *dot_h = p.rowdot + (int64_t)bh * S;

        vec8 kf[NDC];
        load_frags(kh, kj, S, g, kf);
        const float c2 = p.scale * kLog2e;

        // rows that see any of the workgroup's keys: j - win_hi <= i <= j + win_lo
        const int klast = min(k0 + ROWS - 1, S - 1);
        const int u_first = max(0, k0 - p.win_hi) / QB;
        const int u_last = min(S - 1, klast + p.win_lo) / QB;
        // query tiles that see every key of the workgroup
        const int u_in_lo = (max(0, klast - p.win_hi) + QB - 1) / QB;
        const int u_in_hi = (min(S - 1, k0 + p.win_lo) + 1) / QB;
        const bool keys_in = k0 + ROWS <= S;

        Offs o;
        make_offs(o, lane);
        const uint32_t sbase = (uint32_t)(uintptr_t)smem;
        const LDS char *vw = smem + wave * 32 * GQ::RB;  // this wave's V rows
        auto issue = [&](int u, int s) {
            const uint32_t st = sbase + kKvV + s * kKvStage;
            load_tile<kRowSwz, kKvWaves, QB>(qh, u * QB, S, st, wave, lane);
            load_tile<kTrSwz, kKvWaves, QB>(qh, u * QB, S, st + GQ::TILE_BYTES, wave, lane);
            load_tile<kRowSwz, kKvWaves, QB>(doh, u * QB, S, st + 2 * GQ::TILE_BYTES, wave, lane);
            load_tile<kTrSwz, kKvWaves, QB>(doh, u * QB, S, st + 3 * GQ::TILE_BYTES, wave, lane);
        };
        // Within a step the next tile's DMA goes in two halves, Q after the
        // barrier and dO after the S and dP products: issued at once by every
        // wave, the 32 KiB queue up and stall the issuing waves.
        auto issue_q = [&](int u, int s) {
            const uint32_t st = sbase + kKvV + s * kKvStage;
            load_tile<kRowSwz, kKvWaves, QB>(qh, u * QB, S, st, wave, lane);
            load_tile<kTrSwz, kKvWaves, QB>(qh, u * QB, S, st + GQ::TILE_BYTES, wave, lane);
        };
        auto issue_do = [&](int u, int s) {
            const uint32_t st = sbase + kKvV + s * kKvStage;
            load_tile<kRowSwz, kKvWaves, QB>(doh, u * QB, S, st + 2 * GQ::TILE_BYTES, wave, lane);
            load_tile<kTrSwz, kKvWaves, QB>(doh, u * QB, S, st + 3 * GQ::TILE_BYTES, wave, lane);
        };
        // the tile's LSE (base 2) and D_i: fetched by the first QB threads,
        // stored into the stage's arrays once they arrive
        auto fetch_vec = [&](int u, float &l2, float &dr) {
            const int i = u * QB + (int)threadIdx.x;
            l2 = i < S ? lse_h[i] * kLog2e : 0.0f;
            dr = i < S ? -dot_h[i] : 0.0f;
        };
        auto put_vec = [&](int s, float l2, float dr) {
            LDS float *v =
                reinterpret_cast<LDS float *>(smem + kKvV + s * kKvStage + 4 * GQ::TILE_BYTES);
            v[threadIdx.x] = l2;
            v[QB + threadIdx.x] = dr;
        };

        f32x16 dva[NDB], dka[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dva[db] = dka[db] = f32x16{};
        load_tile<kRowSwz, kKvWaves, ROWS>(vh, k0, S, sbase, wave, lane);
        issue(u_first, 0);
        if (threadIdx.x < QB) {
            float l2, dr;
            fetch_vec(u_first, l2, dr);
            put_vec(0, l2, dr);
        }
        for (int u = u_first; u <= u_last; ++u) {
            const int s = (u - u_first) & 1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // tile u and its vectors are in LDS; stage s ^ 1 is free
            float nl2 = 0.0f, ndr = 0.0f;
            const bool more = u < u_last;
            if (more) {
                issue_q(u + 1, s ^ 1);
                if (threadIdx.x < QB) fetch_vec(u + 1, nl2, ndr);
            }
            const LDS char *qr = smem + kKvV + s * kKvStage;
            const LDS char *qtr = qr + GQ::TILE_BYTES;
            const LDS char *dor = qr + 2 * GQ::TILE_BYTES;
            const LDS char *dotr = qr + 3 * GQ::TILE_BYTES;
            const LDS float *vl = reinterpret_cast<const LDS float *>(qr + 4 * GQ::TILE_BYTES);
            const bool full = u >= u_in_lo && u < u_in_hi && (u + 1) * QB <= S && keys_in;
            f32x16 sa = f32x16{}, da;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 d4 = *reinterpret_cast<const LDS f32x4 *>(vl + QB + 8 * a + 4 * g);
#pragma unroll
                for (int w = 0; w < 4; ++w) da[4 * a + w] = d4[w];
            }
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                sa = Elem<T>::mma(read_rows(qr, o, 0, c), kf[c], sa);
                da = Elem<T>::mma(read_rows(dor, o, 0, c), read_rows(vw, o, 0, c), da);
            }
            if (more) issue_do(u + 1, s ^ 1);
            // element e: query u*QB + 8(e/4) + 4g + e%4, key kj. Hidden pairs:
            // exponent -inf by selects under one uniform branch, as in dq.
            float x[16];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 l4 = *reinterpret_cast<const LDS f32x4 *>(vl + 8 * a + 4 * g);
#pragma unroll
                for (int w = 0; w < 4; ++w) x[4 * a + w] = fmaf(sa[4 * a + w], c2, -l4[w]);
            }
            if (!full) mask_block(x, u * QB + 4 * g, kj - p.win_hi,
                                  kj < S ? min(kj + p.win_lo, S - 1) : -1);
            uint32_t pp[8], dsp[8];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float pr[4], ds[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pr[w] = __builtin_amdgcn_exp2f(x[4 * a + w]);
                    ds[w] = pr[w] * da[4 * a + w];
                }
                pp[2 * a] = Elem<T>::pack(pr[0], pr[1]);
                pp[2 * a + 1] = Elem<T>::pack(pr[2], pr[3]);
                dsp[2 * a] = Elem<T>::pack(ds[0], ds[1]);
                dsp[2 * a + 1] = Elem<T>::pack(ds[2], ds[3]);
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dva[db] =
                        Elem<T>::mma(read_tr(dotr, o, db, hh), half_of(pp, hh), dva[db]);
                    dka[db] =
                        Elem<T>::mma(read_tr(qtr, o, db, hh), half_of(dsp, hh), dka[db]);
                }
            if (more && threadIdx.x < QB) put_vec(s ^ 1, nl2, ndr);
        }
        if (kj < S) {
            store_rows(static_cast<uint16_t *>(p.dv) + head, kj, g, dva, 1.0f);
            store_rows(static_cast<uint16_t *>(p.dk) + head, kj, g, dka, p.scale);
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(64 * kDqWaves, 1) void fa_bwd_dq_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * Bwd<T, D>::kDqStage];
    Bwd<T, D>::dq(p, (LDS char *)smem);
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kKvWaves, 1) void fa_bwd_dkdv_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[Bwd<T, D>::kKvV + 2 * Bwd<T, D>::kKvStage];
    Bwd<T, D>::dkdv(p, (LDS char *)smem);
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdParams &p, hipStream_t stream) {
    void *args[] = {const_cast<BwdParams *>(&p)};
    // dQ first: it also writes the row dots D_i that dK/dV reads.
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_dq_kernel<T, D>),
                                   dim3((unsigned)p.dq_plan.grid), dim3(64 * kDqWaves), args, 0,
                                   stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_dkdv_kernel<T, D>),
                           dim3((unsigned)p.kv_plan.grid), dim3(64 * kKvWaves), args, 0, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams &p, int D, int dtype, hipStream_t stream) {
    if (D == 128) return dtype == 0 ? launch_bwd_t<_Float16, 128>(p, stream)
                                    : launch_bwd_t<__bf16, 128>(p, stream);
    if (D == 64) return dtype == 0 ? launch_bwd_t<_Float16, 64>(p, stream)
                                   : launch_bwd_t<__bf16, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
