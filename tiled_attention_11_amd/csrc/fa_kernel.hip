// fa_kernel.hip -- fused attention forward for gfx950 (MI355X), fp16/bf16 in,
// fp32 accumulate, D in {64, 128}.
//
// What it computes: O = softmax(scale * Q K^T + mask) V and the row LSE, with
// the online-softmax recurrence of the Ascend C FlashAttention-2 tile-fusion
// page (ascendai.csdn.net), section 1.2: a running row maximum m and row sum l,
// an unnormalised accumulator rescaled by exp(m_old - m_new) whenever m grows,
// and one division by l at the end. Tiling Q into row blocks and streaming
// K/V column blocks follows section 3 of that page and the ops-transformer
// walkthrough (hwcomputing.csdn.net, 6a0ef689), "core idea: tiling + online
// softmax"; skipping key blocks that the mask hides entirely follows section 6
// of the tile-fusion page; the window mask follows the catlass article
// (lnwmold.com/news/1200460), section "usage".
//
// gfx950 design (not the pages' Ascend design):
//  * One workgroup = 4 waves of 64 lanes = 128 query rows of one (b, h);
//    each wave owns 32 query rows for the whole key loop.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16
//    (A = 32 keys x 16 dims, B = 16 dims x 32 queries). In the accumulator
//    layout lane l then holds query (l % 32) and 16 keys, so the row max and
//    row sum are in-lane reductions plus one exchange with lane l ^ 32, and
//    the per-row rescale of the output is a per-lane scalar.
//  * The output is accumulated transposed as well, O^T += V^T P^T: P^T comes
//    straight out of the score accumulator (rounded to fp16/bf16) as the B
//    operand, and V^T is the A operand, read from a transposed copy of the V
//    tile in LDS.
//  * K and V^T tiles are double-buffered in LDS: global loads of tile t+1 are
//    issued before tile t is computed and written to the other buffer after,
//    with one workgroup barrier per tile.
//  * Key tiles that the mask hides from all 128 rows are never loaded; per
//    wave, tiles hidden from its 32 rows are skipped, tiles fully visible run
//    without any mask arithmetic, and only boundary tiles evaluate the
//    per-element predicate.
//  * The flat workgroup index is remapped so that all query tiles of a head
//    land on one XCD (workgroups are dealt round-robin over the 8 XCDs) and
//    run heaviest-first (longest causal rows first).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = 32;  // query rows per wave
static_assert(kWaves * kWaveRows == kBlockM, "workgroup covers kBlockM rows");

// ---- element type traits --------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<_Float16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // two fp32 -> two fp16, round to nearest even, packed low|high
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        f16x2 h = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
};
template <> struct Elem<__bf16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        bf16x2 h = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
};

// ---- tile geometry per head dimension ---------------------------------------
// D = 128: 64-key tiles; D = 64: 128-key tiles. Both give 32 MFMAs per wave per
// tile and 35 KiB of LDS per stage.
template <int D> struct Geom {
    static constexpr int BN = (D == 128) ? 64 : 128;  // keys per tile
    static constexpr int KS = D + 8;    // K tile row stride in elements (16 B pad)
    static constexpr int VS = BN + 8;   // V^T tile row stride in elements (16 B pad)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;   // elements per LDS stage
    static constexpr int TPR = D / 8;                // threads per 16-byte-chunked row
    static constexpr int KPT = BN * TPR / kThreads;  // keys each thread stages
    static_assert(KPT == 4, "staging assumes 4 keys per thread");
    static_assert((BN / 8) % 8 == 0, "V^T chunk swizzle needs 8-chunk groups");
};

// V^T rows hold the tile's keys in a permuted order: inside each group of 16
// keys, key 8a + 4g + b (a, g in {0,1}, b in 0..3) sits at 8g + 4a + b. That
// is the order in which lane group g = lane / 32 of a 32x32 score accumulator
// holds its keys, so each lane's 8-key slice of P^T is one contiguous 16-byte
// LDS read of V^T. In units of 4-key groups this swaps bits 0 and 1.
__device__ __forceinline__ int vt_group_pos(int kg) {
    return (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
}
// 16-byte chunk swizzle of V^T rows: chunk c of row d lives at c ^ ((d >> 3) & 7),
// so the 8-row-apart transposed writes hit different banks.
__device__ __forceinline__ int vt_chunk(int chunk, int d) { return chunk ^ ((d >> 3) & 7); }

template <typename T, int D>
struct Kernel {
    typedef Geom<D> G;
    typedef typename Elem<T>::vec8 vec8;
    static constexpr int BN = G::BN;
    static constexpr int NKB = BN / 32;   // 32-key score blocks per tile
    static constexpr int NDC = D / 16;    // 16-dim chunks of the QK^T contraction
    static constexpr int NDB = D / 32;    // 32-dim output blocks
    static constexpr int NPC = BN / 16;   // 16-key chunks of the PV contraction

    // Global -> registers: thread t stages keys 4*(t / TPR) + i, i = 0..3, at
    // dims 8*(t % TPR) .. +7 of both K and V. Rows past S read as zero.
    static __device__ __forceinline__ void load_tile(const uint16_t *kh, const uint16_t *vh,
                                                     int k0, int S, u32x4 (&kr)[4],
                                                     u32x4 (&vr)[4]) {
        const int t = threadIdx.x;
        const int kg = t / G::TPR, dc = t % G::TPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = k0 + 4 * kg + i;
            if (key < S) {
                const int64_t off = (int64_t)key * D + 8 * dc;
                kr[i] = *reinterpret_cast<const u32x4 *>(kh + off);
                vr[i] = *reinterpret_cast<const u32x4 *>(vh + off);
            } else {
                kr[i] = u32x4{0, 0, 0, 0};
                vr[i] = u32x4{0, 0, 0, 0};
            }
        }
    }

    // Registers -> LDS stage: K row-major (16-byte writes); V transposed, 4 keys
    // of one dim per 8-byte write, keys permuted and chunks swizzled as above.
    static __device__ __forceinline__ void store_tile(uint16_t *stage, const u32x4 (&kr)[4],
                                                      const u32x4 (&vr)[4]) {
        const int t = threadIdx.x;
        const int kg = t / G::TPR, dc = t % G::TPR;
        uint16_t *ks = stage;
        uint16_t *vt = stage + G::K_ELEMS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(ks + (4 * kg + i) * G::KS + 8 * dc) = kr[i];
        const int pos = 4 * vt_group_pos(kg);  // first of the 4 key slots
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * dc + e;
            const int w = e >> 1;
            uint32_t a0 = vr[0][w], a1 = vr[1][w], a2 = vr[2][w], a3 = vr[3][w];
            u32x2 out;
            if (e & 1) {
                out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
            } else {
                out[0] = (a0 & 0xffffu) | (a1 << 16);
                out[1] = (a2 & 0xffffu) | (a3 << 16);
            }
            const int col = vt_chunk(pos >> 3, d) * 8 + (pos & 7);
            *reinterpret_cast<u32x2 *>(vt + d * G::VS + col) = out;
        }
    }

    // Map the flat workgroup index to (b*H + h, query tile).
    static __device__ __forceinline__ void tile_of(const FwdParams &p, int wg, int *bh,
                                                   int *qt) {
        const int nq = p.n_qtiles;
        if (p.xcd_remap) {
            const int xcd = wg & 7, slot = wg >> 3;
            const int hl = slot / nq;
            *bh = hl * 8 + xcd;
            *qt = nq - 1 - (slot - hl * nq);
        } else {
            *bh = wg / nq;
            *qt = nq - 1 - (wg - *bh * nq);
        }
    }

    static __device__ void run(const FwdParams &p, uint16_t *smem) {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        const int l32 = lane & 31;
        const int g = lane >> 5;
        const int S = p.S;

        int bh, qt;
        tile_of(p, blockIdx.x, &bh, &qt);
        const int64_t head = (int64_t)bh * S * D;
        const uint16_t *qh = static_cast<const uint16_t *>(p.q) + head;
        const uint16_t *kh = static_cast<const uint16_t *>(p.k) + head;
        const uint16_t *vh = static_cast<const uint16_t *>(p.v) + head;

        const int q0 = qt * kBlockM;
        const int qlast = min(q0 + kBlockM - 1, S - 1);
        // Keys visible from any row of the workgroup, in whole tiles.
        const int klo = max(0, q0 - p.win_lo);
        const int khi = min(S - 1, qlast + p.win_hi);
        const int t_first = klo / BN;
        const int t_last = khi / BN;

        // This wave's rows and their visible key range.
        const int r0 = q0 + wave * kWaveRows;
        const bool wave_live = r0 < S;
        const int rlast = min(r0 + kWaveRows - 1, S - 1);
        const int wklo = max(0, r0 - p.win_lo);
        const int wkhi = min(S - 1, rlast + p.win_hi);

        // Q^T fragments (B operand): lane holds query row r0 + l32, dims
        // 16c + 8g .. +7. Rows past S are zero.
        vec8 qf[NDC];
        {
            const int row = r0 + l32;
            const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                u32x4 x = u32x4{0, 0, 0, 0};
                if (row < S)
                    x = *reinterpret_cast<const u32x4 *>(qh + (int64_t)row * D + 16 * c + 8 * g);
                x ^= flip;
                qf[c] = __builtin_bit_cast(vec8, x);
            }
        }

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        float m_run = -INFINITY;  // running max of base-2 scaled scores
        float l_run = 0.0f;       // this lane's share of the running row sum
        const float c2 = p.c2;
        const int qi = r0 + l32;  // this lane's query row

        u32x4 kr[4], vr[4];
        load_tile(kh, vh, t_first * BN, S, kr, vr);
        store_tile(smem, kr, vr);
        __syncthreads();

        for (int t = t_first; t <= t_last; ++t) {
            uint16_t *stage = smem + ((t - t_first) & 1) * G::STAGE;
            const bool more = t < t_last;
            if (more) load_tile(kh, vh, (t + 1) * BN, S, kr, vr);

            const int k0 = t * BN;
            const bool live = wave_live && k0 <= wkhi && k0 + BN - 1 >= wklo;
            if (live) {
                const bool full = k0 + BN - 1 <= S - 1 && k0 + BN - 1 <= r0 + p.win_hi &&
                                  k0 >= rlast - p.win_lo;
                const uint16_t *ks = stage;
                const uint16_t *vt = stage + G::K_ELEMS;

                // ---- S^T = K Q^T for this tile ----
                f32x16 sacc[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const vec8 a = *reinterpret_cast<const vec8 *>(
                            ks + (32 * kb + l32) * G::KS + 16 * c + 8 * g);
                        sacc[kb] = Elem<T>::mma(a, qf[c], sacc[kb]);
                    }
                }

                // ---- mask (boundary tiles only) ----
                // Accumulator element r of block kb holds key
                // k0 + 32kb + 8(r/4) + 4g + r%4 for query qi.
                uint64_t vis = ~0ull;
                if (!full) {
                    vis = 0;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                            const bool ok = j < S && j <= qi + p.win_hi && j >= qi - p.win_lo;
                            vis |= (uint64_t)ok << (16 * kb + r);
                            if (!ok) sacc[kb][r] = -INFINITY;
                        }
                }

                // ---- online softmax (base 2) ----
                float smax = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
                smax = fmaxf(smax, __shfl_xor(smax, 32));
                // c2 >= 0, so the max of the scaled scores is c2 * max(score).
                const float m_tile = (smax == -INFINITY) ? -INFINITY : smax * c2;
                const float m_new = fmaxf(m_run, m_tile);
                const float mu = (m_new == -INFINITY) ? 0.0f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
                m_run = m_new;

                uint32_t pk[NKB][8];
                float psum = 0.0f;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, -mu));
                        float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], c2, -mu));
                        if (!full) {
                            p0 = ((vis >> (16 * kb + r)) & 1) ? p0 : 0.0f;
                            p1 = ((vis >> (16 * kb + r + 1)) & 1) ? p1 : 0.0f;
                        }
                        psum += p0 + p1;
                        pk[kb][r >> 1] = Elem<T>::pack(p0, p1);
                    }
                l_run = l_run * alpha + psum;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

                // ---- O^T += V^T P^T ----
#pragma unroll
                for (int c = 0; c < NPC; ++c) {
                    const int kb = c >> 1, h = c & 1;
                    const u32x4 pw = {pk[kb][4 * h + 0], pk[kb][4 * h + 1], pk[kb][4 * h + 2],
                                      pk[kb][4 * h + 3]};
                    const vec8 b = __builtin_bit_cast(vec8, pw);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const int d = 32 * db + l32;
                        const vec8 a = *reinterpret_cast<const vec8 *>(
                            vt + d * G::VS + vt_chunk(2 * c + g, d) * 8);
                        oacc[db] = Elem<T>::mma(a, b, oacc[db]);
                    }
                }
            }

            if (more) store_tile(smem + ((t + 1 - t_first) & 1) * G::STAGE, kr, vr);
            __syncthreads();
        }

        // ---- epilogue: O = O_acc / l, LSE = ln 2 * (m + log2 l) ----
        if (!wave_live || qi >= S) return;
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t *orow = static_cast<uint16_t *>(p.o) + head + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // elements 4a .. 4a+3 hold dims 32db + 8a + 4g + 0..3
                u32x2 w;
                w[0] = Elem<T>::pack(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv);
                w[1] = Elem<T>::pack(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * a + 4 * g) = w;
            }
        if (p.lse && g == 0) {
            const float lse = l_tot > 0.0f ? 0.69314718055994531f * (m_run + __log2f(l_tot))
                                           : -INFINITY;
            p.lse[(int64_t)bh * S + qi] = lse;
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(FwdParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Geom<D>::STAGE];
    Kernel<T, D>::run(p, smem);
}

template <typename T, int D>
hipError_t launch_t(const FwdParams &p, hipStream_t stream) {
    const int grid = p.B * p.H * p.n_qtiles;
    void *args[] = {const_cast<FwdParams *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_fwd_kernel<T, D>), dim3(grid),
                           dim3(kThreads), args, 0, stream);
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
