// fa_decode.hip -- attention of a few new query rows against a key/value cache
// (incremental decoding) for gfx950 (MI355X): fp16/bf16 in, fp32 accumulate,
// D in {64, 128}, 1 .. 32 query rows.
//
// What it computes: for query row i (position Sk - Sq + i of its sequence,
// the cache holding positions 0 .. Sk-1, the row's own key included),
// O_i = softmax_j(scale * q_i . k_j + mask_ij) V and its LSE: the KV-cache
// section of "FlashAttention on Ascend NPU: from principle to practice"
// (hwcomputing.csdn.net, 6a0fe629), "optimisation 4: KV-cache reuse", read as
// attention of each new row over every visible cached key (the code printed
// there attends to the last key only). The mask rules are those of the
// forward kernel, applied at each row's position.
//
// gfx950 design:
//  * The work is reading the cache (HBM-bound: each cached key is used by at
//    most 32 rows). The visible key range of every head is cut into splits of
//    consecutive 32-key tiles; one workgroup = one wave handles one split of
//    one head, so B*H*nsplit workgroups keep every CU streaming.
//  * Each wave streams its tiles HBM -> LDS with the same direct DMA as the
//    forward kernel (buffer_load_dwordx4 ... lds), through a ring of four
//    (K, V) stages: three tiles are always in flight. The wave is alone in
//    its workgroup, so a vmcnt wait orders each tile; no barrier is needed.
//  * Per tile the wave computes S^T = K Q^T (v_mfma_f32_32x32x16, the query
//    rows padded to 32 with zero rows) and O^T += V^T P^T exactly as the
//    forward kernel does (lane = query row, V^T from the transposing LDS
//    read), with the same online softmax and lazy rescale.
//  * Each split ends with its normalised partial output and its LSE; a merge
//    kernel combines the splits of a row: LSE = log sum_s e^LSE_s and
//    O = sum_s e^(LSE_s - LSE) O_s. With one split the wave writes O and LSE
//    itself.
//  * Paged cache: the keys of a sequence live in fixed-size pages of a pool
//    [num_pages, page_size, H, D] named by a per-sequence block table, each
//    sequence with its own length (both device arrays). A 32-key tile lies in
//    one page, so only the tile's base address and row stride change; a page
//    index outside the pool gets an empty buffer resource (its keys read as
//    zero, nothing outside the pool is touched). Splits are laid over each
//    sequence's own visible tiles; a split with none left reports no keys
//    (LSE -inf), which the merge weighs zero.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Split partials of fa_decode_noalloc: one copy of this array per GPU. Host
// code never passes its name to a kernel (on the host it names a stand-in, not
// device memory); it uses the address decode_scratch() looks up.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *a = nullptr;
        err = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));  // with `dev` current
        if (err != hipSuccess) return err;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

using namespace dev;

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int wait_vmcnt(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <int D> struct DGeom {
    static constexpr int BN = kDecodeBN;           // keys per tile
    static constexpr int RB = 2 * D;               // bytes per K/V row
    static constexpr int CPR = RB / 16;            // 16-byte chunks per row
    static constexpr int TILE_BYTES = BN * RB;     // one K or V tile: 8 KiB (D=128), 4 KiB (D=64)
    static constexpr int ROWS_PER_KB = 1024 / RB;  // rows per 1 KiB DMA block
    static constexpr int NBLK = TILE_BYTES / 1024; // DMA blocks per K or V tile
    static constexpr int NSTAGE = 4;               // ring of (K, V) stages
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
    static constexpr int OPS_PER_TILE = 2 * NBLK;  // DMA instructions per (K, V) tile
    static_assert((NSTAGE - 1) * OPS_PER_TILE <= 63, "vmcnt range");
};

template <typename T, int D>
struct Decode {
    typedef DGeom<D> G;
    typedef typename Elem<T>::vec8 vec8;
    static constexpr int BN = G::BN;
    static constexpr int NDC = D / 16;  // 16-dim chunks of the QK^T contraction
    static constexpr int NDB = D / 32;  // 32-dim output blocks
    static constexpr int NPC = BN / 16; // 16-key chunks of the PV contraction
    // Largest growth of a row maximum absorbed without rescaling (as in the
    // forward kernel: probabilities up to 2^8 relative to a stale maximum).
    static constexpr float kRescaleSlack = 8.0f;

    // Wait until tile i's DMA has landed; the DMA of the tiles after it (at
    // most NSTAGE - 1 of them, fewer near the end) may stay in flight.
    static __device__ __forceinline__ void wait_tile(int later) {
        switch (later) {
        case 0: __builtin_amdgcn_s_waitcnt(wait_vmcnt(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(wait_vmcnt(1 * G::OPS_PER_TILE)); break;
        case 2: __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * G::OPS_PER_TILE)); break;
        default: __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * G::OPS_PER_TILE)); break;
        }
    }

    static __device__ void run(const DecodeParams &p, LDS char *smem) {
        static_assert(G::NSTAGE == 4, "wait_tile covers three later tiles");
        const int lane = threadIdx.x;  // the workgroup is one wave
        const int l32 = lane & 31, g = lane >> 5;
        const int ns = p.nsplit;
        const int bh = blockIdx.x / ns, sp = blockIdx.x - bh * ns;
        const int bb = bh / p.H, hh = bh - bb * p.H;
        const bool paged = p.block_table != nullptr;
        // This sequence's cached keys and the tiles its rows can see (row i at
        // position S - Sq + i); this split's share of them (possibly none).
        const int S = paged ? min(max(__builtin_amdgcn_readfirstlane(p.seq_lens[bb]), 0), p.Sk)
                            : p.Sk;
        const int Sq = p.Sq;
        const int win_lo = p.win_lo, win_hi = p.win_hi;
        const int pos_first = S - Sq, pos_last = S - 1;
        const int key_lo = max(0, pos_first - win_lo);
        const int key_hi = min(S - 1, pos_last + win_hi);
        const int ta = key_lo / BN + sp * p.tiles_per_split;
        const int nt = key_hi < key_lo ? 0 : min(ta + p.tiles_per_split, key_hi / BN + 1) - ta;
        const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
        // Bytes between consecutive keys of one head: a contiguous [B, H, Sk, D]
        // cache has them adjacent, a page pool interleaves the heads.
        const uint32_t rs = paged ? (uint32_t)p.H * G::RB : (uint32_t)G::RB;

        // DMA: 1 KiB block b of a tile holds rows b * ROWS_PER_KB + lane / CPR;
        // lane L lands in physical chunk L % CPR and so fetches the logical
        // chunk the swizzle stores there (XOR swizzles are their own inverse).
        uint32_t kdma[G::NBLK], vdma[G::NBLK];
        {
            const int pc = lane % G::CPR;
#pragma unroll
            for (int b = 0; b < G::NBLK; ++b) {
                const int row = b * G::ROWS_PER_KB + lane / G::CPR;
                kdma[b] = row * rs + kchunk<D>(pc, row) * 16;
                vdma[b] = row * rs + vchunk<D>(pc, row) * 16;
            }
        }
        auto load = [&](int i) {  // tile ta + i into stage i % NSTAGE
            const int k0 = (ta + i) * BN;
            const int rows = min(BN, S - k0);  // rows past S read as zero
            int64_t first;  // element offset of (key k0, head hh) in k and v
            bool ok = true;
            if (paged) {
                const int page = __builtin_amdgcn_readfirstlane(
                    p.block_table[(int64_t)bb * p.max_pages + k0 / p.page_size]);
                ok = page >= 0 && page < p.num_pages;
                first = (((int64_t)page * p.page_size + k0 % p.page_size) * p.H + hh) * D;
            } else {
                first = ((int64_t)bh * p.Sk + k0) * D;
            }
            const uint32_t bytes = ok ? (uint32_t)(rows - 1) * rs + G::RB : 0u;
            const i32x4 rk = buffer_rsrc(static_cast<const uint16_t *>(p.k) + (ok ? first : 0), bytes);
            const i32x4 rv = buffer_rsrc(static_cast<const uint16_t *>(p.v) + (ok ? first : 0), bytes);
            const uint32_t base = smem_addr + (uint32_t)((i % G::NSTAGE) * G::STAGE_BYTES);
#pragma unroll
            for (int b = 0; b < G::NBLK; ++b) dma16(rk, base + (uint32_t)b * 1024u, kdma[b]);
#pragma unroll
            for (int b = 0; b < G::NBLK; ++b)
                dma16(rv, base + (uint32_t)(G::TILE_BYTES + b * 1024), vdma[b]);
        };
#pragma unroll
        for (int i = 0; i < G::NSTAGE - 1; ++i)
            if (i < nt) load(i);

        // Operand offsets within a stage. K (A operand) of chunk c: row l32,
        // logical chunk 2c + g. V^T (A operand, transposing read) of block db:
        // the 16-lane group G16 = lane / 16 (g = G16 / 2, h = G16 % 2) reads
        // rows 4g + (lane % 16) / 4 (+ 16c, + 8), columns 32db + 16h + 4(lane % 4).
        uint32_t ko[NDC], vo[NDB];
#pragma unroll
        for (int c = 0; c < NDC; ++c) ko[c] = l32 * G::RB + kchunk<D>(2 * c + g, l32) * 16;
        {
            const int q = lane & 15, h = (lane >> 4) & 1;
            const int vrow = 4 * g + (q >> 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int col = 32 * db + 16 * h + 4 * (q & 3);
                vo[db] = G::TILE_BYTES + vrow * G::RB + vchunk<D>(col >> 3, vrow) * 16 +
                         (col & 7) * 2;
            }
        }

        // Q^T fragments (B operand): query row l32, dims 16c + 8g .. +7; rows
        // past Sq lie outside the buffer resource and read as zero.
        vec8 qf[NDC];
        {
            const uint16_t *qh = static_cast<const uint16_t *>(p.q) + (int64_t)bh * Sq * D;
            const __amdgpu_buffer_rsrc_t qr =
                __builtin_amdgcn_make_buffer_rsrc((void *)qh, 0, (uint32_t)Sq * G::RB, kBufferFlags);
            const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                u32x4 x = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               qr, (uint32_t)l32 * G::RB + (16 * c + 8 * g) * 2, 0, 0));
                x ^= flip;
                qf[c] = __builtin_bit_cast(vec8, x);
            }
            if (p.rope_cos) {  // rotary embedding of the row at its position
                const int64_t at = (int64_t)min(max(pos_first + l32, 0), p.Sk - 1) * (D / 2);
                rope_fragments<T, D>(qf, g, p.rope_cos + at, p.rope_sin + at,
                                     p.rope_interleaved != 0);
            }
        }

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        float m_run = -INFINITY, l_run = 0.0f;
        const float c2 = p.c2;
        const int pos = pos_first + l32;  // this lane's query position

        for (int i = 0; i < nt; ++i) {
            if (i + G::NSTAGE - 1 < nt) load(i + G::NSTAGE - 1);  // into the stage tile i - 1 used
            wait_tile(min(G::NSTAGE - 1, nt - 1 - i));
            const LDS char *st = smem + (i % G::NSTAGE) * G::STAGE_BYTES;

            // S^T = K Q^T for the 32 keys of the tile.
            f32x16 sacc = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                const vec8 a = *reinterpret_cast<const LDS vec8 *>(st + ko[c]);
                sacc = Elem<T>::mma(a, qf[c], sacc);
            }

            // Mask: element r holds key k0 + 8(r/4) + 4g + r%4 for this lane's
            // row. A tile visible in full from every valid row skips it.
            const int k0 = (ta + i) * BN;
            const bool full = k0 + BN - 1 <= S - 1 && k0 + BN - 1 <= pos_first + win_hi &&
                              k0 >= pos_last - win_lo;
            if (!full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool ok = j < S && j <= pos + win_hi && j >= pos - win_lo;
                    sacc[r] = ok ? sacc[r] : -INFINITY;
                }
            }

            // Online softmax (base 2, c2 > 0) with the lazy rescale.
            float smax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[r]);
            smax = max_with_partner(smax);
            const float m_tile = (smax == -INFINITY) ? -INFINITY : smax * c2;
            if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack)) {
                const float m_new = fmaxf(m_run, m_tile);
                const float alpha =
                    (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            }
            const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
            // bf16 keeps only 8 significant bits of each probability, which
            // moves a short row's output by up to about one bf16 unit before
            // its own rounding. The cache kernel is bound by HBM, not by the
            // matrix cores, so for bf16 it also feeds the rounding remainder
            // p - bf16(p) (itself rounded, 16 bits in all) through a second
            // product with the same V^T operand.
            constexpr bool kSplitP = Elem<T>::kCoarse;
            uint32_t pk[8], pr[8] = {};
            float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, -mu));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], c2, -mu));
                pk[r >> 1] = Elem<T>::pack(p0, p1);
                if constexpr (kSplitP) {
                    const float h0 = __builtin_bit_cast(float, pk[r >> 1] << 16);
                    const float h1 = __builtin_bit_cast(float, pk[r >> 1] & 0xffff0000u);
                    pr[r >> 1] = Elem<T>::pack(p0 - h0, p1 - h1);
                }
                if (Elem<T>::kSumRounded) {
                    ps0 = Elem<T>::sum2(pk[r >> 1], ps0);
                } else {
                    ps0 += p0;
                    ps1 += p1;
                }
            }
            l_run += ps0 + ps1;

            // O^T += V^T P^T: chunk c's B operand is P^T elements 8c .. 8c+7
            // (keys 16c + 8a + 4g + b for element 4a + b); the A operand comes
            // from two transposing reads, rows 16c + 4g + (0..3) and
            // 16c + 8 + 4g + (0..3).
#pragma unroll
            for (int c = 0; c < NPC; ++c) {
                const u32x4 pw = {pk[4 * c + 0], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
                const vec8 b = __builtin_bit_cast(vec8, pw);
                vec8 br{};
                if constexpr (kSplitP)
                    br = __builtin_bit_cast(vec8, u32x4{pr[4 * c + 0], pr[4 * c + 1],
                                                        pr[4 * c + 2], pr[4 * c + 3]});
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const LDS char *base = st + vo[db] + 16 * c * G::RB;
                    const fp16x4_t lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS fp16x4_t *)(base));
                    const fp16x4_t hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS fp16x4_t *)(base + 8 * G::RB));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    const vec8 a = __builtin_bit_cast(vec8, u32x4{l2[0], l2[1], h2[0], h2[1]});
                    oacc[db] = Elem<T>::mma(a, b, oacc[db]);
                    if constexpr (kSplitP) oacc[db] = Elem<T>::mma(a, br, oacc[db]);
                }
            }
            // Every LDS read of this stage has returned (the MFMAs consumed
            // them) before the stage is refilled at the next iteration's DMA.
            pin(oacc);
            conservative_lds_wait();
        }

        // ---- this split's result -------------------------------------------
        const float l_tot = sum_with_partner(l_run);
        if (l32 >= Sq) return;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const float lse = l_tot > 0.0f ? 0.69314718055994531f * (m_run + __log2f(l_tot)) : -INFINITY;
        const int64_t row = (int64_t)bh * Sq + l32;
        if (ns == 1) {
            uint16_t *orow = static_cast<uint16_t *>(p.o) + row * D;
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
            if (p.lse && g == 0) p.lse[row] = lse;
        } else {
            const int64_t prow = ((int64_t)bh * ns + sp) * Sq + l32;
            float *orow = p.ws_o + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 w = {oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv,
                                      oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
                    *reinterpret_cast<float4 *>(orow + 32 * db + 8 * a + 4 * g) = w;
                }
            if (g == 0) p.ws_lse[prow] = lse;
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(64) void fa_decode_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[DGeom<D>::NSTAGE * DGeom<D>::STAGE_BYTES];
    Decode<T, D>::run(p, (LDS char *)smem);
}

// One row (b, h, i) per workgroup, one output dimension per thread:
// LSE = M + log sum_s e^(LSE_s - M) with M = max_s LSE_s, and
// O = sum_s e^(LSE_s - M) O_s / sum_s e^(LSE_s - M). A row no split saw
// (impossible for the supported masks) gets O = 0, LSE = -inf.
template <typename T, int D>
__global__ __launch_bounds__(D) void fa_decode_merge_kernel(DecodeParams p) {
    const int d = threadIdx.x;
    const int row = blockIdx.x;  // (b*H + h) * Sq + i
    const int Sq = p.Sq, ns = p.nsplit;
    const int bh = row / Sq, i = row - bh * Sq;
    const float *ls = p.ws_lse + (int64_t)bh * ns * Sq + i;  // split s at ls[s * Sq]
    const float *os = p.ws_o + ((int64_t)bh * ns * Sq + i) * D + d;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ls[(int64_t)s * Sq]);
    float wsum = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float w = __expf(ls[(int64_t)s * Sq] - M);  // e^-inf = 0
            wsum += w;
            acc += w * os[(int64_t)s * Sq * D];
        }
    }
    const float out = wsum > 0.0f ? acc / wsum : 0.0f;
    const T ot = (T)out;
    static_cast<uint16_t *>(p.o)[(int64_t)row * D + d] = __builtin_bit_cast(uint16_t, ot);
    if (p.lse && d == 0) p.lse[row] = wsum > 0.0f ? M + __logf(wsum) : -INFINITY;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t stream) {
    void *args[] = {const_cast<DecodeParams *>(&p)};
    const unsigned grid = (unsigned)p.B * (unsigned)p.H * (unsigned)p.nsplit;
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&fa_decode_kernel<T, D>),
                                     dim3(grid), dim3(64), args, 0, stream);
    if (err != hipSuccess || p.nsplit == 1) return err;
    const unsigned rows = (unsigned)p.B * (unsigned)p.H * (unsigned)p.Sq;
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_decode_merge_kernel<T, D>),
                           dim3(rows), dim3(D), args, 0, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int D, int dtype, hipStream_t stream) {
    if (D == 128) return dtype == 0 ? launch_decode_t<_Float16, 128>(p, stream)
                                    : launch_decode_t<__bf16, 128>(p, stream);
    if (D == 64) return dtype == 0 ? launch_decode_t<_Float16, 64>(p, stream)
                                   : launch_decode_t<__bf16, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
