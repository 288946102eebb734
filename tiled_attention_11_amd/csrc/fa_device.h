// fa_device.h -- device-side building blocks shared by the gfx950 attention
// kernels (the prefill forward and the key/value-cache kernels): vector types,
// the fp16/bf16 matrix-core and rounding traits, the LDS swizzles, the direct
// HBM -> LDS DMA and small wave-level helpers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace dev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));

#define LDS __attribute__((address_space(3)))

// Word 3 of a gfx9 buffer resource for raw (untyped, stride 0) access.
constexpr int kBufferFlags = 0x00020000;

// ---- element type traits --------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<_Float16> {
    typedef f16x8 vec8;
    typedef f16x2 vec2;
    // The cache kernel's row sum adds the fp16-rounded probabilities (the
    // P V operands), two per v_dot2 against (1, 1); their rounding (relative
    // 2^-12 at most) moves the LSE by under 2.5e-4. (The prefill forward sums
    // the unrounded fp32 probabilities for both types.)
    static constexpr bool kSumRounded = true;
    // 8 significant bits: the cache kernel feeds P to its product in two parts.
    static constexpr bool kCoarse = false;
    // acc + a.lo + a.hi for two packed fp16 values
    static __device__ __forceinline__ float sum2(uint32_t a, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), one, acc, false);
    }
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // two fp32 -> two fp16, round to nearest even, packed low|high
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        vec2 h = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
};
template <> struct Elem<__bf16> {
    typedef bf16x8 vec8;
    typedef bf16x2 vec2;
    // bf16 rounding (relative 2^-9) would move the LSE by up to 2e-3: the row
    // sum adds the unrounded fp32 probabilities instead.
    static constexpr bool kSumRounded = false;
    static constexpr bool kCoarse = true;
    static __device__ __forceinline__ float sum2(uint32_t, float acc) { return acc; }
    static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        vec2 h = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
};

// ---- LDS swizzles ----------------------------------------------------------
// Physical 16-byte chunk of logical chunk q in row r of a K (or Q) tile with
// head dimension D: the 16 rows read together by one 16-lane group land on 16
// different 4-bank groups.
template <int D> __device__ __forceinline__ int kchunk(int q, int r) {
    return D == 128 ? (q ^ (r & 15)) : (q ^ ((r >> 1) & 7));
}
// Physical chunk of logical chunk q in row r of a V tile: the 4 rows x 64
// bytes read by 32 lanes of a transposing load land in 4 different 64-byte
// segments.
template <int D> __device__ __forceinline__ int vchunk(int q, int r) {
    return D == 128 ? (q ^ ((r & 3) << 2)) : (q ^ (((r >> 1) & 1) << 2));
}

// ---- conservative synchronisation (a checking build) ----------------------------
// Compiled with FA_CONSERVATIVE_SYNC=1 the kernels wait for every DMA right
// after issuing it (vmcnt 0), wait for every LDS read at the end of every phase
// (lgkmcnt 0) and put a fenced workgroup barrier between the two halves of
// every step of the forward's key loop. The arithmetic is unchanged, so that
// build must give bit-identical results: a test compares it with the release
// build, which orders its DMA and LDS traffic by hand.
#ifndef FA_CONSERVATIVE_SYNC
#define FA_CONSERVATIVE_SYNC 0
#endif
constexpr bool kConservativeSync = FA_CONSERVATIVE_SYNC != 0;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait for all vector-memory operations, or for all LDS ones.
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (3 << 14);

__device__ __forceinline__ void conservative_lds_wait() {
    if constexpr (kConservativeSync) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        asm volatile("" ::: "memory");
    }
}

// ---- HBM -> LDS DMA ---------------------------------------------------------
// Raw buffer resource (base, num_records bytes, stride 0) as 4 SGPRs.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes,
                 kBufferFlags};
}

// 16 bytes per lane from the buffer at voffset straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds; offsets outside the
// resource read as zero). Issued from inline assembly so that the compiler
// does not guard every later LDS read with a wait for this load: the
// kernel orders DMA and LDS reads itself (vmcnt wait + barrier per tile).
// M0 carries the LDS base and is restored, with the one wait state the
// hardware needs between an SALU write of M0 and its use by the load.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voffset), "s"(rsrc)
        : "memory");
    if constexpr (kConservativeSync) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("" ::: "memory");
    }
}

// ---- wave-level helpers ------------------------------------------------------
// Materialise a value here: the compiler may not move its computation past
// this point (it would otherwise sink the softmax of one phase into the
// next, or the MFMAs of one phase past the barrier that ends it).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x16 &x) { asm volatile("" : "+v"(x)); }
template <int N> __device__ __forceinline__ void pin(f32x16 (&x)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) pin(x[n]);
}
template <int N, int M> __device__ __forceinline__ void pin(uint32_t (&x)[N][M]) {
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
        for (int m = 0; m < M; ++m) asm volatile("" : "+v"(x[n][m]));
}

// A workgroup barrier that is also a compiler memory fence: the compiler
// models s_barrier as touching no memory, so without the empty asm clobbers it
// could move an LDS read of the next step above the barrier (and past the
// refill of the slot it reads) or a DMA issue of this step below it. Costs no
// instruction.
__device__ __forceinline__ void fence_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float max_with_partner(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
                 __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) +
           __builtin_bit_cast(float, (uint32_t)r[1]);
}

// ---- rotary position embedding (RoPE) -----------------------------------------
// Pair (a, b) turned by the angle with cosine c and sine s, in fp32:
// a' = a c - b s, b' = b c + a s. The D dimensions of a row form D/2 pairs,
// pair t being dims (t, t + D/2) ("halves") or (2t, 2t + 1) ("interleaved");
// a row at position p takes c, s from row p of [n_pos, D/2] fp32 tables.
__device__ __forceinline__ void rotate(float &a, float &b, float c, float s) {
    const float na = a * c - b * s;
    const float nb = b * c + a * s;
    a = na;
    b = nb;
}

__device__ __forceinline__ float4 load_f4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

// RoPE of one row held as D/16 fragments of 8 values, fragment c holding dims
// 8 * (2c + g) .. + 7 (the MFMA operand layout of a 32-row block: the lane's
// half g = 0, 1 holds every other 8-dim chunk). cs and sn point at the row's
// table rows. Under halves the partner of dim d < D/2 is d + D/2, which lies
// in fragment c + D/32 of the same lane.
template <typename T, int D>
__device__ __forceinline__ void rope_fragments(typename Elem<T>::vec8 (&x)[D / 16], int g,
                                               const float *cs, const float *sn,
                                               bool interleaved) {
    constexpr int NC = D / 16;
    if (!interleaved) {
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
            const int t0 = 8 * (2 * c + g);
            const float4 c0 = load_f4(cs + t0), c1 = load_f4(cs + t0 + 4);
            const float4 s0 = load_f4(sn + t0), s1 = load_f4(sn + t0 + 4);
            const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = (float)x[c][e], b = (float)x[c + NC / 2][e];
                rotate(a, b, cc[e], ss[e]);
                x[c][e] = (T)a;
                x[c + NC / 2][e] = (T)b;
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int t0 = 4 * (2 * c + g);
            const float4 c0 = load_f4(cs + t0), s0 = load_f4(sn + t0);
            const float cc[4] = {c0.x, c0.y, c0.z, c0.w};
            const float ss[4] = {s0.x, s0.y, s0.z, s0.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a = (float)x[c][2 * e], b = (float)x[c][2 * e + 1];
                rotate(a, b, cc[e], ss[e]);
                x[c][2 * e] = (T)a;
                x[c][2 * e + 1] = (T)b;
            }
        }
    }
}

// ---- persistent work lists (ListPlan) ------------------------------------------
// The list position of this workgroup's item in round r, and its list x
// (list_pos_at and list_item in fa_internal.h, shared with the host).
__device__ __forceinline__ int list_pos(const ListPlan &pl, int r, int &x) {
    return list_pos_at(pl, (int)blockIdx.x, (int)gridDim.x, r, x);
}

}  // namespace dev
}  // namespace fa
