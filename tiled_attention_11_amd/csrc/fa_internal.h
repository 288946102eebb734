// fa_internal.h -- launch parameters shared by the C-ABI host code and the
// gfx950 kernels of the attention forward. Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace fa {

// "Unbounded" window side: larger than any sequence index the ABI accepts,
// small enough that i + kUnbounded does not overflow a 32-bit int.
constexpr int kUnbounded = 1 << 30;

// Everything a kernel needs, computed and validated on the host.
struct FwdParams {
    const void *q, *k, *v;  // [B, H, S, D]
    void *o;                // [B, H, S, D]
    float *lse;             // [B, H, S] or nullptr
    int B, H, S;
    int n_qtiles;           // ceil(S / query rows per workgroup)
    // Key j is visible from query i iff i - win_lo <= j <= i + win_hi and j < S
    // (win_lo, win_hi in [0, kUnbounded]); covers all three mask modes.
    int win_lo, win_hi;
    float c2;               // max(|scale| * log2(e), 2^-100): scores go to base 2 in one multiply
    int negate_q;           // scale < 0: Q's sign is flipped on load instead
    // Work distribution (see the kernel): `grid` workgroups, each running a
    // stream of work items (query tiles). xcd_lists: B*H % 8 == 0 and grid % 8
    // == 0, so list x (heads x, x + 8, ...) is served by workgroups w = x mod 8;
    // otherwise one list holds every head. list_len: items per list;
    // group_heads: heads per group within a list (divides the list's heads).
    int grid;
    int xcd_lists;
    int list_len;
    int group_heads;
};

// Query rows per workgroup of every kernel variant.
constexpr int kBlockM = 256;

// Enqueue the kernel for head dimension D and dtype (0 fp16, 1 bf16).
hipError_t launch_fwd(const FwdParams &p, int D, int dtype, hipStream_t stream);

// ---- new query rows against a key/value cache ---------------------------------
// Keys per tile of the cache kernel.
constexpr int kDecodeBN = 32;
// Query rows of one call: one wave's MFMA block.
constexpr int kDecodeMaxRows = 32;

struct DecodeParams {
    const void *q;          // [B, H, Sq, D]
    const void *k, *v;      // [B, H, Sk, D]
    void *o;                // [B, H, Sq, D]
    float *lse;             // [B, H, Sq] or nullptr
    float *ws_o;            // nsplit > 1: partial outputs [B*H, nsplit, Sq, D]
    float *ws_lse;          // nsplit > 1: partial LSEs [B*H, nsplit, Sq]
    int B, H, Sq, Sk;
    int pos0;               // Sk - Sq: position of query row 0 in the sequence
    int win_lo, win_hi;     // as in FwdParams, relative to each row's position
    float c2;
    int negate_q;
    int t_first, t_last;    // key tiles visible from some row (same for every head)
    int tiles_per_split;    // a split covers this many consecutive tiles (the last may have fewer)
    int nsplit;             // splits per head; 1 writes o and lse directly
};

// Enqueue the cache kernel (and, for nsplit > 1, the merge kernel).
hipError_t launch_decode(const DecodeParams &p, int D, int dtype, hipStream_t stream);

}  // namespace fa
