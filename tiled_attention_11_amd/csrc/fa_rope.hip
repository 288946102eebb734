// fa_rope.hip -- rotary position embedding (RoPE) of a [B, H, S, D] tensor for
// gfx950 (MI355X): row s of every head turns by the angles of table row s.
//
// What it computes: the Ascend C tile-fusion page (ascendai.csdn.net),
// section 9, rotates Q and K by position from a cos/sin table; read as the
// usual rotary embedding, each pair of dims (halves: d and d + D/2, or
// interleaved: 2t and 2t + 1) is turned by the table's angle for the row's
// position, in fp32, and the result rounded once (RNE) to the element type.
//
// gfx950 design: a plain streaming pass (HBM-bound: 2 bytes read and 2
// written per element, the tables staying in L2). A thread handles 8 pairs of
// one row with 16-byte loads and stores; consecutive threads cover
// consecutive 16-byte pieces of consecutive rows, so each wave reads and
// writes whole contiguous rows. Each thread reads and writes only its own
// elements, so the output may be the input (in place).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kRopeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kRopeThreads) void fa_rope_kernel(RopeParams p) {
    typedef typename Elem<T>::vec8 vec8;
    constexpr int TPR = D / 16;  // threads per row, 8 pairs each
    const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    const int64_t row = gid / TPR;
    if (row >= p.rows) return;
    const int part = (int)(gid - row * TPR);
    const int pos = (int)(row % p.S);
    const float *cs = p.cos + (int64_t)pos * (D / 2) + 8 * part;
    const float *sn = p.sin + (int64_t)pos * (D / 2) + 8 * part;
    const float4 c0 = load_f4(cs), c1 = load_f4(cs + 4);
    const float4 s0 = load_f4(sn), s1 = load_f4(sn + 4);
    const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint16_t *xr = static_cast<const uint16_t *>(p.x) + row * D;
    uint16_t *yr = static_cast<uint16_t *>(p.y) + row * D;
    // halves: pairs 8*part .. +7 are dims (t, t + D/2); interleaved: they are
    // dims 16*part .. +15, pair e being elements (2e, 2e + 1)
    const int oa = p.interleaved ? 16 * part : 8 * part;
    const int ob = p.interleaved ? 16 * part + 8 : 8 * part + D / 2;
    vec8 a = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4 *>(xr + oa));
    vec8 b = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4 *>(xr + ob));
    if (!p.interleaved) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float u = (float)a[e], w = (float)b[e];
            rotate(u, w, cc[e], ss[e]);
            a[e] = (T)u;
            b[e] = (T)w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float u = (float)a[2 * e], w = (float)a[2 * e + 1];
            rotate(u, w, cc[e], ss[e]);
            a[2 * e] = (T)u;
            a[2 * e + 1] = (T)w;
            u = (float)b[2 * e];
            w = (float)b[2 * e + 1];
            rotate(u, w, cc[e + 4], ss[e + 4]);
            b[2 * e] = (T)u;
            b[2 * e + 1] = (T)w;
        }
    }
    *reinterpret_cast<u32x4 *>(yr + oa) = __builtin_bit_cast(u32x4, a);
    *reinterpret_cast<u32x4 *>(yr + ob) = __builtin_bit_cast(u32x4, b);
}

template <typename T, int D>
hipError_t launch_rope_t(const RopeParams &p, hipStream_t stream) {
    const int64_t threads = p.rows * (D / 16);
    const int64_t blocks = (threads + kRopeThreads - 1) / kRopeThreads;
    void *args[] = {const_cast<RopeParams *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_rope_kernel<T, D>),
                           dim3((unsigned)blocks), dim3(kRopeThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_rope(const RopeParams &p, int D, int dtype, hipStream_t stream) {
    if (D == 128) return dtype == 0 ? launch_rope_t<_Float16, 128>(p, stream)
                                    : launch_rope_t<__bf16, 128>(p, stream);
    if (D == 64) return dtype == 0 ? launch_rope_t<_Float16, 64>(p, stream)
                                   : launch_rope_t<__bf16, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
