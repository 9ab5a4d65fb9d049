// Coalesced row gather / scatter for the token reorder (SparseAttn article,
// section 3.4: reorder Q, K, V together, undo the reorder on the output).
//
// HBM-bound copies.  One thread moves one 16-byte chunk of a row; consecutive
// threads take consecutive chunks of the same row, so each row is read and
// written as full contiguous segments and only the row index is indirect.
#include "sa_internal.h"

namespace sa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// grid: x over (row, chunk) pairs of one (b,h) slice, y over (b,h) slices.
template <bool kF32>
__global__ __launch_bounds__(256) void k_permute(const void* __restrict__ x, uint16_t* __restrict__ y,
                                                 const int32_t* __restrict__ perm, int64_t bh_count,
                                                 int N, int chunks) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= N * chunks) return;
    const int i = t / chunks;
    const int c = t - i * chunks;
    const int src = perm[i];
    const int64_t D = int64_t(chunks) * 8;
    const bool ok = uint32_t(src) < uint32_t(N);  // an entry outside 0..N-1 reads nothing and writes zeros
    for (int64_t bh = blockIdx.y; bh < bh_count; bh += gridDim.y) {
        const int64_t base = bh * N;
        uint4 out = make_uint4(0, 0, 0, 0);
        if (!ok) {
        } else if constexpr (kF32) {
            const f32x4* xs = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + (base + src) * D) + 2 * c;
            const f32x4 a = __builtin_nontemporal_load(xs);
            const f32x4 b = __builtin_nontemporal_load(xs + 1);
            out.x = bf16_rne_bits(a.x) | (bf16_rne_bits(a.y) << 16);
            out.y = bf16_rne_bits(a.z) | (bf16_rne_bits(a.w) << 16);
            out.z = bf16_rne_bits(b.x) | (bf16_rne_bits(b.y) << 16);
            out.w = bf16_rne_bits(b.z) | (bf16_rne_bits(b.w) << 16);
        } else {
            const u32x4* xs = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + (base + src) * D) + c;
            const u32x4 v = __builtin_nontemporal_load(xs);
            out = make_uint4(v.x, v.y, v.z, v.w);
        }
        uint4* yd = reinterpret_cast<uint4*>(y + (base + i) * D) + c;
        *yd = out;
    }
}

// x[b,h,perm[i],:] = y[b,h,i,:]; chunks of 4 floats.
__global__ __launch_bounds__(256) void k_unpermute(const float* __restrict__ y, float* __restrict__ x,
                                                   const int32_t* __restrict__ perm, int64_t bh_count,
                                                   int N, int chunks) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= N * chunks) return;
    const int i = t / chunks;
    const int c = t - i * chunks;
    const int dst = perm[i];
    if (uint32_t(dst) >= uint32_t(N)) return;  // an entry outside 0..N-1 stores nothing
    const int64_t D = int64_t(chunks) * 4;
    for (int64_t bh = blockIdx.y; bh < bh_count; bh += gridDim.y) {
        const int64_t base = bh * N;
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (base + i) * D) + c);
        *(reinterpret_cast<f32x4*>(x + (base + dst) * D) + c) = v;
    }
}

}  // namespace

hipError_t launch_permute(const void* x, int x_dtype, uint16_t* y, const int32_t* perm,
                          int64_t rows_bh, int64_t N, int D, hipStream_t stream) {
    const int chunks = D / 8;
    const int64_t per_slice = N * chunks;
    if (per_slice > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid(unsigned((per_slice + 255) / 256), unsigned(rows_bh < 65535 ? rows_bh : 65535));
    if (x_dtype == SA_F32)
        hipLaunchKernelGGL(k_permute<true>, grid, dim3(256), 0, stream, x, y, perm, rows_bh, int(N), chunks);
    else
        hipLaunchKernelGGL(k_permute<false>, grid, dim3(256), 0, stream, x, y, perm, rows_bh, int(N), chunks);
    return hipGetLastError();
}

hipError_t launch_unpermute(const float* y, float* x, const int32_t* perm, int64_t rows_bh, int64_t N,
                            int Dv, hipStream_t stream) {
    const int chunks = Dv / 4;
    const int64_t per_slice = N * chunks;
    if (per_slice > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid(unsigned((per_slice + 255) / 256), unsigned(rows_bh < 65535 ? rows_bh : 65535));
    hipLaunchKernelGGL(k_unpermute, grid, dim3(256), 0, stream, y, x, perm, rows_bh, int(N), chunks);
    return hipGetLastError();
}

}  // namespace sa
