// Per-block FP8 E4M3 quantization of the QK operands (SpargeAttn notes,
// section 2.4: the sparse kernel's QK path takes Q and K quantized per block,
// with one dequantization scale per block; the format here is OCP FP8 E4M3,
// the 8-bit float of the gfx950 matrix cores).
//
// One workgroup per block of `block` rows of one (batch, head).  The rows are
// read once (through the token permutation when one is given: block j holds
// the rows perm[j*block ..]) and stay in registers while the workgroup reduces
// the block's largest magnitude; then every element becomes the E4M3 code
// nearest to clamp(x * (448 / amax), -448, 448) (v_cvt_pk_fp8_f32: round to
// nearest even, sign kept), written at the row's own position, and the block's
// scale amax / 448 is stored.  amax, both divisions and the product are IEEE
// float32 operations.  An all-zero block gets scale 1 (and zero codes).
#include "sa_internal.h"

namespace sa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                   int64_t N, int block, int64_t n_blocks,
                                                   uint8_t* __restrict__ codes, float* __restrict__ scales) {
    constexpr int LPR = D / 8;         // lanes per row: 8 bf16 (16 bytes) each
    constexpr int RP = 256 / LPR;      // rows per pass of the workgroup
    constexpr int MAXP = kQuantMaxBlock / RP;
    __shared__ uint32_t wmax[4];
    const int64_t g = blockIdx.x;
    const int64_t bh = g / n_blocks;
    const int64_t r0 = (g % n_blocks) * block;
    const int tid = threadIdx.x;
    const int rr = tid / LPR, c = tid % LPR;
    const uint16_t* xh = x + bh * N * D;

    uint4 v[MAXP];
    int32_t src[MAXP];  // source row of pass p, -1: none
    uint32_t m = 0;     // largest |x| of this lane as a bf16 magnitude pattern
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        v[p] = make_uint4(0u, 0u, 0u, 0u);
        src[p] = -1;
        const int64_t r = r0 + p * RP + rr;
        if (p * RP + rr < block && r < N) {
            int64_t s = r;
            if (perm) {
                const int32_t e = perm[r];
                s = (e >= 0 && e < N) ? e : -1;  // not a permutation entry: the row is skipped
            }
            if (s >= 0) {
                src[p] = int32_t(s);
                v[p] = *reinterpret_cast<const uint4*>(xh + s * D + c * 8);
            }
        }
        const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), o)));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    const uint32_t mb = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float amax = __uint_as_float(mb << 16);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
    if (tid == 0) scales[g] = amax > 0.f ? amax / 448.0f : 1.0f;

    uint8_t* ch = codes + bh * N * D;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (src[p] < 0) continue;
        const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = __uint_as_float(w[i] << 16) * inv;
            y[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * inv;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(y[i], -448.0f), 448.0f);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
        *reinterpret_cast<uint2*>(ch + int64_t(src[p]) * D + c * 8) = make_uint2(uint32_t(lo), uint32_t(hi));
    }
}

}  // namespace

hipError_t launch_quant_fp8(const uint16_t* x, const int32_t* perm, int64_t BH, int64_t N, int D, int block,
                            uint8_t* codes, float* scales, hipStream_t stream) {
    const int64_t n_blocks = (N + block - 1) / block;
    const int64_t grid = BH * n_blocks;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    if (D == 128)
        hipLaunchKernelGGL(k_quant_fp8<128>, dim3(unsigned(grid)), dim3(256), 0, stream, x, perm, N, block, n_blocks,
                           codes, scales);
    else
        hipLaunchKernelGGL(k_quant_fp8<64>, dim3(unsigned(grid)), dim3(256), 0, stream, x, perm, N, block, n_blocks,
                           codes, scales);
    return hipGetLastError();
}

}  // namespace sa
