// Block-sparse FlashAttention-style forward (SpargeAttn notes, section 2.1:
// online softmax with running max m, running sum l and unnormalised output O;
// blocks outside the mask skip both QK^T and PV; section 2.3: PV skip when
// the running-max gap of a row group is below lambda).
//
// k_flash_dma<D, SUB, GATHER, FP8>, k_flash_lam<D, SUB, GATHER, FP8>: the
// kernels for 128-row query blocks without and with PV skip; 128-key blocks
// (SUB = 2) run as two 64-key tiles, with one PV-skip decision per block in
// k_flash_lam.  One workgroup of 4 wavefronts per query block; wavefront w owns
// query rows 32w..32w+31 and is the PV-skip group.  Scores are computed
// transposed, S^T = K Q^T, so that every accumulator a lane holds belongs to
// ONE query row (lane & 31): row max/sum need no cross-lane work beyond one
// exchange with lane ^ 32, and the output rescale is one scalar per lane.
// O^T = V^T P^T reuses the exponentials as the B operand.  GATHER reads q, k,
// v through the token permutation and stores O back in the original order;
// FP8 takes the QK products on E4M3 codes with per-block scales.  See the
// comments at the kernels.
//
// k_flash_small<D>: the 16x16-block case (tiny workloads), plain fp32 ALU; it
// maps rows through the permutation (when given) one load at a time.
#include <cmath>
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
// An exp2 argument below this gives 0 in fp32 (the smallest subnormal is 2^-149),
// with a wide margin for the rounding of the argument.
constexpr float kExpZeroArg = -200.0f;

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// 32 E4M3 codes per lane: the A/B operand of v_mfma_f32_32x32x64_f8f6f4
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ inline i32x8 cat8(uint4 a, uint4 b) {
    return i32x8{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
}
// C += A B over 64 products per element, both operands E4M3 (format code 0);
// with no block scales the compiler emits the unscaled instruction
__device__ inline floatx16 mfma_fp8(i32x8 a, i32x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over one head's rows: loads at or past `bytes` return 0
// (hardware range check), which covers the ragged last block and any
// out-of-range column without branches.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}

__global__ void k_attn_init(int32_t* status, unsigned long long* counters) {
    *status = SA_OK;
    if (counters) counters[0] = counters[1] = counters[2] = 0ull;
}

// Source row of position i of the reordered sequence: perm[i], or i without a
// permutation.  An entry outside 0..N-1 (perm is then no permutation) reads
// row 0 instead of leaving the tensor.
__device__ inline int64_t src_row(const int32_t* perm, int64_t i, int64_t N) {
    if (!perm) return i;
    const int32_t r = perm[i];
    return (r >= 0 && r < N) ? r : 0;
}

// Small helpers of the pipelined kernels.
__device__ inline float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ inline float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// (value of this lane, value of lane ^ 32) combined: returns both halves' values
__device__ inline void swap32(float v, float& lo, float& hi) {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(pr[0]);
    hi = __uint_as_float(pr[1]);
}
// max over lanes 0..31 (lanes 32..63 hold the same values), uniform result
__device__ inline float max_lanes32(float v) {
    v = fmaxf(v, __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), 0x140, 0xF, 0xF, false)));
    const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
    const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
    return fmaxf(r0, r1);
}

// LDS-DMA kernels (the production path for 64-key tiles).  K and V tiles go
// straight from HBM/L2 into LDS with buffer_load ... lds (16 bytes per lane,
// out-of-range rows read as zero).  Each 1 KB DMA instruction moves 8 rows x
// 128 bytes (whole cache lines); in LDS the 16-byte chunks of row r are
// XOR-permuted (K: by (r>>1)&7, V: by r&7) so that the MFMA operand reads are
// bank-conflict free: the K operand (ds_read_b128, key row 32mt+(l&31),
// head-dim chunk 2ks+(l>>5)) and the transposed V operand (ds_read_b64_tr_b16:
// in each 16-lane group lane i slot j receives element i&3 of the 8 bytes
// lane 4j+i/4 read, so lane l reads
// V[16ps + 8ab + 4(l>>5) + ((l&15)>>2)][32tt + 16((l>>4)&1) + 4(l&3) .. +3]).
// All operand read addresses are one of a few per-lane offsets plus an
// immediate.
//
// GATHER: q, k and v stay in the caller's token order and position i of the
// reordered sequence is row perm[i] (the reorder is an index map, not a
// copy).  Each tile's 64 entries of perm are DMA'd into a small LDS ring
// several tiles ahead; every lane reads the source rows of its DMA lines from
// there one iteration before it issues them, and O rows are stored back at
// their original positions.  The arithmetic is unchanged, so the output equals
// that of the same kernel on reordered copies bit for bit.
//
// The exponentials are taken against the running maximum itself, so the
// largest probability of the row is exactly 1 (exact in bf16 for the PV
// product); O and l are rescaled only on tiles where some row's maximum rises.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier without the implied memory waits: the caller has already
// waited for what must be complete (the in-flight DMA of a later tile is not
// waited for); the clobber keeps the compiler from moving memory accesses
// across it.
__device__ inline void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }
// this wave's LDS reads and writes are complete
__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Buffer resource (descriptor words) over `bytes` bytes at `base`, for the DMA
// below; offsets at or past `bytes` read as zero.
typedef int int4v __attribute__((ext_vector_type(4)));
__device__ inline int4v head_desc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return int4v{int(uint32_t(p)), int(uint32_t(p >> 32) & 0xffff), int(bytes), 0x00020000};
}
// LDS byte address of a __shared__ object
__device__ inline uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
// 16 (dma16_at) or 4 (dma4_at) bytes per lane from buffer `r` at byte offset
// `off` into LDS at la + lane * size; `la` is wave-uniform.  Issued as assembly
// so the compiler does not track it (it would otherwise wait for every
// outstanding LDS DMA before any LDS read); the kernels wait explicitly
// (dma_wait) before the barrier that publishes a DMA'd buffer.  M0 is handed
// to the compiler as an operand.  The compiler does not pad hazards into
// inline assembly, so the leading s_nop supplies the five wait states a vector
// memory instruction needs after a VALU write of an SGPR it reads (the
// descriptor can be restored from a spill with v_readlane right before), which
// also covers the one after the write of M0.
__device__ inline void dma16_at(int4v r, uint32_t la, uint32_t off) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(off), "s"(r), "{m0}"(la) : "memory");
}
__device__ inline void dma4_at(int4v r, uint32_t la, uint32_t off) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" :: "v"(off), "s"(r), "{m0}"(la) : "memory");
}
// Marks the Q fragments as consumed here, so the compiler waits for their
// loads once, before the tile loop, instead of inside it (where its count
// would also wait for the untracked tile DMAs in flight).
template <int KS>
__device__ inline void q_ready(const bf16x8_t (&qf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(qf[ks]));
}
// (in 128-bit halves: a wider asm operand silently voids the kernel's host
// launch stub)
template <int KS>
__device__ inline void q_ready(const i32x8 (&qf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(qf[ks].lo), "v"(qf[ks].hi));
}

// FP8 QK operands (D = 128): a query row is 128 bytes of E4M3 codes, so a
// 64-key K tile is 8 KB in LDS, laid out like a bf16 tile of head dim 64: 8-row
// lines of 128-byte rows, 16-byte chunk p of row r holding source chunk
// p ^ ((r >> 1) & 7).  For k-step ks (64 head-dim entries) lane l supplies
// entries 64 ks + 32 (l >> 5) .. +31 of its key row (A operand) or query row
// (B operand), so both operands agree on which products are summed.
// Q codes of this lane's query row, two k-steps
__device__ inline void load_q8(const uint8_t* q8_head, uint32_t head_bytes, int qsrc, int half, i32x8 (&qf)[2]) {
    const __amdgpu_buffer_rsrc_t rQ = head_rsrc(q8_head, head_bytes);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint32_t off = uint32_t(qsrc) * 128u + uint32_t(64 * ks + 32 * half);
        qf[ks] = cat8(bload16(rQ, off), bload16(rQ, off + 16u));
    }
}
// byte offsets of this lane's four 16-byte K operand chunks in an FP8 tile:
// [2 ks + x] = chunk 4 ks + 2 half + x of key row l32 (add 4096 for rows 32..63)
__device__ inline void k8_offsets(int l32, int half, int (&off)[4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int x = 0; x < 2; ++x)
            off[2 * ks + x] = (l32 >> 3) * 1024 + (l32 & 7) * 128 + (((4 * ks + 2 * half + x) ^ ((l32 >> 1) & 7)) * 16);
}
// this lane's K operands of a 64-key FP8 tile: kf[2 ks] for keys 0..31, kf[2 ks + 1]
// for keys 32..63
__device__ inline void load_k8(const uint8_t* K8, const int (&off)[4], i32x8 (&kf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint8_t* p = K8 + off[2 * ks];
        const uint8_t* p1 = K8 + off[2 * ks + 1];
        kf[2 * ks] = cat8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p1));
        kf[2 * ks + 1] = cat8(*reinterpret_cast<const uint4*>(p + 4096), *reinterpret_cast<const uint4*>(p1 + 4096));
    }
}
// raw scores of a 64-key FP8 tile: s0 keys 0..31, s1 keys 32..63 (code units)
__device__ inline void qk_fp8(const i32x8 (&kf)[4], const i32x8 (&qf)[2], floatx16& s0, floatx16& s1) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        s0 = mfma_fp8(kf[2 * ks], qf[ks], s0);
        s1 = mfma_fp8(kf[2 * ks + 1], qf[ks], s1);
    }
}
// vmcnt(N): at most N of this wave's vector memory operations outstanding
template <int N>
__device__ inline void dma_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else static_assert(N == 0 || N == 2 || N == 4, "add the count");
}

constexpr int kRing = 8;  // LDS ring of per-tile source rows (GATHER)
constexpr int kColChunk = 512;  // column indices staged in LDS per chunk (k_flash_lam)

// Per-lane part of the tile DMA.  Instruction c of wave w moves rows
// 8*rg .. 8*rg+7 (rg = 2w + c/SEG) of 128-byte segment c % SEG of a 64-row
// tile; lane L carries row 8*rg + L/8 into LDS position L%8 of that line, so
// it reads source chunk (L%8) ^ swizzle(row).  A lane thus moves rows
// r0 = 16w + L/8 and r0 + 8 of every tile.
template <int D>
struct TileLane {
    static constexpr int SEG = D / 64;
    int r0;
    uint32_t kch[2][SEG];  // K: chunk offset of row r0 + 8x plus segment offset
    uint32_t vch[SEG];     // V: the same (the V swizzle is equal for both rows)
    __device__ TileLane(int wave, int lane) {
        const int dq = lane >> 3, dp = lane & 7;
        r0 = 16 * wave + dq;
#pragma unroll
        for (int s = 0; s < SEG; ++s) {
            kch[0][s] = uint32_t((dp ^ ((dq >> 1) & 7)) * 16 + s * 128);
            kch[1][s] = uint32_t((dp ^ ((4 + (dq >> 1)) & 7)) * 16 + s * 128);
            vch[s] = uint32_t((dp ^ dq) * 16 + s * 128);
        }
    }
    __device__ uint32_t k_off(const uint32_t (&rb)[2], int c) const { return rb[c / SEG] + kch[c / SEG][c % SEG]; }
    __device__ uint32_t v_off(const uint32_t (&rb)[2], int c) const { return rb[c / SEG] + vch[c % SEG]; }
};

// lambda off: every kept tile runs its PV product.  K and V run one tile
// ahead in two LDS buffers each.  128-key blocks run as two 64-key tiles.
template <int D, int SUB, bool GATHER, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_flash_dma(FlashArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                 uint8_t* __restrict__ pv_skip) {
    constexpr int BQ = 128;
    constexpr int BK = 64;
    constexpr int NT = D / 32;               // 32-wide output column tiles
    constexpr int KS = D / 16;               // MFMA k-steps over the head dim
    constexpr int SEG = D / 64;              // 128-byte segments per row
    constexpr int DI = 2 * SEG;              // DMA instructions per wave per tile and tensor
    static_assert(!FP8 || D == 128, "the FP8 QK path has head dim 128");
    constexpr int KT = FP8 ? BK * D / 2 : BK * D;  // uint16 slots of one K tile
    // One array per buffer, selected at compile time, so that operand reads
    // use constant LDS addresses.
    __shared__ __align__(16) uint16_t Ks0[KT];
    __shared__ __align__(16) uint16_t Ks1[KT];
    __shared__ __align__(16) uint16_t Vs0[BK * D];
    __shared__ __align__(16) uint16_t Vs1[BK * D];
    __shared__ __align__(16) int32_t prow[GATHER ? kRing : 1][BK];  // source rows of tile t in slot t % kRing
    __shared__ float ksc[FP8 ? kMaxKeyTiles : 1];  // FP8: the scale of every 64-key tile of the head
    auto kbuf_of = [&](auto I) -> uint16_t* {
        if constexpr (decltype(I)::value == 0) return Ks0;
        else return Ks1;
    };
    auto vbuf_of = [&](auto I) -> uint16_t* {
        if constexpr (decltype(I)::value == 0) return Vs0;
        else return Vs1;
    };

    const int G = a.B * a.Hq * a.n_qb;
    const int per = (G + 7) >> 3;
    const int row = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (row >= G) return;
    const int qb = row % a.n_qb;
    const int bh = row / a.n_qb;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int N = int(a.N);
    const int Nk = int(a.Nk);  // keys per sequence
    const uint32_t head_bytes = uint32_t(N) * D * 2u;
    const uint32_t kv_bytes = uint32_t(Nk) * D * 2u;
    const int4v rK = FP8 ? head_desc(a.k8 + (int64_t(b) * a.Hkv + hk) * Nk * D, uint32_t(Nk) * D)
                         : head_desc(a.k + (int64_t(b) * a.Hkv + hk) * Nk * D, kv_bytes);
    const int4v rV = head_desc(a.v + (int64_t(b) * a.Hkv + hk) * Nk * D, kv_bytes);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int wrow0 = qb * BQ + wave * 32;
    const int qrow = wrow0 + l32;
    const bool row_valid = qrow < N;
    const bool wave_rows = wrow0 < N;
    int qsrc = qrow;  // source row of this lane's query; past the end it reads zeros
    if constexpr (GATHER) qsrc = row_valid ? a.perm[qrow] : N;

    bf16x8_t qf[FP8 ? 1 : KS];
    i32x8 q8f[2];
    float qscale = 1.f;  // FP8: dequantization scale of this query block
    if constexpr (FP8) {
        load_q8(a.q8 + int64_t(bh) * N * D, uint32_t(N) * D, qsrc, half, q8f);
        qscale = a.q_scale[int64_t(bh) * a.n_qb + qb];
        const float* ks_src = a.k_scale + (int64_t(b) * a.Hkv + hk) * a.n_kt;
        // one entry past the last tile: a 128-key block's second tile may lie wholly past the end
        for (int x = tid; x <= a.n_kt; x += 256) ksc[x] = x < a.n_kt ? ks_src[x] : 1.f;
    } else {
        const __amdgpu_buffer_rsrc_t rQ = head_rsrc(a.q + int64_t(bh) * N * D, head_bytes);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = as_bf16x8(bload16(rQ, uint32_t(qsrc * D + ks * 16 + half * 8) * 2u));
    }

    int e0 = row_ptr[row];
    int e1 = row_ptr[row + 1];
    if (e1 > a.col_cap) {
        if (tid == 0) *a.dev_status = SA_ERR_CAPACITY;
        e1 = int(a.col_cap);
    }
    if (e0 < 0) {  // a malformed row_ptr: the row reads no entry
        if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
        e0 = e1 = 0;
    }
    const int nt = (e1 > e0 ? e1 - e0 : 0) * SUB;

    auto tile_key0 = [&](int t) -> int {
        const int j = col_idx[e0 + t / SUB];
        if (j < 0 || j >= a.n_kb) return -1;
        return j * (BK * SUB) + (t % SUB) * BK;
    };
    const TileLane<D> tl(wave, lane);
    const int4v rP = head_desc(a.perm, uint32_t(N) * 4u);
    const uint32_t pr_lds = lds_addr(&prow[0][0]);
    // wave 0 fetches the source rows of tile t (first key key0) into ring slot t % kRing
    auto issue_perm = [&](int t, int key0) {
        if constexpr (GATHER) {
            if (wave == 0 && key0 >= 0)
                dma4_at(rP, pr_lds + uint32_t((t % kRing) * BK * 4), uint32_t(key0 + lane) * 4u);
        }
    };
    // A tile's rows for this lane: its first key and the ring entries of the
    // lane's two rows (GATHER), read one iteration before the DMA and turned
    // into byte offsets only there, so the LDS read latency is hidden.
    struct Rows {
        int key0;
        int32_t src[2];
    };
    auto tile_rows = [&](int t, int key0, Rows& rw) {
        rw.key0 = key0;
        if constexpr (GATHER) {
#pragma unroll
            for (int x = 0; x < 2; ++x) rw.src[x] = prow[t % kRing][tl.r0 + 8 * x];
        }
    };
    // byte offsets of the two source rows (rows of rs bytes); an invalid tile
    // or a row past the end gets an offset beyond the buffer (reads zeros)
    auto row_bytes = [&](const Rows& rw, uint32_t (&rb)[2], uint32_t rs) {
        if constexpr (GATHER) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = tl.r0 + 8 * x;
                rb[x] = (rw.key0 >= 0 && rw.key0 + r < Nk) ? uint32_t(rw.src[x]) * rs : 0x80000000u;
            }
        } else {
            const uint32_t base = rw.key0 < 0 ? 0x80000000u : uint32_t(rw.key0) * rs;
#pragma unroll
            for (int x = 0; x < 2; ++x) rb[x] = base + uint32_t(tl.r0 + 8 * x) * rs;
        }
    };
    auto issue_kv = [&](const Rows& rw, auto KN) {
        uint32_t rb[2];
        row_bytes(rw, rb, uint32_t(D * 2));
        const uint32_t vl = lds_addr(vbuf_of(KN)) + uint32_t(wave * DI * 1024);
        if constexpr (FP8) {  // 2 lines of 8 code rows per wave: rows r0 and r0 + 8
            uint32_t rk[2];
            row_bytes(rw, rk, uint32_t(D));
            const uint32_t kl = lds_addr(kbuf_of(KN)) + uint32_t(wave * 2 * 1024);
#pragma unroll
            for (int c = 0; c < 2; ++c) dma16_at(rK, kl + uint32_t(c * 1024), rk[c] + tl.kch[c][0]);
        } else {
            const uint32_t kl = lds_addr(kbuf_of(KN)) + uint32_t(wave * DI * 1024);
#pragma unroll
            for (int c = 0; c < DI; ++c) dma16_at(rK, kl + uint32_t(c * 1024), tl.k_off(rb, c));
        }
#pragma unroll
        for (int c = 0; c < DI; ++c) dma16_at(rV, vl + uint32_t(c * 1024), tl.v_off(rb, c));
    };
    // operand read offsets (elements): K for ks % 4, V for tt % 2
    int k_off[4], v_off[2];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
        k_off[k4] = ((l32 >> 3) * SEG * 1024 + (l32 & 7) * 128 + (((2 * k4 + half) ^ ((l32 >> 1) & 7)) * 16)) / 2;
    int k8o[4];  // FP8: byte offsets of the K operand chunks
    if constexpr (FP8) k8_offsets(l32, half, k8o);
    {
        const int g = (lane >> 4) & 1, j = (lane & 15) >> 2, m = lane & 3;
#pragma unroll
        for (int x = 0; x < 2; ++x)
            v_off[x] = ((4 * half + j) * 128 + (((4 * x + 2 * g + (m >> 1)) ^ (4 * half + j)) * 16) + 8 * (m & 1)) / 2;
    }

    floatx16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
    float m_run = -INFINITY;  // running max in score units (q.k; FP8: of the dequantized operands)
    float l_part = 0.f;
    const float c2 = a.scale * kLog2e;
    int n_exec = 0;
    bool bad_col = false;
    Rows nr;  // rows of the next tile to fetch
    // first keys of tiles t, t+1, t+2 (one column index is loaded per step,
    // ahead of the ring reads, so waiting for it never waits for them)
    int kc = nt > 0 ? tile_key0(0) : -1, k1 = nt > 1 ? tile_key0(1) : -1, k2 = nt > 2 ? tile_key0(2) : -1;

    // tile t: K and V in buffer KC; tile t+1 goes to buffer KN
    auto step = [&](int t, auto KC, auto KN) {
        const int kb0 = kc;
        const int k3 = t + 3 < nt ? tile_key0(t + 3) : -1;
        if (GATHER && t + 3 < nt) issue_perm(t + 3, k3);
        if (t + 1 < nt) issue_kv(nr, KN);
        // ring slot t+2 was filled during iteration t-1
        if (t + 2 < nt) tile_rows(t + 2, k2, nr);
        if (kb0 < 0) {
            bad_col = true;
        } else if (wave_rows) {
            const uint16_t* K = kbuf_of(KC);
            floatx16 s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
            // FP8: scores in code units; f turns them into q.k of the dequantized operands
            float f = 1.f;
            if constexpr (FP8) {
                f = qscale * ksc[kb0 >> 6];
                i32x8 kf[4];
                load_k8(reinterpret_cast<const uint8_t*>(K), k8o, kf);
                qk_fp8(kf, q8f, s0, s1);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint16_t* Kk = K + k_off[ks & 3] + (ks >> 2) * 512;
                    const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(Kk);
                    const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(Kk + 4 * SEG * 512);
                    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks], s1, 0, 0, 0);
                }
            }
            const float c2t = c2 * f;
            if ((kb0 + BK > Nk) || (a.causal && kb0 + BK - 1 > wrow0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = kb0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool ok0 = kk < Nk && (!a.causal || kk <= qrow);
                    const bool ok1 = kk + 32 < Nk && (!a.causal || kk + 32 <= qrow);
                    s0[i] = ok0 ? s0[i] : -INFINITY;
                    s1[i] = ok1 ? s1[i] : -INFINITY;
                }
            }
            float mx[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float m1 = max3f(s0[4 * r], s0[4 * r + 1], s0[4 * r + 2]);
                const float m2 = max3f(s0[4 * r + 3], s1[4 * r], s1[4 * r + 1]);
                mx[r] = max3f(m1, m2, max2f(s1[4 * r + 2], s1[4 * r + 3]));
            }
            float lo, hi;
            swap32(max3f(mx[0], mx[1], max2f(mx[2], mx[3])), lo, hi);
            const float m_new = max2f(m_run, max2f(lo, hi) * f);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
                const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);  // 0 when m_run = -inf
                l_part *= alpha;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[tt][i] *= alpha;
            }
            m_run = m_new;
            const float mc = (m_new == -INFINITY ? 0.f : m_new) * c2;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c2t, -mc));
                s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c2t, -mc));
            }
            float ps[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ps[i] = (s0[2 * i] + s0[2 * i + 1]) + (s1[2 * i] + s1[2 * i + 1]);
            l_part += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
            ++n_exec;
            bf16x8_t pb[4];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                pb[0][x] = (__bf16)s0[x];
                pb[1][x] = (__bf16)s0[8 + x];
                pb[2][x] = (__bf16)s1[x];
                pb[3][x] = (__bf16)s1[8 + x];
            }
            const uint16_t* Vt = vbuf_of(KC);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                for (int ps4 = 0; ps4 < 4; ++ps4) {
                    const uint16_t* pa = Vt + v_off[tt & 1] + ((2 * ps4) * SEG + (tt >> 1)) * 512;
                    const short4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)pa);
                    const short4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(pa + SEG * 512));
                    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ps4], oacc[tt], 0, 0, 0);
                }
            }
        }
        // the tiles of t+1 (and the source rows of t+3) have landed; the
        // operand reads of tile t are complete (consumed by the MFMAs)
        dma_wait<0>();
        tile_barrier();  // ... everyone's; the buffers of tile t are free again
        kc = k1;
        k1 = k2;
        k2 = k3;
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if constexpr (GATHER) {
        issue_perm(0, kc);
        issue_perm(1, k1);
        issue_perm(2, k2);
        dma_wait<0>();
        tile_barrier();
    }
    if (nt > 0) {
        Rows r0;
        tile_rows(0, kc, r0);
        issue_kv(r0, I0{});
    }
    if (nt > 1) tile_rows(1, k1, nr);
    dma_wait<0>();
    __syncthreads();
    if constexpr (FP8) q_ready(q8f);
    else q_ready(qf);
    for (int t = 0; t < nt; t += 2) {
        step(t, I0{}, I1{});
        if (t + 1 < nt) step(t + 1, I1{}, I0{});
    }
    if (pv_skip && lane == 0)
        for (int e = e0; e < e1; ++e) pv_skip[int64_t(e) * 4 + wave] = 0;
    if (bad_col && tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;

    float l_lo, l_hi;
    swap32(l_part, l_lo, l_hi);
    const float l_tot = l_lo + l_hi;
    if (row_valid && uint32_t(qsrc) < uint32_t(N)) {  // entries of perm outside 0..N-1 store nothing
        const float inv = 1.0f / l_tot;  // l = 0 (no key) -> 0 * inf = NaN
        if (l_tot == 0.f) *a.dev_status = SA_ERR_EMPTY_ROW;
        float* orow = a.o + (int64_t(bh) * N + qsrc) * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 v;
                v.x = oacc[tt][4 * g + 0] * inv;
                v.y = oacc[tt][4 * g + 1] * inv;
                v.z = oacc[tt][4 * g + 2] * inv;
                v.w = oacc[tt][4 * g + 3] * inv;
                *reinterpret_cast<float4*>(orow + 32 * tt + 8 * g + 4 * half) = v;
            }
    }
    if (a.counters) {
        if (tid == 0) atomicAdd(&a.counters[0], (unsigned long long)(e1 > e0 ? e1 - e0 : 0));
        if (lane == 0 && wave_rows) atomicAdd(&a.counters[1], (unsigned long long)((n_exec + SUB - 1) / SUB));
    }
}

// PV-skip variant of k_flash_dma (the production path when lambda is set).
// Same LDS layouts, operand reads and online softmax.  The
// PV product of a tile is deferred by one iteration: during iteration t the
// four waves fetch V of tile t-1 cooperatively (only if some wave kept the PV
// of that tile; the need flags come through LDS), while the scores and
// softmax of tile t run; a barrier then lets the waves that kept it apply
// O <- alpha O + P V for tile t-1.  O therefore lags one tile behind m and l;
// a skipped tile never raises a valid row's maximum (its alpha is 1), so only
// kept tiles carry a pending rescale.  K runs two tiles ahead in three
// buffers; V needs one buffer.  The skip test of a 32-row group is one
// ballot: skip when no valid row's block maximum comes within lambda of its
// new running maximum.
//
// SUB = 2: 128-key blocks as two 64-key tiles with one decision per block, as
// the PV-skip rule defines it (the block's row maximum against the running
// maximum after the whole block).  The first half is scored and added to m and
// l as usual and its P kept pending undecided; the second half decides for
// both.  The first half's V is therefore fetched whatever the decision (during
// the second half's iteration), and its PV product is applied there, after
// the decision, or dropped.  A skipped block never raises a valid row's
// maximum, so dropping needs no rescale; a kept one applies O <- aA O + PA VA,
// then (one iteration later) O <- aB O + PB VB, which equals the block update
// with P taken against the maximum after the block.
template <int D, int SUB, bool GATHER, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_flash_lam(FlashArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                 uint8_t* __restrict__ pv_skip) {
    constexpr int BQ = 128;
    constexpr int BK = 64;
    constexpr int NT = D / 32;               // 32-wide output column tiles
    constexpr int KS = D / 16;               // MFMA k-steps over the head dim
    constexpr int SEG = D / 64;              // 128-byte segments per row
    constexpr int DI = 2 * SEG;              // DMA instructions per wave per tile and tensor
    static_assert(!FP8 || D == 128, "the FP8 QK path has head dim 128");
    constexpr int DK = FP8 ? 2 : DI;         // ... for K (FP8: 8 KB tiles)
    constexpr int KT = FP8 ? BK * D / 2 : BK * D;  // uint16 slots of one K tile
    __shared__ __align__(16) uint16_t Ks[3][KT];
    __shared__ __align__(16) uint16_t Vs[BK * D];
    __shared__ __align__(16) int32_t prow[GATHER ? kRing : 1][BK];  // source rows of tile t in slot t % kRing
    // need[t % 3] byte w: wave w keeps the PV product of tile t (each wave stores its own
    // byte every tile, so no slot needs clearing; the four bytes read as one word)
    __shared__ __align__(4) uint8_t need[3][4];
    // the row's column indices, kColChunk tiles per chunk, two chunks in turn
    __shared__ __align__(16) int32_t colc[2][kColChunk];
    __shared__ float ksc[FP8 ? kMaxKeyTiles : 1];  // FP8: the scale of every 64-key tile of the head

    const int G = a.B * a.Hq * a.n_qb;
    const int per = (G + 7) >> 3;
    const int row = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (row >= G) return;
    const int qb = row % a.n_qb;
    const int bh = row / a.n_qb;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int N = int(a.N);
    const int Nk = int(a.Nk);  // keys per sequence
    const uint32_t head_bytes = uint32_t(N) * D * 2u;
    const uint32_t kv_bytes = uint32_t(Nk) * D * 2u;
    const int4v rK = FP8 ? head_desc(a.k8 + (int64_t(b) * a.Hkv + hk) * Nk * D, uint32_t(Nk) * D)
                         : head_desc(a.k + (int64_t(b) * a.Hkv + hk) * Nk * D, kv_bytes);
    const int4v rV = head_desc(a.v + (int64_t(b) * a.Hkv + hk) * Nk * D, kv_bytes);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int wrow0 = qb * BQ + wave * 32;
    const int qrow = wrow0 + l32;
    const bool row_valid = qrow < N;
    const bool wave_rows = wrow0 < N;
    int qsrc = qrow;  // source row of this lane's query; past the end it reads zeros
    if constexpr (GATHER) qsrc = row_valid ? a.perm[qrow] : N;

    bf16x8_t qf[FP8 ? 1 : KS];
    i32x8 q8f[2];
    float qscale = 1.f;  // FP8: dequantization scale of this query block
    if constexpr (FP8) {
        load_q8(a.q8 + int64_t(bh) * N * D, uint32_t(N) * D, qsrc, half, q8f);
        qscale = a.q_scale[int64_t(bh) * a.n_qb + qb];
        const float* ks_src = a.k_scale + (int64_t(b) * a.Hkv + hk) * a.n_kt;
        // one entry past the last tile: a 128-key block's second tile may lie wholly past the end
        for (int x = tid; x <= a.n_kt; x += 256) ksc[x] = x < a.n_kt ? ks_src[x] : 1.f;
    } else {
        const __amdgpu_buffer_rsrc_t rQ = head_rsrc(a.q + int64_t(bh) * N * D, head_bytes);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = as_bf16x8(bload16(rQ, uint32_t(qsrc * D + ks * 16 + half * 8) * 2u));
    }

    int e0 = row_ptr[row];
    int e1 = row_ptr[row + 1];
    if (e1 > a.col_cap) {
        if (tid == 0) *a.dev_status = SA_ERR_CAPACITY;
        e1 = int(a.col_cap);
    }
    if (e0 < 0) {  // a malformed row_ptr: the row reads no entry
        if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
        e0 = e1 = 0;
    }
    const int ne = e1 > e0 ? e1 - e0 : 0;  // CSR entries (key blocks) of the row
    const int nt = ne * SUB;                // 64-key tiles

    auto tile_key0 = [&](int t) -> int {
        const int j = col_idx[e0 + t / SUB];
        if (j < 0 || j >= a.n_kb) return -1;
        return j * (BK * SUB) + (t % SUB) * BK;
    };
    const TileLane<D> tl(wave, lane);
    const int4v rP = head_desc(a.perm, uint32_t(N) * 4u);
    const uint32_t pr_lds = lds_addr(&prow[0][0]);
    const uint32_t ks_lds = lds_addr(&Ks[0][0]) + uint32_t(wave * DK * 1024);
    const uint32_t vs_lds = lds_addr(&Vs[0]) + uint32_t(wave * DI * 1024);
    // wave 0 fetches the source rows of tile t (first key key0) into ring slot t % kRing;
    // a tile past the row's end (key -1) reads zeros
    auto issue_perm = [&](int t, int key0) {
        if constexpr (GATHER) {
            if (wave == 0)
                dma4_at(rP, pr_lds + uint32_t((t % kRing) * BK * 4),
                        key0 >= 0 ? uint32_t(key0 + lane) * 4u : 0x80000000u);
        }
    };
    // A tile's rows for this lane: its first key and the ring entries of the
    // lane's two rows (GATHER), read one iteration before the DMA and turned
    // into byte offsets only there, so the LDS read latency is hidden.
    struct Rows {
        int key0;
        int32_t src[2];
    };
    auto tile_rows = [&](int key0, int t, Rows& rw) {
        rw.key0 = key0;
        if constexpr (GATHER) {
#pragma unroll
            for (int x = 0; x < 2; ++x) rw.src[x] = prow[t % kRing][tl.r0 + 8 * x];
        }
    };
    // byte offsets of the two source rows (rows of rs bytes); an invalid tile
    // or a row past the end gets an offset beyond the buffer (reads zeros)
    auto row_bytes = [&](const Rows& rw, uint32_t (&rb)[2], uint32_t rs) {
        if constexpr (GATHER) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = tl.r0 + 8 * x;
                rb[x] = (rw.key0 >= 0 && rw.key0 + r < Nk) ? uint32_t(rw.src[x]) * rs : 0x80000000u;
            }
        } else {
            const uint32_t base = rw.key0 < 0 ? 0x80000000u : uint32_t(rw.key0) * rs;
#pragma unroll
            for (int x = 0; x < 2; ++x) rb[x] = base + uint32_t(tl.r0 + 8 * x) * rs;
        }
    };
    auto issue_k = [&](const Rows& rw, int buf) {  // this wave's share of a K tile
        uint32_t rb[2];
        if constexpr (FP8) {  // 2 lines of 8 code rows per wave: rows r0 and r0 + 8
            row_bytes(rw, rb, uint32_t(D));
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dma16_at(rK, ks_lds + uint32_t(buf * BK * D + c * 1024), rb[c] + tl.kch[c][0]);
        } else {
            row_bytes(rw, rb, uint32_t(D * 2));
#pragma unroll
            for (int c = 0; c < DI; ++c)
                dma16_at(rK, ks_lds + uint32_t(buf * BK * D * 2 + c * 1024), tl.k_off(rb, c));
        }
    };
    auto issue_v = [&](const Rows& rw) {  // this wave's share of a V tile
        uint32_t rb[2];
        row_bytes(rw, rb, uint32_t(D * 2));
#pragma unroll
        for (int c = 0; c < DI; ++c) dma16_at(rV, vs_lds + uint32_t(c * 1024), tl.v_off(rb, c));
    };
    // operand read offsets (elements): K for ks % 4, V for tt % 2
    int k_off[4], v_off[2];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
        k_off[k4] = ((l32 >> 3) * SEG * 1024 + (l32 & 7) * 128 + (((2 * k4 + half) ^ ((l32 >> 1) & 7)) * 16)) / 2;
    int k8o[4];  // FP8: byte offsets of the K operand chunks
    if constexpr (FP8) k8_offsets(l32, half, k8o);
    {
        const int g = (lane >> 4) & 1, j = (lane & 15) >> 2, m = lane & 3;
#pragma unroll
        for (int x = 0; x < 2; ++x)
            v_off[x] = ((4 * half + j) * 128 + (((4 * x + 2 * g + (m >> 1)) ^ (4 * half + j)) * 16) + 8 * (m & 1)) / 2;
    }

    floatx16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
    float m_run = -INFINITY;  // running max in score units (q.k; FP8: of the dequantized operands)
    float l_part = 0.f;
    const float c2 = a.scale * kLog2e;
    const float lam_raw = a.lambda / a.scale;
    int n_exec = 0, n_skip = 0;
    bool bad_col = false;
    // the kept tile whose PV product is pending: P (bf16) and its rescale of O
    bool pend = false;
    bf16x8_t pp[4];
    float palpha = 1.f;
    auto apply_pending = [&]() {
        if (__builtin_amdgcn_ballot_w64(palpha != 1.0f)) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[tt][i] *= palpha;
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int ps4 = 0; ps4 < 4; ++ps4) {
                const uint16_t* pa = Vs + v_off[tt & 1] + ((2 * ps4) * SEG + (tt >> 1)) * 512;
                const short4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)pa);
                const short4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(pa + SEG * 512));
                const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pp[ps4], oacc[tt], 0, 0, 0);
            }
        }
    };

    // column indices of entries 0 .. 2*kColChunk-1 (published by the barrier before the
    // loop); later chunks are DMA'd by wave 0 one chunk ahead.  No scalar loads stay in
    // the loop: an outstanding one would make every LDS-operand wait a full lgkmcnt(0).
    {
        constexpr int PER = 2 * kColChunk / 256;
        int cv[PER];
#pragma unroll
        for (int x = 0; x < PER; ++x) cv[x] = tid + 256 * x < ne ? col_idx[e0 + tid + 256 * x] : -1;
#pragma unroll
        for (int x = 0; x < PER; ++x) (&colc[0][0])[tid + 256 * x] = cv[x];
    }
    const int4v rC = head_desc(col_idx + (ne > 0 ? e0 : 0), uint32_t(ne) * 4u);
    // kr: source rows of the next K tile to fetch (t+2 during iteration t);
    // vr: those of tile t-1, whose V may be fetched during iteration t
    Rows kr, vr;
    // first keys of tiles t .. t+4: the column index of tile t+5 is loaded
    // during iteration t and first used in iteration t+1, so its scalar load
    // has a whole iteration to land
    int kc = nt > 0 ? tile_key0(0) : -1, k1 = nt > 1 ? tile_key0(1) : -1;
    int k2 = nt > 2 ? tile_key0(2) : -1, k3 = nt > 3 ? tile_key0(3) : -1;
    int k4 = nt > 4 ? tile_key0(4) : -1;
    if constexpr (GATHER) {
        issue_perm(0, kc);
        issue_perm(1, k1);
        issue_perm(2, k2);
        issue_perm(3, k3);
        dma_wait<0>();
        tile_barrier();
    }
    if (nt > 0) {
        tile_rows(kc, 0, kr);
        issue_k(kr, 0);
    }
    if (nt > 1) {
        tile_rows(k1, 1, kr);
        issue_k(kr, 1);
    }
    if (nt > 2) tile_rows(k2, 2, kr);
    dma_wait<0>();
    __syncthreads();
    if constexpr (FP8) q_ready(q8f);
    else q_ready(qf);
    // bf16: K operands of the next tile's first KPRE k-steps, read right after the barrier
    // that publishes its buffer, so the first score products do not wait for them (the FP8
    // tile's eight operand reads are issued with its products: prefetching them was slower)
    constexpr int KPRE = KS < 4 ? KS : 4;
    bf16x8_t kpre[FP8 ? 1 : 2 * KPRE];
    auto prefetch_k = [&](int buf) {
        if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < KPRE; ++ks) {
                const uint16_t* Kk = Ks[buf] + k_off[ks];
                kpre[2 * ks] = *reinterpret_cast<const bf16x8_t*>(Kk);
                kpre[2 * ks + 1] = *reinterpret_cast<const bf16x8_t*>(Kk + 4 * SEG * 512);
            }
        }
    };
    prefetch_k(0);
    int kbuf = 0;  // t % 3, also the need slot of tile t
    uint32_t need_prev = 0u;  // the need flags of tile t-1, read after the last barrier
    uint64_t skipm = 0ull;    // bit i: PV of entry et - et % 64 + i skipped (this wave's group)
    float mx_first = -INFINITY;  // SUB = 2: the block's first-half row maximum
    int refill_t = kColChunk * SUB;  // next tile that starts a column chunk
    int flush_t = 64 * SUB - 1;      // next tile whose entry ends a run of 64 skip flags
    for (int t = 0; t < nt; ++t) {
        const int kb0 = kc;
        const int et = t / SUB;                        // CSR entry of tile t
        const bool first = SUB == 2 && (t & 1) == 0;   // first half of a 128-key block
        const bool second = SUB == 2 && (t & 1) == 1;  // ... the half that decides
        // V of tile t-1 first (so waiting for it leaves the K prefetch in flight); the
        // first half of a block is fetched whatever the decision
        const uint32_t need_s = __builtin_amdgcn_readfirstlane(need_prev);
        const bool vprev = second || (t > 0 && need_s != 0u);
        // raw column index of the entry of tile t+5 (LDS), checked and turned into a key
        // at the end of the iteration
        // (the two chunks are one ring of 2 kColChunk entries)
        int c5v = (&colc[0][0])[((t + 5) / SUB) & (2 * kColChunk - 1)];  // stale past the row's end
        // the chunk after next: entries et+kColChunk.., into the buffer of the chunk that
        // ended with entry et-1 (its last read was at least five tiles ago); issued before
        // the V and K tiles so the waits below cover it
        if (t == refill_t) {
            refill_t += kColChunk * SUB;
            if (wave == 0 && et + kColChunk < ne) {
                const uint32_t cl = lds_addr(&colc[((et / kColChunk) + 1) & 1][0]);
#pragma unroll
                for (int h = 0; h < kColChunk / 256; ++h)
                    dma16_at(rC, cl + uint32_t(h * 1024),
                             uint32_t(et + kColChunk + h * 256) * 4u + uint32_t(lane) * 16u);
            }
        }
        // prefetches past the row's end (key -1) read zeros into buffers nobody reads,
        // so they need no condition
        if (GATHER) issue_perm(t + 4, k4);
        if (vprev) issue_v(vr);
        issue_k(kr, kbuf == 0 ? 2 : kbuf - 1);
        // rows for the next iteration: V of tile t, K of tile t+3 (its ring
        // slot was filled during iteration t-1)
        tile_rows(kb0, t, vr);
        tile_rows(k3, t + 3, kr);

        int my_need = 0;
        float alpha = 1.f;
        floatx16 s0, s1;
        if (kb0 < 0) {
            bad_col = true;
        } else if (wave_rows) {
            const uint16_t* K = Ks[kbuf];
#pragma unroll
            for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
            // FP8: scores in code units; f turns them into q.k of the dequantized operands
            float f = 1.f;
            if constexpr (FP8) f = qscale * ksc[kb0 >> 6];
            // the score products issue ahead of the other wave of this SIMD, whose
            // softmax then fills the VALU while the matrix core runs
            __builtin_amdgcn_s_setprio(1);
            if constexpr (FP8) {
                i32x8 kf[4];
                load_k8(reinterpret_cast<const uint8_t*>(K), k8o, kf);
                qk_fp8(kf, q8f, s0, s1);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint16_t* Kk = K + k_off[ks & 3] + (ks >> 2) * 512;
                    const bf16x8_t k0 = ks < KPRE ? kpre[2 * ks] : *reinterpret_cast<const bf16x8_t*>(Kk);
                    const bf16x8_t k1 =
                        ks < KPRE ? kpre[2 * ks + 1] : *reinterpret_cast<const bf16x8_t*>(Kk + 4 * SEG * 512);
                    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks], s1, 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            const float c2t = c2 * f;
            if ((kb0 + BK > Nk) || (a.causal && kb0 + BK - 1 > wrow0)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = kb0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool ok0 = kk < Nk && (!a.causal || kk <= qrow);
                    const bool ok1 = kk + 32 < Nk && (!a.causal || kk + 32 <= qrow);
                    s0[i] = ok0 ? s0[i] : -INFINITY;
                    s1[i] = ok1 ? s1[i] : -INFINITY;
                }
            }
            float mx[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float m1 = max3f(s0[4 * r], s0[4 * r + 1], s0[4 * r + 2]);
                const float m2 = max3f(s0[4 * r + 3], s1[4 * r], s1[4 * r + 1]);
                mx[r] = max3f(m1, m2, max2f(s1[4 * r + 2], s1[4 * r + 3]));
            }
            float lo, hi;
            swap32(max3f(mx[0], mx[1], max2f(mx[2], mx[3])), lo, hi);
            const float smax_raw = max2f(lo, hi);  // the row's largest score of this tile
            const float smax = smax_raw * f;
            const float m_new = max2f(m_run, smax);
            // the block's row maximum: this tile's, or (second half) both halves'
            const float bmax = second ? max2f(mx_first, smax) : smax;
            if (first) mx_first = smax;
            // NaN (no key yet) and -inf gaps never reach lambda
            const bool skip = __builtin_amdgcn_ballot_w64(row_valid && bmax - m_new >= lam_raw) == 0ull;
            alpha = m_new > m_run ? __builtin_amdgcn_exp2f((m_run - m_new) * c2) : 1.f;  // 0 when m_run = -inf
            m_run = m_new;
            const float mc = (m_new == -INFINITY ? 0.f : m_new) * c2;
            // A skipped tile leaves alpha at 1 (the maximum did not move) and needs no P,
            // so all it does is add its exponentials to the row sum.  With `arg` the
            // largest exponent argument (the same fma as below, on the row's largest
            // score), a lane adds at most 32 * 2^arg to its l_part: nothing when arg is
            // under -200 (every exp2 is 0), and nothing after rounding when that bound
            // is under half an ulp of l_part (l_part in [2^(E-1), 2^E): arg < E - 31,
            // one step of margin).  When that holds on every row the exponentials are
            // left out, with no change to any result.  NaN scores take the full path.
            const float arg = fmaf(smax_raw, c2t, -mc);
            const bool lost = arg < kExpZeroArg ||
                              (l_part > 0.f && arg < float(__builtin_amdgcn_frexp_expf(l_part) - 31));
            const bool zero = !first && skip && __builtin_amdgcn_ballot_w64(row_valid && !lost) == 0ull;
            if (!zero) {
                if constexpr (!FP8) {
                    // every exponent argument first, in place, then the exponentials: no
                    // instruction waits on the one just before it (measured faster for bf16
                    // scores, slower for the shorter FP8 score phase)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s0[i] = fmaf(s0[i], c2t, -mc);
                        s1[i] = fmaf(s1[i], c2t, -mc);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s0[i] = __builtin_amdgcn_exp2f(s0[i]);
                        s1[i] = __builtin_amdgcn_exp2f(s1[i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c2t, -mc));
                        s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c2t, -mc));
                    }
                }
                float ps[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) ps[i] = (s0[2 * i] + s0[2 * i + 1]) + (s1[2 * i] + s1[2 * i + 1]);
                l_part = fmaf(l_part, alpha, ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7])));
            }
            if (first) {
                my_need = 1;  // undecided: kept pending until the second half decides
            } else if (skip) {
                skipm |= 1ull << (et & 63);
                ++n_skip;
            } else {
                ++n_exec;
                my_need = 1;
            }
        }
        // PV of tile t-1 once every wave's part of its V tile has landed (the second
        // half drops its block's first-half product when the block is skipped)
        if (vprev) {
            dma_wait<DK>();  // only the K DMAs issued after it may still be in flight
            tile_barrier();
            if (pend && (!second || my_need)) apply_pending();
        }
        // tile t becomes the pending one
        pend = my_need != 0;
        if (pend) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                pp[0][x] = (__bf16)s0[x];
                pp[1][x] = (__bf16)s0[8 + x];
                pp[2][x] = (__bf16)s1[x];
                pp[3][x] = (__bf16)s1[8 + x];
            }
            palpha = alpha;
        }
        if (lane == 0) need[kbuf][wave] = uint8_t(my_need);
        // the skip flags of 64 entries leave in one store (lane i: entry et - et % 64 + i)
        if (t == flush_t || t == nt - 1) {
            flush_t += 64 * SUB;
            if (pv_skip && lane <= (et & 63))
                pv_skip[int64_t(e0 + (et & ~63) + lane) * 4 + wave] = uint8_t((skipm >> lane) & 1ull);
            skipm = 0ull;
        }
        // K of tile t+1 and the source rows of tile t+4 have landed (K of t+2
        // may be in flight); V reads and the need flags are complete
        dma_wait<DK>();
        lds_wait();
        tile_barrier();
        // every wave's need flag of tile t is in place: read it now, use it at the
        // top of the next iteration
        need_prev = *reinterpret_cast<const uint32_t*>(need[kbuf]);
        kbuf = kbuf == 2 ? 0 : kbuf + 1;
        prefetch_k(kbuf);
        kc = k1;
        k1 = k2;
        k2 = k3;
        k3 = k4;
        // the LDS read of c5v is consumed only here (the empty asm keeps the
        // compiler from moving the read-first-lane, and its wait, up to the read)
        asm volatile("" : "+v"(c5v));
        const int c5 = __builtin_amdgcn_readfirstlane(c5v);
        k4 = (t + 5 >= nt || c5 < 0 || c5 >= a.n_kb) ? -1 : c5 * (BK * SUB) + ((t + 5) % SUB) * BK;
    }
    dma_wait<0>();  // no LDS write may land after the workgroup ends
    if (nt > 0 && __builtin_amdgcn_readfirstlane(need_prev) != 0u) {
        issue_v(vr);
        dma_wait<0>();
        tile_barrier();
        if (pend) apply_pending();
    }
    if (bad_col && tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;

    float l_lo, l_hi;
    swap32(l_part, l_lo, l_hi);
    const float l_tot = l_lo + l_hi;
    if (row_valid && uint32_t(qsrc) < uint32_t(N)) {  // entries of perm outside 0..N-1 store nothing
        const float inv = 1.0f / l_tot;  // l = 0 (no key) -> 0 * inf = NaN
        if (l_tot == 0.f) *a.dev_status = SA_ERR_EMPTY_ROW;
        float* orow = a.o + (int64_t(bh) * N + qsrc) * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 v;
                v.x = oacc[tt][4 * g + 0] * inv;
                v.y = oacc[tt][4 * g + 1] * inv;
                v.z = oacc[tt][4 * g + 2] * inv;
                v.w = oacc[tt][4 * g + 3] * inv;
                *reinterpret_cast<float4*>(orow + 32 * tt + 8 * g + 4 * half) = v;
            }
    }
    if (a.counters) {
        if (tid == 0) atomicAdd(&a.counters[0], (unsigned long long)ne);
        if (lane == 0 && wave_rows) {
            atomicAdd(&a.counters[1], (unsigned long long)n_exec);
            atomicAdd(&a.counters[2], (unsigned long long)n_skip);
        }
    }
}

// 16x16 blocks: thread (r, c) owns query row r of the block and output
// columns c, c+16, ...; scores go through LDS.  The whole 16-row block is one
// PV-skip group.
template <int D>
__global__ __launch_bounds__(256) void k_flash_small(FlashArgs a) {
    constexpr int B = 16;
    __shared__ float Qs[B][D + 1];
    __shared__ float Ks[B][D + 1];
    __shared__ float Vs[B][D + 1];
    __shared__ float Ss[B][B + 1];
    __shared__ float gaps[B];

    const int row = blockIdx.x;
    const int qb = row % a.n_qb;
    const int bh = row / a.n_qb;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t N = a.N;
    const uint16_t* Qh = a.q + int64_t(bh) * N * D;
    const int64_t Nk = a.Nk;
    const uint16_t* Kh = a.k + (int64_t(b) * a.Hkv + hk) * Nk * D;
    const uint16_t* Vh = a.v + (int64_t(b) * a.Hkv + hk) * Nk * D;
    float* Oh = a.o + int64_t(bh) * N * D;

    const int tid = threadIdx.x;
    const int r = tid / B, c = tid % B;
    const int64_t qrow = int64_t(qb) * B + r;
    const bool valid = qrow < N;
    for (int t = tid; t < B * D; t += 256) {
        const int rr = t / D, dd = t % D;
        const int64_t qq = int64_t(qb) * B + rr;
        Qs[rr][dd] = qq < N ? __uint_as_float(uint32_t(Qh[src_row(a.perm, qq, N) * D + dd]) << 16) : 0.f;
    }
    float m = -INFINITY, l = 0.f;
    float O[D / B];
#pragma unroll
    for (int u = 0; u < D / B; ++u) O[u] = 0.f;
    const bool lam_on = a.lambda > -INFINITY;
    int n_exec = 0, n_skip = 0;
    int e0 = a.row_ptr[row];
    int e1 = a.row_ptr[row + 1];
    if (e1 > a.col_cap) {
        if (tid == 0) *a.dev_status = SA_ERR_CAPACITY;
        e1 = int(a.col_cap);
    }
    if (e0 < 0) {  // a malformed row_ptr: the row reads no entry
        if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
        e0 = e1 = 0;
    }
    for (int e = e0; e < e1; ++e) {
        const int jblk = a.col_idx[e];
        if (jblk < 0 || jblk >= a.n_kb) {
            if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
            continue;
        }
        const int64_t kb0 = int64_t(jblk) * B;
        __syncthreads();
        for (int t = tid; t < B * D; t += 256) {
            const int rr = t / D, dd = t % D;
            const int64_t key = kb0 + rr;
            const int64_t src = key < Nk ? src_row(a.perm, key, Nk) : 0;
            Ks[rr][dd] = key < Nk ? __uint_as_float(uint32_t(Kh[src * D + dd]) << 16) : 0.f;
            Vs[rr][dd] = key < Nk ? __uint_as_float(uint32_t(Vh[src * D + dd]) << 16) : 0.f;
        }
        __syncthreads();
        const int64_t key = kb0 + c;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(Qs[r][d], Ks[c][d], s);
        const bool ok = key < Nk && (!a.causal || key <= qrow);
        Ss[r][c] = ok ? s * a.scale : -INFINITY;
        __syncthreads();
        float rmax = -INFINITY;
        for (int kk = 0; kk < B; ++kk) rmax = fmaxf(rmax, Ss[r][kk]);
        const float m_new = fmaxf(m, rmax);
        if (c == 0) gaps[r] = (valid && rmax > -INFINITY) ? rmax - m_new : -INFINITY;
        __syncthreads();
        bool skip = false;
        if (lam_on) {
            float gmax = -INFINITY;
            for (int kk = 0; kk < B; ++kk) gmax = fmaxf(gmax, gaps[kk]);
            skip = gmax < a.lambda;
        }
        const float msafe = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m - msafe);
        float p[B];
        float ps = 0.f;
        for (int kk = 0; kk < B; ++kk) {
            p[kk] = expf(Ss[r][kk] - msafe);
            ps += p[kk];
        }
        l = l * alpha + ps;
        m = m_new;
        if (!skip) {
#pragma unroll
            for (int u = 0; u < D / B; ++u) {
                float acc = O[u] * alpha;
                for (int kk = 0; kk < B; ++kk) acc = fmaf(p[kk], Vs[kk][c + B * u], acc);
                O[u] = acc;
            }
        }
        if (tid == 0) {
            if (a.pv_skip) a.pv_skip[e] = skip ? 1 : 0;
            n_exec += skip ? 0 : 1;
            n_skip += skip ? 1 : 0;
        }
    }
    if (valid) {
        const float inv = 1.0f / l;
        if (l == 0.f) *a.dev_status = SA_ERR_EMPTY_ROW;
        const int64_t qsrc = src_row(a.perm, qrow, N);
#pragma unroll
        for (int u = 0; u < D / B; ++u) Oh[qsrc * D + c + B * u] = O[u] * inv;
    }
    if (a.counters && tid == 0) {
        atomicAdd(&a.counters[0], (unsigned long long)(e1 > e0 ? e1 - e0 : 0));
        atomicAdd(&a.counters[1], (unsigned long long)n_exec);
        atomicAdd(&a.counters[2], (unsigned long long)n_skip);
    }
}

}  // namespace

hipError_t launch_flash(const FlashArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(k_attn_init, dim3(1), dim3(1), 0, stream, a.dev_status, a.counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = int64_t(a.B) * a.Hq * a.n_qb;
    if (rows > INT32_MAX) return hipErrorInvalidValue;
    const bool lam_on = a.lambda > -INFINITY;
    const dim3 grid{unsigned(rows), 1, 1};
    const dim3 block{256, 1, 1};
    const dim3 pgrid{unsigned((rows + 7) / 8 * 8), 1, 1};
    const bool G = a.perm != nullptr;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, pgrid, block, 0, stream, a, a.row_ptr, a.col_idx, a.pv_skip); };
    if (a.q8) {
        // FP8 QK path: head dim 128, 128-row query blocks; the caller has checked the shape
        if (a.D != 128 || a.bq != 128 || !(a.bk == 64 || a.bk == 128)) return hipErrorInvalidValue;
        if (a.n_kt != (a.Nk + 63) / 64 || a.n_kt >= kMaxKeyTiles) return hipErrorInvalidValue;
        if (lam_on && a.bk == 64) G ? go(k_flash_lam<128, 1, true, true>) : go(k_flash_lam<128, 1, false, true>);
        else if (lam_on) G ? go(k_flash_lam<128, 2, true, true>) : go(k_flash_lam<128, 2, false, true>);
        else if (a.bk == 64) G ? go(k_flash_dma<128, 1, true, true>) : go(k_flash_dma<128, 1, false, true>);
        else G ? go(k_flash_dma<128, 2, true, true>) : go(k_flash_dma<128, 2, false, true>);
    } else if (a.bq == 16 && a.bk == 16) {
        if (a.D == 128) hipLaunchKernelGGL(k_flash_small<128>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(k_flash_small<64>, grid, block, 0, stream, a);
    } else if (a.D == 128) {
        if (lam_on && a.bk == 64) G ? go(k_flash_lam<128, 1, true, false>) : go(k_flash_lam<128, 1, false, false>);
        else if (lam_on) G ? go(k_flash_lam<128, 2, true, false>) : go(k_flash_lam<128, 2, false, false>);
        else if (a.bk == 64) G ? go(k_flash_dma<128, 1, true, false>) : go(k_flash_dma<128, 1, false, false>);
        else G ? go(k_flash_dma<128, 2, true, false>) : go(k_flash_dma<128, 2, false, false>);
    } else {
        if (lam_on && a.bk == 64) G ? go(k_flash_lam<64, 1, true, false>) : go(k_flash_lam<64, 1, false, false>);
        else if (lam_on) G ? go(k_flash_lam<64, 2, true, false>) : go(k_flash_lam<64, 2, false, false>);
        else if (a.bk == 64) G ? go(k_flash_dma<64, 1, true, false>) : go(k_flash_dma<64, 1, false, false>);
        else G ? go(k_flash_dma<64, 2, true, false>) : go(k_flash_dma<64, 2, false, false>);
    }
    return hipGetLastError();
}

}  // namespace sa
