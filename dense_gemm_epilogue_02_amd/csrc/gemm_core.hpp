// gemm_core.hpp -- device building blocks of the gfx950 GEMM
//
//   D = epilogue(alpha * s_A * s_B * (A * B) + beta * C),  fp32 accumulation
//
// The operation is the one stated in "CUTLASS Python接口" section 3.3 and
// "CUTLASS Python 接口全解析" section 2 (D = A*B + C, with alpha/beta and an
// fp32 accumulator); the ReLU epilogue follows "CUTLASS Python接口" section
// 5.2 (activation applied after the linear combination).
//
// Design (CDNA4 / gfx950):
//   * A workgroup owns a BM x BN output tile. K is walked in k-tiles of KB
//     bytes per row (KB = 128: 64 bf16/f16, 128 fp8, 32 fp32 elements).
//   * Both operand tiles live in LDS "K-contiguous": row r (an m of A or an n
//     of B) holds the k-tile's 128 bytes as eight 16-byte chunks. Chunk c of
//     row r is stored at chunk slot c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7,
//     which keeps 16-byte MFMA fragment reads, row-wise staging writes and
//     transposed staging writes free of bank conflicts.
//   * Global -> LDS staging uses 16-byte buffer loads (out-of-range lanes get
//     an offset past num_records and read zeros). An operand whose contiguous
//     dimension is K is copied chunk by chunk; one whose contiguous dimension
//     is M (A ColumnMajor) or N (B RowMajor) is loaded as VEC x VEC element
//     blocks and transposed in registers before the LDS write.
//   * Two LDS stages: the k-tile t+1 is fetched into registers while tile t is
//     multiplied out of LDS, then written to the other stage (one barrier per
//     k-tile).
//   * MFMA 32x32 blocks with src0 = B rows (n) and src1 = A rows (m), so each
//     lane ends up with four consecutive n of one m: RowMajor D gets 8- or
//     16-byte vector stores straight from the accumulators.
//   * The k index inside one MFMA is assigned identically for both operands
//     (lane group g, element e -> k = chunk(g) * VEC + e), so the hardware's
//     sum over its K slots is exactly the sum over this k-tile's k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mg {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;

// FAM_MXF8: e4m3 operands with MX block scales (one E8M0 scale per 32
// elements along K, per row of A and per column of B). FAM_MXF4: e2m1
// operands, two per byte along K (element 2t in the low nibble of byte t),
// under the same block scales; the tile engine addresses them as bytes (the
// host passes K in bytes), a 16-byte chunk being one 32-element block.
enum Family { FAM_F32 = 0, FAM_F16 = 1, FAM_BF16 = 2, FAM_F8 = 3, FAM_MXF8 = 4, FAM_MXF4 = 5 };

constexpr uint32_t OOB_OFFSET = 0x80000000u;
constexpr int NUM_RECORDS = 0x7FFFFFFF;
constexpr int ST_POLICY = 2;   // buffer store cache policy: non-temporal (nt)
constexpr int RSRC_FLAGS = 0x00020000;   // gfx9 raw buffer, 32-bit data format

// ---------------------------------------------------------------- per-family

template <int FAM> struct Fam;

template <> struct Fam<FAM_BF16> {
    static constexpr int ESZ = 2, CPL = 1;
    static constexpr bool MX = false;
    static constexpr int SCW = 0;
    using Out = __bf16;
    static __device__ __forceinline__ void mma(f32x16 &c, const u32x4 *x, const u32x4 *y) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x[0]),
                                                     __builtin_bit_cast(bf16x8, y[0]), c, 0, 0, 0);
    }
};
template <> struct Fam<FAM_F16> {
    static constexpr int ESZ = 2, CPL = 1;
    static constexpr bool MX = false;
    static constexpr int SCW = 0;
    using Out = _Float16;
    static __device__ __forceinline__ void mma(f32x16 &c, const u32x4 *x, const u32x4 *y) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x[0]),
                                                    __builtin_bit_cast(f16x8, y[0]), c, 0, 0, 0);
    }
};
template <> struct Fam<FAM_F32> {
    static constexpr int ESZ = 4, CPL = 1;
    static constexpr bool MX = false;
    static constexpr int SCW = 0;
    using Out = float;
    static __device__ __forceinline__ void mma(f32x16 &c, const u32x4 *x, const u32x4 *y) {
        const f32x4 xv = __builtin_bit_cast(f32x4, x[0]);
        const f32x4 yv = __builtin_bit_cast(f32x4, y[0]);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xv.x, yv.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xv.y, yv.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xv.z, yv.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xv.w, yv.w, c, 0, 0, 0);
    }
};
template <> struct Fam<FAM_F8> {
    static constexpr int ESZ = 1, CPL = 2;
    static constexpr bool MX = false;
    static constexpr int SCW = 0;
    using Out = __bf16;
    static __device__ __forceinline__ void mma(f32x16 &c, const u32x4 *x, const u32x4 *y) {
        i32x8 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (int)x[0][e]; a[e + 4] = (int)x[1][e];
            b[e] = (int)y[0][e]; b[e + 4] = (int)y[1][e];
        }
        // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 1.0
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};
// The 32x32x64 scaled MFMA reads, in lane l, 32 bytes of row l%32: bytes
// 0-15 belong to the first 32-element block of its 64 K positions, bytes
// 16-31 to the second; the E8M0 scale of (row r, block b) comes from lane
// r + 32b, byte OPSEL of its scale register (lane layout measured on gfx950).
// The MX tile kernels therefore give lane group g chunks 2s*2+g and 2s*2+2+g
// of substep s, so each hardware block holds one real 32-element K block.
template <> struct Fam<FAM_MXF8> {
    static constexpr int ESZ = 1, CPL = 2;
    static constexpr bool MX = true;
    static constexpr int SCW = 1;   // 32-bit scale words per row per k-tile (4 blocks)
    using Out = __bf16;
    template <int OPSEL>
    static __device__ __forceinline__ void mma_mx(f32x16 &c, const u32x4 *x, const u32x4 *y,
                                                  uint32_t sx, uint32_t sy) {
        i32x8 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (int)x[0][e]; a[e + 4] = (int)x[1][e];
            b[e] = (int)y[0][e]; b[e + 4] = (int)y[1][e];
        }
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, (int)sx, OPSEL,
                                                             (int)sy);
    }
};

// The 32x32x64 scaled MFMA with FP4 operands reads, in lane l, 16 bytes (32
// elements) of row l%32 that all belong to hardware block l/32 -- its 64 K
// positions are two 32-element blocks, one per lane half (lane layout
// measured on gfx950) -- and takes the scale of (row r, block b) from lane
// r + 32b as for FP8. Lane group g of substep s reads chunk 2s + g of the
// k-tile's 128-byte row: exactly the k-tile's block 2s + g.
template <> struct Fam<FAM_MXF4> {
    static constexpr int ESZ = 1, CPL = 1;
    static constexpr bool MX = true;
    static constexpr int SCW = 2;   // 32-bit scale words per row per k-tile (8 blocks)
    using Out = __bf16;
    template <int OPSEL>
    static __device__ __forceinline__ void mma_mx(f32x16 &c, const u32x4 *x, const u32x4 *y,
                                                  uint32_t sx, uint32_t sy) {
        const i32x8 a = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3], 0, 0, 0, 0};
        const i32x8 b = {(int)y[0][0], (int)y[0][1], (int)y[0][2], (int)y[0][3], 0, 0, 0, 0};
        // format 4 = FP4 E2M1 for both operands (the unused upper half of
        // each operand is not read)
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, OPSEL, (int)sx, OPSEL,
                                                             (int)sy);
    }
};

// ---------------------------------------------------------------- arguments

// One GEMM problem as the tile engine sees it (uniform per workgroup).
struct Prob {
    const char *A;
    const char *B;
    const char *C;
    char *D;
    int64_t M, N, K;
    int tiles_m, tiles_n, ipt;   // tile grid and k-tiles per output tile
    int vec_cd;                  // C/D allow 4-element vector access
    // Batched GEMM: `batch` problems of the same shape whose operands lie
    // stride_* elements apart (a stride of 0 shares an operand); the tile
    // space is batch-major. batch <= 1 is a single GEMM.
    int batch;
    int64_t stride_a, stride_b, stride_c, stride_d;
    // MX block scales (FAM_MXF8 only): E8M0 bytes [M][K/32] for A's rows and
    // [N][K/32] for B's columns; the tile kernels need K % 128 == 0 and
    // 4-byte aligned arrays.
    const uint8_t *mx_a, *mx_b;
};

// Epilogue activations (the values of gemm_epilogue).
enum { ACT_LINEAR = 0, ACT_RELU = 1, ACT_SIGMOID = 2, ACT_TANH = 3 };

// Auxiliary-tensor elementwise ops (the values of gemm_aux_op).
enum { AUX_ADD = 0, AUX_SUB = 1, AUX_MUL = 2, AUX_DIV = 3 };

struct EpiArgs {
    float alpha, beta;
    const float *scale_a, *scale_b;   // device pointers or null (1.0)
    const void *bias;                 // N elements of the output type, or null
    int act;                          // ACT_*
    int lc_row;                       // C/D RowMajor
    // Auxiliary tensors (M x N, output type, C/D layout), each may be null:
    // aux is combined by aux_op before the activation (aux_after == 0) or
    // after it; aux_out receives the activation's input.
    const void *aux;
    void *aux_out;
    int aux_op, aux_after;
};

// act(v): identity, max(v, +0) (NaN -> +0), 1/(1+e^-v), tanh(v). The two
// transcendental ones use the hardware base-2 exponential and reciprocal
// (about one fp32 ulp each): e^x = 2^(x log2 e); tanh|v| = (1 - t)/(1 + t)
// with t = e^(-2|v|) <= 1, so nothing overflows; the absolute error near 0
// stays below 1e-7.
__device__ __forceinline__ float exp_e(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ float apply_act(float v, int act) {
    switch (act) {
    case ACT_RELU: return v > 0.0f ? v : 0.0f;
    case ACT_SIGMOID: return __builtin_amdgcn_rcpf(1.0f + exp_e(-v));
    case ACT_TANH: {
        const float t = exp_e(-2.0f * __builtin_fabsf(v));
        return __builtin_copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), v);
    }
    default: return v;
    }
}

// y op x for the auxiliary tensor (fp32; the division is IEEE, correctly
// rounded). Written as selects, not a switch: the epilogue applies it to
// every accumulator of a fully unrolled tile, where a branch per element
// would multiply the kernel's control flow.
__device__ __forceinline__ float aux_apply(float y, float x, int op) {
    const float q = y / x;
    float r = op == AUX_SUB ? y - x : y + x;
    r = op == AUX_MUL ? y * x : r;
    return op == AUX_DIV ? q : r;
}

// Output value from the linear result v and the auxiliary element x (0
// without a tensor): the op on its side of the activation; z receives the
// activation's input. pre / post: the op applies before / after it.
// apply_act as selects (all three candidates computed), for the same reason.
__device__ __forceinline__ float act_select(float v, int act) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + exp_e(-v));
    const float t = exp_e(-2.0f * __builtin_fabsf(v));
    const float th = __builtin_copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), v);
    float r = act == ACT_RELU ? (v > 0.0f ? v : 0.0f) : v;
    r = act == ACT_SIGMOID ? sg : r;
    return act == ACT_TANH ? th : r;
}

__device__ __forceinline__ float finish_aux(float v, float x, int op, int act, bool pre, bool post,
                                            float &z) {
    const float r = aux_apply(v, x, op);
    v = pre ? r : v;
    z = v;
    const float d = act_select(v, act);
    const float s = aux_apply(d, x, op);
    return post ? s : d;
}
// finish_aux with the op and activation chosen by (uniform) branches: only
// the selected arithmetic runs. For the general epilogues, where the
// branches stay few.
__device__ __forceinline__ float aux_op_branch(float y, float x, int op) {
    switch (op) {
    case AUX_SUB: return y - x;
    case AUX_MUL: return y * x;
    case AUX_DIV: return y / x;
    default: return y + x;
    }
}
__device__ __forceinline__ float finish_aux_branch(float v, float x, int op, int act, bool pre,
                                                   bool post, float &z) {
    if (pre) v = aux_op_branch(v, x, op);
    z = v;
    float d = apply_act(v, act);
    if (post) d = aux_op_branch(d, x, op);
    return d;
}
__device__ __forceinline__ float finish_aux(float v, float x, const EpiArgs &e, float &z) {
    return finish_aux(v, x, e.aux_op, e.act, e.aux && !e.aux_after, e.aux && e.aux_after, z);
}

// Persistent schedule: schedule indices [0, sk_tiles) are split stream-K
// style over `grid` workgroups; [sk_tiles, total) are whole tiles dealt out
// round robin. With split > 0 every tile is instead cut into `split` units
// (grid = tiles * split): unit c takes k-tiles c, c + split, c + 2 split, ...,
// so the units of one tile, which run side by side, read neighbouring
// segments of every operand row (DRAM page locality on skinny, HBM-bound
// shapes).
// Grouped GEMM: per-problem descriptors in device memory.
struct GroupDesc {
    Prob p;
    int tile_start;   // prefix sum of tiles of the problems before this one
    int pad[3];
};

struct Sched {
    int grid;
    int total_tiles;
    int sk_tiles;
    int64_t sk_iters;       // sk_tiles * ipt
    // Workgroups that share the stream-K iterations: virtual ids [0, sk_grid),
    // with 1 <= sk_grid <= min(grid, sk_iters) so that every one of them owns a
    // non-empty range (a tile's expected arrivals count every id between the
    // owners of its first and last iteration). Ids >= sk_grid go straight to
    // the data-parallel tiles.
    int sk_grid;
    int group_m;            // raster: tile rows per swizzle group
    int xcd_remap;          // map consecutive virtual ids onto one XCD
    int split;              // > 0: interleaved split-K, `split` units per tile
    float *partials;        // stream-K workspace: 2 * grid slots of BM*BN fp32
    int *counters;          // one arrival counter per stream-K tile (self-resetting)
    // Grouped GEMM (gcount > 0; data-parallel tiles only): tile t belongs to
    // the last of the gcount problems whose tile_start is <= t.
    const GroupDesc *gdesc;
    int gcount;
    // Optional work queues for the data-parallel tiles (schedules without
    // stream-K or split-K): each workgroup takes tile v first, then the next
    // unclaimed tile when it finishes one, so tiles of unequal cost (grouped
    // problems of different K) spread evenly. With the XCD remap one queue
    // per XCD: the tiles past the first `grid` go in chunks of QUEUE_CHUNK
    // consecutive tiles to the XCDs in turn, so the workgroups of one XCD
    // stay on neighbouring tiles (shared panels in its L2). queue[0 .. 7]
    // count claims, queue[8] finished workgroups; the last workgroup to
    // finish zeroes all nine, so they start at zero for the next launch on
    // the stream.
    unsigned int *queue;
};

struct KArgs {
    Prob p;
    EpiArgs e;
    Sched s;
};


// ---------------------------------------------------------------- helpers

// Wave-uniform copies (the compiler cannot always prove uniformity; buffer
// descriptors and M0 must live in scalar registers).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// The thread index as a value the compiler cannot see through: per-lane
// offsets derived from it are then computed where they are used instead of
// being hoisted out of the persistent tile loop, where they would stay live
// (and spill) through every main loop.
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(uniform_ptr(base)), (short)0,
                                             NUM_RECORDS, RSRC_FLAGS);
}

// Cache policy of the operand loads: device scope (SC1). Each workgroup
// reads its operand panels once, so they need no L1 allocation. On the
// benchmark workloads this measured the same as the default policy
// (same-box A/B within 1 %); in a standalone launcher whose operands had
// just been allocated it ran 13-18 % faster on the 256x256 bf16 k-loop,
// and the non-temporal hint (NT) ran 10 % slower.
constexpr int LD_POLICY = 16;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, LD_POLICY);
}

// LDS rows hold CH 16-byte chunks (CH = 8: 128-byte rows, CH = 4: 64-byte
// rows). Chunk c of row r lives at slot c ^ swz<CH>(r); the XOR keeps the
// 16 lanes that read rows r..r+15 at one chunk index on distinct banks.
template <int CH> __device__ __forceinline__ int swz(int row);
template <> __device__ __forceinline__ int swz<8>(int row) { return (row ^ (row >> 3)) & 7; }
template <> __device__ __forceinline__ int swz<4>(int row) { return ((row >> 2) ^ (row >> 4)) & 3; }

template <int CH> __device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
    return (uint32_t)(row * CH * 16 + ((chunk ^ swz<CH>(row)) << 4));
}

// Workgroup barrier without the release fence of __syncthreads(): the fence
// would wait for every outstanding vector load (vmcnt(0)), draining the
// LDS-DMA copies that a deep pipeline keeps in flight. Callers wait for the
// copies they need with wait_vmcnt<n>() first (LDS-DMA completion is counted
// by vmcnt); the memory clobber keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// In-register transpose of a VEC x VEC block of ESZ-byte elements held as
// VEC rows of 16 bytes: out[j] element i = in[i] element j.
template <int ESZ> struct Transpose;
template <> struct Transpose<4> {
    static __device__ __forceinline__ void run(const u32x4 *in, u32x4 *out) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) out[j][i] = in[i][j];
    }
};
template <> struct Transpose<2> {
    static __device__ __forceinline__ void run(const u32x4 *in, u32x4 *out) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = in[2 * d][j >> 1], hi = in[2 * d + 1][j >> 1];
                out[j][d] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                    : ((lo & 0xFFFFu) | (hi << 16));
            }
    }
};
template <> struct Transpose<1> {
    static __device__ __forceinline__ void run(const u32x4 *in, u32x4 *out) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int sh = 8 * (j & 3);
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    v |= ((in[4 * d + b][j >> 2] >> sh) & 0xFFu) << (8 * b);
                out[j][d] = v;
            }
    }
};

// ---------------------------------------------------------------- staging

// Global -> register -> LDS copy of one operand k-tile with R rows.
// KC: the operand's contiguous dimension is K (A RowMajor, B ColumnMajor).
template <int R, int ESZ, bool KC, int NT, int CH> struct Stager {
    static constexpr int VEC = 16 / ESZ;
    static constexpr int UNITS = KC ? R * CH : (R / VEC) * CH;
    static constexpr int LPU = KC ? 1 : VEC;           // loads per unit
    static constexpr int UPT = (UNITS + NT - 1) / NT;  // units per thread
    static constexpr bool FULL = (UNITS % NT) == 0;
    u32x4 r[UPT * LPU];

    // base: operand element (row r0, k0) for KC, (k0, r0) otherwise.
    // ld_bytes: byte distance between consecutive rows of the storage.
    // r_left: valid rows from r0; k_left: valid k from k0.
    __device__ __forceinline__ void load(const char *base, uint32_t ld_bytes, int r_left,
                                         int k_left, int tid) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int unit = tid + u * NT;
            const bool act = FULL || unit < UNITS;
            if constexpr (KC) {
                const int row = unit / CH, c = unit % CH;
                const bool ok = act && row < r_left && c * VEC < k_left;
                r[u] = buf_load16(rs, ok ? row * ld_bytes + (uint32_t)(c << 4) : OOB_OFFSET);
            } else {
                constexpr int RB = R / VEC;
                const int rb = unit % RB, kb = unit / RB;
                const bool okr = act && rb * VEC < r_left;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const int k = kb * VEC + i;
                    const bool ok = okr && k < k_left;
                    r[u * VEC + i] =
                        buf_load16(rs, ok ? (uint32_t)k * ld_bytes + (uint32_t)(rb << 4) : OOB_OFFSET);
                }
            }
        }
    }

    __device__ __forceinline__ void store(char *lds, int tid) const {
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int unit = tid + u * NT;
            if (!FULL && unit >= UNITS) continue;
            if constexpr (KC) {
                *reinterpret_cast<u32x4 *>(lds + lds_off<CH>(unit / CH, unit % CH)) = r[u];
            } else {
                constexpr int RB = R / VEC;
                const int rb = unit % RB, kb = unit / RB;
                u32x4 t[VEC];
                Transpose<ESZ>::run(&r[u * VEC], t);
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    *reinterpret_cast<u32x4 *>(lds + lds_off<CH>(rb * VEC + j, kb)) = t[j];
            }
        }
    }
};

// Direct global -> LDS copy (buffer_load_dwordx4 ... lds) of a K-contiguous
// operand k-tile with R rows: no staging registers. One instruction moves 64
// lanes x 16 bytes into 1 KiB of consecutive LDS, lane i landing at slot
// base + i; lane i therefore fetches the logical chunk that the swizzle puts
// in that slot. Out-of-range lanes use an offset past num_records and write
// zeros. The per-lane byte offsets do not depend on k: they are computed once
// per output tile, and each k-tile only advances the (scalar) base address.
template <int R, int ESZ, int NT, int CH> struct DirectStager {
    static constexpr int VEC = 16 / ESZ;
    static constexpr int WAVES = NT / 64;
    static constexpr int RPI = 64 / CH;            // rows per instruction
    static constexpr int INSTR = R / RPI;
    static constexpr int IPW = INSTR / WAVES;      // instructions per wave
    static_assert(INSTR % WAVES == 0, "rows per tile must cover all waves");

    const char *base;        // operand element (r0, k = 0), wave-uniform
    uint32_t ld;             // bytes between rows
    uint32_t voff[IPW];      // per-lane offsets (OOB_OFFSET for rows past the edge)

    __device__ __forceinline__ void init(const char *tile_base, uint32_t ld_bytes, int r_left,
                                         int tid) {
        base = static_cast<const char *>(uniform_ptr(tile_base));
        ld = ld_bytes;
        const int lane = tid & 63, wave = uniform(tid >> 6);
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int row = (wave * IPW + i) * RPI + lane / CH;
            const int c = (lane % CH) ^ swz<CH>(row);
            voff[i] = row < r_left ? row * ld_bytes + (uint32_t)(c << 4) : OOB_OFFSET;
        }
    }

    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int kt) const {
        return make_rsrc(base + (size_t)kt * (CH * 16));
    }

    // Instruction i of this wave for a full k-tile (no K tail).
    __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, int i, char *lds,
                                              int wave) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(lds + (wave * IPW + i) * 1024), 16, voff[i],
            0, 0, LD_POLICY);
    }

    // Copy k-tile kt (k_left valid elements from its start) into `lds`.
    __device__ __forceinline__ void issue(int kt, int k_left, char *lds, int tid) const {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (size_t)kt * (CH * 16));
        const int wave = uniform(tid >> 6);
        if (k_left >= CH * VEC) {
#pragma unroll
            for (int i = 0; i < IPW; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(lds + (wave * IPW + i) * 1024), 16,
                    voff[i], 0, 0, LD_POLICY);
        } else {   // ragged K tail: drop the chunks past K
            const int lane = tid & 63;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int row = (wave * IPW + i) * RPI + lane / CH;
                const int c = (lane % CH) ^ swz<CH>(row);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(lds + (wave * IPW + i) * 1024), 16,
                    c * VEC < k_left ? voff[i] : OOB_OFFSET, 0, 0, LD_POLICY);
            }
        }
    }
};

// ---------------------------------------------------------------- tile engine

// KB: bytes of K per LDS row per k-tile (128 or 64); STAGES: LDS stages
// (more than 2 only when both operands are K-contiguous).
// PIPE: 0 = fragment reads scheduled by the compiler; 3 = the fragments of
// substep s+1 are read (as one burst) before the MFMAs of substep s, with
// scheduling fences; 7 = the register-streamed pipeline (mainloop_rs: one
// wave per SIMD; K-contiguous operands, or 16-bit M-/N-contiguous ones read
// with transposing LDS loads).
// COPY_WAVES: how many waves issue the LDS-DMA copies (0 = all). With half
// of them (one per SIMD), the other wave of every SIMD starts its MFMAs right
// after the barrier while its partner waits on the CU's copy queue, which
// takes ~1100 cycles to accept the 64 KiB of a 256x256 k-tile.
template <int FAM_, bool A_KC, bool B_KC, int BM_, int BN_, int WM_, int WN_, int KB = 128,
          int STAGES = 2, int PIPE = 0, int COPY_WAVES = 0>
struct Tile {
    static constexpr int FAM = FAM_, BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int CH = KB / 16;
    using F = Fam<FAM>;
    using Out = typename F::Out;
    static constexpr int ESZ = F::ESZ, CPL = F::CPL;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int VEC = 16 / ESZ;            // elements per 16-byte chunk
    static constexpr int BK = KB / ESZ;             // elements of K per k-tile
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int SUBSTEPS = CH / (2 * CPL);
    static constexpr bool MX = F::MX;
    static_assert(!MX || (CH == 8 && STAGES == 2 && PIPE == 0),
                  "MX tiles: 128-byte rows (four scale blocks per k-tile), two stages");
    static_assert(PIPE != 7 || ((A_KC || ESZ == 2) && (B_KC || ESZ == 2) && !MX && CH == 8 &&
                                STAGES == 2 && COPY_WAVES == 0),
                  "register-streamed pipeline: K-contiguous or 16-bit operands, 128-byte rows, "
                  "two stages");
    // LDS: [A stage 0 .. A stage S-1 | B stage 0 .. B stage S-1]
    static constexpr int A_BYTES = BM * KB, B_BYTES = BN * KB;
    static constexpr int B_OFF = STAGES * A_BYTES;
    // MX: each stage also holds SCW 32-bit words of E8M0 scales per tile row
    // of A and of B (the k-tile's 4 * SCW blocks; word w of row r at
    // (w * rows + r) * 4, rows padded to whole 64-lane copy instructions).
    static constexpr int SCW = MX ? Fam<FAM>::SCW : 0;
    static constexpr int ROWS_A = (BM + 63) / 64 * 64, ROWS_B = (BN + 63) / 64 * 64;
    static constexpr int SC_A = SCW * ROWS_A * 4;
    static constexpr int SC_B = SCW * ROWS_B * 4;
    static constexpr int SC_OFF = STAGES * (A_BYTES + B_BYTES);
    static constexpr int LDS_BYTES = STAGES * (A_BYTES + B_BYTES + SC_A + SC_B);
    static_assert(CH == 8 || CH == 4, "64- or 128-byte LDS rows");
    static_assert(STAGES == 2 || (A_KC && B_KC), "deep pipelines need direct loads");
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // Workgroups that fit twice in a CU's LDS ask the compiler for two waves
    // per SIMD (at most 256 registers per wave), so two of them can share the
    // CU and hide each other's waits; larger ones run one per CU. Byte-wide
    // operands staged through registers (fp8 with an M- or N-contiguous
    // operand) keep the full register file: their in-register transposes
    // would spill within 256 registers.
    static constexpr int WG_PER_CU =
        ((160 * 1024) / LDS_BYTES >= 2 && ((A_KC && B_KC) || ESZ >= 2)) ? 2 : 1;
    static constexpr int WAVES_PER_EU = WG_PER_CU * (NT / 64) / 4 > 0 ? WG_PER_CU * (NT / 64) / 4 : 1;

    // K-contiguous operands go straight to LDS; the others are staged through
    // registers and transposed.
    using SA = Stager<BM, ESZ, false, NT, CH>;
    using SB = Stager<BN, ESZ, false, NT, CH>;
    static constexpr int COPY_NT = COPY_WAVES > 0 ? 64 * COPY_WAVES : NT;
    static_assert(COPY_NT <= NT && NT % COPY_NT == 0, "copy waves");
    static_assert(COPY_NT == NT || STAGES == 2, "subset copies with the two-stage loop only");
    using DA = DirectStager<BM, ESZ, COPY_NT, CH>;
    using DB = DirectStager<BN, ESZ, COPY_NT, CH>;
    static constexpr int LPS = DA::IPW + DB::IPW;   // direct loads per stage per wave

    struct Acc {
        f32x16 v[FN][FM];
    };

    // MX: copy the k-tile's scale words of the tile's rows of A and B into
    // the stage (LDS DMA, 4 bytes a lane; rows past the edge read as zero).
    // Byte b of a row's word w is the scale of the k-tile's block 4w + b.
    static __device__ __forceinline__ void issue_scales(const Prob &p, int tm, int tn, int kt,
                                                        char *sc, int tid) {
        constexpr int GA = ROWS_A / 64, GB = ROWS_B / 64, CW = COPY_NT / 64;
        constexpr int EPB = FAM == FAM_MXF4 ? 2 : 1;   // elements per operand byte
        const int lane = tid & 63, wave = uniform(tid >> 6);
        const uint32_t nb = (uint32_t)((p.K * EPB) >> 5);   // scale bytes per row
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.mx_a), rb = make_rsrc(p.mx_b);
        for (int q = wave; q < SCW * (GA + GB); q += CW) {
            const int w = q / (GA + GB), qq = q - w * (GA + GB);
            const bool is_a = qq < GA;
            const int row = (is_a ? qq : qq - GA) * 64 + lane;
            const int64_t g_row = is_a ? (int64_t)tm * BM + row : (int64_t)tn * BN + row;
            const bool ok = row < (is_a ? BM : BN) && g_row < (is_a ? p.M : p.N);
            const uint32_t voff = ok ? (uint32_t)g_row * nb : OOB_OFFSET;
            char *dst = sc + (is_a ? 0 : SC_A) + (w * (is_a ? ROWS_A : ROWS_B) + row - lane) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                is_a ? ra : rb, (__attribute__((address_space(3))) void *)dst, 4, voff,
                kt * 4 * SCW + 4 * w, 0, 0);
        }
    }

    static __device__ __forceinline__ void zero(Acc &a) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) a.v[i][j][e] = 0.0f;
    }

    // Element pointers of the operand k-tile origins, and row strides.
    static __device__ __forceinline__ void a_tile(const Prob &p, int tm, int kt, const char *&base,
                                                  uint32_t &ld, int &r_left, int &k_left) {
        const int64_t m0 = (int64_t)tm * BM, k0 = (int64_t)kt * BK;
        if constexpr (A_KC) {   // RowMajor A: [M][K]
            base = p.A + (m0 * p.K + k0) * ESZ;
            ld = (uint32_t)(p.K * ESZ);
        } else {                // ColumnMajor A: [K][M]
            base = p.A + (k0 * p.M + m0) * ESZ;
            ld = (uint32_t)(p.M * ESZ);
        }
        r_left = (int)imin64(p.M - m0, BM);
        k_left = (int)imin64(p.K - k0, BK);
    }
    static __device__ __forceinline__ void b_tile(const Prob &p, int tn, int kt, const char *&base,
                                                  uint32_t &ld, int &r_left, int &k_left) {
        const int64_t n0 = (int64_t)tn * BN, k0 = (int64_t)kt * BK;
        if constexpr (B_KC) {   // ColumnMajor B: [N][K]
            base = p.B + (n0 * p.K + k0) * ESZ;
            ld = (uint32_t)(p.K * ESZ);
        } else {                // RowMajor B: [K][N]
            base = p.B + (k0 * p.N + n0) * ESZ;
            ld = (uint32_t)(p.N * ESZ);
        }
        r_left = (int)imin64(p.N - n0, BN);
        k_left = (int)imin64(p.K - k0, BK);
    }

    // The problem that schedule tile t belongs to (its batch entry's
    // operands) and the tile's coordinates within it.
    static __device__ __forceinline__ Prob tile_problem(const Prob &p, const Sched &s, int t, int &tm,
                                                         int &tn);

    // Per-work-unit copy state: direct stagers for K-contiguous operands,
    // register stagers (with in-register transpose) for the others.
    struct Loader {
        DA da;
        DB db;
        SA sa;
        SB sb;
    };

    static __device__ __forceinline__ void loader_init(const Prob &p, int tm, int tn, Loader &L,
                                                       int tid) {
        const char *base;
        uint32_t ld;
        int rl, kl;
        if constexpr (A_KC) {
            a_tile(p, tm, 0, base, ld, rl, kl);
            L.da.init(base, ld, rl, tid);
        }
        if constexpr (B_KC) {
            b_tile(p, tn, 0, base, ld, rl, kl);
            L.db.init(base, ld, rl, tid);
        }
    }

    // Start the copy of k-tile kt: direct operands are issued into `stage`,
    // transposed operands are fetched into registers (stored by store_regs).
    static __device__ __forceinline__ void issue_stage(const Prob &p, int tm, int tn, int kt,
                                                       int k_left, char *lds, int st, Loader &L,
                                                       int tid) {
        char *stage = lds + st * A_BYTES;   // A of stage st; B of stage st at B_OFF + st * B_BYTES
        const char *base;
        uint32_t ld;
        int rl, kl;
        const bool copy_wave = COPY_NT == NT || uniform(tid >> 6) < COPY_NT / 64;
        if constexpr (MX) {
            if (copy_wave) issue_scales(p, tm, tn, kt, lds + SC_OFF + st * (SC_A + SC_B), tid);
        }
        if constexpr (A_KC) {
            if (copy_wave) L.da.issue(kt, k_left, stage, tid);
        } else {
            a_tile(p, tm, kt, base, ld, rl, kl);
            L.sa.load(base, ld, rl, kl, tid);
        }
        if constexpr (B_KC) {
            if (copy_wave) L.db.issue(kt, k_left, lds + B_OFF + st * B_BYTES, tid);
        } else {
            b_tile(p, tn, kt, base, ld, rl, kl);
            L.sb.load(base, ld, rl, kl, tid);
        }
    }

    static __device__ __forceinline__ void store_regs(char *lds, int st, const Loader &L, int tid) {
        if constexpr (!A_KC) L.sa.store(lds + st * A_BYTES, tid);
        if constexpr (!B_KC) L.sb.store(lds + B_OFF + st * B_BYTES, tid);
    }

    struct Frags {
        u32x4 x[FN][CPL], y[FM][CPL];
    };

    static __device__ __forceinline__ void load_frags(const char *sA, const char *sB, int s, Frags &f,
                                                      int lane, int wm, int wn) {
        const int g = lane >> 5, r = lane & 31;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                f.x[i][c] = *reinterpret_cast<const u32x4 *>(
                    sB + lds_off<CH>(wn * WTN + i * 32 + r, s * 2 * CPL + g * CPL + c));
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                f.y[j][c] = *reinterpret_cast<const u32x4 *>(
                    sA + lds_off<CH>(wm * WTM + j * 32 + r, s * 2 * CPL + g * CPL + c));
    }

    static __device__ __forceinline__ void mma_frags(const Frags &f, Acc &acc) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) F::mma(acc.v[i][j], f.x[i], f.y[j]);
    }

    // Pipelined multiply with scheduling fences: the reads of substep s+1 are
    // issued as one burst, then the MFMAs of substep s; the fence keeps the
    // scheduler from interleaving them back into read -> wait -> MFMA pairs.
    static __device__ __forceinline__ void compute_p3(const char *sA, const char *sB, Acc &acc,
                                                      int lane, int wm, int wn) {
        Frags f[2];
        load_frags(sA, sB, 0, f[0], lane, wm, wn);
#pragma unroll
        for (int s = 0; s < SUBSTEPS; ++s) {
            if (s + 1 < SUBSTEPS) load_frags(sA, sB, s + 1, f[(s + 1) & 1], lane, wm, wn);
            __builtin_amdgcn_sched_barrier(0);
            mma_frags(f[s & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    template <int P>
    static __device__ __forceinline__ void compute_any(const char *sA, const char *sB, Acc &acc,
                                                       int lane, int wm, int wn) {
        if constexpr (P == 3) compute_p3(sA, sB, acc, lane, wm, wn);
        else compute(sA, sB, acc, lane, wm, wn);
    }

    // 16-byte chunk of a 128-byte LDS row that lane group g reads as part c
    // of substep s: contiguous 32-element halves for the unscaled types; for
    // MX the two halves of each hardware scale block (see Fam<FAM_MXF8>).
    static __device__ __forceinline__ int frag_chunk(int s, int g, int c) {
        if constexpr (MX) return s * 2 * CPL + c * 2 + g;
        else return s * 2 * CPL + g * CPL + c;
    }

    // Multiply one LDS stage into the accumulators (MX: with the k-tile's
    // block scales).
    static __device__ __forceinline__ void compute(const char *sA, const char *sB, Acc &acc,
                                                   int lane, int wm, int wn,
                                                   const char *sSc = nullptr) {
        const int g = lane >> 5, r = lane & 31;
        // MX: this lane's scale words, shifted so byte 2(s % 2) of word s / 2
        // is the block 2s + g its lane group multiplies in substep s
        uint32_t scx[SCW > 0 ? SCW : 1][FN], scy[SCW > 0 ? SCW : 1][FM];
        if constexpr (MX) {
#pragma unroll
            for (int w = 0; w < SCW; ++w) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    scx[w][i] = *reinterpret_cast<const uint32_t *>(
                                    sSc + SC_A + (w * ROWS_B + wn * WTN + i * 32 + r) * 4) >>
                                (8 * g);
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    scy[w][j] = *reinterpret_cast<const uint32_t *>(
                                    sSc + (w * ROWS_A + wm * WTM + j * 32 + r) * 4) >>
                                (8 * g);
            }
        }
#pragma unroll
        for (int s = 0; s < SUBSTEPS; ++s) {
            u32x4 xf[FN][CPL], yf[FM][CPL];
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int row = wn * WTN + i * 32 + r;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    xf[i][c] = *reinterpret_cast<const u32x4 *>(
                        sB + lds_off<CH>(row, frag_chunk(s, g, c)));
            }
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int row = wm * WTM + j * 32 + r;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    yf[j][c] = *reinterpret_cast<const u32x4 *>(
                        sA + lds_off<CH>(row, frag_chunk(s, g, c)));
            }
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    if constexpr (MX) {
                        const int w = s / 2 < SCW ? s / 2 : 0;
                        if (s % 2 == 0)
                            F::template mma_mx<0>(acc.v[i][j], xf[i], yf[j], scx[w][i], scy[w][j]);
                        else
                            F::template mma_mx<2>(acc.v[i][j], xf[i], yf[j], scx[w][i], scy[w][j]);
                    } else {
                        F::mma(acc.v[i][j], xf[i], yf[j]);
                    }
                }
        }
    }

    // Wait until at most n k-tiles issued after the one needed are in flight
    // (vmcnt counts this wave's direct loads; LPS per k-tile).
    static __device__ __forceinline__ void wait_tiles_after(int n) {
        if constexpr (STAGES >= 5) {
            if (n >= 3) { wait_vmcnt<3 * LPS>(); return; }
        }
        if constexpr (STAGES >= 4) {
            if (n >= 2) { wait_vmcnt<2 * LPS>(); return; }
        }
        if constexpr (STAGES >= 3) {
            if (n >= 1) { wait_vmcnt<LPS>(); return; }
        }
        wait_vmcnt<0>();
    }

    // acc = sum over the n k-tiles kt0, kt0 + stride, ..., kt0 + (n-1) stride
    // of the tile (tm, tn). Ends with a barrier, so LDS may be reused
    // immediately afterwards.
    static __device__ __forceinline__ void mainloop(const Prob &p, int tm, int tn, int kt0_, int n_,
                                                    int stride_, Acc &acc, char *lds) {
        const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const int kt0 = uniform(kt0_), n = uniform(n_), stride = uniform(stride_);
        if constexpr (PIPE == 7) {
            mainloop_rs(p, tm, tn, kt0, n, stride, acc, lds);
            return;
        }
        zero(acc);
        if (n <= 0) return;
        // valid k of the last k-tile of K (the only one that can be partial)
        const int last = uniform(p.ipt) - 1;
        const int k_tail = uniform((int)(p.K - (int64_t)last * BK));
        auto kvalid = [&](int kt) { return kt == last ? k_tail : BK; };
        Loader L;
        loader_init(p, tm, tn, L, tid);
        if constexpr (STAGES > 2) {
            // Deep pipeline: k-tiles i+1 .. i+STAGES-2 stay in flight while i
            // is multiplied; the stage refilled at iteration i held i-1.
#pragma unroll
            for (int j = 0; j < STAGES - 1; ++j)
                if (j < n) issue_stage(p, tm, tn, kt0 + j * stride, kvalid(kt0 + j * stride), lds, j, L, tid);
            int stage = 0;
            for (int i = 0; i < n; ++i) {
                wait_tiles_after(imin64(STAGES - 2, n - 1 - i));
                barrier_no_fence();
                if (i + STAGES - 1 < n) {
                    const int st = stage == 0 ? STAGES - 1 : stage - 1;
                    const int kt = kt0 + (i + STAGES - 1) * stride;
                    issue_stage(p, tm, tn, kt, kvalid(kt), lds, st, L, tid);
                }
                compute_any<PIPE>(lds + stage * A_BYTES, lds + B_OFF + stage * B_BYTES, acc, lane,
                                  wm, wn);
                stage = stage + 1 == STAGES ? 0 : stage + 1;
            }
        } else {
            issue_stage(p, tm, tn, kt0, kvalid(kt0), lds, 0, L, tid);
            store_regs(lds, 0, L, tid);
            for (int i = 0; i < n; ++i) {
                const int par = i & 1;
                wait_vmcnt<0>();   // this wave's copies of k-tile i landed
                __syncthreads();
                const int kt = kt0 + (i + 1) * stride;
                if (i + 1 < n) issue_stage(p, tm, tn, kt, kvalid(kt), lds, par ^ 1, L, tid);
                if constexpr (MX)
                    compute(lds + par * A_BYTES, lds + B_OFF + par * B_BYTES, acc, lane, wm, wn,
                            lds + SC_OFF + par * (SC_A + SC_B));
                else
                    compute_any<PIPE>(lds + par * A_BYTES, lds + B_OFF + par * B_BYTES, acc, lane,
                                      wm, wn);
                if (i + 1 < n) store_regs(lds, par ^ 1, L, tid);
            }
        }
        __syncthreads();
    }

    // ---- register-streamed pipeline (PIPE == 7) -------------------------------
    //
    // One wave per SIMD (2 x 2 waves of 128 x 128 on the 256 x 256 tile). Each
    // thread streams its 16-byte chunks of every k-tile through registers:
    // chunk u of k-tile t+2 is fetched right after chunk u of k-tile t+1 has
    // been written to LDS, so a whole k-tile of loads is always in flight --
    // the registers are the third buffer that two 64 KiB LDS stages leave no
    // room for -- and no barrier ever waits for the memory pipe to drain.
    // Inside a k-tile, the LDS writes of the next k-tile and the fragment
    // reads of the next substep sit between the MFMAs of the current substep;
    // one barrier, before the last substep, publishes the next k-tile's stage
    // and releases the previous one for the writes that follow.
    static constexpr int RS_UA = BM * CH / NT, RS_UB = BN * CH / NT;   // chunks per thread
    static constexpr int RS_OPS = RS_UA + RS_UB;
    static constexpr int RS_RSTEP = NT / CH;   // rows between one thread's chunks
    // Pipeline shape: RS_DEPTH k-tiles of loads in flight in registers (one
    // register set each); the LDS writes of a k-tile spread over substeps
    // [0, RS_WSUB), which all precede the barrier; the global loads over
    // substeps [0, RS_LSUB), each after the write that frees its registers.
    // (Two on tiles of at most 128 x 128, whose accumulators leave room for
    // a second register set: twice the loads in flight for the short-K and
    // latency-bound shapes these tiles serve.)
    static constexpr int RS_DEPTH = BM * BN <= 128 * 128 ? 2 : 1;
    static constexpr int RS_WSUB = SUBSTEPS - 1;
    static constexpr int RS_LSUB = SUBSTEPS;
    static_assert(RS_DEPTH == 1 || RS_DEPTH == 2, "register stages");
    static_assert(RS_WSUB >= 1 && RS_WSUB <= SUBSTEPS - 1 && RS_LSUB >= 1 && RS_LSUB <= SUBSTEPS,
                  "copy distribution");
    // substep of op o's LDS write and of its global load
    static constexpr int rs_ws(int o) { return o * RS_WSUB / RS_OPS; }
    static constexpr int rs_ls(int o) {
        return o * RS_LSUB / RS_OPS > rs_ws(o) ? o * RS_LSUB / RS_OPS : rs_ws(o);
    }
    static constexpr int rs_count_w(int S) {
        int c = 0;
        for (int o = 0; o < RS_OPS; ++o) c += rs_ws(o) == S;
        return c;
    }
    static constexpr int rs_count_l(int S) {
        int c = 0;
        for (int o = 0; o < RS_OPS; ++o) c += rs_ls(o) == S;
        return c;
    }

    // K-contiguous operand: row r of the tile (an M or N index) holds the
    // k-tile's 128 bytes at lds_off<8>(r, chunk).
    template <int U> struct RsStream {
        const char *base;   // operand element (first row of the tile, k = 0), wave-uniform
        uint32_t voff;      // this lane's byte offset in the tile's first row step
        uint32_t step;      // bytes between a thread's consecutive chunks (32 rows), uniform
        int nval;           // chunks of this thread whose rows lie inside the operand
        int kc;             // first k of this thread's chunks within a k-tile
        uint32_t lo[2];     // LDS byte offsets of chunk 0 and of chunk 1 minus one row step
        u32x4 r[RS_DEPTH][U];

        __device__ __forceinline__ void init(const char *tile_base, uint32_t ld, int r_left, int tid) {
            static_assert(RS_RSTEP == 32, "register stream: 256 threads, 128-byte rows");
            base = static_cast<const char *>(uniform_ptr(tile_base));
            const int row0 = tid >> 3, c = tid & 7;
            voff = (uint32_t)row0 * ld + (uint32_t)(c << 4);
            step = (uint32_t)uniform((int)(ld * RS_RSTEP));
            nval = r_left > row0 ? (r_left - row0 + RS_RSTEP - 1) / RS_RSTEP : 0;
            kc = c * VEC;
            // rows row0 + 32u: the row swizzle repeats with period 2 in u
            lo[0] = lds_off<8>(row0, c);
            lo[1] = lds_off<8>(row0 + RS_RSTEP, c) - RS_RSTEP * KB;
        }
        // byte offset of k-tile kt from the tile's origin
        __device__ __forceinline__ size_t koff(int kt) const { return (size_t)kt * KB; }
        // chunk u of the k-tile whose resource starts at its first byte, into
        // register set Q; kl: valid K elements of that k-tile (0: none). The
        // row step goes in the scalar offset; a lane outside the operand
        // reads zeros (offset past the records).
        template <int Q>
        __device__ __forceinline__ void load(int u, __amdgpu_buffer_rsrc_t rs, int kl) {
            const bool in = (kc < kl) & (u < nval);
            r[Q][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? voff : OOB_OFFSET, u * step,
                                                            LD_POLICY);
        }
        template <int Q> __device__ __forceinline__ void store(int u, char *stage) const {
            *reinterpret_cast<u32x4 *>(stage + lo[u & 1] + u * RS_RSTEP * KB) = r[Q][u];
        }
    };

    // M- or N-contiguous 16-bit operand (ColumnMajor A, RowMajor B): k-row k
    // of a stage holds the tile's BMN elements, its 16-byte chunk c at slot
    // c ^ mn_swz(k). A transposing fragment read covers, per 16 lanes, 32
    // bytes of each of 4 consecutive k-rows (per 32 lanes, 64 bytes of
    // each); the XOR puts those pieces on distinct banks whether the LDS
    // serves 128 or 256 bytes a clock, and keeps each row's chunks a
    // permutation within aligned groups of 16 for the 16-byte writes.
    static __device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 2) | (k & 2); }

    template <int U, int BMN> struct RsStreamMN {
        static constexpr int ROWB = BMN * ESZ, CPR = ROWB / 16, RPU = NT / CPR;
        static_assert(CPR >= 16 && RPU % 4 == 0 && RPU * U == BK, "MN register stream shape");
        const char *base;   // operand element (k = 0, first M/N index of the tile), uniform
        uint32_t voff;      // this lane's byte offset within the k-tile's first k-row step
        uint32_t step;      // bytes between a thread's consecutive chunks (RPU k-rows), uniform
        uint32_t kstep;     // bytes between k-tiles (BK k-rows), uniform
        uint32_t lo;        // LDS byte offset of chunk 0 (the swizzle repeats every 4 k-rows)
        int row0;           // k-row of chunk 0
        u32x4 r[RS_DEPTH][U];

        __device__ __forceinline__ void init(const char *tile_base, uint32_t ld, int mn_left, int tid) {
            base = static_cast<const char *>(uniform_ptr(tile_base));
            row0 = tid / CPR;
            const int c = tid % CPR;
            // a thread whose 8 elements lie outside the operand reads zeros
            voff = c * VEC < mn_left ? (uint32_t)row0 * ld + (uint32_t)(c << 4) : OOB_OFFSET;
            step = (uint32_t)uniform((int)(ld * RPU));
            kstep = (uint32_t)uniform((int)(ld * BK));
            lo = (uint32_t)(row0 * ROWB + ((c ^ mn_swz(row0)) << 4));
        }
        __device__ __forceinline__ size_t koff(int kt) const { return (size_t)kt * kstep; }
        template <int Q>
        __device__ __forceinline__ void load(int u, __amdgpu_buffer_rsrc_t rs, int kl) {
            r[Q][u] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, row0 + u * RPU < kl ? voff : OOB_OFFSET, u * step, LD_POLICY);
        }
        template <int Q> __device__ __forceinline__ void store(int u, char *stage) const {
            *reinterpret_cast<u32x4 *>(stage + lo + u * RPU * ROWB) = r[Q][u];
        }
    };

    // MFMA operand (8 consecutive k of one M/N index per lane, the same k
    // split as the K-contiguous fragments) of the 32 M/N indices from mn0,
    // substep s, read from an MN stage with two transposing loads: of a
    // 16-lane group, lane r fetches 4 elements of k-row r/4, and the load
    // hands lane r element r of the group's 16 columns for each of the 4
    // k-rows (lane layout measured on gfx950).
    template <int BMN>
    static __device__ __forceinline__ u32x4 tr_frag(const char *stage, int mn0, int s, int lane) {
        constexpr int ROWB = BMN * ESZ;
        typedef __attribute__((ext_vector_type(4))) short s16x4;
        const int r = lane & 15, g = lane >> 4;
        const int mn = mn0 + ((g & 1) << 4) + ((r & 3) << 2);
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 8 * frag_chunk(s, g >> 1, 0) + 4 * h + (r >> 2);
            const char *ptr = stage + k * ROWB + ((((mn >> 3) ^ mn_swz(k))) << 4) + ((mn & 7) << 1);
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(ptr));
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            out[2 * h] = w.x;
            out[2 * h + 1] = w.y;
        }
        return out;
    }
    static constexpr int RS_READS = FN * (B_KC ? CPL : 2) + FM * (A_KC ? CPL : 2);

    // fragments of substep s of one stage
    static __device__ __forceinline__ void rs_frags(const char *sA, const char *sB, int s, Frags &f,
                                                    int lane, int wm, int wn) {
        const int g = lane >> 5, r = lane & 31;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            if constexpr (B_KC) {
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    f.x[i][c] = *reinterpret_cast<const u32x4 *>(
                        sB + lds_off<CH>(wn * WTN + i * 32 + r, frag_chunk(s, g, c)));
            } else {
                f.x[i][0] = tr_frag<BN>(sB, wn * WTN + i * 32, s, lane);
            }
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            if constexpr (A_KC) {
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    f.y[j][c] = *reinterpret_cast<const u32x4 *>(
                        sA + lds_off<CH>(wm * WTM + j * 32 + r, frag_chunk(s, g, c)));
            } else {
                f.y[j][0] = tr_frag<BM>(sA, wm * WTM + j * 32, s, lane);
            }
        }
    }

    // Scheduling pattern of one substep: the fragment reads ride on the
    // first MFMAs -- a quarter of the substep's 16 on 128x128 wave tiles
    // (issued early, they have the rest of the substep to land: 2-5 % faster
    // than over the first half, 5-10 % faster than over all of it), the
    // first half of the 4 on 64x64 wave tiles (a quarter measured no
    // better there); the LDS writes and the global loads on the rest (the
    // writes go to the other stage, but the compiler cannot prove that, so
    // they stay behind the reads), spread evenly, so the memory instructions
    // issue in the MFMAs' shadow.
    template <int NREAD, int NW, int NL, int Q = 0, bool MIXOK = true>
    static __device__ __forceinline__ void rs_sched() {
        constexpr int NMMA = FN * FM;
        constexpr int H = NMMA >= 16 ? NMMA / 4 : NMMA / 2;
        if constexpr (Q < NMMA) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            if constexpr (Q < H) {
                constexpr int NR = (Q + 1) * NREAD / H - Q * NREAD / H;
                if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);   // DS read
            } else {
                constexpr int W = NMMA - H, h = Q - H, TOT = NW + NL;
                constexpr int e0 = h * TOT / W, e1 = (h + 1) * TOT / W;
                // 128x128 wave tiles of K-contiguous operands: writes and
                // loads interleaved in proportion (1-2 % faster than all
                // writes first), except in the substep that ends at the
                // barrier, whose writes go first so the wait before the
                // barrier is short (another 1-2 %); otherwise writes first
                // (no gain measured)
                constexpr bool MIX = NMMA >= 16 && A_KC && B_KC && MIXOK;
                constexpr int nw = MIX ? NW * (h + 1) / W - NW * h / W
                                       : (e1 < NW ? e1 : NW) - (e0 < NW ? e0 : NW);
                constexpr int nl = MIX ? NL * (h + 1) / W - NL * h / W : (e1 - e0) - nw;
                if constexpr (nw > 0) __builtin_amdgcn_sched_group_barrier(0x200, nw, 0);   // DS write
                if constexpr (nl > 0) __builtin_amdgcn_sched_group_barrier(0x020, nl, 0);   // VMEM read
            }
            rs_sched<NREAD, NW, NL, Q + 1, MIXOK>();
        }
    }

    static __device__ __forceinline__ void mainloop_rs(const Prob &p, int tm, int tn, int kt0, int n,
                                                       int stride, Acc &acc, char *lds) {
        const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        zero(acc);
        if (n <= 0) return;
        const int last = uniform(p.ipt) - 1;
        const int k_tail = uniform((int)(p.K - (int64_t)last * BK));
        std::conditional_t<A_KC, RsStream<RS_UA>, RsStreamMN<RS_UA, BM>> sa;
        std::conditional_t<B_KC, RsStream<RS_UB>, RsStreamMN<RS_UB, BN>> sb;
        {
            const char *base;
            uint32_t ld;
            int rl, kl;
            a_tile(p, tm, 0, base, ld, rl, kl);
            sa.init(base, ld, rl, tid);
            b_tile(p, tn, 0, base, ld, rl, kl);
            sb.init(base, ld, rl, tid);
        }
        // valid K elements of k-tile j of this work unit (j >= n: none; every
        // chunk reads zeros)
        auto kin = [&](int j) {
            const int kt = kt0 + j * stride;
            return j < n ? (kt == last ? k_tail : BK) : 0;
        };
        auto ktile = [&](int j) { return kt0 + (j < n ? j : 0) * stride; };
        // every chunk of k-tile j into register set Q
        auto load_all = [&](auto qc, int j) {
            constexpr int Q = decltype(qc)::value;
            const int k = kin(j);
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(sa.base + sa.koff(ktile(j)));
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(sb.base + sb.koff(ktile(j)));
#pragma unroll
            for (int u = 0; u < RS_UA; ++u) sa.template load<Q>(u, ra, k);
#pragma unroll
            for (int u = 0; u < RS_UB; ++u) sb.template load<Q>(u, rb, k);
        };
        constexpr int Q1 = RS_DEPTH == 2 ? 1 : 0;   // register set of k-tile 1

        // prologue: k-tile 0 into stage 0; k-tiles 1 .. RS_DEPTH into registers
        load_all(std::integral_constant<int, 0>{}, 0);
#pragma unroll
        for (int u = 0; u < RS_UA; ++u) sa.template store<0>(u, lds);
#pragma unroll
        for (int u = 0; u < RS_UB; ++u) sb.template store<0>(u, lds + B_OFF);
        load_all(std::integral_constant<int, Q1>{}, 1);
        if constexpr (RS_DEPTH == 2) load_all(std::integral_constant<int, 0>{}, 2);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes done
        barrier_no_fence();

        Frags f[2];
        rs_frags(lds, lds + B_OFF, 0, f[0], lane, wm, wn);
        // iteration i: multiply k-tile i (stage P = i & 1); write k-tile i+1
        // from its register set into stage P^1 and refill that set with
        // k-tile i+1+RS_DEPTH
        auto iteration = [&](auto pc, int i) {
            constexpr int P = decltype(pc)::value;
            constexpr int Q = RS_DEPTH == 2 ? (P ^ 1) : 0;   // register set of k-tile i+1
            const char *rA = lds + P * A_BYTES, *rB = lds + B_OFF + P * B_BYTES;
            char *wA = lds + (P ^ 1) * A_BYTES, *wB = lds + B_OFF + (P ^ 1) * B_BYTES;
            const int jn = i + 1 + RS_DEPTH;
            const int kn = kin(jn);
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(sa.base + sa.koff(ktile(jn)));
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(sb.base + sb.koff(ktile(jn)));
            auto substep = [&](auto sc) {
                constexpr int S = decltype(sc)::value;
                // fragments for the next substep: this stage, or (after the
                // barrier) the next k-tile's substep 0 from the other stage
                if constexpr (S + 1 < SUBSTEPS) rs_frags(rA, rB, S + 1, f[(S + 1) & 1], lane, wm, wn);
                else rs_frags(wA, wB, 0, f[0], lane, wm, wn);
                mma_frags(f[S & 1], acc);
#pragma unroll
                for (int o = 0; o < RS_OPS; ++o) {
                    if (rs_ws(o) != S) continue;
                    if (o < RS_UA) sa.template store<Q>(o, wA);
                    else sb.template store<Q>(o - RS_UA, wB);
                }
#pragma unroll
                for (int o = 0; o < RS_OPS; ++o) {
                    if (rs_ls(o) != S) continue;
                    if (o < RS_UA) sa.template load<Q>(o, ra, kn);
                    else sb.template load<Q>(o - RS_UA, rb, kn);
                }
                rs_sched<RS_READS, rs_count_w(S), rs_count_l(S), 0, S != SUBSTEPS - 2>();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (S == SUBSTEPS - 2) {
                    // this wave's writes of k-tile i+1 and reads of k-tile i
                    // are done; after the barrier everyone's are
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    barrier_no_fence();
                }
            };
            static_assert(SUBSTEPS == 2 || SUBSTEPS == 4, "substeps per k-tile");
            substep(std::integral_constant<int, 0>{});
            substep(std::integral_constant<int, 1>{});
            if constexpr (SUBSTEPS == 4) {
                substep(std::integral_constant<int, 2>{});
                substep(std::integral_constant<int, 3>{});
            }
        };
        // k-tiles in pairs (the stages, and with two register sets the sets,
        // alternate). With two sets the second iteration is unconditional:
        // a conditional one makes the compiler's wait counts for the other
        // set conservative (one set of loads in flight instead of two); an
        // odd count then ends with one iteration past the last k-tile, whose
        // stage holds zeros (its loads read past K), leaving acc unchanged.
        for (int i = 0; i < n; i += 2) {
            iteration(std::integral_constant<int, 0>{}, i);
            if (RS_DEPTH == 2 || i + 1 < n) iteration(std::integral_constant<int, 1>{}, i + 1);
        }
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
    //
    // v = alpha' * acc + beta * C (C not read when beta == 0) + bias[n],
    // alpha' = alpha times the per-tensor scales; then the activation; one
    // round-to-nearest-even conversion into the output type.

    static __device__ __forceinline__ float eff_alpha(const EpiArgs &e) {
        float a = e.alpha;
        if (e.scale_a) a *= *e.scale_a;
        if (e.scale_b) a *= *e.scale_b;
        return a;
    }

    // Interior tile, RowMajor C/D with 4-element vector access: every lane
    // owns four consecutive n of one m for each (i, j, q).
    // Four consecutive elements of an output-typed vector as floats.
    static __device__ __forceinline__ void load4(const Out *src, int64_t idx, float (&v)[4]) {
        if constexpr (sizeof(Out) == 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(src + idx);
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) v[t4] = t[t4];
        } else {
            const u32x2 t = *reinterpret_cast<const u32x2 *>(src + idx);
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
                v[t4] = (float)__builtin_bit_cast(Out, (uint16_t)(t[t4 >> 1] >> (16 * (t4 & 1))));
        }
    }

    // Four floats to consecutive output-typed elements (one RNE conversion).
    static __device__ __forceinline__ void store4(Out *dst, int64_t idx, const float (&v)[4]) {
        if constexpr (sizeof(Out) == 4) {
            *reinterpret_cast<f32x4 *>(dst + idx) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
            u32x2 t;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                t[h] = (uint32_t)__builtin_bit_cast(uint16_t, (Out)v[2 * h]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (Out)v[2 * h + 1]) << 16);
            *reinterpret_cast<u32x2 *>(dst + idx) = t;
        }
    }

    // The finished output tile can be staged through the (idle) LDS and
    // written back as whole rows: OROW bytes per tile row, the 16-byte chunk
    // k of row r at chunk k ^ (r & 15) -- the per-lane 4-element writes (two
    // or four rows of one chunk column per bank window) and the row-wise
    // 16-byte reads are both free of bank conflicts.
    static constexpr int OSZ = (int)sizeof(Out);
    static constexpr int OROW = BN * OSZ;
    static constexpr int OCPR = OROW / 16;   // 16-byte chunks per tile row
    static constexpr bool STAGE_OUT = BM * OROW <= LDS_BYTES && OCPR >= 16 && (BM * OCPR) % NT == 0;
    static __device__ __forceinline__ uint32_t out_off(int r, int cbyte) {
        return (uint32_t)(r * OROW + ((((cbyte >> 4) ^ (r & 15))) << 4) + (cbyte & 15));
    }

    // Four floats to LDS as output-typed elements (one RNE conversion).
    static __device__ __forceinline__ void store4_lds(char *lds, uint32_t off, const float (&v)[4]) {
        if constexpr (sizeof(Out) == 4) {
            *reinterpret_cast<f32x4 *>(lds + off) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
            u32x2 t;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                t[h] = (uint32_t)__builtin_bit_cast(uint16_t, (Out)v[2 * h]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (Out)v[2 * h + 1]) << 16);
            *reinterpret_cast<u32x2 *>(lds + off) = t;
        }
    }

    // Interior tile, RowMajor D, beta = 0, no bias or auxiliary tensor, a
    // linear or ReLU epilogue, the output tile fitting the LDS: v =
    // act(alpha acc) per lane (four
    // consecutive n of one m for each (i, j, q)) into the LDS (idle on
    // entry), which the workgroup then writes back as whole rows with
    // 16-byte stores (D 16-byte aligned, rows a multiple of 16 bytes): the
    // common case, kept small; the other cases take epi_aux or epi_slow.
    static __device__ __forceinline__ void epi_fast(const Prob &p, const EpiArgs &e, float alpha,
                                                    int64_t m_base, int64_t n_base, const Acc &acc,
                                                    char *lds, int tm, int tn) {
        // LINEAR or RELU only, as a select (a switch per element would put
        // every element behind its own branches); relu(NaN) = relu(-0) = +0
        const bool relu = e.act == ACT_RELU;
        // the per-lane LDS offsets below depend on the lane only; an opaque
        // copy of the thread index keeps the compiler from hoisting all of
        // them out of the persistent tile loop, where they would stay live
        // (64 registers) through every main loop
        const int tid = opaque_tid();
        const int lane = tid & 63, wave = tid >> 6;
        // tile-local row / column of this lane's first group
        const int r_loc = (wave / WN) * WTM + (lane & 31), c_loc = (wave % WN) * WTN + (lane >> 5) * 4;
        // alpha = 1 with no activation (the plain GEMM): conversion only;
        // the choice is made once per tile, not per element
        auto to_lds = [&](auto plain_c) {
            constexpr bool PLAIN = decltype(plain_c)::value;
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        float v[4];
#pragma unroll
                        for (int t4 = 0; t4 < 4; ++t4) {
                            if constexpr (PLAIN) {
                                v[t4] = acc.v[i][j][q * 4 + t4];
                            } else {
                                const float x = alpha * acc.v[i][j][q * 4 + t4];
                                v[t4] = (relu && !(x > 0.0f)) ? 0.0f : x;
                            }
                        }
                        store4_lds(lds, out_off(r_loc + j * 32, (c_loc + i * 32 + q * 8) * OSZ), v);
                    }
        };
        if (!relu && alpha == 1.0f) to_lds(std::true_type{});
        else to_lds(std::false_type{});
        __syncthreads();
        char *Dt = p.D + ((int64_t)tm * BM * p.N + (int64_t)tn * BN) * OSZ;
        const int64_t ld = p.N * OSZ;
        // streaming (non-temporal) stores when the tile's rows stay within
        // 32-bit buffer offsets: D is not read again by this kernel
        if ((int64_t)BM * ld < 0x7FFF0000LL) {
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(Dt);
            const uint32_t ld32 = (uint32_t)ld;
#pragma unroll 8
            for (int it = 0; it < BM * OCPR / NT; ++it) {
                const int c = tid + it * NT;
                const int r = c / OCPR, k = c - (c / OCPR) * OCPR;
                const u32x4 val = *reinterpret_cast<const u32x4 *>(lds + out_off(r, k * 16));
                __builtin_amdgcn_raw_buffer_store_b128(val, rd, (uint32_t)r * ld32 + (uint32_t)(k * 16),
                                                       0, ST_POLICY);
            }
        } else {
#pragma unroll 8
            for (int it = 0; it < BM * OCPR / NT; ++it) {
                const int c = tid + it * NT;
                const int r = c / OCPR, k = c - (c / OCPR) * OCPR;
                const u32x4 val = *reinterpret_cast<const u32x4 *>(lds + out_off(r, k * 16));
                *reinterpret_cast<u32x4 *>(Dt + r * ld + k * 16) = val;
            }
        }
        __syncthreads();
    }

    // Interior tile with C, bias or auxiliary tensors: the same vector
    // accesses as epi_fast (X read like C, Z written like D). The
    // accumulators of fragment rows j0 .. j0+jc-1 arrive through the idle LDS:
    // group ((jj * FN + i) * 4 + q) of thread tid at vals[group * NT + tid].
    static __device__ __forceinline__ void epi_aux(const Prob &p, const EpiArgs &e, float alpha,
                                                   int64_t m_base, int64_t n_base, const f32x4 *vals,
                                                   int j0, int jc) {
        Out *D = reinterpret_cast<Out *>(p.D);
        const Out *C = reinterpret_cast<const Out *>(p.C);
        const Out *bias = reinterpret_cast<const Out *>(e.bias);
        const Out *X = reinterpret_cast<const Out *>(e.aux);
        Out *Z = reinterpret_cast<Out *>(e.aux_out);
        const bool pre = X && !e.aux_after, post = X && e.aux_after;
        const int tid = threadIdx.x;
        for (int jj = 0; jj < jc; ++jj) {
            const int64_t row = (m_base + (j0 + jj) * 32) * p.N;
            for (int i = 0; i < FN; ++i) {
                // the loads of a column block's four groups first, so they
                // are in flight together (one at a time, each waited for,
                // this epilogue cost ~130 us per 256 x 256 tile)
                float c[4][4] = {}, b[4][4] = {}, x[4][4] = {};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = n_base + i * 32 + q * 8;
                    if (e.beta != 0.0f) load4(C, row + col, c[q]);
                    if (bias) load4(bias, col, b[q]);
                    if (X) load4(X, row + col, x[q]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t idx = row + n_base + i * 32 + q * 8;
                    float v[4], z[4];
                    const f32x4 a = vals[((jj * FN + i) * 4 + q) * NT + tid];
#pragma unroll
                    for (int t4 = 0; t4 < 4; ++t4) {
                        const float lin = __builtin_fmaf(alpha, a[t4], e.beta * c[q][t4]) + b[q][t4];
                        v[t4] = finish_aux_branch(lin, x[q][t4], e.aux_op, e.act, pre, post, z[t4]);
                    }
                    if (Z) store4(Z, idx, z);
                    store4(D, idx, v);
                }
            }
        }
    }
    // Fragment rows per LDS hand-off to epi_aux: as many as the tile's LDS holds.
    static constexpr int AUX_JC_FIT = LDS_BYTES / (NT * FN * 4 * 16);
    static constexpr int AUX_JC = AUX_JC_FIT >= FM ? FM : AUX_JC_FIT;
    static_assert(AUX_JC >= 1 && FM % AUX_JC == 0, "LDS hand-off of the auxiliary epilogue");

    // Edge tiles, ColumnMajor C/D or unaligned C/D: element by element, with
    // the accumulators of fragment rows j0 .. j0+jc-1 handed over through the
    // idle LDS exactly as for epi_aux (no private scratch array).
    static __device__ __forceinline__ void epi_slow(const Prob &p, const EpiArgs &e, float alpha,
                                                    int64_t m_base, int64_t n_base, const f32x4 *vals,
                                                    int j0, int jc) {
        Out *D = reinterpret_cast<Out *>(p.D);
        const Out *C = reinterpret_cast<const Out *>(p.C);
        const int tid = threadIdx.x;
        for (int jj = 0; jj < jc; ++jj) {
            const int64_t m = m_base + (j0 + jj) * 32;
            if (m >= p.M) continue;
            for (int i = 0; i < FN; ++i)
                for (int q = 0; q < 4; ++q) {
                    const f32x4 a4 = vals[((jj * FN + i) * 4 + q) * NT + tid];
                    for (int t4 = 0; t4 < 4; ++t4) {
                        const int64_t n = n_base + i * 32 + q * 8 + t4;
                        if (n >= p.N) continue;
                        const int64_t idx = e.lc_row ? m * p.N + n : m + n * p.M;
                        const float a = a4[t4];
                        float v = alpha * a;
                        if (e.beta != 0.0f) v = __builtin_fmaf(alpha, a, e.beta * (float)C[idx]);
                        if (e.bias) v += (float)reinterpret_cast<const Out *>(e.bias)[n];
                        const float x =
                            e.aux ? (float)reinterpret_cast<const Out *>(e.aux)[idx] : 0.0f;
                        float z;
                        D[idx] = (Out)finish_aux_branch(v, x, e.aux_op, e.act,
                                                        e.aux && !e.aux_after,
                                                        e.aux && e.aux_after, z);
                        if (e.aux_out) reinterpret_cast<Out *>(e.aux_out)[idx] = (Out)z;
                    }
                }
        }
    }
    // `lds`: the tile's LDS, idle here (the main loop ends with a barrier);
    // every path but the interior vector one hands the accumulators over
    // through it and closes with a barrier before the next tile's copies may
    // land.
    static __device__ __forceinline__ void epilogue(const Prob &p, const EpiArgs &e, int tm, int tn,
                                                    const Acc &acc, char *lds) {
        const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const float alpha = eff_alpha(e);
        const int64_t m_base = (int64_t)tm * BM + wm * WTM + (lane & 31);
        const int64_t n_base = (int64_t)tn * BN + wn * WTN + (lane >> 5) * 4;
        const bool interior = e.lc_row && p.vec_cd && (int64_t)(tm + 1) * BM <= p.M &&
                              (int64_t)(tn + 1) * BN <= p.N;
        if constexpr (STAGE_OUT) {
            if (interior && !e.aux && !e.aux_out && !e.bias && e.beta == 0.0f &&
                (e.act == ACT_LINEAR || e.act == ACT_RELU) &&
                (reinterpret_cast<uintptr_t>(p.D) & 15) == 0 && ((p.N * OSZ) & 15) == 0) {
                epi_fast(p, e, alpha, m_base, n_base, acc, lds, tm, tn);
                return;
            }
        }
        f32x4 *buf = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
        for (int j0 = 0; j0 < FM; j0 += AUX_JC) {
            // each thread reads back only its own slots: no barrier between
#pragma unroll
            for (int jj = 0; jj < AUX_JC; ++jj)
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        buf[((jj * FN + i) * 4 + q) * NT + tid] =
                            f32x4{acc.v[i][j0 + jj][q * 4], acc.v[i][j0 + jj][q * 4 + 1],
                                  acc.v[i][j0 + jj][q * 4 + 2], acc.v[i][j0 + jj][q * 4 + 3]};
            // inline: an out-of-line call made the kernel save and restore
            // its live accumulators through scratch around every call
            // (256x256 layer GEMMs +2.4 %, 64-problem grouped +2.7 %)
            if (interior) epi_aux(p, e, alpha, m_base, n_base, buf, j0, AUX_JC);
            else epi_slow(p, e, alpha, m_base, n_base, buf, j0, AUX_JC);
        }
        __syncthreads();
    }

    // ---- stream-K partial tiles ---------------------------------------------
    //
    // Partials are written and read with device-scope (sc1) buffer accesses,
    // which stay coherent across the XCDs' private L2s; no L2 write-back or
    // invalidate (what a __threadfence() costs) is needed.

    static constexpr int SC1 = 16;   // cache-policy bit: device scope


    // A partial tile is stored group-major (16-byte group g of thread tid at
    // (g * NT + tid) * 16). Lanes whose M row lies past the problem (rows
    // mrows .. BM-1 of an edge tile, e.g. all but 16 of a 64-row tile for a
    // 16-token decode GEMM) neither store nor load their groups: their lane
    // offset is out of the buffer's range, so the hardware drops the store
    // and returns zeros to the load, and the epilogue never writes those rows.
    static __device__ __forceinline__ uint32_t part_voff(int j, int mrows) {
        const int tid = threadIdx.x, wave = tid >> 6, wm = wave / WN;
        return wm * WTM + j * 32 + (tid & 31) < mrows ? (uint32_t)(tid * 16) : OOB_OFFSET;
    }
    static __device__ __forceinline__ void store_partial(float *slot, const Acc &acc, int mrows) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const uint32_t vo = part_voff(j, mrows);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int grp = (i * FM + j) * 4 + q;
                    const f32x4 t{acc.v[i][j][q * 4], acc.v[i][j][q * 4 + 1], acc.v[i][j][q * 4 + 2],
                                  acc.v[i][j][q * 4 + 3]};
                    // the group's offset in the scalar offset: one lane
                    // offset for all groups instead of one register each
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), rs, vo,
                                                           grp * NT * 16, SC1);
                }
        }
    }

    // acc = sum of the partials slot(0) .. slot(n-1), added in that order.
    // Small accumulators fetch several partials per round (four for at most
    // two fragments, two for at most four), cutting the number of dependent
    // load round trips (the sum and its rounding are unchanged).
    static constexpr int FIXUP_BATCH = FN * FM <= 2 ? 4 : FN * FM <= 4 ? 2 : 1;
    static constexpr bool PAIRED_FIXUP = FIXUP_BATCH > 1;

    static __device__ __forceinline__ void load_partial(const float *slot, f32x4 (&t)[FN * FM * 4],
                                                        int mrows) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot);
#pragma unroll
        for (int g = 0; g < FN * FM * 4; ++g)
            t[g] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, part_voff((g >> 2) % FM, mrows),
                                                             g * NT * 16, SC1));
    }
    static __device__ __forceinline__ void accumulate(const f32x4 (&t)[FN * FM * 4], Acc &acc, bool first) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = t[(i * FM + j) * 4 + q][e];
                        acc.v[i][j][q * 4 + e] = first ? v : acc.v[i][j][q * 4 + e] + v;
                    }
    }

    template <class SlotFn>
    static __device__ __forceinline__ void add_partials(SlotFn slot, int n, Acc &acc, int mrows) {
        if constexpr (PAIRED_FIXUP) {
            constexpr int R = FIXUP_BATCH;
            int u = 0;
            for (; u + R - 1 < n; u += R) {
                f32x4 t[R][FN * FM * 4];
#pragma unroll
                for (int b = 0; b < R; ++b) load_partial(slot(u + b), t[b], mrows);
#pragma unroll
                for (int b = 0; b < R; ++b) accumulate(t[b], acc, u + b == 0);
            }
            if (u < n) {   // the last 1 .. R-1 partials, also in one round
                const int rem = n - u;
                f32x4 t[R - 1][FN * FM * 4];
#pragma unroll
                for (int b = 0; b < R - 1; ++b)
                    if (b < rem) load_partial(slot(u + b), t[b], mrows);
#pragma unroll
                for (int b = 0; b < R - 1; ++b)
                    if (b < rem) accumulate(t[b], acc, u + b == 0);
            }
        } else {
            for (int u = 0; u < n; ++u) add_partial(slot(u), acc, u == 0, mrows);
        }
    }

    // One partial added into acc, its 16-byte groups fetched eight at a time
    // (eight device-scope loads in flight per round trip instead of one).
    static __device__ __forceinline__ void add_partial(const float *slot, Acc &acc, bool first,
                                                       int mrows) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot);
        constexpr int NG = FN * FM * 4, CHUNK = 8;
        static_assert(NG % CHUNK == 0, "partial groups");
#pragma unroll
        for (int g0 = 0; g0 < NG; g0 += CHUNK) {
            f32x4 t[CHUNK];
#pragma unroll
            for (int c = 0; c < CHUNK; ++c)
                t[c] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rs, part_voff(((g0 + c) >> 2) % FM, mrows), (g0 + c) * NT * 16, SC1));
#pragma unroll
            for (int c = 0; c < CHUNK; ++c) {
                const int grp = g0 + c, q = grp & 3, ij = grp >> 2, i = ij / FM, j = ij % FM;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc.v[i][j][q * 4 + e] = first ? t[c][e] : acc.v[i][j][q * 4 + e] + t[c][e];
            }
        }
    }
};

// ---------------------------------------------------------------- schedules

// Raster order of output tiles: groups of `group_m` tile rows, column-major
// inside a group, so consecutive schedule indices form compact 2-D blocks
// that share A and B panels in L2.
__device__ __forceinline__ void tile_coords(int s, int tiles_m, int tiles_n, int group_m, int &tm,
                                            int &tn) {
    const int per_group = group_m * tiles_n;
    const int grp = s / per_group;
    const int first_m = grp * group_m;
    const int gm = min(group_m, tiles_m - first_m);
    const int local = s - grp * per_group;
    tm = first_m + local % gm;
    tn = local / gm;
}

// Workgroups are dealt to the 8 XCDs round robin; give the 32 (or G/8)
// workgroups of one XCD consecutive virtual ids so they work on neighbouring
// tiles and share that XCD's L2.
__device__ __forceinline__ int virtual_id(int w, int grid, int remap) {
    if (!remap || (grid & 7)) return w;
    return (w & 7) * (grid >> 3) + (w >> 3);
}

// Virtual workgroup whose stream-K range holds iteration x:
// ranges are [floor(v T / G), floor((v+1) T / G)).
__device__ __forceinline__ int sk_owner(int64_t x, int64_t T, int G) {
    return (int)(((x + 1) * G + T - 1) / T) - 1;
}

// Tiles per chunk of a per-XCD queue. Small enough that the costly tiles at
// the head of a grouped list spread over the eight XCDs (the XCD that drew
// one chunk more of them finished last with chunks of grid / 8 = 64 tiles:
// 64-problem fp16 mix 362-369 -> 348-354 us with 16, same box), large enough
// for four raster columns of neighbouring tiles.
constexpr int QUEUE_CHUNK = 16;
// Queues of a launch: one per XCD with the remap and a grid of whole XCDs.
__device__ __forceinline__ int queue_count(const Sched &s) {
    return s.xcd_remap && (s.grid & 7) == 0 ? 8 : 1;
}
// The tile after `claim` (the queue's count before this workgroup's claim),
// handed to every thread of the workgroup through the first word of the idle
// LDS: the first barrier waits for the waves still reading the LDS (output
// staging), the last keeps the next copy into LDS from overwriting the word
// before every wave has read it. total_tiles when the queue is exhausted.
__device__ __forceinline__ int queue_next(unsigned int claim, const Sched &s, char *lds) {
    int *slot = reinterpret_cast<int *>(lds);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nq = queue_count(s), chunk = nq == 8 ? QUEUE_CHUNK : s.grid;
        const int x = nq == 8 ? (int)(blockIdx.x & 7) : 0;
        const int64_t t = s.grid + ((int64_t)(claim / chunk) * nq + x) * chunk + claim % chunk;
        *slot = t < s.total_tiles ? (int)t : s.total_tiles;
    }
    __syncthreads();
    const int t = *slot;
    __syncthreads();
    return t;
}

// Count this workgroup's arrival at `counter` (after its partial is stored);
// true in every thread of the workgroup that arrives last, i.e. sees
// `expected` earlier arrivals. The flag passes through the first word of the
// (idle) LDS, so it costs no LDS of its own; the closing barrier keeps the
// next copy into LDS from overwriting it before every wave has read it.
__device__ __forceinline__ bool arrive_last(int *counter, int expected, char *lds) {
    int *flag = reinterpret_cast<int *>(lds);
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = old == expected;
    }
    __syncthreads();
    const bool last = *flag != 0;
    __syncthreads();
    return last;
}

template <int FAM_, bool A_KC, bool B_KC, int BM_, int BN_, int WM_, int WN_, int KB, int STAGES,
          int PIPE, int COPY_WAVES>
__device__ __forceinline__ Prob
Tile<FAM_, A_KC, B_KC, BM_, BN_, WM_, WN_, KB, STAGES, PIPE, COPY_WAVES>::tile_problem(
    const Prob &p, const Sched &s, int t, int &tm, int &tn) {
    if (s.gcount > 0) {
        int lo = 0, hi = s.gcount - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s.gdesc[mid].tile_start <= t) lo = mid;
            else hi = mid - 1;
        }
        lo = uniform(lo);
        const Prob q = s.gdesc[lo].p;
        tile_coords(t - s.gdesc[lo].tile_start, q.tiles_m, q.tiles_n, s.group_m, tm, tn);
        return q;
    }
    if (p.batch <= 1) {
        tile_coords(t, p.tiles_m, p.tiles_n, s.group_m, tm, tn);
        return p;
    }
    const int per = p.tiles_m * p.tiles_n;
    const int b = t / per;
    tile_coords(t - b * per, p.tiles_m, p.tiles_n, s.group_m, tm, tn);
    Prob q = p;
    q.A = p.A + (size_t)(b * p.stride_a) * ESZ;
    q.B = p.B + (size_t)(b * p.stride_b) * ESZ;
    if (p.C) q.C = p.C + (size_t)(b * p.stride_c) * sizeof(Out);
    q.D = p.D + (size_t)(b * p.stride_d) * sizeof(Out);
    return q;
}

// One workgroup's work, as a sequence of units (a tile and a range of its
// k-tiles): the split-K unit, or the stream-K segments, then the
// data-parallel tiles. The kernel has a single main-loop and a single
// epilogue call site, which keeps its code and register allocation to one
// copy of each.
template <class TL>
__global__ void __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::WAVES_PER_EU)))
gemm_persistent(KArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[TL::LDS_BYTES];
    const Prob &p = a.p;
    const Sched &s = a.s;
    const int v = uniform(virtual_id(blockIdx.x, s.grid, s.xcd_remap));
    const size_t slot_elems = (size_t)TL::BM * TL::BN;
    typename TL::Acc acc;

    // stream-K range of this workgroup (empty unless v < sk_grid)
    const bool sk = s.split == 0 && s.sk_tiles > 0 && p.ipt > 0 && v < s.sk_grid;
    const int64_t T = s.sk_iters;
    const int G = s.sk_grid;
    int64_t it = sk ? (int64_t)v * T / G : 0;
    const int64_t end = sk ? (int64_t)(v + 1) * T / G : 0;
    const int first_tile = sk ? (int)(it / p.ipt) : 0;
    // split-K: this workgroup's single unit, if any
    const int S = s.split;
    bool split_pending = S > 0 && v < s.sk_tiles * S;
    int dp_t = S > 0 ? s.total_tiles : s.sk_tiles + v;
    const bool dyn = s.queue != nullptr;

    for (;;) {
        int t, kt0, n, stride;
        int mode;   // 0: whole tile, 1: stream-K segment, 2: split-K unit
        int c = 0, k1 = 0;
        if (split_pending) {
            split_pending = false;
            t = v / S;
            c = v - t * S;
            kt0 = c;
            n = (p.ipt - c + S - 1) / S;
            stride = S;
            mode = S == 1 ? 0 : 2;
        } else if (it < end) {
            t = (int)(it / p.ipt);
            const int64_t tile_it0 = (int64_t)t * p.ipt;
            kt0 = (int)(it - tile_it0);
            k1 = (int)(imin64(end, tile_it0 + p.ipt) - tile_it0);
            n = k1 - kt0;
            stride = 1;
            mode = (kt0 == 0 && k1 == p.ipt) ? 0 : 1;
            it = tile_it0 + k1;
        } else if (dp_t < s.total_tiles) {
            t = dp_t;
            dp_t = dyn ? s.total_tiles : dp_t + s.grid;
            kt0 = 0;
            n = -1;   // every k-tile of the tile's problem
            stride = 1;
            mode = 0;
        } else {
            break;
        }
        t = uniform(t);
        mode = uniform(mode);
        int tm, tn;
        const Prob pt = TL::tile_problem(p, s, t, tm, tn);
        if (n < 0) n = pt.ipt;
        TL::mainloop(pt, tm, tn, kt0, n, stride, acc, lds);
        // claim the next tile now; its number is needed only after the
        // epilogue, whose stores hide the atomic's round trip
        unsigned int claim = 0;
        if (dyn && threadIdx.x == 0)
            claim = __hip_atomic_fetch_add(s.queue + (queue_count(s) == 8 ? (blockIdx.x & 7) : 0), 1u,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool finish = mode == 0;
        int v0 = 0, v1 = 0;
        if (mode != 0) {
            // every contributor publishes its partial; the last to arrive
            // sums all of them in contributor order (deterministic)
            const int my_slot = mode == 2 ? v : 2 * v + (t == first_tile ? 0 : 1);
            const int mrows = (int)imin64(pt.M - (int64_t)tm * TL::BM, TL::BM);
            TL::store_partial(s.partials + (size_t)my_slot * slot_elems, acc, mrows);
            wait_vmcnt<0>();   // this thread's device-scope stores are complete
            __syncthreads();   // ... and every thread's, before the arrival is counted
            if (mode == 2) {
                v1 = S - 1;
            } else {
                const int64_t tile_it0 = (int64_t)t * p.ipt;
                v0 = sk_owner(tile_it0, T, G);
                v1 = sk_owner(tile_it0 + p.ipt - 1, T, G);
            }
            finish = arrive_last(&s.counters[t], v1 - v0, lds);
            if (finish) {
                TL::add_partials(
                    [&](int k) {
                        if (mode == 2) return s.partials + ((size_t)t * S + k) * slot_elems;
                        const int u = v0 + k;
                        const int ft = (int)(((int64_t)u * T / G) / p.ipt);
                        return s.partials + (size_t)(2 * u + (t == ft ? 0 : 1)) * slot_elems;
                    },
                    v1 - v0 + 1, acc, mrows);
            }
        }
        if (finish) {
            TL::epilogue(pt, a.e, tm, tn, acc, lds);
            if (mode != 0 && threadIdx.x == 0)
                __hip_atomic_store(&s.counters[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (mode != 0) __syncthreads();
        if (dyn) dp_t = queue_next(claim, s, lds);
    }
    if (dyn && threadIdx.x == 0) {
        // every claim of this workgroup has been made (its last one came back
        // past the end); the last workgroup to get here resets the queue
        const unsigned int done =
            __hip_atomic_fetch_add(s.queue + 8, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned int)s.grid - 1) {
            for (int q = 0; q < 9; ++q)
                __hip_atomic_store(s.queue + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace mg
