// kernels_wholek.hip -- whole-K GEMM for small problems.
//
// D = epi(alpha*A*B + beta*C) with an fp32 accumulator ("CUTLASS Python接口"
// section 3.3), for problems too small to fill the GPU with output tiles
// (a 1024^3 GEMM is 64 tiles of 128x128 for 256 CUs; 128x64x256 is one) and
// with a short K. Each workgroup owns a 32x32 block of D; its four waves take
// a quarter of K each, and every wave issues all the loads of its quarter at
// once, straight into the MFMA operand registers (no LDS staging), so a
// block costs one memory round trip instead of one per k-tile. The four
// partial blocks meet in LDS and are added in wave order (deterministic),
// then one fused epilogue pass (alpha / scales, beta*C, bias, auxiliary op,
// activation) writes D.
//
// K positions: lane (r, h) = (lane % 32, lane / 32) of wave w supplies, in
// MFMA step t, the VPL values at k = w*KW + (2t + h)*VPL + i (i < VPL), for
// A's row r and B's column r alike; every MFMA step pairs equal k in both
// operands, so the contraction covers each k < K exactly once (k >= K loads
// read zeros). Both halves of a wave read neighbouring 16-byte pieces of a
// row, so four consecutive steps use whole 128-byte lines.
#include "kernels.hpp"

namespace mg {

namespace {

template <int FAM> struct WkOut;
template <> struct WkOut<FAM_F32> { using T = float; };
template <> struct WkOut<FAM_F16> { using T = _Float16; };
template <> struct WkOut<FAM_BF16> { using T = __bf16; };

// Operand values per lane per MFMA step (16 bytes of K).
template <int FAM> constexpr int wk_vpl() { return FAM == FAM_F32 ? 4 : 8; }

// One lane's 16 bytes of an operand for MFMA step t: the K-contiguous form is
// one vector load; the M/N-contiguous form loads its VPL elements one by one
// (k-rows `ld` elements apart; consecutive lanes read consecutive elements).
template <int FAM, bool KC>
__device__ __forceinline__ u32x4 wk_load(__amdgpu_buffer_rsrc_t rs, int64_t row, int64_t rows,
                                         int64_t k, int64_t K, int64_t ld) {
    constexpr int ESZ = FAM == FAM_F32 ? 4 : 2, VPL = wk_vpl<FAM>();
    if constexpr (KC) {   // element (row, k) at row * K + k; K % VPL == 0
        const bool in = row < rows && k < K;
        const uint32_t off = in ? (uint32_t)((row * K + k) * ESZ) : OOB_OFFSET;
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    } else {              // element (row, k) at k * ld + row
        u32x4 v;
        if constexpr (ESZ == 4) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const bool in = row < rows && k + i < K;
                const uint32_t off = in ? (uint32_t)(((k + i) * ld + row) * 4) : OOB_OFFSET;
                v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < VPL; i += 2) {
                const bool in0 = row < rows && k + i < K, in1 = row < rows && k + i + 1 < K;
                const uint32_t o0 = in0 ? (uint32_t)(((k + i) * ld + row) * 2) : OOB_OFFSET;
                const uint32_t o1 = in1 ? (uint32_t)(((k + i + 1) * ld + row) * 2) : OOB_OFFSET;
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, o0, 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, o1, 0, 0);
                v[i / 2] = (lo & 0xFFFFu) | (hi << 16);
            }
        }
        return v;
    }
}

template <int FAM, bool A_KC, bool B_KC, int T, int W>
__global__ void __launch_bounds__(64 * W) gemm_wholek(GenericArgs a) {
    using Out = typename WkOut<FAM>::T;
    constexpr int VPL = wk_vpl<FAM>(), KW = 2 * VPL * T;   // K per wave
    constexpr int NT = 64 * W, OPT = 1024 / NT;             // threads; outputs per thread
    __shared__ float part[W][32][33];   // [wave][m][n], rows padded against bank conflicts
    const Prob &p = a.p;
    // blocks in groups of 8 block-rows, and each XCD (workgroups are dealt
    // to the 8 XCDs in turn) on one contiguous run of them: the operand
    // panels an XCD reads fit its L2
    const int tiles_m = (int)((p.M + 31) / 32), tiles_n = (int)((p.N + 31) / 32);
    int bm, bn;
    tile_coords(virtual_id((int)blockIdx.x, (int)gridDim.x, 1), tiles_m, tiles_n, 8, bm, bn);
    const int64_t m0 = (int64_t)bm * 32, n0 = (int64_t)bn * 32;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 31, h = lane >> 5;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A), rb = make_rsrc(p.B);
    const int64_t kb = (int64_t)w * KW + h * VPL;

    u32x4 av[T], bv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        av[t] = wk_load<FAM, A_KC>(ra, m0 + r, p.M, kb + t * 2 * VPL, p.K, p.M);
        bv[t] = wk_load<FAM, B_KC>(rb, n0 + r, p.N, kb + t * 2 * VPL, p.K, p.N);
    }
    // every load is issued before the first MFMA waits on one (left alone,
    // the scheduler interleaves them to save registers, one round trip each)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int t = 0; t < T; ++t) Fam<FAM>::mma(acc, &bv[t], &av[t]);

    // acc element v of lane (r, h): row m = r, column n = 8 (v / 4) + 4 h + v % 4
#pragma unroll
    for (int v = 0; v < 16; ++v) part[w][r][8 * (v >> 2) + 4 * h + (v & 3)] = acc[v];
    __syncthreads();

    float alpha = a.e.alpha;
    if (a.e.scale_a) alpha *= *a.e.scale_a;
    if (a.e.scale_b) alpha *= *a.e.scale_b;
    Out *D = reinterpret_cast<Out *>(p.D);
    const Out *C = reinterpret_cast<const Out *>(p.C);
    // OPT outputs per thread, consecutive in D's contiguous dimension
    const int i0 = tid / (32 / OPT), j0 = (tid % (32 / OPT)) * OPT;
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
        const int mm = a.e.lc_row ? i0 : j0 + u, nn = a.e.lc_row ? j0 + u : i0;
        const int64_t m = m0 + mm, n = n0 + nn;
        if (m >= p.M || n >= p.N) continue;
        float s = part[0][mm][nn];   // the waves' partial sums in wave order
#pragma unroll
        for (int q = 1; q < W; ++q) s += part[q][mm][nn];
        const int64_t idx = a.e.lc_row ? m * p.N + n : m + n * p.M;
        float v = alpha * s;
        if (a.e.beta != 0.0f) v = __builtin_fmaf(alpha, s, a.e.beta * (float)C[idx]);
        if (a.e.bias) v += (float)reinterpret_cast<const Out *>(a.e.bias)[n];
        const float x = a.e.aux ? (float)reinterpret_cast<const Out *>(a.e.aux)[idx] : 0.0f;
        float z;
        D[idx] = (Out)finish_aux(v, x, a.e, z);
        if (a.e.aux_out) reinterpret_cast<Out *>(a.e.aux_out)[idx] = (Out)z;
    }
}

template <int FAM, bool A_KC, bool B_KC>
hipError_t launch_t(int steps, dim3 grid, const GenericArgs &a, hipStream_t st) {
    const dim3 b4(256), b8(512);
    switch (steps) {
    case 1: hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 1, 4>), grid, b4, 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 2, 4>), grid, b4, 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 4, 4>), grid, b4, 0, st, a); break;
    case 8: hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 8, 4>), grid, b4, 0, st, a); break;
    case 16: hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 16, 4>), grid, b4, 0, st, a); break;
    case 32:   // eight waves of 16 steps (fp32 only)
        if constexpr (FAM == FAM_F32) {
            hipLaunchKernelGGL((gemm_wholek<FAM, A_KC, B_KC, 16, 8>), grid, b8, 0, st, a);
            break;
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int FAM>
hipError_t launch_fam(bool a_kc, bool b_kc, int steps, dim3 grid, const GenericArgs &a,
                      hipStream_t st) {
    if (a_kc) return b_kc ? launch_t<FAM, true, true>(steps, grid, a, st)
                          : launch_t<FAM, true, false>(steps, grid, a, st);
    return b_kc ? launch_t<FAM, false, true>(steps, grid, a, st)
                : launch_t<FAM, false, false>(steps, grid, a, st);
}

}  // namespace

// 16-step waves need at most 152 registers (220 with an element-loaded
// 16-bit operand); fp32, whose MFMA takes 4 K per step, gets an
// eight-wave form (K <= 1024) reported as 32 steps.
int wholek_steps(int fam, int64_t K) {
    if (fam != FAM_F32 && fam != FAM_F16 && fam != FAM_BF16) return 0;
    const int64_t per_step = 8 * (fam == FAM_F32 ? 4 : 8);   // K of one step over 4 waves x 2 halves
    for (int t = 1; t <= 16; t *= 2)
        if ((int64_t)t * per_step >= K) return t;
    if (fam == FAM_F32 && 32 * per_step >= K) return 32;
    return 0;
}

hipError_t launch_wholek(int fam, bool a_kc, bool b_kc, int steps, const GenericArgs &a,
                         hipStream_t st) {
    const int64_t blocks = ((a.p.M + 31) / 32) * ((a.p.N + 31) / 32);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (fam) {
    case FAM_F32: return launch_fam<FAM_F32>(a_kc, b_kc, steps, grid, a, st);
    case FAM_F16: return launch_fam<FAM_F16>(a_kc, b_kc, steps, grid, a, st);
    case FAM_BF16: return launch_fam<FAM_BF16>(a_kc, b_kc, steps, grid, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mg
