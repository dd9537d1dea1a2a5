// kernels_generic.hip -- scalar-load GEMM for operands that vector loads cannot
// serve (unaligned base addresses, contiguous extents that are not a multiple
// of 16 bytes, or offsets beyond 32 bits), plus a small zero-fill kernel.
//
// Same contract as the tile kernels ("CUTLASS Python接口" section 3.3:
// D = alpha*A*B + beta*C with an fp32 accumulator; section 7.2: misaligned
// data still works, only slower): each element is loaded on its own (64-bit
// addressing), decoded to fp32, staged in LDS, and accumulated with fp32 FMA
// in increasing k. The raw loads of the next few k-steps stay in flight while
// one is multiplied.
#include "kernels.hpp"

namespace mg {

namespace {

constexpr int GT = 64;    // output tile edge
constexpr int GK = 16;    // k per step

// OCP E4M3: sign, 4-bit exponent (bias 7), 3-bit fraction, S.1111.111 = NaN.
__device__ __forceinline__ float decode_e4m3(uint32_t u) {
    const uint32_t s = (u & 0x80u) << 24, e = (u >> 3) & 15u, m = u & 7u;
    if (e == 15u && m == 7u) return __builtin_nanf("");
    float v;
    if (e == 0u) v = (float)m * 0.001953125f;   // m * 2^-9
    else v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | s);
}
// OCP FP4 E2M1: sign, 2-bit exponent (bias 1), 1-bit fraction; exponent 0
// holds 0 and 1/2, the largest magnitude is 6; no NaN or infinity.
__device__ __forceinline__ float decode_e2m1(uint32_t u) {
    const uint32_t e = (u >> 1) & 3u, m = u & 1u;
    const float v = e == 0u ? 0.5f * (float)m : (float)(2u + m) * (float)(1u << e) * 0.25f;
    return (u & 8u) ? -v : v;
}
// OCP MX E8M0 scale: 2^(c-127); c = 0 is the fp32 subnormal 2^-127, 255 is NaN.
__device__ __forceinline__ float e8m0(uint32_t c) {
    if (c == 255u) return __builtin_nanf("");
    return __builtin_bit_cast(float, c == 0u ? 0x00400000u : c << 23);
}

template <int FAM> struct OutT;
template <> struct OutT<FAM_F32> { using T = float; };
template <> struct OutT<FAM_F16> { using T = _Float16; };
template <> struct OutT<FAM_BF16> { using T = __bf16; };
template <> struct OutT<FAM_F8> { using T = __bf16; };
template <> struct OutT<FAM_MXF8> { using T = __bf16; };
template <> struct OutT<FAM_MXF4> { using T = __bf16; };

// Raw storage bits of one element (decoded only when staged into LDS, so
// the loads of several k-steps can be in flight at once).
template <int FAM> struct RawT;
template <> struct RawT<FAM_F32> { using T = uint32_t; };
template <> struct RawT<FAM_F16> { using T = uint16_t; };
template <> struct RawT<FAM_BF16> { using T = uint16_t; };
template <> struct RawT<FAM_F8> { using T = uint8_t; };

template <int FAM> __device__ __forceinline__ float decode_raw(uint32_t bits);
template <> __device__ __forceinline__ float decode_raw<FAM_F32>(uint32_t b) {
    return __builtin_bit_cast(float, b);
}
template <> __device__ __forceinline__ float decode_raw<FAM_F16>(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
template <> __device__ __forceinline__ float decode_raw<FAM_BF16>(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}
template <> __device__ __forceinline__ float decode_raw<FAM_F8>(uint32_t b) {
    return decode_e4m3(b & 0xFFu);
}
// FP4: the fetch already extracted the element's nibble
template <> struct RawT<FAM_MXF4> { using T = uint8_t; };
template <> __device__ __forceinline__ float decode_raw<FAM_MXF4>(uint32_t b) {
    return decode_e2m1(b & 15u);
}

// k-steps whose loads are in flight ahead of the one being multiplied.
constexpr int GPF = 4;

template <int FAM>
__global__ void __launch_bounds__(256) gemm_generic(GenericArgs a) {
    using Out = typename OutT<FAM>::T;
    constexpr int LF = FAM == FAM_MXF8 ? FAM_F8 : FAM;   // element decoder
    constexpr bool MX = FAM == FAM_MXF8 || FAM == FAM_MXF4;
    using Raw = typename RawT<LF>::T;
    // k-rows of 64 floats: a thread's 4 consecutive rows / columns are one
    // 16-byte read (4x fewer LDS instructions than element reads: fp32
    // 128x64x256 33 -> 29 us)
    __shared__ __attribute__((aligned(16))) float As[GK][GT];
    __shared__ __attribute__((aligned(16))) float Bs[GK][GT];
    const Prob &p = a.p;
    const int tiles_n = (int)((p.N + GT - 1) / GT);
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * GT;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * GT;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const Raw *Ar = reinterpret_cast<const Raw *>(p.A);
    const Raw *Br = reinterpret_cast<const Raw *>(p.B);
    float acc[4][4] = {};
    // ring of GPF k-steps of raw operand bits (and MX block-scale codes):
    // slot u holds step s with s % GPF == u; out-of-range elements are 0
    uint32_t ra[GPF][4], rb[GPF][4], xa[GPF][4], xb[GPF][4];
    auto fetch = [&](int64_t k0, uint32_t (&va)[4], uint32_t (&vb)[4], uint32_t (&sa)[4],
                     uint32_t (&sb)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = tid + u * 256;      // 0 .. 1023
            const int kk = e / GT, rr = e % GT;
            const int64_t k = k0 + kk;
            const int64_t m = m0 + rr, n = n0 + rr;
            const bool ina = k < p.K && m < p.M, inb = k < p.K && n < p.N;
            const int64_t ia = a.la_row ? m * p.K + k : m + k * p.M;
            const int64_t ib = a.lb_row ? k * p.N + n : k + n * p.K;
            if constexpr (FAM == FAM_MXF4) {   // element t: nibble t & 1 of byte t / 2
                va[u] = ina ? ((uint32_t)Ar[ia >> 1] >> (4 * (ia & 1))) & 15u : 0u;
                vb[u] = inb ? ((uint32_t)Br[ib >> 1] >> (4 * (ib & 1))) & 15u : 0u;
            } else {
                va[u] = ina ? (uint32_t)Ar[ia] : 0u;
                vb[u] = inb ? (uint32_t)Br[ib] : 0u;
            }
            if constexpr (MX) {
                sa[u] = ina ? (uint32_t)p.mx_a[m * (p.K >> 5) + (k >> 5)] : 127u;
                sb[u] = inb ? (uint32_t)p.mx_b[n * (p.K >> 5) + (k >> 5)] : 127u;
            }
        }
    };
    const int64_t steps = (p.K + GK - 1) / GK;
#pragma unroll
    for (int u = 0; u < GPF; ++u)
        if (u < steps) fetch((int64_t)u * GK, ra[u], rb[u], xa[u], xb[u]);
    for (int64_t s0 = 0; s0 < steps; s0 += GPF) {
#pragma unroll
        for (int u = 0; u < GPF; ++u) {
            const int64_t s = s0 + u;
            if (s >= steps) break;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int e = tid + w * 256;
                const int kk = e / GT, rr = e % GT;
                float av = decode_raw<LF>(ra[u][w]), bv = decode_raw<LF>(rb[u][w]);
                if constexpr (MX) {
                    // block scales of A's row and B's column (K % 32 == 0); a
                    // power of two, so the scaled element is exact
                    av *= e8m0(xa[u][w]);
                    bv *= e8m0(xb[u][w]);
                }
                As[kk][rr] = av;
                Bs[kk][rr] = bv;
            }
            __syncthreads();
            // refill this slot with step s + GPF while step s is multiplied
            if (s + GPF < steps) fetch((s + GPF) * GK, ra[u], rb[u], xa[u], xb[u]);
#pragma unroll
            for (int kk = 0; kk < GK; ++kk) {
                const f32x4 xv = *reinterpret_cast<const f32x4 *>(&As[kk][ty * 4]);
                const f32x4 yv = *reinterpret_cast<const f32x4 *>(&Bs[kk][tx * 4]);
                const float x[4] = {xv.x, xv.y, xv.z, xv.w}, y[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(x[i], y[j], acc[i][j]);
            }
            __syncthreads();
        }
    }
    float alpha = a.e.alpha;
    if (a.e.scale_a) alpha *= *a.e.scale_a;
    if (a.e.scale_b) alpha *= *a.e.scale_b;
    Out *D = reinterpret_cast<Out *>(p.D);
    const Out *C = reinterpret_cast<const Out *>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m >= p.M || n >= p.N) continue;
            const int64_t idx = a.e.lc_row ? m * p.N + n : m + n * p.M;
            float v = alpha * acc[i][j];
            if (a.e.beta != 0.0f) v = __builtin_fmaf(alpha, acc[i][j], a.e.beta * (float)C[idx]);
            if (a.e.bias) v += (float)reinterpret_cast<const Out *>(a.e.bias)[n];
            const float x = a.e.aux ? (float)reinterpret_cast<const Out *>(a.e.aux)[idx] : 0.0f;
            float z;
            D[idx] = (Out)finish_aux(v, x, a.e, z);
            if (a.e.aux_out) reinterpret_cast<Out *>(a.e.aux_out)[idx] = (Out)z;
        }
}

__global__ void zero_u32(uint32_t *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_generic(int fam, const GenericArgs &a, hipStream_t st) {
    const int64_t tiles = ((a.p.M + GT - 1) / GT) * ((a.p.N + GT - 1) / GT);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles), block(256);
    switch (fam) {
    case FAM_F32: hipLaunchKernelGGL(gemm_generic<FAM_F32>, grid, block, 0, st, a); break;
    case FAM_F16: hipLaunchKernelGGL(gemm_generic<FAM_F16>, grid, block, 0, st, a); break;
    case FAM_BF16: hipLaunchKernelGGL(gemm_generic<FAM_BF16>, grid, block, 0, st, a); break;
    case FAM_F8: hipLaunchKernelGGL(gemm_generic<FAM_F8>, grid, block, 0, st, a); break;
    case FAM_MXF8: hipLaunchKernelGGL(gemm_generic<FAM_MXF8>, grid, block, 0, st, a); break;
    case FAM_MXF4: hipLaunchKernelGGL(gemm_generic<FAM_MXF4>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace mg
