// kernels.hpp -- registry of the compiled GEMM kernels (host-visible)
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_core.hpp"

namespace mg {

enum TileId { TILE_256x256 = 1, TILE_128x128 = 2, TILE_64x256 = 3, TILE_32x256 = 4 };

using PersistentLaunch = hipError_t (*)(const KArgs &, int grid, hipStream_t);

struct KernelEntry {
    int fam, a_kc, b_kc, tile;
    int bm, bn, bk, nt, lds_bytes;
    const void *fn_persistent;   // for occupancy queries
    PersistentLaunch run;        // single, batched and grouped GEMMs
};

template <class TL>
hipError_t launch_persistent(const KArgs &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(gemm_persistent<TL>, dim3(grid), dim3(TL::NT), 0, st, a);
    return hipGetLastError();
}

template <class TL>
KernelEntry make_entry(int tile, bool a_kc, bool b_kc) {
    return KernelEntry{TL::FAM, a_kc ? 1 : 0, b_kc ? 1 : 0, tile, TL::BM, TL::BN, TL::BK, TL::NT,
                       TL::LDS_BYTES, reinterpret_cast<const void *>(&gemm_persistent<TL>),
                       &launch_persistent<TL>};
}

// Per-family tables (one translation unit each).
const KernelEntry *entries_bf16(int *count);
const KernelEntry *entries_f16(int *count);
const KernelEntry *entries_f32(int *count);
const KernelEntry *entries_f8(int *count);
const KernelEntry *entries_mxf8(int *count);
const KernelEntry *entries_mxf4(int *count);

// Scalar-load kernel for any alignment / stride (kernels_generic.hip).
struct GenericArgs {
    Prob p;
    EpiArgs e;
    int la_row, lb_row;
};
hipError_t launch_generic(int fam, const GenericArgs &a, hipStream_t st);

// Whole-K kernel for small problems (kernels_wholek.hip): 32x32 blocks of D,
// each of a workgroup's four waves loading its quarter of K at once. Steps:
// MFMA steps per wave (1, 2, 4, 8 or 16; 32 = eight waves of 16, fp32
// only), from wholek_steps (0: K too long or not an fp32/fp16/bf16
// family): K <= 32 * steps * (fp32 ? 4 : 8). K-contiguous operands need
// 16-byte aligned bases and K * element size % 16 == 0; every operand's
// byte span must stay below 2^31.
int wholek_steps(int fam, int64_t K);
hipError_t launch_wholek(int fam, bool a_kc, bool b_kc, int steps, const GenericArgs &a,
                         hipStream_t st);

// Grid-stride zero fill for 32-bit words (graph-capture safe, unlike memset nodes).
hipError_t launch_zero_u32(uint32_t *p, size_t n, hipStream_t st);

}  // namespace mg
