// kernels_inst.hpp -- instantiation helper: one table row per tile kernel
#pragma once

#include "kernels.hpp"

// 128-byte LDS rows, two stages, compiler-scheduled fragment reads (PIPE 0):
// in interleaved same-box measurements this matched or beat the hand-ordered
// pipelines (PIPE 3) on the layer GEMMs.
namespace mg {
template <int FAM, bool AKC, bool BKC, int BM, int BN, int WM, int WN> struct TileCfg {
    using type = Tile<FAM, AKC, BKC, BM, BN, WM, WN, 128, 2, 0>;
};
// 256x256 with both operands K-contiguous: the LDS-DMA copies are issued by
// four of the eight waves (one per SIMD); 2-4 % faster than all eight on the
// transformer-layer shapes in interleaved same-box runs.
template <int FAM> struct TileCfg<FAM, true, true, 256, 256, 2, 4> {
    using type = Tile<FAM, true, true, 256, 256, 2, 4, 128, 2, 0, 4>;
};
// 16-bit types, both operands K-contiguous: the register-streamed pipeline
// (four waves of 128 x 128, one per SIMD; loads one k-tile ahead in
// registers, LDS writes and fragment reads slotted between the MFMAs).
template <> struct TileCfg<FAM_BF16, true, true, 256, 256, 2, 4> {
    using type = Tile<FAM_BF16, true, true, 256, 256, 2, 2, 128, 2, 7>;
};
template <> struct TileCfg<FAM_F16, true, true, 256, 256, 2, 4> {
    using type = Tile<FAM_F16, true, true, 256, 256, 2, 2, 128, 2, 7>;
};
}  // namespace mg

#define MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN) \
    typename mg::TileCfg<FAM, AKC, BKC, BM, BN, WM, WN>::type

#define MG_ROW(FAM, AKC, BKC, TILEID, BM, BN, WM, WN, GROUPED) \
    mg::make_entry<MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN), GROUPED>(TILEID, AKC, BKC)

// The four operand-layout combinations of one tile shape.
#define MG_LAYOUTS(FAM, TILEID, BM, BN, WM, WN, GROUPED)          \
    MG_ROW(FAM, true, true, TILEID, BM, BN, WM, WN, GROUPED),     \
    MG_ROW(FAM, true, false, TILEID, BM, BN, WM, WN, GROUPED),    \
    MG_ROW(FAM, false, true, TILEID, BM, BN, WM, WN, GROUPED),    \
    MG_ROW(FAM, false, false, TILEID, BM, BN, WM, WN, GROUPED)
