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
// 16-bit types with an M- or N-contiguous operand: the same pipeline, that
// operand kept k-row-major in LDS and read with transposing loads.
template <int FAM, bool AKC, bool BKC> struct Rs256 {
    using type = Tile<FAM, AKC, BKC, 256, 256, 2, 2, 128, 2, 7>;
};
template <> struct TileCfg<FAM_BF16, true, false, 256, 256, 2, 4> : Rs256<FAM_BF16, true, false> {};
template <> struct TileCfg<FAM_BF16, false, true, 256, 256, 2, 4> : Rs256<FAM_BF16, false, true> {};
template <> struct TileCfg<FAM_BF16, false, false, 256, 256, 2, 4> : Rs256<FAM_BF16, false, false> {};
template <> struct TileCfg<FAM_F16, true, false, 256, 256, 2, 4> : Rs256<FAM_F16, true, false> {};
template <> struct TileCfg<FAM_F16, false, true, 256, 256, 2, 4> : Rs256<FAM_F16, false, true> {};
template <> struct TileCfg<FAM_F16, false, false, 256, 256, 2, 4> : Rs256<FAM_F16, false, false> {};
// 128x128 (two workgroups per CU): four waves of 64 x 64, every layout.
template <bool AKC, bool BKC> struct TileCfg<FAM_BF16, AKC, BKC, 128, 128, 2, 2> {
    using type = Tile<FAM_BF16, AKC, BKC, 128, 128, 2, 2, 128, 2, 7>;
};
template <bool AKC, bool BKC> struct TileCfg<FAM_F16, AKC, BKC, 128, 128, 2, 2> {
    using type = Tile<FAM_F16, AKC, BKC, 128, 128, 2, 2, 128, 2, 7>;
};
// fp8 with both operands K-contiguous on the skinny and mid tiles (the
// decode shapes, bound by streaming B from HBM): four LDS stages keep three
// k-tiles of copies in flight; 5-6 % more bandwidth than two stages on the
// six decode shapes (same-box A/B; three stages measured the same as four).
template <> struct TileCfg<FAM_F8, true, true, 32, 256, 1, 4> {
    using type = Tile<FAM_F8, true, true, 32, 256, 1, 4, 128, 4, 0>;
};
template <> struct TileCfg<FAM_F8, true, true, 64, 256, 1, 4> {
    using type = Tile<FAM_F8, true, true, 64, 256, 1, 4, 128, 4, 0>;
};
template <> struct TileCfg<FAM_F8, true, true, 128, 128, 2, 2> {
    using type = Tile<FAM_F8, true, true, 128, 128, 2, 2, 128, 4, 0>;
};
}  // namespace mg

#define MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN) \
    typename mg::TileCfg<FAM, AKC, BKC, BM, BN, WM, WN>::type

#define MG_ROW(FAM, AKC, BKC, TILEID, BM, BN, WM, WN) \
    mg::make_entry<MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN)>(TILEID, AKC, BKC)

// The four operand-layout combinations of one tile shape.
#define MG_LAYOUTS(FAM, TILEID, BM, BN, WM, WN)          \
    MG_ROW(FAM, true, true, TILEID, BM, BN, WM, WN),     \
    MG_ROW(FAM, true, false, TILEID, BM, BN, WM, WN),    \
    MG_ROW(FAM, false, true, TILEID, BM, BN, WM, WN),    \
    MG_ROW(FAM, false, false, TILEID, BM, BN, WM, WN)
