// kernels_inst.hpp -- instantiation helper: one table row per tile kernel
#pragma once

#include "kernels.hpp"

// 128-byte LDS rows, two stages, compiler-scheduled fragment reads (PIPE 0):
// in interleaved same-box measurements this matched or beat the hand-ordered
// pipelines (PIPE 3 / 5) on the layer GEMMs.
#define MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN) mg::Tile<FAM, AKC, BKC, BM, BN, WM, WN, 128, 2, 0>

#define MG_ROW(FAM, AKC, BKC, TILEID, BM, BN, WM, WN, GROUPED) \
    mg::make_entry<MG_TILE(FAM, AKC, BKC, BM, BN, WM, WN), GROUPED>(TILEID, AKC, BKC)

// The four operand-layout combinations of one tile shape.
#define MG_LAYOUTS(FAM, TILEID, BM, BN, WM, WN, GROUPED)          \
    MG_ROW(FAM, true, true, TILEID, BM, BN, WM, WN, GROUPED),     \
    MG_ROW(FAM, true, false, TILEID, BM, BN, WM, WN, GROUPED),    \
    MG_ROW(FAM, false, true, TILEID, BM, BN, WM, WN, GROUPED),    \
    MG_ROW(FAM, false, false, TILEID, BM, BN, WM, WN, GROUPED)
