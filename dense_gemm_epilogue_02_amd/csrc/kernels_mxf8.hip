// kernels_mxf8.hip -- MX (block-scaled e4m3) tile kernels for every operand
// layout and tile shape; not offered to grouped GEMM
#include "kernels_inst.hpp"

namespace mg {

static const KernelEntry kTable[] = {
    MG_LAYOUTS(FAM_MXF8, TILE_256x256, 256, 256, 2, 4),
    MG_LAYOUTS(FAM_MXF8, TILE_128x128, 128, 128, 2, 2),
    MG_LAYOUTS(FAM_MXF8, TILE_64x256, 64, 256, 1, 4),
    MG_LAYOUTS(FAM_MXF8, TILE_32x256, 32, 256, 1, 4),
};

const KernelEntry *entries_mxf8(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace mg
