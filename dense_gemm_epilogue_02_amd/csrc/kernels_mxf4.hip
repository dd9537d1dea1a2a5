// kernels_mxf4.hip -- MXFP4 (block-scaled e2m1) tile kernels. The elements
// are packed two per byte along K, so only K-contiguous operands (A
// RowMajor, B ColumnMajor) have tile kernels; other layouts run on the
// scalar kernel. Not offered to grouped GEMM.
#include "kernels_inst.hpp"

namespace mg {

static const KernelEntry kTable[] = {
    MG_ROW(FAM_MXF4, true, true, TILE_256x256, 256, 256, 2, 4),
    MG_ROW(FAM_MXF4, true, true, TILE_128x128, 128, 128, 2, 2),
    MG_ROW(FAM_MXF4, true, true, TILE_64x256, 64, 256, 1, 4),
    MG_ROW(FAM_MXF4, true, true, TILE_32x256, 32, 256, 1, 4),
};

const KernelEntry *entries_mxf4(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace mg
