// kernels_bf16.hip -- bf16 tile kernels for every operand layout and tile shape
#include "kernels_inst.hpp"

namespace mg {

static const KernelEntry kTable[] = {
    MG_LAYOUTS(FAM_BF16, TILE_256x256, 256, 256, 2, 4),
    MG_LAYOUTS(FAM_BF16, TILE_128x128, 128, 128, 2, 2),
    MG_LAYOUTS(FAM_BF16, TILE_64x256, 64, 256, 1, 4),
    MG_LAYOUTS(FAM_BF16, TILE_32x256, 32, 256, 1, 4),
};

const KernelEntry *entries_bf16(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace mg
