// kernels_f32.hip -- fp32 tile kernels (fp32 MFMA) for every operand layout
#include "kernels_inst.hpp"

namespace mg {

static const KernelEntry kTable[] = {
    MG_LAYOUTS(FAM_F32, TILE_128x128, 128, 128, 2, 2),
};

const KernelEntry *entries_f32(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace mg
