// rec_bf16_wide.hip -- the k_rec instances for bf16 with the wide exchange words (rec.h).
#include "rec.h"

namespace lstm_amd {

const void *rec_kernel_bf16_wide(RecTile t, bool wreg, bool fused) {
    return rec_kernel_variant<BF16, true>(t, wreg, fused);
}

}  // namespace lstm_amd
