// rec_bf16.hip -- the k_rec instances for bf16 with the pair exchange words (rec.h).
#include "rec.h"

namespace lstm_amd {

const void *rec_kernel_bf16(RecTile t, bool wreg, bool fused) {
    return rec_kernel_variant<BF16, false>(t, wreg, fused);
}

}  // namespace lstm_amd
