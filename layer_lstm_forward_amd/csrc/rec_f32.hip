// rec_f32.hip -- the k_rec instances for fp32 (rec.h).
#include "rec.h"

namespace lstm_amd {

const void *rec_kernel_f32(RecTile t, bool wreg, bool fused) {
    return rec_kernel_variant<F32, false>(t, wreg, fused);
}

}  // namespace lstm_amd
