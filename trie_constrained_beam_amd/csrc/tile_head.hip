// Tile kernel variants for lm_head steps: fp32 rows from the dense head, and the children's
// logits computed in the tile for requests with the sparse-head flag (device code in
// beam_device.h).
#include "beam_device.h"

namespace tcb {
hipError_t launch_tile_f32_head(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                                int64_t ld, bool vec, int mode, hipStream_t s) {
    if (!vec || w.norm != TCB_NORM_CHILDREN) return hipErrorInvalidValue;
    launch_tile_t<TCB_F32, TCB_NORM_CHILDREN, true, false, true>(t, w, rp, R, logits, ld, mode, s);
    return hipGetLastError();
}
}  // namespace tcb
