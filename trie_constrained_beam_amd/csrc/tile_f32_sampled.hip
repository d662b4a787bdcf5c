// Tile kernel variants for fp32 logits, sampled steps (device code in beam_device.h).
#include "beam_device.h"

namespace tcb {
hipError_t launch_tile_f32_sampled(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits, int64_t ld,
                bool vec, int mode, hipStream_t s) {
    launch_tile_dt<TCB_F32, true>(t, w, rp, R, logits, ld, vec, mode, s);
    return hipGetLastError();
}
}  // namespace tcb
