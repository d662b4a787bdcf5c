// Tile kernel variants for bf16 logits (device code in beam_device.h).
#include "beam_device.h"

namespace tcb {
hipError_t launch_tile_bf16(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits, int64_t ld,
                bool vec, int mode, hipStream_t s) {
    launch_tile_dt<TCB_BF16, false>(t, w, rp, R, logits, ld, vec, mode, s);
    return hipGetLastError();
}
}  // namespace tcb
