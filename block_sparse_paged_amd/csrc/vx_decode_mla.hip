// K4 (MFMA) for MLA-shaped decode: placeholder until the kernel lands; the
// API layer rejects MLA shapes before reaching it.
#include "vx_internal.h"

namespace vx {
hipError_t launch_decode_mla(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace vx
