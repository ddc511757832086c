// Paged decode attention, split-K partial pass, matrix-core version (placeholder
// until the MFMA kernel lands: reports no supported shape).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

bool mfma_supported(int, int, int, int, int) { return false; }

hipError_t launch_attend_mfma(const AttendArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
