// attn_fwd_mxfp8.hip -- block-scaled e4m3 attention forward for gfx950.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {

hipError_t launch_fwd_mxfp8(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
