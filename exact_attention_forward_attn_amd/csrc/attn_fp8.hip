// FP8 path (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
int launch_fwd_fp8(const FwdArgs&, void*) { return (int)hipErrorNotSupported; }
int launch_fp8_prepare(const PrepArgs&, void*) { return (int)hipErrorNotSupported; }
}  // namespace attn
