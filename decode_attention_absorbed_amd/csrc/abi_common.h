// Internal: the error state of the C ABI (owned by mla_decode.hip) for the
// entry points defined in other files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode.h"

namespace mla {

// Record `msg` as the calling thread's last error and return `s`.
mla_status abi_fail(mla_status s, const char* msg);
// MLA_ERR_HIP with "what: <HIP's message>".
mla_status abi_hip_fail(hipError_t e, const char* what);
// A successful call: clear the calling thread's last error.
void abi_ok();
bool abi_aligned(const void* p, uintptr_t a);

}  // namespace mla
