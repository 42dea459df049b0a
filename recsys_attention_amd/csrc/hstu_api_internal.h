// hstu_api_internal.h - helpers of the C ABI shared by its source files (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu.h"

namespace hstu {
namespace api {

// Sets the thread-local message hstu_last_error() returns and returns st.
hstu_status_t fail(hstu_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// The attention argument check of hstu_validate_args.
hstu_status_t validate_fwd(const hstu_fwd_args_t *a);
hstu_status_t hip_status(hipError_t e, const char *what);
// Query tokens of an attention argument block (batched: batch * seqlen_q).
int64_t rows_q(const hstu_fwd_args_t *a);

}  // namespace api
}  // namespace hstu
