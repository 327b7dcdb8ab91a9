// api_util.h -- helpers shared by the host entry points (api.cpp,
// prefill_api.cpp): the thread-local last-error message and descriptor
// checks.  Internal; not part of the C ABI.
#pragma once

#include "pkvd.h"

namespace pkvd {
namespace api {

// Records a printf-style message as the calling thread's last error and
// returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's last error (every entry point starts with it).
void clear_error();
bool aligned16(const void* p);
// Dense row-major strides (size-1 dimensions may have any stride).
bool contiguous(const pkvd_tensor* t);
// CUs of the current device (cached per device; 256 when no device answers).
int device_cus();
// Whether the byte ranges two tensors' elements may occupy (from shape,
// strides and element size; negative strides are not accepted anywhere)
// intersect.  Empty tensors overlap nothing.
bool overlaps(const pkvd_tensor* a, const pkvd_tensor* b);

}  // namespace api
}  // namespace pkvd
