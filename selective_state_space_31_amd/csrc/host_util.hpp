// host_util.hpp -- host-side helpers shared by the library's translation
// units: the per-thread error message behind ssm_last_error(), argument
// checks and the device queries.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ssm {

// Records the message for ssm_last_error() and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message at the start of an entry point.
void clear_error();

bool aligned(const void* p, size_t k);

struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};
bool overlap(const Span& a, const Span& b);

// SSM_OK, or SSM_ERR_HIP with the launch error's text.
int launch_status(const char* what);

// Compute units of the current device (256 on MI355X if the query fails).
int device_cus();

}  // namespace ssm
