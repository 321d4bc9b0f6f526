// Internal declarations shared by the host and device translation units of
// libqgemv.so.  Not part of the public ABI (that is include/qgemv.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "qgemv.h"

namespace qg {

struct FormatInfo {
    int block;       // weights per block (one meta entry)
    int code_bytes;  // codes per block
    int meta_bytes;  // meta per block
};

// nullptr for an unknown format
const FormatInfo* format_info(int fmt);

// Records a thread-local message and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Host-side argument checks shared by the device entry points.
int check_matrix(int fmt, int64_t N, int64_t K);
bool aligned(const void* p, size_t a);
// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb);

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// Host checks of a GEMV call (format, shape, batch, pointers, alignment);
// QG_OK or the error code with the detail recorded.
int check_gemv_args(int fmt, const void* w, const float* x, const float* y, int64_t N, int64_t K, int B);

}  // namespace qg
