// Pinned host staging for plan uploads (staging.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fi {

// Copies n bytes of host memory `src` to device memory `dst`, asynchronously
// on `stream`, through a pinned block from a process-wide cache. `src` may be
// reused as soon as this returns. Thread-safe. Not for use under stream
// capture (the block returns to the cache once the copy has run).
hipError_t staged_upload(void* dst, const void* src, size_t n, hipStream_t stream);

}  // namespace fi
