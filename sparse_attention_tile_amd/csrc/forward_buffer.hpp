// The forward pass with its tile map in caller-chosen device memory: the
// host side of na_forward_noalloc (defined in na_api.cpp, called from
// noalloc.hip, which owns the fixed device buffer).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>

#include "na.h"

namespace na {

// na_forward's form 2 (bf16, head_dim 64 / 128: the kernel reads q, k, v and
// writes out, lse in grid order) with the tile map copied on `stream` into
// the device memory *get_buffer returns (buffer_bytes long) instead of a
// cached allocation.  Validates everything, including the map's size against
// buffer_bytes, before get_buffer is called.
na_status forward_in_buffer(const void* q, const void* k, const void* v, void* out, float* lse, int batch,
                            int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                            float scale, na_dtype dtype, void* stream, size_t buffer_bytes,
                            hipError_t (*get_buffer)(void** ptr));

}  // namespace na
