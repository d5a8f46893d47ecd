// scan.hpp -- device-wide exclusive prefix sum (internal helper of libmsa).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {
// Workspace bytes for scanning n int32 values.
size_t scan_workspace_bytes(int64_t n);
// out[i] = sum_{j<i} in[j] (in == out allowed); *total = sum of all (total may be NULL).
hipError_t launch_exclusive_scan(const int* in, int* out, int64_t n, int* total, void* ws,
                                 hipStream_t st);
}  // namespace msa
