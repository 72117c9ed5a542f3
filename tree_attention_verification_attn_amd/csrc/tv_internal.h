// Internal helpers of libtreeverify (device code and host launch glue).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

constexpr int kMaxT = 128;      // tree nodes per sequence (two 64-bit mask words)
constexpr int kMaxW = 2;

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline long long ceil_div_ll(long long a, long long b) {
  return (a + b - 1) / b;
}

// Checks the launch that was just enqueued.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

// Compute units of the current device (256 on MI355X); cached per device.
int device_cu_count();

}  // namespace tv
