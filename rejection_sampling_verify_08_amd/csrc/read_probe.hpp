// read_probe.hpp -- a streaming-read kernel with the row pass's load pattern,
// used only to measure the chip's practical read bandwidth (included once, by
// spec_verify.hip).  It is not part of the verify step.
//
// One wave reads 8 KB: lane l loads the 16-byte blocks l, l + 64, ...,
// l + 448 of its wave's block range (each load instruction covers 1 KB of
// contiguous memory), exactly as a row-pass wave task reads 4096 bf16
// logits.  The wave folds the data into one word with XOR and writes it only
// if it equals a fixed improbable value, so the loads cannot be removed and
// the kernel writes (almost) nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerLane = 8;
constexpr int64_t kProbeWaveBytes = 64LL * 16 * kProbeBlocksPerLane;   // 8192

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src,
                                                                    int64_t waves,
                                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  if (w >= waves) return;
  const u32x4* p = src + w * (64 * kProbeBlocksPerLane) + lane;
  u32x4 v[kProbeBlocksPerLane];
#pragma unroll
  for (int j = 0; j < kProbeBlocksPerLane; ++j)
    v[j] = NT ? __builtin_nontemporal_load(p + j * 64) : p[j * 64];
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kProbeBlocksPerLane; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0 && x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace sv
