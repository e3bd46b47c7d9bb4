// Chunk order of the split-K decode and prefill grids (device code only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// The chunk that workgroup x (0 <= x < n) of the pair (KV head y, sequence z)
// takes: x rotated by the pair's index.  The dispatcher hands workgroups to
// the eight XCDs in turn by linear index, so in a grid of n chunks (n a
// multiple of eight) without the rotation XCD k would take the chunks k, k+8,
// ... of every pair, and in a ragged batch the leading chunks, which every
// sequence has, would pile onto the first XCDs while the last ones idle.  For
// each pair the map is a rotation of 0..n-1, so every chunk is still taken
// once.
__device__ __forceinline__ int rotated_chunk(uint32_t x, uint32_t y, uint32_t z, uint32_t hkv, uint32_t n) {
  return (int)((x + (y + hkv * z) % n) % n);
}

}  // namespace tq
