// Tile geometry shared by the host work planner and the HIP kernels.
#pragma once

namespace cpa {

constexpr int kBlock = 16;          // tokens per KV page
constexpr int kChunkRows = 128;     // (token, head) query rows per chunk workgroup: 4 waves x 32
constexpr int kKvTile = 64;         // keys per LDS-staged K/V tile in the chunk kernel (4 pages)
constexpr int kDecodeWavesTarget = 4096;  // decode waves to aim for when sizing splits

// Query tokens one chunk workgroup covers when G query heads share a KV head.
inline int chunk_tile_tokens(int group) { return kChunkRows / group; }

inline bool supported_group(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}
inline bool supported_head_dim(int d) { return d == 64 || d == 128; }

}  // namespace cpa
