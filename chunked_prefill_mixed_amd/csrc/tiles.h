// Tile geometry shared by the host work planner and the HIP kernels.
#pragma once

namespace cpa {

constexpr int kBlock = 16;          // tokens per KV page
constexpr int kKvTile = 64;         // keys per LDS-staged K/V tile in the chunk kernel (4 pages)

// (token, head) query rows of a chunk tile, workgroup and partial slot: 32
// per wave, all sharing every K/V tile the workgroup loads into LDS.  At
// head_dim 128 the kernel's registers allow two waves per SIMD: 256 rows (8
// waves) fill a CU with one workgroup and share each tile load (half the
// loads per matrix operation), or 128 rows (4 waves) put two workgroups on a
// CU.  At 64 they allow three, and three 128-row workgroups per CU fill it.
constexpr int default_chunk_rows(int head_dim) { return head_dim > 64 ? 256 : 128; }
// The rows a plan's chunk_tile_rows field selects (0: the head_dim's
// default); 0 when the head_dim does not allow the value.
inline int plan_chunk_rows(int field, int head_dim) {
  if (field == 0) return default_chunk_rows(head_dim);
  if (field == 128 || (field == 256 && head_dim > 64)) return field;
  return 0;
}
constexpr int chunk_waves(int rows) { return rows / 32; }
// Decode waves per launch round: one per SIMD of the 256 CUs.  The kernel's
// registers would allow 3 waves per SIMD at head_dim 128 and 5 at 64, but
// longer pieces at one wave per SIMD read as fast or faster (less start-up
// and fewer partial results per byte), and a whole number of workgroups per
// CU keeps every CU's share of the bytes equal; the planner adds whole
// rounds only when pieces would exceed 64 pages.
inline int decode_waves_target(int head_dim) {
  (void)head_dim;
  return 256 * 4;
}
constexpr int kDecodeMaxSplit = 64 * kBlock;  // a decode split spans at most 64 pages
constexpr int kChunkMinSplit = 256;       // fewest prefix keys worth a separate chunk piece

// Chunk workgroups the planner aims at when it cuts tiles into key pieces:
// one resident round of 256-row workgroups (one per CU); 512 of 128 rows.
inline int chunk_wg_target(int rows) { return rows == 256 ? 256 : 512; }

// Resident workgroups of the chunk kernel and of the mixed launch on 256 CUs:
// one per CU with 256-row tiles, two with 128-row tiles at head_dim 128,
// three at 64.  A step runs its decode pieces and chunk tiles as one launch
// only when the chunk tiles alone fill a round: then decode workgroups either
// run beside them or fill the slots their last round leaves idle.  With fewer
// chunk tiles the two run as separate launches, which measured as fast or
// faster there.
inline int mixed_slots(int head_dim, int rows) {
  return 256 * (rows == 256 ? 1 : head_dim > 64 ? 2 : 3);
}

// Query tokens one chunk workgroup covers when G query heads share a KV head.
inline int chunk_tile_tokens(int group, int rows) { return rows / group; }

inline bool supported_group(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}
inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
// at most 256 KV heads: one page of all KV heads then spans under 2^21 bytes,
// and the chunk kernel forms page offsets as 32 x 32-bit products
constexpr int kMaxKvHeads = 256;
inline bool supported_kv_heads(int h) { return h >= 1 && h <= kMaxKvHeads; }

}  // namespace cpa

#include <stddef.h>
#include <stdint.h>

namespace cpa {

// Byte offsets of the fp32 partial-result regions inside the caller's
// workspace.  Decode slot: acc [Hq][D], m [Hq], l [Hq].  Chunk slot: acc
// [Hkv][R rows][D], m and l [Hkv][R], R the plan's chunk tile rows.  Max
// values are stored in log2 units of the scaled score.
struct WorkspaceLayout {
  size_t dec_acc, dec_m, dec_l, chk_acc, chk_m, chk_l, total;
};

inline WorkspaceLayout workspace_layout(int64_t dec_slots, int64_t chk_slots, int num_q_heads,
                                        int num_kv_heads, int head_dim, int rows) {
  auto up = [](int64_t bytes) { return (size_t)((bytes + 255) / 256 * 256); };
  WorkspaceLayout w;
  size_t at = 0;
  const int64_t dr = dec_slots * num_q_heads;
  const int64_t cr = chk_slots * num_kv_heads * rows;
  w.dec_acc = at; at += up(dr * head_dim * 4);
  w.dec_m = at;   at += up(dr * 4);
  w.dec_l = at;   at += up(dr * 4);
  w.chk_acc = at; at += up(cr * head_dim * 4);
  w.chk_m = at;   at += up(cr * 4);
  w.chk_l = at;   at += up(cr * 4);
  w.total = at;
  return w;
}

}  // namespace cpa
