// Tile geometry shared by the host work planner and the HIP kernels.
#pragma once

namespace cpa {

constexpr int kBlock = 16;          // tokens per KV page
constexpr int kKvTile = 64;         // keys per LDS-staged K/V tile in the chunk kernel (4 pages)

// Waves of one chunk workgroup, each owning 32 (token, head) query rows; all
// of them share every K/V tile the workgroup loads into LDS.  At head_dim 128
// the kernel's registers allow two waves per SIMD, so 8 waves fill a CU with
// one workgroup, whose 256 rows then share each tile load (half the loads per
// matrix operation of two 4-wave workgroups).  At 64 they allow three, and
// three 4-wave workgroups per CU fill it.
constexpr int chunk_waves(int head_dim) { return head_dim > 64 ? 8 : 4; }
// (token, head) query rows of one chunk workgroup, tile and partial slot
constexpr int chunk_rows(int head_dim) { return 32 * chunk_waves(head_dim); }
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
// one resident round at head_dim 128 (one workgroup per CU); 512 at 64.
inline int chunk_wg_target(int head_dim) { return head_dim > 64 ? 256 : 512; }

// Resident workgroups of the chunk kernel and of the mixed launch (one per CU
// at head_dim 128, three at 64, on 256 CUs).  A step runs its decode pieces
// and chunk tiles as one launch only when the chunk tiles alone fill a round:
// then decode workgroups either run beside them or fill the slots their last
// round leaves idle.  With fewer chunk tiles the two run as separate
// launches, which measured as fast or faster there.
inline int mixed_slots(int head_dim) { return 256 * (head_dim > 64 ? 1 : 3); }

// Query tokens one chunk workgroup covers when G query heads share a KV head
// (its last chunk_rows % G rows, if any, hold no query and store nothing).
inline int chunk_tile_tokens(int group, int head_dim) { return chunk_rows(head_dim) / group; }

// Query heads one block of a decode wave serves: the 16 columns of its S^T
// product.
constexpr int kDecodeCols = 16;
constexpr int decode_column_blocks(int group) { return (group + kDecodeCols - 1) / kDecodeCols; }
// A wave of the run-time-group decode holds up to kDecodeWaveBlocks such
// blocks against the same K/V registers, so a group of up to 32 heads reads
// each page once; larger groups take ceil(blocks / 2) waves per (piece, KV
// head).  The compiled groups (at most 8 heads) take one wave.
constexpr int kDecodeWaveBlocks = 2;
constexpr int decode_group_waves(int group) {
  return (decode_column_blocks(group) + kDecodeWaveBlocks - 1) / kDecodeWaveBlocks;
}

// Any number of query heads per KV head up to one chunk tile's rows, so that
// a tile holds at least one token.  G = 1, 2, 4 and 8 have kernels compiled
// for them; any other G runs the same kernels with G read at run time, which
// only changes the row -> (token, head) index arithmetic.
inline bool supported_group(int group, int head_dim) {
  return group >= 1 && group <= chunk_rows(head_dim);
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

// Byte offsets of the partial-result regions inside the caller's workspace.
// Decode slot: acc [Hq][D], m [Hq], l [Hq], fp32 (acc unnormalised).  Chunk
// slot: out [Hkv][R rows][D] bf16 (each piece's output divided by its own
// sum), m and l [Hkv][R] fp32, R = chunk_rows(D).  Max values are stored in
// log2 units of the scaled score.
struct WorkspaceLayout {
  size_t dec_acc, dec_m, dec_l, chk_acc, chk_m, chk_l, total;
};

inline WorkspaceLayout workspace_layout(int64_t dec_slots, int64_t chk_slots, int num_q_heads,
                                        int num_kv_heads, int head_dim) {
  auto up = [](int64_t bytes) { return (size_t)((bytes + 255) / 256 * 256); };
  WorkspaceLayout w;
  size_t at = 0;
  const int64_t dr = dec_slots * num_q_heads;
  const int64_t cr = chk_slots * num_kv_heads * chunk_rows(head_dim);
  w.dec_acc = at; at += up(dr * head_dim * 4);
  w.dec_m = at;   at += up(dr * 4);
  w.dec_l = at;   at += up(dr * 4);
  w.chk_acc = at; at += up(cr * head_dim * 2);
  w.chk_m = at;   at += up(cr * 4);
  w.chk_l = at;   at += up(cr * 4);
  w.total = at;
  return w;
}

}  // namespace cpa
