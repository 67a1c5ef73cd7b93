// Launchers shared between the kernel files and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpa {

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* qsl,
                         const int32_t* ctx, const int32_t* bt, int bt_stride, int num_seqs,
                         int num_tokens, int num_kv_heads, int head_dim, void* k_cache,
                         void* v_cache, hipStream_t stream);

// fp32 partial results of split work items (see WorkspaceLayout in tiles.h);
// m is in log2 units of the scaled score.
struct Partials {
  float* acc;
  float* m;
  float* l;
};

// A split chunk tile's pieces: each piece's output divided by its own sum, in
// bf16 (a weighted mean of V rows, so within V's range), with that sum and
// the running max in fp32.
struct ChunkPartials {
  uint16_t* out;
  float* m;
  float* l;
};

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* bt, int bt_stride, const int32_t* qsl,
                         const int32_t* splits, int num_splits, int num_q_heads, int num_kv_heads,
                         int head_dim, float scale_log2, void* out, float* lse, Partials ws,
                         hipStream_t stream);

hipError_t launch_chunk(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                        int bt_stride, const int32_t* qsl, const int32_t* ctx,
                        const int32_t* tiles, int num_tiles, int num_q_heads, int num_kv_heads,
                        int head_dim, float scale_log2, void* out, float* lse, ChunkPartials part,
                        hipStream_t stream);

// Decode pieces and chunk tiles of one step in one launch (mixed.hip); both
// counts > 0.
hipError_t launch_mixed(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                        int bt_stride, const int32_t* qsl, const int32_t* ctx,
                        const int32_t* tiles, int num_tiles, const int32_t* splits, int num_splits,
                        int num_q_heads, int num_kv_heads, int head_dim, float scale_log2,
                        void* out, float* lse, ChunkPartials cpart, Partials dpart,
                        hipStream_t stream);

// Both merges of a step in one launch (either count may be 0).
hipError_t launch_merges(const int32_t* dmerges, int num_decode_merges, const int32_t* cmerges,
                         int num_chunk_merges, const int32_t* qsl, int num_q_heads,
                         int num_kv_heads, int head_dim, Partials dws, ChunkPartials cws, void* out,
                         float* lse, hipStream_t stream);

}  // namespace cpa
