// C-ABI device entry points: argument checks, then kernel launches on the
// caller's stream.  Declarations and contracts are in include/cpa.h.

#include <atomic>

#include "../../include/cpa.h"
#include "internal.h"
#include "tiles.h"

namespace {

int check_heads(int num_q_heads, int num_kv_heads, int head_dim, int block_size) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return CPA_ERR_INVALID;
  if (block_size != cpa::kBlock) return CPA_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_head_dim(head_dim)) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_group(num_q_heads / num_kv_heads, head_dim)) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_kv_heads(num_kv_heads)) return CPA_ERR_UNSUPPORTED;
  return CPA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? CPA_OK : CPA_ERR_DEVICE; }

}  // namespace

extern "C" int cpa_append_kv(const void* k_new, const void* v_new, const int32_t* d_query_start_loc,
                             const int32_t* d_context_lens, const int32_t* d_block_table,
                             int bt_stride, int num_seqs, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, void* k_cache, void* v_cache,
                             void* stream) {
  if (head_dim <= 0 || num_kv_heads <= 0) return CPA_ERR_INVALID;
  if (block_size != cpa::kBlock) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_head_dim(head_dim)) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_kv_heads(num_kv_heads)) return CPA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_seqs < 0 || bt_stride <= 0) return CPA_ERR_INVALID;
  if (num_tokens == 0) return CPA_OK;
  if (num_seqs == 0 || !k_new || !v_new || !d_query_start_loc || !d_context_lens ||
      !d_block_table || !k_cache || !v_cache)
    return CPA_ERR_INVALID;
  return status_of(cpa::launch_append(k_new, v_new, d_query_start_loc, d_context_lens,
                                      d_block_table, bt_stride, num_seqs, num_tokens, num_kv_heads,
                                      head_dim, k_cache, v_cache, (hipStream_t)stream));
}

extern "C" int cpa_attention(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* d_block_table, int bt_stride,
                             const int32_t* d_query_start_loc, const int32_t* d_seq_lens,
                             const int32_t* d_context_lens, const int32_t* d_plan,
                             const cpa_plan_counts_t* counts, int num_seqs, int num_decodes,
                             int num_tokens, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, float softmax_scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  (void)d_seq_lens;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != CPA_OK) return st;
  if (!counts || num_seqs < 0 || num_decodes < 0 || num_decodes > num_seqs || num_tokens < 0 ||
      bt_stride <= 0)
    return CPA_ERR_INVALID;
  const cpa_plan_counts_t& n = *counts;
  if (n.num_decode_splits < 0 || n.num_decode_merges < 0 || n.num_chunk_tiles < 0 ||
      n.num_chunk_merges < 0 || n.num_decode_partials < 0 || n.num_chunk_partials < 0)
    return CPA_ERR_INVALID;
  if (num_tokens == 0) return CPA_OK;
  if (!q || !k_cache || !v_cache || !d_block_table || !d_query_start_loc || !d_context_lens ||
      !d_plan || !out)
    return CPA_ERR_INVALID;
  if (!(softmax_scale > 0.f)) return CPA_ERR_INVALID;
  const cpa::WorkspaceLayout wl =
      cpa::workspace_layout(n.num_decode_partials, n.num_chunk_partials, num_q_heads, num_kv_heads,
                            head_dim);
  if (wl.total > 0 && (workspace == nullptr || workspace_bytes < wl.total)) return CPA_ERR_CAPACITY;

  hipStream_t s = (hipStream_t)stream;
  const float sl2 = softmax_scale * 1.4426950408889634f;
  cpa::Partials dws{nullptr, nullptr, nullptr};
  cpa::ChunkPartials cws{nullptr, nullptr, nullptr};
  if (wl.total > 0) {
    char* base = static_cast<char*>(workspace);
    dws = {reinterpret_cast<float*>(base + wl.dec_acc), reinterpret_cast<float*>(base + wl.dec_m),
           reinterpret_cast<float*>(base + wl.dec_l)};
    cws = {reinterpret_cast<uint16_t*>(base + wl.chk_acc),
           reinterpret_cast<float*>(base + wl.chk_m), reinterpret_cast<float*>(base + wl.chk_l)};
  }
  const int32_t* splits = d_plan;
  const int32_t* tiles = splits + (size_t)n.num_decode_splits * CPA_DECODE_SPLIT_WORDS;
  const int32_t* dmerges = tiles + (size_t)n.num_chunk_tiles * CPA_CHUNK_TILE_WORDS;
  const int32_t* cmerges = dmerges + (size_t)n.num_decode_merges * CPA_DECODE_MERGE_WORDS;

  // decode splits and chunk tiles are independent (one launch when both are
  // present and the chunk tiles fill a resident round); the merges (one
  // launch) follow them
  const bool mixed = n.num_decode_splits > 0 &&
                     (int64_t)n.num_chunk_tiles * num_kv_heads >= cpa::mixed_slots(head_dim);
  if (mixed) {
    st = status_of(cpa::launch_mixed(q, k_cache, v_cache, d_block_table, bt_stride,
                                     d_query_start_loc, d_context_lens, tiles, n.num_chunk_tiles,
                                     splits, n.num_decode_splits, num_q_heads, num_kv_heads,
                                     head_dim, sl2, out, lse, cws, dws, s));
    if (st != CPA_OK) return st;
  } else if (n.num_decode_splits > 0) {
    st = status_of(cpa::launch_decode(q, k_cache, v_cache, d_block_table, bt_stride,
                                      d_query_start_loc, splits, n.num_decode_splits, num_q_heads,
                                      num_kv_heads, head_dim, sl2, out, lse, dws, s));
    if (st != CPA_OK) return st;
  }
  if (!mixed && n.num_chunk_tiles > 0) {
    st = status_of(cpa::launch_chunk(q, k_cache, v_cache, d_block_table, bt_stride,
                                     d_query_start_loc, d_context_lens, tiles, n.num_chunk_tiles,
                                     num_q_heads, num_kv_heads, head_dim, sl2, out, lse, cws, s));
    if (st != CPA_OK) return st;
  }
  if (n.num_decode_merges > 0 || n.num_chunk_merges > 0) {
    st = status_of(cpa::launch_merges(dmerges, n.num_decode_merges, cmerges, n.num_chunk_merges,
                                      d_query_start_loc, num_q_heads, num_kv_heads, head_dim, dws,
                                      cws, out, lse, s));
    if (st != CPA_OK) return st;
  }
  return CPA_OK;
}

// ---------------------------------------------------------------------------
// cpa_attention_noalloc: the same call with the partial-result workspace in a
// file-scope device array, for callers that cannot allocate.
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // CPA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == CPA_NOALLOC_SCRATCH_BYTES, "header and library agree");

// One copy per GPU, held until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in): the device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_address[kMaxDevices];

// Device address of the current device's scratch array.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CPA_ERR_DEVICE;
  void* p = scratch_address[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return CPA_ERR_DEVICE;
    scratch_address[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return CPA_OK;
}

}  // namespace

extern "C" int cpa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* d_block_table, int bt_stride,
                                     const int32_t* d_query_start_loc, const int32_t* d_seq_lens,
                                     const int32_t* d_context_lens, const int32_t* d_plan,
                                     const cpa_plan_counts_t* counts, int num_seqs,
                                     int num_decodes, int num_tokens, int num_q_heads,
                                     int num_kv_heads, int head_dim, int block_size,
                                     float softmax_scale, void* out, float* lse, void* stream) {
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != CPA_OK) return st;
  if (!counts || counts->num_decode_partials < 0 || counts->num_chunk_partials < 0)
    return CPA_ERR_INVALID;
  const cpa::WorkspaceLayout wl =
      cpa::workspace_layout(counts->num_decode_partials, counts->num_chunk_partials, num_q_heads,
                            num_kv_heads, head_dim);
  if (wl.total > kScratchBytes) return CPA_ERR_CAPACITY;
  void* ws = nullptr;
  if (wl.total > 0 && num_tokens > 0) {
    st = current_scratch(&ws);
    if (st != CPA_OK) return st;
  }
  return cpa_attention(q, k_cache, v_cache, d_block_table, bt_stride, d_query_start_loc,
                       d_seq_lens, d_context_lens, d_plan, counts, num_seqs, num_decodes,
                       num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, softmax_scale,
                       out, lse, ws, ws ? kScratchBytes : 0, stream);
}
