// Host-side decode-first budget split and device work plan (cpa_build_metadata).
//
// Budget split: every running decode takes one token, the rest of the budget
// goes to prefills in queue order and a prompt that does not fit is cut to
// what remains ("Chunked Prefill" (deepconcepts.dev), "Why a chunk can be
// nearly free"; "05. Chunked Prefill" section 5; tbr8.org deep dive 3.1;
// "How Chunked Prefill Stops Decode Starvation", "The fix").  A budget below
// the number of decodes is rejected ("Chunked Prefill", "The budget points in
// two directions").
//
// Work plan: decode rows are cut into page-aligned key pieces sized so that
// every wave is resident at once and none reads more pages than needed
// (lognormal context lengths then balance over the GPU); rows with several
// pieces get a log-sum-exp merge entry.  Chunk rows are cut into query tiles of
// floor(chunk_rows(head_dim) / (Hq/Hkv)) tokens whose visible prefix may be cut
// into key pieces, ordered longest key range first (dealt over the XCD ranges
// of a KV head when there are fewer than 8 KV heads).
//
// Pure host code: no HIP call, safe to run on a machine without a GPU.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <functional>
#include <queue>
#include <vector>

#include "../../include/cpa.h"
#include "tiles.h"

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_params(const cpa_build_params_t* p) {
  if (!p) return CPA_ERR_INVALID;
  if (p->token_budget <= 0 || p->long_prefill_cap < 0) return CPA_ERR_INVALID;
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0) return CPA_ERR_INVALID;
  if (p->decode_split_tokens < 0 || p->chunk_split_tokens < 0) return CPA_ERR_INVALID;
  if (p->block_size != cpa::kBlock) return CPA_ERR_UNSUPPORTED;
  if (p->num_q_heads % p->num_kv_heads) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_head_dim(p->head_dim)) return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_group(p->num_q_heads / p->num_kv_heads, p->head_dim))
    return CPA_ERR_UNSUPPORTED;
  if (!cpa::supported_kv_heads(p->num_kv_heads)) return CPA_ERR_UNSUPPORTED;
  if (p->decode_split_tokens % cpa::kBlock || p->decode_split_tokens > cpa::kDecodeMaxSplit)
    return CPA_ERR_INVALID;
  if (p->chunk_split_tokens % cpa::kKvTile) return CPA_ERR_INVALID;
  const int base = p->policy & ~(CPA_POLICY_ADAPTIVE_CHUNK | CPA_POLICY_BLOCK_ALIGNED);
  if (base != CPA_POLICY_TRUNCATE && base != CPA_POLICY_DEFER && base != CPA_POLICY_QUOTA)
    return CPA_ERR_INVALID;
  if (base == CPA_POLICY_QUOTA &&
      (p->max_prefill_tokens <= 0 || p->max_prefill_tokens > INT32_MAX - p->token_budget))
    return CPA_ERR_INVALID;
  if ((p->policy & CPA_POLICY_ADAPTIVE_CHUNK) && p->long_prefill_cap <= 0) return CPA_ERR_INVALID;
  return CPA_OK;
}

// Per-request chunk size from the decode queue depth (tbr8.org deep dive 7.1).
// The rule is a table: the first row whose bound exceeds the decode count
// scales the base chunk by mul / div (at least one token, at most INT32_MAX).
struct AdaptiveRow {
  int64_t below;
  int64_t mul, div;
};
constexpr AdaptiveRow kAdaptiveRows[] = {{1, 4, 1}, {10, 2, 1}, {50, 1, 1}, {INT64_MAX, 1, 2}};

int adaptive_cap(int base_chunk, int num_decodes) {
  for (const AdaptiveRow& r : kAdaptiveRows)
    if (num_decodes < r.below)
      return (int)std::min<int64_t>(INT32_MAX, std::max<int64_t>(1, base_chunk * r.mul / r.div));
  return base_chunk;
}

// Pages per decode piece when the caller leaves the split size to the
// planner.  Decode is bound by HBM bandwidth, so its time is the time of the
// longest wave: pick the fewest rounds k of R waves (R = decode_waves_target,
// one per SIMD) for which pieces of at most 64 pages exist, then the
// smallest page count p such that the rows, each cut into ceil(pages/p)
// pieces, give at most k * R waves (piece x KV head x 32 query heads of the
// group: one wave for G <= 32).  Every wave then
// starts in pass 1..k and no wave reads more than p pages.  p is kept at 8 pages or
// more: a shorter piece is mostly start-up latency and lengthens the merge.
int pick_piece_pages(const std::vector<int64_t>& row_pages, int waves_per_piece, int head_dim) {
  constexpr int64_t kMinPages = 8;
  const int64_t max_pages = cpa::kDecodeMaxSplit / cpa::kBlock;
  auto waves = [&](int64_t p) {
    int64_t n = 0;
    for (int64_t pg : row_pages) n += ceil_div(pg, p);
    return n * waves_per_piece;
  };
  const int64_t target = cpa::decode_waves_target(head_dim);
  const int64_t budget = ceil_div(std::max<int64_t>(waves(max_pages), 1), target) * target;
  int64_t lo = kMinPages, hi = max_pages;  // waves(p) is non-increasing in p; waves(hi) <= budget
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (waves(mid) <= budget) hi = mid; else lo = mid + 1;
  }
  return (int)lo;
}

// Pieces per tile for a grid of at most `target` workgroups: none when the
// tiles alone reach it; otherwise each tile's keys are cut into ceil(L / S)
// equal pieces, with S the smallest size (a multiple of the KV tile, at
// least kChunkMinSplit) for which all pieces of all KV heads fit the target.
std::vector<int32_t> pieces_within(const std::vector<int64_t>& tile_keys, int num_kv_heads,
                                   int64_t target) {
  std::vector<int32_t> n(tile_keys.size(), 1);
  if ((int64_t)tile_keys.size() * num_kv_heads >= target) return n;
  int64_t total_keys = 0;
  for (int64_t L : tile_keys) total_keys += L;
  int64_t S = ceil_div(total_keys * num_kv_heads, target);
  S = std::max<int64_t>(ceil_div(S, cpa::kKvTile) * cpa::kKvTile, cpa::kChunkMinSplit);
  for (;;) {
    int64_t pieces = 0;
    for (size_t t = 0; t < tile_keys.size(); ++t) {
      n[t] = (int32_t)std::max<int64_t>(1, ceil_div(tile_keys[t], S));
      pieces += n[t];
    }
    if (pieces * num_kv_heads <= target) return n;
    S += std::max<int64_t>(cpa::kKvTile, S / 16);
  }
}

// Keys' worth of time a piece of a split tile costs beyond its own keys
// (writing its partial output and the merge's read of it), and what a plan with any
// split tile costs once more for the merging.  Both were fitted to same-box
// timings: a one-round step whose causal tiles run up to twice the mean (a
// 2048-token chunk at prefix 0) gains less from splitting than its merges
// cost, and stays unsplit.
constexpr int64_t kPieceCost = 128;
constexpr int64_t kMergeCost = 512;

// Finish time of the chunk launch, in keys, estimated as list scheduling:
// the pieces' workgroups (one per KV head) taken longest first by `slots`
// resident workgroups, each starting the next one when it frees (the order
// the grid is dispatched in).
int64_t estimated_finish(const std::vector<int64_t>& tile_keys, const std::vector<int32_t>& n,
                         int num_kv_heads, int slots) {
  std::vector<int64_t> work;
  for (size_t t = 0; t < tile_keys.size(); ++t)
    for (int32_t k = 0; k < n[t]; ++k)
      work.push_back(ceil_div(tile_keys[t], n[t]) + (n[t] > 1 ? kPieceCost : 0));
  std::sort(work.begin(), work.end(), std::greater<int64_t>());
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0);
  int64_t end = 0;
  for (int64_t w : work)
    for (int h = 0; h < num_kv_heads; ++h) {
      const int64_t t = free_at.top() + w;
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  const bool split = std::any_of(n.begin(), n.end(), [](int32_t k) { return k > 1; });
  return end + (split ? kMergeCost : 0);
}

// Pieces per chunk tile when the caller leaves the split size to the library.
// The base plan fills one resident round (pieces_within the resident slots;
// nothing is split when the tiles alone fill it).  With tiles of very
// different lengths that round waits for its longest piece, so plans of two
// and three rounds of smaller pieces are estimated too, and one replaces the
// base plan when it is estimated to finish in under kSplitGain of the base
// plan's time.  Steps of three rounds of tiles or more are left unsplit
// without estimating (list scheduling balances them).
constexpr double kSplitGain = 0.85;

std::vector<int32_t> pick_chunk_pieces(const std::vector<int64_t>& tile_keys, int num_kv_heads,
                                       int head_dim) {
  const int slots = cpa::chunk_wg_target(head_dim);
  std::vector<int32_t> best = pieces_within(tile_keys, num_kv_heads, slots);
  if ((int64_t)tile_keys.size() * num_kv_heads >= 3LL * slots) return best;
  const int64_t base = estimated_finish(tile_keys, best, num_kv_heads, slots);
  int64_t best_time = base;
  for (int rounds = 2; rounds <= 3; ++rounds) {
    std::vector<int32_t> n = pieces_within(tile_keys, num_kv_heads, (int64_t)rounds * slots);
    const int64_t t = estimated_finish(tile_keys, n, num_kv_heads, slots);
    if (t < kSplitGain * base && t < best_time) {
      best = n;
      best_time = t;
    }
  }
  return best;
}

}  // namespace

extern "C" int cpa_build_metadata(const cpa_req_t* reqs, int n_reqs, const cpa_build_params_t* params,
                                  const int32_t* bt, int bt_stride, int num_blocks, cpa_meta_t* out) {
  int st = check_params(params);
  if (st != CPA_OK) return st;
  if (!out || n_reqs < 0 || (n_reqs > 0 && !reqs)) return CPA_ERR_INVALID;
  if (bt && (bt_stride <= 0 || num_blocks <= 0)) return CPA_ERR_INVALID;

  const int budget = params->token_budget;
  const int policy = params->policy & ~(CPA_POLICY_ADAPTIVE_CHUNK | CPA_POLICY_BLOCK_ALIGNED);
  const bool aligned = params->policy & CPA_POLICY_BLOCK_ALIGNED;
  // most tokens one step can hold (the quota policy may go past the budget)
  const int step_max = budget + (policy == CPA_POLICY_QUOTA ? params->max_prefill_tokens : 0);
  const int group = params->num_q_heads / params->num_kv_heads;

  // validate requests; positions must stay addressable as int32 slot indices
  int n_dec = 0;
  for (int i = 0; i < n_reqs; ++i) {
    const cpa_req_t& r = reqs[i];
    if (r.num_computed < 0) return CPA_ERR_INVALID;
    if (!r.is_decode && r.target_len < r.num_computed) return CPA_ERR_INVALID;
    if (r.num_computed > (INT32_MAX - step_max)) return CPA_ERR_INVALID;
    n_dec += r.is_decode ? 1 : 0;
  }
  if (n_dec > budget) return CPA_ERR_BUDGET;
  const int cap = (params->policy & CPA_POLICY_ADAPTIVE_CHUNK)
                      ? adaptive_cap(params->long_prefill_cap, n_dec)
                      : params->long_prefill_cap;

  // decode-first split of the budget
  std::vector<int32_t> order, nsched;
  order.reserve(n_reqs);
  nsched.reserve(n_reqs);
  for (int i = 0; i < n_reqs; ++i)
    if (reqs[i].is_decode) {
      order.push_back(i);
      nsched.push_back(1);
    }
  // what the prefills may take: the budget left by the decodes, or the
  // quota policy's own prefill budget (cut back once decodes take > 70%)
  int64_t remaining = budget - n_dec;
  if (policy == CPA_POLICY_QUOTA && 10LL * n_dec <= 7LL * budget)
    remaining = params->max_prefill_tokens;
  for (int i = 0; i < n_reqs; ++i) {
    const cpa_req_t& r = reqs[i];
    if (r.is_decode) continue;
    int64_t want = (int64_t)r.target_len - r.num_computed;
    if (cap) want = std::min<int64_t>(want, cap);
    int64_t n;
    if (policy == CPA_POLICY_DEFER) {
      if (want > remaining) break;  // the first prefill that does not fit ends the scan
      n = want;
    } else {
      if (remaining == 0) break;
      n = std::min(want, remaining);
    }
    // a chunk that stops short of its prompt's end may stop on a page boundary
    if (aligned && n > 0 && n < (int64_t)r.target_len - r.num_computed) {
      const int64_t end = (r.num_computed + n) / cpa::kBlock * cpa::kBlock;
      if (end > r.num_computed) n = end - r.num_computed;
    }
    if (n > 0) {
      order.push_back(i);
      nsched.push_back((int32_t)n);
      remaining -= n;
    }
  }

  const int nseq = (int)order.size();
  if (nseq > out->max_seqs) return CPA_ERR_CAPACITY;
  if (!out->order || !out->num_scheduled || !out->query_start_loc || !out->seq_lens ||
      !out->context_lens)
    return CPA_ERR_INVALID;

  int32_t qsl = 0;
  out->query_start_loc[0] = 0;
  for (int s = 0; s < nseq; ++s) {
    const cpa_req_t& r = reqs[order[s]];
    out->order[s] = order[s];
    out->num_scheduled[s] = nsched[s];
    out->context_lens[s] = r.num_computed;
    out->seq_lens[s] = r.num_computed + nsched[s];
    if (out->new_blocks)
      out->new_blocks[s] = (int32_t)(ceil_div(out->seq_lens[s], cpa::kBlock) -
                                     ceil_div(r.num_computed, cpa::kBlock));
    qsl += nsched[s];
    out->query_start_loc[s + 1] = qsl;
  }
  out->num_seqs = nseq;
  out->num_decodes = n_dec;
  out->num_tokens = qsl;

  // optional host block-table checks and slot mapping
  if (bt) {
    if (out->slot_mapping && out->max_tokens < qsl) return CPA_ERR_CAPACITY;
    std::vector<int64_t> fresh, cached;
    fresh.reserve(qsl);
    for (int s = 0; s < nseq; ++s) {
      const int32_t* row = bt + (int64_t)order[s] * bt_stride;
      const int c = out->context_lens[s], L = out->seq_lens[s];
      const int64_t pages = ceil_div(L, cpa::kBlock);
      if (pages > bt_stride) return CPA_ERR_INVALID;
      for (int64_t pg = 0; pg < pages; ++pg)
        if (row[pg] < 0 || row[pg] >= num_blocks) return CPA_ERR_INVALID;
      for (int p = 0; p < L; ++p) {
        int64_t slot = (int64_t)row[p / cpa::kBlock] * cpa::kBlock + p % cpa::kBlock;
        if (p >= c) {
          if (out->slot_mapping) out->slot_mapping[out->query_start_loc[s] + (p - c)] = slot;
          fresh.push_back(slot);
        } else {
          cached.push_back(slot);
        }
      }
    }
    std::sort(fresh.begin(), fresh.end());
    if (std::adjacent_find(fresh.begin(), fresh.end()) != fresh.end()) return CPA_ERR_INVALID;
    // a fresh slot that another row reads as cached context would race with it
    std::sort(cached.begin(), cached.end());
    size_t a = 0, b = 0;
    while (a < fresh.size() && b < cached.size()) {
      if (fresh[a] == cached[b]) return CPA_ERR_INVALID;
      if (fresh[a] < cached[b]) ++a; else ++b;
    }
  }

  // ---- work plan --------------------------------------------------------
  // a row of L keys is cut into n pieces of nearly equal, page-aligned size:
  // n = ceil(L / split) for a caller-given split, else ceil(pages / p) with p
  // from pick_piece_pages.  Pieces are emitted longest first so the last
  // waves to start are short ones.
  std::vector<int64_t> row_pages(n_dec);
  for (int s = 0; s < n_dec; ++s) row_pages[s] = ceil_div(out->seq_lens[s], cpa::kBlock);
  const int split = params->decode_split_tokens;
  const int piece_pages =
      split ? 0
            : pick_piece_pages(row_pages,
                               params->num_kv_heads * cpa::decode_group_waves(group),
                               params->head_dim);
  std::vector<int32_t> dsplits, dmerges, tiles;
  int partials = 0;
  struct DPiece { int32_t row, kb, ke, slot; };
  std::vector<DPiece> dp;
  for (int s = 0; s < n_dec; ++s) {
    const int L = out->seq_lens[s];
    const int64_t pages = row_pages[s];
    const int n = (int)(split ? ceil_div(L, split) : ceil_div(pages, piece_pages));
    if (n == 1) {
      dp.push_back({s, 0, L, -1});
      continue;
    }
    dmerges.insert(dmerges.end(), {s, partials, n, 0});
    for (int k = 0; k < n; ++k) {
      const int32_t kb = (int32_t)(pages * k / n) * cpa::kBlock;
      const int32_t ke = k + 1 < n ? (int32_t)(pages * (k + 1) / n) * cpa::kBlock : L;
      dp.push_back({s, kb, ke, partials + k});
    }
    partials += n;
  }
  std::stable_sort(dp.begin(), dp.end(),
                   [](const DPiece& x, const DPiece& y) { return x.ke - x.kb > y.ke - y.kb; });
  for (const DPiece& p : dp) dsplits.insert(dsplits.end(), {p.row, p.kb, p.ke, p.slot});

  // chunk tiles: chunk_rows(head_dim) (token, head) rows of one KV head each.  Keys below
  // context + q_begin are visible to every row of the tile, so a long prefix
  // may be cut into pieces there; the last piece holds the rest, including
  // the causal diagonal.
  const int tile_tokens = cpa::chunk_tile_tokens(group, params->head_dim);
  struct Tile { int32_t row, qb, qe; int64_t prefix, keys; };
  std::vector<Tile> tl;
  for (int s = n_dec; s < nseq; ++s) {
    const int n = out->num_scheduled[s];
    for (int qb = 0; qb < n; qb += tile_tokens) {
      const int qe = std::min(n, qb + tile_tokens);
      const int64_t c = out->context_lens[s];
      tl.push_back({s, qb, qe, c + qb, c + qe});
    }
  }
  // Inner cut points of each tile's keys [0, keys): multiples of the KV tile,
  // at or before the tile's first query's limit (prefix), so every row of the
  // tile sees at least one key of every piece.  A caller's split size cuts at
  // its multiples; by default the cuts divide the keys into equal pieces.
  std::vector<int32_t> auto_n;
  if (!params->chunk_split_tokens) {
    std::vector<int64_t> keys(tl.size());
    for (size_t i = 0; i < tl.size(); ++i) keys[i] = tl[i].keys;
    auto_n = pick_chunk_pieces(keys, params->num_kv_heads, params->head_dim);
  }
  struct Piece { int32_t row, qb, qe, kb, ke, slot; };
  std::vector<Piece> pieces;
  std::vector<int32_t> cmerges;
  std::vector<int64_t> cuts;
  int cpartials = 0;
  for (size_t i = 0; i < tl.size(); ++i) {
    const Tile& t = tl[i];
    const int64_t last = t.prefix / cpa::kKvTile * cpa::kKvTile;  // latest allowed cut
    cuts.clear();
    if (params->chunk_split_tokens) {
      const int64_t S = params->chunk_split_tokens;
      for (int64_t c = S; c <= t.prefix; c += S) cuts.push_back(c);
    } else {
      const int64_t n = auto_n[i];
      for (int64_t k = 1; k < n; ++k) {
        const int64_t c = std::min(k * t.keys / n / cpa::kKvTile * cpa::kKvTile, last);
        if (c > 0 && (cuts.empty() || c > cuts.back())) cuts.push_back(c);
      }
    }
    const int32_t n = (int32_t)cuts.size() + 1;
    if (n == 1) {
      pieces.push_back({t.row, t.qb, t.qe, 0, (int32_t)t.keys, -1});
      continue;
    }
    cmerges.insert(cmerges.end(), {t.row, t.qb, t.qe, cpartials, n, 0, 0, 0});
    for (int32_t k = 0; k < n; ++k) {
      const int64_t kb = k ? cuts[k - 1] : 0, ke = k + 1 < n ? cuts[k] : t.keys;
      pieces.push_back({t.row, t.qb, t.qe, (int32_t)kb, (int32_t)ke, cpartials + k});
    }
    cpartials += n;
  }
  // longest key range first, so the last workgroups to start are short ones
  std::stable_sort(pieces.begin(), pieces.end(),
                   [](const Piece& x, const Piece& y) { return x.ke - x.kb > y.ke - y.kb; });
  // The chunk grid is (KV head, piece) items, head-major, and each of the 8
  // XCDs runs one contiguous range of them (xcd_remap).  With 8 KV heads an
  // XCD's range is one head's whole list; with fewer, 8 / Hkv XCDs split a
  // head's list into consecutive ranges, and the longest-first order would
  // give the first of them all the long pieces.  Deal the pieces round-robin
  // over those ranges instead (each range stays longest first).
  const int hkv = params->num_kv_heads;
  if (hkv < 8 && 8 % hkv == 0 && pieces.size() > 1) {
    const size_t f = (size_t)(8 / hkv);
    std::vector<Piece> dealt;
    dealt.reserve(pieces.size());
    for (size_t r = 0; r < f; ++r)
      for (size_t j = r; j < pieces.size(); j += f) dealt.push_back(pieces[j]);
    pieces.swap(dealt);
  }
  for (const Piece& p : pieces) tiles.insert(tiles.end(), {p.row, p.qb, p.qe, p.kb, p.ke, p.slot, 0, 0});

  out->counts.num_decode_splits = (int32_t)(dsplits.size() / CPA_DECODE_SPLIT_WORDS);
  out->counts.num_decode_merges = (int32_t)(dmerges.size() / CPA_DECODE_MERGE_WORDS);
  out->counts.num_chunk_tiles = (int32_t)(tiles.size() / CPA_CHUNK_TILE_WORDS);
  out->counts.num_chunk_merges = (int32_t)(cmerges.size() / CPA_CHUNK_MERGE_WORDS);
  out->counts.num_decode_partials = partials;
  out->counts.num_chunk_partials = cpartials;
  const int64_t words = (int64_t)dsplits.size() + dmerges.size() + tiles.size() + cmerges.size();
  if (words > INT32_MAX) return CPA_ERR_CAPACITY;
  out->plan_words = (int32_t)words;
  if (out->plan) {
    if (words > out->plan_capacity) return CPA_ERR_CAPACITY;
    int32_t* w = out->plan;
    for (const std::vector<int32_t>* sec : {&dsplits, &tiles, &dmerges, &cmerges}) {
      std::memcpy(w, sec->data(), sec->size() * sizeof(int32_t));
      w += sec->size();
    }
  }
  return CPA_OK;
}

extern "C" size_t cpa_workspace_size(const cpa_plan_counts_t* counts, int num_q_heads,
                                     int num_kv_heads, int head_dim) {
  if (!counts || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  const cpa::WorkspaceLayout w =
      cpa::workspace_layout(counts->num_decode_partials, counts->num_chunk_partials, num_q_heads,
                            num_kv_heads, head_dim);
  return w.total;
}

extern "C" const char* cpa_status_string(int status) {
  switch (status) {
    case CPA_OK: return "CPA_OK";
    case CPA_ERR_INVALID: return "CPA_ERR_INVALID: malformed input";
    case CPA_ERR_BUDGET: return "CPA_ERR_BUDGET: more running decodes than budget tokens";
    case CPA_ERR_CAPACITY: return "CPA_ERR_CAPACITY: output array or workspace too small";
    case CPA_ERR_UNSUPPORTED: return "CPA_ERR_UNSUPPORTED: shape not supported";
    case CPA_ERR_DEVICE: return "CPA_ERR_DEVICE: kernel launch failed";
    default: return "unknown cpa status";
  }
}
