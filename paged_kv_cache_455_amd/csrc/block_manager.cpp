// Host-side block manager: the bookkeeping that feeds the device calls.
//
// uml.org.cn "PagedAttention": a request's KV cache is a list of fixed-size
// physical blocks, taken from a free pool as the request grows, and found through
// its block table.  5688vip chapter 3, section 3.2: a new token goes at the end of
// the request's last block; a full block is followed by a fresh one.
// uml.org.cn "Prefix Sharing": requests with the same prompt prefix map it to the
// same physical blocks (reference counted); a request that writes into a shared
// block first gets its own copy of it (copy-on-write).  uml.org.cn "Continuous
// Batching": each step runs whatever requests are active, so the step's block
// tables, lengths and query ranges are rebuilt every step.
//
// The device work of one step runs in this order on one stream: the step's
// copy-on-write pairs (kv_block_copy), the K/V writes of its query tokens, then
// attention.  The manager keeps every hand-out consistent with that order:
//  * a request's query rows in a step are exactly its tokens not yet written, so
//    every token is written once, by the request that holds it;
//  * a block enters the prefix cache only in the step that writes its last token,
//    so a request that hits it in a later step reads written rows;
//  * a request is forked only when all its tokens are written, so two requests
//    never write the same slot in one step;
//  * a step's pairs have unique destinations disjoint from their sources: a
//    destination is a fresh block of a request with unwritten tokens, so it is
//    neither forked nor a cache hit (nor a source) before the step; a source whose
//    last reference goes waits for the step before it is free again; a
//    destination whose last reference goes takes its pair with it.
//
// Swapping (uml.org.cn "PagedAttention": under memory pressure a request's pages
// go out to CPU memory and come back when it runs again) moves the blocks a
// request holds alone to slots of a host pool, and back into fresh device blocks.
// Blocks it shares stay on the device, held by it as before.  A step's device
// work then starts with the swap-outs and the swap-ins (pa_bm_swaps hands them
// out), in that order, before the copy-on-write pairs: a swap-out source freed in
// the phase may be taken again by a swap-in, a copy or a write, all of which run
// after it; a host slot a swap-in reads stays off the host free list until the
// step; a request moves at most once between two steps.  The least recently
// stepped resident request is offered as the victim (pa_bm_lru).
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pa.h"
#include "status.h"

namespace {

uint64_t mix(uint64_t h, uint64_t x) {  // splitmix64 step over the running hash
  h ^= x + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}

// prefix hash through one more full block of bs tokens (0 is kept for "none")
uint64_t chain(uint64_t prev, const int32_t *tokens, int bs) {
  uint64_t h = prev;
  for (int k = 0; k < bs; ++k) h = mix(h, (uint32_t)tokens[k]);
  return h == 0 ? 1 : h;
}

constexpr uint64_t kSeed = 0x6a09e667f3bcc909ull;

struct Request {
  std::vector<int32_t> blocks;  // device block ids, logical order (-1: in a host slot)
  std::vector<int32_t> host;    // host slot of each logical block (-1: on the device)
  std::vector<int32_t> tokens;  // every token so far
  int32_t written = 0;          // leading tokens whose K/V a handed-out step writes
  int32_t published = 0;        // leading full blocks already offered to the cache
  uint64_t hash = kSeed;        // prefix hash through block `published - 1`
  bool swapped = false;         // swapped out: not runnable until swapped in
  bool moved = false;           // swapped out or in since the last step
  int64_t stamp = 0;            // the last step that listed it (LRU order)
};

struct Pair {
  int32_t src, dst;
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t bs = 16;                      // tokens per block (16 or 32)
  std::vector<int32_t> free_list;       // stack of free block ids
  std::vector<int32_t> refs;            // references per block
  std::vector<uint64_t> cached_hash;    // prefix-cache key of a block, 0 if not cached
  std::vector<int32_t> cached_parent;   // block before it in the request that cached it
  std::vector<std::vector<int32_t>> cached_tokens;  // the bs tokens a cached block holds
  std::unordered_map<uint64_t, int32_t> cache;      // hash -> block
  std::unordered_map<int64_t, Request> reqs;
  std::vector<Pair> pending;            // copy-on-write pairs for the next step
  std::vector<int32_t> held;            // freed pending sources, free after the step
  int32_t num_host = 0;
  std::vector<int32_t> host_free;       // stack of free host slots
  std::vector<int32_t> host_held;       // host slots read by pending swap-ins
  std::vector<Pair> swap_out;           // (device block, host slot) for the next step
  std::vector<Pair> swap_in;            // (host slot, device block) for the next step
  std::vector<int64_t> moved_reqs;      // requests with `moved` set
  int64_t steps = 0;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] > 0) return;
    if (cached_hash[b] != 0) {
      auto it = cache.find(cached_hash[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      cached_hash[b] = 0;
    }
    for (const Pair &p : pending)
      if (p.src == b) {  // its step-start rows are still to be copied
        held.push_back(b);
        return;
      }
    const auto to_b = [b](const Pair &p) { return p.dst == b; };
    pending.erase(std::remove_if(pending.begin(), pending.end(), to_b), pending.end());
    swap_in.erase(std::remove_if(swap_in.begin(), swap_in.end(), to_b), swap_in.end());
    free_list.push_back(b);
  }
  void mark_moved(int64_t id, Request &r) {
    r.moved = true;
    moved_reqs.push_back(id);
  }
  // offer request r's full blocks to the prefix cache (first holder of a hash wins)
  void publish(Request &r) {
    const int32_t full = r.written / bs;
    for (; r.published < full; ++r.published) {
      const int32_t i = r.published;
      r.hash = chain(r.hash, r.tokens.data() + (size_t)i * bs, bs);
      const int32_t b = r.blocks[i];
      if (cache.count(r.hash) != 0 || cached_hash[b] != 0) continue;
      cache.emplace(r.hash, b);
      cached_hash[b] = r.hash;
      cached_parent[b] = i == 0 ? -1 : r.blocks[i - 1];
      cached_tokens[b].assign(r.tokens.begin() + (size_t)i * bs,
                              r.tokens.begin() + (size_t)(i + 1) * bs);
    }
  }
  // Append tokens to r: fresh blocks at block boundaries, a private copy of a
  // shared last block before writing into it.  Fails (changing nothing) when the
  // free list cannot cover it.
  pa_status_t append(Request &r, const int32_t *tokens, int32_t n) {
    if (n == 0) return PA_OK;
    const int32_t len = (int32_t)r.tokens.size();
    const int32_t have = (int32_t)r.blocks.size();
    int32_t needed = (len + n + bs - 1) / bs - have;
    const bool cow = len % bs != 0 && refs[r.blocks.back()] > 1;
    if (cow) ++needed;
    if (needed > (int32_t)free_list.size())
      return pa::set_error(PA_E_NO_BLOCKS, "no free block for the request's new tokens");
    if (cow) {
      const int32_t src = r.blocks.back();
      const int32_t dst = take();
      pending.push_back({src, dst});
      r.blocks.back() = dst;
      drop(src);  // still referenced by the other holders
    }
    for (int32_t i = 0; i < n; ++i) {
      if ((int32_t)r.tokens.size() == (int32_t)r.blocks.size() * bs) {
        r.blocks.push_back(take());
        r.host.push_back(-1);
      }
      r.tokens.push_back(tokens[i]);
    }
    return PA_OK;
  }
};

extern "C" {

pa_block_manager_t *pa_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size) {
  if (num_blocks <= 0 || num_host_blocks < 0 || (block_size != 16 && block_size != 32))
    return nullptr;
  pa_block_manager *bm = new (std::nothrow) pa_block_manager();
  if (bm == nullptr) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->bs = block_size;
    bm->free_list.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = num_blocks - 1 - i;  // 0 first
    bm->refs.assign(num_blocks, 0);
    bm->cached_hash.assign(num_blocks, 0);
    bm->cached_parent.assign(num_blocks, -1);
    bm->cached_tokens.resize(num_blocks);
    bm->num_host = num_host_blocks;
    bm->host_free.resize(num_host_blocks);
    for (int32_t i = 0; i < num_host_blocks; ++i) bm->host_free[i] = num_host_blocks - 1 - i;
  } catch (const std::bad_alloc &) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager_t *bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager_t *bm) {
  return bm ? (int32_t)bm->free_list.size() : -1;
}

int32_t pa_bm_num_free_host(const pa_block_manager_t *bm) {
  return bm ? (int32_t)bm->host_free.size() : -1;
}

int32_t pa_bm_refcount(const pa_block_manager_t *bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refs[block];
}

pa_status_t pa_bm_add(pa_block_manager_t *bm, int64_t req, const int32_t *tokens, int32_t n,
                      int32_t *cached) {
  if (!bm || !tokens || n < 1) return pa::set_error(PA_E_ARG, "pa_bm_add: bad argument");
  if (bm->reqs.count(req)) return pa::set_error(PA_E_ARG, "pa_bm_add: request id already in use");
  // leading full blocks found in the prefix cache; a hit must hold the same 16
  // tokens and follow the block matched before it, so the whole prefix is equal.
  // The last prompt token is always computed: at most (n - 1) / bs blocks reused.
  const int bs = bm->bs;
  const int32_t max_hit = (n - 1) / bs;
  std::vector<int32_t> shared;
  uint64_t h = kSeed;
  for (int32_t i = 0; i < max_hit; ++i) {
    const uint64_t key = chain(h, tokens + (size_t)i * bs, bs);
    auto it = bm->cache.find(key);
    if (it == bm->cache.end()) break;
    const int32_t b = it->second;
    if (bm->cached_parent[b] != (i == 0 ? -1 : shared.back())) break;
    if (!std::equal(bm->cached_tokens[b].begin(), bm->cached_tokens[b].end(),
                    tokens + (size_t)i * bs))
      break;
    shared.push_back(b);
    h = key;
  }
  const int32_t hit = (int32_t)shared.size();
  const int32_t fresh = (n + bs - 1) / bs - hit;
  if (fresh > (int32_t)bm->free_list.size())
    return pa::set_error(PA_E_NO_BLOCKS, "pa_bm_add: not enough free blocks for the prompt");
  for (int32_t b : shared) ++bm->refs[b];
  Request r;
  r.blocks = shared;
  r.host.assign(shared.size(), -1);
  r.stamp = bm->steps;
  r.tokens.assign(tokens, tokens + (size_t)hit * bs);
  r.written = hit * bs;
  r.published = hit;
  r.hash = h;
  Request &rr = bm->reqs.emplace(req, std::move(r)).first->second;
  bm->append(rr, tokens + (size_t)hit * bs, n - hit * bs);  // fits: checked
  if (cached) *cached = hit * bs;
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_block_manager_t *bm, int64_t parent, int64_t child) {
  if (!bm) return pa::set_error(PA_E_ARG, "pa_bm_fork: NULL manager");
  auto it = bm->reqs.find(parent);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_fork: unknown parent");
  if (bm->reqs.count(child)) return pa::set_error(PA_E_ARG, "pa_bm_fork: child id in use");
  if (it->second.swapped) return pa::set_error(PA_E_ARG, "pa_bm_fork: the parent is swapped out");
  if (it->second.written != (int32_t)it->second.tokens.size())
    return pa::set_error(PA_E_ARG, "pa_bm_fork: the parent has tokens no step has written yet");
  Request c = it->second;
  c.moved = false;
  for (int32_t b : c.blocks) ++bm->refs[b];
  bm->reqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status_t pa_bm_append(pa_block_manager_t *bm, int64_t req, const int32_t *tokens, int32_t n) {
  if (!bm || n < 0 || (!tokens && n > 0)) return pa::set_error(PA_E_ARG, "pa_bm_append: bad argument");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_append: unknown request");
  if (it->second.swapped) return pa::set_error(PA_E_ARG, "pa_bm_append: request is swapped out");
  return bm->append(it->second, tokens, n);
}

pa_status_t pa_bm_release(pa_block_manager_t *bm, int64_t req) {
  if (!bm) return pa::set_error(PA_E_ARG, "pa_bm_release: NULL manager");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_release: unknown request");
  const Request &r = it->second;
  for (size_t i = 0; i < r.blocks.size(); ++i) {
    if (r.host[i] < 0) {
      bm->drop(r.blocks[i]);
      continue;
    }
    const int32_t h = r.host[i];  // its swap-out, if still pending, is not needed now
    bm->swap_out.erase(std::remove_if(bm->swap_out.begin(), bm->swap_out.end(),
                                      [h](const Pair &p) { return p.dst == h; }),
                       bm->swap_out.end());
    bm->host_free.push_back(h);
  }
  bm->reqs.erase(it);
  return PA_OK;
}

pa_status_t pa_bm_swap_out(pa_block_manager_t *bm, int64_t req, int32_t *moved) {
  if (!bm) return pa::set_error(PA_E_ARG, "pa_bm_swap_out: NULL manager");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_swap_out: unknown request");
  Request &r = it->second;
  if (r.swapped) return pa::set_error(PA_E_ARG, "pa_bm_swap_out: already swapped out");
  if (r.moved) return pa::set_error(PA_E_ARG, "pa_bm_swap_out: request moved since the last step");
  if (r.written != (int32_t)r.tokens.size())
    return pa::set_error(PA_E_ARG, "pa_bm_swap_out: the request has tokens no step has written yet");
  int32_t alone = 0;
  for (int32_t b : r.blocks) alone += bm->refs[b] == 1;
  if (alone > (int32_t)bm->host_free.size())
    return pa::set_error(PA_E_NO_BLOCKS, "pa_bm_swap_out: %d host slots needed, %d free", alone,
                         (int32_t)bm->host_free.size());
  for (size_t i = 0; i < r.blocks.size(); ++i) {
    const int32_t b = r.blocks[i];
    if (bm->refs[b] != 1) continue;  // shared: stays on the device
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    bm->swap_out.push_back({b, h});
    r.host[i] = h;
    r.blocks[i] = -1;
    bm->drop(b);
  }
  r.swapped = true;
  bm->mark_moved(req, r);
  if (moved) *moved = alone;
  return PA_OK;
}

pa_status_t pa_bm_swap_in(pa_block_manager_t *bm, int64_t req) {
  if (!bm) return pa::set_error(PA_E_ARG, "pa_bm_swap_in: NULL manager");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_swap_in: unknown request");
  Request &r = it->second;
  if (!r.swapped) return pa::set_error(PA_E_ARG, "pa_bm_swap_in: not swapped out");
  if (r.moved) return pa::set_error(PA_E_ARG, "pa_bm_swap_in: request moved since the last step");
  int32_t out = 0;
  for (int32_t h : r.host) out += h >= 0;
  if (out > (int32_t)bm->free_list.size())
    return pa::set_error(PA_E_NO_BLOCKS, "pa_bm_swap_in: %d device blocks needed, %d free", out,
                         (int32_t)bm->free_list.size());
  for (size_t i = 0; i < r.blocks.size(); ++i) {
    const int32_t h = r.host[i];
    if (h < 0) continue;
    const int32_t d = bm->take();
    bm->swap_in.push_back({h, d});
    bm->host_held.push_back(h);
    r.blocks[i] = d;
    r.host[i] = -1;
  }
  r.swapped = false;
  bm->mark_moved(req, r);
  return PA_OK;
}

pa_status_t pa_bm_lru(const pa_block_manager_t *bm, int64_t *req) {
  if (!bm || !req) return pa::set_error(PA_E_ARG, "pa_bm_lru: bad argument");
  bool found = false;
  int64_t best = 0, best_stamp = 0;
  for (const auto &kv : bm->reqs) {
    const Request &r = kv.second;
    if (r.swapped || r.moved || r.written != (int32_t)r.tokens.size()) continue;
    if (!found || r.stamp < best_stamp || (r.stamp == best_stamp && kv.first < best)) {
      found = true;
      best = kv.first;
      best_stamp = r.stamp;
    }
  }
  if (!found) return pa::set_error(PA_E_NO_BLOCKS, "pa_bm_lru: no resident request to swap out");
  *req = best;
  return PA_OK;
}

pa_status_t pa_bm_blocks(const pa_block_manager_t *bm, int64_t req, int32_t *device_blocks,
                         int32_t *host_slots, int32_t max_blocks, int32_t *num_blocks) {
  if (!bm || !num_blocks || max_blocks < 0) return pa::set_error(PA_E_ARG, "pa_bm_blocks: bad argument");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_blocks: unknown request");
  const Request &r = it->second;
  const int32_t n = (int32_t)r.blocks.size();
  if (n > max_blocks || (n > 0 && (!device_blocks || !host_slots)))
    return pa::set_error(PA_E_ARG, "pa_bm_blocks: %d blocks, room for %d", n, max_blocks);
  for (int32_t i = 0; i < n; ++i) {
    device_blocks[i] = r.blocks[i];
    host_slots[i] = r.host[i];
  }
  *num_blocks = n;
  return PA_OK;
}

pa_status_t pa_bm_swaps(pa_block_manager_t *bm, int32_t *out_pairs, int32_t max_out,
                        int32_t *num_out, int32_t *in_pairs, int32_t max_in, int32_t *num_in) {
  if (!bm || !num_out || !num_in || max_out < 0 || max_in < 0)
    return pa::set_error(PA_E_ARG, "pa_bm_swaps: bad argument");
  const int32_t no = (int32_t)bm->swap_out.size(), ni = (int32_t)bm->swap_in.size();
  if (no > max_out || ni > max_in || (no > 0 && !out_pairs) || (ni > 0 && !in_pairs))
    return pa::set_error(PA_E_ARG, "pa_bm_swaps: %d out / %d in pairs pending, room for %d / %d",
                         no, ni, max_out, max_in);
  for (int32_t i = 0; i < no; ++i) {
    out_pairs[2 * i] = bm->swap_out[i].src;
    out_pairs[2 * i + 1] = bm->swap_out[i].dst;
  }
  for (int32_t i = 0; i < ni; ++i) {
    in_pairs[2 * i] = bm->swap_in[i].src;
    in_pairs[2 * i + 1] = bm->swap_in[i].dst;
  }
  *num_out = no;
  *num_in = ni;
  bm->swap_out.clear();
  bm->swap_in.clear();
  return PA_OK;
}

pa_status_t pa_bm_step(pa_block_manager_t *bm, const int64_t *reqs, int32_t n,
                       int32_t max_blocks_per_seq, int32_t *block_tables, int32_t *seq_lens,
                       int32_t *query_start_loc, int32_t *copy_pairs, int32_t max_pairs,
                       int32_t *num_pairs) {
  if (!bm || n < 0 || max_blocks_per_seq <= 0 || max_pairs < 0 || !num_pairs ||
      !query_start_loc || (n > 0 && (!reqs || !block_tables || !seq_lens)))
    return pa::set_error(PA_E_ARG, "pa_bm_step: bad argument");
  if (!bm->swap_out.empty() || !bm->swap_in.empty())
    return pa::set_error(PA_E_ARG, "pa_bm_step: swap pairs pending; pa_bm_swaps hands them out first");
  const int32_t pairs = (int32_t)bm->pending.size();
  if (pairs > max_pairs || (pairs > 0 && !copy_pairs))
    return pa::set_error(PA_E_ARG, "pa_bm_step: %d copy pairs pending, room for %d", pairs,
                         max_pairs);
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->reqs.find(reqs[i]);
    if (it == bm->reqs.end()) return pa::set_error(PA_E_ARG, "pa_bm_step: unknown request");
    if (!seen.insert(reqs[i]).second)
      return pa::set_error(PA_E_ARG, "pa_bm_step: request listed twice");
    const Request &r = it->second;
    if (r.swapped) return pa::set_error(PA_E_ARG, "pa_bm_step: request is swapped out");
    if ((int32_t)r.blocks.size() > max_blocks_per_seq)
      return pa::set_error(PA_E_ARG, "pa_bm_step: request needs %d blocks > %d",
                           (int32_t)r.blocks.size(), max_blocks_per_seq);
    if (r.written == (int32_t)r.tokens.size())
      return pa::set_error(PA_E_ARG, "pa_bm_step: request has no new token");
  }
  int32_t q = 0;
  ++bm->steps;
  for (int32_t i = 0; i < n; ++i) {
    Request &r = bm->reqs.find(reqs[i])->second;
    r.stamp = bm->steps;
    int32_t *row = block_tables + (int64_t)i * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)r.blocks.size() ? r.blocks[j] : -1;
    const int32_t len = (int32_t)r.tokens.size();
    seq_lens[i] = len;
    query_start_loc[i] = q;
    q += len - r.written;
    r.written = len;
    bm->publish(r);
  }
  query_start_loc[n] = q;
  for (int32_t i = 0; i < pairs; ++i) {
    copy_pairs[2 * i] = bm->pending[i].src;
    copy_pairs[2 * i + 1] = bm->pending[i].dst;
  }
  *num_pairs = pairs;
  bm->pending.clear();
  for (int32_t b : bm->held) bm->free_list.push_back(b);
  bm->held.clear();
  for (int32_t h : bm->host_held) bm->host_free.push_back(h);
  bm->host_held.clear();
  for (int64_t id : bm->moved_reqs) {
    auto it = bm->reqs.find(id);
    if (it != bm->reqs.end()) it->second.moved = false;
  }
  bm->moved_reqs.clear();
  return PA_OK;
}

}  // extern "C"
