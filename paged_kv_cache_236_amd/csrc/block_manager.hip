// Host-side KV block manager with prefix caching: hands out the cache blocks
// that the paged kernels address through block_tables and slot_mapping.
//
// The paged KV cache is cut into fixed-size blocks and the scheduler asks a
// block manager for cached blocks (lunaryes/nano-vllm diagram, "Components"
// and "Connections"); full blocks of a prompt that were computed before are
// reused (nano-vllm-sansho README, "Key Features": prefix caching).  The pages
// give no algorithm; this is the plain reading:
//  * a full block is identified by a chain hash of (previous block's hash, its
//    block_size token ids), so its identity covers the whole prefix; its own
//    token ids are kept and compared on every hit as well;
//  * a new sequence reuses the leading run of its prompt's full blocks that are
//    cached (stopping at the first miss) and always computes at least one
//    token: a prompt that is cached in full recomputes its last block into a
//    block of its own;
//  * a block's reference count is the number of sequences holding it; freeing
//    a sequence drops its references, last block first, and a block with none
//    joins the back of the free queue while staying findable by hash until its
//    space is handed out again (least recently freed first);
//  * a decode step appends one token: a sequence that crosses a block boundary
//    gets a new block, and a block that becomes full gets its hash;
//  * a block that became full is pending until pk_bm_commit: its K/V are
//    computed and stored by the step the caller is about to run, so a hit on
//    it in the same step would read rows not yet written (the fused store +
//    prefill writes them inside the very launch that reads the prefix).  The
//    commit, called once the step's kernels are enqueued, makes the pending
//    blocks findable; a pending block that is freed first is dropped.
// Only full blocks are ever shared, so the block a token is written to belongs
// to one sequence.  Host code only: nothing here touches the GPU.
#include <stdint.h>

#include <cstdio>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"

namespace pk {
pk_status record_status(pk_status s, const char* message);   // api.hip

namespace {

constexpr uint64_t kNoHash = 0;   // a block that is not registered

// The splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014) as a 64-bit mixing function.
uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ULL;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebULL;
  x ^= x >> 31;
  return x;
}

uint64_t chain_hash(uint64_t prev, const int32_t* tokens, int32_t n) {
  uint64_t h = mix64(prev + 0x9e3779b97f4a7c15ULL);
  for (int32_t i = 0; i < n; ++i)
    h = mix64(h ^ static_cast<uint64_t>(static_cast<uint32_t>(tokens[i])));
  return h == kNoHash ? 1 : h;
}

struct Block {
  int32_t ref = 0;
  uint64_t hash = kNoHash;        // chain hash of a full block (pending or registered)
  uint32_t gen = 0;               // bumped each time the block joins the free queue
  bool free = true;
  bool pending = false;           // full, hashed, not yet findable (waits for pk_bm_commit)
  std::vector<int32_t> tokens;    // token ids of a full block
};

struct Seq {
  std::vector<int32_t> tokens;    // every token of the sequence so far
  std::vector<int32_t> blocks;    // its block table
  std::vector<uint64_t> hashes;   // chain hash of each of its full blocks
  int32_t num_cached = 0;         // leading tokens whose K/V were reused at allocation
};

}  // namespace
}  // namespace pk

struct pk_block_manager {
  int32_t block_size = 0;
  int32_t num_free = 0;
  std::vector<pk::Block> blocks;
  std::deque<std::pair<int32_t, uint32_t>> free_q;     // (block, gen); stale entries skipped
  // Registered full blocks by chain hash.  Two blocks can hold the same
  // content (a fully cached prompt recomputes its last block), so a hash maps
  // to every holder and evicting one leaves the others findable.
  std::unordered_map<uint64_t, std::vector<int32_t>> by_hash;
  std::unordered_map<int64_t, pk::Seq> seqs;
  std::vector<int32_t> pending;   // blocks filled since the last commit, in fill order
};

namespace pk {
namespace {

pk_status fail(pk_status s, const char* msg) { return record_status(s, msg); }
pk_status ok() { return record_status(PK_OK, ""); }

bool live_entry(const pk_block_manager* m, const std::pair<int32_t, uint32_t>& e) {
  const Block& b = m->blocks[e.first];
  return b.free && b.gen == e.second;
}

void push_free(pk_block_manager* m, int32_t b) {
  Block& blk = m->blocks[b];
  if (blk.pending) {
    // Freed before its step was committed: its rows may never have been
    // written, so it is not offered for reuse (pk_bm_commit skips it).
    blk.pending = false;
    blk.hash = kNoHash;
    blk.tokens.clear();
  }
  blk.free = true;
  ++blk.gen;
  ++m->num_free;
  m->free_q.emplace_back(b, blk.gen);
  // Entries of blocks revived by cache hits stay queued until skipped; drop
  // them once they outnumber the blocks.
  if (m->free_q.size() > 2 * m->blocks.size() + 64) {
    std::deque<std::pair<int32_t, uint32_t>> q;
    for (const auto& e : m->free_q)
      if (live_entry(m, e)) q.push_back(e);
    m->free_q.swap(q);
  }
}

// A cache hit on a block with no holders takes it out of the free pool.
void revive(pk_block_manager* m, int32_t b) {
  m->blocks[b].free = false;
  --m->num_free;
}

// The least recently freed block, emptied for new content (-1 if none).
int32_t take_free(pk_block_manager* m) {
  while (!m->free_q.empty()) {
    const auto e = m->free_q.front();
    m->free_q.pop_front();
    if (!live_entry(m, e)) continue;
    const int32_t b = e.first;
    Block& blk = m->blocks[b];
    if (blk.hash != kNoHash) {
      auto it = m->by_hash.find(blk.hash);
      auto& holders = it->second;
      for (size_t i = 0; i < holders.size(); ++i)
        if (holders[i] == b) {
          holders[i] = holders.back();
          holders.pop_back();
          break;
        }
      if (holders.empty()) m->by_hash.erase(it);
      blk.hash = kNoHash;
      blk.tokens.clear();
    }
    blk.free = false;
    blk.ref = 1;
    --m->num_free;
    return b;
  }
  return -1;
}

void release(pk_block_manager* m, int32_t b) {
  if (--m->blocks[b].ref == 0) push_free(m, b);
}

// A registered block with this chain hash and these tokens, preferring one
// that a sequence holds (so that a hit does not shrink the free pool); -1 if
// there is none.
int32_t lookup(const pk_block_manager* m, uint64_t h, const int32_t* tokens) {
  auto it = m->by_hash.find(h);
  if (it == m->by_hash.end()) return -1;
  int32_t found = -1;
  for (int32_t b : it->second) {
    const Block& blk = m->blocks[b];
    if (std::memcmp(blk.tokens.data(), tokens, sizeof(int32_t) * m->block_size) != 0) continue;
    if (blk.ref > 0) return b;
    if (found < 0) found = b;
  }
  return found;
}

// Hash block `index` of `s`, which has just become (or was born) full, and
// queue it for the next commit (the sequence's chain continues from it at once).
void fill_full(pk_block_manager* m, Seq& s, int32_t index) {
  const int32_t b = s.blocks[index];
  Block& blk = m->blocks[b];
  const uint64_t prev = index > 0 ? s.hashes[index - 1] : 0;
  const int32_t* t = s.tokens.data() + static_cast<int64_t>(index) * m->block_size;
  const uint64_t h = chain_hash(prev, t, m->block_size);
  s.hashes.push_back(h);
  blk.hash = h;
  blk.tokens.assign(t, t + m->block_size);
  blk.pending = true;
  m->pending.push_back(b);
}

const Seq* find_seq(const pk_block_manager* m, int64_t id) {
  auto it = m->seqs.find(id);
  return it == m->seqs.end() ? nullptr : &it->second;
}

}  // namespace
}  // namespace pk

extern "C" {

pk_status pk_bm_create(int32_t num_blocks, int32_t block_size, pk_block_manager** out) {
  if (!out) return pk::fail(PK_ERR_INVALID_ARG, "out must not be NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pk::fail(PK_ERR_INVALID_ARG, "num_blocks and block_size must be > 0");
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return pk::fail(PK_ERR_INVALID_ARG, "num_blocks * block_size must fit an int32 slot index");
  pk_block_manager* m = new (std::nothrow) pk_block_manager();
  if (!m) return pk::fail(PK_ERR_INVALID_ARG, "out of host memory");
  m->block_size = block_size;
  m->blocks.resize(num_blocks);
  m->num_free = num_blocks;
  for (int32_t b = 0; b < num_blocks; ++b) m->free_q.emplace_back(b, 0u);
  *out = m;
  return pk::ok();
}

void pk_bm_destroy(pk_block_manager* m) { delete m; }

pk_status pk_bm_num_free_blocks(const pk_block_manager* m, int32_t* out) {
  if (!m || !out) return pk::fail(PK_ERR_INVALID_ARG, "NULL argument");
  *out = m->num_free;
  return pk::ok();
}

pk_status pk_bm_block_info(const pk_block_manager* m, int32_t block, int32_t* ref_count,
                           int32_t* cached) {
  if (!m || !ref_count || !cached) return pk::fail(PK_ERR_INVALID_ARG, "NULL argument");
  if (block < 0 || block >= static_cast<int32_t>(m->blocks.size()))
    return pk::fail(PK_ERR_INVALID_ARG, "block index out of range");
  const pk::Block& blk = m->blocks[block];
  *ref_count = blk.ref;
  *cached = blk.hash != pk::kNoHash && !blk.pending;
  return pk::ok();
}

pk_status pk_bm_allocate(pk_block_manager* m, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, int32_t* num_cached_tokens) {
  if (!m || !tokens || !num_cached_tokens) return pk::fail(PK_ERR_INVALID_ARG, "NULL argument");
  if (num_tokens <= 0) return pk::fail(PK_ERR_INVALID_ARG, "a sequence needs at least one token");
  if (m->seqs.count(seq_id)) return pk::fail(PK_ERR_INVALID_ARG, "sequence id already allocated");
  const int32_t bs = m->block_size;
  const int32_t nblocks = (num_tokens - 1) / bs + 1;
  const int32_t nfull = num_tokens / bs;
  // The leading full blocks already cached, checked token by token.
  std::vector<int32_t> hits;
  std::vector<uint64_t> hit_hashes;
  uint64_t prev = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    const int32_t* t = tokens + static_cast<int64_t>(i) * bs;
    const uint64_t h = pk::chain_hash(prev, t, bs);
    const int32_t b = pk::lookup(m, h, t);
    if (b < 0) break;
    hits.push_back(b);
    hit_hashes.push_back(h);
    prev = h;
  }
  if (static_cast<int64_t>(hits.size()) * bs >= num_tokens) {
    hits.pop_back();
    hit_hashes.pop_back();
  }
  int32_t revived = 0;
  for (int32_t b : hits) revived += m->blocks[b].ref == 0;
  const int32_t fresh = nblocks - static_cast<int32_t>(hits.size());
  if (m->num_free - revived < fresh) return pk::fail(PK_ERR_WORKSPACE, "not enough free blocks");
  // Nothing below can fail: the manager changes only on success.
  pk::Seq& s = m->seqs[seq_id];
  s.tokens.assign(tokens, tokens + num_tokens);
  s.hashes = hit_hashes;
  for (int32_t b : hits) {
    if (m->blocks[b].ref == 0) pk::revive(m, b);
    ++m->blocks[b].ref;
    s.blocks.push_back(b);
  }
  s.num_cached = static_cast<int32_t>(hits.size()) * bs;
  for (int32_t i = 0; i < fresh; ++i) s.blocks.push_back(pk::take_free(m));
  for (int32_t i = static_cast<int32_t>(hits.size()); i < nfull; ++i) pk::fill_full(m, s, i);
  *num_cached_tokens = s.num_cached;
  return pk::ok();
}

pk_status pk_bm_append(pk_block_manager* m, int64_t seq_id, int32_t token) {
  if (!m) return pk::fail(PK_ERR_INVALID_ARG, "NULL manager");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pk::fail(PK_ERR_INVALID_ARG, "unknown sequence id");
  pk::Seq& s = it->second;
  const int32_t bs = m->block_size;
  const int64_t n = static_cast<int64_t>(s.tokens.size());
  if (n >= INT32_MAX) return pk::fail(PK_ERR_INVALID_ARG, "sequence length overflows int32");
  if (n % bs == 0) {   // the new token opens a block
    const int32_t b = pk::take_free(m);
    if (b < 0) return pk::fail(PK_ERR_WORKSPACE, "not enough free blocks");
    s.blocks.push_back(b);
  }
  s.tokens.push_back(token);
  if ((n + 1) % bs == 0) pk::fill_full(m, s, static_cast<int32_t>(n / bs));
  return pk::ok();
}

pk_status pk_bm_commit(pk_block_manager* m, int32_t* num_registered) {
  if (!m) return pk::fail(PK_ERR_INVALID_ARG, "NULL manager");
  int32_t n = 0;
  for (int32_t b : m->pending) {
    pk::Block& blk = m->blocks[b];
    if (!blk.pending) continue;   // freed (and possibly reused) since it was filled
    blk.pending = false;
    m->by_hash[blk.hash].push_back(b);
    ++n;
  }
  m->pending.clear();
  if (num_registered) *num_registered = n;
  return pk::ok();
}

pk_status pk_bm_free(pk_block_manager* m, int64_t seq_id) {
  if (!m) return pk::fail(PK_ERR_INVALID_ARG, "NULL manager");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pk::fail(PK_ERR_INVALID_ARG, "unknown sequence id");
  const auto& bl = it->second.blocks;
  for (auto b = bl.rbegin(); b != bl.rend(); ++b) pk::release(m, *b);
  m->seqs.erase(it);
  return pk::ok();
}

pk_status pk_bm_seq_info(const pk_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                         int32_t* num_blocks, int32_t* num_cached_tokens) {
  if (!m) return pk::fail(PK_ERR_INVALID_ARG, "NULL manager");
  const pk::Seq* s = pk::find_seq(m, seq_id);
  if (!s) return pk::fail(PK_ERR_INVALID_ARG, "unknown sequence id");
  if (num_tokens) *num_tokens = static_cast<int32_t>(s->tokens.size());
  if (num_blocks) *num_blocks = static_cast<int32_t>(s->blocks.size());
  if (num_cached_tokens) *num_cached_tokens = s->num_cached;
  return pk::ok();
}

pk_status pk_bm_prepare(const pk_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                        const int32_t* num_new, int32_t max_blocks_per_seq,
                        int32_t* block_tables, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                        int32_t* slot_mapping) {
  if (!m || !cu_seqlens_q || !cu_seqlens_k) return pk::fail(PK_ERR_INVALID_ARG, "NULL argument");
  if (num_seqs < 0 || max_blocks_per_seq <= 0)
    return pk::fail(PK_ERR_INVALID_ARG, "num_seqs must be >= 0 and max_blocks_per_seq > 0");
  if (num_seqs > 0 && (!seq_ids || !num_new || !block_tables))
    return pk::fail(PK_ERR_INVALID_ARG, "NULL argument");
  // Check everything before writing anything.
  int64_t total_q = 0, total_k = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pk::Seq* s = pk::find_seq(m, seq_ids[i]);
    if (!s) return pk::fail(PK_ERR_INVALID_ARG, "unknown sequence id");
    if (num_new[i] < 0 || num_new[i] > static_cast<int64_t>(s->tokens.size()))
      return pk::fail(PK_ERR_INVALID_ARG, "num_new outside [0, sequence length]");
    if (static_cast<int64_t>(s->blocks.size()) > max_blocks_per_seq)
      return pk::fail(PK_ERR_INVALID_ARG, "max_blocks_per_seq is smaller than a block table");
    total_q += num_new[i];
    total_k += static_cast<int64_t>(s->tokens.size());
  }
  if (total_q > INT32_MAX || total_k > INT32_MAX)
    return pk::fail(PK_ERR_INVALID_ARG, "token totals overflow int32");
  if (total_q > 0 && !slot_mapping) return pk::fail(PK_ERR_INVALID_ARG, "NULL slot_mapping");
  const int32_t bs = m->block_size;
  cu_seqlens_q[0] = cu_seqlens_k[0] = 0;
  int64_t k = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pk::Seq& s = *pk::find_seq(m, seq_ids[i]);
    const int32_t L = static_cast<int32_t>(s.tokens.size());
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nb ? s.blocks[j] : -1;
    for (int32_t pos = L - num_new[i]; pos < L; ++pos)
      slot_mapping[k++] = s.blocks[pos / bs] * bs + pos % bs;
    cu_seqlens_q[i + 1] = cu_seqlens_q[i] + num_new[i];
    cu_seqlens_k[i + 1] = cu_seqlens_k[i] + L;
  }
  return pk::ok();
}

}  // extern "C"
