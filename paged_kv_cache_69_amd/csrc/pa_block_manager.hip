// Host-side block manager: the pool's free list and reference counts, per-sequence block tables
// with copy-on-write, and the prefix cache ([P1] "25. Paged attention and prefix caching", sections
// "The allocator", "The paged cache", "Sharing blocks: forks and copy-on-write", "Prefix caching";
// [P2] "Модуль 09: PagedAttention: пейджинг KV-кэша", section 4). Host code only: it decides which
// physical blocks hold what; the block copies that copy-on-write needs are returned to the caller,
// who runs them on the GPU with pa_copy_blocks before writing.
//
// Prefix cache layout: a trie over full blocks. The node of a block stands for the whole token
// prefix that ends with that block (its parent is the prefix before it), so two blocks with equal
// tokens but different histories are different nodes, with no hashing collisions. A node holds the
// cached physical block, if any, and its place in the least-recently-used list. Nodes without a
// block stay while they have children (a later lookup still walks through them) and are removed
// when the last child goes.
#include <stdint.h>

#include <deque>
#include <list>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

struct TokensHash {
  size_t operator()(const std::vector<int32_t>& v) const {
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the 32-bit tokens
    for (int32_t t : v) {
      h ^= (uint32_t)t;
      h *= 1099511628211ull;
    }
    return (size_t)h;
  }
};

struct Node {
  Node* parent = nullptr;
  std::vector<int32_t> tokens;  // this block's tokens (the key under the parent)
  std::unordered_map<std::vector<int32_t>, std::unique_ptr<Node>, TokensHash> children;
  int32_t block = -1;           // cached physical block, or -1
  std::list<Node*>::iterator lru;
};

struct Seq {
  std::vector<int32_t> table;
  int32_t length = 0;
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;  // first in, first out
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Seq> seqs;
  Node root;
  std::list<Node*> lru;  // front: least recently used cache entry
  int32_t entries = 0;

  int32_t blocks_for(int64_t tokens) const { return (int32_t)((tokens + block_size - 1) / block_size); }

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }

  // Remove nodes that hold no block and have no children, walking up from n.
  void collect(Node* n) {
    while (n != &root && n->block < 0 && n->children.empty()) {
      Node* up = n->parent;
      const std::vector<int32_t> key = n->tokens;
      up->children.erase(key);  // destroys n
      n = up;
    }
  }
};

namespace {

Seq* find_seq(pa_block_manager* m, int64_t id) {
  auto it = m->seqs.find(id);
  return it == m->seqs.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->refs.assign((size_t)num_blocks, 0);
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_num_free(const pa_block_manager* m) { return m ? (int32_t)m->free_list.size() : PA_ERR_INVALID_ARG; }

int32_t pa_bm_refcount(const pa_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return PA_ERR_INVALID_ARG;
  return m->refs[block];
}

int pa_bm_add_seq(pa_block_manager* m, int64_t seq) {
  if (!m || m->seqs.count(seq)) return PA_ERR_INVALID_ARG;
  m->seqs.emplace(seq, Seq{});
  return PA_OK;
}

int pa_bm_reserve(pa_block_manager* m, int64_t seq, int32_t new_tokens, int32_t* copies, int32_t copies_capacity,
                  int32_t* num_copies) {
  if (!m || new_tokens < 0 || !num_copies) return PA_ERR_INVALID_ARG;
  Seq* s = find_seq(m, seq);
  if (!s) return PA_ERR_INVALID_ARG;
  *num_copies = 0;
  if (new_tokens == 0) return PA_OK;  // nothing is written, so nothing needs a private copy
  const int64_t end = (int64_t)s->length + new_tokens;
  const int32_t want = m->blocks_for(end);
  const int32_t have = (int32_t)s->table.size();
  std::vector<int32_t> shared;  // table slots about to be written whose block others reference
  for (int32_t j = s->length / m->block_size; j < (have < want ? have : want); ++j)
    if (m->refs[s->table[j]] > 1) shared.push_back(j);
  const int64_t grow = want > have ? want - have : 0;
  if ((int64_t)shared.size() + grow > (int64_t)m->free_list.size()) return PA_ERR_NO_BLOCKS;
  if ((int32_t)shared.size() > copies_capacity || (!shared.empty() && !copies)) return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  for (int32_t j : shared) {
    const int32_t fresh = m->take();
    copies[2 * n] = s->table[j];
    copies[2 * n + 1] = fresh;
    ++n;
    m->drop(s->table[j]);
    s->table[j] = fresh;
  }
  for (int64_t k = 0; k < grow; ++k) s->table.push_back(m->take());
  *num_copies = n;
  return PA_OK;
}

int pa_bm_commit(pa_block_manager* m, int64_t seq, int32_t length) {
  Seq* s = m ? find_seq(m, seq) : nullptr;
  if (!s || length < 0 || (int64_t)length > (int64_t)s->table.size() * m->block_size) return PA_ERR_INVALID_ARG;
  if (length > s->length) s->length = length;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m || parent == child || m->seqs.count(child)) return PA_ERR_INVALID_ARG;
  Seq* p = find_seq(m, parent);
  if (!p) return PA_ERR_INVALID_ARG;
  Seq c = *p;  // copy first: emplace may rehash and move *p
  for (int32_t b : c.table) ++m->refs[b];
  m->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_bm_free_seq(pa_block_manager* m, int64_t seq) {
  Seq* s = m ? find_seq(m, seq) : nullptr;
  if (!s) return PA_ERR_INVALID_ARG;
  for (int32_t b : s->table) m->drop(b);
  m->seqs.erase(seq);
  return PA_OK;
}

int pa_bm_truncate(pa_block_manager* m, int64_t seq, int32_t length) {
  Seq* s = m ? find_seq(m, seq) : nullptr;
  if (!s || length < 0 || length > s->length) return PA_ERR_INVALID_ARG;
  const int32_t keep = m->blocks_for(length);
  for (size_t j = (size_t)keep; j < s->table.size(); ++j) m->drop(s->table[j]);
  s->table.resize((size_t)keep);
  s->length = length;
  return PA_OK;
}

int32_t pa_bm_seq_length(const pa_block_manager* m, int64_t seq) {
  if (!m) return PA_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq);
  return it == m->seqs.end() ? PA_ERR_INVALID_ARG : it->second.length;
}

int32_t pa_bm_seq_blocks(const pa_block_manager* m, int64_t seq, int32_t* out, int32_t capacity) {
  if (!m) return PA_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_INVALID_ARG;
  const std::vector<int32_t>& t = it->second.table;
  if (out) {
    if ((int32_t)t.size() > capacity) return PA_ERR_INVALID_ARG;
    for (size_t j = 0; j < t.size(); ++j) out[j] = t[j];
  }
  return (int32_t)t.size();
}

int pa_bm_build_tables(const pa_block_manager* m, const int64_t* seqs, int32_t num_seqs, int32_t width, int32_t pad,
                       int32_t* tables, int32_t* lengths) {
  if (!m || num_seqs < 0 || width < 1 || (num_seqs > 0 && (!seqs || !tables || !lengths))) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {  // validate everything before writing anything
    auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end() || (int32_t)it->second.table.size() > width) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = m->seqs.find(seqs[i])->second;
    int32_t* row = tables + (int64_t)i * width;
    for (int32_t j = 0; j < width; ++j) row[j] = j < (int32_t)s.table.size() ? s.table[j] : pad;
    lengths[i] = s.length;
  }
  return PA_OK;
}

int32_t pa_bm_prefix_attach(pa_block_manager* m, int64_t seq, const int32_t* tokens, int32_t num_tokens) {
  if (!m || num_tokens < 0 || (num_tokens > 0 && !tokens) || m->seqs.count(seq)) return PA_ERR_INVALID_ARG;
  Seq s;
  const int32_t b = m->block_size;
  Node* node = &m->root;
  int32_t reused = 0;
  std::vector<int32_t> key((size_t)b);
  while ((int64_t)reused + b <= (int64_t)num_tokens - 1) {  // one prompt token is always left to prefill
    key.assign(tokens + reused, tokens + reused + b);
    auto it = node->children.find(key);
    if (it == node->children.end() || it->second->block < 0) break;
    Node* child = it->second.get();
    m->lru.splice(m->lru.end(), m->lru, child->lru);  // most recently used
    ++m->refs[child->block];
    s.table.push_back(child->block);
    reused += b;
    node = child;
  }
  s.length = reused;
  m->seqs.emplace(seq, std::move(s));
  return reused;
}

int32_t pa_bm_prefix_remember(pa_block_manager* m, int64_t seq, const int32_t* tokens, int32_t num_tokens) {
  Seq* s = m ? find_seq(m, seq) : nullptr;
  if (!s || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
  const int32_t b = m->block_size;
  const int32_t full = num_tokens / b;
  if (full > (int32_t)s->table.size()) return PA_ERR_INVALID_ARG;
  Node* node = &m->root;
  int32_t published = 0;
  for (int32_t j = 0; j < full; ++j) {
    std::vector<int32_t> key(tokens + (int64_t)j * b, tokens + (int64_t)(j + 1) * b);
    auto it = node->children.find(key);
    Node* child;
    if (it == node->children.end()) {
      auto fresh = std::make_unique<Node>();
      fresh->parent = node;
      fresh->tokens = key;
      child = fresh.get();
      node->children.emplace(std::move(key), std::move(fresh));
    } else {
      child = it->second.get();
    }
    if (child->block < 0) {
      child->block = s->table[j];
      ++m->refs[child->block];
      child->lru = m->lru.insert(m->lru.end(), child);
      ++m->entries;
      ++published;
    }
    node = child;
  }
  return published;
}

int32_t pa_bm_prefix_evict(pa_block_manager* m, int32_t blocks_wanted) {
  if (!m) return PA_ERR_INVALID_ARG;
  for (auto it = m->lru.begin(); it != m->lru.end();) {
    if ((int64_t)m->free_list.size() >= blocks_wanted) break;
    Node* n = *it;
    if (m->refs[n->block] == 1) {  // only the cache holds it
      it = m->lru.erase(it);
      --m->entries;
      m->drop(n->block);
      n->block = -1;
      m->collect(n);
    } else {
      ++it;
    }
  }
  return (int32_t)m->free_list.size();
}

int32_t pa_bm_prefix_entries(const pa_block_manager* m) { return m ? m->entries : PA_ERR_INVALID_ARG; }

int32_t pa_bm_num_seqs(const pa_block_manager* m) { return m ? (int32_t)m->seqs.size() : PA_ERR_INVALID_ARG; }

}  // extern "C"
