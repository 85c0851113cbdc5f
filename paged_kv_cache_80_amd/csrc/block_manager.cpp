// block_manager.cpp -- host-side KV-cache block allocation (declared in
// include/pkv_blocks.h), after the three-layer design of the "KV Cache
// management design document" page: BlockPool (section 2.4), one manager per
// attention type (section 2.3: full attention, sliding window), and the
// request-level two-phase allocate_slots (sections 2.2 and 3).
//
// Host C++ only: no device memory, no HIP calls.  Ids are int32 (the block
// table's type); request ids are any int64.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_blocks.h"
#include "pkv_error.h"

namespace {

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pkv::set_last_error(buf);
  return s;
}

pkv_status ok() {
  pkv::clear_last_error();
  return PKV_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Every C entry point runs its body through this: host allocations (queues,
// tables, strings) may throw, and no exception may cross the C ABI.
template <typename F>
pkv_status guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  } catch (...) {
    return fail(PKV_ERR_INVALID_ARG, "unexpected host error");
  }
}

// Section 2.4: ids 0..n-1 queued in order; the first one popped is the null
// block; issue from the head, return to the tail; `is_free` is the set that
// catches double frees in O(1).
class BlockPool {
 public:
  explicit BlockPool(int32_t num_blocks) : num_blocks_(num_blocks), is_free_(num_blocks, 1) {
    for (int32_t b = 1; b < num_blocks; ++b) queue_.push_back(b);
    null_block_ = 0;
    is_free_[0] = 0;
  }
  int32_t num_blocks() const { return num_blocks_; }
  int32_t null_block() const { return null_block_; }
  int32_t num_free() const { return (int32_t)queue_.size(); }

  bool get_new_blocks(int32_t n, int32_t* out) {
    if (n < 0 || n > num_free()) return false;
    for (int32_t i = 0; i < n; ++i) {
      out[i] = queue_.front();
      queue_.pop_front();
      is_free_[out[i]] = 0;
    }
    return true;
  }

  // Checks the whole list first, so a rejected call changes nothing; the bad
  // id goes to *bad.
  bool free_blocks(const int32_t* ids, int32_t n, int32_t* bad) {
    std::vector<int32_t> marked;
    bool good = true;
    for (int32_t i = 0; i < n && good; ++i) {
      const int32_t b = ids[i];
      if (b < 0 || b >= num_blocks_ || b == null_block_ || is_free_[b]) {
        *bad = b;
        good = false;
        break;
      }
      is_free_[b] = 2;  // seen in this list: a repeat is a double free
      marked.push_back(b);
    }
    for (int32_t b : marked) is_free_[b] = 0;
    if (!good) return false;
    for (int32_t i = 0; i < n; ++i) {
      queue_.push_back(ids[i]);
      is_free_[ids[i]] = 1;
    }
    return true;
  }

 private:
  int32_t num_blocks_;
  int32_t null_block_;
  std::deque<int32_t> queue_;
  std::vector<uint8_t> is_free_;
};

// Section 2.3: the blocks of one attention type.
class TypeManager {
 public:
  TypeManager(int32_t attn_type, int32_t num_blocks, int32_t block_size, int32_t window)
      : attn_type_(attn_type), block_size_(block_size), window_(window), pool_(num_blocks) {}

  int32_t attn_type() const { return attn_type_; }
  BlockPool& pool() { return pool_; }
  const BlockPool& pool() const { return pool_; }

  // 2.3.1: full attention skips nothing; 2.3.2: with c tokens computed, the next
  // query (position c) sees c - W + 1 .. c, so the first c - W + 1 are skipped.
  int64_t skipped_tokens(int64_t computed) const {
    if (attn_type_ == PKV_ATTN_FULL) return 0;
    return computed - window_ + 1 > 0 ? computed - window_ + 1 : 0;
  }
  int64_t skipped_blocks(int64_t computed) const { return skipped_tokens(computed) / block_size_; }

  const std::vector<int32_t>* blocks_of(int64_t req) const {
    const auto it = req_to_blocks_.find(req);
    return it == req_to_blocks_.end() ? nullptr : &it->second;
  }

  // Entries past the held ones up to ceil(need / bs), minus those that fall
  // wholly inside the skipped tokens (they take the null block).
  int64_t blocks_to_allocate(int64_t req, int64_t need, int64_t computed) const {
    const std::vector<int32_t>* b = blocks_of(req);
    const int64_t required = ceil_div(need, block_size_);
    const int64_t existing = b ? (int64_t)b->size() : 0;
    const int64_t first_real = existing > skipped_blocks(computed) ? existing : skipped_blocks(computed);
    return required > first_real ? required - first_real : 0;
  }

  // Phase 2: cannot fail once blocks_to_allocate passed the free-block check.
  void allocate_new_blocks(int64_t req, int64_t need, int64_t computed) {
    std::vector<int32_t>& b = req_to_blocks_[req];
    const int64_t required = ceil_div(need, block_size_);
    const int64_t skipped = skipped_blocks(computed);
    while ((int64_t)b.size() < required && (int64_t)b.size() < skipped) b.push_back(pool_.null_block());
    const int64_t n = required - (int64_t)b.size();
    if (n > 0) {
      const size_t at = b.size();
      b.resize(at + (size_t)n);
      pool_.get_new_blocks((int32_t)n, b.data() + at);
    }
  }

  // Entries that slid out of every future window become the null block; walk
  // back from the last skipped entry, stop at the first null (those before it
  // were dropped earlier) and free in that order.
  void remove_skipped_blocks(int64_t req, int64_t computed) {
    const auto it = req_to_blocks_.find(req);
    if (it == req_to_blocks_.end()) return;
    std::vector<int32_t>& b = it->second;
    const int64_t skipped = skipped_blocks(computed);
    std::vector<int32_t> freed;
    for (int64_t i = (skipped < (int64_t)b.size() ? skipped : (int64_t)b.size()) - 1; i >= 0; --i) {
      if (b[i] == pool_.null_block()) break;
      freed.push_back(b[i]);
      b[i] = pool_.null_block();
    }
    int32_t bad = 0;
    pool_.free_blocks(freed.data(), (int32_t)freed.size(), &bad);  // held blocks: cannot be rejected
  }

  void free(int64_t req) {
    const auto it = req_to_blocks_.find(req);
    if (it == req_to_blocks_.end()) return;
    std::vector<int32_t> real;
    for (int32_t id : it->second)
      if (id != pool_.null_block()) real.push_back(id);
    req_to_blocks_.erase(it);
    int32_t bad = 0;
    pool_.free_blocks(real.data(), (int32_t)real.size(), &bad);
  }

  int32_t num_used() const { return pool_.num_blocks() - 1 - pool_.num_free(); }

 private:
  int32_t attn_type_;
  int32_t block_size_;
  int32_t window_;
  BlockPool pool_;
  std::unordered_map<int64_t, std::vector<int32_t>> req_to_blocks_;
};

}  // namespace

struct pkv_block_pool {
  BlockPool pool;
  explicit pkv_block_pool(int32_t n) : pool(n) {}
};

struct pkv_kv_manager {
  int32_t block_size;
  int32_t max_model_len;
  std::vector<std::unique_ptr<TypeManager>> managers;
};

extern "C" {

pkv_status pkv_pool_create(int32_t num_blocks, pkv_block_pool** out) {
  return guarded([&]() -> pkv_status {
    if (!out) return fail(PKV_ERR_INVALID_ARG, "NULL output pointer");
    *out = nullptr;
    if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "a pool needs at least the null block (num_blocks %d)", num_blocks);
    *out = new (std::nothrow) pkv_block_pool(num_blocks);
    if (!*out) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
    return ok();
  });
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

pkv_status pkv_pool_num_free(const pkv_block_pool* pool, int32_t* count) {
  return guarded([&]() -> pkv_status {
    if (!pool || !count) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    *count = pool->pool.num_free();
    return ok();
  });
}

pkv_status pkv_pool_get_new_blocks(pkv_block_pool* pool, int32_t n, int32_t* ids) {
  return guarded([&]() -> pkv_status {
    if (!pool || (n > 0 && !ids)) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (!pool->pool.get_new_blocks(n, ids))
      return fail(PKV_ERR_INVALID_ARG, "%d blocks asked, %d free", n, pool->pool.num_free());
    return ok();
  });
}

pkv_status pkv_pool_free_blocks(pkv_block_pool* pool, const int32_t* ids, int32_t n) {
  return guarded([&]() -> pkv_status {
    if (!pool || n < 0 || (n > 0 && !ids)) return fail(PKV_ERR_INVALID_ARG, "bad argument");
    int32_t bad = 0;
    if (!pool->pool.free_blocks(ids, n, &bad))
      return fail(PKV_ERR_INVALID_ARG, "block %d cannot be freed (out of range, the null block, or already free)", bad);
    return ok();
  });
}

pkv_status pkv_kvm_create(const pkv_attn_group* groups, int32_t num_groups, int32_t block_size,
                          int32_t max_model_len, pkv_kv_manager** out) {
  return guarded([&]() -> pkv_status {
    if (!out) return fail(PKV_ERR_INVALID_ARG, "NULL output pointer");
    *out = nullptr;
    if (!groups || num_groups < 1) return fail(PKV_ERR_INVALID_ARG, "at least one attention group is needed");
    if (block_size < 1 || max_model_len < 1)
      return fail(PKV_ERR_INVALID_ARG, "block_size %d and max_model_len %d must be > 0", block_size, max_model_len);
    for (int32_t g = 0; g < num_groups; ++g) {
      const pkv_attn_group& s = groups[g];
      if (s.attn_type != PKV_ATTN_FULL && s.attn_type != PKV_ATTN_SLIDING)
        return fail(PKV_ERR_INVALID_ARG, "group %d: unknown attention type %d", g, s.attn_type);
      if (s.num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "group %d: num_blocks %d < 1", g, s.num_blocks);
      if (s.attn_type == PKV_ATTN_SLIDING && s.sliding_window < 1)
        return fail(PKV_ERR_INVALID_ARG, "group %d: sliding window %d < 1", g, s.sliding_window);
    }
    auto m = std::unique_ptr<pkv_kv_manager>(new (std::nothrow) pkv_kv_manager());
    if (!m) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
    m->block_size = block_size;
    m->max_model_len = max_model_len;
    for (int32_t g = 0; g < num_groups; ++g)
      m->managers.push_back(std::make_unique<TypeManager>(
          groups[g].attn_type, groups[g].num_blocks, block_size,
          groups[g].attn_type == PKV_ATTN_SLIDING ? groups[g].sliding_window : 0));
    *out = m.release();
    return ok();
  });
}

void pkv_kvm_destroy(pkv_kv_manager* m) { delete m; }

pkv_status pkv_kvm_allocate_slots(pkv_kv_manager* m, int64_t request_id, int32_t computed_tokens,
                                  int32_t num_new_tokens, int32_t lookahead_tokens, int32_t* allocated) {
  return guarded([&]() -> pkv_status {
    if (!m || !allocated) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    *allocated = 0;
    if (computed_tokens < 0 || num_new_tokens < 0 || lookahead_tokens < 0)
      return fail(PKV_ERR_INVALID_ARG, "token counts must be >= 0");
    const int64_t cap = m->max_model_len;
    const int64_t computed = computed_tokens < cap ? computed_tokens : cap;
    const int64_t want = (int64_t)computed_tokens + num_new_tokens + lookahead_tokens;
    const int64_t need = want < cap ? want : cap;
    // Phase 1: converge every group's state, then check it can grow.
    for (auto& t : m->managers) {
      t->remove_skipped_blocks(request_id, computed);
      if (t->blocks_to_allocate(request_id, need, computed) > t->pool().num_free()) return ok();
    }
    // Phase 2: every group has room.
    for (auto& t : m->managers) t->allocate_new_blocks(request_id, need, computed);
    *allocated = 1;
    return ok();
  });
}

pkv_status pkv_kvm_free(pkv_kv_manager* m, int64_t request_id) {
  return guarded([&]() -> pkv_status {
    if (!m) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    for (auto& t : m->managers) t->free(request_id);
    return ok();
  });
}

pkv_status pkv_kvm_get_block_ids(const pkv_kv_manager* m, int64_t request_id, int32_t group, int32_t* ids,
                                 int32_t capacity, int32_t* count) {
  return guarded([&]() -> pkv_status {
    if (!m || !count) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (group < 0 || group >= (int32_t)m->managers.size()) return fail(PKV_ERR_INVALID_ARG, "no group %d", group);
    const std::vector<int32_t>* b = m->managers[group]->blocks_of(request_id);
    *count = b ? (int32_t)b->size() : 0;
    if (ids && b) {
      const int32_t n = *count < capacity ? *count : capacity;
      if (n > 0) std::memcpy(ids, b->data(), sizeof(int32_t) * (size_t)n);
    }
    return ok();
  });
}

pkv_status pkv_kvm_num_free_blocks(const pkv_kv_manager* m, int32_t group, int32_t* count) {
  return guarded([&]() -> pkv_status {
    if (!m || !count) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (group < 0 || group >= (int32_t)m->managers.size()) return fail(PKV_ERR_INVALID_ARG, "no group %d", group);
    *count = m->managers[group]->pool().num_free();
    return ok();
  });
}

pkv_status pkv_kvm_format_usage(const pkv_kv_manager* m, char* buf, size_t capacity) {
  return guarded([&]() -> pkv_status {
    if (!m || !buf) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    std::string s;
    for (size_t g = 0; g < m->managers.size(); ++g) {
      const TypeManager& t = *m->managers[g];
      if (g) s += ",";
      s += t.attn_type() == PKV_ATTN_FULL ? "full:" : "sliding:";
      s += std::to_string(t.num_used()) + "/" + std::to_string(t.pool().num_blocks());
    }
    if (s.size() + 1 > capacity) return fail(PKV_ERR_INVALID_ARG, "usage string needs %zu bytes", s.size() + 1);
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return ok();
  });
}

pkv_status pkv_kvm_prepare_block_table(const pkv_kv_manager* m, int32_t group, const int64_t* request_ids,
                                       int32_t batch, int32_t max_blocks_per_seq, int32_t* table) {
  return guarded([&]() -> pkv_status {
    if (!m || (batch > 0 && (!request_ids || !table))) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
    if (group < 0 || group >= (int32_t)m->managers.size()) return fail(PKV_ERR_INVALID_ARG, "no group %d", group);
    if (batch < 0 || max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "bad table shape");
    const TypeManager& t = *m->managers[group];
    for (int32_t r = 0; r < batch; ++r) {
      const std::vector<int32_t>* b = t.blocks_of(request_ids[r]);
      if (b && (int64_t)b->size() > max_blocks_per_seq)
        return fail(PKV_ERR_INVALID_ARG, "request %lld holds %zu table entries, more than %d",
                    (long long)request_ids[r], b->size(), max_blocks_per_seq);
    }
    for (int32_t r = 0; r < batch; ++r) {
      const std::vector<int32_t>* b = t.blocks_of(request_ids[r]);
      int32_t* row = table + (int64_t)r * max_blocks_per_seq;
      const int32_t n = b ? (int32_t)b->size() : 0;
      if (n > 0) std::memcpy(row, b->data(), sizeof(int32_t) * (size_t)n);
      for (int32_t i = n; i < max_blocks_per_seq; ++i) row[i] = t.pool().null_block();
    }
    return ok();
  });
}

pkv_status pkv_block_num_fixed(int32_t max_concurrency, int32_t sliding_window, int32_t next_n, int32_t block_size,
                               int64_t* num_blocks) {
  return guarded([&]() -> pkv_status {
    if (!num_blocks || max_concurrency < 0 || sliding_window < 1 || next_n < 0 || block_size < 1)
      return fail(PKV_ERR_INVALID_ARG, "bad sizing argument");
    *num_blocks = (int64_t)max_concurrency * (ceil_div((int64_t)sliding_window + 2 * (int64_t)next_n, block_size) + 1) + 1;
    return ok();
  });
}

pkv_status pkv_block_num_full(int32_t max_len, int32_t max_concurrency, int32_t block_size, int64_t* num_blocks) {
  return guarded([&]() -> pkv_status {
    if (!num_blocks || max_len < 0 || max_concurrency < 0 || block_size < 1)
      return fail(PKV_ERR_INVALID_ARG, "bad sizing argument");
    *num_blocks = ceil_div(max_len, block_size) * max_concurrency + 1;
    return ok();
  });
}

pkv_status pkv_block_num_budget(int64_t budget_bytes, int64_t fixed_bytes, int64_t per_token_bytes, int32_t block_size,
                                int64_t* num_blocks) {
  return guarded([&]() -> pkv_status {
    if (!num_blocks || per_token_bytes < 1 || block_size < 1 || budget_bytes < 0 || fixed_bytes < 0)
      return fail(PKV_ERR_INVALID_ARG, "bad sizing argument");
    const int64_t left = budget_bytes > fixed_bytes ? budget_bytes - fixed_bytes : 0;
    *num_blocks = left / per_token_bytes / block_size + 1;
    return ok();
  });
}

}  // extern "C"
