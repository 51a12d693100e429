// Host-side owner of the KV page pool (see include/pa_pager.h for the
// policy and the contract).  Plain C++17; no GPU calls.
#include "pa_pager.h"

#include <algorithm>
#include <array>
#include <cstring>
#include <deque>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

namespace {

constexpr int kMaxPageSize = 64;

// One step of the splitmix64 generator's output function (Steele, Lea and
// Flood, "Fast splittable pseudorandom number generators", 2014; constants
// as published with Vigna's splitmix64): add the golden-ratio increment,
// then the variant-13 finalizer.
uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int page_size) {
  uint64_t h = mix(parent ^ 0x5A17C0DEu);
  for (int i = 0; i < page_size; ++i) h = mix(h ^ uint64_t(uint32_t(tokens[i])));
  return h;
}

struct Page {
  int32_t ref = 0;
  bool registered = false;  // in the hash table (this page is the entry)
  uint64_t hash = 0, parent = 0;
  std::array<int32_t, kMaxPageSize> tokens{};
  int64_t released_at = 0;  // LRU key while cached
};

struct Sequence {
  std::vector<int32_t> pages;
  int64_t len = 0;
  uint64_t full_hash = 0;                       // chained hash through the last full page
  std::array<int32_t, kMaxPageSize> tail{};     // tokens of the partial last page
};

struct Event {
  int32_t kind;
  int64_t page;
  uint64_t hash;
};

}  // namespace

struct pa_pager {
  int64_t num_pages;
  int page_size;
  int max_pages;
  std::vector<Page> pages;
  std::set<int32_t> empty;                   // free, nothing registered: lowest id first
  std::map<int64_t, int32_t> cached;         // free, registered: release tick -> page (LRU)
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Sequence> seqs;
  std::deque<Event> events;
  int64_t tick = 0;
  int64_t hits = 0, evictions = 0, cows = 0;

  // A page for new content, or -1 when every page is in use.
  int32_t allocate() {
    int32_t p;
    if (!empty.empty()) {
      p = *empty.begin();
      empty.erase(empty.begin());
    } else if (!cached.empty()) {
      p = cached.begin()->second;
      cached.erase(cached.begin());
      Page& pg = pages[p];
      by_hash.erase(pg.hash);
      pg.registered = false;
      events.push_back({PA_PAGER_EVENT_REMOVED, p, pg.hash});
      ++evictions;
    } else {
      return -1;
    }
    pages[p].ref = 1;
    return p;
  }

  void take(int32_t p) {  // one more holder of a registered page
    Page& pg = pages[p];
    if (pg.ref == 0) cached.erase(pg.released_at);
    ++pg.ref;
  }

  void release(int32_t p) {
    Page& pg = pages[p];
    if (--pg.ref > 0) return;
    if (pg.registered) {
      pg.released_at = ++tick;
      cached.emplace(pg.released_at, p);
    } else {
      empty.insert(p);
    }
  }

  // Register page p (now full, held by the caller) under hash h unless the
  // hash is already taken.
  void register_full(int32_t p, uint64_t h, uint64_t parent, const int32_t* tokens) {
    if (by_hash.count(h)) return;
    Page& pg = pages[p];
    pg.registered = true;
    pg.hash = h;
    pg.parent = parent;
    std::copy(tokens, tokens + page_size, pg.tokens.begin());
    by_hash.emplace(h, p);
    events.push_back({PA_PAGER_EVENT_STORED, p, h});
  }

  // The registered page for (parent, tokens), or -1.
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* tokens) const {
    auto it = by_hash.find(h);
    if (it == by_hash.end()) return -1;
    const Page& pg = pages[it->second];
    if (pg.parent != parent || !std::equal(tokens, tokens + page_size, pg.tokens.begin()))
      return -1;
    return it->second;
  }
};

namespace {
// Length of the common prefix of a[0..n) and b[0..n): whole 16-id blocks
// by memcmp (vectorised), then the first differing block id by id.
int common_prefix(const int32_t* a, const int32_t* b, int n) {
  constexpr int kBlock = 16;
  int l = 0;
  while (l + kBlock <= n && std::memcmp(a + l, b + l, kBlock * sizeof(int32_t)) == 0) l += kBlock;
  while (l < n && a[l] == b[l]) ++l;
  return l;
}
}  // namespace

extern "C" {

pa_pager* pa_pager_create(int64_t num_pages, int page_size, int max_pages_per_seq) {
  if (num_pages <= 0 || num_pages > INT32_MAX || page_size <= 0 || page_size > kMaxPageSize ||
      max_pages_per_seq <= 0)
    return nullptr;
  pa_pager* p = new (std::nothrow) pa_pager();
  if (!p) return nullptr;
  p->num_pages = num_pages;
  p->page_size = page_size;
  p->max_pages = max_pages_per_seq;
  p->pages.resize(size_t(num_pages));
  for (int64_t i = 0; i < num_pages; ++i) p->empty.insert(int32_t(i));
  return p;
}

void pa_pager_destroy(pa_pager* pager) { delete pager; }

int pa_pager_add_sequence(pa_pager* pg, int64_t seq_id, const int32_t* tokens, int64_t n,
                          int64_t* slot_mapping, int64_t* num_cached) {
  if (!pg || n < 0 || !num_cached || (n > 0 && (!tokens || !slot_mapping)))
    return PA_PAGER_INVALID_ARGUMENT;
  if (pg->seqs.count(seq_id)) return PA_PAGER_SEQUENCE_EXISTS;
  const int P = pg->page_size;
  const int64_t npages = (n + P - 1) / P;
  if (npages > pg->max_pages) return PA_PAGER_SEQUENCE_FULL;

  // The longest registered prefix of full pages, found without changing
  // anything, so that a pool too small for the rest fails cleanly.
  std::vector<int32_t> reuse;
  uint64_t h = 0;
  for (int64_t k = 0; k < n / P; ++k) {
    const uint64_t hk = chain_hash(h, tokens + k * P, P);
    const int32_t p = pg->lookup(hk, h, tokens + k * P);
    if (p < 0) break;
    reuse.push_back(p);
    h = hk;
  }
  const int64_t reused = int64_t(reuse.size());
  int64_t reuse_cached = 0;  // reused pages that are free now (leaving the evictable set)
  for (int32_t p : reuse) reuse_cached += pg->pages[size_t(p)].ref == 0 ? 1 : 0;
  const int64_t available = int64_t(pg->empty.size() + pg->cached.size()) - reuse_cached;
  if (npages - reused > available) return PA_PAGER_OUT_OF_PAGES;

  Sequence s;
  for (int32_t p : reuse) {
    pg->take(p);
    s.pages.push_back(p);
  }
  for (int64_t k = reused; k < npages; ++k) s.pages.push_back(pg->allocate());  // cannot fail
  for (int64_t k = reused; k < n / P; ++k) {
    const uint64_t hk = chain_hash(h, tokens + k * P, P);
    pg->register_full(s.pages[size_t(k)], hk, h, tokens + k * P);
    h = hk;
  }
  s.full_hash = h;
  s.len = n;
  for (int64_t t = (n / P) * P; t < n; ++t) s.tail[size_t(t % P)] = tokens[t];
  for (int64_t t = 0; t < n; ++t) slot_mapping[t] = int64_t(s.pages[size_t(t / P)]) * P + t % P;
  *num_cached = reused * P;
  pg->hits += reused * P;
  pg->seqs.emplace(seq_id, std::move(s));
  return PA_PAGER_OK;
}

int pa_pager_append(pa_pager* pg, int64_t seq_id, int32_t token, int64_t* slot,
                    int64_t* copy_src, int64_t* copy_dst) {
  if (!pg || !slot || !copy_src || !copy_dst) return PA_PAGER_INVALID_ARGUMENT;
  auto it = pg->seqs.find(seq_id);
  if (it == pg->seqs.end()) return PA_PAGER_UNKNOWN_SEQUENCE;
  Sequence& s = it->second;
  const int P = pg->page_size;
  const int off = int(s.len % P);
  *copy_src = *copy_dst = -1;
  if (off == 0) {  // the token opens a new page
    if (int64_t(s.pages.size()) >= pg->max_pages) return PA_PAGER_SEQUENCE_FULL;
    const int32_t p = pg->allocate();
    if (p < 0) return PA_PAGER_OUT_OF_PAGES;
    s.pages.push_back(p);
  } else {
    const int32_t tail = s.pages.back();
    if (pg->pages[size_t(tail)].ref > 1) {  // shared by a fork: move to a private copy
      const int32_t p = pg->allocate();
      if (p < 0) return PA_PAGER_OUT_OF_PAGES;
      pg->release(tail);
      s.pages.back() = p;
      *copy_src = tail;
      *copy_dst = p;
      ++pg->cows;
    }
  }
  const int32_t page = s.pages.back();
  *slot = int64_t(page) * P + off;
  s.tail[size_t(off)] = token;
  ++s.len;
  if (s.len % P == 0) {  // the page is full: register it
    const uint64_t h = chain_hash(s.full_hash, s.tail.data(), P);
    pg->register_full(page, h, s.full_hash, s.tail.data());
    s.full_hash = h;
  }
  return PA_PAGER_OK;
}

int pa_pager_append_batch(pa_pager* pg, const int64_t* seq_ids, const int32_t* tokens,
                          int64_t n, int64_t* slots, int64_t* copy_src, int64_t* copy_dst,
                          int64_t* num_done) {
  if (!pg || n < 0 || !num_done ||
      (n > 0 && (!seq_ids || !tokens || !slots || !copy_src || !copy_dst)))
    return PA_PAGER_INVALID_ARGUMENT;
  *num_done = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int st = pa_pager_append(pg, seq_ids[i], tokens[i], slots + i, copy_src + i, copy_dst + i);
    if (st != PA_PAGER_OK) return st;
    *num_done = i + 1;
  }
  return PA_PAGER_OK;
}

int pa_pager_fork(pa_pager* pg, int64_t parent, int64_t child) {
  if (!pg) return PA_PAGER_INVALID_ARGUMENT;
  auto it = pg->seqs.find(parent);
  if (it == pg->seqs.end()) return PA_PAGER_UNKNOWN_SEQUENCE;
  if (pg->seqs.count(child)) return PA_PAGER_SEQUENCE_EXISTS;
  Sequence c = it->second;
  for (int32_t p : c.pages) ++pg->pages[size_t(p)].ref;
  pg->seqs.emplace(child, std::move(c));
  return PA_PAGER_OK;
}

int pa_pager_free_sequence(pa_pager* pg, int64_t seq_id) {
  if (!pg) return PA_PAGER_INVALID_ARGUMENT;
  auto it = pg->seqs.find(seq_id);
  if (it == pg->seqs.end()) return PA_PAGER_UNKNOWN_SEQUENCE;
  const std::vector<int32_t>& ps = it->second.pages;
  for (auto p = ps.rbegin(); p != ps.rend(); ++p) pg->release(*p);
  pg->seqs.erase(it);
  return PA_PAGER_OK;
}

int pa_pager_block_tables(const pa_pager* pg, const int64_t* seq_ids, int64_t n, int32_t* tables,
                          int32_t* context_lens) {
  if (!pg || n < 0 || (n > 0 && (!seq_ids || !tables || !context_lens)))
    return PA_PAGER_INVALID_ARGUMENT;
  std::vector<const Sequence*> found(size_t(n), nullptr);
  for (int64_t i = 0; i < n; ++i) {
    auto it = pg->seqs.find(seq_ids[i]);
    if (it == pg->seqs.end()) return PA_PAGER_UNKNOWN_SEQUENCE;  // nothing written
    found[size_t(i)] = &it->second;
  }
  for (int64_t i = 0; i < n; ++i) {
    const Sequence& s = *found[size_t(i)];
    int32_t* row = tables + i * pg->max_pages;
    std::copy(s.pages.begin(), s.pages.end(), row);
    std::fill(row + s.pages.size(), row + pg->max_pages, -1);
    context_lens[i] = int32_t(s.len);
  }
  return PA_PAGER_OK;
}

int pa_pager_get_stats(const pa_pager* pg, pa_pager_stats* out) {
  if (!pg || !out) return PA_PAGER_INVALID_ARGUMENT;
  std::memset(out, 0, sizeof(*out));
  out->num_pages = pg->num_pages;
  out->cached_free = int64_t(pg->cached.size());
  out->empty_free = int64_t(pg->empty.size());
  out->in_use = pg->num_pages - out->cached_free - out->empty_free;
  out->registered = int64_t(pg->by_hash.size());
  out->live_sequences = int64_t(pg->seqs.size());
  out->prefix_hit_tokens = pg->hits;
  out->evictions = pg->evictions;
  out->cow_copies = pg->cows;
  return PA_PAGER_OK;
}

int pa_pager_drain_events(pa_pager* pg, int32_t* kinds, int64_t* pages, uint64_t* hashes,
                          int64_t capacity, int64_t* count) {
  if (!pg || !count || capacity < 0 || (capacity > 0 && (!kinds || !pages || !hashes)))
    return PA_PAGER_INVALID_ARGUMENT;
  int64_t k = 0;
  while (k < capacity && !pg->events.empty()) {
    const Event& e = pg->events.front();
    kinds[k] = e.kind;
    pages[k] = e.page;
    hashes[k] = e.hash;
    pg->events.pop_front();
    ++k;
  }
  *count = k;
  return PA_PAGER_OK;
}

int pa_pager_prefix_groups(const int32_t* block_tables, const int32_t* context_lens,
                           int64_t num_seqs, int max_pages_per_seq, int pages_per_partition,
                           int32_t* group_start, int32_t* group_seqs, int32_t* group_partitions,
                           int32_t* seq_first_partition, int64_t* num_groups,
                           int64_t* max_group_size, int64_t* max_group_partitions,
                           int64_t* max_suffix_partitions) {
  if (num_seqs < 0 || max_pages_per_seq <= 0 || pages_per_partition <= 0 || !num_groups ||
      !max_group_size || !max_group_partitions || !max_suffix_partitions || !group_start)
    return PA_PAGER_INVALID_ARGUMENT;
  if (num_seqs > 0 && (!block_tables || !context_lens || !group_seqs || !group_partitions ||
                       !seq_first_partition))
    return PA_PAGER_INVALID_ARGUMENT;
  const int P = 16;
  auto row = [&](int64_t b) { return block_tables + b * max_pages_per_seq; };
  auto whole = [&](int64_t b) {  // pages wholly before the last token
    const int L = context_lens[b];
    return std::min(L > 0 ? (L - 1) / P : 0, max_pages_per_seq);
  };
  // Eligible sequences keyed by the page in column 0.  Sorting the (page,
  // sequence) pairs makes every bucket a run whose members are in batch
  // order; the runs are then taken in order of their first member.
  std::vector<std::pair<int32_t, int32_t>> keyed;
  keyed.reserve(size_t(num_seqs));
  for (int64_t b = 0; b < num_seqs; ++b) {
    seq_first_partition[b] = 0;
    if (whole(b) >= pages_per_partition) keyed.emplace_back(row(b)[0], int32_t(b));
  }
  std::sort(keyed.begin(), keyed.end());
  struct Run {
    int32_t first_member, begin, end;
  };
  std::vector<Run> runs;
  for (size_t i = 0; i < keyed.size();) {
    size_t k = i + 1;
    while (k < keyed.size() && keyed[k].first == keyed[i].first) ++k;
    if (k - i >= 2) runs.push_back({keyed[i].second, int32_t(i), int32_t(k)});
    i = k;
  }
  std::sort(runs.begin(), runs.end(),
            [](const Run& a, const Run& b) { return a.first_member < b.first_member; });
  int64_t g = 0, at = 0, max_size = 0, max_parts = 0;
  group_start[0] = 0;
  for (const Run& run : runs) {
    const int32_t* first = row(run.first_member);
    int lcp = whole(run.first_member);
    for (int32_t i = run.begin + 1; i < run.end && lcp > 0; ++i) {
      const int32_t* r = row(keyed[size_t(i)].second);
      lcp = common_prefix(r, first, std::min(lcp, whole(keyed[size_t(i)].second)));
    }
    const int parts = lcp / pages_per_partition;
    if (parts < 1) continue;
    for (int32_t i = run.begin; i < run.end; ++i) {
      const int32_t b = keyed[size_t(i)].second;
      group_seqs[at++] = b;
      seq_first_partition[b] = parts;
    }
    group_partitions[g] = parts;
    group_start[++g] = int32_t(at);
    max_size = std::max<int64_t>(max_size, run.end - run.begin);
    max_parts = std::max<int64_t>(max_parts, parts);
  }
  int64_t max_suffix = 0;
  for (int64_t b = 0; b < num_seqs; ++b) {
    const int64_t L = std::max(context_lens[b], 0);
    const int64_t pages = std::min<int64_t>((L + P - 1) / P, max_pages_per_seq);
    const int64_t parts = (pages + pages_per_partition - 1) / pages_per_partition;
    max_suffix = std::max(max_suffix, parts - seq_first_partition[b]);
  }
  *num_groups = g;
  *max_group_size = max_size;
  *max_group_partitions = max_parts;
  *max_suffix_partitions = max_suffix;
  return PA_PAGER_OK;
}

uint64_t pa_pager_page_hash(uint64_t parent, const int32_t* tokens, int page_size) {
  if (!tokens || page_size <= 0) return 0;
  return chain_hash(parent, tokens, page_size);
}

}  // extern "C"
