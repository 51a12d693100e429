// Host build of the decode's unit grid (unit_of, unit_pages and
// merged_partitions from pa_device.hpp), for a CPU test of its indexing.
// stdin: num_seqs num_kv_heads group num_partitions grid_partitions
//        pages_per_partition max_pages_per_seq use_first, then num_seqs
//        context lengths, then (use_first) num_seqs first partitions.
// stdout: one line per grid index:
//   "skip u" or "unit u seq kvh part has_tokens lo hi merged_partitions".
#include <cstdio>
#include <vector>

#include "pa_device.hpp"

int main() {
  int B, Hkv, G, NP, GP, PP, MP, use_first;
  if (std::scanf("%d %d %d %d %d %d %d %d", &B, &Hkv, &G, &NP, &GP, &PP, &MP, &use_first) != 8)
    return 2;
  std::vector<int32_t> lens(B), first(B, 0);
  for (int b = 0; b < B; ++b)
    if (std::scanf("%d", &lens[b]) != 1) return 2;
  if (use_first)
    for (int b = 0; b < B; ++b)
      if (std::scanf("%d", &first[b]) != 1) return 2;
  pa::DecodeParams p{};
  p.context_lens = lens.data();
  p.first_partition = use_first ? first.data() : nullptr;
  p.num_seqs = B;
  p.num_kv_heads = Hkv;
  p.group = G;
  p.num_q_heads = Hkv * G;
  p.num_partitions = NP;
  p.grid_partitions = GP;
  p.pages_per_partition = PP;
  p.max_pages_per_seq = MP;
  p.num_units = B * Hkv * GP;
  for (int u = 0; u < p.num_units; ++u) {
    int seq, kvh, part, lo = 0, hi = 0;
    if (!pa::unit_of(p, u, seq, kvh, part)) {
      std::printf("skip %d\n", u);
      continue;
    }
    const bool has = pa::unit_pages(p, seq, part, lens[seq], lo, hi);
    std::printf("unit %d %d %d %d %d %d %d %d\n", u, seq, kvh, part, int(has), lo, hi,
                pa::merged_partitions(p, lens[seq]));
  }
  return 0;
}
