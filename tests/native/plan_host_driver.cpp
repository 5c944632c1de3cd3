// Runs the library's host wave planner (pe::host_plan_step) over a trace read
// from stdin, for a build under AddressSanitizer and UndefinedBehaviorSanitizer.
// The block and work arrays are sized exactly as the library sizes them, so any
// access past them is reported.
//
// stdin:  E K k max_tokens steps, then per step: T, then T*k ids
// stdout: per step one line "rc n_waves | count experts.. slots.. evicted.. |
//         ... | slot_of.. | slot_expert.. | last_use.. | tick | entries..
//         | used_off.."
#include <cstdio>
#include <vector>

#include "../../host_paged_expert_amd/csrc/pe_layout.h"

int main() {
  int E, K, k, max_tokens, steps;
  if (std::scanf("%d %d %d %d %d", &E, &K, &k, &max_tokens, &steps) != 5) return 2;
  pe::Dims d = pe::make_dims(1, E, K, k, 8, 8, max_tokens);
  const pe::LayerLayout ll = pe::make_layer_layout(d);
  const pe::WorkLayout wl = pe::make_work_layout(d);
  std::vector<int32_t> blk(ll.total, 0), work(wl.total, 0);
  int32_t* st = blk.data() + ll.state(0);
  st[ll.tick] = 1;
  for (int e = 0; e < E; ++e) st[ll.expert_slot + e] = -1;
  for (int j = 0; j < K; ++j) { st[ll.slot_expert + j] = -1; st[ll.last_use + j] = 0; }
  pe::HostPlanSummary* sum = new pe::HostPlanSummary;
  for (int s = 0; s < steps; ++s) {
    int T;
    if (std::scanf("%d", &T) != 1 || T < 1 || T > max_tokens) return 3;
    std::vector<int32_t> ids((size_t)T * k);
    for (auto& v : ids)
      if (std::scanf("%d", &v) != 1) return 4;
    const int rc = pe::host_plan_step(d, ll, wl, ids.data(), (int)ids.size(), blk.data(), work.data(), sum);
    const int nw = rc == 0 ? blk[ll.n_waves] : 0;
    std::printf("%d %d |", rc, nw);
    for (int w = 0; w < nw; ++w) {
      const int c = blk[ll.plan_count + w];
      std::printf(" %d", c);
      for (const size_t base : {ll.plan_expert, ll.plan_slot, ll.plan_evicted})
        for (int r = 0; r < c; ++r) std::printf(" %d", blk[base + (size_t)w * K + r]);
      std::printf(" |");
    }
    for (int i = 0; i < T * k; ++i) std::printf(" %d", blk[ll.slot_of + i]);
    std::printf(" |");
    for (int j = 0; j < K; ++j) std::printf(" %d", st[ll.slot_expert + j]);
    std::printf(" |");
    for (int j = 0; j < K; ++j) std::printf(" %u", (unsigned)st[ll.last_use + j]);
    std::printf(" | %u |", (unsigned)st[ll.tick]);
    const int n_used = rc == 0 ? work[wl.hdr + pe::hdr_wave_u(d.max_waves, nw)] : 0;
    const int n_valid = rc == 0 ? work[wl.used_off + n_used] : 0;
    for (int i = 0; i < n_valid; ++i) std::printf(" %d", work[wl.entries + i]);
    std::printf(" |");
    for (int u = 0; u <= n_used; ++u) std::printf(" %d", work[wl.used_off + u]);
    std::printf("\n");
  }
  delete sum;
  return 0;
}
