// Host wave planner of libpe: the multi-wave step of one layer.
//
// SGLang "Paged Experts" docs page, "A step: waves, page-in, merge", steps 1-2,
// and "Captured decode" (which steps the host plans, and that it shares the
// layer's LRU state with the device planner).  For one step of one layer: the
// routed experts are grouped into waves of at most K, those holding a slot
// first; per wave, each expert without a slot takes the slot of an expert the
// wave does not use, least recently used first, and only those are copied in.
//
// Readings where the page is silent (the device planner makes the same ones):
// resident-first order with ascending ids inside each part; waves are
// consecutive chunks of K; a wave is one use (all its experts get the current
// tick, then the tick advances); victims are slots whose expert is outside the
// wave, by ascending (last_use, slot); the i-th missing expert (ascending id)
// takes the i-th victim; ids outside [0, E) are ignored.
#include <algorithm>
#include <cstring>
#include <vector>

#include "pe_layout.h"

namespace pe {

int host_plan_step(const Dims& d, const LayerLayout& ll, const WorkLayout& wl,
                   const int32_t* ids, int n_entries, int32_t* blk, int32_t* work,
                   HostPlanSummary* sum) {
  const int E = d.E, K = d.K, MW = d.max_waves;
  int32_t* st = blk + ll.state(blk[ll.cur] & 1);
  uint32_t tick = (uint32_t)st[ll.tick];
  int32_t* slot_expert = st + ll.slot_expert;
  int32_t* expert_slot = st + ll.expert_slot;
  uint32_t* last_use = reinterpret_cast<uint32_t*>(st + ll.last_use);
  int32_t* slot_of = blk + ll.slot_of;

  // scratch kept per thread (a host-planned step runs on the caller's thread),
  // reached once through references: the per-entry loops then touch plain arrays
  struct Scratch {
    std::vector<int> cnt, order, u_of, in_wave, seen, wave;
    std::vector<std::pair<uint32_t, int>> cand;
    std::vector<char> hit, was_hit;
  };
  thread_local Scratch tls;
  Scratch& sc = tls;
  std::vector<int>&cnt = sc.cnt, &order = sc.order, &u_of = sc.u_of, &in_wave = sc.in_wave, &seen = sc.seen,
  &wave = sc.wave;
  std::vector<std::pair<uint32_t, int>>& cand = sc.cand;
  std::vector<char>&hit = sc.hit, &was_hit = sc.was_hit;
  cnt.assign(E, 0);
  int bad = 0, valid = 0;
  {
    int* c = cnt.data();
    for (int i = 0; i < n_entries; ++i) {
      const int e = ids[i];
      if ((unsigned)e >= (unsigned)E) { ++bad; continue; }
      ++c[e];
    }
    valid = n_entries - bad;
  }
  order.clear();
  for (int e = 0; e < E; ++e) if (cnt[e] && expert_slot[e] >= 0) order.push_back(e);
  for (int e = 0; e < E; ++e) if (cnt[e] && expert_slot[e] < 0) order.push_back(e);
  const int D = (int)order.size();
  const int n_waves = ceil_div(D, K);
  if (n_waves > MW) return -1;

  int32_t* hdr = work + wl.hdr;
  int32_t* used_expert = work + wl.used_expert;
  int32_t* used_slot = work + wl.used_slot;
  int32_t* used_off = work + wl.used_off;
  int32_t* gemv_u = work + wl.gemv_u;
  int32_t* gemv_desc = work + wl.gemv_desc;
  int32_t* tile_desc = work + wl.tile_desc;
  int32_t* entries = work + wl.entries;

  u_of.assign(E, -1);
  in_wave.assign(E, -1);
  int u = 0, off = 0, ng = 0, nt = 0, page_ins = 0, max_gemv = 0;
  hdr[0] = n_waves;
  hdr[hdr_wave_u(MW, 0)] = 0;
  hdr[hdr_gemv(MW, 0)] = 0;
  hdr[hdr_tile(MW, 0)] = 0;
  for (int w = 0; w < n_waves; ++w) {
    const int b = w * K, n = std::min(K, D - b);
    for (int i = 0; i < n; ++i) in_wave[order[b + i]] = w;
    // victims: slots whose occupant is outside this wave, by (last_use, slot)
    cand.clear();
    for (int j = 0; j < K; ++j) {
      int occ = slot_expert[j];
      if (occ < 0 || in_wave[occ] != w) cand.push_back({last_use[j], j});
    }
    std::sort(cand.begin(), cand.end());
    int r = 0;
    int32_t* pe_ = blk + ll.plan_expert + (size_t)w * K;
    int32_t* ps_ = blk + ll.plan_slot + (size_t)w * K;
    int32_t* pv_ = blk + ll.plan_evicted + (size_t)w * K;
    hit.assign(n, 0);
    for (int i = 0; i < n; ++i) hit[i] = expert_slot[order[b + i]] >= 0;
    for (int i = 0; i < n; ++i) {
      int e = order[b + i];
      if (hit[i]) continue;
      int j = cand[r].second;
      int old = slot_expert[j];
      if (old >= 0) expert_slot[old] = -1;
      slot_expert[j] = e;
      expert_slot[e] = j;
      pe_[r] = e; ps_[r] = j; pv_[r] = old;
      ++r;
    }
    blk[ll.plan_count + w] = r;
    page_ins += r;
    for (int i = 0; i < n; ++i) last_use[expert_slot[order[b + i]]] = tick;
    ++tick;
    // used experts of this wave, ascending id; GEMV items and MFMA tiles list the
    // experts resident before the wave first, then the ones paged in
    wave.assign(order.begin() + b, order.begin() + b + n);
    was_hit.assign(E, 0);
    for (int i = 0; i < n; ++i) was_hit[order[b + i]] = hit[i];
    std::sort(wave.begin(), wave.end());
    int g0 = ng, t0 = nt;
    const int u0 = u;
    for (int e : wave) {
      u_of[e] = u;
      used_expert[u] = e;
      used_slot[u] = expert_slot[e];
      used_off[u] = off;
      off += cnt[e];
      ++u;
    }
    for (int pass = 0; pass < 2; ++pass) {          // 0: hits, 1: paged in
      for (int uu = u0; uu < u; ++uu) {
        const int e = used_expert[uu];
        if (was_hit[e] != (pass == 0)) continue;
        if (cnt[e] < d.mfma_min) {
          int32_t* dsc = gemv_desc + 4 * (size_t)ng;
          dsc[0] = used_slot[uu]; dsc[1] = used_off[uu]; dsc[2] = cnt[e]; dsc[3] = e;
          gemv_u[ng++] = uu;
          max_gemv = std::max(max_gemv, cnt[e]);
        } else {
          for (int q = 0; q < cnt[e]; q += kTileM) {
            int32_t* td = tile_desc + 4 * (size_t)nt++;
            td[0] = used_slot[uu]; td[1] = used_off[uu] + q; td[2] = std::min(kTileM, cnt[e] - q); td[3] = e;
          }
        }
      }
      if (pass == 0) {
        hdr[hdr_gemv_split(MW, w)] = ng;
        hdr[hdr_tile_split(MW, w)] = nt;
        sum->gemv_hits[w] = ng - g0;
        sum->tile_hits[w] = nt - t0;
      }
    }
    hdr[hdr_wave_u(MW, w + 1)] = u;
    hdr[hdr_gemv(MW, w + 1)] = ng;
    hdr[hdr_tile(MW, w + 1)] = nt;
    sum->gemv_items[w] = ng - g0;
    sum->tiles[w] = nt - t0;
  }
  used_off[u] = off;
  // entries in ascending index at their expert's positions; slot map at wave
  // time (per expert: its next free position and its slot, looked up once)
  seen.assign(2 * (size_t)E, 0);
  {
    int* next = seen.data();          // [E] next sorted position of expert e
    int* slot = seen.data() + E;      // [E] its slot
    for (int e = 0; e < E; ++e) {
      if (cnt[e] == 0) continue;
      next[e] = used_off[u_of[e]];
      slot[e] = used_slot[u_of[e]];
    }
    for (int i = 0; i < n_entries; ++i) {
      const int e = ids[i];
      if ((unsigned)e >= (unsigned)E) { slot_of[i] = -1; continue; }
      entries[next[e]++] = i;
      slot_of[i] = slot[e];
    }
  }
  st[ll.tick] = (int32_t)tick;
  blk[ll.n_waves] = n_waves;

  sum->n_waves = n_waves;
  sum->distinct = D;
  sum->page_ins = page_ins;
  sum->valid_entries = valid;
  sum->bad_ids = bad;
  sum->max_gemv_tokens = max_gemv;
  return 0;
}

}  // namespace pe
