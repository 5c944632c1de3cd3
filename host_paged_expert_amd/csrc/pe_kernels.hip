// HIP kernels of libpe for gfx950 (CDNA4, 64-wide wavefronts).
//
// Steps of one MoE-layer forward with paged experts (SGLang "Paged Experts"
// docs page, "A step: waves, page-in, merge" and "Captured decode"):
//   plan_single_wave  the LRU decision made on the device, writing the page-in
//                     plan (experts, slots, count) to device buffers, plus the
//                     slot remap and per-slot entry lists;
//   page_in           copies the planned expert blobs from pinned host memory,
//                     read through its mapped address, with the count read on
//                     the device;
//   gemv_gate_up      per used slot: h = silu(W1 x) * (W3 x) (fp32 accumulation,
//                     inline dequantisation), stored as bf16;
//   gemv_down         per used slot: merged[t,j] = w[t,j] * (W2 h) in fp32,
//                     no top-k sum;
//   topk_sum          the fixed-order top-k sum of the merged entries.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "../../include/pe.h"
#include "pe_kernels.h"

namespace pe {

Offsets make_offsets(const LayerLayout& ll, const WorkLayout& wl) {
  Offsets o;
  o.tick = (int)ll.tick; o.slot_expert = (int)ll.slot_expert; o.expert_slot = (int)ll.expert_slot;
  o.last_use = (int)ll.last_use;
  o.cur = (int)ll.cur; o.state0 = (int)ll.state0; o.state_stride = (int)ll.state_stride;
  o.n_waves = (int)ll.n_waves; o.plan_count = (int)ll.plan_count;
  o.plan_expert = (int)ll.plan_expert; o.plan_slot = (int)ll.plan_slot;
  o.plan_evicted = (int)ll.plan_evicted; o.slot_of = (int)ll.slot_of;
  o.hdr = (int)wl.hdr; o.used_expert = (int)wl.used_expert; o.used_slot = (int)wl.used_slot;
  o.used_off = (int)wl.used_off; o.gemv_u = (int)wl.gemv_u; o.gemv_desc = (int)wl.gemv_desc;
  o.tile_desc = (int)wl.tile_desc; o.entries = (int)wl.entries;
  return o;
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// out[t] = bf16(((m0 + m1) + ...) + m_{k-1}) over the valid entries of token t,
// four columns per thread, threads tid, tid + nthreads, ...
__device__ __forceinline__ void topk_sum_rows(const float* __restrict__ merged, const int32_t* __restrict__ ids,
                                              int T, int k, int E, int H, uint16_t* __restrict__ out, size_t tid,
                                              size_t nthreads) {
  const int q4 = H / 4;
  for (size_t i = tid; i < (size_t)T * q4; i += nthreads) {
    const int t = (int)(i / q4), c = (int)(i - (size_t)t * q4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int id = ids[t * k + j];
      if (id < 0 || id >= E) continue;
      const float4 v = reinterpret_cast<const float4*>(merged + ((size_t)t * k + j) * H)[c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    ushort4 o;
    o.x = f32_to_bf16(acc.x); o.y = f32_to_bf16(acc.y); o.z = f32_to_bf16(acc.z); o.w = f32_to_bf16(acc.w);
    reinterpret_cast<ushort4*>(out + (size_t)t * H)[c] = o;
  }
}

// Inclusive scan across the 64 lanes of a wavefront with DPP lane moves (no LDS
// round trips): Kogge-Stone within each row of 16 lanes (row_shr 1, 2, 4, 8; a
// lane with no source adds 0), then row 0's total into row 1 and row 2's into
// row 3 (row_bcast:15), then rows 0-1's total into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// ------------------------------------------------------------------ page-in copy

namespace {
constexpr int kCopyThreads = 256;
}

// Every thread of the grid takes 16-byte chunks gtid, gtid + gstride, ...,
// two loads in flight before the stores (named registers, no private array).
__device__ __forceinline__ void copy_chunks(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                            size_t n16, size_t gtid, size_t gstride) {
  for (size_t i0 = gtid; i0 < n16; i0 += 2 * gstride) {
    const size_t i1 = i0 + gstride;
    const bool two = i1 < n16;
    const uint4 v0 = src[i0];
    uint4 v1 = make_uint4(0, 0, 0, 0);
    if (two) v1 = src[i1];
    dst[i0] = v0;
    if (two) dst[i1] = v1;
  }
}

// ------------------------------------------------------------------ planning + page-in

namespace {
constexpr int kPlanThreads = kCopyThreads;
constexpr int kPlanWaves = kPlanThreads / 64;
// prefix values: missing, present, entries, GEMV hit/miss, MFMA tiles hit/miss
constexpr int kScanVals = 7;
constexpr size_t al16(size_t b) { return (b + 15) / 16 * 16; }
}  // namespace

// LDS of one planning workgroup, sized by E experts, K slots and n entries.
struct PlanLds {
  int *es, *cnt, *se;
  unsigned* lu;
  int *victim, *plan_e, *ids, *wtot, *tot, *bad;
  short* pref;
  unsigned char* cand;
};

constexpr size_t plan_lds_bytes(int E, int K, int n) {
  return 2 * al16(4 * (size_t)E) + 4 * al16(4 * (size_t)K) + al16(4 * (size_t)n) +
         al16(4 * kScanVals * kPlanWaves) + al16(4 * kScanVals) + 16 + al16(2 * kScanVals * (size_t)E) +
         al16((size_t)K);
}

__device__ __forceinline__ PlanLds carve_plan(char* p, int E, int K, int n) {
  PlanLds L;
  L.es = reinterpret_cast<int*>(p); p += al16(4 * (size_t)E);
  L.cnt = reinterpret_cast<int*>(p); p += al16(4 * (size_t)E);
  L.se = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.lu = reinterpret_cast<unsigned*>(p); p += al16(4 * (size_t)K);
  L.victim = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.plan_e = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.ids = reinterpret_cast<int*>(p); p += al16(4 * (size_t)n);
  L.wtot = reinterpret_cast<int*>(p); p += al16(4 * kScanVals * kPlanWaves);
  L.tot = reinterpret_cast<int*>(p); p += al16(4 * kScanVals);
  L.bad = reinterpret_cast<int*>(p); p += 16;
  L.pref = reinterpret_cast<short*>(p); p += al16(2 * kScanVals * (size_t)E);
  L.cand = reinterpret_cast<unsigned char*>(p);
  return L;
}

struct PlanArgs {
  int32_t* blk;
  const int32_t* ids;
  int n, E, K, MW;
  Offsets o;
  int mfma_min;
  int32_t* work;
  unsigned long long* stats;
  const uint8_t* host_rows;
  uint8_t* slots;
  size_t stride, copy_bytes;
  int do_copy;
};

// One device-planned wave (all routed experts of a step with T*k <= K), in LDS.
// Each of the ncopy + 1 planning workgroups computes the same plan from state
// copy `cur`; workgroup `ncopy` publishes it (plan, new state in the other copy,
// slot map, work lists, counters) while workgroups [0, ncopy) go on to copy
// their share of the missing experts.  Returns the number of missing experts;
// the plan stays in LDS (carve_plan): the r-th missing expert plan_e[r] goes to
// slot victim[r].
__device__ int plan_page_in_block(const PlanArgs& p, int block, int ncopy, char* lds) {
  const int E = p.E, K = p.K, n = p.n, MW = p.MW;
  const Offsets& o = p.o;
  int32_t* __restrict__ blk = p.blk;
  int32_t* __restrict__ work = p.work;
  unsigned long long* __restrict__ stats = p.stats;
  const int32_t* __restrict__ ids = p.ids;
  const int mfma_min = p.mfma_min;
  PlanLds L = carve_plan(lds, E, K, n);
  int* s_es = L.es;            // expert -> slot (updated in place)
  int* s_cnt = L.cnt;          // entries per expert
  int* s_se = L.se;            // slot -> expert
  unsigned* s_lu = L.lu;       // slot last use
  unsigned char* s_cand = L.cand;   // slot is evictable in this wave
  int* s_victim = L.victim;    // victims by rank
  int* s_plan_e = L.plan_e;    // r-th missing expert
  int* s_ids = L.ids;          // valid id or -1
  int* s_tot = L.tot;
  int& s_bad = *L.bad;
  auto s_pref = [&](int v, int e) -> short& { return L.pref[v * E + e]; };
  auto s_wtot = [&](int v, int w) -> int& { return L.wtot[v * kPlanWaves + w]; };

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // Copier workgroups (block < ncopy) start copying as soon as they hold the plan;
  // the one workgroup past them (block == ncopy) publishes it instead.
  const bool publish = block == ncopy;
  // One round of global loads: the current-copy index, the routed ids (n <= K <=
  // kMaxExperts = 4 per thread) and both state copies; the current copy is picked
  // once everything has arrived.
  const int32_t* st0 = blk + o.state0;
  const int32_t* st1 = blk + o.state0 + o.state_stride;
  const int cur_word = blk[o.cur];
  const unsigned tick0 = (unsigned)st0[o.tick], tick1 = (unsigned)st1[o.tick];
  int idv[kMaxExperts / kPlanThreads];
#pragma unroll
  for (int q = 0; q < kMaxExperts / kPlanThreads; ++q) {
    const int i = tid + q * kPlanThreads;
    idv[q] = i < n ? ids[i] : -1;
  }
  const int cur = cur_word & 1;
  int32_t* nst = blk + o.state0 + (cur ^ 1) * o.state_stride;           // written by the publisher
  const unsigned tick = cur ? tick1 : tick0;
  if (tid == 0) s_bad = 0;
  for (int e = tid; e < E; e += kPlanThreads) {
    const int a0 = st0[o.expert_slot + e], a1 = st1[o.expert_slot + e];
    s_es[e] = cur ? a1 : a0;
    s_cnt[e] = 0;
  }
  for (int j = tid; j < K; j += kPlanThreads) {
    const int a0 = st0[o.slot_expert + j], a1 = st1[o.slot_expert + j];
    const int b0 = st0[o.last_use + j], b1 = st1[o.last_use + j];
    s_se[j] = cur ? a1 : a0;
    s_lu[j] = (unsigned)(cur ? b1 : b0);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kMaxExperts / kPlanThreads; ++q) {
    const int i = tid + q * kPlanThreads;
    if (i >= n) break;
    const int id = idv[q];
    const bool ok = id >= 0 && id < E;
    s_ids[i] = ok ? id : -1;
    if (ok) atomicAdd(&s_cnt[id], 1); else atomicAdd(&s_bad, 1);
  }
  __syncthreads();

  // Exclusive prefixes over experts of: missing, present, entry count, GEMV
  // items of resident / missing experts, MFMA tiles of resident / missing
  // experts.  Thread t owns experts [t*per, (t+1)*per).
  const int per = (E + kPlanThreads - 1) / kPlanThreads;
  const int e0 = tid * per;
  int loc[kScanVals] = {0, 0, 0, 0, 0, 0, 0};
  for (int q = 0; q < per; ++q) {
    int e = e0 + q;
    if (e >= E) break;
    int c = s_cnt[e];
    if (c > 0) {
      const int miss = s_es[e] < 0;
      loc[0] += miss;
      loc[1] += 1;
      loc[2] += c;
      const int tl = (c + kTileM - 1) / kTileM;
      const bool gv = c < mfma_min;
      loc[3] += gv && !miss;
      loc[4] += gv && miss;
      loc[5] += gv || miss ? 0 : tl;
      loc[6] += !gv && miss ? tl : 0;
    }
  }
  int inc[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) inc[v] = wave_incl_scan(loc[v], lane);
  if (lane == 63) {
#pragma unroll
    for (int v = 0; v < kScanVals; ++v) s_wtot(v, wv) = inc[v];
  }
  __syncthreads();
  int base[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) {
    int b = 0, t = 0;
    for (int w = 0; w < kPlanWaves; ++w) { if (w < wv) b += s_wtot(v, w); t += s_wtot(v, w); }
    base[v] = b + inc[v] - loc[v];
    if (tid == 0) s_tot[v] = t;
  }
  {
    int run[kScanVals];
#pragma unroll
    for (int v = 0; v < kScanVals; ++v) run[v] = base[v];
    for (int q = 0; q < per; ++q) {
      int e = e0 + q;
      if (e >= E) break;
#pragma unroll
      for (int v = 0; v < kScanVals; ++v) s_pref(v, e) = (short)run[v];
      int c = s_cnt[e];
      if (c > 0) {
        const int miss = s_es[e] < 0;
        run[0] += miss;
        run[1] += 1;
        run[2] += c;
        const int tl = (c + kTileM - 1) / kTileM;
        const bool gv = c < mfma_min;
        run[3] += gv && !miss;
        run[4] += gv && miss;
        run[5] += gv || miss ? 0 : tl;
        run[6] += !gv && miss ? tl : 0;
      }
    }
  }
  // Evictable slots: empty, or holding an expert outside this wave (the wave is
  // every routed expert of the step).
  for (int j = tid; j < K; j += kPlanThreads) {
    int occ = s_se[j];
    s_cand[j] = occ < 0 || s_cnt[occ] == 0;
  }
  __syncthreads();
  const int n_miss = s_tot[0], D = s_tot[1], n_valid = s_tot[2];
  const int g_hit = s_tot[3], n_gemv = s_tot[3] + s_tot[4], t_hit = s_tot[5], n_tiles = s_tot[5] + s_tot[6];
  // Victims: the n_miss evictable slots of smallest (last_use, slot).  Up to 256
  // slots, wavefront 0 selects them in registers, one per round: the wavefront
  // minimum of 64-bit keys (last_use << 32 | slot) by an xor butterfly, which its
  // owner lane then retires.  Larger tables rank every candidate against all.
  if (K <= 4 * 64) {
    if (wv == 0 && n_miss > 0) {
      unsigned long long key[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = lane + 64 * q;
        key[q] = (j < K && s_cand[j]) ? ((unsigned long long)s_lu[j] << 32 | (unsigned)j) : ~0ull;
      }
      for (int r = 0; r < n_miss; ++r) {
        unsigned long long m = key[0] < key[1] ? key[0] : key[1];
        const unsigned long long m2 = key[2] < key[3] ? key[2] : key[3];
        m = m < m2 ? m : m2;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const unsigned long long o = __shfl_xor(m, off, 64);
          m = o < m ? o : m;
        }
        const int j = (int)(unsigned)(m & 0xFFFFFFFFull);
        if (lane == 0) s_victim[r] = j;
        if (lane == (j & 63)) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == (j >> 6)) key[q] = ~0ull;
        }
      }
    }
  } else {
    for (int j = tid; j < K; j += kPlanThreads) {
      if (!s_cand[j]) continue;
      const unsigned lj = s_lu[j];
      int r = 0;
      for (int q = 0; q < K; ++q) {
        const unsigned lq = s_lu[q];
        r += (int)s_cand[q] & ((int)(lq < lj) | ((int)(lq == lj) & (int)(q < j)));
      }
      if (r < n_miss) s_victim[r] = j;
    }
  }
  __syncthreads();
  // Place the i-th missing expert (ascending id) into the i-th victim.
  for (int e = tid; e < E; e += kPlanThreads) {
    if (s_cnt[e] == 0 || s_es[e] >= 0) continue;
    int r = s_pref(0, e);
    int j = s_victim[r];
    int old = s_se[j];
    s_plan_e[r] = e;
    if (publish) {
      blk[o.plan_expert + r] = e; blk[o.plan_slot + r] = j; blk[o.plan_evicted + r] = old;
    }
    s_se[j] = e;
    s_es[e] = j;
    if (old >= 0) s_es[old] = -1;      // old is outside the wave: no other thread reads it
  }
  __syncthreads();
  if (publish) {
    // The wave is one use: stamp every routed expert's slot; emit work lists.
    int32_t* used_expert = work + o.used_expert;
    int32_t* used_slot = work + o.used_slot;
    int32_t* used_off = work + o.used_off;
    int32_t* gemv_u = work + o.gemv_u;
    int4* tile_desc = reinterpret_cast<int4*>(work + o.tile_desc);
    for (int e = tid; e < E; e += kPlanThreads) {
      int c = s_cnt[e];
      if (c == 0) continue;
      int j = s_es[e];
      s_lu[j] = tick;
      int u = s_pref(1, e);
      used_expert[u] = e;
      used_slot[u] = j;
      used_off[u] = s_pref(2, e);
      // was this expert missing? (its missing-prefix steps up right after it)
      const bool miss = (e + 1 < E ? (int)s_pref(0, e + 1) : n_miss) > (int)s_pref(0, e);
      if (c < mfma_min) {
        const int g = miss ? g_hit + s_pref(4, e) : s_pref(3, e);
        gemv_u[g] = u;
        reinterpret_cast<int4*>(work + o.gemv_desc)[g] = make_int4(j, s_pref(2, e), c, e);
      } else {
        int t0 = miss ? t_hit + s_pref(6, e) : s_pref(5, e);
        for (int q = 0; q * kTileM < c; ++q)
          tile_desc[t0 + q] = make_int4(j, s_pref(2, e) + q * kTileM, min(kTileM, c - q * kTileM), e);
      }
    }
    __syncthreads();
    // Entries: ascending entry index inside each expert; slot map.
    int32_t* entries = work + o.entries;
    int32_t* slot_of = blk + o.slot_of;
    for (int i = tid; i < n; i += kPlanThreads) {
      int id = s_ids[i];
      if (id < 0) { slot_of[i] = -1; continue; }
      int r = 0;
      for (int q = 0; q < i; ++q) r += s_ids[q] == id;
      entries[s_pref(2, id) + r] = i;
      slot_of[i] = s_es[id];
    }
    // The new LRU state goes into the other copy; a later kernel of the step flips `cur`.
    for (int e = tid; e < E; e += kPlanThreads) nst[o.expert_slot + e] = s_es[e];
    for (int j = tid; j < K; j += kPlanThreads) {
      nst[o.slot_expert + j] = s_se[j];
      nst[o.last_use + j] = (int32_t)s_lu[j];
    }
    if (tid == 0) {
      const int nw = D > 0 ? 1 : 0;
      nst[o.tick] = (int32_t)(tick + nw);
      blk[o.n_waves] = nw;
      blk[o.plan_count] = n_miss;
      int32_t* hdr = work + o.hdr;
      hdr[0] = nw;
      hdr[hdr_wave_u(MW, 0)] = 0; hdr[hdr_wave_u(MW, 1)] = D;
      hdr[hdr_gemv(MW, 0)] = 0;   hdr[hdr_gemv(MW, 1)] = n_gemv;
      hdr[hdr_tile(MW, 0)] = 0;   hdr[hdr_tile(MW, 1)] = n_tiles;
      hdr[hdr_gemv_split(MW, 0)] = g_hit;
      hdr[hdr_tile_split(MW, 0)] = t_hit;
      used_off[D] = n_valid;
      atomicAdd(stats + ST_STEPS, 1ull);
      atomicAdd(stats + ST_DEVICE_PLANNED, 1ull);
      atomicAdd(stats + ST_WAVES, (unsigned long long)nw);
      atomicAdd(stats + ST_PAGE_INS, (unsigned long long)n_miss);
      atomicAdd(stats + ST_DISTINCT, (unsigned long long)D);
      atomicAdd(stats + ST_ENTRIES, (unsigned long long)n_valid);
      if (s_bad) atomicAdd(stats + ST_BAD_IDS, (unsigned long long)s_bad);
    }
  }
  return n_miss;
}

// LDS of the copiers' planner (copier_plan), sized by E experts, K slots and n
// entries.
struct CopierLds {
  int *es, *cnt, *se;
  unsigned* lu;
  int *ids, *plan_e, *victim, *off, *nm;
};

constexpr size_t copier_lds_bytes(int E, int K, int n) {
  return 2 * al16(4 * (size_t)E) + 5 * al16(4 * (size_t)K) + al16(4 * (size_t)n) + 16;
}

__device__ __forceinline__ CopierLds carve_copier(char* p, int E, int K, int n) {
  CopierLds L;
  L.es = reinterpret_cast<int*>(p); p += al16(4 * (size_t)E);
  L.cnt = reinterpret_cast<int*>(p); p += al16(4 * (size_t)E);
  L.se = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.lu = reinterpret_cast<unsigned*>(p); p += al16(4 * (size_t)K);
  L.plan_e = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.victim = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.off = reinterpret_cast<int*>(p); p += al16(4 * (size_t)K);
  L.ids = reinterpret_cast<int*>(p); p += al16(4 * (size_t)n);
  L.nm = reinterpret_cast<int*>(p);
  return L;
}

// The part of a device-planned wave's plan that a copier workgroup needs, made
// by one wavefront from the current state copy: the missing experts in
// ascending id (plan_e), the first sorted position of each (off: the prefix of
// entry counts over experts by id, where the planner puts its entries) and its
// victim slot (victim) -- the decisions plan_page_in_block makes, without the
// work lists, counters and new state that the publishing workgroup writes.
// Victims are the evictable slots (empty, or holding an expert outside the
// wave) of smallest (last_use, slot), one per round: the wavefront minimum of
// 64-bit keys by an xor butterfly, retired by its owner lane.  Needs E, K <=
// 256.  Returns the number of missing experts.
__device__ int copier_plan(const PlanArgs& p, char* lds) {
  const int E = p.E, K = p.K, n = p.n;
  const Offsets& o = p.o;
  const int32_t* __restrict__ blk = p.blk;
  const CopierLds L = carve_copier(lds, E, K, n);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // one round of global loads: current-copy index, both state copies, the ids
  const int32_t* st0 = blk + o.state0;
  const int32_t* st1 = blk + o.state0 + o.state_stride;
  const int cur = blk[o.cur] & 1;
  const int id = tid < n ? p.ids[tid] : -1;      // n <= K <= 256 = blockDim.x
  for (int e = tid; e < E; e += blockDim.x) {
    const int a0 = st0[o.expert_slot + e], a1 = st1[o.expert_slot + e];
    L.es[e] = cur ? a1 : a0;
    L.cnt[e] = 0;
  }
  for (int j = tid; j < K; j += blockDim.x) {
    const int a0 = st0[o.slot_expert + j], a1 = st1[o.slot_expert + j];
    const int b0 = st0[o.last_use + j], b1 = st1[o.last_use + j];
    L.se[j] = cur ? a1 : a0;
    L.lu[j] = (unsigned)(cur ? b1 : b0);
  }
  __syncthreads();
  if (tid < n) {
    const bool ok = id >= 0 && id < E;
    L.ids[tid] = ok ? id : -1;
    if (ok) atomicAdd(&L.cnt[id], 1);
  }
  __syncthreads();
  if (wv == 0) {
    int nm = 0, base = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {                  // experts 64q + lane, ascending
      const int e = 64 * q + lane;
      const int c = e < E ? L.cnt[e] : 0;
      const bool miss = c > 0 && L.es[e] < 0;
      const int inc = wave_incl_scan(c, lane);
      const unsigned long long mask = __ballot(miss);
      if (miss) {
        const int r = nm + __popcll(mask & ((1ull << lane) - 1ull));
        L.plan_e[r] = e;
        L.off[r] = base + inc - c;
      }
      nm += __popcll(mask);
      base += __shfl(inc, 63, 64);
    }
    unsigned long long key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = lane + 64 * q;
      const int occ = j < K ? L.se[j] : 0;
      const bool cand = j < K && (occ < 0 || L.cnt[occ] == 0);
      key[q] = cand ? ((unsigned long long)L.lu[j] << 32 | (unsigned)j) : ~0ull;
    }
    for (int r = 0; r < nm; ++r) {
      unsigned long long m = key[0] < key[1] ? key[0] : key[1];
      const unsigned long long m2 = key[2] < key[3] ? key[2] : key[3];
      m = m < m2 ? m : m2;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long v = __shfl_xor(m, off, 64);
        m = v < m ? v : m;
      }
      const int j = (int)(unsigned)(m & 0xFFFFFFFFull);
      if (lane == 0) L.victim[r] = j;
      if (lane == (j & 63)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (j >> 6)) key[q] = ~0ull;
      }
    }
    if (lane == 0) *L.nm = nm;
  }
  __syncthreads();
  return *L.nm;
}

// Page-in of a planned wave: the r-th missing expert's blob into its victim
// slot, copier workgroup `block` of `ncopy` taking its share of the 16-byte
// chunks.
__device__ void copy_planned(const PlanArgs& p, int block, int ncopy, const char* lds, int n_miss) {
  const PlanLds L = carve_plan(const_cast<char*>(lds), p.E, p.K, p.n);
  const size_t n16 = p.copy_bytes / 16;
  const size_t gtid = (size_t)block * blockDim.x + threadIdx.x;
  const size_t gstride = (size_t)ncopy * blockDim.x;
  for (int r = 0; r < n_miss; ++r) {
    const uint4* src = reinterpret_cast<const uint4*>(p.host_rows + (size_t)L.plan_e[r] * p.stride);
    uint4* dst = reinterpret_cast<uint4*>(p.slots + (size_t)L.victim[r] * p.stride);
    copy_chunks(dst, src, n16, gtid, gstride);
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_page_in_kernel(PlanArgs p, int ncopy) {
  extern __shared__ __align__(16) char lds[];
  const int n_miss = plan_page_in_block(p, blockIdx.x, ncopy, lds);
  if ((int)blockIdx.x < ncopy && p.do_copy) copy_planned(p, blockIdx.x, ncopy, lds, n_miss);
}

static PlanArgs plan_args(int32_t* blk, const int32_t* ids, int n, const Dims& d, const Offsets& o, int mfma_min,
                          int32_t* work, unsigned long long* stats, const uint8_t* host_rows, uint8_t* slots,
                          size_t stride, size_t copy_bytes, bool copy) {
  PlanArgs p;
  p.blk = blk; p.ids = ids; p.n = n; p.E = d.E; p.K = d.K; p.MW = d.max_waves; p.o = o; p.mfma_min = mfma_min;
  p.work = work; p.stats = stats; p.host_rows = host_rows; p.slots = slots; p.stride = stride;
  p.copy_bytes = copy_bytes; p.do_copy = copy ? 1 : 0;
  return p;
}

void launch_plan_page_in(int32_t* blk, const int32_t* ids, int n, const Dims& d, const Offsets& o,
                         int mfma_min, int32_t* work, unsigned long long* stats, const uint8_t* host_rows,
                         uint8_t* slots, size_t stride, size_t copy_bytes, bool copy, int grid, hipStream_t s) {
  const PlanArgs p = plan_args(blk, ids, n, d, o, mfma_min, work, stats, host_rows, slots, stride, copy_bytes, copy);
  const int ncopy = copy ? grid : 0;
  plan_page_in_kernel<<<ncopy + 1, kPlanThreads, plan_lds_bytes(d.E, d.K, n), s>>>(p, ncopy);
}

// Copy the planned experts of one host-planned wave (plan already in the layer block).
__global__ __launch_bounds__(kCopyThreads) void page_in_kernel(
    const int32_t* __restrict__ blk, Offsets o, int wave, int K, const uint8_t* __restrict__ host_rows,
    uint8_t* __restrict__ slots, size_t stride, size_t copy_bytes) {
  int cnt = blk[o.plan_count + wave];
  if (cnt > K) cnt = K;
  const int32_t* pe_ = blk + o.plan_expert + (size_t)wave * K;
  const int32_t* ps_ = blk + o.plan_slot + (size_t)wave * K;
  const size_t n16 = copy_bytes / 16;
  const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t gstride = (size_t)gridDim.x * blockDim.x;
  for (int r = 0; r < cnt; ++r) {
    const uint4* src = reinterpret_cast<const uint4*>(host_rows + (size_t)pe_[r] * stride);
    uint4* dst = reinterpret_cast<uint4*>(slots + (size_t)ps_[r] * stride);
    copy_chunks(dst, src, n16, gtid, gstride);
  }
}

void launch_page_in(const int32_t* blk, const Offsets& o, int wave, int K,
                    const uint8_t* host_rows, uint8_t* slots, size_t stride, size_t copy_bytes,
                    int grid, hipStream_t s) {
  page_in_kernel<<<grid, kCopyThreads, 0, s>>>(blk, o, wave, K, host_rows, slots, stride, copy_bytes);
}

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(uint4* __restrict__ dst,
                                                            const uint4* __restrict__ src, size_t n16) {
  copy_chunks(dst, src, n16, (size_t)blockIdx.x * blockDim.x + threadIdx.x,
              (size_t)gridDim.x * blockDim.x);
}

void launch_copy(void* dst, const void* src, size_t bytes, int grid, hipStream_t s) {
  copy_kernel<<<grid, kCopyThreads, 0, s>>>(static_cast<uint4*>(dst), static_cast<const uint4*>(src),
                                            bytes / 16);
}

// ------------------------------------------------------------------ GEMV expert kernels
//
// Weights are row-major; a row is read in 16-byte chunks by a group of LG lanes
// (LG = 8..64, 64/LG rows per wavefront at a time): lane g of the group takes
// chunks g, g + LG, ... so each load instruction of the wave reads contiguous
// memory.  Each lane accumulates its chunks in fp32 for every token of the
// expert, then the group reduces by an xor butterfly.  The arithmetic of one
// (token, row) dot product depends only on the row length and the format, never
// on which slot, wave or batch the expert is in.

namespace {
constexpr int kGemvThreads = 256;
constexpr int kMaxChunksInFlight = 4;

template <int FMT> struct Fmt;
template <> struct Fmt<PE_W_BF16> { static constexpr int VPC = 8; };        // values per 16-B chunk
template <> struct Fmt<PE_W_FP8_B128> { static constexpr int VPC = 16; };
template <> struct Fmt<PE_W_INT4_G128> { static constexpr int VPC = 32; };
template <> struct Fmt<PE_W_INT8_G128> { static constexpr int VPC = 16; };
template <> struct Fmt<PE_W_MXFP4_B32> { static constexpr int VPC = 32; };
// Per-row scales: int4 and int8 keep one fp16 scale per row and 128 columns,
// MXFP4 one E8M0 byte per row and 32 columns (one 16-byte chunk).
template <int FMT> constexpr bool kGroupScales = FMT == PE_W_INT4_G128 || FMT == PE_W_INT8_G128;
template <int FMT> constexpr bool kRowScales = kGroupScales<FMT> || FMT == PE_W_MXFP4_B32;
template <int FMT> constexpr int kScaleCols = FMT == PE_W_MXFP4_B32 ? 32 : 128;
template <int FMT> constexpr int kScaleBytes = FMT == PE_W_MXFP4_B32 ? 1 : 2;
}  // namespace

// Byte offset of row `row`'s scales in the row-scale region of a matrix with C columns.
template <int FMT>
__host__ __device__ __forceinline__ size_t row_scale_off(size_t row, int C) {
  return row * (size_t)(C / kScaleCols<FMT>) * kScaleBytes<FMT>;
}

// OCP E8M0 scale byte: 2^(e - 127) (e = 0 gives the fp32 subnormal 2^-127; 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : e == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float(e << 23);
}

// Loads of one row's chunks for one lane: chunks lig, lig + LG, ... (at most
// kMaxChunksInFlight per call, starting at chunk c0).
__device__ __forceinline__ void load_row(const uint4* __restrict__ row, int n_ch, int c0, int LG,
                                         uint4 (&w)[kMaxChunksInFlight]) {
#pragma unroll
  for (int q = 0; q < kMaxChunksInFlight; ++q) {
    const int c = c0 + q * LG;
    if (c < n_ch) w[q] = row[c];
  }
}

// The scale of the 16-byte chunk starting at column `col` of a row: the FP8
// block scale (one per 128 x 128 block), the int4 / int8 group scale (fp16,
// one per row and 128 columns) or the MXFP4 block scale (E8M0, one per row and
// 32 columns); 1 for bf16 (unused).  `s_row` points at the row's scales.
template <int FMT>
__device__ __forceinline__ float chunk_scale(const float* __restrict__ s_fp8_row,
                                             const uint8_t* __restrict__ s_row, int col) {
  if constexpr (FMT == PE_W_FP8_B128) return s_fp8_row[col >> 7];
  else if constexpr (kGroupScales<FMT>) return half_bits_to_f32(reinterpret_cast<const uint16_t*>(s_row)[col >> 7]);
  else if constexpr (FMT == PE_W_MXFP4_B32) return e8m0_to_f32(s_row[col >> 5]);
  else return 1.0f;
}

// The GEMV blocks stage the scales of their rows in LDS with the token vectors,
// so that a chunk's scale is an LDS read rather than a global load issued
// behind the previous chunk's arithmetic.  A row range's scales are one
// contiguous byte range of the scale region (FP8: the scale rows of the 128-row
// blocks it touches), staged in 16-byte words from `begin`, a multiple of 16.
// The rounding never leaves the blob: each scale region ends within 15 bytes of
// a 256-byte boundary that is the next region's start or the end of the copied
// blob.
struct ScaleSpan {
  size_t begin;
  int words;
};

// Scale bytes before row `row` of a C-column matrix (FP8: before its 128-row block).
template <int FMT>
__host__ __device__ __forceinline__ size_t scale_row_off(int row, int C) {
  if constexpr (FMT == PE_W_FP8_B128) return (size_t)(row >> 7) * (C / 128) * 4;
  else return row_scale_off<FMT>(row, C);
}

// Words of the staged scales of rows [r0, r1) (r0 < r1).
template <int FMT>
__device__ __forceinline__ ScaleSpan scale_span(int r0, int r1, int C) {
  size_t e;
  if constexpr (FMT == PE_W_FP8_B128) e = scale_row_off<FMT>(r1 - 1, C) + (C / 128) * 4;
  else e = scale_row_off<FMT>(r1, C);
  const size_t b = scale_row_off<FMT>(r0, C) & ~(size_t)15;
  return {b, (int)(((e + 15) & ~(size_t)15) - b) / 16};
}

// Most words scale_span can give for `rows` consecutive rows (0 for bf16).
template <int FMT>
__host__ __device__ __forceinline__ int scale_stage_words(int rows, int C) {
  if constexpr (FMT == PE_W_BF16) {
    return 0;
  } else {
    const size_t bytes = FMT == PE_W_FP8_B128 ? (size_t)((rows + 126) / 128 + 1) * (C / 128) * 4
                                              : row_scale_off<FMT>(rows, C);
    return (int)((bytes + 15) / 16 + 2);
  }
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// a.lo * b.lo + a.hi * b.hi + c, a and b packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Two fp32 values that bf16 holds exactly, packed as a bf16 pair (lo, hi).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Dot product of one 16-byte weight chunk (columns col .. col + VPC - 1) with m
// <= MB token vectors [MB][C] (bf16; in LDS or global memory), accumulated into
// acc in fp32 in a fixed order.  The chunk is decoded once into bf16 pairs
// (exact for every format) and each token takes one v_dot2 per pair, pair by
// pair; for the quantized formats the chunk's partial sum is then multiplied by
// its scale `sc` and added.  int4 nibbles are decoded as (q - 8) / 16 (exact), so
// their partial sum is 1/16 of the true one and the scale is taken times 16:
// the product is the same number.  MXFP4 codes are decoded to their E2M1 values
// (at most two significant bits: exact in bf16) and the chunk's one E8M0 scale
// multiplies the partial sum.  Every GEMV path runs a row as these chunk
// steps in ascending chunk order per lane, so a (token, row) dot product never
// depends on the launch it ran in.
template <int FMT, int MB>
__device__ __forceinline__ void dot_chunk(const uint4 w, int col, const uint16_t* __restrict__ xs, int C, int m,
                                          float sc, float (&acc)[MB]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  if constexpr (FMT == PE_W_BF16) {
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t >= m) break;
      const uint4 xv = *reinterpret_cast<const uint4*>(xs + t * C + col);
      float a = acc[t];
      a = dot2_bf16(wd[0], xv.x, a);
      a = dot2_bf16(wd[1], xv.y, a);
      a = dot2_bf16(wd[2], xv.z, a);
      a = dot2_bf16(wd[3], xv.w, a);
      acc[t] = a;
    }
  } else if constexpr (FMT == PE_W_FP8_B128) {
    // 16 e4m3 codes (OCP e4m3fn, hardware conversion), element pairs in order
    uint32_t wb[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[p], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[p], true);
      wb[2 * p] = pack_bf16x2(lo[0], lo[1]);
      wb[2 * p + 1] = pack_bf16x2(hi[0], hi[1]);
    }
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t >= m) break;
      const uint4* xp = reinterpret_cast<const uint4*>(xs + t * C + col);
      const uint4 x0 = xp[0], x1 = xp[1];
      const uint32_t xd[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float part = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) part = dot2_bf16(wb[p], xd[p], part);
      acc[t] = __builtin_fmaf(sc, part, acc[t]);
    }
  } else if constexpr (FMT == PE_W_INT8_G128) {
    // 16 bytes q, value q - 128 (an integer bf16 holds exactly), pairs in order
    uint32_t wb[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      wb[2 * p] = pack_bf16x2((float)(wd[p] & 0xFFu) - 128.0f, (float)((wd[p] >> 8) & 0xFFu) - 128.0f);
      wb[2 * p + 1] = pack_bf16x2((float)((wd[p] >> 16) & 0xFFu) - 128.0f, (float)(wd[p] >> 24) - 128.0f);
    }
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t >= m) break;
      const uint4* xp = reinterpret_cast<const uint4*>(xs + t * C + col);
      const uint4 x0 = xp[0], x1 = xp[1];
      const uint32_t xd[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float part = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) part = dot2_bf16(wb[p], xd[p], part);
      acc[t] = __builtin_fmaf(sc, part, acc[t]);
    }
  } else if constexpr (FMT == PE_W_MXFP4_B32) {
    // 32 E2M1 codes, element 2i the low nibble of byte i; v_cvt_scalef32_pk_bf16_fp4
    // with scale 1 turns the two codes of one byte into a bf16 pair (low first)
    uint32_t wb[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      wb[4 * v] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], 1.0f, 0));
      wb[4 * v + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], 1.0f, 1));
      wb[4 * v + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], 1.0f, 2));
      wb[4 * v + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], 1.0f, 3));
    }
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t >= m) break;
      const uint4* xp = reinterpret_cast<const uint4*>(xs + t * C + col);
      float part = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 xv = xp[v];
        part = dot2_bf16(wb[4 * v], xv.x, part);
        part = dot2_bf16(wb[4 * v + 1], xv.y, part);
        part = dot2_bf16(wb[4 * v + 2], xv.z, part);
        part = dot2_bf16(wb[4 * v + 3], xv.w, part);
      }
      acc[t] = __builtin_fmaf(sc, part, acc[t]);
    }
  } else {
    // 32 nibbles, element 2i the low nibble of byte i; q ^ 8 read as a signed
    // 4-bit value is q - 8, which v_cvt_off_f32_i4 turns into (q - 8) / 16
    uint32_t wb[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tw = (int)(wd[v] ^ 0x88888888u);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        wb[4 * v + b] = pack_bf16x2(__builtin_amdgcn_cvt_off_f32_i4(tw >> (8 * b)),
                                    __builtin_amdgcn_cvt_off_f32_i4(tw >> (8 * b + 4)));
    }
    const float sc16 = 16.0f * sc;
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t >= m) break;
      const uint4* xp = reinterpret_cast<const uint4*>(xs + t * C + col);
      float part = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 xv = xp[v];
        part = dot2_bf16(wb[4 * v], xv.x, part);
        part = dot2_bf16(wb[4 * v + 1], xv.y, part);
        part = dot2_bf16(wb[4 * v + 2], xv.z, part);
        part = dot2_bf16(wb[4 * v + 3], xv.w, part);
      }
      acc[t] = __builtin_fmaf(sc16, part, acc[t]);
    }
  }
}

// Dot products of the loaded chunks c0, c0 + LG, ... (at most
// kMaxChunksInFlight, below n_ch) of one row with m token vectors.
template <int FMT, int MB>
__device__ __forceinline__ void dot_row(const uint4 (&w)[kMaxChunksInFlight], int n_ch, int c0, int LG,
                                        const uint16_t* __restrict__ xs, int C, int m,
                                        const float* __restrict__ s_fp8_row,   // fp8: scales of this row's 128-row block
                                        const uint8_t* __restrict__ s_row,     // per-row formats: this row's scales
                                        float (&acc)[MB]) {
  constexpr int VPC = Fmt<FMT>::VPC;
#pragma unroll
  for (int q = 0; q < kMaxChunksInFlight; ++q) {
    const int c = c0 + q * LG;
    if (c >= n_ch) break;
    const int col = c * VPC;
    dot_chunk<FMT, MB>(w[q], col, xs, C, m, chunk_scale<FMT>(s_fp8_row, s_row, col), acc);
  }
}

// The value of lane (this lane xor m) for m = 1, 2, 4, 8 by DPP lane moves
// (quad_perm 1,0,3,2; quad_perm 2,3,0,1; row_half_mirror, which reads lane xor
// 7 within 8, then quad_perm 3,2,1,0; row_ror:8 within a row of 16), m = 16 by
// ds_swizzle (xor 16 within 32) and m = 32 through ds_bpermute.
__device__ __forceinline__ float lane_xor(float v, int m) {
  const int x = __float_as_int(v);
  switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    case 4: {
      const int h = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
      return __int_as_float(__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, false));
    }
    case 8: return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
    case 16: return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
    default: return __shfl_xor(v, m, 64);
  }
}

// Sum over the LG lanes of a group (xor butterfly, partners LG/2, ..., 2, 1;
// every lane gets the same total).  The masks are uniform, so the branches
// on them are scalar.  ROLL keeps the loop over the partners rolled (the same
// operations in the same order), for callers whose registers an unrolled
// butterfly would push into scratch.
template <int MB, bool ROLL = false>
__device__ __forceinline__ void group_reduce(float (&acc)[MB], int LG) {
  if constexpr (ROLL) {
#pragma unroll 1
    for (int off = 32; off > 0; off >>= 1) {
      if (off >= LG) continue;
#pragma unroll
      for (int t = 0; t < MB; ++t) acc[t] += lane_xor(acc[t], off);
    }
  } else {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      if (off >= LG) continue;
#pragma unroll
      for (int t = 0; t < MB; ++t) acc[t] += lane_xor(acc[t], off);
    }
  }
}

// Copy n 16-byte words into LDS, word i from src_of(i) to dst_of(i), every
// thread of the block taking words threadIdx.x, + blockDim.x, ...  Each thread
// issues up to four loads before it stores them (the last round too), so a copy
// of more words than threads costs one load latency per four words instead of
// one per word.
template <class SrcOf, class DstOf>
__device__ __forceinline__ void copy_words_to_lds(int n, SrcOf src_of, DstOf dst_of) {
  const int st = blockDim.x;
  int i = threadIdx.x;
  for (; i + 3 * st < n; i += 4 * st) {
    const uint4 v0 = *src_of(i), v1 = *src_of(i + st), v2 = *src_of(i + 2 * st), v3 = *src_of(i + 3 * st);
    *dst_of(i) = v0;
    *dst_of(i + st) = v1;
    *dst_of(i + 2 * st) = v2;
    *dst_of(i + 3 * st) = v3;
  }
  if (i < n) {
    const bool h1 = i + st < n, h2 = i + 2 * st < n;
    const uint4 v0 = *src_of(i);
    uint4 v1 = v0, v2 = v0;
    if (h1) v1 = *src_of(i + st);
    if (h2) v2 = *src_of(i + 2 * st);
    *dst_of(i) = v0;
    if (h1) *dst_of(i + st) = v1;
    if (h2) *dst_of(i + 2 * st) = v2;
  }
}

template <class SrcOf>
__device__ __forceinline__ void copy_words_to_lds(uint4* dst, int n, SrcOf src_of) {
  copy_words_to_lds(n, src_of, [=](int i) { return dst + i; });
}

// Stage rows `entries[pos0 + t] / k` (t < mb) of a bf16 [*, C] matrix into LDS.
__device__ __forceinline__ void stage_rows(uint16_t* xs, const uint16_t* __restrict__ src, int C,
                                           const int32_t* __restrict__ row_idx, int mb, int divisor) {
  const int n16 = C / 8;
  copy_words_to_lds(reinterpret_cast<uint4*>(xs), mb * n16, [=](int i) {
    const int t = i / n16, c = i - t * n16;
    return reinterpret_cast<const uint4*>(src + (size_t)(row_idx[t] / divisor) * C) + c;
  });
}

struct GemvItem {
  int slot, off, m;
  const int32_t* ent;   // the expert's entries (t*k + j), ascending, at sorted positions off..off+m-1
};

// Range [b, e) of a wave's list selected by a.part: 0 all, 1 resident before
// the wave ("hits"), 2 paged in by it.
__device__ __forceinline__ void part_range(const ExpertArgs& a, int begin, int split, int end, int& b, int& e) {
  b = a.part == 2 ? split : begin;
  e = a.part == 1 ? split : end;
}

// LDS of the lean expert discovery for n routed entries.
constexpr size_t lean_lds_bytes(int n) { return 3 * al16(4 * (size_t)n) + 16 + al16((size_t)n); }

// The item-th GEMV expert among those already resident, found from the routed
// ids and the current LRU-state copy without the published plan, so it can run
// while the planning + page-in workgroups are still in flight.  Same numbering
// as the planner: present experts by ascending id (sorted positions are the
// prefix of their entry counts), GEMV hits in ascending id.  Block-wide; n = T*k.
__device__ bool lean_hit_item(const ExpertArgs& a, int item, GemvItem& it, char* lds) {
  const int n = a.T * a.k, tid = threadIdx.x;
  int* s_id = reinterpret_cast<int*>(lds);
  int* s_cnt = reinterpret_cast<int*>(lds + al16(4 * (size_t)n));      // entries with this id, first occurrences
  int* s_ent = reinterpret_cast<int*>(lds + 2 * al16(4 * (size_t)n));
  int* s_sel = reinterpret_cast<int*>(lds + 3 * al16(4 * (size_t)n));
  unsigned char* s_hitg = reinterpret_cast<unsigned char*>(lds + 3 * al16(4 * (size_t)n) + 16);
  const int32_t* st = a.blk + a.o.state0 + (a.blk[a.o.cur] & 1) * a.o.state_stride;
  if (tid == 0) s_sel[0] = -1;
  for (int i = tid; i < n; i += blockDim.x) {
    const int id = a.ids[i];
    s_id[i] = (id >= 0 && id < a.E) ? id : -1;
  }
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int id = s_id[i];
    int cnt = 0;
    bool first = id >= 0;
    for (int j = 0; j < n; ++j) {
      if (s_id[j] != id) continue;
      ++cnt;
      if (j < i) first = false;
    }
    s_cnt[i] = first ? cnt : 0;
    s_hitg[i] = first && cnt < a.mfma_min && st[a.o.expert_slot + id] >= 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    if (!s_hitg[i]) continue;
    const int id = s_id[i];
    int rank = 0, off = 0;
    for (int j = 0; j < n; ++j) {
      if (s_cnt[j] == 0 || s_id[j] >= id) continue;
      off += s_cnt[j];
      rank += s_hitg[j];
    }
    if (rank == item) { s_sel[0] = id; s_sel[1] = off; s_sel[2] = s_cnt[i]; s_sel[3] = st[a.o.expert_slot + id]; }
  }
  __syncthreads();
  const int e = s_sel[0];
  if (e < 0) return false;
  for (int i = tid; i < n; i += blockDim.x) {
    if (s_id[i] != e) continue;
    int r = 0;
    for (int j = 0; j < i; ++j) r += s_id[j] == e;
    s_ent[r] = i;
  }
  __syncthreads();
  it.off = s_sel[1];
  it.m = s_sel[2];
  it.slot = s_sel[3];
  it.ent = s_ent;
  return true;
}

__device__ __forceinline__ bool gemv_item(const ExpertArgs& a, int item, GemvItem& it, char* lds) {
  if (a.lean) return lean_hit_item(a, item, it, lds);
  int g0, g1;
  if (a.hdr_known) {
    part_range(a, a.g0, a.gsplit, a.g1, g0, g1);
  } else {
    const int32_t* hdr = a.work + a.o.hdr;
    part_range(a, hdr[hdr_gemv(a.MW, a.wave)], hdr[hdr_gemv_split(a.MW, a.wave)], hdr[hdr_gemv(a.MW, a.wave + 1)], g0,
               g1);
  }
  if (item >= g1 - g0) return false;
  const int4 dsc = reinterpret_cast<const int4*>(a.work + a.o.gemv_desc)[g0 + item];
  it.slot = dsc.x;
  it.off = dsc.y;
  it.m = dsc.z;
  it.ent = a.work + a.o.entries + it.off;
  return true;
}

// LDS ahead of the staged token vectors: the lean discovery's arrays, if used.
__device__ __forceinline__ size_t gemv_lds_head(const ExpertArgs& a) {
  return a.lean ? lean_lds_bytes(a.T * a.k) : 0;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// LDS the GEMV blocks stage beyond the lean discovery's: MB token vectors of C
// values, then `sides` scale areas of scale_stage_words(rows, C) words each.
template <int FMT>
__host__ __device__ __forceinline__ size_t gemv_stage_bytes(int MB, int C, int rows, int sides) {
  return al16((size_t)MB * C * 2) + (size_t)sides * 16 * scale_stage_words<FMT>(rows, C);
}

// Gate/up projection + SwiGLU of one workgroup: used expert `by`, `nr` blocks of
// intermediate rows from bx * nr * rows_per_block; every lane group takes one
// row i of each block and computes h[pos, i] = bf16(silu(W1[i].x) * (W3[i].x)).
// The first block's weight loads are issued before the token vectors and the
// scales of all the workgroup's rows are staged in LDS; the blocks then run
// one after another on one set of weight registers, so `nr` changes neither a
// row's arithmetic nor the registers a lane needs (a launch picks it so that
// all its workgroups are resident).
template <int FMT, int MB>
__device__ void gate_up_block(const ExpertArgs& a, int bx, int by, int LG, int rows_per_block, char* lds,
                              int nr = 1) {
  GemvItem it;
  if (!gemv_item(a, by, it, lds)) return;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + gemv_lds_head(a));   // [MB][H]
  constexpr int VPC = Fmt<FMT>::VPC;
  const int H = a.H, I = a.I;
  const int n_ch = H / VPC;
  const uint8_t* blob = a.slots + (size_t)it.slot * a.slot_stride;
  const uint4* W13 = reinterpret_cast<const uint4*>(blob + a.off_w13);
  const uint8_t* S13b = blob + a.off_s13;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int groups = 64 / LG, lig = lane % LG, grp = lane / LG;
  const int i0 = bx * nr * rows_per_block + wv * groups + grp;     // this group's row in the first block
  // the workgroup's gate rows [R0, R1) and up rows I + [R0, R1): their scales
  // are staged at s_sc (gate) and s_sc + 16 SW (up)
  const int R0 = bx * nr * rows_per_block, R1 = min(I, R0 + nr * rows_per_block);
  const int SW = scale_stage_words<FMT>(nr * rows_per_block, H);
  char* s_sc = lds + gemv_lds_head(a) + al16((size_t)MB * H * 2);
  int* s_e8 = reinterpret_cast<int*>(s_sc + 32 * (size_t)SW);     // the token batch's entries
  ScaleSpan gs{0, 0}, us{0, 0};
  if constexpr (FMT != PE_W_BF16) {
    gs = scale_span<FMT>(R0, R1, H);
    us = scale_span<FMT>(I + R0, I + R1, H);
  }
  const uint16_t* x = a.x;
  const int32_t* ent = it.ent;
  const int k = a.k;
  for (int tb = 0; tb < it.m; tb += MB) {
    const int mb = min(MB, it.m - tb);
    uint4 wg[kMaxChunksInFlight], wu[kMaxChunksInFlight];
    if (i0 < I) {
      load_row(W13 + (size_t)i0 * n_ch, n_ch, lig, LG, wg);
      load_row(W13 + (size_t)(I + i0) * n_ch, n_ch, lig, LG, wu);
    }
    if (tb > 0) __syncthreads();     // the previous batch's token vectors are consumed
    // the batch's entries (the work lists may be in host memory: one read each)
    if ((int)threadIdx.x < mb) s_e8[threadIdx.x] = ent[tb + threadIdx.x];
    __syncthreads();
    // the batch's token vectors, and with the first batch the scales
    const int n16 = H / 8, xw = mb * n16, sw = tb == 0 ? gs.words + us.words : 0;
    copy_words_to_lds(
        xw + sw,
        [=](int i) -> const uint4* {
          if (i < xw) {
            const int t = i / n16;
            return reinterpret_cast<const uint4*>(x + (size_t)(s_e8[t] / k) * H) + (i - t * n16);
          }
          const int j = i - xw;
          return j < gs.words ? reinterpret_cast<const uint4*>(S13b + gs.begin) + j
                              : reinterpret_cast<const uint4*>(S13b + us.begin) + (j - gs.words);
        },
        [=](int i) -> uint4* {
          if (i < xw) return reinterpret_cast<uint4*>(xs) + i;
          const int j = i - xw;
          return reinterpret_cast<uint4*>(s_sc) + (j < gs.words ? j : SW + j - gs.words);
        });
    __syncthreads();
#pragma unroll 1
    for (int r = 0; r < nr; ++r) {
      const int ir = i0 + r * rows_per_block, ru = I + ir;
      if (ir >= I) break;
      if (r > 0) {
        load_row(W13 + (size_t)ir * n_ch, n_ch, lig, LG, wg);
        load_row(W13 + (size_t)ru * n_ch, n_ch, lig, LG, wu);
      }
      float g[MB], u[MB];
#pragma unroll
      for (int t = 0; t < MB; ++t) { g[t] = 0.0f; u[t] = 0.0f; }
      const char* sg = s_sc;
      const char* su = s_sc + 16 * (size_t)SW;
      if constexpr (FMT != PE_W_BF16) {
        sg += scale_row_off<FMT>(ir, H) - gs.begin;
        su += scale_row_off<FMT>(ru, H) - us.begin;
      }
      const float* sgf = reinterpret_cast<const float*>(sg);
      const float* suf = reinterpret_cast<const float*>(su);
      const uint8_t* sgh = reinterpret_cast<const uint8_t*>(sg);
      const uint8_t* suh = reinterpret_cast<const uint8_t*>(su);
      for (int c0 = lig;; c0 += LG * kMaxChunksInFlight) {
        dot_row<FMT, MB>(wg, n_ch, c0, LG, xs, H, mb, sgf, sgh, g);
        dot_row<FMT, MB>(wu, n_ch, c0, LG, xs, H, mb, suf, suh, u);
        if (c0 + LG * kMaxChunksInFlight >= n_ch) break;
        load_row(W13 + (size_t)ir * n_ch, n_ch, c0 + LG * kMaxChunksInFlight, LG, wg);
        load_row(W13 + (size_t)ru * n_ch, n_ch, c0 + LG * kMaxChunksInFlight, LG, wu);
      }
      group_reduce<MB>(g, LG);
      group_reduce<MB>(u, LG);
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        if (t < mb && lig == t)
          a.h[(size_t)(it.off + tb + t) * I + ir] = f32_to_bf16(silu_f(g[t]) * u[t]);
      }
    }
  }
}

// Down projection of one workgroup: used expert `by`, rows from bx *
// rows_per_block; every lane group takes two rows n, n+1 and writes
// merged[entry, n] = w[entry] * (W2[n] . h[pos]).  The scales of the
// workgroup's rows are staged in LDS with the first batch of h rows.
template <int FMT, int MB>
__device__ void down_block(const ExpertArgs& a, int bx, int by, int LG, int rows_per_block, char* lds) {
  GemvItem it;
  if (!gemv_item(a, by, it, lds)) return;
  uint16_t* hs = reinterpret_cast<uint16_t*>(lds + gemv_lds_head(a));   // [MB][I]
  constexpr int VPC = Fmt<FMT>::VPC;
  const int H = a.H, I = a.I;
  const int n_ch = I / VPC;
  const uint8_t* blob = a.slots + (size_t)it.slot * a.slot_stride;
  const uint4* W2 = reinterpret_cast<const uint4*>(blob + a.off_w2);
  const uint8_t* S2b = blob + a.off_s2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int groups = 64 / LG, lig = lane % LG, grp = lane / LG;
  const int n0 = bx * rows_per_block + 2 * (wv * groups + grp);   // rows n0, n0 + 1
  const bool act0 = n0 < H, act1 = n0 + 1 < H;
  const uint4* r0 = W2 + (size_t)n0 * n_ch;
  const uint4* r1 = W2 + (size_t)(n0 + 1) * n_ch;
  // the workgroup's rows [R0, R1): their scales are staged at s_sc
  const int R0 = bx * rows_per_block, R1 = min(H, R0 + rows_per_block);
  char* s_sc = lds + gemv_lds_head(a) + al16((size_t)MB * I * 2);
  ScaleSpan ss{0, 0};
  if constexpr (FMT != PE_W_BF16) ss = scale_span<FMT>(R0, R1, I);
  const char* sc0 = s_sc;
  const char* sc1 = s_sc;
  if constexpr (FMT != PE_W_BF16) {
    sc0 += scale_row_off<FMT>(n0, I) - ss.begin;
    sc1 += scale_row_off<FMT>(act1 ? n0 + 1 : n0, I) - ss.begin;
  }
  const uint16_t* h = a.h;
  const int32_t* ent = it.ent;
  for (int tb = 0; tb < it.m; tb += MB) {
    const int mb = min(MB, it.m - tb);
    // lane lig stores token lig of the batch: its entry now, its router weight
    // once the entry has arrived (both in flight during the dot products)
    const int e_l = lig < mb ? ent[tb + lig] : 0;
    uint4 w0[kMaxChunksInFlight], w1[kMaxChunksInFlight];
    if (act0) load_row(r0, n_ch, lig, LG, w0);
    if (act1) load_row(r1, n_ch, lig, LG, w1);
    if (tb > 0) __syncthreads();     // the previous batch's h rows are consumed
    // the batch's h rows (consecutive sorted positions), and with the first batch the scales
    const int hw = mb * (I / 8), sw = tb == 0 ? ss.words : 0;
    const uint4* hsrc = reinterpret_cast<const uint4*>(h + (size_t)(it.off + tb) * I);
    copy_words_to_lds(
        hw + sw,
        [=](int i) { return i < hw ? hsrc + i : reinterpret_cast<const uint4*>(S2b + ss.begin) + (i - hw); },
        [=](int i) { return i < hw ? reinterpret_cast<uint4*>(hs) + i : reinterpret_cast<uint4*>(s_sc) + (i - hw); });
    __syncthreads();
    if (!act0) continue;
    const float w_l = lig < mb ? a.topk_w[e_l] : 0.0f;
    float y0[MB], y1[MB];
#pragma unroll
    for (int t = 0; t < MB; ++t) { y0[t] = 0.0f; y1[t] = 0.0f; }
    for (int c0 = lig;; c0 += LG * kMaxChunksInFlight) {
      dot_row<FMT, MB>(w0, n_ch, c0, LG, hs, I, mb, reinterpret_cast<const float*>(sc0),
                       reinterpret_cast<const uint8_t*>(sc0), y0);
      if (act1)
        dot_row<FMT, MB>(w1, n_ch, c0, LG, hs, I, mb, reinterpret_cast<const float*>(sc1),
                         reinterpret_cast<const uint8_t*>(sc1), y1);
      if (c0 + LG * kMaxChunksInFlight >= n_ch) break;
      load_row(r0, n_ch, c0 + LG * kMaxChunksInFlight, LG, w0);
      if (act1) load_row(r1, n_ch, c0 + LG * kMaxChunksInFlight, LG, w1);
    }
    group_reduce<MB>(y0, LG);
    group_reduce<MB>(y1, LG);
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t < mb && lig == t) {
        a.merged[(size_t)e_l * H + n0] = w_l * y0[t];
        if (act1) a.merged[(size_t)e_l * H + n0 + 1] = w_l * y1[t];
      }
    }
  }
}

// Geometry of one GEMV launch: lanes per row, rows per workgroup, workgroups per
// expert along the rows.
struct GemvGeom {
  int LG, rows_per_block, gx;
};

template <int FMT, int MB>
__global__ __launch_bounds__(kGemvThreads) void gemv_gate_up_kernel(ExpertArgs a, GemvGeom g) {
  extern __shared__ __align__(16) char lds[];
  gate_up_block<FMT, MB>(a, blockIdx.x, blockIdx.y, g.LG, g.rows_per_block, lds);
}

template <int FMT, int MB>
__global__ __launch_bounds__(kGemvThreads) void gemv_down_kernel(ExpertArgs a, GemvGeom g) {
  extern __shared__ __align__(16) char lds[];
  down_block<FMT, MB>(a, blockIdx.x, blockIdx.y, g.LG, g.rows_per_block, lds);
}

// LDS for the gate/up scales one stream_gate_up_rows block stages (gate rows in
// the first half, up rows in the second): at most 1024 bytes each for hidden <=
// 4096 (int4 / int8: rows_per_block * hidden / 128 fp16, at most 512; MXFP4:
// rows_per_block * hidden / 32 bytes, at most 1024; FP8: one 128-row block row).
constexpr size_t kStreamScaleLds = 2048;
// LDS for one token batch's entries (at most 8), staged by every GEMV gate/up
// block before it reads the batch's token vectors.
constexpr size_t kEntStage = 32;

// Gate/up row block gi of a missing expert, paged in and projected in one pass:
// rows i of the block (gemv_gate_up_kernel's geometry) are read from the mapped
// host row `src`, stored into the slot `dst` and, as each 16-byte chunk arrives,
// dotted with the expert's m token vectors (entries `ent`, staged in LDS `xs`),
// one chunk per row in flight ahead of the arithmetic.  The block's scales are
// staged once through LDS `s_sc` (one contiguous read per side, in 2-byte units)
// and stored into the slot as well.  The lane's chunk order and the reduction are
// those of gate_up_block, so h is bit-identical to a gate/up projection read
// back from the slot.
template <int FMT, int MB>
__device__ void stream_gate_up_rows(const ExpertArgs& a, const GemvGeom& g, const uint8_t* __restrict__ src,
                                    uint8_t* __restrict__ dst, int gi, const int* ent, int m, int off,
                                    uint16_t* xs, char* s_sc, int* s_e8) {
  constexpr int VPC = Fmt<FMT>::VPC;
  const int H = a.H, I = a.I, n_ch = H / VPC, LG = g.LG;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int groups = 64 / LG, lig = lane % LG, grp = lane / LG;
  const int i0 = gi * g.rows_per_block;
  const int i = i0 + wv * groups + grp;    // this group's gate row; up row I + i
  const bool active = i < I;
  const uint4* sg = reinterpret_cast<const uint4*>(src + a.off_w13) + (size_t)i * n_ch;
  const uint4* su = reinterpret_cast<const uint4*>(src + a.off_w13) + (size_t)(I + i) * n_ch;
  uint4* dg = reinterpret_cast<uint4*>(dst + a.off_w13) + (size_t)i * n_ch;
  uint4* du = reinterpret_cast<uint4*>(dst + a.off_w13) + (size_t)(I + i) * n_ch;
  // the block's scale bytes [og, og + nb) (gate) and [ou, ou + nb) (up) of the S13 region
  size_t og = 0, ou = 0;
  int nb = 0;
  if constexpr (kRowScales<FMT>) {
    og = row_scale_off<FMT>(i0, H);
    ou = row_scale_off<FMT>(I + i0, H);
    nb = (int)row_scale_off<FMT>(min(g.rows_per_block, I - i0), H);
  } else if constexpr (FMT == PE_W_FP8_B128) {
    og = (size_t)(i0 >> 7) * (H / 128) * 4;
    ou = (size_t)((I + i0) >> 7) * (H / 128) * 4;
    nb = (H / 128) * 4;
  }
  const bool store_sc = kRowScales<FMT> || (i0 & 127) == 0;   // one block per FP8 block row
  const float* sgf = reinterpret_cast<const float*>(s_sc);
  const float* suf = reinterpret_cast<const float*>(s_sc + kStreamScaleLds / 2);
  const uint8_t* sgh = reinterpret_cast<const uint8_t*>(s_sc) + row_scale_off<FMT>(i - i0, H);
  const uint8_t* suh = reinterpret_cast<const uint8_t*>(s_sc + kStreamScaleLds / 2) + row_scale_off<FMT>(i - i0, H);
  // the first token batch also stores the rows (tb == 0 runs even for m == 0)
  for (int tb = 0; tb == 0 || tb < m; tb += MB) {
    const int mb = max(0, min(MB, m - tb));
    int c = lig;
    uint4 wg = make_uint4(0, 0, 0, 0), wu = wg;
    if (active && c < n_ch) { wg = sg[c]; wu = su[c]; }     // in flight during the staging
    __syncthreads();
    if ((int)threadIdx.x < mb) s_e8[threadIdx.x] = ent[tb + threadIdx.x];    // the entries may be in host memory
    __syncthreads();
    stage_rows(xs, a.x, H, s_e8, mb, a.k);
    if (FMT != PE_W_BF16 && tb == 0) {
      const uint16_t* hs = reinterpret_cast<const uint16_t*>(src + a.off_s13);
      uint16_t* ds = reinterpret_cast<uint16_t*>(dst + a.off_s13);
      uint16_t* ls = reinterpret_cast<uint16_t*>(s_sc);
      const int nu = nb / 2;
      for (int q = threadIdx.x; q < 2 * nu; q += blockDim.x) {
        const bool up = q >= nu;
        const size_t at = (up ? ou : og) / 2 + (q - (up ? nu : 0));
        const uint16_t v = hs[at];
        ls[(up ? kStreamScaleLds / 4 : 0) + (q - (up ? nu : 0))] = v;
        if (store_sc) ds[at] = v;
      }
    }
    __syncthreads();
    if (!active) continue;
    float gacc[MB], uacc[MB];
#pragma unroll
    for (int t = 0; t < MB; ++t) { gacc[t] = 0.0f; uacc[t] = 0.0f; }
    while (c < n_ch) {
      const int cn = c + LG;
      uint4 ng = make_uint4(0, 0, 0, 0), nu = ng;
      if (cn < n_ch) { ng = sg[cn]; nu = su[cn]; }
      if (tb == 0) { dg[c] = wg; du[c] = wu; }
      dot_chunk<FMT, MB>(wg, c * VPC, xs, H, mb, chunk_scale<FMT>(sgf, sgh, c * VPC), gacc);
      dot_chunk<FMT, MB>(wu, c * VPC, xs, H, mb, chunk_scale<FMT>(suf, suh, c * VPC), uacc);
      c = cn; wg = ng; wu = nu;
    }
    group_reduce<MB>(gacc, LG);
    group_reduce<MB>(uacc, LG);
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t < mb && lig == t)
        a.h[(size_t)(off + tb + t) * I + i] = f32_to_bf16(silu_f(gacc[t]) * uacc[t]);
    }
  }
}

// The part of an expert blob a streamed page-in copies plainly: the down
// weights [off_w2, off_s13) and their scales [off_s2, copy_bytes) (the gate/up
// rows and scales are stored by stream_gate_up_rows).
__device__ __forceinline__ void copy_blob_rest(const ExpertArgs& a, const uint8_t* src, uint8_t* dst,
                                               size_t copy_bytes, size_t gtid, size_t gstride) {
  copy_chunks(reinterpret_cast<uint4*>(dst + a.off_w2), reinterpret_cast<const uint4*>(src + a.off_w2),
              (a.off_s13 - a.off_w2) / 16, gtid, gstride);
  copy_chunks(reinterpret_cast<uint4*>(dst + a.off_s2), reinterpret_cast<const uint4*>(src + a.off_s2),
              (copy_bytes - a.off_s2) / 16, gtid, gstride);
}

// Page-in of a device-planned wave's missing experts with their gate/up
// projection fused in (copier workgroup w of P): the gate/up row blocks of all
// missing experts are dealt round-robin, block gi of the r-th missing expert
// being item r * gx + gi; then the rest of every blob (down weights, scales) is
// copied plainly.  The missing experts' weights cross the host link once and are
// never read back from HBM in this step's gate/up.
template <int FMT, int MB>
__device__ void stream_in(const PlanArgs& p, const ExpertArgs& a, const GemvGeom& g, int w, int P, char* lds,
                          int n_miss) {
  const CopierLds L = carve_copier(lds, p.E, p.K, p.n);
  const size_t plan_b = copier_lds_bytes(p.E, p.K, p.n);
  int* s_ent = reinterpret_cast<int*>(lds + plan_b);                                    // [n]
  char* s_sc = lds + plan_b + al16(4 * (size_t)p.n);                                    // scales
  uint16_t* xs = reinterpret_cast<uint16_t*>(s_sc + kStreamScaleLds);                   // [MB][H]
  int* s_e8 = reinterpret_cast<int*>(s_sc + kStreamScaleLds + al16((size_t)MB * a.H * 2));   // [MB]
  for (int r = 0; r < n_miss; ++r) {
    int gi = ((w - (r * g.gx) % P) % P + P) % P;     // this workgroup's first block of expert r
    if (gi >= g.gx) continue;
    const int e = L.plan_e[r];
    for (int i = threadIdx.x; i < p.n; i += blockDim.x) {     // entries of e, ascending
      if (L.ids[i] != e) continue;
      int rank = 0;
      for (int q = 0; q < i; ++q) rank += L.ids[q] == e;
      s_ent[rank] = i;
    }
    const int m = L.cnt[e], off = L.off[r];
    const uint8_t* src = p.host_rows + (size_t)e * p.stride;
    uint8_t* dst = p.slots + (size_t)L.victim[r] * p.stride;
    for (; gi < g.gx; gi += P) stream_gate_up_rows<FMT, MB>(a, g, src, dst, gi, s_ent, m, off, xs, s_sc, s_e8);
    __syncthreads();     // s_ent is rebuilt for the next expert
  }
  for (int r = 0; r < n_miss; ++r)
    copy_blob_rest(a, p.host_rows + (size_t)L.plan_e[r] * p.stride, p.slots + (size_t)L.victim[r] * p.stride,
                   p.copy_bytes, (size_t)w * blockDim.x + threadIdx.x, (size_t)P * blockDim.x);
}

// Host-planned wave with no MFMA tiles, launch A: workgroups [0, P) page in the
// wave's missing experts (its GEMV items past the hit split), computing their
// gate/up projection from the rows as they arrive (stream_gate_up_rows), then
// copy the rest of each blob; the next ceil(gx / nr) x hit items run the
// gate/up projection of the wave's experts that were already resident
// (`a.part` = 1), nr row blocks each.  If `up_bytes` is not 0, one more
// workgroup copies the host's plan (layer block and work lists, `up_bytes`
// from the mapped host mirror `up_src`) into device memory at `up_dst`, while
// the others read their work lists from the mirror itself (`a.work`, with the
// wave's GEMV ranges in `a.g0 / a.gsplit / a.g1`): the step's first wave then
// needs no launch of its own for the upload.  The wave's down projection
// follows as its own launch.
template <int FMT, int MB>
__global__ __launch_bounds__(kGemvThreads) void wave_a_kernel(ExpertArgs a, GemvGeom g, int P, int nr,
                                                              const uint8_t* __restrict__ host_rows,
                                                              size_t stride, size_t copy_bytes,
                                                              const uint4* __restrict__ up_src,
                                                              uint4* __restrict__ up_dst, size_t up_bytes) {
  extern __shared__ __align__(16) char lds[];
  if (up_bytes && blockIdx.x == gridDim.x - 1) {
    copy_chunks(up_dst, up_src, up_bytes / 16, threadIdx.x, blockDim.x);
    return;
  }
  if ((int)blockIdx.x >= P) {
    const int gxn = (g.gx + nr - 1) / nr;
    const int b = blockIdx.x - P;
    gate_up_block<FMT, MB>(a, b % gxn, b / gxn, g.LG, g.rows_per_block, lds, nr);
    return;
  }
  const int w = blockIdx.x;
  int split, g1;
  if (a.hdr_known) {
    split = a.gsplit;
    g1 = a.g1;
  } else {
    const int32_t* hdr = a.work + a.o.hdr;
    split = hdr[hdr_gemv_split(a.MW, a.wave)];
    g1 = hdr[hdr_gemv(a.MW, a.wave + 1)];
  }
  const int4* desc = reinterpret_cast<const int4*>(a.work + a.o.gemv_desc);
  char* s_sc = lds;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + kStreamScaleLds);
  int* s_e8 = reinterpret_cast<int*>(lds + kStreamScaleLds + al16((size_t)MB * a.H * 2));
  const int n_miss = g1 - split;
  for (int r = 0; r < n_miss; ++r) {
    int gi = ((w - (r * g.gx) % P) % P + P) % P;
    if (gi >= g.gx) continue;
    const int4 d = desc[split + r];     // {slot, first sorted position, entries, expert}
    const uint8_t* src = host_rows + (size_t)d.w * stride;
    uint8_t* dst = const_cast<uint8_t*>(a.slots) + (size_t)d.x * a.slot_stride;
    for (; gi < g.gx; gi += P)
      stream_gate_up_rows<FMT, MB>(a, g, src, dst, gi, a.work + a.o.entries + d.y, d.z, d.y, xs, s_sc, s_e8);
  }
  for (int r = 0; r < n_miss; ++r) {
    const int4 d = desc[split + r];
    copy_blob_rest(a, host_rows + (size_t)d.w * stride, const_cast<uint8_t*>(a.slots) + (size_t)d.x * a.slot_stride,
                   copy_bytes, (size_t)w * blockDim.x + threadIdx.x, (size_t)P * blockDim.x);
  }
}

// Device-planned step with no many-token expert (E, K <= 256), launch A:
// workgroups [0, P) make the copiers' part of the plan (copier_plan) and page in
// the wave's missing experts with their gate/up projection (stream_in);
// workgroup P makes the whole plan and publishes it (plan, new LRU state, work
// lists, counters); the rest run the gate/up projection of the experts that were
// already resident (lean discovery, `a.lean` set).  Every planning workgroup
// decides from the same state copy by the same rules, and no workgroup waits
// for another.
template <int FMT, int MB>
__global__ __launch_bounds__(kGemvThreads) void step_a_kernel(PlanArgs p, int P, ExpertArgs a, GemvGeom g,
                                                              int nr) {
  extern __shared__ __align__(16) char lds[];
  if ((int)blockIdx.x < P) {
    stream_in<FMT, MB>(p, a, g, blockIdx.x, P, lds, copier_plan(p, lds));
  } else if ((int)blockIdx.x == P) {
    plan_page_in_block(p, P, P, lds);
  } else {
    // nr row blocks per workgroup, so every workgroup of the launch is resident at once
    const int gxn = (g.gx + nr - 1) / nr;
    const int b = blockIdx.x - P - 1;
    gate_up_block<FMT, MB>(a, b % gxn, b / gxn, g.LG, g.rows_per_block, lds, nr);
  }
}

// First round of one down-projection lane group's loads for rows n0 and n0 + 1
// of expert blob `blob`: chunks lig, lig + LG, ... (kMaxChunksInFlight at most)
// and each chunk's scale.
struct DownRows {
  uint4 w0[kMaxChunksInFlight], w1[kMaxChunksInFlight];
  float s0[kMaxChunksInFlight], s1[kMaxChunksInFlight];
};

template <int FMT>
__device__ __forceinline__ void fetch_down_rows(const ExpertArgs& a, const uint8_t* blob, int n0, bool act0,
                                                bool act1, int c0, int LG, int n_ch, DownRows& r) {
  constexpr int VPC = Fmt<FMT>::VPC;
  const int I = a.I;
  const uint4* W2 = reinterpret_cast<const uint4*>(blob + a.off_w2);
  const float* S2f = reinterpret_cast<const float*>(blob + a.off_s2);
  const uint8_t* S2b = blob + a.off_s2;
  if (act0) load_row(W2 + (size_t)n0 * n_ch, n_ch, c0, LG, r.w0);
  if (act1) load_row(W2 + (size_t)(n0 + 1) * n_ch, n_ch, c0, LG, r.w1);
#pragma unroll
  for (int q = 0; q < kMaxChunksInFlight; ++q) {
    const int c = c0 + q * LG;
    r.s0[q] = r.s1[q] = 1.0f;
    if (c >= n_ch) continue;
    if (act0) r.s0[q] = chunk_scale<FMT>(S2f + (size_t)(n0 >> 7) * (I / 128), S2b + row_scale_off<FMT>(n0, I), c * VPC);
    if (act1)
      r.s1[q] = chunk_scale<FMT>(S2f + (size_t)((n0 + 1) >> 7) * (I / 128), S2b + row_scale_off<FMT>(n0 + 1, I),
                                 c * VPC);
  }
}

// One GEMV expert's down projection for rows n0, n0 + 1 of one lane group:
// s_y[e * RB + row - r0] = w[e] * (W2[row] . h[pos]) for each of its entries e
// (s_ent: the entry at each sorted position, s_w: router weights by entry,
// both staged in LDS).  `r` holds the first round of loads of token batch 0.
// Per lane the chunks run in ascending order and the group reduces by the xor
// butterfly, as in down_block.
template <int FMT, int MB, bool ROLL>
__device__ __forceinline__ void down_rows_item(const ExpertArgs& a, const int4 dsc, DownRows& r, int n0,
                                               bool act0, bool act1, int lig, int LG, int n_ch,
                                               const uint16_t* hbase, float* s_y, int RB, int r0,
                                               const int* s_ent, const float* s_w) {
  constexpr int VPC = Fmt<FMT>::VPC;
  const int I = a.I, off = dsc.y, m = dsc.z;
  const uint8_t* blob = a.slots + (size_t)dsc.x * a.slot_stride;
  const int* ent = s_ent + off;
  for (int tb = 0; tb < m; tb += MB) {
    const int mb = min(MB, m - tb);
    if (tb > 0) fetch_down_rows<FMT>(a, blob, n0, act0, act1, lig, LG, n_ch, r);
    const uint16_t* hs = hbase + (size_t)(off + tb) * I;
    float y0[MB], y1[MB];
#pragma unroll
    for (int t = 0; t < MB; ++t) { y0[t] = 0.0f; y1[t] = 0.0f; }
    if (act0) {
      for (int c0 = lig;; c0 += LG * kMaxChunksInFlight) {
#pragma unroll
        for (int q = 0; q < kMaxChunksInFlight; ++q) {
          const int c = c0 + q * LG;
          if (c >= n_ch) break;
          dot_chunk<FMT, MB>(r.w0[q], c * VPC, hs, I, mb, r.s0[q], y0);
          if (act1) dot_chunk<FMT, MB>(r.w1[q], c * VPC, hs, I, mb, r.s1[q], y1);
        }
        if (c0 + LG * kMaxChunksInFlight >= n_ch) break;
        fetch_down_rows<FMT>(a, blob, n0, act0, act1, c0 + LG * kMaxChunksInFlight, LG, n_ch, r);
      }
    }
    group_reduce<MB, ROLL>(y0, LG);
    group_reduce<MB, ROLL>(y1, LG);
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (t < mb && lig == t && act0) {
        const int e = ent[tb + t];
        const float we = s_w[e];
        s_y[(size_t)e * RB + n0 - r0] = we * y0[t];
        if (act1) s_y[(size_t)e * RB + n0 + 1 - r0] = we * y1[t];
      }
    }
  }
}

// One wave's down projection (every GEMV expert of wave 0) and the fixed-order
// top-k sum, by output rows (launch B of a device-planned step, and the last
// launch of a one-wave host-planned step).  Workgroup b owns the RB = 2 GR rows
// [b*RB, b*RB + RB).  A wavefront's 64 / LG lane groups (LG lanes per row, as in
// gemv_down_kernel) are GR row pairs times GE = 64 / (LG GR) experts: group g
// takes rows r0 + 2 (g % GR) and + 1 of expert slot g / GR, so fewer rows per
// workgroup spread short rows over more workgroups without changing a row's
// lanes, chunk order or reduction.  The NW (1..8) wavefronts take the wave's
// GEMV experts round-robin, GE at a time; each lane group issues the weight
// loads of its first two experts (their descriptors are one load away) before
// the workgroup stages the step's h rows (if STAGE) and routed ids in LDS, and
// a later expert's as soon as a register set is free.  Every entry's w[e] * (W2
// h)[row] goes to LDS; then each token's k entries are summed in j order
// (invalid ids skipped) and rounded once to bf16: the arithmetic of down_block +
// topk_sum_rows.  Workgroup 0 makes the new LRU-state copy current, if `flip`.
template <int FMT, int MB, bool STAGE>
__global__ __launch_bounds__(512) void down_sum_kernel(ExpertArgs a, int LG, int GR, uint16_t* __restrict__ out,
                                                        int32_t* flip) {
  extern __shared__ __align__(16) char lds[];
  constexpr int VPC = Fmt<FMT>::VPC;
  const int T = a.T, k = a.k, n = T * k, H = a.H, I = a.I, n_ch = I / VPC;
  const int NW = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int groups = 64 / LG, lig = lane % LG, grp = lane / LG;
  const int GE = groups / GR, gr = grp % GR, ge = grp / GR;
  const int RB = 2 * GR, r0 = blockIdx.x * RB;
  float* s_y = reinterpret_cast<float*>(lds);                                          // [n][RB]
  int* s_id = reinterpret_cast<int*>(lds + al16(4 * (size_t)n * RB));                  // [n] routed ids
  int* s_ent = s_id + al16(4 * (size_t)n) / 4;                                         // [n] entry by sorted position
  float* s_w = reinterpret_cast<float*>(s_ent + al16(4 * (size_t)n) / 4);              // [n] router weights
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_w + al16(4 * (size_t)n) / 4);           // [n][I]
  const int32_t* hdr = a.work + a.o.hdr;
  const int4* desc = reinterpret_cast<const int4*>(a.work + a.o.gemv_desc);
  const int n_items = a.hdr_known ? a.g1 : hdr[hdr_gemv(a.MW, 1)];     // wave 0's GEMV items start at 0
  const int n0 = r0 + 2 * gr;
  const bool act0 = n0 < H, act1 = n0 + 1 < H;
  // this lane group's experts i, i + NW GE, i + 2 NW GE, ... (i = wv GE + ge):
  // the first two experts' first rounds of weight loads are issued before the
  // staging, and each later one's as soon as its buffer is free (ping-pong
  // between two named register sets)
  const int step = NW * GE;
  int i0 = wv * GE + ge, i1 = i0 + step;
  int4 d0 = i0 < a.E ? desc[i0] : make_int4(0, 0, 0, 0);
  int4 d1 = i1 < a.E ? desc[i1] : make_int4(0, 0, 0, 0);
  DownRows rA, rB;
  if (i0 < n_items) fetch_down_rows<FMT>(a, a.slots + (size_t)d0.x * a.slot_stride, n0, act0, act1, lig, LG, n_ch, rA);
  if (i1 < n_items) fetch_down_rows<FMT>(a, a.slots + (size_t)d1.x * a.slot_stride, n0, act0, act1, lig, LG, n_ch, rB);
  // the routed ids, the sorted entry order (the step's valid entries, at most
  // n; positions past them are read but never used) and the router weights
  const int32_t* ents = a.work + a.o.entries;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int id = a.ids[i], en = ents[i];
    const float w = a.topk_w[i];
    s_id[i] = id;
    s_ent[i] = en;
    s_w[i] = w;
  }
  if constexpr (STAGE) {
    const uint4* hw = reinterpret_cast<const uint4*>(a.h);
    copy_words_to_lds(reinterpret_cast<uint4*>(s_h), n * I / 8, [=](int i) { return hw + i; });
  }
  __syncthreads();
  const uint16_t* hbase = STAGE ? s_h : a.h;
  // int4 and MXFP4 dot products with eight tokens per item, or with h read
  // from global memory, leave no registers for an unrolled butterfly (it
  // spilled 0.3-0.4 KB per lane); bf16 and FP8 are faster unrolled
  constexpr bool kRollReduce = (FMT == PE_W_INT4_G128 || FMT == PE_W_MXFP4_B32) && (MB >= 8 || !STAGE);
  while (i0 < n_items) {
    down_rows_item<FMT, MB, kRollReduce>(a, d0, rA, n0, act0, act1, lig, LG, n_ch, hbase, s_y, RB, r0, s_ent, s_w);
    i0 += 2 * step;
    if (i0 < n_items) {
      d0 = desc[i0];
      fetch_down_rows<FMT>(a, a.slots + (size_t)d0.x * a.slot_stride, n0, act0, act1, lig, LG, n_ch, rA);
    }
    if (i1 >= n_items) break;
    down_rows_item<FMT, MB, kRollReduce>(a, d1, rB, n0, act0, act1, lig, LG, n_ch, hbase, s_y, RB, r0, s_ent, s_w);
    i1 += 2 * step;
    if (i1 < n_items) {
      d1 = desc[i1];
      fetch_down_rows<FMT>(a, a.slots + (size_t)d1.x * a.slot_stride, n0, act0, act1, lig, LG, n_ch, rB);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * RB; idx += blockDim.x) {
    const int t = idx / RB, r = idx - t * RB, row = r0 + r;
    if (row >= H) continue;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int e = t * k + j;
      const int id = s_id[e];
      if (id < 0 || id >= a.E) continue;
      acc += s_y[(size_t)e * RB + r];
    }
    out[(size_t)t * H + row] = f32_to_bf16(acc);
  }
  if (flip && blockIdx.x == 0 && threadIdx.x == 0) *flip ^= 1;
}

// Lanes per row: the smallest power of two (8..64) that keeps a row at most
// kMaxChunksInFlight chunks per lane, so a lane group issues a whole row in one
// round of loads and short rows give a wave several rows at once.
static int lanes_per_row(int n_ch) {
  int lg = 8;
  while (lg < 64 && n_ch > lg * kMaxChunksInFlight) lg <<= 1;
  return lg;
}

static int pick_mb(int max_m) {
  if (max_m <= 1) return 1;
  if (max_m <= 2) return 2;
  if (max_m <= 4) return 4;
  return 8;
}

static int vpc_of(int wtype) {
  return wtype == PE_W_BF16 ? Fmt<PE_W_BF16>::VPC
         : wtype == PE_W_FP8_B128 ? Fmt<PE_W_FP8_B128>::VPC
         : wtype == PE_W_INT8_G128 ? Fmt<PE_W_INT8_G128>::VPC
         : wtype == PE_W_MXFP4_B32 ? Fmt<PE_W_MXFP4_B32>::VPC
                                   : Fmt<PE_W_INT4_G128>::VPC;
}

static GemvGeom gate_up_geom(int wtype, const ExpertArgs& a) {
  GemvGeom g;
  g.LG = lanes_per_row(a.H / vpc_of(wtype));
  g.rows_per_block = (kGemvThreads / 64) * (64 / g.LG);
  g.gx = (a.I + g.rows_per_block - 1) / g.rows_per_block;
  return g;
}

static GemvGeom down_geom(int wtype, const ExpertArgs& a) {
  GemvGeom g;
  g.LG = lanes_per_row(a.I / vpc_of(wtype));
  g.rows_per_block = (kGemvThreads / 64) * (64 / g.LG) * 2;
  g.gx = (a.H + g.rows_per_block - 1) / g.rows_per_block;
  return g;
}

static size_t lean_head(const ExpertArgs& a) { return a.lean ? lean_lds_bytes(a.T * a.k) : 0; }

// gemv_stage_bytes for a format given at run time.
static size_t gemv_stage(int wtype, int mb, int C, int rows, int sides) {
  switch (wtype) {
    case PE_W_BF16: return gemv_stage_bytes<PE_W_BF16>(mb, C, rows, sides);
    case PE_W_FP8_B128: return gemv_stage_bytes<PE_W_FP8_B128>(mb, C, rows, sides);
    case PE_W_INT8_G128: return gemv_stage_bytes<PE_W_INT8_G128>(mb, C, rows, sides);
    case PE_W_MXFP4_B32: return gemv_stage_bytes<PE_W_MXFP4_B32>(mb, C, rows, sides);
    default: return gemv_stage_bytes<PE_W_INT4_G128>(mb, C, rows, sides);
  }
}

// Workgroups of kGemvThreads threads with `lds` bytes of LDS each that the
// device holds at once (per-CU occupancy times CUs), cached per kernel and LDS
// size; 0 if the runtime cannot tell.
static int resident_blocks(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kernel, lds);
  auto hit = cache.find(key);
  if (hit != cache.end()) return hit->second;
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kGemvThreads, lds) != hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    per_cu = cus = 0;
  }
  return cache[key] = per_cu * cus;
}

// Instantiate a kernel template over the weight format and token batch.
#define PE_DISPATCH(wtype, mb, CALL)                                              \
  do {                                                                            \
    if ((wtype) == PE_W_BF16) {                                                   \
      constexpr int F_ = PE_W_BF16;                                               \
      if (mb == 1) { constexpr int M_ = 1; CALL; }                                \
      else if (mb == 2) { constexpr int M_ = 2; CALL; }                           \
      else if (mb == 4) { constexpr int M_ = 4; CALL; }                           \
      else { constexpr int M_ = 8; CALL; }                                        \
    } else if ((wtype) == PE_W_FP8_B128) {                                        \
      constexpr int F_ = PE_W_FP8_B128;                                           \
      if (mb == 1) { constexpr int M_ = 1; CALL; }                                \
      else if (mb == 2) { constexpr int M_ = 2; CALL; }                           \
      else if (mb == 4) { constexpr int M_ = 4; CALL; }                           \
      else { constexpr int M_ = 8; CALL; }                                        \
    } else if ((wtype) == PE_W_INT8_G128) {                                       \
      constexpr int F_ = PE_W_INT8_G128;                                          \
      if (mb == 1) { constexpr int M_ = 1; CALL; }                                \
      else if (mb == 2) { constexpr int M_ = 2; CALL; }                           \
      else if (mb == 4) { constexpr int M_ = 4; CALL; }                           \
      else { constexpr int M_ = 8; CALL; }                                        \
    } else if ((wtype) == PE_W_MXFP4_B32) {                                       \
      constexpr int F_ = PE_W_MXFP4_B32;                                          \
      if (mb == 1) { constexpr int M_ = 1; CALL; }                                \
      else if (mb == 2) { constexpr int M_ = 2; CALL; }                           \
      else if (mb == 4) { constexpr int M_ = 4; CALL; }                           \
      else { constexpr int M_ = 8; CALL; }                                        \
    } else {                                                                      \
      constexpr int F_ = PE_W_INT4_G128;                                          \
      if (mb == 1) { constexpr int M_ = 1; CALL; }                                \
      else if (mb == 2) { constexpr int M_ = 2; CALL; }                           \
      else if (mb == 4) { constexpr int M_ = 4; CALL; }                           \
      else { constexpr int M_ = 8; CALL; }                                        \
    }                                                                             \
  } while (0)

void launch_gemv_gate_up(int wtype, const ExpertArgs& a, int items, int max_m, hipStream_t s) {
  if (items <= 0) return;
  const int mb = pick_mb(max_m);
  const GemvGeom g = gate_up_geom(wtype, a);
  const size_t lds = lean_head(a) + gemv_stage(wtype, mb, a.H, g.rows_per_block, 2) + kEntStage;
  const dim3 grid(g.gx, items);
  PE_DISPATCH(wtype, mb, (gemv_gate_up_kernel<F_, M_><<<grid, kGemvThreads, lds, s>>>(a, g)));
}

void launch_gemv_down(int wtype, const ExpertArgs& a, int items, int max_m, hipStream_t s) {
  if (items <= 0) return;
  const int mb = pick_mb(max_m);
  const GemvGeom g = down_geom(wtype, a);
  const size_t lds = lean_head(a) + gemv_stage(wtype, mb, a.I, g.rows_per_block, 1);
  const dim3 grid(g.gx, items);
  PE_DISPATCH(wtype, mb, (gemv_down_kernel<F_, M_><<<grid, kGemvThreads, lds, s>>>(a, g)));
}

void launch_step_a(int wtype, int32_t* blk, const int32_t* ids, int n, const Dims& d, const Offsets& o,
                   int mfma_min, int32_t* work, unsigned long long* stats, const uint8_t* host_rows,
                   uint8_t* slots, size_t stride, size_t copy_bytes, int P, const ExpertArgs& a, int items,
                   int max_m, hipStream_t s) {
  const PlanArgs p = plan_args(blk, ids, n, d, o, mfma_min, work, stats, host_rows, slots, stride, copy_bytes, true);
  const int mb = pick_mb(max_m);
  const GemvGeom g = gate_up_geom(wtype, a);
  const size_t copier = copier_lds_bytes(d.E, d.K, n) + al16(4 * (size_t)n) + kStreamScaleLds +
                        al16((size_t)mb * a.H * 2) + kEntStage;
  const size_t fixed = std::max(copier, plan_lds_bytes(d.E, d.K, n));
  // LDS for nr row blocks per gate/up workgroup (their scales grow with nr)
  auto lds_for = [&](int nr) {
    return std::max(fixed, lean_head(a) + gemv_stage(wtype, mb, a.H, nr * g.rows_per_block, 2) + kEntStage);
  };
  // Row blocks per gate/up workgroup: the fewest that leave every workgroup of
  // the launch resident at once (a second dispatch round would start its
  // workgroups only after the first ones end).
  auto resident_at = [&](int nr) {
    int r = 0;
    PE_DISPATCH(wtype, mb, (r = resident_blocks(reinterpret_cast<const void*>(&step_a_kernel<F_, M_>), lds_for(nr))));
    return r;
  };
  int nr = 1;
  if (resident_at(1) <= 0) {
    nr = 2;
  } else {
    while (nr < g.gx && P + 1 + ceil_div(g.gx, nr) * items > resident_at(nr)) ++nr;
  }
  const size_t lds = lds_for(nr);
  const int blocks = P + 1 + ceil_div(g.gx, nr) * items;
  PE_DISPATCH(wtype, mb, (step_a_kernel<F_, M_><<<blocks, kGemvThreads, lds, s>>>(p, P, a, g, nr)));
}

void launch_wave_a(int wtype, const ExpertArgs& a, int hit_items, int max_m, int P, const uint8_t* host_rows,
                   size_t stride, size_t copy_bytes, const void* up_src, void* up_dst, size_t up_bytes,
                   hipStream_t s) {
  const int mb = pick_mb(max_m);
  const GemvGeom g = gate_up_geom(wtype, a);
  const size_t copier = kStreamScaleLds + al16((size_t)mb * a.H * 2) + kEntStage;
  auto lds_for = [&](int nr) {
    return std::max(copier, gemv_stage(wtype, mb, a.H, nr * g.rows_per_block, 2) + kEntStage);
  };
  // Row blocks per gate/up workgroup: the fewest that leave every workgroup of
  // the launch resident at once, as in launch_step_a.
  auto resident_at = [&](int nr) {
    int r = 0;
    PE_DISPATCH(wtype, mb, (r = resident_blocks(reinterpret_cast<const void*>(&wave_a_kernel<F_, M_>), lds_for(nr))));
    return r;
  };
  const int extra = up_bytes ? 1 : 0;
  int nr = 1;
  if (hit_items > 0) {
    if (resident_at(1) <= 0) {
      nr = 2;
    } else {
      while (nr < g.gx && P + extra + ceil_div(g.gx, nr) * hit_items > resident_at(nr)) ++nr;
    }
  }
  const size_t lds = lds_for(nr);
  const int blocks = P + ceil_div(g.gx, nr) * hit_items + extra;
  PE_DISPATCH(wtype, mb, (wave_a_kernel<F_, M_><<<blocks, kGemvThreads, lds, s>>>(
                             a, g, P, nr, host_rows, stride, copy_bytes, static_cast<const uint4*>(up_src),
                             static_cast<uint4*>(up_dst), up_bytes)));
}

void launch_down_sum(int wtype, const ExpertArgs& a, int max_m, uint16_t* out, int32_t* flip, hipStream_t s) {
  const int mb = pick_mb(max_m);
  const int LG = lanes_per_row(a.I / vpc_of(wtype));
  const int groups = 64 / LG;
  // row pairs per workgroup: a power of two, at most one per lane group, and few
  // enough for a workgroup on every CU (256) when the rows allow it
  int GR = groups;
  while (GR > 1 && ceil_div(a.H, 2 * GR) < 256) GR >>= 1;
  const int RB = 2 * GR, GE = groups / GR;
  const int n = a.T * a.k;
  // wavefronts per workgroup: enough for the wave's experts GE at a time, at
  // most 8, and no more than keep every workgroup of the launch resident at
  // once (about 2048 wavefronts of this kernel's size on 256 CUs)
  const int grid_x = ceil_div(a.H, RB);
  const int items = std::min(n, a.E);
  const int nw = std::max(1, std::min(std::min(8, ceil_div(items, GE)), std::max(1, 2048 / grid_x)));
  const size_t head = al16(4 * (size_t)n * RB) + 3 * al16(4 * (size_t)n);
  const size_t staged = head + (size_t)n * a.I * 2;
  const dim3 grid(grid_x), block(64 * nw);
  if (staged <= 64 * 1024) {
    PE_DISPATCH(wtype, mb, (down_sum_kernel<F_, M_, true><<<grid, block, staged, s>>>(a, LG, GR, out, flip)));
  } else {
    PE_DISPATCH(wtype, mb, (down_sum_kernel<F_, M_, false><<<grid, block, head, s>>>(a, LG, GR, out, flip)));
  }
}

// ------------------------------------------------------------------ MFMA grouped GEMM
//
// Experts with at least kMfmaMinTokens entries in a step (prefill waves) run on
// v_mfma_f32_16x16x32_bf16.  A block computes a tile of kTileM = 128 token rows
// of one used expert against 64 weight rows, staging K in blocks of 128 through
// LDS (rows padded by 8 bf16 against bank conflicts); each wavefront takes 16 of
// the weight rows against all 128 token rows, so a weight tile staged once
// serves eight 16-row MFMA blocks.  FP8 and int4 weights are
// decoded into LDS as exact bf16 (every e4m3 value and every nibble - 8 is a
// bf16 number); their block / group scale multiplies the fp32 partial product
// of each 128-wide K block.  MXFP4 codes are decoded with their 32-column E8M0
// scale applied (an E2M1 value times a power of two: exact in bf16 within
// bf16's range), so its K blocks take no scale, and bf16 and MXFP4 MFMAs
// accumulate straight into the output accumulators.  Every output element's
// arithmetic depends only on its own token row and weight row, never on the
// other rows of the tile.

namespace {
constexpr int kMfmaThreads = 256;
constexpr int kNT = 64;          // weight rows per block (16 per wavefront)
constexpr int kKB = 128;         // K per LDS stage = one FP8 block / int4 group
constexpr int kLdsRow = kKB + 8; // padded LDS row, bf16 elements
constexpr int kMH = kTileM / 16; // 16-row MFMA blocks per tile (every wavefront covers all of them)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
}  // namespace

// Entry index and router weight of each row of a down tile, staged in LDS
// (`s_ent`, `s_w`: kTileM words each, over the last K block's operands) for
// the epilogue, which would otherwise load both, one after the other, for
// every output element it stores.
__device__ __forceinline__ void stage_tile_entries(const ExpertArgs& a, const int32_t* __restrict__ ent, int rows,
                                                   int* s_ent, float* s_w) {
  __syncthreads();     // every wavefront is done with the operands in this LDS area
  if ((int)threadIdx.x < kTileM) {
    const int r = threadIdx.x;
    const int e = r < rows ? ent[r] : 0;
    s_ent[r] = e;
    s_w[r] = r < rows ? a.topk_w[e] : 0.f;
  }
  __syncthreads();
}

// The (tile, column block) item of this workgroup.  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2) in linear block order; the
// items are given out so that every XCD takes a contiguous run of them, tile by
// tile, so the column blocks of one token tile (which share its rows of x or h)
// and the tiles of one expert (which share its weights) meet in one L2.  Only
// the order changes: every item is computed the same way wherever it runs.
__device__ __forceinline__ void mfma_item(int& tile_idx, int& nblk) {
  constexpr int kXcds = 8;
  const int nb = gridDim.x, total = gridDim.x * gridDim.y;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int xcd = b % kXcds, k = b / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  const int q = xcd * per + min(xcd, rem) + k;
  tile_idx = q / nb;
  nblk = q - tile_idx * nb;
}

// The descriptor of the wave's tile_idx-th MFMA tile of this launch's part
// (all, resident before the wave's page-in, or paged in by it): {slot, first
// sorted position, rows, expert id}.  False past the part's last tile.
__device__ __forceinline__ bool mfma_tile(const ExpertArgs& a, int tile_idx, int4& td) {
  int t0, t1;
  if (a.hdr_known) {
    part_range(a, a.t0, a.tsplit, a.t1, t0, t1);
  } else {
    const int32_t* hdr = a.work + a.o.hdr;
    part_range(a, hdr[hdr_tile(a.MW, a.wave)], hdr[hdr_tile_split(a.MW, a.wave)], hdr[hdr_tile(a.MW, a.wave + 1)], t0,
               t1);
  }
  const int tile = t0 + tile_idx;
  if (tile >= t1) return false;
  td = reinterpret_cast<const int4*>(a.work + a.o.tile_desc)[tile];
  return true;
}

// Decode one 16-byte chunk of weights of format FMT into bf16 in LDS at `dst`
// (VPC values); returns nothing, writes VPC/8 16-byte LDS words.  `sc` (MXFP4
// only) is the chunk's block scale, applied here.
template <int FMT>
__device__ __forceinline__ void decode_chunk_to_lds(uint4 w, uint16_t* dst, float sc) {
  if constexpr (FMT == PE_W_BF16) {
    *reinterpret_cast<uint4*>(dst) = w;
  } else if constexpr (FMT == PE_W_FP8_B128) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[p], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[p], true);
      // e4m3 values have at most 4 significant bits: the top half of the fp32 is exact
      o[2 * p] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
      o[2 * p + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
    }
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else if constexpr (FMT == PE_W_INT8_G128) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // q - 128 is an integer of at most 8 bits: the top half of its fp32 is exact
      const float v0 = (float)(wd[p] & 0xFFu) - 128.0f, v1 = (float)((wd[p] >> 8) & 0xFFu) - 128.0f;
      const float v2 = (float)((wd[p] >> 16) & 0xFFu) - 128.0f, v3 = (float)(wd[p] >> 24) - 128.0f;
      o[2 * p] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
      o[2 * p + 1] = (__float_as_uint(v2) >> 16) | (__float_as_uint(v3) & 0xFFFF0000u);
    }
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else if constexpr (FMT == PE_W_MXFP4_B32) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[16];
    // e2m1 * 2^k has at most two significant bits: the top half of the fp32 is exact
    auto top = [sc](auto v) { return (__float_as_uint(v[0] * sc) >> 16) | (__float_as_uint(v[1] * sc) & 0xFFFF0000u); };
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      o[4 * p] = top(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[p], 1.0f, 0));
      o[4 * p + 1] = top(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[p], 1.0f, 1));
      o[4 * p + 2] = top(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[p], 1.0f, 2));
      o[4 * p + 3] = top(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[p], 1.0f, 3));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<uint4*>(dst)[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  } else {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wd[p] >> (8 * b)) & 0xFFu;
        const float lo = (float)(int)(byte & 0xFu) - 8.0f, hi = (float)(int)(byte >> 4) - 8.0f;
        o[4 * p + b] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<uint4*>(dst)[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
}

// One K block's staging per thread: kAPer 16-byte chunks of token rows and
// kWPer<FMT> chunks of each weight matrix.  All of a thread's loads of a block
// are issued before any of them is stored to LDS, so they are in flight
// together.
constexpr int kAPer = kTileM * (kKB / 8) / kMfmaThreads;
// FP8, int4 and int8 multiply each 128-wide K block's partial product by its scale.
template <int FMT> constexpr bool kBlockScaled = FMT == PE_W_FP8_B128 || kGroupScales<FMT>;
template <int FMT> constexpr int kWPer = kNT * (kKB / Fmt<FMT>::VPC) / kMfmaThreads;

// Loads of kNT weight rows [row0, row0 + kNT) x K block kb of a row-major matrix
// with C columns (and, for MXFP4, each chunk's scale from the row-scale region S).
template <int FMT>
__device__ __forceinline__ void load_weights(uint4 (&v)[kWPer<FMT>], float (&sc)[kWPer<FMT>],
                                             const uint8_t* __restrict__ W, const uint8_t* __restrict__ S,
                                             int C, int row0, int kb) {
  constexpr int VPC = Fmt<FMT>::VPC;
  constexpr int CPR = kKB / VPC;                       // chunks per row per stage
  const size_t row_chunks = (size_t)(C / VPC);         // 16 bytes per VPC columns
  const uint4* base = reinterpret_cast<const uint4*>(W);
#pragma unroll
  for (int q = 0; q < kWPer<FMT>; ++q) {
    const int i = threadIdx.x + q * kMfmaThreads;
    const int r = i / CPR, c = i - r * CPR;
    v[q] = base[(size_t)(row0 + r) * row_chunks + (size_t)kb * CPR + c];
    sc[q] = 1.0f;
    if constexpr (FMT == PE_W_MXFP4_B32)
      sc[q] = chunk_scale<FMT>(nullptr, S + row_scale_off<FMT>(row0 + r, C), (kb * CPR + c) * VPC);
  }
}

// Decode the loaded chunks into LDS rows (bf16, padded).
template <int FMT>
__device__ __forceinline__ void store_weights(const uint4 (&v)[kWPer<FMT>], const float (&sc)[kWPer<FMT>],
                                              uint16_t* sB) {
  constexpr int VPC = Fmt<FMT>::VPC;
  constexpr int CPR = kKB / VPC;
#pragma unroll
  for (int q = 0; q < kWPer<FMT>; ++q) {
    const int i = threadIdx.x + q * kMfmaThreads;
    const int r = i / CPR, c = i - r * CPR;
    decode_chunk_to_lds<FMT>(v[q], sB + r * kLdsRow + c * VPC, sc[q]);
  }
}

// Gate/up + SwiGLU on MFMA: one token tile of the wave x 64 intermediate rows
// (the item mfma_item gives this workgroup).
template <int FMT>
__global__ __launch_bounds__(kMfmaThreads) void mfma_gate_up_kernel(ExpertArgs a) {
  __shared__ __align__(16) uint16_t sA[kTileM * kLdsRow];
  __shared__ __align__(16) uint16_t sG[kNT * kLdsRow];
  __shared__ __align__(16) uint16_t sU[kNT * kLdsRow];
  __shared__ int sTok[kTileM];
  int tile_idx, nblk;
  mfma_item(tile_idx, nblk);
  int4 td;
  if (!mfma_tile(a, tile_idx, td)) return;
  const int slot = td.x, pos = td.y, rows = td.z;     // the tile's sorted positions pos .. pos + rows - 1
  const int H = a.H, I = a.I;
  const int n0 = nblk * kNT;
  const uint8_t* blob = a.slots + (size_t)slot * a.slot_stride;
  const uint8_t* W13 = blob + a.off_w13;
  const float* S13f = reinterpret_cast<const float*>(blob + a.off_s13);
  const uint16_t* S13h = reinterpret_cast<const uint16_t*>(blob + a.off_s13);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lk = lane >> 4;
  if (threadIdx.x < kTileM)
    sTok[threadIdx.x] = threadIdx.x < rows ? a.work[a.o.entries + pos + threadIdx.x] / a.k : -1;
  f32x4_t accg[kMH], accu[kMH];
#pragma unroll
  for (int h = 0; h < kMH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) { accg[h][i] = 0.f; accu[h][i] = 0.f; }
  const int ncol = n0 + 16 * wv + ln;     // this lane's output column (intermediate row)
  // Formats without a per-block scale accumulate straight into accg / accu, and
  // with the registers that saves they load K block kb + 1 while block kb's
  // MFMAs run; the scaled formats keep a per-block partial and load each block
  // at its start.
  constexpr bool kPipe = !kBlockScaled<FMT>;
  uint4 va[kAPer], vg[kWPer<FMT>], vu[kWPer<FMT>];
  float sg_[kWPer<FMT>], su_[kWPer<FMT>];
  __syncthreads();     // sTok
  auto load_block = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB / 8), c = i - r * (kKB / 8);
      const int tok = sTok[r];
      va[q] = tok >= 0 ? reinterpret_cast<const uint4*>(a.x + (size_t)tok * H + kb * kKB)[c] : make_uint4(0, 0, 0, 0);
    }
    load_weights<FMT>(vg, sg_, W13, blob + a.off_s13, H, n0, kb);
    load_weights<FMT>(vu, su_, W13, blob + a.off_s13, H, I + n0, kb);
  };
  const int nK = H / kKB;
  if constexpr (kPipe) load_block(0);
  for (int kb = 0; kb < nK; ++kb) {
    __syncthreads();
    if constexpr (!kPipe) load_block(kb);
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB / 8), c = i - r * (kKB / 8);
      *reinterpret_cast<uint4*>(sA + r * kLdsRow + c * 8) = va[q];
    }
    store_weights<FMT>(vg, sg_, sG);
    store_weights<FMT>(vu, su_, sU);
    __syncthreads();
    if constexpr (kPipe) {
      if (kb + 1 < nK) load_block(kb + 1);
#pragma unroll
      for (int ks = 0; ks < kKB / 32; ++ks) {
        const int kc = ks * 32 + 8 * lk;
        const bf16x8_t bg = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sG + (16 * wv + ln) * kLdsRow + kc));
        const bf16x8_t bu = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sU + (16 * wv + ln) * kLdsRow + kc));
#pragma unroll
        for (int h = 0; h < kMH; ++h) {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (16 * h + ln) * kLdsRow + kc));
          accg[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bg, accg[h], 0, 0, 0);
          accu[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bu, accu[h], 0, 0, 0);
        }
      }
      continue;
    }
    f32x4_t pg[kMH], pu[kMH];
#pragma unroll
    for (int h = 0; h < kMH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) { pg[h][i] = 0.f; pu[h][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < kKB / 32; ++ks) {
      const int kc = ks * 32 + 8 * lk;
      const bf16x8_t bg = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sG + (16 * wv + ln) * kLdsRow + kc));
      const bf16x8_t bu = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sU + (16 * wv + ln) * kLdsRow + kc));
#pragma unroll
      for (int h = 0; h < kMH; ++h) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (16 * h + ln) * kLdsRow + kc));
        pg[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bg, pg[h], 0, 0, 0);
        pu[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bu, pu[h], 0, 0, 0);
      }
    }
    float sg = 1.f, su = 1.f;
    if constexpr (FMT == PE_W_FP8_B128) {
      sg = S13f[(size_t)(n0 >> 7) * (H / 128) + kb];
      su = S13f[(size_t)((I + n0) >> 7) * (H / 128) + kb];
    } else if constexpr (kGroupScales<FMT>) {
      sg = half_bits_to_f32(S13h[(size_t)ncol * (H / 128) + kb]);
      su = half_bits_to_f32(S13h[(size_t)(I + ncol) * (H / 128) + kb]);
    }
#pragma unroll
    for (int h = 0; h < kMH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[h][i] = __builtin_fmaf(sg, pg[h][i], accg[h][i]);
        accu[h][i] = __builtin_fmaf(su, pu[h][i], accu[h][i]);
      }
  }
#pragma unroll
  for (int h = 0; h < kMH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * h + 4 * lk + i;
      if (r < rows)
        a.h[(size_t)(pos + r) * I + ncol] = f32_to_bf16(silu_f(accg[h][i]) * accu[h][i]);
    }
}

// Down projection x router weight on MFMA: one token tile x 64 output columns
// (the item mfma_item gives this workgroup).
template <int FMT>
__global__ __launch_bounds__(kMfmaThreads) void mfma_down_kernel(ExpertArgs a) {
  __shared__ __align__(16) uint16_t sA[kTileM * kLdsRow];
  __shared__ __align__(16) uint16_t sB[kNT * kLdsRow];
  int tile_idx, nblk;
  mfma_item(tile_idx, nblk);
  int4 td;
  if (!mfma_tile(a, tile_idx, td)) return;
  const int slot = td.x, pos = td.y, rows = td.z;     // the tile's sorted positions pos .. pos + rows - 1
  const int H = a.H, I = a.I;
  const int n0 = nblk * kNT;
  const uint8_t* blob = a.slots + (size_t)slot * a.slot_stride;
  const uint8_t* W2 = blob + a.off_w2;
  const float* S2f = reinterpret_cast<const float*>(blob + a.off_s2);
  const uint16_t* S2h = reinterpret_cast<const uint16_t*>(blob + a.off_s2);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lk = lane >> 4;
  f32x4_t acc[kMH];
#pragma unroll
  for (int h = 0; h < kMH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;
  const int ncol = n0 + 16 * wv + ln;
  // K block kb + 1 is loaded while block kb's MFMAs run; formats without a
  // per-block scale accumulate straight into acc.
  uint4 va[kAPer], vb[kWPer<FMT>];
  float sb_[kWPer<FMT>];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB / 8), c = i - r * (kKB / 8);
      va[q] = r < rows ? reinterpret_cast<const uint4*>(a.h + (size_t)(pos + r) * I + kb * kKB)[c]
                       : make_uint4(0, 0, 0, 0);
    }
    load_weights<FMT>(vb, sb_, W2, blob + a.off_s2, I, n0, kb);
  };
  const int nK = I / kKB;
  load_block(0);
  for (int kb = 0; kb < nK; ++kb) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB / 8), c = i - r * (kKB / 8);
      *reinterpret_cast<uint4*>(sA + r * kLdsRow + c * 8) = va[q];
    }
    store_weights<FMT>(vb, sb_, sB);
    __syncthreads();
    if (kb + 1 < nK) load_block(kb + 1);
    if constexpr (!kBlockScaled<FMT>) {
#pragma unroll
      for (int ks = 0; ks < kKB / 32; ++ks) {
        const int kc = ks * 32 + 8 * lk;
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sB + (16 * wv + ln) * kLdsRow + kc));
#pragma unroll
        for (int h = 0; h < kMH; ++h) {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (16 * h + ln) * kLdsRow + kc));
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[h], 0, 0, 0);
        }
      }
      continue;
    }
    f32x4_t p[kMH];
#pragma unroll
    for (int h = 0; h < kMH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[h][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKB / 32; ++ks) {
      const int kc = ks * 32 + 8 * lk;
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sB + (16 * wv + ln) * kLdsRow + kc));
#pragma unroll
      for (int h = 0; h < kMH; ++h) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (16 * h + ln) * kLdsRow + kc));
        p[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, p[h], 0, 0, 0);
      }
    }
    float sc = 1.f;
    if constexpr (FMT == PE_W_FP8_B128) sc = S2f[(size_t)(n0 >> 7) * (I / 128) + kb];
    else if constexpr (kGroupScales<FMT>) sc = half_bits_to_f32(S2h[(size_t)ncol * (I / 128) + kb]);
#pragma unroll
    for (int h = 0; h < kMH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] = __builtin_fmaf(sc, p[h][i], acc[h][i]);
  }
  int* s_ent = reinterpret_cast<int*>(sA);
  float* s_w = reinterpret_cast<float*>(sA) + kTileM;
  stage_tile_entries(a, a.work + a.o.entries + pos, rows, s_ent, s_w);
#pragma unroll
  for (int h = 0; h < kMH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * h + 4 * lk + i;
      if (r < rows) a.merged[(size_t)s_ent[r] * H + ncol] = s_w[r] * acc[h][i];
    }
}

// ---- 32x32 MFMA kernels for the formats without per-block scales (bf16, MXFP4)
//
// v_mfma_f32_32x32x16_bf16 does twice the multiply-adds of the 16x16x32 form
// for the same two 16-byte operand reads per lane, and every wavefront here
// covers all 128 token rows of the tile against 32 (gate/up: 32 gate and the
// matching 32 up rows) or 64 (down) weight rows, so each staged K block feeds
// 8 MFMAs per 6 LDS operand reads.  K is staged 64 wide (rows padded to 72
// bf16: conflict-free 16-byte reads), so any H and I that are multiples of 64
// take these kernels (gpt-oss-20b's 2880 included); weight rows past the
// matrix are zero-filled and their outputs dropped.  Operand layout of the
// 32x32x16 form: lane l holds A[m = l % 32][k = 8 (l / 32) .. +8] and
// B[k = 8 (l / 32) .. +8][n = l % 32]; result register i of lane l is
// D[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32].  The next K block is loaded
// into registers while the current one's MFMAs run.
namespace {
constexpr int kKB2 = 64;
constexpr int kRow2 = kKB2 + 8;
constexpr int kNG2 = 128;        // gate/up: intermediate rows per block (32 per wavefront)
constexpr int kND2 = 256;        // down: output rows per block (64 per wavefront)
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
template <int FMT> constexpr int kCpr2 = kKB2 / Fmt<FMT>::VPC;    // 16-byte chunks per row per K block
}  // namespace

template <int FMT>
constexpr bool kMfma32 = FMT == PE_W_BF16 || FMT == PE_W_MXFP4_B32;

// Chunks q of one K block of weight rows [row0, row0 + NR) (rows >= nrows
// zero): thread-strided, chunk i = threadIdx.x + q * 256 is row i / CPR,
// chunk i % CPR.  MXFP4 takes each chunk's E8M0 scale too.
template <int FMT, int NR>
__device__ __forceinline__ void load_w2(uint4 (&v)[NR * kCpr2<FMT> / kMfmaThreads], float (&sc)[NR * kCpr2<FMT> / kMfmaThreads],
                                        const uint8_t* __restrict__ W, const uint8_t* __restrict__ S, int C,
                                        int row0, int nrows, int kb) {
  constexpr int VPC = Fmt<FMT>::VPC, CPR = kCpr2<FMT>, NQ = NR * CPR / kMfmaThreads;
  const size_t row_chunks = (size_t)(C / VPC);
  const uint4* base = reinterpret_cast<const uint4*>(W);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int i = threadIdx.x + q * kMfmaThreads;
    const int r = i / CPR, c = i - r * CPR;
    const bool ok = row0 + r < nrows;
    v[q] = ok ? base[(size_t)(row0 + r) * row_chunks + (size_t)kb * CPR + c] : make_uint4(0, 0, 0, 0);
    sc[q] = 1.0f;
    if constexpr (FMT == PE_W_MXFP4_B32)
      if (ok) sc[q] = chunk_scale<FMT>(nullptr, S + row_scale_off<FMT>(row0 + r, C), (kb * CPR + c) * VPC);
  }
}

template <int FMT, int NR>
__device__ __forceinline__ void store_w2(const uint4 (&v)[NR * kCpr2<FMT> / kMfmaThreads],
                                         const float (&sc)[NR * kCpr2<FMT> / kMfmaThreads], uint16_t* sB) {
  constexpr int VPC = Fmt<FMT>::VPC, CPR = kCpr2<FMT>, NQ = NR * CPR / kMfmaThreads;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int i = threadIdx.x + q * kMfmaThreads;
    const int r = i / CPR, c = i - r * CPR;
    decode_chunk_to_lds<FMT>(v[q], sB + r * kRow2 + c * VPC, sc[q]);
  }
}

// Gate/up + SwiGLU: one token tile x 128 intermediate rows (the item mfma_item
// gives this workgroup); wavefront wv takes rows n0 + 32 wv .. + 32.
template <int FMT>
__global__ __launch_bounds__(kMfmaThreads, 2) void mfma32_gate_up_kernel(ExpertArgs a) {
  __shared__ __align__(16) uint16_t sA[kTileM * kRow2];
  __shared__ __align__(16) uint16_t sG[kNG2 * kRow2];
  __shared__ __align__(16) uint16_t sU[kNG2 * kRow2];
  __shared__ int sTok[kTileM];
  constexpr int NQ = kNG2 * kCpr2<FMT> / kMfmaThreads;
  constexpr int AQ = kTileM * (kKB2 / 8) / kMfmaThreads;
  int tile_idx, nblk;
  mfma_item(tile_idx, nblk);
  int4 td;
  if (!mfma_tile(a, tile_idx, td)) return;
  const int slot = td.x, pos = td.y, rows = td.z;     // the tile's sorted positions pos .. pos + rows - 1
  const int H = a.H, I = a.I;
  const int n0 = nblk * kNG2;
  const uint8_t* blob = a.slots + (size_t)slot * a.slot_stride;
  const uint8_t* W13 = blob + a.off_w13;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  if (threadIdx.x < kTileM)
    sTok[threadIdx.x] = (int)threadIdx.x < rows ? a.work[a.o.entries + pos + threadIdx.x] / a.k : -1;
  f32x16_t accg[4], accu[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) { accg[mb][i] = 0.f; accu[mb][i] = 0.f; }
  uint4 va[AQ], vg[NQ], vu[NQ];
  float sg_[NQ], su_[NQ];
  __syncthreads();     // sTok
  auto load_block = [&](int kb) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB2 / 8), c = i - r * (kKB2 / 8);
      const int tok = sTok[r];
      va[q] = tok >= 0 ? reinterpret_cast<const uint4*>(a.x + (size_t)tok * H + kb * kKB2)[c] : make_uint4(0, 0, 0, 0);
    }
    // gate rows [n0, n0 + 128) of the first I rows, up rows I + [n0, n0 + 128)
    load_w2<FMT, kNG2>(vg, sg_, W13, blob + a.off_s13, H, n0, I, kb);
    load_w2<FMT, kNG2>(vu, su_, W13 + (size_t)I * (H / Fmt<FMT>::VPC) * 16, blob + a.off_s13 + row_scale_off<FMT>(I, H),
                       H, n0, I, kb);
  };
  const int nK = H / kKB2;
  load_block(0);
  for (int kb = 0; kb < nK; ++kb) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB2 / 8), c = i - r * (kKB2 / 8);
      *reinterpret_cast<uint4*>(sA + r * kRow2 + c * 8) = va[q];
    }
    store_w2<FMT, kNG2>(vg, sg_, sG);
    store_w2<FMT, kNG2>(vu, su_, sU);
    __syncthreads();
    if (kb + 1 < nK) load_block(kb + 1);
#pragma unroll
    for (int ks = 0; ks < kKB2 / 16; ++ks) {
      const int kc = ks * 16 + 8 * lh;
      const bf16x8_t bg = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sG + (32 * wv + l32) * kRow2 + kc));
      const bf16x8_t bu = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sU + (32 * wv + l32) * kRow2 + kc));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (32 * mb + l32) * kRow2 + kc));
        accg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bg, accg[mb], 0, 0, 0);
        accu[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bu, accu[mb], 0, 0, 0);
      }
    }
  }
  const int ncol = n0 + 32 * wv + l32;     // this lane's intermediate row
  if (ncol >= I) return;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * mb + 8 * (i / 4) + 4 * lh + (i % 4);
      if (r < rows) a.h[(size_t)(pos + r) * I + ncol] = f32_to_bf16(silu_f(accg[mb][i]) * accu[mb][i]);
    }
}

// Down projection x router weight: one token tile x 256 output rows; wavefront
// wv takes rows n0 + 64 wv .. + 64 (two 32-row MFMA blocks).
template <int FMT>
__global__ __launch_bounds__(kMfmaThreads, 2) void mfma32_down_kernel(ExpertArgs a) {
  __shared__ __align__(16) uint16_t sA[kTileM * kRow2];
  __shared__ __align__(16) uint16_t sB[kND2 * kRow2];
  constexpr int NQ = kND2 * kCpr2<FMT> / kMfmaThreads;
  constexpr int AQ = kTileM * (kKB2 / 8) / kMfmaThreads;
  int tile_idx, nblk;
  mfma_item(tile_idx, nblk);
  int4 td;
  if (!mfma_tile(a, tile_idx, td)) return;
  const int slot = td.x, pos = td.y, rows = td.z;     // the tile's sorted positions pos .. pos + rows - 1
  const int H = a.H, I = a.I;
  const int n0 = nblk * kND2;
  const uint8_t* blob = a.slots + (size_t)slot * a.slot_stride;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  f32x16_t acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  uint4 va[AQ], vb[NQ];
  float sb_[NQ];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB2 / 8), c = i - r * (kKB2 / 8);
      va[q] = r < rows ? reinterpret_cast<const uint4*>(a.h + (size_t)(pos + r) * I + kb * kKB2)[c]
                       : make_uint4(0, 0, 0, 0);
    }
    load_w2<FMT, kND2>(vb, sb_, blob + a.off_w2, blob + a.off_s2, I, n0, H, kb);
  };
  const int nK = I / kKB2;
  load_block(0);
  for (int kb = 0; kb < nK; ++kb) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int i = threadIdx.x + q * kMfmaThreads;
      const int r = i / (kKB2 / 8), c = i - r * (kKB2 / 8);
      *reinterpret_cast<uint4*>(sA + r * kRow2 + c * 8) = va[q];
    }
    store_w2<FMT, kND2>(vb, sb_, sB);
    __syncthreads();
    if (kb + 1 < nK) load_block(kb + 1);
#pragma unroll
    for (int ks = 0; ks < kKB2 / 16; ++ks) {
      const int kc = ks * 16 + 8 * lh;
      bf16x8_t bv[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bv[nb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sB + (64 * wv + 32 * nb + l32) * kRow2 + kc));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + (32 * mb + l32) * kRow2 + kc));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }
  int* s_ent = reinterpret_cast<int*>(sA);
  float* s_w = reinterpret_cast<float*>(sA) + kTileM;
  stage_tile_entries(a, a.work + a.o.entries + pos, rows, s_ent, s_w);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * mb + 8 * (i / 4) + 4 * lh + (i % 4);
      if (r >= rows) continue;
      float* dst = a.merged + (size_t)s_ent[r] * H;
      const float wr = s_w[r];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int ncol = n0 + 64 * wv + 32 * nb + l32;
        if (ncol < H) dst[ncol] = wr * acc[mb][nb][i];
      }
    }
}

void launch_mfma_gate_up(int wtype, const ExpertArgs& a, int tiles, hipStream_t s) {
  if (tiles <= 0) return;
  if (wtype == PE_W_BF16 || wtype == PE_W_MXFP4_B32) {
    const dim3 grid(ceil_div(a.I, kNG2), tiles);
    if (wtype == PE_W_BF16) mfma32_gate_up_kernel<PE_W_BF16><<<grid, kMfmaThreads, 0, s>>>(a);
    else mfma32_gate_up_kernel<PE_W_MXFP4_B32><<<grid, kMfmaThreads, 0, s>>>(a);
    return;
  }
  dim3 grid(a.I / kNT, tiles);
  if (wtype == PE_W_FP8_B128) mfma_gate_up_kernel<PE_W_FP8_B128><<<grid, kMfmaThreads, 0, s>>>(a);
  else if (wtype == PE_W_INT8_G128) mfma_gate_up_kernel<PE_W_INT8_G128><<<grid, kMfmaThreads, 0, s>>>(a);
  else mfma_gate_up_kernel<PE_W_INT4_G128><<<grid, kMfmaThreads, 0, s>>>(a);
}

void launch_mfma_down(int wtype, const ExpertArgs& a, int tiles, hipStream_t s) {
  if (tiles <= 0) return;
  if (wtype == PE_W_BF16 || wtype == PE_W_MXFP4_B32) {
    const dim3 grid(ceil_div(a.H, kND2), tiles);
    if (wtype == PE_W_BF16) mfma32_down_kernel<PE_W_BF16><<<grid, kMfmaThreads, 0, s>>>(a);
    else mfma32_down_kernel<PE_W_MXFP4_B32><<<grid, kMfmaThreads, 0, s>>>(a);
    return;
  }
  dim3 grid(a.H / kNT, tiles);
  if (wtype == PE_W_FP8_B128) mfma_down_kernel<PE_W_FP8_B128><<<grid, kMfmaThreads, 0, s>>>(a);
  else if (wtype == PE_W_INT8_G128) mfma_down_kernel<PE_W_INT8_G128><<<grid, kMfmaThreads, 0, s>>>(a);
  else mfma_down_kernel<PE_W_INT4_G128><<<grid, kMfmaThreads, 0, s>>>(a);
}

int mfma_multiple(int wtype) { return wtype == PE_W_BF16 || wtype == PE_W_MXFP4_B32 ? kKB2 : kKB; }

// ------------------------------------------------------------------ top-k sum

// `flip` (device-planned steps): the layer's current-state index, flipped to the
// copy the planning kernel wrote; nothing reads it while this kernel runs.
__global__ __launch_bounds__(256) void topk_sum_kernel(const float* __restrict__ merged,
                                                       const int32_t* __restrict__ ids, int T, int k,
                                                       int E, int H, uint16_t* __restrict__ out, int32_t* flip) {
  topk_sum_rows(merged, ids, T, k, E, H, out, (size_t)blockIdx.x * blockDim.x + threadIdx.x,
                (size_t)gridDim.x * blockDim.x);
  if (flip && blockIdx.x == 0 && threadIdx.x == 0) *flip ^= 1;
}

void launch_topk_sum(const float* merged, const int32_t* ids, int T, int k, int E, int H,
                     uint16_t* out, int32_t* flip, hipStream_t s) {
  const size_t n = (size_t)T * (H / 4);
  const int grid = (int)((n + 255) / 256);
  topk_sum_kernel<<<grid, 256, 0, s>>>(merged, ids, T, k, E, H, out, flip);
}

// ------------------------------------------------------------------ LRU reset

__global__ void reset_lru_kernel(int32_t* blocks, size_t layer_words, int l0, Offsets o, int E, int K,
                                 int identity) {
  int32_t* blk = blocks + (size_t)(l0 + blockIdx.x) * layer_words;
  for (int c = 0; c < 2; ++c) {
    int32_t* st = blk + o.state0 + c * o.state_stride;
    for (int e = threadIdx.x; e < E; e += blockDim.x) st[o.expert_slot + e] = identity ? e : -1;
    for (int j = threadIdx.x; j < K; j += blockDim.x) {
      st[o.slot_expert + j] = identity ? j : -1;
      st[o.last_use + j] = 0;
    }
    if (threadIdx.x == 0) st[o.tick] = 1;
  }
  if (threadIdx.x == 0) { blk[o.cur] = 0; blk[o.n_waves] = 0; }
}

void launch_reset_lru(int32_t* blocks, size_t layer_words, int l0, int l1, const Offsets& o,
                      int E, int K, bool identity, hipStream_t s) {
  if (l1 <= l0) return;
  reset_lru_kernel<<<l1 - l0, 256, 0, s>>>(blocks, layer_words, l0, o, E, K, identity ? 1 : 0);
}

// ------------------------------------------------------------------ host-planned step: read-back

// Every thread makes its own stores visible to the host (system-scope fence)
// before the barrier, so once thread 0 has published `seq` the host can read
// everything the workgroup wrote.
__global__ __launch_bounds__(256) void gather_state_kernel(const int32_t* __restrict__ blk, int state_words,
                                                           const int32_t* __restrict__ ids, int n,
                                                           int32_t* __restrict__ host_blk,
                                                           int32_t* __restrict__ host_ids, uint32_t* flag,
                                                           uint32_t seq) {
  for (int i = threadIdx.x; i < state_words; i += blockDim.x) host_blk[i] = blk[i];
  for (int i = threadIdx.x; i < n; i += blockDim.x) host_ids[i] = ids[i];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

void launch_gather_state(const int32_t* blk, int state_words, const int32_t* ids, int n, int32_t* host_blk,
                         int32_t* host_ids, uint32_t* flag, uint32_t seq, hipStream_t s) {
  gather_state_kernel<<<1, 256, 0, s>>>(blk, state_words, ids, n, host_blk, host_ids, flag, seq);
}

// ------------------------------------------------------------------ plan log

// One workgroup: the record of the step that just ended goes to ring slot
// seq % cap.  Runs after every kernel of the step, so the block's current
// state copy is the state after the step.
__global__ __launch_bounds__(256) void plan_log_kernel(const int32_t* __restrict__ blk, Offsets o, int K,
                                                       int plan0, int plan_words, int T,
                                                       int32_t* __restrict__ ring, int cap, int rec_words,
                                                       uint32_t* __restrict__ seq) {
  const uint32_t q = *seq;
  int32_t* rec = ring + (size_t)(q % (uint32_t)cap) * rec_words;
  const int32_t* st = blk + o.state0 + (blk[o.cur] & 1) * o.state_stride;
  const int p_se = 4 + plan_words, p_lu = p_se + K;
  if (threadIdx.x == 0) {
    rec[0] = (int32_t)q;
    rec[1] = T;
    rec[2] = st[o.tick];
    rec[3] = 0;
  }
  for (int i = threadIdx.x; i < plan_words; i += blockDim.x) rec[4 + i] = blk[plan0 + i];
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    rec[p_se + j] = st[o.slot_expert + j];
    rec[p_lu + j] = st[o.last_use + j];
  }
  for (int i = p_lu + K + threadIdx.x; i < rec_words; i += blockDim.x) rec[i] = 0;
  __syncthreads();     // every thread has read *seq
  if (threadIdx.x == 0) *seq = q + 1;
}

void launch_plan_log(const int32_t* blk, const Offsets& o, int K, int plan0, int plan_words, int T,
                     int32_t* ring, int cap, int rec_words, uint32_t* seq, hipStream_t s) {
  plan_log_kernel<<<1, 256, 0, s>>>(blk, o, K, plan0, plan_words, T, ring, cap, rec_words, seq);
}

// ------------------------------------------------------------------ fixed scratch area

// The activations of pe_forward_static (h, then the merged buffer) live here
// instead of in the context's allocations.  Each device the library runs on
// holds its own copy until the process ends.  Host code never passes this name
// to a kernel: in host code it is only a stand-in for the symbol, and the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

void* static_scratch(int device) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(device);
  if (it != addr.end()) return it->second;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != device) {
    (void)hipGetLastError();
    return nullptr;      // the caller makes `device` current first
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  addr[device] = ptr;
  return ptr;
}

}  // namespace pe
