// Memory layout shared by the host orchestration, the host wave planner and
// the HIP kernels of libpe.  Plain C++ (no HIP types) so the host planner can
// be built and tested without a GPU toolchain.
#pragma once
#include <cstddef>
#include <cstdint>

namespace pe {

constexpr int kMaxExperts = 1024;
// In a step of at least this many tokens, an expert whose entries number at
// least this many runs on the MFMA grouped-GEMM kernels, otherwise on the GEMV
// kernels.  The choice depends only on the step's token count and the expert's
// entry count, which no wave split and no K changes, so a paged step and an
// unpaged step run every expert through the same arithmetic.
constexpr int kMfmaMinTokens = 16;
constexpr int kNoMfma = 1 << 30;   // threshold that sends every expert to the GEMV kernels
constexpr int kTileM = 128;  // token rows per MFMA tile

// Device statistic counters (uint64 each).
enum StatIdx {
  ST_STEPS = 0, ST_DEVICE_PLANNED, ST_HOST_PLANNED, ST_WAVES, ST_PAGE_INS,
  ST_DISTINCT, ST_ENTRIES, ST_BAD_IDS, ST_COUNT
};

struct Dims {
  int L, E, K, k, H, I;
  int max_tokens;
  int max_entries;   // max_tokens * k
  int max_waves;     // ceil(min(max_entries, E) / K)
  int max_tiles;     // MFMA tiles one step can need
  int mfma_min;      // experts with at least this many entries take the MFMA kernels
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

inline Dims make_dims(int L, int E, int K, int k, int H, int I, int max_tokens) {
  Dims d{L, E, K, k, H, I, max_tokens, max_tokens * k, 0, 0, kMfmaMinTokens};
  int most = d.max_entries < E ? d.max_entries : E;
  d.max_waves = ceil_div(most, K);
  if (d.max_waves < 1) d.max_waves = 1;
  d.max_tiles = ceil_div(d.max_entries, kTileM) + E;
  return d;
}

// Per-layer block (int32 words): two copies of the LRU state, the index of the
// current one, the last step's plans and slot map.  A device-planned step reads
// copy `cur` in every block of its planning kernel and writes the new state into
// the other copy; a later kernel of the same step flips `cur`.  No block can
// therefore read a half-written state.  Host-planned steps update copy `cur` in
// place.  tick / slot_expert / expert_slot / last_use are offsets inside a copy.
struct LayerLayout {
  size_t tick;          // [1]    uint32: tick of the next wave
  size_t slot_expert;   // [K]    expert in slot j, -1 = empty
  size_t expert_slot;   // [E]    slot of expert e, -1 = not resident
  size_t last_use;      // [K]    uint32: tick of the wave that last used slot j
  size_t state_words;   // words of one state copy
  size_t cur;           // [1]    current state copy (0 or 1)
  size_t state0;        // first state copy; the second follows at state0 + state_stride
  size_t state_stride;
  size_t n_waves;       // [1]    waves of the last step
  size_t plan_count;    // [MW]   page-ins of wave w
  size_t plan_expert;   // [MW*K] expert copied in
  size_t plan_slot;     // [MW*K] slot it went to
  size_t plan_evicted;  // [MW*K] previous occupant (-1 = empty)
  size_t slot_of;       // [max_entries] slot entry t*k+j ran in (-1 invalid id)
  size_t state_prefix;  // words from the block start through both state copies
  size_t total;         // words per layer (rounded to 64)

  size_t state(int copy) const { return state0 + (size_t)copy * state_stride; }
};

inline LayerLayout make_layer_layout(const Dims& d) {
  LayerLayout l{};
  l.tick = 0;
  l.slot_expert = 1;
  l.expert_slot = 1 + (size_t)d.K;
  l.last_use = 1 + (size_t)d.K + d.E;
  l.state_words = 1 + 2 * (size_t)d.K + d.E;
  size_t o = 0;
  l.cur = o; o += 1;
  l.state0 = o;
  l.state_stride = l.state_words;
  o += 2 * l.state_words;
  l.state_prefix = o;
  l.n_waves = o; o += 1;
  l.plan_count = o; o += d.max_waves;
  l.plan_expert = o; o += (size_t)d.max_waves * d.K;
  l.plan_slot = o; o += (size_t)d.max_waves * d.K;
  l.plan_evicted = o; o += (size_t)d.max_waves * d.K;
  l.slot_of = o; o += d.max_entries;
  l.total = (o + 63) / 64 * 64;
  return l;
}

// One plan-log record (int32 words): what one step of one layer decided.
//   [0] seq        the layer's step number since the context was created (from 0)
//   [1] T          tokens of the step
//   [2] tick       the layer's tick after the step
//   [3] 0
//   [4 ...]        the block's plan area as the step left it, word for word:
//                  n_waves, count[MW], experts[MW*K], slots[MW*K], evicted[MW*K]
//                  (wave-major, entries r < count[w] valid), slot_of[max_entries]
//                  (first T*k valid)
//   then           slot_expert[K] and last_use[K] after the step
// padded to a multiple of 16 words.
struct PlanLogLayout {
  size_t plan;          // first word of the copied plan area
  size_t plan_words;    // words of the plan area (ll.slot_of + max_entries - ll.n_waves)
  size_t slot_expert;   // [K]
  size_t last_use;      // [K]
  size_t total;         // words per record
};

inline PlanLogLayout make_plan_log_layout(const Dims& d, const LayerLayout& ll) {
  PlanLogLayout p{};
  p.plan = 4;
  p.plan_words = ll.slot_of + (size_t)d.max_entries - ll.n_waves;
  p.slot_expert = p.plan + p.plan_words;
  p.last_use = p.slot_expert + (size_t)d.K;
  p.total = (p.last_use + (size_t)d.K + 15) / 16 * 16;
  return p;
}

// Step work arena (int32 words), shared by all layers (steps run in stream order).
// "Used" experts are those with at least one valid entry; they are numbered u in
// wave order and, inside a wave, by ascending expert id.  Entries of used expert
// u occupy sorted positions [used_off[u], used_off[u+1]) in ascending entry index.
struct WorkLayout {
  size_t hdr;           // header, see hdr_* below
  size_t used_expert;   // [E]
  size_t used_slot;     // [E]
  size_t used_off;      // [E+1]
  size_t gemv_u;        // [E]          used experts on the GEMV kernels, per wave
  size_t gemv_desc;     // [E][4]       the same GEMV items as {slot, first sorted position,
                        //              entry count, expert id}, 16-byte aligned
  size_t tile_desc;     // [max_tiles][4] MFMA tiles as {slot, first sorted position, rows (<= kTileM),
                        //              expert id}, 16-byte aligned
  size_t entries;       // [max_entries] entry index t*k+j at each sorted position
  size_t total;
};

// Header words (constexpr, so kernels can use them too): [0] n_waves, then
// wave_u_begin[MW+1], gemv_begin[MW+1], tile_begin[MW+1], gemv_split[MW],
// tile_split[MW].  Inside a wave, GEMV items and MFMA tiles list first the
// experts that were resident before the wave's page-in ("hits"), then the ones
// it copies in; *_split[w] is where the second group starts, so the hits can
// run while the page-in is in flight.
constexpr size_t hdr_wave_u(int MW, int w) { return (void)MW, 1 + (size_t)w; }
constexpr size_t hdr_gemv(int MW, int w) { return 1 + (size_t)(MW + 1) + w; }
constexpr size_t hdr_tile(int MW, int w) { return 1 + 2 * (size_t)(MW + 1) + w; }
constexpr size_t hdr_gemv_split(int MW, int w) { return 1 + 3 * (size_t)(MW + 1) + w; }
constexpr size_t hdr_tile_split(int MW, int w) { return 1 + 3 * (size_t)(MW + 1) + MW + w; }
constexpr size_t hdr_words(int MW) { return 1 + 3 * (size_t)(MW + 1) + 2 * (size_t)MW; }

inline WorkLayout make_work_layout(const Dims& d) {
  WorkLayout w{};
  size_t o = 0;
  w.hdr = o; o += (hdr_words(d.max_waves) + 15) / 16 * 16;
  w.used_expert = o; o += d.E;
  w.used_slot = o; o += d.E;
  w.used_off = o; o += d.E + 1;
  w.gemv_u = o; o += d.E;
  o = (o + 3) / 4 * 4;
  w.gemv_desc = o; o += 4 * (size_t)d.E;
  w.tile_desc = o; o += 4 * (size_t)d.max_tiles;
  w.entries = o; o += d.max_entries;
  w.total = (o + 63) / 64 * 64;
  return w;
}

// Result of one host-planned step, beyond what is written into the layer
// block and the work arena.
struct HostPlanSummary {
  int n_waves;
  int distinct;
  int page_ins;
  int valid_entries;
  int bad_ids;
  int max_gemv_tokens;   // largest entry count among GEMV experts
  int gemv_items[kMaxExperts];   // per wave: experts on the GEMV kernels
  int gemv_hits[kMaxExperts];    // per wave: of which resident before the wave
  int tiles[kMaxExperts];        // per wave: MFMA tiles
  int tile_hits[kMaxExperts];    // per wave: of which for resident experts
};

// Plan one step of one layer on the host (the multi-wave path).  `blk` is a
// host mirror of the layer block whose state copy `cur` is current; on return
// that copy holds the new state, and the block the plans of every wave and the
// slot map.  `work` is a
// host mirror of the work arena, filled for the step.  Returns 0 or -1 if the
// step needs more waves than the layout holds.
int host_plan_step(const Dims& d, const LayerLayout& ll, const WorkLayout& wl,
                   const int32_t* ids, int n_entries, int32_t* blk, int32_t* work,
                   HostPlanSummary* sum);

}  // namespace pe
