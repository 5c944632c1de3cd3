// Launchers of the libpe HIP kernels (defined in pe_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "pe_layout.h"

namespace pe {

// Offsets of the layer block and the work arena, in int32 words, as kernel arguments.
struct Offsets {
  int tick, slot_expert, expert_slot, last_use;   // inside a state copy
  int cur, state0, state_stride;                  // current copy, copies
  int n_waves, plan_count, plan_expert, plan_slot, plan_evicted, slot_of;
  int hdr, used_expert, used_slot, used_off, gemv_u, gemv_desc, tile_desc, entries;
};

Offsets make_offsets(const LayerLayout& ll, const WorkLayout& wl);

// Everything the expert kernels read: one layer's slot table, the step work
// lists and the activations.
struct ExpertArgs {
  const uint8_t* slots;       // slot 0 of the layer
  size_t slot_stride;         // bytes between slots
  size_t off_w13, off_w2, off_s13, off_s2;   // sub-tensor offsets inside a blob
  const int32_t* work;        // work arena
  Offsets o;
  int MW;                     // header capacity (max waves)
  int wave;                   // wave whose experts this launch runs
  int part;                   // 0: all its experts; 1: those resident before the
                              // wave's page-in; 2: those it pages in
  const uint16_t* x;          // [T, H] bf16
  const float* topk_w;        // [T*k]
  uint16_t* h;                // [max_entries, I] bf16, by sorted position
  float* merged;              // [T*k, H] fp32, by entry index
  int H, I, k;
  // lean = 1 (device-planned steps, part 1): each workgroup finds its resident
  // expert from the routed ids and the current LRU-state copy instead of the
  // published work lists, so it can run alongside the planning + page-in kernel.
  int lean;
  // hdr_known = 1: this launch's GEMV ranges of the wave (start, end of the
  // experts resident before the wave, end) are g0 / gsplit / g1 and its MFMA
  // tile ranges t0 / tsplit / t1, instead of the work arena's header (which
  // may be in host memory, or one dependent load away)
  int hdr_known, g0, gsplit, g1, t0, tsplit, t1;
  int mfma_min;
  const int32_t* ids;         // [T*k] routed ids
  int T, E;
  const int32_t* blk;         // the layer block
};

// Single-wave device-planned step (T*k <= K), planning and page-in in one launch:
// every workgroup makes the same LRU decision in LDS from the current state copy
// (no workgroup waits for another); workgroup 0 publishes the plan, slot map,
// work lists, counters and the new state (into the other copy); then every
// workgroup copies its share of the planned experts from the mapped host rows
// (`grid` workgroups; with copy == false one workgroup, planning only).
void launch_plan_page_in(int32_t* blk, const int32_t* ids, int n, const Dims& d, const Offsets& o,
                         int mfma_min, int32_t* work, unsigned long long* stats, const uint8_t* host_rows,
                         uint8_t* slots, size_t stride, size_t copy_bytes, bool copy, int grid, hipStream_t s);

// Copy the planned experts of wave `wave` from the mapped host rows into their
// slots, reading the page-in count on the device.
void launch_page_in(const int32_t* blk, const Offsets& o, int wave, int K,
                    const uint8_t* host_rows, uint8_t* slots, size_t stride, size_t copy_bytes,
                    int grid, hipStream_t s);

// Raw mapped-read copy (the page-in copy routine on plain buffers).
void launch_copy(void* dst, const void* src, size_t bytes, int grid, hipStream_t s);

// GEMV expert kernels for the experts of one wave with few tokens each.
// `items` bounds the experts of the launch; `max_m` bounds their token counts.
void launch_gemv_gate_up(int wtype, const ExpertArgs& a, int items, int max_m, hipStream_t s);
void launch_gemv_down(int wtype, const ExpertArgs& a, int items, int max_m, hipStream_t s);

// Device-planned step with no many-token expert, two launches on one queue.
// Launch A: `P` workgroups plan the wave (as launch_plan_page_in) and page in its
// missing experts, computing their gate/up projection from the rows as they
// arrive from the host; one more workgroup publishes the plan; the others run
// the gate/up projection of the experts already resident (`a`: lean = 1, ids, T,
// E, blk set).  Launch B (launch_down_sum): the down projection of every expert
// of the wave and the fixed-order top-k sum into `out` by output-row blocks
// (`a`: ids, T, E set); it toggles `flip` (the layer's current LRU-state copy).
// The merged buffer is not used.
void launch_step_a(int wtype, int32_t* blk, const int32_t* ids, int n, const Dims& d, const Offsets& o,
                   int mfma_min, int32_t* work, unsigned long long* stats, const uint8_t* host_rows,
                   uint8_t* slots, size_t stride, size_t copy_bytes, int P, const ExpertArgs& a, int items,
                   int max_m, hipStream_t s);
void launch_down_sum(int wtype, const ExpertArgs& a, int max_m, uint16_t* out, int32_t* flip, hipStream_t s);

// Host-planned wave with no MFMA tiles (`a` = the wave, part 1): `P` workgroups
// page in the wave's missing experts from the mapped host rows with their
// gate/up projection computed on the way; the others run the gate/up
// projection of its `hit_items` resident experts.  With up_bytes > 0, one more
// workgroup copies `up_bytes` from the mapped host address `up_src` (the host's
// plan) to `up_dst` (the layer block and work lists in device memory), and
// `a.work` may point at the host's copy of the work lists.  Follow with
// launch_gemv_down over all of the wave's GEMV items (part 0).
void launch_wave_a(int wtype, const ExpertArgs& a, int hit_items, int max_m, int P, const uint8_t* host_rows,
                   size_t stride, size_t copy_bytes, const void* up_src, void* up_dst, size_t up_bytes,
                   hipStream_t s);

// MFMA grouped-GEMM expert kernels for the tiles of one wave (experts with many
// tokens).  Need H and I multiples of mfma_multiple(wtype): 64 for bf16 and
// MXFP4 (32x32 MFMA kernels, K staged 64 wide), 128 for the block- and
// group-scaled formats (one scale per 128-wide K block).
void launch_mfma_gate_up(int wtype, const ExpertArgs& a, int tiles, hipStream_t s);
void launch_mfma_down(int wtype, const ExpertArgs& a, int tiles, hipStream_t s);
int mfma_multiple(int wtype);

// out[t] = bf16(sum_j merged[t,j]) over valid entries, j in order; if `flip` is
// set, it toggles that word (the layer's current LRU-state copy).
void launch_topk_sum(const float* merged, const int32_t* ids, int T, int k, int E, int H,
                     uint16_t* out, int32_t* flip, hipStream_t s);

// Reset the LRU state of layers [l0, l1): empty, or the identity map.
void launch_reset_lru(int32_t* blocks, size_t layer_words, int l0, int l1, const Offsets& o,
                      int E, int K, bool identity, hipStream_t s);

// Host-planned step, before the host plans: copy the layer block's first
// `state_words` words (current-copy index and both LRU-state copies) to
// `host_blk` and the n routed ids to `host_ids`, both page-locked coherent host
// memory written through its mapped device address (one launch, no copy
// engine), then store `seq` to the host word `flag` once those writes are
// visible to the host.
void launch_gather_state(const int32_t* blk, int state_words, const int32_t* ids, int n, int32_t* host_blk,
                         int32_t* host_ids, uint32_t* flag, uint32_t seq, hipStream_t s);

// Append one record (PlanLogLayout) of the step that just ended to the layer's
// plan-log ring: `ring` holds `cap` records of `rec_words` words; *seq counts
// the layer's logged steps and is advanced.  Reads the layer block's plan area
// (`plan_words` words from word `plan0`) and its current LRU-state copy.
void launch_plan_log(const int32_t* blk, const Offsets& o, int K, int plan0, int plan_words, int T,
                     int32_t* ring, int cap, int rec_words, uint32_t* seq, hipStream_t s);

// The library's fixed device scratch area (no allocation): its size, and its
// address on the current device (looked up once per device with
// hipGetSymbolAddress; NULL if the lookup failed).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
void* static_scratch(int device);

}  // namespace pe
