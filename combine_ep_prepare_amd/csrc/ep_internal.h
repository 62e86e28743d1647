// ep_internal.h -- handle layout and kernel launchers shared by the C-ABI
// entry points (ep_api.hip) and the gfx950 kernels (ep_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace epmi {

constexpr int kWave = 64;
constexpr int kMaxTopk = 64;
constexpr int kMaxExperts = 2048;
constexpr int kKeyBits = 11;  // bits of an expert id below kMaxExperts
constexpr uint32_t kHandleMagic = 0x45504D49u;  // "EPMI"

// Routes per prepare work unit (one wavefront): kPrepRounds x 64.
constexpr int kPrepRounds = 8;
constexpr int kUnitRoutes = kPrepRounds * kWave;

// Run entries. The routes are cut into chunks of run_units consecutive
// prepare units (RU * 512 routes, RU in {1, 2, 4}), and chunk c belongs to
// XCD stream c mod 8. A chunk's entries are its routes that hold a row, in
// ascending received-row order (so the rows an expert receives from the
// chunk, one contiguous run, are adjacent), then one empty entry for each of
// its valid routes dropped past the capacity. Each stream's chunks are laid
// out one after another in that stream's list, which starts at
// x * stream_cap(U) entries; the header holds each list's length.
struct RunEntry {
  int32_t row;    // received row, or -1 for an empty entry
  int32_t route;  // route index s = t*K + k
};
constexpr int kRunXcds = 8;             // chunks are dealt round-robin to 8 streams
constexpr int kRunMaxUnits = 4;         // at most 4 units (2048 routes) per chunk
constexpr int64_t kRunChunkBytes = 3584 * 1024;   // token rows of one chunk, at most

// Units per chunk: the most (up to 4) whose tokens' rows (RU * 512 / K of
// them) fit in kRunChunkBytes, so that a chunk's token rows stay in one XCD's
// 4 MB L2 while its runs are written; fewer if that leaves some stream with
// no chunk. Chosen by prepare from its layout's row size and kept in the
// header, so payload ops of another payload type read the same entries.
// Measured on the MI355X (dsv3 routing, the copy launched one step a block):
// 3.5 MiB (four units a chunk for 14 KiB rows, two for fp32 rows of 28 KiB)
// against 2.5 MiB takes combine_bwd from 127 to 120 us warm and 128 to 125
// cold, dispatch and the masked shares level, with the same bytes fetched
// (fp32 dispatch 1506 MB for 1505 algorithmic); the weighted backward on
// dsv3 fetches 707 MB for 625 (its y rows push token rows out of the L2) in
// the same time, and its row gradient alone is 8 us faster on dsv3 and 8 us
// slower on the hot-expert share.
inline int32_t run_chunk_units(int32_t units, int32_t K, int64_t row_bytes) {
  int32_t ru = kRunMaxUnits;
  while (ru > 1 && (int64_t)ru * kUnitRoutes / K * row_bytes > kRunChunkBytes) ru /= 2;
  while (ru > 1 && (units + ru - 1) / ru < kRunXcds) ru /= 2;
  return ru;
}

// Entries each stream's list can hold: its chunks, at most ceil(ceil(U/RU)/8)
// of RU * 512 entries, which is at most 64 U + 2048 for any RU <= 4.
__host__ __device__ inline int64_t run_stream_cap(int32_t units) {
  return (int64_t)units * (kUnitRoutes / kRunXcds) + (int64_t)kRunMaxUnits * kUnitRoutes;
}

// The most entries one stream receives when every route holds a row, over
// the chunk sizes prepare may choose: what a run copy's grid is sized for.
inline int64_t run_stream_dense(int32_t units, int64_t routes) {
  int64_t m = 0;
  for (int32_t ru = 1; ru <= kRunMaxUnits; ru *= 2) {
    const int64_t nch = (units + ru - 1) / ru;
    const int64_t e = (nch + kRunXcds - 1) / kRunXcds * ru * kUnitRoutes;
    if (e > m) m = e;
  }
  return m < routes ? m : routes;
}

// Header at the start of every handle (256 bytes reserved).
struct HandleHeader {
  uint32_t status;      // EP_STATUS_* bits of the last prepare
  uint32_t magic;       // kHandleMagic once prepared
  int64_t num_tokens;
  int32_t topk;
  int32_t num_experts;
  int32_t alignment;
  int32_t num_units;
  int64_t recv_capacity;
  int32_t total;        // offsets[E]
  int32_t pads_live;    // pad rows below recv_capacity
  int32_t run_units;    // units per run chunk (RU)
  int32_t stream_live[kRunXcds];  // entries in each stream's run list
};
static_assert(sizeof(HandleHeader) <= 256, "header too large");

// Byte offsets of the regions of a handle; every region is 256-byte aligned.
// The routing maps come first (maps_bytes of them: everything the payload ops
// read); prepare's scratch (the per-unit histograms and bad-id flags of its
// two-kernel form) closes the handle.
struct HandleLayout {
  size_t header, counts, offsets, pad_offsets, slot, row_src, pad_rows, runs, maps_bytes,
      unit_hist, unit_flags, bytes;
  int32_t num_units;
};

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline int32_t prep_units(int64_t routes) {
  return (int32_t)((routes + kUnitRoutes - 1) / kUnitRoutes);
}

// LDS one prepare block may take.
constexpr size_t kPrepLdsBudget = 65536;

// Up to this many block-sum rows every block of the slot kernel sums them
// itself (about 64 * E loads each); past it the column scan takes its own
// launch, so that prepare's work stays linear in the routes.
constexpr int kPrepDirectBlockRows = 64;

// Units per block of the histogram kernel (one wave-private E-entry
// histogram each): four while the block rows stay within
// kPrepDirectBlockRows, else eight; fewer when they do not fit the LDS
// budget. Its wavefronts spend most of their time matching peers one round
// after another, so while the direct sums allow, smaller blocks spread them
// over more CUs. Measured on the MI355X (prepare us, four units a block
// against eight): top-8 of 256 at 4096 tokens 19.3 against 20.3, top-8 of
// 128 at 8192 18.1 against 19.0, top-2 of 8 at 16384 16.5 against 16.7; the
// 32-expert masked share at 32768 (512 units) 21.6 against 19.3, where four
// would take the column scan; two units a block were slower.
inline int32_t hist_block_units(int32_t num_units, int32_t E) {
  int32_t nw = num_units <= 4 * kPrepDirectBlockRows ? 4 : 8;
  while (nw > 1 && sizeof(int32_t) * (size_t)nw * (size_t)E > kPrepLdsBudget) nw /= 2;
  return nw;
}

// Block-sum rows of the histogram kernel: one per block, then one more for
// the totals (written by the column scan when it runs).
inline int32_t hist_block_rows(int32_t num_units, int32_t E) {
  const int32_t nw = hist_block_units(num_units, E);
  return (num_units + nw - 1) / nw + 1;
}

// Bytes of prepare's histograms (the first part of its scratch): the
// per-unit rows [num_units][E], then the block-sum rows.
inline size_t scratch_hist_bytes(int32_t num_units, int32_t E) {
  return align256(sizeof(int32_t) * ((size_t)num_units + (size_t)hist_block_rows(num_units, E)) *
                  (size_t)E);
}

// Bytes of prepare's per-unit words: each unit's flag word, then (for as
// many chunks as there can be, one per unit) each chunk's start in its
// stream's run list, which the column scan writes for large routings.
inline size_t scratch_unit_bytes(int32_t num_units) {
  return align256(2 * sizeof(int32_t) * (size_t)num_units);
}

// Bytes of prepare's whole scratch: the histograms, then the per-unit words.
inline size_t scratch_bytes(int32_t num_units, int32_t E) {
  return scratch_hist_bytes(num_units, E) + scratch_unit_bytes(num_units);
}

inline HandleLayout handle_layout(int64_t T, int32_t K, int32_t E, int64_t cap) {
  HandleLayout h{};
  const int64_t routes = T * (int64_t)K;
  h.num_units = prep_units(routes);
  size_t at = 0;
  h.header = at;       at += 256;
  h.counts = at;       at += align256(sizeof(int32_t) * (size_t)E);
  h.offsets = at;      at += align256(sizeof(int32_t) * (size_t)(E + 1));
  h.pad_offsets = at;  at += align256(sizeof(int32_t) * (size_t)(E + 1));
  h.slot = at;         at += align256(sizeof(int32_t) * (size_t)routes);
  h.row_src = at;      at += align256(sizeof(int32_t) * (size_t)cap);
  h.pad_rows = at;     at += align256(sizeof(int32_t) * (size_t)cap);
  h.runs = at;
  at += align256(sizeof(RunEntry) * (size_t)kRunXcds * (size_t)run_stream_cap(h.num_units));
  h.maps_bytes = at;
  h.unit_hist = at;    at += scratch_hist_bytes(h.num_units, E);
  h.unit_flags = at;   at += scratch_unit_bytes(h.num_units);
  h.bytes = at;
  return h;
}

// Device pointers into one handle, passed by value to every kernel.
struct HandleView {
  HandleHeader* header;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pad_offsets;
  int32_t* slot;
  int32_t* row_src;
  int32_t* pad_rows;
  int32_t* unit_hist;
  int32_t* unit_flags;   // per unit: (valid routes << 1) | bad-id flag; then
                         // per chunk: its start in its stream's list
  RunEntry* runs;
};

inline HandleView handle_view(void* mem, const HandleLayout& h) {
  char* b = static_cast<char*>(mem);
  HandleView v;
  v.header = reinterpret_cast<HandleHeader*>(b + h.header);
  v.counts = reinterpret_cast<int32_t*>(b + h.counts);
  v.offsets = reinterpret_cast<int32_t*>(b + h.offsets);
  v.pad_offsets = reinterpret_cast<int32_t*>(b + h.pad_offsets);
  v.slot = reinterpret_cast<int32_t*>(b + h.slot);
  v.row_src = reinterpret_cast<int32_t*>(b + h.row_src);
  v.pad_rows = reinterpret_cast<int32_t*>(b + h.pad_rows);
  v.unit_hist = reinterpret_cast<int32_t*>(b + h.unit_hist);
  v.unit_flags = reinterpret_cast<int32_t*>(b + h.unit_flags);
  v.runs = reinterpret_cast<RunEntry*>(b + h.runs);
  return v;
}

// Sizes every kernel receives.
struct Dims {
  int64_t T;
  int32_t K;
  int32_t E;
  int32_t A;
  int32_t num_units;
  int64_t cap;
  int64_t H;
  int64_t V;          // 16-byte vectors per payload row: H * element size / 16
  int32_t dtype;      // EP_DTYPE_* of the payload rows
  int32_t fill_pads;  // 1: payload ops zero the live pad rows; 0: leave them
  int32_t zero_tail;  // 1: payload ops also zero rows [min(total, cap), cap)
};

// Launchers (ep_kernels.hip). Each returns the hipError_t of its launch.
hipError_t launch_prepare(const Dims& d, const HandleView& hv, const int64_t* topk_idx,
                          int32_t* user_counts, int32_t* user_offsets, int num_cus,
                          hipStream_t stream);
// Payload pointers are raw rows of d.dtype.
hipError_t launch_scatter_rows(const Dims& d, const HandleView& hv, const void* src,
                               const float* w, void* dst, float* dst_w, int num_cus,
                               hipStream_t stream);
// The map D over the run entries (every routing): one launch sized for a
// dense routing, its work read on the device.
hipError_t launch_run_rows(const Dims& d, const HandleView& hv, const void* src,
                           const float* w, void* dst, float* dst_w, int num_cus,
                           hipStream_t stream);
hipError_t launch_reduce_rows(const Dims& d, const HandleView& hv, const void* src,
                              const float* rw, const float* g_w, void* dst, float* dst_w,
                              int num_cus, hipStream_t stream);
hipError_t launch_weighted_bwd(const Dims& d, const HandleView& hv, const void* g,
                               const void* y, const float* rw, void* grad_rows, float* grad_w,
                               int num_cus, hipStream_t stream);

}  // namespace epmi
