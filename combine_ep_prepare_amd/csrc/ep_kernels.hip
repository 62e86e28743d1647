// ep_kernels.hip -- gfx950 (CDNA4) kernels for MoE expert-parallel routing.
//
// Four kernel families serve the five ops of "Expert Parallelism: common C
// API + NCCL EP backend" (section "Per-step (allocation-free, CUDA-graph
// capturable)") at one GPU's share, and the fused weighted combine with its
// backward:
//
//   prepare      prepare_hist_kernel + prepare_slots_kernel: a per-wavefront
//                expert histogram privatised in LDS, a block-wide wavefront-
//                shuffle exclusive scan of the aligned segment lengths, and a
//                stable (route-ordered) slot map; prepare_fused_kernel does
//                the same in one block and one launch for small routings.
//                Both also write the run entries: each chunk of routes' rows
//                in received-row order, chunk c on list c mod 8.
//   dispatch,    run_rows_kernel: the linear map D that copies token row t
//   combine_bwd  into the received row of each of its valid routes and
//                zero-fills pad rows, walking the run entries so that the
//                blocks of one XCD write dense bands of received rows and
//                read each chunk's token rows from memory once, then from
//                that XCD's L2. scatter_rows_kernel is the fallback for
//                sizes past the run copy's 32-bit piece indices.
//   combine,     reduce_rows_kernel: the transpose of D. Each token row is the
//   dispatch_bwd fp32 sum, k ascending, of the received rows of its valid
//                routes, rounded once to the payload type; the dispatch_bwd
//                weight gradient is gathered in the same pass. With the
//                received weights it is the fused weighted combine.
//   weighted     run_wbwd_kernel: the weighted combine's row gradient (w * g
//   backward     copied along the run entries) and weight gradient (a dot
//                product per route, summed in a fixed order);
//                weighted_bwd_kernel is its token-group fallback.
//
// None of this is a dense contraction, so no MFMA: every kernel is bound by
// HBM traffic (or, for prepare, by latency). Rows move as 16-byte vectors,
// 64 lanes x 16 B = 1 KiB per wavefront instruction, fully coalesced.
// Work is split into units handed out in a grid-stride loop whose bound is
// read on the device, so no host sync is ever needed and every launch is
// graph-capturable.

#include <hip/hip_runtime.h>

#include <utility>

#include "ep.h"
#include "ep_internal.h"

namespace epmi {

namespace {

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N). Keeps
// every index of the small per-lane register arrays a constant, so they stay
// in VGPRs instead of being demoted to LDS or scratch.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return static_cast<uint64_t>(__ballot(p));
}

// Lanes whose (valid) key equals this lane's key: the intersection, over the
// key's bits, of the ballot of lanes agreeing on that bit. nbits ballots
// instead of one iteration per distinct key.
__device__ __forceinline__ uint64_t match_peers(uint32_t key, bool valid, int nbits) {
  uint64_t m = wave_ballot(valid);
  // all kKeyBits bits, unrolled: bits at or above nbits are zero in every
  // valid key and leave m unchanged
  static_for<kKeyBits>([&](auto b) {
    if (b < nbits) {
      const bool bit = (key >> b) & 1u;
      const uint64_t ones = wave_ballot(valid && bit);
      m &= bit ? ones : ~ones;
    }
  });
  return m;
}

// The whole header is copied in one go and then tested without
// short-circuits, so it costs one round trip instead of one per field.
__device__ __forceinline__ bool handle_matches(const HandleHeader& hh, const Dims& d) {
  return (hh.magic == kHandleMagic) & (hh.num_tokens == d.T) & (hh.topk == d.K) &
         (hh.num_experts == d.E) & (hh.alignment == d.A) & (hh.recv_capacity == d.cap) &
         (hh.total >= 0) & (hh.pads_live >= 0);
}

// Rows a payload op writes as zeros, in this order: the live pad rows
// (pad_rows[0, npads), ascending) when pads are filled, then the rows past the
// live total (live .. cap-1) when the tail is zeroed.
struct ZeroRows {
  int64_t npads;  // pad rows among them
  int64_t n;      // all of them
  int64_t live;   // min(total, cap): the first tail row
};

__device__ __forceinline__ ZeroRows zero_rows_of(const HandleHeader& hh, const Dims& d) {
  ZeroRows z;
  z.live = (int64_t)hh.total < d.cap ? (int64_t)hh.total : d.cap;
  z.npads = d.fill_pads ? (int64_t)hh.pads_live : 0;
  z.n = z.npads + (d.zero_tail ? d.cap - z.live : 0);
  return z;
}

__device__ __forceinline__ int64_t zero_row(const ZeroRows& z,
                                            const int32_t* __restrict__ pad_rows, int64_t i) {
  return i < z.npads ? (int64_t)pad_rows[i] : z.live + (i - z.npads);
}

// fp32 -> bf16 bits, round to nearest even; any NaN -> 0x7FC0. Adding
// 0x7FFF plus the lowest kept bit carries into the kept half exactly when the
// discarded half is above one half ulp, or equal to it with an odd kept half.
__device__ __forceinline__ uint32_t rne_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace

// ---------------------------------------------------------------------------
// prepare
// ---------------------------------------------------------------------------

namespace {

// The kPrepRounds x 64 routing ids of one unit. Every load is issued
// unconditionally (lanes past the last route re-read it; unit_id() masks
// them where the ids are used), so all of them are in flight together.
__device__ __forceinline__ void load_unit_ids(const int64_t* __restrict__ topk_idx,
                                              int64_t base, int64_t routes, int lane,
                                              int64_t (&ids)[kPrepRounds]) {
  static_for<kPrepRounds>([&](auto i) {
    const int64_t s = base + i * kWave + lane;
    ids[i] = topk_idx[s < routes ? s : routes - 1];
  });
}

__device__ __forceinline__ int64_t unit_id(const int64_t (&ids)[kPrepRounds], int i,
                                           int64_t s, int64_t routes) {
  return s < routes ? ids[i] : -1;
}

}  // namespace

// One wavefront per unit of kUnitRoutes consecutive routes. Histogram of the
// unit's valid expert ids in a wave-private LDS row; each distinct id of a
// 64-route round is added once, by its lowest lane, with the peer count. The
// count before the add plus the route's rank among its peers is the route's
// rank among the unit's routes of its expert: it is left in slot[s], packed
// with the expert id, for prepare_slots_kernel. The unit's flag word holds
// its count of valid routes and whether it saw a bad id.
__global__ void __launch_bounds__(512)
prepare_hist_kernel(Dims d, HandleView hv, const int64_t* __restrict__ topk_idx, int nbits) {
  extern __shared__ int32_t lds[];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int E = d.E;
  int32_t* hist = lds + w * E;
  for (int e = lane; e < E; e += kWave) hist[e] = 0;
  __syncthreads();

  const int64_t routes = d.T * d.K;
  const int32_t u = blockIdx.x * nw + w;
  bool bad_any = false;
  int32_t nvalid = 0;
  if (u < d.num_units) {
    const int64_t base = (int64_t)u * kUnitRoutes;
    int64_t ids[kPrepRounds];
    load_unit_ids(topk_idx, base, routes, lane, ids);
    // All rounds are matched first, then all claims are issued back to back
    // (one wavefront's LDS atomics are served in order), so each route's
    // rank among the unit's routes of its expert comes out in route order.
    uint64_t peers[kPrepRounds];
    uint32_t key[kPrepRounds];
    bool valid[kPrepRounds];
    static_for<kPrepRounds>([&](auto i) {
      const int64_t id = unit_id(ids, i, base + i * kWave + lane, routes);
      valid[i] = id >= 0 && id < E;
      const bool bad = !valid[i] && id != -1;
      bad_any |= wave_ballot(bad) != 0;
      nvalid += __popcll(wave_ballot(valid[i]));
      key[i] = valid[i] ? (uint32_t)id : 0u;
      peers[i] = match_peers(key[i], valid[i], nbits);
    });
    int32_t first[kPrepRounds];
    int leader[kPrepRounds];
    static_for<kPrepRounds>([&](auto i) {
      leader[i] = valid[i] ? __ffsll((unsigned long long)peers[i]) - 1 : lane;
      first[i] = 0;
      if (valid[i] && lane == leader[i])
        first[i] = atomicAdd(&hist[key[i]], (int32_t)__popcll(peers[i]));
    });
    static_for<kPrepRounds>([&](auto i) { first[i] = __shfl(first[i], leader[i]); });
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    static_for<kPrepRounds>([&](auto i) {
      const int64_t s = base + i * kWave + lane;
      if (s < routes) {
        const int32_t rank = first[i] + __popcll(peers[i] & lanes_below);
        hv.slot[s] = valid[i] ? (rank << kKeyBits) | (int32_t)key[i] : -1;
      }
    });
  }
  __syncthreads();
  if (u < d.num_units) {
    int32_t* out = hv.unit_hist + (int64_t)u * E;
    for (int e = lane; e < E; e += kWave) out[e] = hist[e];
    if (lane == 0) hv.unit_flags[u] = (nvalid << 1) | (bad_any ? 1 : 0);
  }
  // the block's row of unit sums (rows of waves past the last unit are zero)
  int32_t* brow = hv.unit_hist + ((int64_t)d.num_units + blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t sum = 0;
    for (int q = 0; q < nw; ++q) sum += lds[q * E + e];
    brow[e] = sum;
  }
}

// For routings of many units: an exclusive scan down each expert's column of
// the block-sum rows (in place), and the column totals in the row after the
// last block's. Block b takes 64 experts, one per lane; its eight wavefronts
// split the rows into eight ranges, sum them, and rewrite them as running
// sums from the ranges' starts. Linear in the rows; prepare_slots_kernel then
// reads one row for its units' predecessors.
__global__ void __launch_bounds__(512)
prepare_scan_kernel(Dims d, HandleView hv, int32_t nb, int32_t ru) {
  __shared__ int32_t s_tot[8][kWave];
  constexpr int kBatch = 16;
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int E = d.E;
  const int e = blockIdx.x * kWave + lane;
  const int ec = e < E ? e : E - 1;
  int32_t* blk = hv.unit_hist + (int64_t)d.num_units * E;
  const int32_t per = (nb + 7) / 8;
  const int32_t r0 = w * per < nb ? w * per : nb;
  const int32_t r1 = r0 + per < nb ? r0 + per : nb;
  int32_t sum = 0;
  for (int32_t rb = r0; rb < r1; rb += kBatch) {
    int32_t v[kBatch];
    static_for<kBatch>([&](auto j) {
      const int32_t r = rb + j;
      v[j] = blk[(int64_t)(r < r1 ? r : r1 - 1) * E + ec];
    });
    static_for<kBatch>([&](auto j) { sum += rb + j < r1 ? v[j] : 0; });
  }
  s_tot[w][lane] = sum;
  __syncthreads();
  int32_t run = 0, total = 0;
  for (int q = 0; q < 8; ++q) {
    run += q < w ? s_tot[q][lane] : 0;
    total += s_tot[q][lane];
  }
  for (int32_t rb = r0; rb < r1; rb += kBatch) {
    int32_t v[kBatch];
    static_for<kBatch>([&](auto j) {
      const int32_t r = rb + j;
      v[j] = blk[(int64_t)(r < r1 ? r : r1 - 1) * E + ec];
    });
    static_for<kBatch>([&](auto j) {
      const int32_t r = rb + j;
      if (r < r1 && e < E) blk[(int64_t)r * E + e] = run;
      run += r < r1 ? v[j] : 0;
    });
  }
  if (w == 0 && e < E) blk[(int64_t)nb * E + e] = total;
  if (blockIdx.x != 0) return;
  // Block 0 also gives every chunk of ru units its start in its stream's run
  // list: wavefront x walks stream x's chunks c = x + 8 j in order, 64 at a
  // time, and scans their valid routes (from the unit flags).
  const int32_t U = d.num_units;
  const int32_t nch = (U + ru - 1) / ru;
  int32_t* cbase = hv.unit_flags + U;
  int32_t base = 0;
  for (int32_t j0 = 0; w + kRunXcds * j0 < nch; j0 += kWave) {
    const int32_t c = w + kRunXcds * (j0 + lane);
    int32_t v = 0;
    if (c < nch)
      for (int32_t i = 0; i < ru; ++i) {
        const int32_t u = c * ru + i;
        if (u < U) v += hv.unit_flags[u] >> 1;
      }
    int32_t inc = v;
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    if (c < nch) cbase[c] = base + inc - v;
    base += __shfl(inc, kWave - 1);
  }
}

// Every block derives the same counts and aligned offsets from the
// histograms (block 0 publishes them), then its wavefronts hand out the rows
// of their units: slot = segment start + routes of the same expert in earlier
// units + the route's rank in its unit, which prepare_hist_kernel left in
// slot[s]. The counts and the routes of earlier units come from the
// histogram kernel's block-sum rows (nw1 units each): summed here when there
// are few of them (scanned = 0), else read from the column scan's output.
__global__ void __launch_bounds__(512)
prepare_slots_kernel(Dims d, HandleView hv, int32_t* __restrict__ user_counts,
                     int32_t* __restrict__ user_offsets, int32_t ru, int32_t in_slot,
                     int32_t nw1, int32_t scanned) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t s_wave_tot[2][16];
  __shared__ int32_t s_pads_live;
  __shared__ int32_t s_run_tot[16];     // kept entries of each of this block's chunks
  __shared__ int32_t s_run_valid[16];   // valid routes of each of this block's chunks
  __shared__ int32_t s_run_base[16];    // each chunk's start in its stream's list
  __shared__ int32_t s_wave_vb[16];     // per wavefront: its share of a chunk's start
  __shared__ int32_t s_wave_vo[16];     // per wavefront: its share of a chunk's valid routes
  __shared__ int32_t s_live[kRunXcds];
  const int32_t run_units = in_slot ? ru : 0;
  const int nthr = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int nw = nthr / kWave;
  const int E = d.E;
  const int32_t A = d.A;
  const int32_t U = d.num_units;
  const int32_t u0 = blockIdx.x * nw;
  int32_t* s_counts = lds;              // [E]
  int32_t* s_pre = s_counts + E;        // [E] routes in units before this block
  int32_t* s_offs = s_pre + E;          // [E+1]
  int32_t* s_padoff = s_offs + E + 1;   // [E+1]
  int32_t* s_red = s_padoff + E + 1;    // [2*nthr]
  int32_t* s_cursor = s_red + 2 * nthr; // [(nw+1)*E]: own units' counts, then cursors
  int32_t* s_rbase = s_cursor + (nw + 1) * E;   // [nw/run_units * E] when run_units > 0

  // The packed ranks of this wavefront's unit are loaded first, so that their
  // latency overlaps the histogram loads below.
  const int64_t routes = d.T * d.K;
  const int32_t my_unit = u0 + w;
  const int64_t base = (int64_t)my_unit * kUnitRoutes;
  int32_t pk[kPrepRounds];                // (rank in unit << kKeyBits) | expert, or -1
  if (my_unit < U)
    static_for<kPrepRounds>([&](auto i) {
      const int64_t s = base + i * kWave + lane;
      pk[i] = hv.slot[s < routes ? s : routes - 1];
    });

  // 1. Per expert: the routes of all units (counts) and of the units before
  //    this block (s_pre), from the block-sum rows, then the rows of the
  //    units between the start of unit u0's histogram block and u0; this
  //    block's own unit rows are kept in LDS. Loads are issued kBatch at a
  //    time per thread so that many are in flight.
  const int32_t nb = (U + nw1 - 1) / nw1;
  const int32_t hb0 = u0 / nw1 < nb ? u0 / nw1 : nb;
  const int32_t* blk = hv.unit_hist + (int64_t)U * E;
  if (scanned) {
    for (int e = tid; e < E; e += nthr) {
      s_counts[e] = blk[(int64_t)nb * E + e];
      s_pre[e] = blk[(int64_t)hb0 * E + e];
    }
  } else {
    constexpr int kBatch = 16;
    const int ncols = E < nthr ? E : nthr;
    const int nparts = nthr / ncols;
    for (int e0 = 0; e0 < E; e0 += ncols) {
      const int col = tid % ncols;
      const int part = tid / ncols;
      const int e = e0 + col;
      int32_t all = 0, pre = 0;
      if (part < nparts && e < E && nb > 0) {
        for (int32_t rb = part; rb < nb; rb += kBatch * nparts) {
          int32_t v[kBatch];
          static_for<kBatch>([&](auto j) {
            const int32_t r = rb + j * nparts;
            v[j] = blk[(int64_t)(r < nb ? r : nb - 1) * E + e];
          });
          static_for<kBatch>([&](auto j) {
            const int32_t r = rb + j * nparts;
            const int32_t c = r < nb ? v[j] : 0;
            all += c;
            pre += r < hb0 ? c : 0;
          });
        }
      }
      s_red[tid] = all;
      s_red[nthr + tid] = pre;
      __syncthreads();
      if (tid < ncols && e < E) {
        int32_t a = 0, p = 0;
        for (int q = 0; q < nparts; ++q) {
          a += s_red[q * ncols + tid];
          p += s_red[nthr + q * ncols + tid];
        }
        s_counts[e] = a;
        s_pre[e] = p;
      }
      __syncthreads();
    }
  }
  const int nq = U - u0 < nw ? (U - u0 > 0 ? U - u0 : 0) : nw;   // units of this block
  for (int e = tid; e < E; e += nthr) {
    int32_t p = 0;
    for (int32_t u = hb0 * nw1; u < u0; ++u) p += hv.unit_hist[(int64_t)u * E + e];
    s_pre[e] += p;
    for (int q = 0; q < nq; ++q) s_cursor[q * E + e] = hv.unit_hist[(int64_t)(u0 + q) * E + e];
  }
  __syncthreads();

  // 2. Exclusive scans over experts of the aligned segment lengths and of the
  //    pad rows: a contiguous chunk per thread, a shuffle scan inside each
  //    wavefront, then the wavefront totals.
  const int per = (E + nthr - 1) / nthr;
  const int b0 = tid * per;
  int32_t loc_a = 0, loc_p = 0;
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < E) {
      const int32_t c = s_counts[e];
      const int32_t padded = (c + A - 1) / A * A;
      loc_a += padded;
      loc_p += padded - c;
    }
  }
  int32_t inc_a = loc_a, inc_p = loc_p;
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t ta = __shfl_up(inc_a, off);
    const int32_t tp = __shfl_up(inc_p, off);
    if (lane >= off) {
      inc_a += ta;
      inc_p += tp;
    }
  }
  if (lane == kWave - 1) {
    s_wave_tot[0][w] = inc_a;
    s_wave_tot[1][w] = inc_p;
  }
  __syncthreads();
  int32_t ex_a = inc_a - loc_a, ex_p = inc_p - loc_p;
  for (int q = 0; q < w; ++q) {
    ex_a += s_wave_tot[0][q];
    ex_p += s_wave_tot[1][q];
  }
  // Pad rows below the capacity: all of them, unless the capacity falls
  // inside expert e's segment; then the pads of the experts before e plus
  // those of e's pad rows that lie below it. Exactly one thread writes.
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < E) {
      const int32_t c = s_counts[e];
      const int32_t padded = (c + A - 1) / A * A;
      s_offs[e] = ex_a;
      s_padoff[e] = ex_p;
      if ((int64_t)ex_a <= d.cap && d.cap < (int64_t)ex_a + padded) {
        const int64_t first_pad = (int64_t)ex_a + c;
        s_pads_live = ex_p + (int32_t)(d.cap > first_pad ? d.cap - first_pad : 0);
      }
      ex_a += padded;
      ex_p += padded - c;
    }
  }
  if (tid == nthr - 1) {
    s_offs[E] = ex_a;
    s_padoff[E] = ex_p;
    if ((int64_t)ex_a <= d.cap) s_pads_live = ex_p;
  }
  __syncthreads();

  // 3. Block 0 publishes counts, offsets and the header, with the length of
  //    each stream's run list (the valid routes of its chunks).
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += nthr) {
      hv.offsets[e] = s_offs[e];
      hv.pad_offsets[e] = s_padoff[e];
      if (user_offsets) user_offsets[e] = s_offs[e];
      if (e < E) {
        hv.counts[e] = s_counts[e];
        user_counts[e] = s_counts[e];
      }
    }
    if (tid < kRunXcds) s_live[tid] = 0;
    __syncthreads();
    int32_t f = 0;
    for (int32_t u = tid; u < U; u += nthr) {
      const int32_t fl = hv.unit_flags[u];
      f |= fl & 1;
      atomicAdd(&s_live[(u / ru) % kRunXcds], fl >> 1);
    }
    const int any_bad = __syncthreads_or(f);
    if (tid < kRunXcds) hv.header->stream_live[tid] = s_live[tid];
    if (tid == 0) {
      HandleHeader* h = hv.header;
      const int32_t total = s_offs[E];
      h->status = (any_bad ? EP_STATUS_BAD_EXPERT : 0u) |
                  ((int64_t)total > d.cap ? EP_STATUS_OVERFLOW : 0u);
      h->num_tokens = d.T;
      h->topk = d.K;
      h->num_experts = d.E;
      h->alignment = d.A;
      h->num_units = d.num_units;
      h->recv_capacity = d.cap;
      h->total = total;
      h->pads_live = s_pads_live;
      h->run_units = ru;
      h->magic = kHandleMagic;
    }
  }

  // 4. Per-wavefront cursors: segment start + routes of earlier units
  //    (turns the own-unit counts kept in LDS into running starts, in place).
  for (int e = tid; e < E; e += nthr) {
    int32_t run = s_offs[e] + s_pre[e];
    for (int q = 0; q < nq; ++q) {
      const int32_t c = s_cursor[q * E + e];
      s_cursor[q * E + e] = run;
      run += c;
    }
    s_cursor[nq * E + e] = run;           // end of this block's units
  }
  __syncthreads();

  // 4b. Run entries, when chunks of run_units units line up with this
  //     block's units: chunk q's routes to expert e hold rows
  //     [cursor(first unit of q), cursor(first unit of q + 1)), of which those
  //     below the capacity are kept; an exclusive scan of the kept counts over
  //     experts gives each run's start among the chunk's entries. The block's
  //     chunks are handled side by side: chunk q by the run_units wavefronts
  //     that own its units (thread group q), with two block barriers in all.
  const int nchb = run_units > 0 ? (nq + run_units - 1) / run_units : 0;
  if (run_units > 0) {
    const int q = w / run_units;                 // this thread's chunk
    const int gsz = run_units * kWave;           // threads of a group
    const int gt = tid - q * gsz;
    const bool active = q < nchb;
    const int qa = q * run_units;
    const int qb = qa + run_units < nq ? qa + run_units : nq;
    const int per_g = (E + gsz - 1) / gsz;
    const int b0g = gt * per_g;
    int32_t loc = 0, vb = 0, vo = 0;
    if (active) {
      for (int i = 0; i < per_g; ++i) {
        const int e = b0g + i;
        if (e < E) {
          const int32_t first = s_cursor[qa * E + e];
          const int32_t cnt = s_cursor[qb * E + e] - first;
          const int64_t room = d.cap - (int64_t)first;
          loc += room <= 0 ? 0 : (room < cnt ? (int32_t)room : cnt);
        }
      }
      // the chunk's start in its stream's list: the valid routes of the
      // stream's earlier chunks (whole chunks of ru units each), and the
      // chunk's own valid routes
      const int32_t c = (u0 + qa) / ru;
      if (scanned) {
        if (gt == 0) vb = hv.unit_flags[U + c];    // from the column scan
      } else {
        const int32_t nprev = c / kRunXcds * ru;
        for (int32_t i = gt; i < nprev; i += gsz) {
          const int32_t cp = c % kRunXcds + kRunXcds * (i / ru);
          vb += hv.unit_flags[cp * ru + i % ru] >> 1;
        }
      }
      for (int32_t i = gt; i < qb - qa; i += gsz) vo += hv.unit_flags[u0 + qa + i] >> 1;
    }
    int32_t inc = loc;
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
      vb += __shfl_xor(vb, off);
      vo += __shfl_xor(vo, off);
    }
    if (lane == kWave - 1) s_wave_tot[0][w] = inc;
    if (lane == 0) {
      s_wave_vb[w] = vb;
      s_wave_vo[w] = vo;
    }
    __syncthreads();
    if (active) {
      int32_t ex = inc - loc;
      for (int qq = q * run_units; qq < w; ++qq) ex += s_wave_tot[0][qq];
      for (int i = 0; i < per_g; ++i) {
        const int e = b0g + i;
        if (e < E) {
          const int32_t first = s_cursor[qa * E + e];
          const int32_t cnt = s_cursor[qb * E + e] - first;
          const int64_t room = d.cap - (int64_t)first;
          s_rbase[q * E + e] = ex;
          ex += room <= 0 ? 0 : (room < cnt ? (int32_t)room : cnt);
        }
      }
      if (gt == gsz - 1) s_run_tot[q] = ex;
      if (gt == 0) {
        int32_t sb = 0, so = 0;
        for (int qq = q * run_units; qq < (q + 1) * run_units; ++qq) {
          sb += s_wave_vb[qq];
          so += s_wave_vo[qq];
        }
        s_run_base[q] = sb;
        s_run_valid[q] = so;
      }
    }
    __syncthreads();
  }
  const int64_t scap = run_stream_cap(U);

  // 5. Stable slots: the unit's start row of the route's expert plus the
  //    route's rank among the unit's routes of that expert.
  if (my_unit < U) {
    const int32_t* cursor = s_cursor + w * E;
    static_for<kPrepRounds>([&](auto i) {
      const int64_t s = base + i * kWave + lane;
      if (s < routes) {
        const int32_t p = pk[i];
        const bool valid = p >= 0;
        const int32_t e = p & ((1 << kKeyBits) - 1);
        const int64_t row = valid ? (int64_t)cursor[e] + (p >> kKeyBits) : 0;
        const bool keep = valid && row < d.cap;
        hv.slot[s] = keep ? (int32_t)row : -1;
        if (keep) hv.row_src[row] = (int32_t)s;
        if (keep && run_units > 0) {
          const int q = w / run_units;
          const int32_t first = s_cursor[q * run_units * E + e];
          const int32_t chunk = (u0 + q * run_units) / run_units;
          hv.runs[(chunk % kRunXcds) * scap + s_run_base[q] + s_rbase[q * E + e] +
                  ((int32_t)row - first)] = RunEntry{(int32_t)row, (int32_t)s};
        }
      }
    });
  }
  // a chunk's valid routes dropped past the capacity leave empty entries
  for (int q = 0; q < nchb; ++q) {
    const int32_t chunk = (u0 + q * run_units) / run_units;
    for (int32_t i = s_run_tot[q] + tid; i < s_run_valid[q]; i += nthr)
      hv.runs[(chunk % kRunXcds) * scap + s_run_base[q] + i] = RunEntry{-1, -1};
  }

  // 6. Pad rows: row_src = -1 and the list of live pad rows (ascending, so
  //    the live ones form a prefix). One wavefront per expert, spread over
  //    every wavefront of the grid; its lanes cover the expert's pad rows.
  for (int e = blockIdx.x * nw + w; e < E; e += gridDim.x * nw) {
    const int64_t lo = (int64_t)s_offs[e] + s_counts[e];
    const int64_t hi_full = s_offs[e + 1];
    const int64_t hi = hi_full < d.cap ? hi_full : d.cap;
    const int32_t p0 = s_padoff[e];
    for (int64_t r = lo + lane; r < hi; r += kWave) {
      hv.row_src[r] = -1;
      hv.pad_rows[p0 + (r - lo)] = (int32_t)r;
    }
  }
}

// Single-block prepare for small routings, where the two-kernel form is bound
// by its launches. The kFusedWaves wavefronts of one block each take a
// contiguous run of at most kPrepRounds 64-route rounds (so wavefront order is
// route order), load their ids once and count them into a wavefront-private
// LDS row; the block turns the rows into counts, aligned offsets and
// per-wavefront cursors; each wavefront then hands out rows from its ids
// exactly as the two-kernel form does. With runs_here it also writes the run
// entries (each one-unit chunk alone in its stream's list), so that the whole
// prepare is one launch; the histograms stay in LDS. Measured on the MI355X it
// beats the two launches up to a few thousand routes; one CU is too slow
// beyond.
constexpr int kFusedWaves = 16;

__global__ void __launch_bounds__(kFusedWaves * kWave)
prepare_fused_kernel(Dims d, HandleView hv, const int64_t* __restrict__ topk_idx,
                     int32_t* __restrict__ user_counts, int32_t* __restrict__ user_offsets,
                     int nbits, int32_t ru, int32_t runs_here) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t s_wave_tot[2][kFusedWaves];
  __shared__ int32_t s_pads_live;
  __shared__ int32_t s_bad;
  constexpr int nthr = kFusedWaves * kWave;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int E = d.E;
  const int32_t A = d.A;
  int32_t* s_cur = lds;                          // [kFusedWaves][E]: counts, then cursors
  int32_t* s_counts = s_cur + kFusedWaves * E;   // [E]
  int32_t* s_offs = s_counts + E;                // [E+1]
  int32_t* s_padoff = s_offs + E + 1;            // [E+1]
  // with runs_here: per chunk (one unit each, at most kRunXcds of them), each
  // expert's first row and its run's start among the chunk's entries
  int32_t* s_cfirst = s_padoff + E + 1;          // [kRunXcds][E]
  int32_t* s_crb = s_cfirst + kRunXcds * E;      // [kRunXcds][E]
  __shared__ int32_t s_ckept[kRunXcds];
  __shared__ int32_t s_cvalid[kRunXcds];

  for (int i = tid; i < kFusedWaves * E; i += nthr) s_cur[i] = 0;
  if (tid == 0) {
    s_bad = 0;
    s_pads_live = 0;
  }
  __syncthreads();

  // 1. Per-wavefront histograms of this wavefront's rounds; the ids stay in
  //    registers for step 5.
  const int64_t routes = d.T * d.K;
  const int32_t n_rounds = (int32_t)((routes + kWave - 1) / kWave);
  // a power of two (<= kPrepRounds), so that each 8-round unit is the rounds
  // of whole wavefronts
  int32_t per_wave = 1;
  while (per_wave * kFusedWaves < n_rounds) per_wave *= 2;
  const int32_t ra = min(n_rounds, w * per_wave);
  const int32_t nr = min(n_rounds, ra + per_wave) - ra;
  const int64_t base = (int64_t)ra * kWave;
  int32_t* hist = s_cur + w * E;
  int64_t ids[kPrepRounds];
  static_for<kPrepRounds>([&](auto i) {
    const int64_t s = base + i * kWave + lane;
    ids[i] = (i < nr && s < routes) ? topk_idx[s] : -1;
  });
  bool bad_any = false;
  static_for<kPrepRounds>([&](auto i) {
    if (i < nr) {
      const int64_t id = ids[i];
      const bool valid = id >= 0 && id < E;
      const bool bad = !valid && id != -1;
      bad_any |= wave_ballot(bad) != 0;
      const uint32_t key = valid ? (uint32_t)id : 0u;
      const uint64_t peers = match_peers(key, valid, nbits);
      if (valid && lane == __ffsll((unsigned long long)peers) - 1)
        atomicAdd(&hist[key], (int32_t)__popcll(peers));
    }
  });
  if (bad_any && lane == 0) s_bad = 1;
  __syncthreads();

  // 2. Counts, and each row turned into the routes of earlier wavefronts.
  for (int e = tid; e < E; e += nthr) {
    int32_t run = 0;
    for (int q = 0; q < kFusedWaves; ++q) {
      const int32_t c = s_cur[q * E + e];
      s_cur[q * E + e] = run;
      run += c;
    }
    s_counts[e] = run;
  }
  __syncthreads();

  // 3. Exclusive scans over experts of the aligned segment lengths and of the
  //    pad rows (a contiguous chunk per thread, a shuffle scan inside each
  //    wavefront, then the wavefront totals), and the live pad rows.
  const int per = (E + nthr - 1) / nthr;
  const int b0 = tid * per;
  int32_t loc_a = 0, loc_p = 0;
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < E) {
      const int32_t c = s_counts[e];
      const int32_t padded = (c + A - 1) / A * A;
      loc_a += padded;
      loc_p += padded - c;
    }
  }
  int32_t inc_a = loc_a, inc_p = loc_p;
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t ta = __shfl_up(inc_a, off);
    const int32_t tp = __shfl_up(inc_p, off);
    if (lane >= off) {
      inc_a += ta;
      inc_p += tp;
    }
  }
  if (lane == kWave - 1) {
    s_wave_tot[0][w] = inc_a;
    s_wave_tot[1][w] = inc_p;
  }
  __syncthreads();
  int32_t ex_a = inc_a - loc_a, ex_p = inc_p - loc_p;
  for (int q = 0; q < w; ++q) {
    ex_a += s_wave_tot[0][q];
    ex_p += s_wave_tot[1][q];
  }
  for (int i = 0; i < per; ++i) {
    const int e = b0 + i;
    if (e < E) {
      const int32_t c = s_counts[e];
      const int32_t padded = (c + A - 1) / A * A;
      s_offs[e] = ex_a;
      s_padoff[e] = ex_p;
      if ((int64_t)ex_a <= d.cap && d.cap < (int64_t)ex_a + padded) {
        const int64_t first_pad = (int64_t)ex_a + c;
        s_pads_live = ex_p + (int32_t)(d.cap > first_pad ? d.cap - first_pad : 0);
      }
      ex_a += padded;
      ex_p += padded - c;
    }
  }
  if (tid == nthr - 1) {
    s_offs[E] = ex_a;
    s_padoff[E] = ex_p;
    if ((int64_t)ex_a <= d.cap) s_pads_live = ex_p;
  }
  __syncthreads();

  // 4. Publish counts, offsets and the header; cursors = segment start +
  //    routes of earlier wavefronts.
  for (int e = tid; e <= E; e += nthr) {
    hv.offsets[e] = s_offs[e];
    hv.pad_offsets[e] = s_padoff[e];
    if (user_offsets) user_offsets[e] = s_offs[e];
    if (e < E) {
      hv.counts[e] = s_counts[e];
      user_counts[e] = s_counts[e];
    }
  }
  if (tid == 0) {
    HandleHeader* h = hv.header;
    const int32_t total = s_offs[E];
    h->status = (s_bad ? EP_STATUS_BAD_EXPERT : 0u) |
                ((int64_t)total > d.cap ? EP_STATUS_OVERFLOW : 0u);
    h->num_tokens = d.T;
    h->topk = d.K;
    h->num_experts = d.E;
    h->alignment = d.A;
    h->num_units = d.num_units;
    h->recv_capacity = d.cap;
    h->total = total;
    h->pads_live = s_pads_live;
    h->run_units = ru;
    h->magic = kHandleMagic;
  }
  // the run lists' lengths: set below with runs_here, else by the run-entry
  // kernel that follows (no route: every list stays empty)
  if (tid < kRunXcds && !runs_here) hv.header->stream_live[tid] = 0;
  for (int i = tid; i < kFusedWaves * E; i += nthr) s_cur[i] += s_offs[i % E];
  __syncthreads();

  // 4b. Run entries (runs_here): the routing has at most 8 units and prepare
  //     cuts it into one-unit chunks, so chunk q is the rounds of wavefronts
  //     [q wpc, (q + 1) wpc) and stream q's whole list. Its routes to expert
  //     e hold rows [cursor of its first wavefront, cursor of the next
  //     chunk's), of which those below the capacity are kept; wavefront q
  //     scans the kept counts over experts.
  const int32_t nch = (int32_t)((routes + kUnitRoutes - 1) / kUnitRoutes);
  const int wpc = kPrepRounds / per_wave;
  if (runs_here) {
    if (w < nch) {
      const int q = w;
      int32_t run = 0, valid = 0;
      for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int32_t kept = 0;
        if (e < E) {
          const int32_t first = s_cur[q * wpc * E + e];
          const int32_t next = (q + 1) * wpc < kFusedWaves ? s_cur[(q + 1) * wpc * E + e]
                                                         : s_offs[e] + s_counts[e];
          const int64_t room = d.cap - (int64_t)first;
          const int32_t cnt = next - first;
          kept = room <= 0 ? 0 : (room < cnt ? (int32_t)room : cnt);
          valid += cnt;
          s_cfirst[q * E + e] = first;
        }
        int32_t inc = kept;
        for (int off = 1; off < kWave; off <<= 1) {
          const int32_t t = __shfl_up(inc, off);
          if (lane >= off) inc += t;
        }
        if (e < E) s_crb[q * E + e] = run + inc - kept;
        run += __shfl(inc, kWave - 1);
      }
      for (int off = kWave / 2; off > 0; off >>= 1) valid += __shfl_xor(valid, off);
      if (lane == 0) {
        s_ckept[q] = run;
        s_cvalid[q] = valid;
      }
    }
    __syncthreads();
    if (tid < kRunXcds) hv.header->stream_live[tid] = tid < nch ? s_cvalid[tid] : 0;
  }
  const int64_t scap = run_stream_cap(d.num_units);

  // 5. Stable slots, round by round in route order: the lowest lane of each
  //    distinct id claims popc(peers) rows from the wavefront's cursor; every
  //    peer adds its rank among earlier lanes.
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  static_for<kPrepRounds>([&](auto i) {
    if (i < nr) {
      const int64_t id = ids[i];
      const bool valid = id >= 0 && id < E;
      const uint32_t key = valid ? (uint32_t)id : 0u;
      const uint64_t peers = match_peers(key, valid, nbits);
      const int leader = valid ? __ffsll((unsigned long long)peers) - 1 : lane;
      int32_t first = 0;
      if (valid && lane == leader) first = atomicAdd(&hist[key], (int32_t)__popcll(peers));
      first = __shfl(first, leader);
      const int64_t s = base + i * kWave + lane;
      if (s < routes) {
        const int64_t row = (int64_t)first + __popcll(peers & lanes_below);
        const bool keep = valid && row < d.cap;
        hv.slot[s] = keep ? (int32_t)row : -1;
        if (keep) hv.row_src[row] = (int32_t)s;
        if (keep && runs_here) {
          const int q = (int)(s / kUnitRoutes);
          hv.runs[(int64_t)q * scap + s_crb[q * E + key] +
                  ((int32_t)row - s_cfirst[q * E + key])] = RunEntry{(int32_t)row, (int32_t)s};
        }
      }
    }
  });

  // a chunk's valid routes dropped past the capacity leave empty entries
  if (runs_here)
    for (int q = 0; q < nch; ++q)
      for (int32_t i = s_ckept[q] + tid; i < s_cvalid[q]; i += nthr)
        hv.runs[(int64_t)q * scap + i] = RunEntry{-1, -1};

  // 6. Pad rows: row_src = -1 and the ascending list of live pad rows.
  for (int e = w; e < E; e += kFusedWaves) {
    const int64_t lo = (int64_t)s_offs[e] + s_counts[e];
    const int64_t hi_full = s_offs[e + 1];
    const int64_t hi = hi_full < d.cap ? hi_full : d.cap;
    const int32_t p0 = s_padoff[e];
    for (int64_t r = lo + lane; r < hi; r += kWave) {
      hv.row_src[r] = -1;
      hv.pad_rows[p0 + (r - lo)] = (int32_t)r;
    }
  }
}

// ---------------------------------------------------------------------------
// prepare: run entries
// ---------------------------------------------------------------------------

// Run entries (after the slot map is final). One block per chunk of ru
// units: the chunk's routes to expert e hold a contiguous run of e's rows
// (rows of a segment follow route order, and a chunk's routes are
// consecutive), starting at the smallest of them. A route's entry goes to the
// count of the chunk's routes of lower experts plus its row's offset in its
// run, so the chunk's entries are in ascending row order; its valid routes
// dropped past the capacity then leave empty entries. The chunk's entries
// start, in the list of stream c mod 8, after the valid routes of the
// stream's earlier chunks (read from the units' flag words). With
// write_live (routings of at most 8 units, prepared by the one-block kernel,
// which writes no unit flags: each stream then has at most one chunk, whose
// entries start its list) the block also publishes its stream's list length.
constexpr int kRunThreads = 1024;

__global__ void __launch_bounds__(kRunThreads)
prepare_runs_kernel(Dims d, HandleView hv, const int64_t* __restrict__ topk_idx, int32_t ru,
                    int32_t write_live, int32_t scanned) {
  extern __shared__ int32_t s_run[];                // base[E] (counts first), first[E]
  __shared__ int32_t s_wave_tot[kRunThreads / kWave];
  __shared__ int32_t s_total;
  __shared__ int32_t s_valid;
  __shared__ int32_t s_sbase;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & (kWave - 1), w = tid / kWave;
  const int E = d.E;
  int32_t* s_base = s_run;
  int32_t* s_first = s_run + E;
  const int32_t c = blockIdx.x;
  const int64_t CK = (int64_t)ru * kUnitRoutes;
  const int64_t routes = d.T * (int64_t)d.K;
  const int64_t s0 = (int64_t)c * CK;
  const int64_t s1 = s0 + CK < routes ? s0 + CK : routes;
  const int n = (int)(s1 - s0);
  for (int e = tid; e < E; e += nthr) {
    s_base[e] = 0;
    s_first[e] = 0x7FFFFFFF;
  }
  if (tid == 0) {
    s_valid = 0;
    s_sbase = 0;
  }
  __syncthreads();
  // the chunk's start in its stream's list
  if (!write_live && scanned) {
    if (tid == 0) atomicAdd(&s_sbase, hv.unit_flags[d.num_units + c]);   // from the column scan
  } else if (!write_live) {
    const int32_t nprev = c / kRunXcds * ru;
    int32_t vb = 0;
    for (int32_t i = tid; i < nprev; i += nthr)
      vb += hv.unit_flags[(c % kRunXcds + kRunXcds * (i / ru)) * ru + i % ru] >> 1;
    for (int off = kWave / 2; off > 0; off >>= 1) vb += __shfl_xor(vb, off);
    if (lane == 0 && vb != 0) atomicAdd(&s_sbase, vb);
  }
  int32_t nv = 0;
  for (int i = tid; i < n; i += nthr) {
    const int64_t id = topk_idx[s0 + i];
    nv += (id >= 0 && id < E) ? 1 : 0;
    const int32_t sl = hv.slot[s0 + i];
    if (sl >= 0) {
      atomicAdd(&s_base[id], 1);
      atomicMin(&s_first[id], sl);
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) nv += __shfl_xor(nv, off);
  if (lane == 0 && nv != 0) atomicAdd(&s_valid, nv);
  __syncthreads();
  // exclusive scan of the counts over experts, in place: a contiguous block
  // of experts per thread, a shuffle scan per wavefront, then wave totals
  const int per = (E + nthr - 1) / nthr;
  const int b0 = tid * per;
  int32_t loc = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < E) loc += s_base[b0 + i];
  int32_t inc = loc;
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == kWave - 1) s_wave_tot[w] = inc;
  __syncthreads();
  int32_t ex = inc - loc;
  for (int q = 0; q < w; ++q) ex += s_wave_tot[q];
  for (int i = 0; i < per; ++i) {
    if (b0 + i < E) {
      const int32_t cnt = s_base[b0 + i];
      s_base[b0 + i] = ex;
      ex += cnt;
    }
  }
  if (tid == nthr - 1) s_total = ex;
  __syncthreads();
  const int total = s_total;
  RunEntry* list = hv.runs + (int64_t)(c % kRunXcds) * run_stream_cap(d.num_units) + s_sbase;
  for (int i = tid; i < n; i += nthr) {
    const int32_t sl = hv.slot[s0 + i];
    if (sl >= 0) {
      const int e = (int)topk_idx[s0 + i];
      list[s_base[e] + (sl - s_first[e])] = RunEntry{sl, (int32_t)(s0 + i)};
    }
  }
  for (int i = total + tid; i < s_valid; i += nthr) list[i] = RunEntry{-1, -1};
  if (write_live && tid == 0) {
    hv.header->stream_live[c] = s_valid;
    if (c == 0)
      for (int x = (int)gridDim.x; x < kRunXcds; ++x) hv.header->stream_live[x] = 0;
  }
}

// ---------------------------------------------------------------------------
// row vectors and tunables
// ---------------------------------------------------------------------------

// 16 bytes per lane (8 bf16 or fp16, or 4 fp32); a wavefront moves 1 KiB per
// instruction.
typedef uint32_t row16_t __attribute__((ext_vector_type(4)));

// Launch shapes and cache policy, as measured on the MI355X.
//
// Output rows are written once, so every payload kernel stores them with the
// streaming store below (non-temporal, written through the L2): it keeps one
// op's dirty lines from being written back during the next op. The reduce
// streams its input rows through once and loads them non-temporally too; with
// plain loads its rows fill the caches that the next run-entry copy needs for
// its token rows (that copy measured 23% slower). Token rows, which several
// wavefronts or routes share, are loaded with the default (temporal) policy.
constexpr bool kScatterNtStore = true;
constexpr bool kScatterNtLoad = false;
constexpr bool kReduceNtStore = true;
constexpr bool kReduceNtLoad = true;
// The scatter (the fallback copy for sizes past the run copy's 32-bit piece
// indices): two 1 KiB column blocks per work item; rows over 8 KiB take the
// plain unit order on 64 blocks per CU, shorter rows the interleaved order
// (token and pad units spread evenly over the grid) on 32 blocks per CU.
constexpr int kScatterCH = 2;
constexpr int kScatterBlocksPerCU = 64;
constexpr int64_t kScatterIlvMaxRow = 8192;
constexpr int kScatterIlvBlocksPerCU = 32;
// The reduce's grid cap, in blocks per CU.
constexpr int kBlocksPerCU = 128;
// The token-group weighted backward's grid, in blocks per CU.
constexpr int kBwdBlocksPerCU = 16;

namespace {

template <bool NT>
__device__ __forceinline__ row16_t load_row16(const row16_t* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

// Streaming stores write through the XCD's L2: non-temporal at system scope
// (cache-policy bits sc0 sc1 nt of the CDNA3/CDNA4 vector memory
// instructions). A plain non-temporal store (nt alone) leaves its lines
// dirty in the L2 until they are evicted, where they push out rows that are
// still to be read; measured on the MI355X, the dsv3 dispatch by run entries
// takes 118 µs with the write-through form against 125 µs (its token rows
// are then read from HBM once), and no op is slower. The compiler emits no
// such store from C++, so it is written out. A store of more than 64 bits of
// data needs two wait states on the gfx940 family (gfx950 included) before a
// VALU instruction may overwrite its data registers, and the compiler inserts
// none after an asm statement: `s_nop 1` gives both. With one (`s_nop 0`) a
// GPU test saw the next loop step's index stored in place of the data.
__device__ __forceinline__ void store_stream16(row16_t* p, row16_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" ::"v"(p), "v"(v)
               : "memory");
}

template <bool NT>
__device__ __forceinline__ void store_row16(row16_t* p, row16_t v) {
  if constexpr (NT) {
    store_stream16(p, v);
  } else {
    *p = v;
  }
}

// The reduce's blocks: two wavefronts each. Its wavefronts mostly handle one
// item and exit, and measured on the MI355X small blocks start faster than
// blocks of 4 or more wavefronts at the same wavefronts per CU.
constexpr int kBlock = 128;

// Lanes past the end of a row (a ragged last column block) load the row's
// last vector instead, so every load is unconditional and never reads out of
// bounds; their stores are skipped. No register is zero-filled ahead of a
// load, which would make the compiler wait for all loads in flight.

// Marks the loaded registers as used, so the compiler waits for the loads
// once here instead of before every conditional store that follows.
template <int N>
__device__ __forceinline__ void consume(const row16_t (&buf)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" ::"v"(buf[j]));
}

// Index of this wavefront among all wavefronts of the grid, as a scalar.
__device__ __forceinline__ int64_t wave_index() {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  return (int64_t)blockIdx.x * (blockDim.x / kWave) + w;
}

// fp32 -> fp16 bits: the hardware conversion rounds to nearest even and keeps
// fp16 subnormals; any NaN -> 0x7E00. The fp32 value is first made opaque to
// the compiler: otherwise it may fold the multiply or fused multiply-add that
// produced it into one mixed-precision instruction (v_fma_mixlo_f16) that
// rounds the exact result straight to fp16, skipping the fp32 rounding the
// result is defined by.
__device__ __forceinline__ uint32_t rne_f16(float f) {
  asm("" : "+v"(f));
  if (__builtin_isnan(f)) return 0x7E00u;
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f));
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(bits16)));
}

// fp32 result bits: the value itself, any NaN -> 0x7FC00000.
__device__ __forceinline__ uint32_t canon_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : u;
}

// Payload element types. A 16-byte vector holds N elements; get<I> widens
// element I exactly to fp32 and pack rounds N fp32 values once to the type.
template <int DT>
struct Payload;

template <>
struct Payload<EP_DTYPE_BF16> {
  static constexpr int N = 8;
  template <int I>
  __device__ static __forceinline__ float get(const row16_t& v) {
    return (I & 1) ? bf16_hi(v[I >> 1]) : bf16_lo(v[I >> 1]);
  }
  __device__ static __forceinline__ row16_t pack(const float (&a)[N]) {
    row16_t o;
    static_for<4>([&](auto q) {
      constexpr int i = q;
      o[i] = rne_bf16(a[2 * i]) | (rne_bf16(a[2 * i + 1]) << 16);
    });
    return o;
  }
};

template <>
struct Payload<EP_DTYPE_FP16> {
  static constexpr int N = 8;
  template <int I>
  __device__ static __forceinline__ float get(const row16_t& v) {
    return f16_to_f32((I & 1) ? (v[I >> 1] >> 16) : (v[I >> 1] & 0xFFFFu));
  }
  __device__ static __forceinline__ row16_t pack(const float (&a)[N]) {
    row16_t o;
    static_for<4>([&](auto q) {
      constexpr int i = q;
      o[i] = rne_f16(a[2 * i]) | (rne_f16(a[2 * i + 1]) << 16);
    });
    return o;
  }
};

template <>
struct Payload<EP_DTYPE_FP32> {
  static constexpr int N = 4;
  template <int I>
  __device__ static __forceinline__ float get(const row16_t& v) {
    return __uint_as_float(v[I]);
  }
  __device__ static __forceinline__ row16_t pack(const float (&a)[N]) {
    row16_t o;
    static_for<4>([&](auto q) {
      constexpr int i = q;
      o[i] = canon_f32(a[i]);
    });
    return o;
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// D: dispatch (token rows + weights) and combine_bwd (gradient rows)
// ---------------------------------------------------------------------------

// A 512-thread block (kScatterWaves wavefronts) takes one unit: a group of
// G = 64 / K consecutive tokens (at most 64 routes, one per lane) and one
// column block of CH KiB. The valid routes of the group are ranked with a
// ballot and dealt round-robin to the wavefronts; each wavefront copies the
// block's slice of the token row of each of its routes to the route's
// received row. The token slices of a dense group are read once from memory
// and then from the caches by the wavefronts that share them, and each
// wavefront stores to one row at a time: measured on the MI355X, this writes
// faster than one wavefront storing a token's slice to all of its rows, and
// a sparse group still gives every wavefront its share of the work.
// Pad units are kScatterWaves 1 KiB pieces of live pad rows, zeroed, when pads
// are filled. A bit copy: the payload type only sets the row length.
// Unit order: all token units, then the pad units; or, with `interleave`, the
// token units spread evenly among the pad units (position i of the grid-stride
// sequence is a token unit when floor((i+1)q/n) > floor(iq/n), q token units
// of n). Measured on the MI355X, rows of up to 8 KiB copy faster
// interleaved and longer rows faster in the plain order.
constexpr int kScatterWaves = 8;

template <int CH>
__global__ void __launch_bounds__(kScatterWaves * kWave)
scatter_rows_kernel(Dims d, const HandleHeader* __restrict__ h,
                    const int32_t* __restrict__ slot, const int32_t* __restrict__ pad_rows,
                    uint32_t* status, const row16_t* __restrict__ src4,
                    const float* __restrict__ w, row16_t* __restrict__ dst4,
                    float* __restrict__ dst_w, int interleave) {
  const HandleHeader hh = *h;
  if (!handle_matches(hh, d)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, EP_STATUS_LAYOUT);
    return;
  }
  const int lane = lane_id();
  const int K = d.K;
  const int G = kWave / K;                               // tokens per group
  const int64_t V = d.V;
  constexpr int64_t CB = (int64_t)kWave * CH;
  const int64_t ncb = (V + CB - 1) / CB;                 // column blocks per row
  const int64_t npc = (V + kWave - 1) / kWave;           // 1 KiB pieces per row
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t tok_units = (d.T + G - 1) / G * ncb;
  const ZeroRows zr = zero_rows_of(hh, d);
  const int64_t pad_pieces = zr.n * npc;
  const int64_t n_units = tok_units + (pad_pieces + kScatterWaves - 1) / kScatterWaves;
  const bool weights = w != nullptr && dst_w != nullptr;
  const int64_t routes = d.T * (int64_t)K;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));   // lanes < this one
  const int tok_of_lane = lane / K;                      // token of lane l within a group
  // Unit and piece indices fit 32 bits whenever the buffers fit in memory;
  // the 64-bit divisions stay for a launch where they would not.
  const bool small = n_units < ((int64_t)1 << 31) && pad_pieces < ((int64_t)1 << 31);
  auto udiv = [&](int64_t x, int64_t y) -> int64_t {
    return small ? (int64_t)((uint32_t)x / (uint32_t)y) : x / y;
  };

  for (int64_t i = blockIdx.x; i < n_units; i += gridDim.x) {
    int64_t u = i;
    if (interleave) {
      const int64_t c0 = i * tok_units / n_units;        // token units before i
      const int64_t c1 = (i + 1) * tok_units / n_units;
      u = c1 > c0 ? c0 : tok_units + (i - c1);
    }
    if (u < tok_units) {
      const int64_t g = udiv(u, ncb);
      const int64_t cb = u - g * ncb;
      const int64_t first = g * G * (int64_t)K;          // first route of the group
      const int64_t s = first + lane;
      const int32_t sl = (lane < G * K && s < routes) ? slot[s] : -1;
      const bool valid = sl >= 0;
      const int rank = __builtin_popcountll(wave_ballot(valid) & below);
      uint64_t mine = wave_ballot(valid && (rank % kScatterWaves) == wv);
      const int64_t v0 = cb * CB + lane;
      while (mine) {
        const int l = __ffsll((unsigned long long)mine) - 1;
        mine &= mine - 1;
        const int32_t r = __builtin_amdgcn_readlane(sl, l);
        const int64_t t = g * G + __builtin_amdgcn_readlane(tok_of_lane, l);
        row16_t buf[CH];
        static_for<CH>([&](auto j) {
          const int64_t v = v0 + j * kWave;
          buf[j] = load_row16<kScatterNtLoad>(src4 + t * V + (v < V ? v : V - 1));
        });
        consume(buf);
        static_for<CH>([&](auto j) {
          const int64_t v = v0 + j * kWave;
          if (v < V) store_row16<kScatterNtStore>(dst4 + (int64_t)r * V + v, buf[j]);
        });
        if (cb == 0 && weights && lane == 0) dst_w[r] = w[first + l];
      }
    } else {
      const int64_t pi = (u - tok_units) * kScatterWaves + wv;
      if (pi >= pad_pieces) continue;
      const int64_t p = udiv(pi, npc);
      const int64_t c = pi - p * npc;
      const int64_t r = zero_row(zr, pad_rows, p);
      const int64_t v = c * kWave + lane;
      if (v < V) store_row16<kScatterNtStore>(dst4 + r * V + v, row16_t{0u, 0u, 0u, 0u});
      if (c == 0 && dst_w != nullptr && lane == 0) dst_w[r] = 0.0f;
    }
  }
}

// D over the run entries, for every routing. Block (x, k) = (i mod 8, i div 8)
// of the copy blocks takes stream x's list and in it the step of 8P
// consecutive 1 KiB pieces starting at 8P k, P per wavefront and
// interleaved, so that each step of a block writes 8 consecutive pieces; then
// the steps 8P (k + bps), 8P (k + 2 bps), ... while the stream has pieces
// (bps = blocks per stream). Piece q of a stream is column piece q mod npc
// of the list's entry q div npc. The hardware deals blocks round-robin over
// the eight XCDs, so one stream's blocks share one L2: a chunk's token rows
// are read from memory once and then from that L2, and consecutive blocks
// write consecutive pieces of the chunk's runs (the rows an expert receives
// from the chunk, adjacent in memory). Each block also zeroes its slice of its
// XCD's share of the zero rows (live pads; the tail under the tail policy).
// Blocks are issued in order and, when the grid covers every step once (the
// launcher sizes it for a dense routing, capped), run once and exit, so each
// XCD's write front stays one dense band; measured on the MI355X, runs of
// 128 KiB and more written this way reach 6.5 TB/s against 5.1 TB/s for rows
// in scattered order. A routing with masked routes has shorter lists, read
// from the header on the device: the same grid covers them with fewer steps
// per block, and blocks past the end only zero their pad slice.
//
// The first step's entries are loaded before the header (they lie inside the
// list's capacity whatever it holds), so that the header, entry and token
// loads of a dense routing are two dependent rounds, not three.
//
// npf leading blocks, when the launcher asks for them, first stream the
// token rows through the caches with plain loads: when the rows are few
// (they fit the 256 MB Infinity Cache with room) and each is read by many
// routes, they are then served from there instead of from HBM at the start
// of every chunk. Measured on the MI355X with the caches flushed before the
// op: dsv3 dispatch 139.9 -> 134.7 us, combine_bwd 138.3 -> 129.9 us; with
// two routes per token (mixtral) it costs 7 us instead, so it is not used
// there.
//
// Where the token rows are not streamed, leading blocks instead read the
// run lists, each on the XCD that copies its list and at most
// kRunListBlockBytes of it, so that the copy blocks find their entries in
// their XCD's L2 rather than in HBM after the caches were flushed. Measured
// on the MI355X with the caches flushed before the op: qwen3 dispatch 70.7
// -> 66.4-67.2 us, combine_bwd 67.5 -> 65.3-66.2; mixtral and the masked
// share level, warm runs level; beside the token-row streaming (dsv3) it made
// the cold combine_bwd 6 us slower.
//
// P, the pieces per wavefront, is 4, or 8 for narrow rows with the pad fill.
// Measured on the MI355X with A/B runs on one device (dispatch µs): rows of
// 14 KiB (dsv3) take 121-125 at P = 4 against 131-132 at P = 3 and 135 at
// P = 5, fp32 rows of 28 KiB 252 against 256 at P = 3; rows of 8 KiB
// (mixtral) lose 3-7% at P = 3 or 6; rows of 4 KiB (qwen3) take 58.4 / 54.7
// (dispatch / combine_bwd) at P = 6 against 60.1 / 56.3 at P = 4, and
// 57.4-58.0 / 53.5-53.8 at P = 8 against 59.9-60.6 / 54.3-55.1 at P = 6 on
// warm steps, 68.0-68.3 / 68.2-68.3 against 66.3-66.8 / 64.9-65.5 after a
// cache flush (P = 5 level with 6). A launch-bound routing of 1 KiB rows in
// 16 blocks (T = 256) loses 0.8 µs at P = 6, so the wide steps need a grid
// that fills the device.
constexpr int kRunWaves = 8;
constexpr int kRunPieces = 4;
constexpr int kRunPiecesNarrow = 8;   // rows of kRunNarrowRow pieces or fewer, pads filled
constexpr int64_t kRunNarrowRow = 4;  // 1 KiB pieces
constexpr int64_t kRunNarrowMinBlocks = 2048;
// The copy grid is sized for a dense routing, one step of kRunWaves * P
// pieces per block, and launched whole while that is at most kRunBlocksPerCU
// blocks per CU. A larger grid is capped at kRunCapBlocksPerCU per CU, its
// blocks then taking steps bps apart. Large routings are mostly one GPU's
// share of an expert-parallel layer, where most routes are masked and the
// blocks past a stream's live pieces have no work: they exit at once, but
// they are still dispatched after all the working ones. Measured on the
// MI355X (dispatch µs): the masked share (about one route in eight local,
// 14 KiB rows) takes 140 at 64 blocks per CU, 154 at 96 and 167.5 at 128;
// the hot-expert share, whose live pieces need 1.6 steps a block at 64,
// takes 235 against 225 at 96; dsv3 in fp32 (28 KiB rows, 112 blocks per CU
// when dense) takes 222 whole against 251 at 96 and 265 at 64, where blocks
// of two steps kept two regions of the lists in flight. On the masked share,
// sizing each block's share from the live count on the device, taking the
// next step's entries early, or dispatching the empty blocks among the
// working ones (front and back halves in turn, or each block's steps from
// the live step count) took 141, 142.5, 150 and 140 µs at 64 blocks per CU
// and 178, 167, 189 and 162 at 96 or 128.
constexpr int64_t kRunBlocksPerCU = 128;
constexpr int64_t kRunCapBlocksPerCU = 64;

// Copy blocks per stream for bps_dense one-step blocks.
inline int64_t run_copy_blocks(int64_t bps_dense, int num_cus) {
  if (bps_dense > (int64_t)num_cus * kRunBlocksPerCU / kRunXcds)
    bps_dense = (int64_t)num_cus * kRunCapBlocksPerCU / kRunXcds;
  return bps_dense < 1 ? 1 : bps_dense;
}
// Token rows streamed by leading blocks when they are at most this many bytes
// in all, each row is at least kRunPrefetchMinRow bytes and each token has at
// least kRunPrefetchMinK routes.
constexpr int64_t kRunPrefetchMaxBytes = (int64_t)96 << 20;
constexpr int kRunPrefetchMinK = 4;
constexpr int64_t kRunPrefetchMinRow = 8192;
constexpr int64_t kRunPrefetchBlocks = 2048;
// Run-list bytes one leading block reads, and such blocks per XCD at most.
constexpr int64_t kRunListBlockBytes = (int64_t)64 << 10;
constexpr int64_t kRunListBlocks = 64;

// Sizes of a run-entry copy, computed on the host; every piece index of the
// launch is below 2^32 (the launcher checks), so index arithmetic is 32-bit.
struct RunGeom {
  uint32_t npc;       // 1 KiB pieces per row
  uint32_t bps;       // copy blocks per stream
  uint32_t npf;       // leading blocks that stream the token rows
  uint32_t pf_per;    // 16-byte vectors each lane of a streaming block loads
  uint32_t nlp;       // leading blocks that read the run lists: 0, or a
                      // multiple of kRunXcds when npf is 0
  uint32_t lp_ent;    // entries of each list they read (even, at most scap)
  uint32_t cap_pieces;  // pieces a stream's list can hold: scap * npc
  int64_t scap;       // entries a stream's list can hold
};

namespace {

// A leading block's work (W wavefronts): stream its slice of the token rows
// [T, H] through the caches with plain loads.
template <int W>
__device__ __forceinline__ void stream_token_rows(const Dims& d, const RunGeom& g,
                                                  const row16_t* __restrict__ src4,
                                                  uint32_t wv, uint32_t lane) {
  const int64_t nvec = d.T * d.V;
  const int64_t base = ((int64_t)blockIdx.x * W + wv) * g.pf_per * kWave + lane;
  row16_t acc = row16_t{0u, 0u, 0u, 0u};
  for (uint32_t i = 0; i < g.pf_per; ++i) {
    const int64_t vv = base + (int64_t)i * kWave;
    if (vv < nvec) acc ^= src4[vv];
  }
  asm volatile("" ::"v"(acc));      // the loads are kept (and waited for)
}

// A leading block's work when the token rows are not streamed: its share
// (part of per) of the first lp_ent entries of run list x, 16 bytes (two
// entries) a lane, read into the caches with plain loads.
__device__ __forceinline__ void read_run_list(const RunEntry* __restrict__ runs,
                                              const RunGeom& g, uint32_t x, uint32_t part,
                                              uint32_t per) {
  const row16_t* __restrict__ l4 = reinterpret_cast<const row16_t*>(runs + (int64_t)x * g.scap);
  row16_t acc = row16_t{0u, 0u, 0u, 0u};
  for (uint32_t i = part * blockDim.x + threadIdx.x; i < g.lp_ent / 2; i += per * blockDim.x)
    acc ^= l4[i];
  asm volatile("" ::"v"(acc));      // the loads are kept (and waited for)
}

// The entries of one step: piece base + 8 j + wv of the stream (j < P), its
// column piece and entry; a piece past the list's capacity gets an empty entry
// (and reads entry 0, so every load is in bounds and unconditional).
template <int P>
__device__ __forceinline__ void run_step_entries(const RunEntry* __restrict__ list,
                                                 uint32_t base, uint32_t wv,
                                                 const RunGeom& g, RunEntry (&ent)[P],
                                                 uint32_t (&col)[P]) {
  static_for<P>([&](auto j) {
    const uint32_t q = base + j * kRunWaves + wv;
    const bool in = q < g.cap_pieces;
    const uint32_t qq = in ? q : 0u;
    const uint32_t qe = qq / g.npc;
    col[j] = qq - qe * g.npc;
    ent[j] = list[qe];
    if (!in) ent[j].row = -1;
  });
}

// Copies one step's pieces: those below `pieces` whose entry names a row
// below the capacity and a route of the routing. All token loads are issued
// before the first store.
template <int P>
__device__ __forceinline__ void run_step_copy(const Dims& d, uint32_t base, uint32_t wv,
                                              uint32_t lane, uint32_t pieces, uint32_t routes,
                                              RunEntry (&ent)[P], const uint32_t (&col)[P],
                                              const row16_t* __restrict__ src4,
                                              const float* __restrict__ w,
                                              row16_t* __restrict__ dst4,
                                              float* __restrict__ dst_w) {
  const int64_t V = d.V;
  static_for<P>([&](auto j) {
    if (base + j * kRunWaves + wv >= pieces || (int64_t)ent[j].row >= d.cap ||
        (uint32_t)ent[j].route >= routes)
      ent[j].row = -1;
  });
  row16_t val[P];
  static_for<P>([&](auto j) {
    const uint32_t t = ent[j].row >= 0 ? (uint32_t)ent[j].route / (uint32_t)d.K : 0u;
    const int64_t v = (int64_t)(col[j] * kWave + lane);
    val[j] = load_row16<kScatterNtLoad>(src4 + (int64_t)t * V + (v < V ? v : V - 1));
  });
  // the weights of the pieces that start a row are loaded with the token
  // slices, not after the stores, so that their latency overlaps
  const bool weights = w != nullptr && dst_w != nullptr;
  float wt[P];
  static_for<P>([&](auto j) {
    wt[j] = (weights && ent[j].row >= 0 && col[j] == 0) ? w[ent[j].route] : 0.0f;
  });
  consume(val);
  static_for<P>([&](auto j) {
    const int64_t v = (int64_t)(col[j] * kWave + lane);
    if (ent[j].row >= 0 && v < V)
      store_row16<kScatterNtStore>(dst4 + (int64_t)ent[j].row * V + v, val[j]);
  });
  if (weights && lane == 0) {
    static_for<P>([&](auto j) {
      if (ent[j].row >= 0 && col[j] == 0) dst_w[ent[j].row] = wt[j];
    });
  }
}

}  // namespace

template <int P>
__global__ void __launch_bounds__(kRunWaves * kWave)
run_rows_kernel(Dims d, const HandleHeader* __restrict__ h, const RunEntry* __restrict__ runs,
                const int32_t* __restrict__ pad_rows, uint32_t* status,
                const row16_t* __restrict__ src4, const float* __restrict__ w,
                row16_t* __restrict__ dst4, float* __restrict__ dst_w, RunGeom g) {
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t V = d.V;
  if (blockIdx.x < g.npf) {
    stream_token_rows<kRunWaves>(d, g, src4, wv, lane);
    return;
  }
  if (blockIdx.x < g.nlp) {
    // npf is 0 here and nlp a multiple of kRunXcds, so block i runs on the
    // XCD that copies list i mod kRunXcds
    read_run_list(runs, g, blockIdx.x % kRunXcds, blockIdx.x / kRunXcds, g.nlp / kRunXcds);
    return;
  }
  const uint32_t tb = blockIdx.x - g.npf - g.nlp;
  const uint32_t x = tb % kRunXcds;
  const uint32_t k = tb / kRunXcds;
  const RunEntry* __restrict__ list = runs + (int64_t)x * g.scap;
  constexpr uint32_t kStep = kRunWaves * P;
  // the first step's entries, before the header
  RunEntry ent[P];
  uint32_t col[P];
  run_step_entries<P>(list, k * kStep, wv, g, ent, col);
  const HandleHeader hh = *h;
  if (!handle_matches(hh, d)) {
    if (tb == 0 && threadIdx.x == 0) atomicOr(status, EP_STATUS_LAYOUT);
    return;
  }
  // the list's length (read from the handle itself: indexing the header copy
  // by x would put the copy in private memory), bounded by its capacity; an
  // entry is used only if it names a row below the capacity and a route of
  // the routing
  const uint32_t live = (uint32_t)h->stream_live[x];
  const uint32_t pieces = (live < (uint32_t)g.scap ? live : (uint32_t)g.scap) * g.npc;
  const uint32_t routes = (uint32_t)(d.T * d.K);
  if (k * kStep < pieces)
    run_step_copy<P>(d, k * kStep, wv, lane, pieces, routes, ent, col, src4, w, dst4, dst_w);
  // later steps, when the grid holds fewer blocks than the stream has steps
  for (uint32_t b = (k + g.bps) * kStep; b < pieces; b += g.bps * kStep) {
    RunEntry e2[P];
    uint32_t c2[P];
    run_step_entries<P>(list, b, wv, g, e2, c2);
    run_step_copy<P>(d, b, wv, lane, pieces, routes, e2, c2, src4, w, dst4, dst_w);
  }
  if (d.fill_pads || d.zero_tail) {
    // Zero rows (the live pads, and the tail under the tail policy): their
    // pieces are split into kRunXcds contiguous shares and share x is split
    // over stream x's blocks in order, so the zeros of each XCD are written
    // as one dense band alongside its token runs (two pieces per wavefront
    // and step).
    const ZeroRows zr = zero_rows_of(hh, d);
    const uint32_t all = (uint32_t)zr.n * g.npc;
    const uint32_t share = (all + kRunXcds - 1) / kRunXcds;
    const uint32_t qn = (share + g.bps - 1) / g.bps;
    const uint32_t send = (x + 1) * share < all ? (x + 1) * share : all;
    const uint32_t lo = x * share + k * qn;
    const uint32_t hi = lo + qn < send ? lo + qn : send;
    for (uint32_t p0 = lo + wv; p0 < hi; p0 += 2 * kRunWaves) {
      const uint32_t p1 = p0 + kRunWaves;
      const int64_t r0 = zero_row(zr, pad_rows, p0 / g.npc);
      const int64_t r1 = zero_row(zr, pad_rows, (p1 < hi ? p1 : p0) / g.npc);
      const uint32_t c0 = p0 - (p0 / g.npc) * g.npc;
      const uint32_t c1 = p1 - (p1 / g.npc) * g.npc;
      const int64_t v0 = (int64_t)(c0 * kWave + lane), v1 = (int64_t)(c1 * kWave + lane);
      if (v0 < V) store_row16<kScatterNtStore>(dst4 + r0 * V + v0, row16_t{0u, 0u, 0u, 0u});
      if (c0 == 0 && dst_w != nullptr && lane == 0) dst_w[r0] = 0.0f;
      if (p1 < hi) {
        if (v1 < V)
          store_row16<kScatterNtStore>(dst4 + r1 * V + v1, row16_t{0u, 0u, 0u, 0u});
        if (c1 == 0 && dst_w != nullptr && lane == 0) dst_w[r1] = 0.0f;
      }
    }
  }
}

// The weighted combine's backward over the run entries. For the received
// row r of route s (token t = s / K) with weight w_r:
//   grad_rows[r] = payload(fp32(w_r * g_t))    grad_w[r] = sum_h g_t[h] * y_r[h]
// Block (x, k) of stream x takes the rows of R consecutive entries of x's
// list per step (entries kR, (k + bps)R, ...), their R * npc pieces dealt to
// the block's wavefronts as in the run copy (so the block writes each row's
// pieces as one dense band, and a chunk's token rows are read from memory
// once and then from its XCD's L2). Each piece's share of the dot product is
// a per-lane chain of fused multiply-adds over the piece's elements, then a
// fixed xor butterfly over the 64 lanes; the partials go to LDS, and one
// thread per row sums its npc partials in column order. So the weight
// gradient has the same bits on every run, and each product passes through
// at most N + npc + 5 roundings (N elements per 16-byte vector: N in the
// lane's chain, six in the butterfly, npc - 1 over the pieces). Zero rows
// (pads, and the tail under the tail policy) are zeroed, with their weight
// gradients, in each XCD's share as in the run copy.
//
// With the weight gradient, when fewer than half of the routes hold a row
// (one GPU's share of an expert-parallel layer), the blocks walk the
// received rows in order instead, block b taking rows bR, (b + nb)R, ... and
// skipping the pads: each token row is then read about once either way, and
// the rows of y and of the gradient stream in address order. Same pieces,
// same partial sums, same bits. Measured on the MI355X (µs, warm / cold):
// the masked share 209-212 / 220-222 against 211-212 / 235-236 along the
// run lists, the hot-expert share 377-379 / 386-388 against 394-395 /
// 392-393; dsv3 takes 289 in received order against 248, qwen3 and mixtral
// 5-10% more. The row gradient alone keeps the run lists: with both walks
// in one kernel it ran 4-6 us slower on qwen3 and mixtral.
//
// With the weight gradient a block has four wavefronts, and the grid cap
// doubles, so the waves per CU stay the same: each block step's two barriers
// then hold fewer wavefronts. Measured on the MI355X (µs, warm / cold,
// against eight wavefronts): dsv3 245.4 / 245.0 against 247.3 / 246.5, the
// masked share 206.9 / 219.4 against 210.3 / 221.0, the hot-expert share
// 367.8 / 388.3 against 377.2 / 386.9, qwen3 117.0 / 121.2 against 119.2 /
// 122.6, mixtral 112.9 / 131.3 against 112.2 / 128.5. The row gradient
// alone keeps eight (four made dsv3's 3-8 us slower).
constexpr int kWbwdPieces = 4;                 // pieces per wavefront and round
constexpr int kWbwdRounds = 2;                 // rounds per block step (weight gradient)
constexpr int kWbwdWaves = 4;                  // wavefronts per block (weight gradient)
constexpr int kWbwdBlocksPerCU = 64;           // grid cap (weight gradient)
constexpr int kWbwdMaxPartials = 1024;         // LDS partials of one block step

__host__ __device__ constexpr int wbwd_waves(bool want_w) {
  return want_w ? kWbwdWaves : kRunWaves;
}

template <int DT, bool WANT_W>
__global__ void __launch_bounds__(wbwd_waves(WANT_W) * kWave)
run_wbwd_kernel(Dims d, const HandleHeader* __restrict__ h, const RunEntry* __restrict__ runs,
                const int32_t* __restrict__ pad_rows, uint32_t* status,
                const row16_t* __restrict__ g4, const row16_t* __restrict__ y4,
                const float* __restrict__ rw, row16_t* __restrict__ o4,
                float* __restrict__ grad_w, RunGeom g, uint32_t rows_per_step,
                const int32_t* __restrict__ row_src) {
  using Pl = Payload<DT>;
  constexpr int kW = wbwd_waves(WANT_W);
  __shared__ float s_part[kWbwdMaxPartials];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t V = d.V;
  if (blockIdx.x < g.npf) {
    stream_token_rows<kW>(d, g, g4, wv, lane);
    return;
  }
  const uint32_t tb = blockIdx.x - g.npf;
  const uint32_t x = tb % kRunXcds;
  const uint32_t k = tb / kRunXcds;
  const RunEntry* __restrict__ list = runs + (int64_t)x * g.scap;
  const HandleHeader hh = *h;
  if (!handle_matches(hh, d)) {
    if (tb == 0 && threadIdx.x == 0) atomicOr(status, EP_STATUS_LAYOUT);
    return;
  }
  const uint32_t routes = (uint32_t)(d.T * d.K);
  const uint32_t R = rows_per_step;
  constexpr uint32_t kRound = kW * kWbwdPieces;
  // The walk over `live` entries, this block taking entries kb R, (kb +
  // kstride) R, ...; entry(e) gives entry e. Instantiated once per walk, so
  // that neither tests the walk per piece.
  auto walk = [&](auto entry, uint32_t live, uint32_t kb, uint32_t kstride) {
    for (uint32_t e0 = kb * R; e0 < live; e0 += kstride * R) {
      const uint32_t nrows = live - e0 < R ? live - e0 : R;
      const uint32_t npieces = nrows * g.npc;
      for (uint32_t r0 = 0; r0 < npieces; r0 += kRound) {
        RunEntry ent[kWbwdPieces];
        uint32_t col[kWbwdPieces];
        bool use[kWbwdPieces];
        static_for<kWbwdPieces>([&](auto j) {
          const uint32_t pp = r0 + j * kW + wv;
          const bool in = pp < npieces;
          const uint32_t pq = in ? pp : 0u;
          const uint32_t ei = pq / g.npc;
          col[j] = pq - ei * g.npc;
          ent[j] = entry(e0 + ei);
          use[j] = in && ent[j].row >= 0 && (int64_t)ent[j].row < d.cap &&
                   (uint32_t)ent[j].route < routes;
        });
        row16_t gv[kWbwdPieces], yv[kWbwdPieces];
        float wk[kWbwdPieces];
        static_for<kWbwdPieces>([&](auto j) {
          const uint32_t t = use[j] ? (uint32_t)ent[j].route / (uint32_t)d.K : 0u;
          const int64_t r = use[j] ? (int64_t)ent[j].row : 0;
          const int64_t v = (int64_t)(col[j] * kWave + lane);
          const int64_t vc = v < V ? v : V - 1;
          gv[j] = load_row16<kScatterNtLoad>(g4 + (int64_t)t * V + vc);
          if constexpr (WANT_W) yv[j] = load_row16<kReduceNtLoad>(y4 + r * V + vc);
          wk[j] = rw[r];
        });
        static_for<kWbwdPieces>([&](auto j) {
          const int64_t v = (int64_t)(col[j] * kWave + lane);
          float prod[Pl::N];
          float pd = 0.0f;
          static_for<Pl::N>([&](auto q) {
            constexpr int i = q;
            const float gi = Pl::template get<i>(gv[j]);
            prod[i] = wk[j] * gi;
            if constexpr (WANT_W) pd = __builtin_fmaf(gi, Pl::template get<i>(yv[j]), pd);
          });
          if (use[j] && v < V)
            store_row16<kScatterNtStore>(o4 + (int64_t)ent[j].row * V + v, Pl::pack(prod));
          if constexpr (WANT_W) {
            pd = v < V ? pd : 0.0f;
            for (int off = kWave / 2; off > 0; off >>= 1) pd += __shfl_xor(pd, off);
            const uint32_t pp = r0 + j * kW + wv;
            if (lane == 0 && pp < npieces) s_part[pp] = pd;
          }
        });
      }
      if constexpr (WANT_W) {
        __syncthreads();
        if (threadIdx.x < nrows) {
          const RunEntry e = entry(e0 + threadIdx.x);
          if (e.row >= 0 && (int64_t)e.row < d.cap && (uint32_t)e.route < routes) {
            float sum = 0.0f;
            for (uint32_t c = 0; c < g.npc; ++c) sum += s_part[threadIdx.x * g.npc + c];
            grad_w[e.row] = sum;
          }
        }
        __syncthreads();
      }
    }
  };
  // with the weight gradient, the received rows in order on sparse routings
  // (a pad giving row -1); else the run list
  bool by_rows = false;
  if constexpr (WANT_W) {
    const int64_t rows_total = (int64_t)hh.total < d.cap ? (int64_t)hh.total : d.cap;
    if (2 * (rows_total - (int64_t)hh.pads_live) < (int64_t)routes) {
      by_rows = true;
      walk([&](uint32_t e) -> RunEntry {
        const int32_t s = row_src[e];
        return RunEntry{s >= 0 ? (int32_t)e : -1, s};
      }, (uint32_t)rows_total, tb, g.bps * kRunXcds);
    }
  }
  if (!by_rows) {
    const uint32_t live0 = (uint32_t)h->stream_live[x];
    walk([&](uint32_t e) -> RunEntry { return list[e]; },
         live0 < (uint32_t)g.scap ? live0 : (uint32_t)g.scap, k, g.bps);
  }
  if (d.fill_pads || d.zero_tail) {
    const ZeroRows zr = zero_rows_of(hh, d);
    const uint32_t all = (uint32_t)zr.n * g.npc;
    const uint32_t share = (all + kRunXcds - 1) / kRunXcds;
    const uint32_t qn = (share + g.bps - 1) / g.bps;
    const uint32_t send = (x + 1) * share < all ? (x + 1) * share : all;
    const uint32_t lo = x * share + k * qn;
    const uint32_t hi = lo + qn < send ? lo + qn : send;
    for (uint32_t p0 = lo + wv; p0 < hi; p0 += kW) {
      const int64_t r0 = zero_row(zr, pad_rows, p0 / g.npc);
      const uint32_t c0 = p0 - (p0 / g.npc) * g.npc;
      const int64_t v0 = (int64_t)(c0 * kWave + lane);
      if (v0 < V) store_row16<kScatterNtStore>(o4 + r0 * V + v0, row16_t{0u, 0u, 0u, 0u});
      if (WANT_W && c0 == 0 && lane == 0) grad_w[r0] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// D^T: combine (expert rows -> token rows) and dispatch_bwd
// ---------------------------------------------------------------------------

namespace {

}  // namespace

// Items: (group of G consecutive tokens, 1 KiB column block), G a power of
// two up to 64 / K, so that a group's routes fit one wavefront. Lane l loads
// the slot of the group's route l (one coalesced load) and the wavefront
// walks the group's valid routes in ascending route order, kReduceBatch row
// slices in flight at a time. A token's slices are summed in fp32 in
// ascending k from its first valid one; when its routes end, the sum is
// rounded once to the payload type and stored; a token with no valid route
// gets +0. Everything that steers the walk comes from a ballot, so its
// branches are scalar.
//
// G follows the routing's density, read from the handle header on the
// device: the largest power of two up to T*K / R (R the live valid routes),
// so that a group holds about K valid routes, capped by the launcher (g_max)
// so that the items still fill the grid. A dense routing (G = 1) loads a
// token's K rows at once, as a per-token walk would; a sparse one (masking
// leaves one in eight routes valid) keeps eight slices in flight per
// wavefront instead of about one, and writes its tokens' zero rows from the
// same wavefronts. The first item's G = 1 slots are loaded together with the
// header and reloaded only when G > 1; later items' slots are loaded before
// the current item's stores.
constexpr int kReduceBatch = 8;

template <int KT, bool WEIGHTED, int DT>
__global__ void __launch_bounds__(kBlock)
reduce_rows_kernel(Dims d, const HandleHeader* __restrict__ h,
                   const int32_t* __restrict__ slot, uint32_t* status,
                   const row16_t* __restrict__ src4, const float* __restrict__ rw,
                   const float* __restrict__ g_w, row16_t* __restrict__ dst4,
                   float* __restrict__ dst_w, int g_max) {
  using P = Payload<DT>;
  const int K = KT > 0 ? KT : d.K;
  const int lane = lane_id();
  const int64_t V = d.V;
  const int64_t ncb = (V + kWave - 1) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t routes = d.T * (int64_t)K;
  const int64_t w0 = wave_index();
  // items and their indices fit 32 bits whenever the buffers fit in memory;
  // the 64-bit division stays for a launch where they would not
  const bool small = d.T * ncb + nwaves < ((int64_t)1 << 31);
  auto udiv = [&](int64_t x, int64_t y) -> int64_t {
    return small ? (int64_t)((uint32_t)x / (uint32_t)y) : x / y;
  };
  if (w0 >= d.T * ncb) return;
  // the first token's slots (the G = 1 guess) are loaded with the header
  constexpr bool kUnrolled = KT > 0 && KT <= kReduceBatch;
  int32_t sl1[kUnrolled ? KT : 1];
  if constexpr (kUnrolled) {
    const int64_t t = udiv(w0, ncb);
    static_for<KT>([&](auto k) { sl1[k] = slot[t * KT + k]; });
  }
  const HandleHeader hh = *h;
  if (!handle_matches(hh, d)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, EP_STATUS_LAYOUT);
    return;
  }
  int G = 1;
  {
    const int64_t live = (int64_t)hh.total < d.cap ? (int64_t)hh.total : d.cap;
    const int64_t R = live - (int64_t)hh.pads_live;
    while (2 * G <= g_max && (int64_t)2 * G * (R > 0 ? R : 1) <= routes) G *= 2;
  }

  if constexpr (kUnrolled) {
    if (G == 1) {
      // One token per item, its K routes unrolled at compile time: a dense
      // routing spends less here than on the walk's bookkeeping.
      bool first = true;
      for (int64_t it = w0; it < d.T * ncb; it += nwaves) {
        const int64_t t = udiv(it, ncb);
        const int64_t cb = it - t * ncb;
        const int64_t v = cb * kWave + lane;
        const int64_t vc = v < V ? v : V - 1;
        int32_t sl[KT];
        static_for<KT>([&](auto k) { sl[k] = first ? sl1[k] : slot[t * KT + k]; });
        first = false;
        int32_t mine = -1;
        static_for<KT>([&](auto k) {
          if (lane == k) mine = sl[k];
        });
        // the gathered weight gradient is loaded here and stored after the
        // row loads, so that the row loads do not wait for it
        const bool wgrad = cb == 0 && dst_w != nullptr;
        float gwv = 0.0f;
        if (wgrad && g_w != nullptr && lane < KT && mine >= 0) gwv = g_w[mine];
        float wl = 0.0f;
        if constexpr (WEIGHTED) {
          if (lane < KT && mine >= 0) wl = rw[mine];
        }
        row16_t buf[KT];
        static_for<KT>([&](auto k) {
          if (sl[k] >= 0) buf[k] = load_row16<kReduceNtLoad>(src4 + (int64_t)sl[k] * V + vc);
        });
        // the terms are kept or dropped with selects, not branches, so that
        // every buffer is read on every path and no load is left possibly in
        // flight when the sum is stored
        float acc[P::N];
        bool have = false;
        static_for<KT>([&](auto k) {
          const bool use = sl[k] >= 0;
          float wk = 0.0f;
          if constexpr (WEIGHTED)
            wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k));
          static_for<P::N>([&](auto q) {
            constexpr int i = q;
            const float x = P::template get<i>(buf[k]);
            float term;
            if constexpr (WEIGHTED) {
              term = have ? __builtin_fmaf(wk, x, acc[i]) : wk * x;
            } else {
              term = have ? acc[i] + x : x;
            }
            acc[i] = use ? term : acc[i];
          });
          have |= use;
        });
        if (v < V)
          store_row16<kReduceNtStore>(dst4 + t * V + v,
                                      have ? P::pack(acc) : row16_t{0u, 0u, 0u, 0u});
        if (wgrad && lane < KT) dst_w[t * KT + lane] = gwv;
      }
      return;
    }
  }

  // The walk over groups of G tokens.
  const int GK = G * K;
  const int64_t n_items = (d.T + G - 1) / G * ncb;
  auto group_slot = [&](int64_t item) -> int32_t {
    const int64_t s = udiv(item, ncb) * GK + lane;
    return (lane < GK && s < routes) ? slot[s] : -1;
  };
  if (w0 >= n_items) return;
  int32_t sl_next = group_slot(w0);
  for (int64_t it = w0; it < n_items; it += nwaves) {
    const int64_t g = udiv(it, ncb);
    const int64_t cb = it - g * ncb;
    const int32_t sl = sl_next;
    const int64_t v = cb * kWave + lane;
    const bool vin = v < V;
    const int64_t vc = vin ? v : V - 1;
    const int64_t t0 = g * G;
    const int ntok = (int)((int64_t)G < d.T - t0 ? (int64_t)G : d.T - t0);
    const int64_t s = g * GK + lane;
    // the gathered weight gradient: loaded here, stored after the rows
    const bool wgrad = cb == 0 && dst_w != nullptr;
    float gwv = 0.0f;
    if (wgrad && g_w != nullptr && lane < GK && s < routes && sl >= 0) gwv = g_w[sl];
    float wl = 0.0f;
    if constexpr (WEIGHTED) {
      if (sl >= 0) wl = rw[sl];
    }
    uint64_t vm = wave_ballot(sl >= 0);
    float acc[P::N];
    auto store_tok = [&](int tk, bool have) {
      if (vin)
        store_row16<kReduceNtStore>(dst4 + (t0 + tk) * V + v,
                                    have ? P::pack(acc) : row16_t{0u, 0u, 0u, 0u});
    };
    int cur = -1;     // token (in the group) whose sum is in acc
    int done = 0;     // tokens of the group stored so far
    while (vm) {
      int lb[kReduceBatch];
      row16_t buf[kReduceBatch];
      // the batch's routes (lane numbers, ascending), one load each; the
      // branches are uniform, and a place past the end loads nothing
      static_for<kReduceBatch>([&](auto j) {
        lb[j] = vm ? __ffsll((unsigned long long)vm) - 1 : -1;
        vm &= vm - 1;
        if (lb[j] >= 0) {
          const int32_t r = __builtin_amdgcn_readlane(sl, lb[j]);
          buf[j] = load_row16<kReduceNtLoad>(src4 + (int64_t)r * V + vc);
        }
      });
      static_for<kReduceBatch>([&](auto j) {
        if (lb[j] >= 0) {
          const int tk = lb[j] / K;
          float wk = 0.0f;
          if constexpr (WEIGHTED)
            wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), lb[j]));
          if (tk != cur) {
            if (cur >= 0) {
              store_tok(cur, true);
              done = cur + 1;
            }
            for (; done < tk; ++done) store_tok(done, false);
            cur = tk;
            static_for<P::N>([&](auto q) {
              constexpr int i = q;
              const float x = P::template get<i>(buf[j]);
              if constexpr (WEIGHTED) {
                acc[i] = wk * x;
              } else {
                acc[i] = x;
              }
            });
          } else {
            static_for<P::N>([&](auto q) {
              constexpr int i = q;
              const float x = P::template get<i>(buf[j]);
              if constexpr (WEIGHTED) {
                acc[i] = __builtin_fmaf(wk, x, acc[i]);
              } else {
                acc[i] = acc[i] + x;
              }
            });
          }
        }
      });
    }
    if (it + nwaves < n_items) sl_next = group_slot(it + nwaves);
    if (cur >= 0) {
      store_tok(cur, true);
      done = cur + 1;
    }
    for (; done < ntok; ++done) store_tok(done, false);
    if (wgrad && lane < GK && s < routes) dst_w[s] = gwv;
  }
}

// ---------------------------------------------------------------------------
// backward of the weighted combine
// ---------------------------------------------------------------------------

// For token t with valid routes k (received rows r_k, weights w_k):
//   grad_rows[r_k] = payload(fp32(w_k * g_t))
//   grad_w[r_k]    = sum_h g_t[h] * y[r_k][h]
// Units are the token groups of the scatter (64 / K tokens, up to 64 routes)
// with the valid routes dealt round-robin to the 8 wavefronts of a block; a
// wavefront handles a whole row per route, kBwdUnroll vectors per lane at a
// time, so the token's gradient row is read from memory once and then from
// L2 by the wavefronts of its other routes. Each lane accumulates its share
// of the dot product with fused multiply-adds over its vectors in ascending
// order, then the wavefront sums the lanes with a fixed butterfly (lane 0's
// result is stored): the same bits on every run. Pad pieces (1 KiB of pad
// rows, and their weight gradients) are zeroed when pads are filled.
constexpr int kBwdWaves = 8;
constexpr int kBwdUnroll = 8;

template <int DT, bool WANT_W>
__global__ void __launch_bounds__(kBwdWaves * kWave)
weighted_bwd_kernel(Dims d, const HandleHeader* __restrict__ h,
                    const int32_t* __restrict__ slot, const int32_t* __restrict__ pad_rows,
                    uint32_t* status, const row16_t* __restrict__ g4,
                    const row16_t* __restrict__ y4, const float* __restrict__ rw,
                    row16_t* __restrict__ o4, float* __restrict__ grad_w) {
  using P = Payload<DT>;
  const HandleHeader hh = *h;
  if (!handle_matches(hh, d)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, EP_STATUS_LAYOUT);
    return;
  }
  const int lane = lane_id();
  const int K = d.K;
  const int G = kWave / K;
  const int64_t V = d.V;
  const int64_t npc = (V + kWave - 1) / kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t n_groups = (d.T + G - 1) / G;
  const ZeroRows zr = zero_rows_of(hh, d);
  const int64_t pad_pieces = zr.n * npc;
  const int64_t n_units = n_groups + (pad_pieces + kBwdWaves - 1) / kBwdWaves;
  const int64_t routes = d.T * (int64_t)K;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));

  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    if (u < n_groups) {
      const int64_t first = u * G * (int64_t)K;
      const int64_t s = first + lane;
      const int32_t sl = (lane < G * K && s < routes) ? slot[s] : -1;
      const bool valid = sl >= 0;
      const int rank = __builtin_popcountll(wave_ballot(valid) & below);
      uint64_t mine = wave_ballot(valid && (rank % kBwdWaves) == wv);
      while (mine) {
        const int l = __ffsll((unsigned long long)mine) - 1;
        mine &= mine - 1;
        const int32_t r = __builtin_amdgcn_readlane(sl, l);
        const int64_t t = (first + l) / K;
        const float wk = rw[r];
        const row16_t* grow = g4 + t * V;
        const row16_t* yrow = y4 + (int64_t)r * V;
        row16_t* orow = o4 + (int64_t)r * V;
        float pd = 0.0f;
        for (int64_t vb = lane; vb < V; vb += (int64_t)kWave * kBwdUnroll) {
          row16_t gv[kBwdUnroll], yv[kBwdUnroll];
          static_for<kBwdUnroll>([&](auto j) {
            const int64_t v = vb + j * kWave;
            const int64_t vc = v < V ? v : V - 1;
            gv[j] = load_row16<false>(grow + vc);
            if constexpr (WANT_W) yv[j] = load_row16<kReduceNtLoad>(yrow + vc);
          });
          static_for<kBwdUnroll>([&](auto j) {
            const int64_t v = vb + j * kWave;
            if (v < V) {
              float prod[P::N];
              static_for<P::N>([&](auto q) {
                constexpr int i = q;
                const float gi = P::template get<i>(gv[j]);
                prod[i] = wk * gi;
                if constexpr (WANT_W) pd = __builtin_fmaf(gi, P::template get<i>(yv[j]), pd);
              });
              store_row16<kScatterNtStore>(orow + v, P::pack(prod));
            }
          });
        }
        if constexpr (WANT_W) {
          for (int off = kWave / 2; off > 0; off >>= 1) pd += __shfl_xor(pd, off);
          if (lane == 0) grad_w[r] = pd;
        }
      }
    } else {
      const int64_t pi = (u - n_groups) * kBwdWaves + wv;
      if (pi >= pad_pieces) continue;
      const int64_t p = pi / npc;
      const int64_t c = pi - p * npc;
      const int64_t r = zero_row(zr, pad_rows, p);
      const int64_t v = c * kWave + lane;
      if (v < V) store_row16<kScatterNtStore>(o4 + r * V + v, row16_t{0u, 0u, 0u, 0u});
      if (WANT_W && c == 0 && lane == 0) grad_w[r] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

int key_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

constexpr size_t kLdsBudget = kPrepLdsBudget;
// Routings of at most this many routes take the single-block prepare.
constexpr int64_t kPrepFusedMaxRoutes = 4096;
static_assert(kPrepFusedMaxRoutes <= (int64_t)kFusedWaves * kPrepRounds * kWave,
              "the one-block prepare holds at most kPrepRounds rounds per wavefront");

size_t slots_lds_bytes(int E, int nw, int run_chunks) {
  return sizeof(int32_t) * (size_t)(4 * E + 2 + 2 * kWave * nw + (nw + 1) * E + run_chunks * E);
}



int grid_for(int64_t items, int num_cus) {
  const int64_t waves_per_block = kBlock / kWave;
  int64_t blocks = (items + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * kBlocksPerCU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

// Calls f(std::integral_constant<int, K>) for the top-k values that have a
// compile-time kernel, f(integral_constant<int, 0>) for any other.
template <typename F>
hipError_t with_topk(int K, F&& f) {
  switch (K) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return f(std::integral_constant<int, 0>{});
  }
}

template <typename F>
hipError_t with_dtype(int dt, F&& f) {
  switch (dt) {
    case EP_DTYPE_FP16: return f(std::integral_constant<int, EP_DTYPE_FP16>{});
    case EP_DTYPE_FP32: return f(std::integral_constant<int, EP_DTYPE_FP32>{});
    default: return f(std::integral_constant<int, EP_DTYPE_BF16>{});
  }
}

const row16_t* rows_in(const void* p) { return static_cast<const row16_t*>(p); }
row16_t* rows_out(void* p) { return static_cast<row16_t*>(p); }

}  // namespace

namespace {

hipError_t launch_prepare_runs(const Dims& d, const HandleView& hv, const int64_t* topk_idx,
                               int32_t ru, int write_live, int scanned, hipStream_t stream) {
  if (d.T == 0) return hipSuccess;
  const int64_t chunks = ((int64_t)d.num_units + ru - 1) / ru;
  hipLaunchKernelGGL(prepare_runs_kernel, dim3((unsigned)chunks), dim3(kRunThreads),
                     2 * sizeof(int32_t) * (size_t)d.E, stream, d, hv, topk_idx, ru, write_live,
                     scanned);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const Dims& d, const HandleView& hv, const int64_t* topk_idx,
                          int32_t* user_counts, int32_t* user_offsets, int num_cus,
                          hipStream_t stream) {
  const int nbits = key_bits(d.E);
  const int U = d.num_units;
  // run chunks sized from this layout's payload row
  const int32_t ru = run_chunk_units(U, d.K, d.V * (int64_t)sizeof(row16_t));
  const size_t fused_lds = sizeof(int32_t) * ((size_t)(kFusedWaves + 3) * d.E + 2);
  if (d.T * (int64_t)d.K <= (int64_t)kPrepFusedMaxRoutes && fused_lds <= kLdsBudget) {
    // the run entries in the same block when their rows fit its LDS (and
    // the chunks are one unit each, which at most 8 units always are)
    const size_t runs_lds = fused_lds + sizeof(int32_t) * 2 * kRunXcds * (size_t)d.E;
    const int runs_here = ru == 1 && runs_lds <= kLdsBudget;
    hipLaunchKernelGGL(prepare_fused_kernel, dim3(1), dim3(kFusedWaves * kWave),
                       runs_here ? runs_lds : fused_lds, stream, d, hv, topk_idx, user_counts,
                       user_offsets, nbits, ru, runs_here);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return runs_here ? hipSuccess : launch_prepare_runs(d, hv, topk_idx, ru, 1, 0, stream);
  }
  const int nw1 = hist_block_units(U, d.E);
  const int nb = (U + nw1 - 1) / nw1;
  const int scanned = nb > kPrepDirectBlockRows;
  if (U > 0) {
    hipLaunchKernelGGL(prepare_hist_kernel, dim3(nb), dim3(nw1 * kWave),
                       sizeof(int32_t) * (size_t)nw1 * d.E, stream, d, hv, topk_idx, nbits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (scanned) {
    hipLaunchKernelGGL(prepare_scan_kernel, dim3((d.E + kWave - 1) / kWave), dim3(8 * kWave), 0,
                       stream, d, hv, (int32_t)nb, ru);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // The slot kernel also builds the run entries when its blocks hold whole
  // chunks (its LDS allowing); otherwise they take their own launch.
  // Measured on the MI355X with the block's chunks scanned side by side
  // (prepare us, in the slot kernel against a launch of their own): top-8 of
  // 256 experts with 2-unit chunks 22.3 against 23.4 at 4096 tokens and 28.5
  // against 30.8 at 65536; top-2 of 8 with 1-unit chunks 20.7 against 21.3
  // at 16384 tokens and 28.6 against 43.0 at 524288.
  // A block holds one chunk (ru wavefronts), or whole chunks up to 8 units
  // while it has fewer threads than experts (its per-expert steps then take
  // one pass) or one chunk a block would give more blocks than CUs: a
  // wavefront hands out its unit's rows one round after another, so while
  // the grid fits the CUs, smaller blocks spread the work over more of them,
  // and past that they queue and repeat each block's setup. Measured
  // (prepare us, one chunk a block against eight units): top-8 of 256 at
  // 4096 tokens 20.3 against 22.1, top-8 of 128 at 8192 19.0 against 20.5,
  // the 32-expert masked share at 32768 19.3 against 20.7, top-2 of 8 at
  // 16384 16.8 against 20.6 and at 131072 18.7 against 22.0; level at 256
  // blocks; top-8 of 256 at 524288 tokens (2048 blocks) 104 against 95, and
  // at 1024 tokens (2-unit chunks, 128 threads) 26.0 against 24.5.
  int nw2 = ru;
  while (nw2 < 8 && (nw2 * kWave < d.E || (U + nw2 - 1) / nw2 > num_cus)) nw2 *= 2;
  while (nw2 > ru && slots_lds_bytes(d.E, nw2, nw2 / ru) > kLdsBudget) nw2 /= 2;
  const int in_slots = slots_lds_bytes(d.E, nw2, nw2 / ru) <= kLdsBudget;
  if (!in_slots) {
    nw2 = 8;
    while (nw2 > 1 && slots_lds_bytes(d.E, nw2, 0) > kLdsBudget) nw2 /= 2;
  }
  int grid2 = (U + nw2 - 1) / nw2;
  if (grid2 < 1) grid2 = 1;
  hipLaunchKernelGGL(prepare_slots_kernel, dim3(grid2), dim3(nw2 * kWave),
                     slots_lds_bytes(d.E, nw2, in_slots ? nw2 / ru : 0), stream, d, hv,
                     user_counts, user_offsets, ru, in_slots, (int32_t)nw1, (int32_t)scanned);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return in_slots ? hipSuccess : launch_prepare_runs(d, hv, topk_idx, ru, 0, scanned, stream);
}

hipError_t launch_scatter_rows(const Dims& d, const HandleView& hv, const void* src,
                               const float* w, void* dst, float* dst_w, int num_cus,
                               hipStream_t stream) {
  const int64_t CB = (int64_t)kWave * kScatterCH;
  const int64_t ncb = (d.V + CB - 1) / CB;
  const int64_t npc = (d.V + kWave - 1) / kWave;
  const int64_t G = kWave / d.K;
  const int64_t max_units =
      (d.T + G - 1) / G * ncb +
      (d.fill_pads || d.zero_tail ? (d.cap * npc + kScatterWaves - 1) / kScatterWaves : 0);
  if (max_units == 0) return hipSuccess;
  const bool interleave = d.V * (int64_t)sizeof(row16_t) <= kScatterIlvMaxRow;
  int64_t grid = max_units;
  const int64_t limit =
      (int64_t)num_cus * (interleave ? kScatterIlvBlocksPerCU : kScatterBlocksPerCU);
  if (grid > limit) grid = limit;
  hipLaunchKernelGGL((scatter_rows_kernel<kScatterCH>), dim3((int)grid),
                     dim3(kScatterWaves * kWave), 0, stream, d, hv.header, hv.slot, hv.pad_rows,
                     &hv.header->status, rows_in(src), w, rows_out(dst), dst_w,
                     (int)interleave);
  return hipGetLastError();
}

hipError_t launch_run_rows(const Dims& d, const HandleView& hv, const void* src,
                           const float* w, void* dst, float* dst_w, int num_cus,
                           hipStream_t stream) {
  if (d.cap == 0) return hipSuccess;        // nothing to write
  // no token: no route, so no entry and no pad row; a zeroed tail still
  // needs a grid, which the scatter sizes from the capacity
  if (d.T == 0)
    return d.zero_tail ? launch_scatter_rows(d, hv, src, w, dst, dst_w, num_cus, stream)
                       : hipSuccess;
  const int64_t npc = (d.V + kWave - 1) / kWave;
  const int64_t routes = d.T * (int64_t)d.K;
  const int64_t scap = run_stream_cap(d.num_units);
  const int64_t dense = run_stream_dense(d.num_units, routes);
  int P = d.fill_pads && npc <= kRunNarrowRow ? kRunPiecesNarrow : kRunPieces;
  // narrow rows take eight pieces only while the grid still fills the device
  if (P == kRunPiecesNarrow &&
      (dense * npc + kRunWaves * P - 1) / (kRunWaves * P) * kRunXcds < kRunNarrowMinBlocks)
    P = kRunPieces;
  const int64_t per_block = (int64_t)kRunWaves * P;
  const int64_t bps = run_copy_blocks((dense * npc + per_block - 1) / per_block, num_cus);
  const int64_t zero_max = d.zero_tail ? d.cap : ((int64_t)d.E * (d.A - 1) < d.cap
                                                      ? (int64_t)d.E * (d.A - 1) : d.cap);
  // 32-bit piece indices: a stream's list, the steps past it, the zero rows
  const int64_t lim = (int64_t)1 << 31;
  if (scap * npc + bps * per_block >= lim || zero_max * npc >= lim) {
    // a size no buffer in memory reaches; the scatter takes any size
    return launch_scatter_rows(d, hv, src, w, dst, dst_w, num_cus, stream);
  }
  RunGeom g;
  g.npc = (uint32_t)npc;
  g.bps = (uint32_t)bps;
  g.cap_pieces = (uint32_t)(scap * npc);
  g.scap = scap;
  g.npf = 0;
  g.pf_per = 0;
  const int64_t row_bytes = d.V * (int64_t)sizeof(row16_t);
  if (d.K >= kRunPrefetchMinK && row_bytes >= kRunPrefetchMinRow &&
      d.T * row_bytes <= kRunPrefetchMaxBytes) {
    const int64_t nvec = d.T * d.V;
    int64_t npf = (nvec + (int64_t)kRunWaves * kWave * 4 - 1) / ((int64_t)kRunWaves * kWave * 4);
    if (npf > kRunPrefetchBlocks) npf = kRunPrefetchBlocks;
    g.npf = (uint32_t)npf;
    g.pf_per = (uint32_t)((nvec + npf * kRunWaves * kWave - 1) / (npf * kRunWaves * kWave));
  }
  g.nlp = 0;
  g.lp_ent = 0;
  if (g.npf == 0) {
    int64_t ent = dense < scap ? dense : scap;
    int64_t per = (ent * (int64_t)sizeof(RunEntry) + kRunListBlockBytes - 1) / kRunListBlockBytes;
    if (per < 1) per = 1;
    if (per > kRunListBlocks) per = kRunListBlocks;
    if (ent > per * kRunListBlockBytes / (int64_t)sizeof(RunEntry))
      ent = per * kRunListBlockBytes / (int64_t)sizeof(RunEntry);
    g.nlp = (uint32_t)(kRunXcds * per);
    g.lp_ent = (uint32_t)ent & ~1u;
  }
  const int64_t grid = (int64_t)g.npf + g.nlp + kRunXcds * bps;
  if (P == kRunPiecesNarrow)
    hipLaunchKernelGGL(run_rows_kernel<kRunPiecesNarrow>, dim3((unsigned)grid),
                       dim3(kRunWaves * kWave), 0, stream, d, hv.header, hv.runs, hv.pad_rows,
                       &hv.header->status, rows_in(src), w, rows_out(dst), dst_w, g);
  else
    hipLaunchKernelGGL(run_rows_kernel<kRunPieces>, dim3((unsigned)grid),
                       dim3(kRunWaves * kWave), 0, stream, d, hv.header, hv.runs, hv.pad_rows,
                       &hv.header->status, rows_in(src), w, rows_out(dst), dst_w, g);
  return hipGetLastError();
}

hipError_t launch_reduce_rows(const Dims& d, const HandleView& hv, const void* src,
                              const float* rw, const float* g_w, void* dst, float* dst_w,
                              int num_cus, hipStream_t stream) {
  const int64_t ncb = (d.V + kWave - 1) / kWave;
  if (d.T * ncb == 0) return hipSuccess;
  // tokens per item: chosen on the device from the routing's density, at
  // most g_max, the largest power of two up to 64 / K that leaves at least
  // half a grid's worth of items
  const int grid = grid_for(d.T * ncb, num_cus);
  const int64_t half = (int64_t)grid * (kBlock / kWave) / 2;
  int g_max = 1;
  while (2 * g_max * d.K <= kWave && (d.T + 2 * g_max - 1) / (2 * g_max) * ncb >= half)
    g_max *= 2;
  return with_dtype(d.dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    return with_topk(d.K, [&](auto kt) {
      constexpr int KT = decltype(kt)::value;
      if (rw != nullptr) {
        hipLaunchKernelGGL((reduce_rows_kernel<KT, true, DT>), dim3(grid), dim3(kBlock), 0,
                           stream, d, hv.header, hv.slot, &hv.header->status, rows_in(src), rw,
                           g_w, rows_out(dst), dst_w, g_max);
      } else {
        hipLaunchKernelGGL((reduce_rows_kernel<KT, false, DT>), dim3(grid), dim3(kBlock), 0,
                           stream, d, hv.header, hv.slot, &hv.header->status, rows_in(src),
                           nullptr, g_w, rows_out(dst), dst_w, g_max);
      }
      return hipGetLastError();
    });
  });
}

namespace {

// The token-group form of the weighted backward: the fallback for sizes the
// run form's 32-bit indices or LDS partials do not take.
hipError_t launch_weighted_bwd_groups(const Dims& d, const HandleView& hv, const void* g,
                                      const void* y, const float* rw, void* grad_rows,
                                      float* grad_w, int num_cus, hipStream_t stream) {
  const int64_t npc = (d.V + kWave - 1) / kWave;
  const int64_t G = kWave / d.K;
  const int64_t max_units =
      (d.T + G - 1) / G +
      (d.fill_pads || d.zero_tail ? (d.cap * npc + kBwdWaves - 1) / kBwdWaves : 0);
  if (max_units == 0) return hipSuccess;
  int64_t grid = max_units;
  const int64_t limit = (int64_t)num_cus * kBwdBlocksPerCU;
  if (grid > limit) grid = limit;
  return with_dtype(d.dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (grad_w != nullptr) {
      hipLaunchKernelGGL((weighted_bwd_kernel<DT, true>), dim3((int)grid),
                         dim3(kBwdWaves * kWave), 0, stream, d, hv.header, hv.slot, hv.pad_rows,
                         &hv.header->status, rows_in(g), rows_in(y), rw, rows_out(grad_rows),
                         grad_w);
    } else {
      hipLaunchKernelGGL((weighted_bwd_kernel<DT, false>), dim3((int)grid),
                         dim3(kBwdWaves * kWave), 0, stream, d, hv.header, hv.slot, hv.pad_rows,
                         &hv.header->status, rows_in(g), nullptr, rw, rows_out(grad_rows),
                         nullptr);
    }
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_weighted_bwd(const Dims& d, const HandleView& hv, const void* g,
                               const void* y, const float* rw, void* grad_rows, float* grad_w,
                               int num_cus, hipStream_t stream) {
  if (d.cap == 0) return hipSuccess;
  const int64_t npc = (d.V + kWave - 1) / kWave;
  const int64_t routes = d.T * (int64_t)d.K;
  const int64_t scap = run_stream_cap(d.num_units);
  const int64_t zero_max = d.zero_tail ? d.cap : ((int64_t)d.E * (d.A - 1) < d.cap
                                                      ? (int64_t)d.E * (d.A - 1) : d.cap);
  const int64_t lim = (int64_t)1 << 31;
  if (d.T == 0 || npc > kWbwdMaxPartials || scap * npc >= lim || zero_max * npc >= lim)
    return launch_weighted_bwd_groups(d, hv, g, y, rw, grad_rows, grad_w, num_cus, stream);
  // rows per block step: as many whole rows as fill the step's rounds of
  // waves * kWbwdPieces pieces, at least one. With the weight gradient a step
  // ends in two block barriers: two rounds a step and at most 256 wavefronts
  // per CU (each block taking more steps) measured best on the MI355X, with
  // eight-wavefront blocks (dsv3 247 us against 257 us with one round and 96
  // blocks per CU, the masked share 209 against 231); the row gradient alone
  // has no barrier and takes one round and the run copy's grid.
  const bool want_w = grad_w != nullptr;
  const int waves = wbwd_waves(want_w);
  const int64_t round = (int64_t)waves * kWbwdPieces * (want_w ? kWbwdRounds : 1);
  int64_t R = round / npc;
  if (R < 1) R = 1;
  const int64_t dense = run_stream_dense(d.num_units, routes);
  int64_t bps = (dense + R - 1) / R;
  if (want_w) {
    const int64_t bps_cap = (int64_t)num_cus * kWbwdBlocksPerCU / kRunXcds;
    if (bps > bps_cap) bps = bps_cap;
    if (bps < 1) bps = 1;
  } else {
    bps = run_copy_blocks(bps, num_cus);
  }
  RunGeom geo;
  geo.npc = (uint32_t)npc;
  geo.bps = (uint32_t)bps;
  geo.cap_pieces = (uint32_t)(scap * npc);
  geo.scap = scap;
  geo.npf = 0;
  geo.pf_per = 0;
  geo.nlp = 0;
  geo.lp_ent = 0;
  const int64_t row_bytes = d.V * (int64_t)sizeof(row16_t);
  if (d.K >= kRunPrefetchMinK && row_bytes >= kRunPrefetchMinRow &&
      d.T * row_bytes <= kRunPrefetchMaxBytes) {
    const int64_t nvec = d.T * d.V;
    int64_t npf = (nvec + (int64_t)waves * kWave * 4 - 1) / ((int64_t)waves * kWave * 4);
    if (npf > kRunPrefetchBlocks) npf = kRunPrefetchBlocks;
    geo.npf = (uint32_t)npf;
    geo.pf_per = (uint32_t)((nvec + npf * waves * kWave - 1) / (npf * waves * kWave));
  }
  const int64_t grid = (int64_t)geo.npf + kRunXcds * bps;
  return with_dtype(d.dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (grad_w != nullptr) {
      hipLaunchKernelGGL((run_wbwd_kernel<DT, true>), dim3((unsigned)grid),
                         dim3(waves * kWave), 0, stream, d, hv.header, hv.runs, hv.pad_rows,
                         &hv.header->status, rows_in(g), rows_in(y), rw, rows_out(grad_rows),
                         grad_w, geo, (uint32_t)R, hv.row_src);
    } else {
      hipLaunchKernelGGL((run_wbwd_kernel<DT, false>), dim3((unsigned)grid),
                         dim3(waves * kWave), 0, stream, d, hv.header, hv.runs, hv.pad_rows,
                         &hv.header->status, rows_in(g), nullptr, rw, rows_out(grad_rows),
                         nullptr, geo, (uint32_t)R, hv.row_src);
    }
    return hipGetLastError();
  });
}

}  // namespace epmi
