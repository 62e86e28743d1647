// ep_ceilings.hip -- memory-pattern ceilings of the MI355X, measured beside
// the routing kernels.
//
// MEASUREMENT ONLY. These kernels are not part of the routing library and
// are built into their own shared object; the benchmark times them on the
// same device as the routing ops so that each op's bandwidth can be read
// against what the memory system gives for the same access pattern, not
// only against the 8 TB/s HBM peak.
//
// Every kernel moves 16-byte vectors with non-temporal loads and with the
// routing kernels' streaming stores (non-temporal, system scope: they write
// through the L2), one wavefront per piece and no grid-stride loop, so that
// blocks are issued in address order:
//   write_linear   a dense write front: wavefront i zeroes bytes [1024 i, 1024 i + 1024)
//   write_rows     the dispatch pattern: rows of `row_bytes` in a scrambled
//                  order (row r -> r * 2654435761 mod nrows, nrows a power of
//                  two), written in 2 KiB pieces, the pieces of a row on
//                  consecutive wavefronts
//   read_linear    a dense read front (the loaded values are folded into a
//                  sink that is written only under a condition that does not
//                  hold for the zero-filled input)
//   copy_linear    dense read and write fronts, 1 KiB per wavefront
//   flush          not a pattern: plain (cache-allocating) stores over one
//                  buffer, then plain loads over a second one, so that the
//                  L2s and the Infinity Cache end up holding clean lines of
//                  the second buffer and nothing a following kernel uses
//   gather_sum     the combine pattern: for each of `ntok` tokens and each
//                  1 KiB column block, k rows picked by a multiplicative
//                  hash of (token, k) are read and summed as 32-bit integers,
//                  and the sum is written to the token's row; no routing
//                  table is read
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epceil {

typedef uint32_t vec4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr uint32_t kScramble = 2654435761u;

// The routing kernels' streaming store (cache-policy bits sc0 sc1 nt), with
// the two wait states a 128-bit store needs on gfx950 before a VALU
// instruction may overwrite its data registers.
__device__ __forceinline__ void store_stream(vec4* p, vec4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" ::"v"(p), "v"(v)
               : "memory");
}

__device__ __forceinline__ int64_t piece_index() {
  return (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
write_linear_kernel(vec4* __restrict__ dst, int64_t pieces) {
  const int64_t p = piece_index();
  if (p >= pieces) return;
  store_stream(dst + p * kWave + (threadIdx.x & (kWave - 1)), vec4{0u, 0u, 0u, 0u});
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
write_rows_kernel(vec4* __restrict__ dst, int64_t nrows, int64_t row_vecs, int64_t per_row) {
  const int64_t p = piece_index();
  const int64_t r = p / per_row;
  if (r >= nrows) return;
  const int64_t c = p - r * per_row;
  const int64_t rr = (int64_t)(((uint64_t)r * kScramble) & (uint64_t)(nrows - 1));
  const int64_t v = c * 2 * kWave + (threadIdx.x & (kWave - 1));
  vec4* row = dst + rr * row_vecs;
  if (v < row_vecs) store_stream(row + v, vec4{0u, 0u, 0u, 0u});
  if (v + kWave < row_vecs) store_stream(row + v + kWave, vec4{0u, 0u, 0u, 0u});
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
read_linear_kernel(const vec4* __restrict__ src, int64_t pieces, vec4* __restrict__ sink) {
  const int64_t p = piece_index();
  if (p >= pieces) return;
  const vec4 v = __builtin_nontemporal_load(src + p * kWave + (threadIdx.x & (kWave - 1)));
  if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9E3779B9u) sink[threadIdx.x & (kWave - 1)] = v;
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
copy_linear_kernel(const vec4* __restrict__ src, vec4* __restrict__ dst, int64_t pieces) {
  const int64_t p = piece_index();
  if (p >= pieces) return;
  const int64_t i = p * kWave + (threadIdx.x & (kWave - 1));
  store_stream(dst + i, __builtin_nontemporal_load(src + i));
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
write_plain_kernel(vec4* __restrict__ dst, int64_t pieces) {
  const int64_t p = piece_index();
  if (p >= pieces) return;
  dst[p * kWave + (threadIdx.x & (kWave - 1))] = vec4{(uint32_t)p, 0u, 0u, 0u};
}

__global__ void __launch_bounds__(kWavesPerBlock * kWave)
read_plain_kernel(const vec4* __restrict__ src, int64_t pieces, vec4* __restrict__ sink) {
  const int64_t p = piece_index();
  if (p >= pieces) return;
  const vec4 v = src[p * kWave + (threadIdx.x & (kWave - 1))];
  if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9E3779B9u) sink[threadIdx.x & (kWave - 1)] = v;
}

template <int K>
__global__ void __launch_bounds__(kWavesPerBlock * kWave)
gather_sum_kernel(const vec4* __restrict__ rows, int64_t nrows, int64_t row_vecs,
                  int64_t ntok, vec4* __restrict__ out) {
  const int64_t ncb = (row_vecs + kWave - 1) / kWave;
  const int64_t p = piece_index();
  const int64_t t = p / ncb;
  if (t >= ntok) return;
  const int64_t cb = p - t * ncb;
  int64_t v = cb * kWave + (threadIdx.x & (kWave - 1));
  const bool live = v < row_vecs;
  if (!live) v = row_vecs - 1;
  vec4 b[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint64_t key = (uint64_t)t * (uint64_t)K + (uint64_t)j;
    const int64_t r = (int64_t)((key * kScramble) % (uint64_t)nrows);
    b[j] = __builtin_nontemporal_load(rows + r * row_vecs + v);
  }
  vec4 acc = b[0];
#pragma unroll
  for (int j = 1; j < K; ++j) acc += b[j];
  if (live) store_stream(out + t * row_vecs + v, acc);
}

int64_t blocks_for(int64_t pieces) { return (pieces + kWavesPerBlock - 1) / kWavesPerBlock; }

// A grid of more blocks than this is refused (the x dimension of a launch).
constexpr int64_t kMaxBlocks = (int64_t)1 << 30;

int finish(int64_t blocks) {
  if (blocks > kMaxBlocks) return 2;
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace epceil

using namespace epceil;

// Each entry point returns 0 on success, 1 on a launch error, 2 for sizes it
// does not take (nothing is launched then). Pointers are device pointers,
// 16-byte aligned; byte counts are multiples of 1024.
extern "C" {

int epc_write_linear(void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t pieces = bytes / 1024;
  const int64_t blocks = blocks_for(pieces);
  if (dst == nullptr || bytes % 1024 != 0 || blocks > kMaxBlocks) return 2;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(write_linear_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<vec4*>(dst), pieces);
  return finish(blocks);
}

// nrows must be a power of two; the buffer holds nrows * row_bytes bytes.
int epc_write_rows(void* dst, int64_t nrows, int64_t row_bytes, hipStream_t stream) {
  if (dst == nullptr || nrows < 1 || (nrows & (nrows - 1)) != 0 || row_bytes < 16 ||
      row_bytes % 16 != 0)
    return 2;
  const int64_t row_vecs = row_bytes / 16;
  const int64_t per_row = (row_vecs + 2 * kWave - 1) / (2 * kWave);
  const int64_t blocks = blocks_for(nrows * per_row);
  if (blocks > kMaxBlocks) return 2;
  hipLaunchKernelGGL(write_rows_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<vec4*>(dst), nrows, row_vecs, per_row);
  return finish(blocks);
}

// sink: 1 KiB of device memory.
int epc_read_linear(const void* src, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t pieces = bytes / 1024;
  const int64_t blocks = blocks_for(pieces);
  if (src == nullptr || sink == nullptr || bytes % 1024 != 0 || blocks > kMaxBlocks) return 2;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(read_linear_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<const vec4*>(src), pieces, static_cast<vec4*>(sink));
  return finish(blocks);
}

int epc_copy_linear(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t pieces = bytes / 1024;
  const int64_t blocks = blocks_for(pieces);
  if (src == nullptr || dst == nullptr || bytes % 1024 != 0 || blocks > kMaxBlocks) return 2;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(copy_linear_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<const vec4*>(src), static_cast<vec4*>(dst), pieces);
  return finish(blocks);
}

// Evicts the caches: plain stores over `a`, then plain loads over `b` (both
// `bytes` long, a multiple of 1024; sink: 1 KiB). Two launches on `stream`.
int epc_flush(void* a, const void* b, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t pieces = bytes / 1024;
  const int64_t blocks = blocks_for(pieces);
  if (a == nullptr || b == nullptr || sink == nullptr || bytes % 1024 != 0 ||
      blocks > kMaxBlocks)
    return 2;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(write_plain_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<vec4*>(a), pieces);
  if (hipGetLastError() != hipSuccess) return 1;
  hipLaunchKernelGGL(read_plain_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                     stream, static_cast<const vec4*>(b), pieces, static_cast<vec4*>(sink));
  return finish(blocks);
}

// rows: nrows * row_bytes bytes; out: ntok * row_bytes bytes; k in {1, 2, 4, 8}.
int epc_gather_sum(const void* rows, int64_t nrows, int64_t row_bytes, int64_t ntok, int k,
                   void* out, hipStream_t stream) {
  if (rows == nullptr || out == nullptr || nrows < 1 || ntok < 0 || row_bytes < 16 ||
      row_bytes % 16 != 0 || (k != 1 && k != 2 && k != 4 && k != 8))
    return 2;
  const int64_t row_vecs = row_bytes / 16;
  const int64_t ncb = (row_vecs + kWave - 1) / kWave;
  const int64_t blocks = blocks_for(ntok * ncb);
  if (blocks > kMaxBlocks) return 2;
  if (blocks == 0) return 0;
  const dim3 grid((unsigned)blocks), block(kWavesPerBlock * kWave);
  const vec4* r = static_cast<const vec4*>(rows);
  vec4* o = static_cast<vec4*>(out);
  switch (k) {
    case 1: hipLaunchKernelGGL(gather_sum_kernel<1>, grid, block, 0, stream, r, nrows, row_vecs, ntok, o); break;
    case 2: hipLaunchKernelGGL(gather_sum_kernel<2>, grid, block, 0, stream, r, nrows, row_vecs, ntok, o); break;
    case 4: hipLaunchKernelGGL(gather_sum_kernel<4>, grid, block, 0, stream, r, nrows, row_vecs, ntok, o); break;
    default: hipLaunchKernelGGL(gather_sum_kernel<8>, grid, block, 0, stream, r, nrows, row_vecs, ntok, o); break;
  }
  return finish(blocks);
}

}  // extern "C"
