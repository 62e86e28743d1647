/*
 * ep_oracle.c -- plain CPU oracle for MoE expert-parallel prepare, dispatch,
 * combine, dispatch_bwd and combine_bwd at one GPU's share of the work.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct model
 * that the HIP library is checked against. Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the library itself never
 * calls it, and it shares no code, header or table with the library.
 *
 * Everything here is scalar C, one loop per step of the definition. When
 * built with OpenMP, the loops over received rows and over tokens (each
 * iteration writes outputs no other iteration touches, and every output's
 * arithmetic stays inside one iteration) are shared among threads; prepare,
 * a sequential counting sort, always runs on one thread. The thread count
 * changes no result bit. Integer work is exact; the only floating point is an ordered
 * binary32 sum followed by one round-to-nearest-even to the payload type
 * (bf16, fp16 or fp32), and, for the weighted combine, products and fused
 * multiply-adds in binary32.
 *
 * Sources (the expert-parallel pull requests these ops come from):
 *  - "Expert Parallelism: common C API + NCCL EP backend", section "Per-step
 *    (allocation-free, CUDA-graph capturable)": the five per-step calls and
 *    their one-line meanings (prepare writes the routing maps for a handle;
 *    dispatch sends token rows and routing weights to their experts; combine
 *    is an unweighted scatter-sum back to the sources, the caller having
 *    already multiplied by the received weights; dispatch_bwd and combine_bwd
 *    are the two backward ops; combine_bwd leaves padded rows zero).
 *  - "[PyTorch] Expert Parallelism: PyTorch wrapper + autograd ops with
 *    symm-mem zero-copy", section "Public Python API": payloads are bf16 and
 *    topk_idx is int64; section "Testing": identity round trip, VJP,
 *    bit stability.
 *  - "Expert Parallelism: common C API + NCCL EP backend", section
 *    "Important Files Changed": its C++ tests cover BF16, FP16 and FP32
 *    payloads, so the oracle takes all three.
 *  - "Expert-parallel implementations for ep_dispatch_experts", table
 *    "Implementations": a rank masks the routes that go to other ranks'
 *    experts; here a masked route carries the id -1.
 *
 * Readings where the pages leave a step open (each one is also a test):
 *  - Rows of an expert's segment are in ascending flattened route order
 *    s = t*K + k (a stable counting sort keyed by expert id).
 *  - An expert's segment is its route count rounded up to a multiple of the
 *    alignment A; pad rows sit at the end of the segment and are zero in
 *    every expert-major output (or, under the no-pad-fill policy, not
 *    written). An expert with no routes has an empty segment.
 *  - token_counts are the raw (unpadded) per-expert route counts.
 *  - Exactly -1 marks a masked route. Any other id outside [0,E) raises the
 *    BAD_EXPERT status bit and is then treated as masked.
 *  - If the padded total exceeds the receive capacity, the OVERFLOW bit is
 *    raised and every route whose row would lie at or past the capacity is
 *    dropped (slot -1); rows past the capacity are never written.
 *  - combine sums, in ascending k, the fp32 values of the rows of the token's
 *    valid routes, starting from the first valid row (so a single route is a
 *    bit copy, -0.0 included), then rounds once to the payload type. A token
 *    with no valid route gets +0.
 *  - fp32 -> bf16 and fp32 -> fp16 round to nearest, ties to even, keep
 *    subnormals, carry into infinity on overflow, and return the canonical
 *    quiet NaN (0x7FC0, 0x7E00) for any NaN (the sign and payload of a NaN
 *    produced by an add are not portable). An fp32 result is the sum itself
 *    with any NaN replaced by 0x7FC00000.
 */
#include <fenv.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#ifdef _OPENMP
#include <omp.h>
#define ORACLE_PARALLEL_FOR _Pragma("omp parallel for schedule(static)")
#else
#define ORACLE_PARALLEL_FOR
#endif

#define ORACLE_STATUS_BAD_EXPERT 1u
#define ORACLE_STATUS_OVERFLOW 2u

/* Return codes of the oracle entry points. */
#define ORACLE_OK 0
#define ORACLE_ERR_ARGS 1
#define ORACLE_ERR_FPENV 2

/* The oracle relies on IEEE binary32 with round-to-nearest and with
 * subnormals neither flushed on output (FTZ) nor treated as zero on input
 * (DAZ). Refuse to run in any other floating-point environment. */
static int fpenv_is_ieee(void) {
  unsigned csr = _mm_getcsr();
  if (csr & (1u << 15)) return 0; /* FTZ */
  if (csr & (1u << 6)) return 0;  /* DAZ */
  return fegetround() == FE_TONEAREST;
}

/* Threads the row and token loops may use (the OpenMP default is every
 * core); returns the count now in force, always 1 without OpenMP. */
int ep_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* bf16 -> fp32: a bf16 value is the upper half of the binary32 pattern. */
static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (IEEE 754 roundTiesToEven
 * applied to the 8-bit significand of bfloat16). The two candidates are the
 * truncation and the next representable value above it in magnitude; the
 * discarded low half decides between them. */
uint16_t ep_oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
    return 0x7FC0u; /* canonical quiet NaN */
  uint16_t truncated = (uint16_t)(u >> 16);
  uint32_t discarded = u & 0xFFFFu;
  int round_up;
  if (discarded > 0x8000u) {
    round_up = 1;
  } else if (discarded < 0x8000u) {
    round_up = 0;
  } else {
    round_up = (truncated & 1u) != 0u; /* exact tie: go to the even one */
  }
  /* For finite values, the next bf16 pattern up is the next value in
   * magnitude (the carry moves into the exponent, up to infinity). */
  return (uint16_t)(truncated + (round_up ? 1u : 0u));
}

float ep_oracle_bf16_to_f32(uint16_t h) { return bf16_to_float(h); }

/* fp16 -> fp32 from the binary16 definition: sign, 5-bit exponent with bias
 * 15, 10-bit fraction; exponent 0 holds the subnormals m * 2^-24, exponent
 * 31 infinities and NaNs. Every binary16 value is exact in binary32. */
float ep_oracle_f16_to_f32(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  float mag;
  if (e == 0x1F) {
    mag = m ? NAN : INFINITY;
  } else if (e == 0) {
    mag = ldexpf((float)m, -24);
  } else {
    mag = ldexpf((float)(1024 + m), e - 25);
  }
  return sign ? -mag : mag;
}

/* fp32 -> fp16, round to nearest, ties to even. The result is n * q where q
 * is the spacing of binary16 values at the magnitude of f (2^(e-10) for a
 * normal exponent e, the subnormal spacing 2^-24 below 2^-14) and n the
 * integer nearest |f| / q, ties to even; n = 2048 moves to the next binade,
 * past the largest finite value (65504) the result is infinity. */
uint16_t ep_oracle_f32_to_f16(float f) {
  if (isnan(f)) return 0x7E00u;
  const uint16_t sign = signbit(f) ? 0x8000u : 0u;
  const float a = fabsf(f);
  if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
  if (a == 0.0f) return sign;
  int ex;
  frexpf(a, &ex);                /* a = m * 2^ex, m in [0.5, 1) */
  int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
  if (e < -14) e = -14;          /* subnormal range: fixed spacing */
  const float y = ldexpf(a, 10 - e);   /* a / q, exact (power-of-two scale) */
  const float fl = floorf(y);
  const float frac = y - fl;           /* exact: y has at most 24 bits */
  long n = (long)fl;
  if (frac > 0.5f || (frac == 0.5f && (n & 1))) n += 1;
  if (n == 2048) {               /* rounded up into the next binade */
    n = 1024;
    e += 1;
  }
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  if (n < 1024) return (uint16_t)(sign | (uint16_t)n);   /* subnormal (e == -14) */
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024));
}

/* Payload element types of the rows. */
#define ORACLE_BF16 0
#define ORACLE_FP16 1
#define ORACLE_FP32 2

static int dtype_ok(int dt) { return dt == ORACLE_BF16 || dt == ORACLE_FP16 || dt == ORACLE_FP32; }

static size_t elem_bytes(int dt) { return dt == ORACLE_FP32 ? 4u : 2u; }

/* Element i of a payload array, exactly as binary32. */
static float load_elem(const void* base, int64_t i, int dt) {
  if (dt == ORACLE_BF16) return bf16_to_float(((const uint16_t*)base)[i]);
  if (dt == ORACLE_FP16) return ep_oracle_f16_to_f32(((const uint16_t*)base)[i]);
  float f;
  memcpy(&f, (const char*)base + 4 * i, sizeof f);
  return f;
}

/* Store a binary32 value into element i, rounded once to the payload type. */
static void store_elem(void* base, int64_t i, int dt, float f) {
  if (dt == ORACLE_BF16) {
    ((uint16_t*)base)[i] = ep_oracle_f32_to_bf16(f);
  } else if (dt == ORACLE_FP16) {
    ((uint16_t*)base)[i] = ep_oracle_f32_to_f16(f);
  } else {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0x7FC00000u;
    memcpy((char*)base + 4 * i, &u, sizeof u);
  }
}

/* +0 in element i. */
static void store_zero(void* base, int64_t i, int dt) {
  memset((char*)base + (size_t)i * elem_bytes(dt), 0, elem_bytes(dt));
}

/* Worst-case number of received rows: every token sends min(K,E) distinct
 * routes and every expert adds up to A-1 pad rows. */
int64_t ep_oracle_recv_capacity_worst(int64_t T, int32_t K, int32_t E, int32_t A) {
  int64_t per_token = K < E ? K : E;
  return T * per_token + (int64_t)E * (int64_t)(A - 1);
}

/*
 * prepare: routing ids -> per-expert counts, aligned segment offsets, the
 * slot of every route and the source route of every received row.
 *
 *   topk_idx  int64 [T*K]   routing id of route s = t*K + k
 *   counts    int32 [E]     valid routes per expert (unpadded)
 *   offsets   int32 [E+1]   segment starts; offsets[E] = padded total
 *   slot      int32 [T*K]   received row of route s, -1 if masked or dropped
 *   row_src   int32 [cap]   route s held by received row r, -1 for pad rows
 *                           (rows at or past offsets[E] are left untouched)
 *   status    uint32        BAD_EXPERT / OVERFLOW bits
 */
int ep_oracle_prepare(int64_t T, int32_t K, int32_t E, int32_t A, int64_t cap,
                      const int64_t* topk_idx, int32_t* counts, int32_t* offsets,
                      int32_t* slot, int32_t* row_src, uint32_t* status) {
  if (T < 0 || K < 1 || E < 1 || A < 1 || cap < 0) return ORACLE_ERR_ARGS;
  if (!counts || !offsets || !status) return ORACLE_ERR_ARGS;
  const int64_t routes = T * (int64_t)K;
  if (routes > 0 && (!topk_idx || !slot)) return ORACLE_ERR_ARGS;
  uint32_t st = 0;

  /* Step 1: classify each route and count the valid ones per expert. */
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < routes; ++s) {
    int64_t e = topk_idx[s];
    if (e == -1) continue;                  /* masked */
    if (e < 0 || e >= E) {                  /* out of range: flag, then mask */
      st |= ORACLE_STATUS_BAD_EXPERT;
      continue;
    }
    counts[e] += 1;
  }

  /* Step 2: segment e is counts[e] rounded up to a multiple of A. */
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    int64_t padded = ((int64_t)counts[e] + A - 1) / A * A;
    offsets[e + 1] = (int32_t)(offsets[e] + padded);
  }
  const int64_t total = offsets[E];
  if (total > cap) st |= ORACLE_STATUS_OVERFLOW;

  /* Step 3: fill the segments in route order. Every row first counts as a
   * pad; a route then claims the next free row of its expert's segment. */
  const int64_t live = total < cap ? total : cap;
  for (int64_t r = 0; r < live; ++r) row_src[r] = -1;
  int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!cursor) return ORACLE_ERR_ARGS;
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t s = 0; s < routes; ++s) {
    int64_t e = topk_idx[s];
    if (e < 0 || e >= E) {
      slot[s] = -1;
      continue;
    }
    int64_t r = cursor[e]++;
    if (r >= cap) {
      slot[s] = -1;                         /* dropped on overflow */
      continue;
    }
    slot[s] = (int32_t)r;
    row_src[r] = (int32_t)s;
  }
  free(cursor);
  *status = st;
  return ORACLE_OK;
}

/*
 * dispatch (token part and weight part): received row r holds the token row
 * of the route it came from (a bit copy of its elements), or zeros for a pad
 * row (left as they are if fill_pads is 0). Rows at or past min(total, cap)
 * are not touched, unless zero_tail is 1: then they are zeros too (the tail
 * policy, under which the whole receive buffer is defined).
 *
 *   x        payload [T*H]  token rows
 *   w        f32  [T*K]     routing weights (may be NULL: then no weight output)
 *   recv     payload [cap*H]
 *   recv_w   f32  [cap]
 */
int ep_oracle_dispatch(int64_t T, int32_t K, int64_t H, int dtype, int fill_pads,
                       int zero_tail, int64_t cap, int64_t total, const int32_t* row_src,
                       const void* x, const float* w, void* recv, float* recv_w) {
  if (T < 0 || K < 1 || H < 1 || cap < 0 || total < 0 || !dtype_ok(dtype))
    return ORACLE_ERR_ARGS;
  const size_t eb = elem_bytes(dtype);
  const int64_t live = total < cap ? total : cap;
  if (zero_tail) {
    ORACLE_PARALLEL_FOR
    for (int64_t r = live; r < cap; ++r) {
      for (int64_t h = 0; h < H; ++h) store_zero(recv, r * H + h, dtype);
      if (w && recv_w) recv_w[r] = 0.0f;
    }
  }
  ORACLE_PARALLEL_FOR
  for (int64_t r = 0; r < live; ++r) {
    int32_t s = row_src[r];
    if (s >= 0) {
      int64_t t = s / K;
      for (int64_t h = 0; h < H; ++h)
        memcpy((char*)recv + (size_t)(r * H + h) * eb, (const char*)x + (size_t)(t * H + h) * eb,
               eb);
      if (w && recv_w) recv_w[r] = w[s];
    } else if (fill_pads) {
      for (int64_t h = 0; h < H; ++h) store_zero(recv, r * H + h, dtype);
      if (w && recv_w) recv_w[r] = 0.0f;
    }
  }
  return ORACLE_OK;
}

/* combine_bwd is the same row map as dispatch's token part, applied to the
 * gradient of the combined output. */
int ep_oracle_combine_bwd(int64_t T, int32_t K, int64_t H, int dtype, int fill_pads,
                          int zero_tail, int64_t cap, int64_t total, const int32_t* row_src,
                          const void* g_result, void* g_expert_out) {
  return ep_oracle_dispatch(T, K, H, dtype, fill_pads, zero_tail, cap, total, row_src,
                            g_result, NULL, g_expert_out, NULL);
}

/*
 * combine: for each token, the ordered binary32 sum over its valid routes
 * (k ascending) of the received rows, rounded once to the payload type.
 *
 *   rows     payload [cap*H]   expert outputs, expert-major
 *   out      payload [T*H]
 */
int ep_oracle_combine(int64_t T, int32_t K, int64_t H, int dtype, const int32_t* slot,
                      const void* rows, void* out) {
  if (T < 0 || K < 1 || H < 1 || !dtype_ok(dtype)) return ORACLE_ERR_ARGS;
  if (!fpenv_is_ieee()) return ORACLE_ERR_FPENV;
  ORACLE_PARALLEL_FOR
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      int have = 0;
      for (int32_t k = 0; k < K; ++k) {
        int32_t r = slot[t * K + k];
        if (r < 0) continue;
        float v = load_elem(rows, (int64_t)r * H + h, dtype);
        if (!have) {
          acc = v;
          have = 1;
        } else {
          acc = acc + v;
        }
      }
      if (have) {
        store_elem(out, t * H + h, dtype, acc);
      } else {
        store_zero(out, t * H + h, dtype);
      }
    }
  }
  return ORACLE_OK;
}

/*
 * dispatch_bwd: the token gradient is combine applied to the gradient of the
 * received rows; the weight gradient of route s is the gradient of the
 * received weight in its slot, or +0 when the route is masked or no weight
 * gradient is given (g_recv_w NULL).
 */
int ep_oracle_dispatch_bwd(int64_t T, int32_t K, int64_t H, int dtype, const int32_t* slot,
                           const void* g_recv, const float* g_recv_w, void* grad_tokens,
                           float* grad_w) {
  int rc = ep_oracle_combine(T, K, H, dtype, slot, g_recv, grad_tokens);
  if (rc != ORACLE_OK) return rc;
  if (!grad_w) return ORACLE_OK;
  ORACLE_PARALLEL_FOR
  for (int64_t s = 0; s < T * (int64_t)K; ++s) {
    int32_t r = slot[s];
    grad_w[s] = (r >= 0 && g_recv_w) ? g_recv_w[r] : 0.0f;
  }
  return ORACLE_OK;
}

/*
 * Weighted combine (the weight multiply folded into combine, the option the
 * review of "[PyTorch] Expert Parallelism: PyTorch wrapper + autograd ops
 * with symm-mem zero-copy" settles on in its thread on the weight multiply,
 * so the caller no longer pre-multiplies). For each token, over its valid
 * routes in ascending k with received row r:
 *   acc = w[r] * y[r]                     (first valid route: one fp32 product)
 *   acc = fmaf(w[r], y[r], acc)           (later routes: one fused rounding)
 * then one rounding to the payload type; +0 if no valid route.
 *   rows  payload [cap*H], w f32 [cap], out payload [T*H]
 */
int ep_oracle_combine_weighted(int64_t T, int32_t K, int64_t H, int dtype, const int32_t* slot,
                               const void* rows, const float* w, void* out) {
  if (T < 0 || K < 1 || H < 1 || !dtype_ok(dtype)) return ORACLE_ERR_ARGS;
  if (!fpenv_is_ieee()) return ORACLE_ERR_FPENV;
  ORACLE_PARALLEL_FOR
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      int have = 0;
      for (int32_t k = 0; k < K; ++k) {
        int32_t r = slot[t * K + k];
        if (r < 0) continue;
        float y = load_elem(rows, (int64_t)r * H + h, dtype);
        if (!have) {
          acc = w[r] * y;
          have = 1;
        } else {
          acc = fmaf(w[r], y, acc);
        }
      }
      if (have) {
        store_elem(out, t * H + h, dtype, acc);
      } else {
        store_zero(out, t * H + h, dtype);
      }
    }
  }
  return ORACLE_OK;
}

/*
 * Backward of the weighted combine, for every live received row r holding
 * route s of token t = s / K:
 *   grad_rows[r, h] = payload(fp32(w[r] * g[t, h]))       (pads: +0)
 *   grad_w[r]       = sum over h of g[t, h] * rows[r, h]   (pads: +0)
 * Pads are left as they are when fill_pads is 0; rows at or past
 * min(total, cap) are zeros when zero_tail is 1, else untouched. The weight
 * gradient is a
 * dot product whose summation order the method does not fix; the oracle
 * returns it from a double-precision sum of the exact products (grad_w64)
 * together with the sum of their magnitudes (abs_dot64), and the tests
 * compare the GPU's fp32 result within the summation error bound. grad_w64
 * may be NULL (then rows is not read).
 */
int ep_oracle_combine_weighted_bwd(int64_t T, int32_t K, int64_t H, int dtype, int fill_pads,
                                   int zero_tail, int64_t cap, int64_t total,
                                   const int32_t* row_src, const void* g, const void* rows,
                                   const float* w, void* grad_rows, double* grad_w64,
                                   double* abs_dot64) {
  if (T < 0 || K < 1 || H < 1 || cap < 0 || total < 0 || !dtype_ok(dtype))
    return ORACLE_ERR_ARGS;
  if (!fpenv_is_ieee()) return ORACLE_ERR_FPENV;
  const int64_t live = total < cap ? total : cap;
  if (zero_tail) {
    ORACLE_PARALLEL_FOR
    for (int64_t r = live; r < cap; ++r) {
      for (int64_t h = 0; h < H; ++h) store_zero(grad_rows, r * H + h, dtype);
      if (grad_w64) grad_w64[r] = 0.0;
      if (abs_dot64) abs_dot64[r] = 0.0;
    }
  }
  ORACLE_PARALLEL_FOR
  for (int64_t r = 0; r < live; ++r) {
    int32_t s = row_src[r];
    if (s < 0) {
      if (!fill_pads) continue;
      for (int64_t h = 0; h < H; ++h) store_zero(grad_rows, r * H + h, dtype);
      if (grad_w64) grad_w64[r] = 0.0;
      if (abs_dot64) abs_dot64[r] = 0.0;
      continue;
    }
    int64_t t = s / K;
    double dot = 0.0, adot = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      float gv = load_elem(g, t * H + h, dtype);
      float p = w[r] * gv;
      store_elem(grad_rows, r * H + h, dtype, p);
      if (grad_w64) {
        /* a product of two binary32 values is exact in binary64 */
        double term = (double)gv * (double)load_elem(rows, r * H + h, dtype);
        dot += term;
        adot += term < 0 ? -term : term;
      }
    }
    if (grad_w64) grad_w64[r] = dot;
    if (abs_dot64) abs_dot64[r] = adot;
  }
  return ORACLE_OK;
}
