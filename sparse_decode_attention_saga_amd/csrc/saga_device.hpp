// Device helpers for the SAGA + Atop-N decode kernels (gfx950, wave64).
//
// Score tiles use the CDNA matrix cores: a 16-key x 16-query-head tile of logits
// A = K q^T (eq. (2) of the paper's "Attention Mechanism Formalization") is one
// chain of MFMA instructions. The key tile is the A operand (rows = keys) and the
// query heads are the B operand (columns = heads). Each lane supplies the same
// slice of the head dimension to both operands, so the contraction is a plain
// dot product whatever order the hardware sums the slices in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saga {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 16 bytes seen as raw words, eight bf16 or four fp32.
union V16 {
  uint4 u;
  bf16x8 h;
  float f[4];
};

typedef uint16_t bf16_t;  // bf16 values are carried as their bit patterns

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }


__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Elements of type T in 16 bytes, as fp32. bf16: 8 values; fp32: 4 values.
template <typename T> struct Unpack;
template <> struct Unpack<bf16_t> {
  static constexpr int kN = 8;
  __device__ __forceinline__ static void run(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
};
template <> struct Unpack<float> {
  static constexpr int kN = 4;
  __device__ __forceinline__ static void run(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
};

// Order-preserving map fp32 -> uint32 (larger float <=> larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_to_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ----------------------------------------------------------------------------
// QK score tiles. One wave computes the logits of 16 consecutive keys against up
// to 16 query heads. After mma(): lane l holds A[key = 4*(l>>4) + r][head = l&15]
// in element r (the 16x16 MFMA accumulator layout).
template <typename T, int D> struct QK;

template <int D> struct QK<bf16_t, D> {
  static_assert(D % 32 == 0, "head dim must be a multiple of 32");
  static constexpr int kLoads = D / 32;  // 16-byte loads per lane per 16-key tile
  bf16x8 qf[kLoads];

  // q of local heads 0..nh-1 starts at `qh` (rows of D values). Columns hh >= nh
  // repeat head nh-1 (an unconditional load keeps every key load free to issue at
  // once); callers never use those columns.
  __device__ __forceinline__ void load_q(const bf16_t* qh, int nh, int lane) {
    const int hh = min(lane & 15, nh - 1), kq = lane >> 4;
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      V16 x;
      x.u = ld16(qh + (size_t)hh * D + 32 * s + 8 * kq);
      qf[s] = x.h;
    }
  }
  // This lane's slices of key row `krow` (the row of key 16*tile + (lane & 15)).
  __device__ __forceinline__ static void load_k(uint4 (&kb)[kLoads], const bf16_t* krow, int lane) {
    const int kq = lane >> 4;
#pragma unroll
    for (int s = 0; s < kLoads; ++s) kb[s] = ld16(krow + 32 * s + 8 * kq);
  }
  __device__ __forceinline__ floatx4 mma(const uint4 (&kb)[kLoads]) const {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      V16 x;
      x.u = kb[s];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.h, qf[s], acc, 0, 0, 0);
    }
    return acc;
  }
};

template <int D> struct QK<float, D> {
  static_assert(D % 16 == 0, "head dim must be a multiple of 16");
  static constexpr int kLoads = D / 16;
  float4 qf[kLoads];

  __device__ __forceinline__ void load_q(const float* qh, int nh, int lane) {
    const int hh = min(lane & 15, nh - 1), kq = lane >> 4;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      V16 x;
      x.u = ld16(qh + (size_t)hh * D + 16 * u + 4 * kq);
      qf[u] = make_float4(x.f[0], x.f[1], x.f[2], x.f[3]);
    }
  }
  __device__ __forceinline__ static void load_k(uint4 (&kb)[kLoads], const float* krow, int lane) {
    const int kq = lane >> 4;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) kb[u] = ld16(krow + 16 * u + 4 * kq);
  }
  __device__ __forceinline__ floatx4 mma(const uint4 (&kb)[kLoads]) const {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      V16 x;
      x.u = kb[u];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.f[0], qf[u].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.f[1], qf[u].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.f[2], qf[u].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.f[3], qf[u].w, acc, 0, 0, 0);
    }
    return acc;
  }
};

// Scaled logits of TPW consecutive 16-key tiles starting at key `wbase` (wave-uniform)
// of one key head, whose rows `rows` locates (row(i), and tile(t0) for the first row
// of a tile). Rows past the valid length L are clamped to L-1 for the load (always
// in bounds); callers mask them. Requires L >= 1. All TPW*kLoads loads of a lane are
// in flight together (the K stream is latency-bound per wave).
template <typename T, int D, int TPW, typename R>
__device__ __forceinline__ void score_tiles(floatx4 (&sc)[TPW], const QK<T, D>& qk, const R& rows,
                                            int wbase, int L, int lane, float scale) {
  uint4 kb[TPW][QK<T, D>::kLoads];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if constexpr (R::kPaged) {
      // a tile lies inside one page: one page lookup per tile, for the clamped tile
      const int t0 = min(wbase + 16 * t, (L - 1) & ~15);
      const int key = min(t0 + (lane & 15), L - 1);
      QK<T, D>::load_k(kb[t], rows.tile(t0) + (size_t)(key - t0) * D, lane);
    } else {
      const int key = min(wbase + 16 * t + (lane & 15), L - 1);
      QK<T, D>::load_k(kb[t], rows.row(key), lane);
    }
  }
  // every key load of the wave is issued before the first MFMA waits on one
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const floatx4 a = qk.mma(kb[t]);
    sc[t] = a * scale;
  }
}

// ----------------------------------------------------------------------------
// Block-wide helpers for blocks of NT threads (a multiple of 64, at most 1024).
// Every thread of the block must call them. Scratch arrays are __shared__.

template <int CTRL, int ROWS = 0xf, int BANKS = 0xf>
__device__ __forceinline__ int dpp_add_src(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, BANKS, false);
}

// Inclusive prefix sum over the 64 lanes (gfx9 DPP: shifts within rows of 16 lanes,
// then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int x, int /*lane*/) {
  int s = x;
  s += dpp_add_src<0x111>(0, x);             // row_shr:1
  s += dpp_add_src<0x112>(0, x);             // row_shr:2
  s += dpp_add_src<0x113>(0, x);             // row_shr:3  (lane i: x[i-3..i] within its row)
  s += dpp_add_src<0x114, 0xf, 0xe>(0, s);   // row_shr:4, lanes 4..15 of each row
  s += dpp_add_src<0x118, 0xf, 0xc>(0, s);   // row_shr:8, lanes 8..15 of each row
  s += dpp_add_src<0x142, 0xa>(0, s);        // row_bcast:15 into rows 1 and 3
  s += dpp_add_src<0x143, 0xc>(0, s);        // row_bcast:31 into rows 2 and 3
  return s;
}

// Inclusive prefix sum within each row of 16 lanes (the row-local steps above).
__device__ __forceinline__ int row_incl_scan(int x) {
  int s = x;
  s += dpp_add_src<0x111>(0, x);             // row_shr:1
  s += dpp_add_src<0x112>(0, x);             // row_shr:2
  s += dpp_add_src<0x113>(0, x);             // row_shr:3
  s += dpp_add_src<0x114, 0xf, 0xe>(0, s);   // row_shr:4, lanes 4..15 of each row
  s += dpp_add_src<0x118, 0xf, 0xc>(0, s);   // row_shr:8, lanes 8..15 of each row
  return s;
}

// Exclusive prefix sum in thread order; `total` gets the block sum. tmp: int[NT/64].
template <int NT = kBlock>
__device__ __forceinline__ int block_excl_scan(int x, int* tmp, int& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int inc = wave_incl_scan(x, lane);
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = tmp[i];
    off += (i < w) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + inc - x;
}

// Two exclusive prefix sums at once (one pass of barriers); totals in ta and tb.
// tmp: int[2 * NT/64].
template <int NT = kBlock>
__device__ __forceinline__ int2 block_excl_scan2(int a, int b, int* tmp, int& ta, int& tb) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
  if (lane == kWave - 1) {
    tmp[w] = ia;
    tmp[NW + w] = ib;
  }
  __syncthreads();
  int oa = 0, ob = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = tmp[i], y = tmp[NW + i];
    oa += (i < w) ? x : 0;
    ob += (i < w) ? y : 0;
    sa += x;
    sb += y;
  }
  __syncthreads();
  ta = sa;
  tb = sb;
  return make_int2(oa + ia - a, ob + ib - b);
}

// Wave reductions with DPP row operations (gfx9): sums and maxima within quads, then
// half-rows, rows of 16, and across the four rows with the row broadcasts of lanes
// 15 and 31; the total ends in lane 63 and is read back as a wave-uniform value.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

constexpr int kDppRor4 = 0x124;       // row_ror:4
constexpr int kDppRor8 = 0x128;       // row_ror:8

// Sum of lanes i, i+4, i+8, i+12 (mod 16) within each row of 16 lanes, in every lane.
__device__ __forceinline__ float row_stride4_sum(float x) {
  x += __int_as_float(dpp_i<kDppRor4>(0, __float_as_int(x)));
  x += __int_as_float(dpp_i<kDppRor8>(0, __float_as_int(x)));
  return x;
}

// x[l] op x[l ^ m] for m = 8 (DPP rotate by 8 within rows of 16 lanes), 16 and 32
// (gfx950 permlane swaps: the two returned halves hold x and its partner).
template <int M, typename Op>
__device__ __forceinline__ float xor_lanes(float x, Op op) {
  static_assert(M == 8 || M == 16 || M == 32, "lane distance 8, 16 or 32");
  if constexpr (M == 8) {
    return op(x, __int_as_float(dpp_i<kDppRor8>(0, __float_as_int(x))));
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}
// Sum (or maximum) over lanes l, l + G, l + 2G, ... of the wave (G = 8, 16 or 32).
template <int G>
__device__ __forceinline__ float strided_lane_sum(float x) {
  auto add = [](float u, float v) { return u + v; };
  if constexpr (G <= 8) x = xor_lanes<8>(x, add);
  if constexpr (G <= 16) x = xor_lanes<16>(x, add);
  return xor_lanes<32>(x, add);
}
template <int G>
__device__ __forceinline__ float strided_lane_max(float x) {
  auto mx = [](float u, float v) { return fmaxf(u, v); };
  if constexpr (G <= 8) x = xor_lanes<8>(x, mx);
  if constexpr (G <= 16) x = xor_lanes<16>(x, mx);
  return xor_lanes<32>(x, mx);
}

template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int x, int neutral, Op op) {
  x = op(x, dpp_i<kDppXor1>(neutral, x));
  x = op(x, dpp_i<kDppXor2>(neutral, x));
  x = op(x, dpp_i<kDppHalfMirror>(neutral, x));
  x = op(x, dpp_i<kDppMirror>(neutral, x));
  x = op(x, dpp_i<kDppBcast15, 0xA>(neutral, x));
  x = op(x, dpp_i<kDppBcast31, 0xC>(neutral, x));
  return __builtin_amdgcn_readlane(x, kWave - 1);
}
__device__ __forceinline__ float wave_max(float x) {
  return __int_as_float(wave_reduce_i(__float_as_int(x), __float_as_int(-INFINITY), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum(float x) {
  return __int_as_float(wave_reduce_i(__float_as_int(x), 0, [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}
__device__ __forceinline__ int wave_sum_i(int x) {
  return wave_reduce_i(x, 0, [](int a, int b) { return a + b; });
}

// Block maximum of `mx` and exclusive prefix sum of `x` in thread order, with one
// barrier; `total` gets the block sum. fmp: float[NT/64], itmp: int[NT/64]; neither
// may be written again before the caller's next barrier.
template <int NT = kBlock>
__device__ __forceinline__ int block_max_excl_scan(float mx, int x, float* fmp, int* itmp, float& M, int& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const float wm = wave_max(mx);
  const int inc = wave_incl_scan(x, lane);
  if (lane == kWave - 1) {
    itmp[w] = inc;
    fmp[w] = wm;
  }
  __syncthreads();
  int off = 0, tot = 0;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = itmp[i];
    off += (i < w) ? t : 0;
    tot += t;
    m = fmaxf(m, fmp[i]);
  }
  M = m;
  total = tot;
  return off + inc - x;
}

// tmp: float[NT/64] (int[NT/64] for the integer sum).
template <int NT = kBlock>
__device__ __forceinline__ float block_max(float x, float* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_max(x);
  if (lane == 0) tmp[w] = x;
  __syncthreads();
  float r = tmp[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, tmp[i]);
  __syncthreads();
  return r;
}
template <int NT = kBlock>
__device__ __forceinline__ float block_sum(float x, float* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_sum(x);
  if (lane == 0) tmp[w] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}
template <int NT = kBlock>
__device__ __forceinline__ int block_sum_i(int x, int* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_sum_i(x);
  if (lane == 0) tmp[w] = x;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}

// ----------------------------------------------------------------------------
// MSB-first radix selection of the k-th largest (k >= 1) order key, 8 bits per pass.

// Given a 256-bin histogram `hist` (shared), find the digit whose bin holds the k-th
// largest element counting from the top bin; res[0] = digit, res[1] = rank of the
// element inside that bin. If the bins hold fewer than k elements res is left at
// (0, 1). With `bin_count`, *bin_count = the count of the chosen bin (0 if none). The
// first wave does the search (four bins per lane from the top, a prefix sum over the
// lanes); one barrier follows. itmp is unused.
template <int NT = kBlock>
__device__ __forceinline__ void digit_of_kth_largest(const unsigned* hist, unsigned k, int* /*itmp*/,
                                                     unsigned* res, unsigned* bin_count = nullptr) {
  static_assert(NT >= kWave, "at least one wave");
  const int t = threadIdx.x;
  if (t < kWave) {
    unsigned c[4];
    unsigned sum = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = hist[255 - 4 * t - e];
      sum += c[e];
    }
    unsigned above = (unsigned)wave_incl_scan((int)sum, t) - sum;  // elements in the bins above lane t's
    if (t == 0) {
      res[0] = 0u;
      res[1] = 1u;
      if (bin_count) *bin_count = 0u;
    }
    // the lane holding the k-th largest writes after the default (same wave, in order)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (above < k && k <= above + c[e]) {
        res[0] = (unsigned)(255 - 4 * t - e);
        res[1] = k - above;
        if (bin_count) *bin_count = c[e];
      }
      above += c[e];
    }
  }
  __syncthreads();
}

// The order key of the k-th largest of vals[0..n) among the values whose key
// matches `prefix` on the bits of `mask`, resolving bits shift_start+7..0, 8 per
// pass. Once at most kWave values match the resolved prefix, they are copied to LDS
// and the first wave ranks them directly (each lane counts the values above and not
// below its own), which takes the place of the remaining passes.
// `vals` may point to global or shared memory.
template <int NT = kBlock>
__device__ __forceinline__ uint32_t radix_select_block(const float* vals, long long n, uint32_t prefix,
                                                       uint32_t mask, int shift_start, unsigned k,
                                                       unsigned* hist, int* itmp, unsigned* res) {
  __shared__ uint32_t s_few[kWave];
  __shared__ unsigned s_nfew, s_left;
  const int tid = threadIdx.x;
  for (int shift = shift_start; shift >= 0; shift -= 8) {
    for (int e = tid; e < 256; e += NT) hist[e] = 0u;
    __syncthreads();
    for (long long i0 = 0; i0 < n; i0 += 4LL * NT) {
      float v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long long i = i0 + (long long)u * NT + tid;
        v4[u] = (i < n) ? vals[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long long i = i0 + (long long)u * NT + tid;
        const uint32_t key = order_key(v4[u]);
        if (i < n && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    digit_of_kth_largest<NT>(hist, k, itmp, res, &s_left);
    // the next pass clears hist (no longer read) and writes res and s_left only after
    // two barriers
    prefix |= res[0] << shift;
    mask |= 255u << shift;
    k = res[1];
    const unsigned left = s_left;  // values matching the new prefix
    if (shift > 0 && left <= (unsigned)kWave) {
      if (tid == 0) s_nfew = 0u;
      __syncthreads();
      for (long long i0 = 0; i0 < n; i0 += 4LL * NT) {
        float v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const long long i = i0 + (long long)u * NT + tid;
          v4[u] = (i < n) ? vals[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const long long i = i0 + (long long)u * NT + tid;
          const uint32_t key = order_key(v4[u]);
          if (i < n && (key & mask) == prefix) s_few[atomicAdd(&s_nfew, 1u)] = key;
        }
      }
      __syncthreads();
      if (tid < kWave) {
        // the k-th largest of the `left` values (k <= left): a lane whose value has
        // fewer than k values above it and at least k not below it
        const uint32_t mine = tid < (int)left ? s_few[tid] : 0u;
        unsigned above = 0u, not_below = 0u;
        for (unsigned i = 0; i < left; ++i) {
          const uint32_t o = s_few[i];
          above += o > mine ? 1u : 0u;
          not_below += o >= mine ? 1u : 0u;
        }
        if (tid < (int)left && above < k && k <= not_below) res[0] = mine;  // equal values write the same
      }
      __syncthreads();
      prefix = res[0];
      break;
    }
  }
  __syncthreads();
  return prefix;
}

}  // namespace saga
