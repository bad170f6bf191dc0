// Kernels of the SAGA + Atop-N decode step and of the dense GQA baseline (gfx950).
//
// Stale-threshold step:  k_qk_select -> k_gather_split
// Refresh step:          k_scores_hist -> k_cand_collect -> k_select_finish
//                        -> k_qk_select<from stored logits> -> k_gather_split
// Dense GQA baseline:    k_dense_partial -> k_dense_combine
//
// No kernel waits on another workgroup: exchanges go through kernel boundaries, or
// through device-scope atomics whose last arrival finishes the work (device-scope
// fences are avoided: on this GPU they write back and invalidate the whole L2).
//
// Paper: "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
// (summary page picx.dev DRD92V): eq. (2) logits, section "Methodology > Atop-N
// Attention" (threshold = N-th largest logit, elementwise comparison, exact
// threshold refreshed every n steps), eq. (7) sparse softmax-PV, section "SAGA
// Architecture" (h_k key heads, h_v value heads).
#pragma once

#include "saga_device.cuh"

namespace saga {

// Keys per block of the key-streaming kernels: 4 waves x TPW tiles x 16 keys.
#ifndef SAGA_KEY_BYTES_PER_WAVE
#define SAGA_KEY_BYTES_PER_WAVE 16384  // K bytes one wave has in flight per chunk
#endif
template <typename T, int D> struct StreamCfg {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kTPW = SAGA_KEY_BYTES_PER_WAVE / (16 * kRowBytes) > 0 ? SAGA_KEY_BYTES_PER_WAVE / (16 * kRowBytes) : 1;  // 16-key tiles per wave
  static_assert(kTPW >= 1, "at least one tile per wave");
  static constexpr int kChunk = 16 * kTPW * kWaves;
};

constexpr int kBufDword3 = 0x00020000;  // buffer resource word 3 for raw gfx9 buffers
constexpr int kCoherent = 16;           // sc1 cache policy: coherent across the device's L2s

// ----------------------------------------------------------------------------
// Shared argument blocks (passed by value).

struct StreamArgs {
  const void* q;           // [B, h_q, D]
  const void* k;           // [B, h_k, l_max, D]
  const int32_t* l_kv;     // [B]
  const float* tau;        // [B*h_q] threshold (select kernels)
  float* scores;           // [B*h_q, lpad] fp32 logits (refresh steps and forced refresh)
  int32_t* surv_idx;       // [B*h_q, lpad] kept indices, one CH-segment per chunk
  float* surv_val;         // [B*h_q, lpad] kept logits; also the threshold candidates
  int32_t* chunk_cnt;      // [B*h_q, nch] kept entries per chunk
  float* chunk_max;        // [B*h_q, nch] largest kept logit per chunk
  unsigned* hist;          // [B*h_q, 256] top-digit histogram (zero between calls)
  unsigned* cand_cnt;      // [B*h_q] candidates of the threshold select (zero between calls)
  int h_q, h_k, g_k, htiles, l_max, nch, N;
  int max_l_kv;            // host bound of l_kv[]; larger device values are clamped
  long long lpad;
  float scale;
  float* zero_f;           // k_qk_select clears [zero_n] floats here (the gather's accumulators)
  long long zero_n;
};

// Source of the logits of k_qk_select.
enum SelectMode { kFromKeys = 0, kFromKeysSpeculative = 1, kFromScores = 2 };

// ----------------------------------------------------------------------------
// Logits of one chunk of keys for the (up to) 16 query heads of one head tile, then
// the Atop-N comparison against each head's threshold. Kept (index, logit) pairs go
// to the chunk's segment of the row's kept list; the chunk's count and largest kept
// logit are recorded. MODE kFromScores reads the logits stored by k_scores_hist (a
// refresh step: the fp32 values the threshold was selected from); MODE
// kFromKeysSpeculative (one sequence) issues the key loads before l_kv arrives.
// Every block also clears its share of the gather's accumulators.
// grid = (nch, h_k * htiles, B), block = 256.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kBlock) void k_qk_select(const StreamArgs a) {
  constexpr int TPW = StreamCfg<T, D>::kTPW;
  constexpr int CH = StreamCfg<T, D>::kChunk;
  const int c = blockIdx.x, gy = blockIdx.y, b = blockIdx.z;
  const int g = gy / a.htiles, ht = gy - g * a.htiles;
  const int j0 = g * a.g_k + ht * 16;
  const int nh = min(16, a.g_k - ht * 16);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * a.h_q + j0;
  const int base = c * CH;
  const int wbase = base + wv * 16 * TPW;
  const bool live = hh < nh;

  floatx4 sc[TPW];
  QK<T, D> qk;
  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.h_k + g) * a.l_max * D;
  if constexpr (MODE == kFromKeysSpeculative) {
    qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, nh, lane);
    score_tiles<T, D, TPW>(sc, qk, kh, wbase, a.max_l_kv, lane, a.scale);
  }
  {
    const long long nblk = (long long)gridDim.x * gridDim.y * gridDim.z;
    const long long id = blockIdx.x + (long long)gridDim.x * (blockIdx.y + (long long)gridDim.y * blockIdx.z);
    const long long per = (a.zero_n + nblk - 1) / nblk;
    for (long long i = id * per + tid; i < min(a.zero_n, (id + 1) * per); i += kBlock) a.zero_f[i] = 0.f;
  }
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (base >= L) return;

  __shared__ int s_cnt[16];
  __shared__ unsigned s_max[16];
  if (tid < 16) {
    s_cnt[tid] = 0;
    s_max[tid] = 0u;
  }
  const float tau_l = live ? a.tau[row0 + hh] : 0.f;
  if constexpr (MODE == kFromScores) {
    const float* srow = a.scores + (long long)(row0 + (live ? hh : 0)) * a.lpad;
#pragma unroll
    for (int t = 0; t < TPW; ++t) sc[t] = *reinterpret_cast<const floatx4*>(srow + wbase + 16 * t + 4 * kq);
  } else if constexpr (MODE == kFromKeys) {
    qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, nh, lane);
    score_tiles<T, D, TPW>(sc, qk, kh, wbase, L, lane, a.scale);
  }
  __syncthreads();

  const long long seg = (long long)(row0 + hh) * a.lpad + base;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = wbase + 16 * t + 4 * kq + r;
      const float v = sc[t][r];
      if (live && key < L && v >= tau_l) {
        const int slot = atomicAdd(&s_cnt[hh], 1);
        a.surv_idx[seg + slot] = key;
        a.surv_val[seg + slot] = v;
        atomicMax(&s_max[hh], order_key(v));
      }
    }
  }
  __syncthreads();
  if (tid < nh) {
    const long long o = (long long)(row0 + tid) * a.nch + c;
    a.chunk_cnt[o] = s_cnt[tid];
    a.chunk_max[o] = order_key_to_f32(s_max[tid]);
  }
}

// ----------------------------------------------------------------------------
// Refresh, pass 1: logits of every cached key stored as fp32, plus a histogram of
// the top 8 bits of their order keys per query head (accumulated into a.hist).
// grid = (nch, h_k * htiles, B), block = 256.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void k_scores_hist(const StreamArgs a) {
  constexpr int TPW = StreamCfg<T, D>::kTPW;
  constexpr int CH = StreamCfg<T, D>::kChunk;
  const int c = blockIdx.x, gy = blockIdx.y, b = blockIdx.z;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int base = c * CH;
  if (base >= L) return;
  const int g = gy / a.htiles, ht = gy - g * a.htiles;
  const int j0 = g * a.g_k + ht * 16;
  const int nh = min(16, a.g_k - ht * 16);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * a.h_q + j0;

  __shared__ unsigned s_hist[16 * 256];
  for (int e = tid; e < 16 * 256; e += kBlock) s_hist[e] = 0u;

  QK<T, D> qk;
  qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, nh, lane);
  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.h_k + g) * a.l_max * D;
  const int wbase = base + wv * 16 * TPW;
  floatx4 sc[TPW];
  score_tiles<T, D, TPW>(sc, qk, kh, wbase, L, lane, a.scale);
  __syncthreads();

  const bool live = hh < nh;
  if (live) {
    float* srow = a.scores + (long long)(row0 + hh) * a.lpad;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      floatx4 v = sc[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = wbase + 16 * t + 4 * kq + r;
        if (key < L) atomicAdd(&s_hist[hh * 256 + (order_key(v[r]) >> 24)], 1u);
        else v[r] = -INFINITY;
      }
      *reinterpret_cast<floatx4*>(srow + wbase + 16 * t + 4 * kq) = v;
    }
  }
  __syncthreads();
  for (int e = tid; e < nh * 256; e += kBlock) {
    const unsigned h = s_hist[e];
    if (h) atomicAdd(&a.hist[(long long)(row0 + e / 256) * 256 + (e & 255)], h);
  }
}

// ----------------------------------------------------------------------------
// Refresh, pass 2: candidates for the exact threshold. The top-digit histogram of a
// row gives the 8-bit bin that holds its N-th largest logit; each block copies the
// logits of its slice that fall in that bin to the row's candidate list (stored in
// the row's kept-logit buffer, free at this point of a refresh step).
// grid = (P, h_q, B) with P = ceil(max_l_kv / kSelSlice), block = 256.
constexpr int kSelSlice = 4096;   // logits scanned per block
constexpr int kCandLds = 8192;    // candidates the finishing block stages in LDS
constexpr int kRowThreads = 1024; // threads of the one-block-per-row kernels

__global__ __launch_bounds__(kBlock) void k_cand_collect(const StreamArgs a) {
  const int p = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const long long row = (long long)b * a.h_q + j;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int N = a.N;
  const int tid = threadIdx.x;
  const int lo = p * kSelSlice;
  if (L <= 0 || N >= L || lo >= L) return;  // uniform over the block
  const long long rbase = row * a.lpad;

  __shared__ unsigned s_hist[256];
  __shared__ int s_itmp[kWaves];
  __shared__ unsigned s_res[2];
  __shared__ float s_cand[kSelSlice];
  __shared__ int s_cc, s_base;

  s_hist[tid] = a.hist[row * 256 + tid];
  if (tid == 0) s_cc = 0;
  __syncthreads();
  digit_of_kth_largest(s_hist, (unsigned)N, s_itmp, s_res);
  const unsigned d1 = s_res[0];
  const int hi = min(lo + kSelSlice, L);
  constexpr int PER = kSelSlice / kBlock;
  float vals[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = lo + u * kBlock + tid;
    vals[u] = (i < hi) ? a.scores[rbase + i] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = lo + u * kBlock + tid;
    if (i < hi && (order_key(vals[u]) >> 24) == d1) s_cand[atomicAdd(&s_cc, 1)] = vals[u];
  }
  __syncthreads();
  const int cnt = s_cc;
  if (tid == 0 && cnt > 0) s_base = (int)atomicAdd(&a.cand_cnt[row], (unsigned)cnt);
  __syncthreads();
  for (int i = tid; i < cnt; i += kBlock) a.surv_val[rbase + s_base + i] = s_cand[i];
}

// Refresh, pass 3: the remaining 24 bits of the N-th largest logit resolved on the
// candidates (counting repeats); writes tau (-inf when N >= l_kv, unchanged when
// l_kv == 0) and returns the row's histogram and candidate count to zero.
// grid = (h_q, B), block = 1024.
__global__ __launch_bounds__(kRowThreads) void k_select_finish(const StreamArgs a, float* tau_out) {
  constexpr int NT = kRowThreads;
  const int j = blockIdx.x, b = blockIdx.y;
  const long long row = (long long)b * a.h_q + j;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int N = a.N;
  const int tid = threadIdx.x;
  if (L <= 0) return;

  __shared__ unsigned s_hist[256];
  __shared__ int s_itmp[NT / kWave];
  __shared__ unsigned s_res[2];
  __shared__ float s_cand[kCandLds];

  if (N >= L) {
    if (tid == 0) tau_out[row] = -INFINITY;
    if (tid < 256) a.hist[row * 256 + tid] = 0u;
    return;
  }
  if (tid < 256) s_hist[tid] = a.hist[row * 256 + tid];
  __syncthreads();
  digit_of_kth_largest<NT>(s_hist, (unsigned)N, s_itmp, s_res);
  const unsigned d1 = s_res[0], k1 = s_res[1];
  const unsigned C = a.cand_cnt[row];
  const float* cand = a.surv_val + row * a.lpad;
  if (C <= (unsigned)kCandLds) {
    for (int i0 = 0; i0 < (int)C; i0 += 4 * NT) {
      float t4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        t4[u] = (i < (int)C) ? cand[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        if (i < (int)C) s_cand[i] = t4[u];
      }
    }
    __syncthreads();
    cand = s_cand;
  }
  const uint32_t key = radix_select_block<NT>(cand, (long long)C, d1 << 24, 0xff000000u, 16, k1, s_hist,
                                              s_itmp, s_res);
  if (tid == 0) {
    tau_out[row] = order_key_to_f32(key);
    a.cand_cnt[row] = 0u;
  }
  if (tid < 256) a.hist[row * 256 + tid] = 0u;
}

// ----------------------------------------------------------------------------
// Sparse softmax and value gather (eq. (7)) over the kept entries of one row.

struct GatherArgs {
  StreamArgs s;           // q, k, l_kv, logit buffer, kept lists and counts
  const void* v;          // [B, h_v, l_max, D]
  float* tau;             // [B*h_q] (written only where a row is refreshed)
  void* out;              // [B*h_q, D]
  int32_t* sel_count;     // [B*h_q] or null
  int32_t* sel_idx;       // [B*h_q, sel_cap] or null
  int32_t* flags;         // [B*h_q] or null
  int h_v, sel_cap, out_bf16, refreshed;
  float* acc;             // [B*h_q][D+4] sum of w*v (D), sum of w; cleared by k_qk_select
  unsigned* row_done;     // [B*h_q] finished blocks per row; cleared by k_qk_select
};

template <int D>
__device__ __forceinline__ void store_out(const GatherArgs& a, long long row, int d, float x) {
  if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16(x);
  else reinterpret_cast<float*>(a.out)[row * D + d] = x;
}

// Work split of a value-row gather: groups of G lanes read one 16-byte slice each of
// a D-wide row; NG groups per block of NT threads.
template <typename T, int D, int NT>
struct RowGather {
  static constexpr int EPL = Unpack<T>::kN;  // columns per lane
  static constexpr int G = D / EPL;          // lanes per value row
  static constexpr int NG = NT / G;          // rows in flight per block pass (x U)
  static constexpr int U = 8;                // rows per group per pass
};

// Sum the per-lane accumulators of a block into s_red[0][0..D) and the weight sums
// into s_z[0] (shuffles inside each wave, then one LDS pass). s_red: [NT/64][D].
template <typename T, int D, int NT>
__device__ __forceinline__ void reduce_rows(float* acc, float z, float (*s_red)[D], float* s_z) {
  using RG = RowGather<T, D, NT>;
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
#pragma unroll
  for (int off = RG::G; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < RG::EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
    z += __shfl_xor(z, off);
  }
  if (lane < RG::G) {
#pragma unroll
    for (int e = 0; e < RG::EPL; ++e) s_red[wv][lane * RG::EPL + e] = acc[e];
  }
  if (lane == 0) s_z[wv] = z;
  __syncthreads();
  for (int col = tid; col < D; col += NT) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) x += s_red[w][col];
    s_red[0][col] = x;  // each column is read and written by one thread only
  }
  if (tid == 0) {
    float zz = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) zz += s_z[w];
    s_z[0] = zz;
  }
  __syncthreads();
}

// One row (b, j) computed exactly by one block: the logits of every key with the same
// tiles as the streaming kernels (into the row's logit buffer), optionally the exact
// N-th largest as a new threshold (a forced refresh), then the kept set, its maximum
// and the sparse softmax-PV. Used where the fast paths cannot answer: a stale
// threshold that keeps nothing, or a logit range too wide for the fixed-reference
// accumulation. Writes out, tau (refresh only), sel_count, sel_idx and flags.
template <typename T, int D, int NT>
__device__ void exact_row(const GatherArgs& a, int b, int j, int L, bool refresh_tau, float (*s_red)[D],
                          float* s_z) {
  constexpr int NW = NT / kWave;
  constexpr int TPW = StreamCfg<T, D>::kTPW;
  using RG = RowGather<T, D, NT>;
  const StreamArgs& s = a.s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const long long row = (long long)b * s.h_q + j;
  const long long rbase = row * s.lpad;
  const int g = j / s.g_k;
  const int jt = (j - g * s.g_k) / 16;
  const int j0 = g * s.g_k + jt * 16;
  const int nh = min(16, s.g_k - jt * 16);
  const int jj = j - j0;

  {
    QK<T, D> qk;
    qk.load_q(reinterpret_cast<const T*>(s.q) + (size_t)(b * s.h_q + j0) * D, nh, lane);
    const T* kh = reinterpret_cast<const T*>(s.k) + (size_t)(b * s.h_k + g) * s.l_max * D;
    const int kq = lane >> 4;
    for (int base = 0; base < L; base += NW * 16 * TPW) {
      const int wbase = base + wv * 16 * TPW;
      if (wbase < L) {
        floatx4 sc[TPW];
        score_tiles<T, D, TPW>(sc, qk, kh, wbase, L, lane, s.scale);
        if ((lane & 15) == jj) {
#pragma unroll
          for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = wbase + 16 * t + 4 * kq + r;
              if (key < L) s.scores[rbase + key] = sc[t][r];
            }
        }
      }
    }
  }
  __syncthreads();

  __shared__ unsigned s_hist[256];
  __shared__ int s_itmp[NW];
  __shared__ unsigned s_res[2];
  __shared__ float s_ftmp[NW];
  __shared__ int s_list_i[NT];
  __shared__ float s_list_v[NT];
  __shared__ int s_n;

  const float* srow = s.scores + rbase;
  float tau = a.tau[row];
  if (refresh_tau) {
    tau = -INFINITY;
    if (s.N < L)
      tau = order_key_to_f32(radix_select_block<NT>(srow, L, 0u, 0u, 24, (unsigned)s.N, s_hist, s_itmp, s_res));
  }
  float m = -INFINITY;
  for (int i = tid; i < L; i += NT) {
    const float v = srow[i];
    if (v >= tau) m = fmaxf(m, v);
  }
  m = block_max<NT>(m, s_ftmp);

  const int vh = (int)(((long long)j * a.h_v) / s.h_q);
  const int grp = tid / RG::G, gl = tid - grp * RG::G;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.h_v + vh) * s.l_max * D + gl * RG::EPL;
  float acc[RG::EPL];
#pragma unroll
  for (int e = 0; e < RG::EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
  int kept = 0;
  for (int base = 0; base < L; base += NT) {
    if (tid == 0) s_n = 0;
    __syncthreads();
    const int i = base + tid;
    if (i < L) {
      const float v = srow[i];
      if (v >= tau) {
        const int slot = atomicAdd(&s_n, 1);
        s_list_i[slot] = i;
        s_list_v[slot] = v;
      }
    }
    __syncthreads();
    const int n = s_n;
    for (int p = grp; p < n; p += RG::NG) {
      const int idx = s_list_i[p];
      const float w = expf(s_list_v[p] - m);
      float x[RG::EPL];
      Unpack<T>::run(ld16(vbase + (size_t)idx * D), x);
#pragma unroll
      for (int e = 0; e < RG::EPL; ++e) acc[e] += w * x[e];
      z += w;
      if (gl == 0 && a.sel_idx && kept + p < a.sel_cap) a.sel_idx[row * a.sel_cap + kept + p] = idx;
    }
    kept += n;
    __syncthreads();
  }
  reduce_rows<T, D, NT>(acc, z, s_red, s_z);
  for (int d = tid; d < D; d += NT) store_out<D>(a, row, d, kept > 0 ? s_red[0][d] / s_z[0] : 0.f);
  if (tid == 0) {
    if (refresh_tau) a.tau[row] = tau;
    if (a.sel_count) a.sel_count[row] = kept;
    if (a.flags) a.flags[row] = refresh_tau ? 3 : (a.refreshed ? 1 : 0);
  }
  __syncthreads();
}

// Split gather: P blocks per row (b, j). Every block reads the row's chunk counts
// and maxima (so all use the row maximum m as the softmax reference and their sums
// add directly), takes list positions [T*s/P, T*(s+1)/P) of the row's kept list
// (chunk order), gathers those value rows of value head v(j) and adds its sum of
// w*v and of w, w = exp(A - m), to the row's accumulator (device-scope atomics,
// fan-in P). The last of the P blocks to finish divides and writes the row. A row
// that kept nothing is recomputed exactly by block 0 (forced refresh).
// grid = (P, h_q, B), block = 256.
constexpr int kSplitWindow = 1024;  // list positions a block stages in LDS per pass
constexpr int kChunkRegs = 8;       // chunk counts a thread keeps in registers

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void k_gather_split(const GatherArgs a) {
  constexpr int NT = kBlock;
  constexpr int NW = NT / kWave;
  constexpr int CH = StreamCfg<T, D>::kChunk;
  constexpr int AS = D + 4;
  using RG = RowGather<T, D, NT>;
  constexpr int U = 4;
  const StreamArgs& sa = a.s;
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int P = gridDim.x;
  const long long row = (long long)b * sa.h_q + j;
  const int L = min(sa.l_kv[b], sa.max_l_kv);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

  __shared__ int s_itmp[NW];
  __shared__ float s_ftmp[NW];
  __shared__ int s_li[kSplitWindow];
  __shared__ float s_lv[kSplitWindow];
  __shared__ float s_red[NW][D];
  __shared__ float s_z[NW];
  __shared__ int s_last;

  if (L <= 0) {
    if (s == 0) {
      for (int d = tid; d < D; d += NT) store_out<D>(a, row, d, 0.f);
      if (tid == 0) {
        if (a.sel_count) a.sel_count[row] = 0;
        if (a.flags) a.flags[row] = 0;
      }
    }
    return;
  }
  const long long rbase = row * sa.lpad;
  const long long cbase = row * sa.nch;
  const int nch_b = (L + CH - 1) / CH;
  const int cpt = (nch_b + NT - 1) / NT;  // consecutive chunks per thread
  const int c0 = tid * cpt, c1 = min(nch_b, c0 + cpt);

  // counts and maxima of this thread's chunks (kept in registers when few)
  int nreg[kChunkRegs];
  float m = -INFINITY;
  int tsum = 0;
#pragma unroll
  for (int k = 0; k < kChunkRegs; ++k) {
    const int c = c0 + k;
    nreg[k] = 0;
    if (c < c1) {
      const int n = sa.chunk_cnt[cbase + c];
      const float mx = sa.chunk_max[cbase + c];
      nreg[k] = n;
      tsum += n;
      m = fmaxf(m, n > 0 ? mx : -INFINITY);
    }
  }
  for (int c = c0 + kChunkRegs; c < c1; ++c) {
    const int n = sa.chunk_cnt[cbase + c];
    tsum += n;
    if (n > 0) m = fmaxf(m, sa.chunk_max[cbase + c]);
  }
  m = block_max<NT>(m, s_ftmp);
  int total;
  const int tpre = block_excl_scan<NT>(tsum, s_itmp, total);
  if (total == 0) {
    if (s == 0) exact_row<T, D, NT>(a, b, j, L, true, s_red, s_z);
    return;
  }
  const int lo = (int)(((long long)total * s) / P), hi = (int)(((long long)total * (s + 1)) / P);

  const int vh = (int)(((long long)j * a.h_v) / sa.h_q);
  const int grp = tid / RG::G, gl = tid - grp * RG::G;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.h_v + vh) * sa.l_max * D + gl * RG::EPL;
  float acc[RG::EPL];
#pragma unroll
  for (int e = 0; e < RG::EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
  for (int w0 = lo; w0 < hi; w0 += kSplitWindow) {
    const int w1 = min(hi, w0 + kSplitWindow);
    // each thread stages its own chunks' kept entries that fall in [w0, w1)
    int pos = tpre;
#pragma unroll
    for (int k = 0; k < kChunkRegs; ++k) {
      const int c = c0 + k;
      if (c < c1 && pos < w1) {
        const int n = nreg[k];
        const int q0 = max(pos, w0), q1 = min(pos + n, w1);
        for (int q = q0; q < q1; ++q) {
          const long long off = rbase + (long long)c * CH + (q - pos);
          s_li[q - w0] = sa.surv_idx[off];
          s_lv[q - w0] = sa.surv_val[off];
        }
        pos += n;
      }
    }
    for (int c = c0 + kChunkRegs; c < c1 && pos < w1; ++c) {
      const int n = sa.chunk_cnt[cbase + c];
      const int q0 = max(pos, w0), q1 = min(pos + n, w1);
      for (int q = q0; q < q1; ++q) {
        const long long off = rbase + (long long)c * CH + (q - pos);
        s_li[q - w0] = sa.surv_idx[off];
        s_lv[q - w0] = sa.surv_val[off];
      }
      pos += n;
    }
    __syncthreads();
    const int wn = w1 - w0;
    for (int p0 = 0; p0 < wn; p0 += RG::NG * U) {
      int idx[U];
      uint4 vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + u * RG::NG + grp;
        idx[u] = (p < wn) ? s_li[p] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) vr[u] = (idx[u] >= 0) ? ld16(vbase + (size_t)idx[u] * D) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (idx[u] >= 0) {
          const int p = p0 + u * RG::NG + grp;
          const float w = expf(s_lv[p] - m);
          float x[RG::EPL];
          Unpack<T>::run(vr[u], x);
#pragma unroll
          for (int e = 0; e < RG::EPL; ++e) acc[e] += w * x[e];
          z += w;
          if (gl == 0 && a.sel_idx && w0 + p < a.sel_cap) a.sel_idx[row * a.sel_cap + w0 + p] = idx[u];
        }
      }
    }
    __syncthreads();
  }
  if (lo < hi) {
    reduce_rows<T, D, NT>(acc, z, s_red, s_z);
    float* ar = a.acc + row * AS;
    for (int d = tid; d < D; d += NT) atomicAdd(&ar[d], s_red[0][d]);
    if (tid == 0) atomicAdd(&ar[D], s_z[0]);
  }
  // every thread's atomics have completed before the block is counted
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&a.row_done[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(P - 1);
  __syncthreads();
  if (!s_last) return;
  // last block of the row: coherent (sc1) loads of the accumulated sums
  __shared__ float s_fin[AS];
  if (tid < AS / 4) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(a.acc + row * AS, (short)0, AS * 4, kBufDword3);
    const floatx4 q = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 16, 0, kCoherent);
#pragma unroll
    for (int e = 0; e < 4; ++e) s_fin[tid * 4 + e] = q[e];
  }
  __syncthreads();
  for (int d = tid; d < D; d += NT) store_out<D>(a, row, d, s_fin[d] / s_fin[D]);
  if (tid == 0) {
    if (a.sel_count) a.sel_count[row] = total;
    if (a.flags) a.flags[row] = a.refreshed ? 1 : 0;
  }
}

// ----------------------------------------------------------------------------
// Dense grouped-query attention (eq. (2)-(4)), split over the cached keys.

struct DenseArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* l_kv;
  float* part;     // [B*h_q, nchd, D+4] per-chunk (m, Z, -, -, o[D])
  void* out;
  int h_q, h_kv, g, l_max, nchd, out_bf16;
  int max_l_kv;
  float scale;
};

// grid = (nchd, h_kv, B), block = 256. Each block: logits of CHD keys for the g query
// heads of one key/value head (MFMA), the chunk's softmax numerator relative to the
// chunk maximum, and its product with the chunk's value rows (VALU).
template <typename T, int D, int GH>
__global__ __launch_bounds__(kBlock) void k_dense_partial(const DenseArgs a) {
  constexpr int TPW = StreamCfg<T, D>::kTPW;
  constexpr int CHD = StreamCfg<T, D>::kChunk;
  constexpr int EPL = Unpack<T>::kN;
  constexpr int G = D / EPL;                         // lanes per value row
  constexpr int VL = (16 * D) / (EPL * kWave);       // 16-byte value loads per lane per tile
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int base = c * CHD;
  if (base >= L) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int j0 = g * a.g;
  const int row0 = b * a.h_q + j0;

  __shared__ float s_p[kWaves][TPW][16][GH];
  __shared__ float s_m[kWaves][GH], s_z[kWaves][GH];
  __shared__ float s_o[kWaves][GH][D];

  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.h_kv + g) * a.l_max * D;
  const T* vh = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.h_kv + g) * a.l_max * D;
  const int wbase = base + wv * 16 * TPW;

  // value tiles: load r of tile t covers flat element (r*64 + lane) of the 16 x G grid
  uint4 vb[TPW][VL];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int e = r * kWave + lane;
      const int key = min(wbase + 16 * t + e / G, L - 1);
      vb[t][r] = ld16(vh + (size_t)key * D + (e % G) * EPL);
    }

  QK<T, D> qk;
  qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, a.g, lane);
  floatx4 sc[TPW];
  score_tiles<T, D, TPW>(sc, qk, kh, wbase, L, lane, a.scale);

  float mh = -INFINITY;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = wbase + 16 * t + 4 * kq + r;
      if (key >= L) sc[t][r] = -INFINITY;
      mh = fmaxf(mh, sc[t][r]);
    }
  mh = fmaxf(mh, __shfl_xor(mh, 16));
  mh = fmaxf(mh, __shfl_xor(mh, 32));
  float zh = 0.f;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = (mh == -INFINITY) ? 0.f : expf(sc[t][r] - mh);
      zh += p;
      if (hh < GH) s_p[wv][t][4 * kq + r][hh] = p;
    }
  zh += __shfl_xor(zh, 16);
  zh += __shfl_xor(zh, 32);
  if (lane < GH) {
    s_m[wv][lane] = mh;
    s_z[wv][lane] = zh;
  }
  __syncthreads();

  float o[GH][EPL];
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int e = r * kWave + lane;
      const int k16 = e / G;
      float x[EPL];
      Unpack<T>::run(vb[t][r], x);
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const float p = s_p[wv][t][k16][h];
#pragma unroll
        for (int q = 0; q < EPL; ++q) o[h][q] += p * x[q];
      }
    }
  // lanes with the same column group (lane % G) hold partial sums over different keys
#pragma unroll
  for (int off = G; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int q = 0; q < EPL; ++q) o[h][q] += __shfl_xor(o[h][q], off);
  if (lane < G) {
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int q = 0; q < EPL; ++q) s_o[wv][h][lane * EPL + q] = o[h][q];
  }
  __syncthreads();

  // merge the 4 waves (each relative to its own maximum) and write the chunk partial
  for (int idx = tid; idx < a.g * (D + 1); idx += kBlock) {
    const int h = idx / (D + 1), d = idx - h * (D + 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][h];
      const float sw = (mw == -INFINITY) ? 0.f : expf(mw - M);
      acc += sw * (d < D ? s_o[w][h][d] : s_z[w][h]);
    }
    float* pp = a.part + ((long long)(row0 + h) * a.nchd + c) * (D + 4);
    if (d < D) pp[4 + d] = acc;
    else {
      pp[0] = M;
      pp[1] = acc;
    }
  }
}

// Log-sum-exp merge of the chunk partials of each row (b, j). Thread t takes chunks
// t, t+256, ... and 16 columns (four 16-byte loads per chunk).
// grid = (D / 16, h_q, B), block = 256.
template <int D>
__global__ __launch_bounds__(kBlock) void k_dense_combine(const DenseArgs a, int chd) {
  const int cg = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const long long row = (long long)b * a.h_q + j;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  __shared__ float s_ftmp[kWaves];
  __shared__ float s_acc[kWaves][17];
  if (L <= 0) {
    if (tid < 16) {
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[row * D + cg * 16 + tid] = 0;
      else reinterpret_cast<float*>(a.out)[row * D + cg * 16 + tid] = 0.f;
    }
    return;
  }
  const int nch_b = (L + chd - 1) / chd;
  const float* rp = a.part + row * a.nchd * (D + 4);
  float m = -INFINITY;
  for (int c = tid; c < nch_b; c += kBlock) m = fmaxf(m, rp[(long long)c * (D + 4)]);
  const float M = block_max(m, s_ftmp);
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  float z = 0.f;
  for (int c = tid; c < nch_b; c += kBlock) {
    const float* pc = rp + (long long)c * (D + 4);
    const float w = expf(pc[0] - M);
    z += w * pc[1];
    const float4* p4 = reinterpret_cast<const float4*>(pc + 4 + cg * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = p4[q];
      o[4 * q] += w * x.x;
      o[4 * q + 1] += w * x.y;
      o[4 * q + 2] += w * x.z;
      o[4 * q + 3] += w * x.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = wave_sum(o[e]);
  z = wave_sum(z);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s_acc[wv][e] = o[e];
    s_acc[wv][16] = z;
  }
  __syncthreads();
  if (tid < 16) {
    float oo = 0.f, zz = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      oo += s_acc[w][tid];
      zz += s_acc[w][16];
    }
    const float x = oo / zz;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[row * D + cg * 16 + tid] = f32_to_bf16(x);
    else reinterpret_cast<float*>(a.out)[row * D + cg * 16 + tid] = x;
  }
}

// Zero fill (workspace initialisation) with 16-byte stores plus a byte tail.
__global__ void k_zero_fill(uint8_t* p, size_t n) {
  const size_t n16 = n / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < (n & 15)) p[n16 * 16 + threadIdx.x] = 0;
}

}  // namespace saga
