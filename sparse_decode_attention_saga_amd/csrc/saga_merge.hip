// GQA-to-SAGA key-head merge: the closed-form initialisation that turns a teacher
// with h_k key heads into a SAGA student with h_k / 2 key heads (paper "More Value
// per Key: Asymmetric Sparse Attention for Faster LLM Decoding", summary page
// picx.dev DRD92V, section "GQA-to-SAGA Conversion > Stage 1: Closed-Form
// Initialization": eq. (13) loss, Lemma 4.1 eq. (15) merged projection, Theorem 4.2
// minimum-weight perfect matching of eq. (14)). Host side of the merge entry points
// of include/saga.h and their kernels.
//
// Notation (the pages'): X [T, D] calibration hidden states; W_Q^j, W_K^a [D, d];
// Q^j = X W_Q^j; S_a = sum over the query heads j of key head a of Q^j^T Q^j.
//
// The loss of eq. (13) is evaluated from Gram matrices instead of T x T logit
// matrices. With C = X^T X and Delta = M - W_a, the sum over j of
// ||Q^j Delta^T X^T||_F^2 equals trace(Delta^T C Delta S_a). Writing the merged
// projection of eq. (15) as M = W_a A + W_b B with A = S_a P, B = S_b P and
// P = (S_a + S_b)^+, Delta_a = [W_a W_b] Z_a with Z_a = [A - I; B] (and Z_b =
// [A; B - I] for head b), so Delta_a^T C Delta_a = Z_a^T Hab Z_a where Hab is the
// 2d x 2d block of H = K^T K (K = X [W_K^1 .. W_K^h_k], the teacher's keys) for the
// heads a and b. Every quantity is then a d x d or 2d x 2d matrix:
//   k_proj    Y = X [W_Q W_K] (bf16 MFMA, fp32 out): all queries and keys;
//   k_gram    partial Grams of the query groups (S_a) and of the keys (H) over
//             token chunks (fp32 MFMA), k_gram_sum adds the chunks;
//   k_pair    per pair (a, b): P = (S_a + S_b)^+ (fp64: a Gauss-Jordan inverse when
//             it is certified to equal the pseudo-inverse with the cut, else a
//             cyclic Jacobi eigendecomposition), A, B, and
//             L_ab = <Z_a^T Hab Z_a, S_a> + <Z_b^T Hab Z_b, S_b>;
//   (host)    the minimum-weight perfect matching of the h_k heads;
//   k_merge   the merged projections of the chosen pairs.
#include "saga.h"

#include <cmath>
#include <cstddef>
#include <vector>

#include "saga_device.hpp"

using namespace saga;

namespace {

constexpr int kMaxMergeHeads = 16;       // teacher key heads (even)
constexpr double kPinvRcond = 1e-5;      // eigenvalues below rcond * largest count as zero
constexpr int kJacobiSweeps = 16;        // upper bound; sweeps stop once converged
constexpr int kGramSteps = 16;      // 4-token MFMA steps per load round of k_gram
constexpr int kGramRound = 4 * kGramSteps;  // tokens per load round (all loads of a round in flight)
constexpr int kGramChunk = 64;      // calibration tokens per partial Gram, at least
constexpr int kGramMaxChunks = 64;  // partial Grams per output tile, at most
static_assert(kGramChunk % kGramRound == 0, "whole load rounds per chunk");
constexpr int kGramTile = 64;            // output tile of one wave in k_gram
constexpr int kPairScratch = 16;         // d x d fp64 matrices of scratch per pair

// --- workspace layout ------------------------------------------------------------

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct MergeLayout {
  int n_cols;          // columns of Y: (h_q + h_k) d
  int chunk_tokens;    // calibration tokens per partial Gram (whole load rounds)
  int chunks;          // token chunks of the partial Grams
  int s_tiles, h_tiles;  // 64 x 64 output tiles of one S_a and of H
  int items;           // partial Gram work items (one wave each)
  int pairs;           // h_k (h_k - 1) / 2
  size_t y, part, s, h, pair_f64, coef, total;
};

MergeLayout merge_layout(const saga_merge_shape* s) {
  MergeLayout m{};
  const int d = s->d, hk = s->h_k;
  m.n_cols = (s->h_q + hk) * d;
  // chunks of kGramChunk tokens (many short serial loops in parallel), longer ones
  // past kGramMaxChunks chunks so that the partials stay a bounded multiple of the Grams
  const int per = (s->tokens + kGramMaxChunks - 1) / kGramMaxChunks;
  m.chunk_tokens = per > kGramChunk ? (per + kGramRound - 1) / kGramRound * kGramRound : kGramChunk;
  m.chunks = (s->tokens + m.chunk_tokens - 1) / m.chunk_tokens;
  m.s_tiles = (d / kGramTile) * (d / kGramTile);
  m.h_tiles = (hk * d / kGramTile) * (hk * d / kGramTile);
  m.items = (hk * m.s_tiles + m.h_tiles) * m.chunks;
  m.pairs = hk * (hk - 1) / 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  m.y = take((size_t)s->tokens * m.n_cols * 4);
  m.part = take((size_t)m.items * kGramTile * kGramTile * 4);
  m.s = take((size_t)hk * d * d * 4);
  m.h = take((size_t)hk * d * hk * d * 4);
  // per pair, fp64: V^T, P, A, B, S_a, S_b (d x d), Z, Z^T, Hab Z (2 d^2 each), Hab (4 d^2)
  m.pair_f64 = take((size_t)m.pairs * (kPairScratch * (size_t)d * d) * 8);
  m.coef = take((size_t)hk * hk * 2 * d * d * 4);  // (A, B) of pair (a, b) at [a][b], fp32
  m.total = off;
  return m;
}

saga_status check_merge_shape(const saga_merge_shape* s) {
  if (!s) return SAGA_ERR_NULL;
  if (s->tokens < 1 || s->d_model < 1 || s->h_q < 1 || s->h_k < 2 || s->d < 1) return SAGA_ERR_SHAPE;
  if (s->h_k % 2 || s->h_q % s->h_k || s->d_model % 32) return SAGA_ERR_SHAPE;
  if (s->d != 64 && s->d != 128) return SAGA_ERR_UNSUPPORTED;
  if (s->h_k > kMaxMergeHeads || s->d_model > (1 << 16) || s->h_q > 256 || s->tokens > (1 << 22))
    return SAGA_ERR_UNSUPPORTED;
  return SAGA_OK;
}

saga_status launched() { return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP; }

// --- k_proj: Y[t, n] = sum_x X[t, x] W[n, x] ----------------------------------------
// W rows n < nq come from w_q, the others from w_k (both [rows, D], D-contiguous: the
// transposes of the pages' W_Q and W_K). A wave computes a 64 x 64 tile of Y as
// 4 x 4 MFMA tiles (bf16 16x16x32): X rows as the A operand, W rows as the B
// operand, each lane loading its 16-byte K slices straight from memory as the score
// tiles do (each load feeds four MFMAs). Rows past T are clamped on load and never
// stored. grid = (ceil(n_cols / 128), ceil(T / 128)), block = 256 (waves 2 x 2).
struct ProjArgs {
  const bf16_t* x;
  const bf16_t* wq;
  const bf16_t* wk;
  float* y;
  int T, D, nq, n_cols;
};

constexpr int kProjTile = 64;  // rows and columns of Y per wave

__global__ __launch_bounds__(kBlock) void k_proj(const ProjArgs a) {
  constexpr int NT = kProjTile / 16;  // MFMA tiles per side
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int m0 = blockIdx.y * 2 * kProjTile + (wv >> 1) * kProjTile;
  const int n0 = blockIdx.x * 2 * kProjTile + (wv & 1) * kProjTile;
  const bf16_t* xr[NT];
  const bf16_t* wr[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    xr[i] = a.x + (size_t)min(m0 + 16 * i + r16, a.T - 1) * a.D + 8 * kq;
    const int n = min(n0 + 16 * i + r16, a.n_cols - 1);
    wr[i] = (n < a.nq ? a.wq + (size_t)n * a.D : a.wk + (size_t)(n - a.nq) * a.D) + 8 * kq;
  }
  floatx4 acc[NT][NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[i][k] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.D; k0 += 32) {  // D is a multiple of 32
    V16 xa[NT], wb[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      xa[i].u = ld16(xr[i] + k0);
      wb[i].u = ld16(wr[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int k = 0; k < NT; ++k)
        acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i].h, wb[k].h, acc[i][k], 0, 0, 0);
  }
  // accumulator layout: lane l holds Y[m + 4 (l >> 4) + r][n + (l & 15)]
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int n = n0 + 16 * k + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * kq + r;
        if (m < a.T && n < a.n_cols) a.y[(size_t)m * a.n_cols + n] = acc[i][k][r];
      }
    }
}

// --- k_gram: partial Grams over one chunk of tokens ---------------------------------
// Work item w (one wave): an output o (S_a for o < h_k, else H), a 64 x 64 tile of it
// and a chunk of a.chunk_tokens tokens. S_a tile (i, k) sums Y[t, jd + 64i + m] *
// Y[t, jd + 64k + n] over the chunk's tokens t and the query heads j of key head a;
// H tile (i, k) sums Y[t, c0 + 64i + m] Y[t, c0 + 64k + n] with c0 = h_q d (the key
// columns). fp32 MFMA 16x16x4 (lane l supplies row/column l & 15 at token l >> 4 of
// each 4-token step), 4 x 4 MFMA tiles per wave. grid = ceil(items / 4), block = 256.
struct GramArgs {
  const float* y;
  float* part;     // [items, 64, 64]
  int T, n_cols, h_q, h_k, d, chunks, s_tiles, h_tiles, items, chunk_tokens;
};

__global__ __launch_bounds__(kBlock) void k_gram(const GramArgs a) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int item = blockIdx.x * kWaves + wv;
  if (item >= a.items) return;  // uniform over the wave
  const int chunk = item % a.chunks, tile_id = item / a.chunks;
  const int r16 = lane & 15, kq = lane >> 4;
  int tiles_per_row, tile, col_base, heads, head_stride;
  if (tile_id < a.h_k * a.s_tiles) {
    const int o = tile_id / a.s_tiles;
    tile = tile_id - o * a.s_tiles;
    tiles_per_row = a.d / kGramTile;
    heads = a.h_q / a.h_k;
    col_base = o * heads * a.d;
    head_stride = a.d;
  } else {
    tile = tile_id - a.h_k * a.s_tiles;
    tiles_per_row = a.h_k * a.d / kGramTile;
    heads = 1;
    col_base = a.h_q * a.d;
    head_stride = 0;
  }
  const int ti = tile / tiles_per_row, tk = tile - ti * tiles_per_row;
  const int t_lo = chunk * a.chunk_tokens, t_hi = min(t_lo + a.chunk_tokens, a.T);
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < heads; ++h) {
    const float* ya = a.y + col_base + h * head_stride + ti * kGramTile + r16;
    const float* yb = a.y + col_base + h * head_stride + tk * kGramTile + r16;
    for (int t0 = t_lo; t0 < t_hi; t0 += kGramRound) {
      float va[kGramSteps][4], vb[kGramSteps][4];  // [token step][subtile]
#pragma unroll
      for (int u = 0; u < kGramSteps; ++u) {
        const int t = t0 + 4 * u + kq;
        const bool ok = t < t_hi;
        const size_t row = (size_t)min(t, a.T - 1) * a.n_cols;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[u][i] = ok ? ya[row + 16 * i] : 0.f;
          vb[u][i] = ok ? yb[row + 16 * i] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kGramSteps; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[u][i], vb[u][k], acc[i][k], 0, 0, 0);
    }
  }
  float* out = a.part + (size_t)item * kGramTile * kGramTile;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(16 * i + 4 * kq + r) * kGramTile + 16 * k + r16] = acc[i][k][r];
}

// Sum of the chunk partials into S [h_k, d, d] and H [h_k d, h_k d]: one thread per
// output element. grid = ceil((h_k d^2 + (h_k d)^2) / 256), block = 256.
__global__ __launch_bounds__(kBlock) void k_gram_sum(const GramArgs a, float* S, float* H) {
  const int d = a.d, hd = a.h_k * a.d;
  const long long n_s = (long long)a.h_k * d * d, n_h = (long long)hd * hd;
  const long long e = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (e >= n_s + n_h) return;
  int tile_id, m, n;
  float* dst;
  if (e < n_s) {
    const int o = (int)(e / ((long long)d * d));
    const int rem = (int)(e - (long long)o * d * d);
    const int row = rem / d, col = rem - (rem / d) * d;
    tile_id = o * a.s_tiles + (row / kGramTile) * (d / kGramTile) + col / kGramTile;
    m = row % kGramTile;
    n = col % kGramTile;
    dst = S + e;
  } else {
    const long long f = e - n_s;
    const int row = (int)(f / hd), col = (int)(f - (long long)row * hd);
    tile_id = a.h_k * a.s_tiles + (row / kGramTile) * (hd / kGramTile) + col / kGramTile;
    m = row % kGramTile;
    n = col % kGramTile;
    dst = H + f;
  }
  float sum = 0.f;
  const float* p = a.part + ((size_t)tile_id * a.chunks) * kGramTile * kGramTile + m * kGramTile + n;
  for (int c = 0; c < a.chunks; ++c) sum += p[(size_t)c * kGramTile * kGramTile];
  *dst = sum;
}

// --- k_pair: Lemma 4.1 and eq. (13) for one pair of teacher heads --------------------
struct PairArgs {
  const float* S;    // [h_k, d, d]
  const float* H;    // [h_k d, h_k d]
  double* scratch;   // [pairs, 9 d^2]
  float* coef;       // [h_k, h_k, 2, d, d]: (A, B) of pair (a, b) at [a][b]
  float* loss;       // [h_k, h_k]
  int h_k, d;
};

// Block-wide sum of one double per thread (all threads receive it).
__device__ double block_sum_f64(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += red[w];
  return t;
}

// C[M x N] = X[M x K] Y[K x N] in fp64, all row-major in global memory, by every
// thread of the block: 64 x 64 output tiles, each thread a 4 x 4 register tile, K
// staged through LDS in slices of 16 (`lds`: 64 * 17 + 16 * 64 doubles), the next
// slice's loads in flight while the current one is multiplied. M and N are multiples
// of 64, K of 16.
constexpr int kGemmLds = 64 * 17 + 16 * 64;

__device__ void block_gemm_f64(double* C, int ldc, const double* X, int ldx, const double* Y, int ldy, int M, int N,
                               int K, double* lds) {
  double* xs = lds;            // [64][17]
  double* ys = lds + 64 * 17;  // [16][64]
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  for (int mt = 0; mt < M; mt += 64)
    for (int nt = 0; nt < N; nt += 64) {
      double acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
      // the next K slice is loaded into registers while the current one is used
      double xv[4], yv[4];
      auto load = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = u * kBlock + tid;
          xv[u] = X[(size_t)(mt + e / 16) * ldx + k0 + e % 16];
          yv[u] = Y[(size_t)(k0 + e / 64) * ldy + nt + e % 64];
        }
      };
      load(0);
      for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = u * kBlock + tid;
          xs[(e / 16) * 17 + e % 16] = xv[u];
          ys[e] = yv[u];
        }
        __syncthreads();
        if (k0 + 16 < K) load(k0 + 16);
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
          double xr[4], yr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[i] = xs[(tr * 4 + i) * 17 + kk];
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[j] = ys[kk * 64 + tc * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += xr[i] * yr[j];
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) C[(size_t)(mt + tr * 4 + i) * ldc + nt + tc * 4 + j] = acc[i][j];
    }
  __syncthreads();
}

// Pseudo-inverse of S_a + S_b by its eigendecomposition, with the cut: the sum
// (symmetrised, fp64) is diagonalised in LDS by cyclic Jacobi rotations. Each round
// rotates d/2 disjoint index pairs (a round-robin schedule visits every pair once
// per sweep of d - 1 rounds) with the angle that zeroes their off-diagonal entry;
// eigenvectors accumulate as the rows of V^T. Then P = V diag(lambda+) V^T. Called by
// every thread of the block; s_* are the kernel's LDS arrays.
template <int D>
__device__ void jacobi_pinv(double* s_m, double* vt, int* s_p, int* s_q, double* s_c, double* s_s, double* s_red,
                            double* s_linv, const double* Ssa, const double* Ssb, double* P) {
  constexpr int HALF = D / 2;
  const int tid = threadIdx.x;
  __syncthreads();
  for (int e = tid; e < D * D; e += kBlock) {
    const int i = e / D, k = e - (e / D) * D;
    s_m[e] = Ssa[e] + Ssb[e];
    vt[e] = i == k ? 1.0 : 0.0;
  }
  __syncthreads();

  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    for (int round = 0; round < D - 1; ++round) {
      if (tid < HALF) {
        // round-robin: position 0 stays, positions 1..D-1 rotate by `round`
        auto idx = [&](int pos) { return pos == 0 ? 0 : ((pos - 1 + round) % (D - 1)) + 1; };
        int p = idx(tid), q = idx(D - 1 - tid);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = s_m[p * D + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (s_m[q * D + q] - s_m[p * D + p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        s_p[tid] = p;
        s_q[tid] = q;
        s_c[tid] = c;
        s_s[tid] = s;
      }
      __syncthreads();
      // M <- J^T M J with J[p][p] = J[q][q] = c, J[p][q] = s = -J[q][p] for every pair
      // of the round: the 2 x 2 block of rows (p1, q1) and columns (p2, q2) depends on
      // itself only, so each thread rotates its own blocks in place
      for (int blk = tid; blk < HALF * HALF; blk += kBlock) {
        const int r1 = blk / HALF, r2 = blk - (blk / HALF) * HALF;
        const int p1 = s_p[r1], q1 = s_q[r1], p2 = s_p[r2], q2 = s_q[r2];
        const double c1 = s_c[r1], s1 = s_s[r1], c2 = s_c[r2], s2 = s_s[r2];
        const double m_pp = s_m[p1 * D + p2], m_pq = s_m[p1 * D + q2];
        const double m_qp = s_m[q1 * D + p2], m_qq = s_m[q1 * D + q2];
        // rows: p' = c p - s q, q' = s p + c q
        const double r_pp = c1 * m_pp - s1 * m_qp, r_pq = c1 * m_pq - s1 * m_qq;
        const double r_qp = s1 * m_pp + c1 * m_qp, r_qq = s1 * m_pq + c1 * m_qq;
        // columns, the same rotation
        s_m[p1 * D + p2] = c2 * r_pp - s2 * r_pq;
        s_m[p1 * D + q2] = s2 * r_pp + c2 * r_pq;
        s_m[q1 * D + p2] = c2 * r_qp - s2 * r_qq;
        s_m[q1 * D + q2] = s2 * r_qp + c2 * r_qq;
      }
      // eigenvector rows: V^T[p] = c V^T[p] - s V^T[q], V^T[q] = s V^T[p] + c V^T[q]
      for (int e = tid; e < HALF * D; e += kBlock) {
        const int r = e / D, col = e - (e / D) * D;
        const int p = s_p[r], q = s_q[r];
        const double c = s_c[r], s = s_s[r];
        const double vp = vt[p * D + col], vq = vt[q * D + col];
        vt[p * D + col] = c * vp - s * vq;
        vt[q * D + col] = s * vp + c * vq;
      }
      __syncthreads();
    }
    // converged when the off-diagonal mass is below 1e-26 of the diagonal's (entries
    // below 1e-13 of the matrix: far under the fp32 rounding of its inputs)
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < D * D; e += kBlock) {
      const int i = e / D, k = e - (e / D) * D;
      const double x = s_m[e] * s_m[e];
      if (i == k) dia += x;
      else off += x;
    }
    off = block_sum_f64(off, s_red);
    dia = block_sum_f64(dia, s_red);
    if (off <= 1e-26 * dia) break;  // the same value in every thread
  }
  __syncthreads();

  // P = V diag(lambda+) V^T, lambda+ = 1 / lambda above rcond * max |lambda|, else 0
  if (tid < D) {
    double lmax = 0.0;
    for (int i = 0; i < D; ++i) lmax = fmax(lmax, fabs(s_m[i * D + i]));
    const double l = s_m[tid * D + tid];
    s_linv[tid] = l > kPinvRcond * lmax ? 1.0 / l : 0.0;
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += kBlock) {
    const int m = e / D, n = e - (e / D) * D;
    double sum = 0.0;
#pragma unroll 8
    for (int i = 0; i < D; ++i) sum += vt[i * D + m] * vt[i * D + n] * s_linv[i];
    P[e] = sum;
  }
}

// One pair (a, b), a < b, per block of 256 threads: P = (S_a + S_b)^+ (the inverse
// when it is certified to equal the pseudo-inverse with the cut, else jacobi_pinv),
// A = S_a P, B = S_b P, and L_ab = <Z_a^T Hab Z_a, S_a> + <Z_b^T Hab Z_b, S_b>.
template <int D>
__global__ __launch_bounds__(kBlock) void k_pair(const PairArgs a) {
  constexpr int HALF = D / 2;
  constexpr bool kVtLds = D <= 64;         // V^T in LDS too (d = 128: in the scratch)
  __shared__ double s_m[D * D];
  __shared__ double s_vt[kVtLds ? D * D : 1];
  __shared__ int s_p[HALF], s_q[HALF];     // the rotation round's index pairs (p < q)
  __shared__ double s_c[HALF], s_s[HALF];  // and their rotations
  __shared__ double s_red[kWaves];
  __shared__ double s_linv[D];             // 1 / eigenvalue, 0 below the cut
  __shared__ double s_gemm[kGemmLds];

  // pair index -> (a, b) with a < b
  int pa = 0, rem = blockIdx.x;
  while (rem >= a.h_k - 1 - pa) {
    rem -= a.h_k - 1 - pa;
    ++pa;
  }
  const int pb = pa + 1 + rem;
  const int tid = threadIdx.x;
  const float* Sa = a.S + (size_t)pa * D * D;
  const float* Sb = a.S + (size_t)pb * D * D;
  double* const vt_g = a.scratch + (size_t)blockIdx.x * kPairScratch * D * D;
  double* const vt = kVtLds ? s_vt : vt_g;                    // V^T [D][D]
  double* const P = vt_g + D * D;
  double* const Am = P + D * D;
  double* const Bm = Am + D * D;
  double* const Ssa = Bm + D * D;    // S_a, S_b symmetrised
  double* const Ssb = Ssa + D * D;
  double* const Z = Ssb + D * D;       // [2D][D]
  double* const Zt = Z + 2 * D * D;    // Z^T [D][2D]
  double* const HZ = Zt + 2 * D * D;   // Hab Z [2D][D]
  double* const Hab = HZ + 2 * D * D;  // [2D][2D]

  for (int e = tid; e < D * D; e += kBlock) {
    const int i = e / D, k = e - (e / D) * D;
    const double sa = 0.5 * ((double)Sa[i * D + k] + (double)Sa[k * D + i]);
    const double sb = 0.5 * ((double)Sb[i * D + k] + (double)Sb[k * D + i]);
    Ssa[e] = sa;
    Ssb[e] = sb;
    s_m[e] = sa + sb;
  }
  __syncthreads();

  // Fast path: S_a + S_b inverted in place by Gauss-Jordan elimination (no pivoting
  // is needed for a positive definite matrix: every pivot is a positive Schur
  // complement diagonal). The inverse is the pseudo-inverse with the cut whenever no
  // eigenvalue lies below rcond times the largest, which ||S||_F ||S^-1||_F <
  // 1 / rcond guarantees (the Frobenius norms bound lambda_max and 1 / lambda_min
  // from above). Otherwise (a singular or badly conditioned sum, or a non-positive
  // pivot) the eigendecomposition below applies the cut.
  double fro_s = 0.0;
  for (int e = tid; e < D * D; e += kBlock) fro_s += s_m[e] * s_m[e];
  fro_s = block_sum_f64(fro_s, s_red);
  bool inverted = true;
  for (int k = 0; k < D; ++k) {
    const double piv = s_m[k * D + k];  // the same value in every thread
    if (!(piv > 0.0)) {
      inverted = false;
      break;
    }
    const double rp = 1.0 / piv;
    constexpr int PER = D * D / kBlock;
    double nv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * kBlock + tid;
      const int i = e / D, j = e - (e / D) * D;
      const double aij = s_m[e], aik = s_m[i * D + k], akj = s_m[k * D + j];
      nv[u] = i == k ? (j == k ? rp : akj * rp) : (j == k ? -aik * rp : aij - aik * akj * rp);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) s_m[u * kBlock + tid] = nv[u];
    __syncthreads();
  }
  double fro_p = 0.0;
  if (inverted) {
    for (int e = tid; e < D * D; e += kBlock) fro_p += s_m[e] * s_m[e];
    fro_p = block_sum_f64(fro_p, s_red);
  }
  const bool certified = inverted && sqrt(fro_s) * sqrt(fro_p) < 1.0 / kPinvRcond;
  if (certified) {
    for (int e = tid; e < D * D; e += kBlock) {
      const int i = e / D, k = e - (e / D) * D;
      P[e] = 0.5 * (s_m[e] + s_m[k * D + i]);
    }
  } else {
    jacobi_pinv<D>(s_m, vt, s_p, s_q, s_c, s_s, s_red, s_linv, Ssa, Ssb, P);
  }
  __syncthreads();
  // A = S_a P, B = S_b P
  block_gemm_f64(Am, D, Ssa, D, P, D, D, D, D, s_gemm);
  block_gemm_f64(Bm, D, Ssb, D, P, D, D, D, D, s_gemm);
  float* ca = a.coef + ((size_t)(pa * a.h_k + pb) * 2) * D * D;
  for (int e = tid; e < D * D; e += kBlock) {
    ca[e] = (float)Am[e];
    ca[D * D + e] = (float)Bm[e];
  }
  // Hab: the rows and columns of H for heads a and b, in fp64
  const int hd = a.h_k * D;
  for (int e = tid; e < 4 * D * D; e += kBlock) {
    const int k = e / (2 * D), t = e - (e / (2 * D)) * (2 * D);
    Hab[e] = (double)a.H[(size_t)((k < D ? pa : pb) * D + k % D) * hd + (t < D ? pa : pb) * D + t % D];
  }

  // L = sum over the two heads r of <Z_r^T Hab Z_r, S_r>, Z_a = [A - I; B],
  // Z_b = [A; B - I]
  double total = 0.0;
  for (int side = 0; side < 2; ++side) {
    for (int e = tid; e < 2 * D * D; e += kBlock) {
      const int k = e / D, n = e - (e / D) * D;
      const double id = (side == 0 ? k == n : k - D == n) ? 1.0 : 0.0;
      const double z = (k < D ? Am[k * D + n] : Bm[(k - D) * D + n]) - id;
      Z[e] = z;
      Zt[(size_t)n * 2 * D + k] = z;
    }
    __syncthreads();
    block_gemm_f64(HZ, D, Hab, 2 * D, Z, D, 2 * D, D, 2 * D, s_gemm);
    double* const G = P;  // P is no longer needed once A and B are formed
    block_gemm_f64(G, D, Zt, 2 * D, HZ, D, D, D, 2 * D, s_gemm);
    const double* Sr = side == 0 ? Ssa : Ssb;
    double part = 0.0;
    for (int e = tid; e < D * D; e += kBlock) part += G[e] * Sr[e];  // S_r is symmetric
    total += block_sum_f64(part, s_red);
    __syncthreads();
  }
  if (tid == 0) {
    a.loss[pa * a.h_k + pb] = (float)total;
    a.loss[pb * a.h_k + pa] = (float)total;
  }
}

// Diagonal of the loss matrix (a head is not merged with itself): zero.
__global__ void k_loss_diag(float* loss, int h_k) {
  if ((int)threadIdx.x < h_k) loss[threadIdx.x * h_k + threadIdx.x] = 0.f;
}

// --- k_merge: the merged projections of the chosen pairs ------------------------------
// out[i d + c, x] = sum_c' wk[a d + c', x] A[c', c] + wk[b d + c', x] B[c', c] for the
// i-th pair (a, b): row c of merged head i is column c of M = W_a A + W_b B.
// grid = (ceil(D / 256), h_k / 2 * d), block = 256.
struct MergeArgs {
  const bf16_t* wk;  // [h_k d, D]
  const float* coef;
  float* out;        // [h_k / 2 * d, D]
  int D, d, h_k;
  int pa[kMaxMergeHeads / 2], pb[kMaxMergeHeads / 2];
};

__global__ __launch_bounds__(kBlock) void k_merge(const MergeArgs a) {
  const int x = blockIdx.x * kBlock + threadIdx.x;
  const int row = blockIdx.y, i = row / a.d, c = row - (row / a.d) * a.d;
  if (x >= a.D) return;
  const int pa = a.pa[i], pb = a.pb[i];
  const float* A = a.coef + ((size_t)(pa * a.h_k + pb) * 2) * a.d * a.d;
  const float* B = A + (size_t)a.d * a.d;
  float sum = 0.f;
  for (int k = 0; k < a.d; ++k) {
    sum += bf16_to_f32(a.wk[(size_t)(pa * a.d + k) * a.D + x]) * A[k * a.d + c];
    sum += bf16_to_f32(a.wk[(size_t)(pb * a.d + k) * a.D + x]) * B[k * a.d + c];
  }
  a.out[(size_t)row * a.D + x] = sum;
}

}  // namespace

extern "C" {

size_t saga_merge_workspace_bytes(const saga_merge_shape* s) {
  if (check_merge_shape(s) != SAGA_OK) return 0;
  return merge_layout(s).total;
}

saga_status saga_merge_losses(const saga_merge_shape* s, const void* x, const void* w_q, const void* w_k,
                              float* loss, void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !x || !w_q || !w_k || !loss || !workspace) return SAGA_ERR_NULL;
  const saga_status st = check_merge_shape(s);
  if (st != SAGA_OK) return st;
  const MergeLayout m = merge_layout(s);
  if (workspace_bytes < m.total) return SAGA_ERR_WORKSPACE;
  const hipStream_t hs = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  (void)hipGetLastError();

  ProjArgs pj{};
  pj.x = reinterpret_cast<const bf16_t*>(x);
  pj.wq = reinterpret_cast<const bf16_t*>(w_q);
  pj.wk = reinterpret_cast<const bf16_t*>(w_k);
  pj.y = reinterpret_cast<float*>(ws + m.y);
  pj.T = s->tokens;
  pj.D = s->d_model;
  pj.nq = s->h_q * s->d;
  pj.n_cols = m.n_cols;
  hipLaunchKernelGGL(k_proj, dim3((m.n_cols + 2 * kProjTile - 1) / (2 * kProjTile), (s->tokens + 2 * kProjTile - 1) / (2 * kProjTile)),
                     dim3(kBlock), 0, hs, pj);

  GramArgs g{};
  g.y = pj.y;
  g.part = reinterpret_cast<float*>(ws + m.part);
  g.T = s->tokens;
  g.n_cols = m.n_cols;
  g.h_q = s->h_q;
  g.h_k = s->h_k;
  g.d = s->d;
  g.chunks = m.chunks;
  g.chunk_tokens = m.chunk_tokens;
  g.s_tiles = m.s_tiles;
  g.h_tiles = m.h_tiles;
  g.items = m.items;
  hipLaunchKernelGGL(k_gram, dim3((m.items + kWaves - 1) / kWaves), dim3(kBlock), 0, hs, g);
  float* S = reinterpret_cast<float*>(ws + m.s);
  float* H = reinterpret_cast<float*>(ws + m.h);
  const long long n_out = (long long)s->h_k * s->d * s->d + (long long)s->h_k * s->d * s->h_k * s->d;
  hipLaunchKernelGGL(k_gram_sum, dim3((unsigned)((n_out + kBlock - 1) / kBlock)), dim3(kBlock), 0, hs, g, S, H);

  PairArgs pa{};
  pa.S = S;
  pa.H = H;
  pa.scratch = reinterpret_cast<double*>(ws + m.pair_f64);
  pa.coef = reinterpret_cast<float*>(ws + m.coef);
  pa.loss = loss;
  pa.h_k = s->h_k;
  pa.d = s->d;
  if (s->d == 64) hipLaunchKernelGGL((k_pair<64>), dim3(m.pairs), dim3(kBlock), 0, hs, pa);
  else hipLaunchKernelGGL((k_pair<128>), dim3(m.pairs), dim3(kBlock), 0, hs, pa);
  hipLaunchKernelGGL(k_loss_diag, dim3(1), dim3(kMaxMergeHeads), 0, hs, loss, s->h_k);
  return launched();
}

saga_status saga_min_weight_pairing(int32_t n, const float* weight, int32_t* partner, double* total) {
  if (!weight || !partner) return SAGA_ERR_NULL;
  if (n < 2 || n % 2 || n > kMaxMergeHeads) return SAGA_ERR_SHAPE;
  for (int a = 0; a < n; ++a)
    for (int b = 0; b < n; ++b)
      if (a != b && !std::isfinite(weight[a * n + b])) return SAGA_ERR_SHAPE;
  // exact minimum over all perfect matchings: best[mask] = least weight matching the
  // heads in `mask`, always pairing the lowest unmatched head first
  const int full = (1 << n) - 1;
  std::vector<double> best(1u << n, INFINITY);
  std::vector<int> choice(1u << n, -1);
  best[0] = 0.0;
  for (int mask = 0; mask < full; ++mask) {
    if (best[mask] == INFINITY) continue;
    int i = 0;
    while (mask & (1 << i)) ++i;
    for (int j = i + 1; j < n; ++j) {
      if (mask & (1 << j)) continue;
      const int next = mask | (1 << i) | (1 << j);
      const double w = best[mask] + (double)weight[i * n + j];
      if (w < best[next]) {
        best[next] = w;
        choice[next] = i * n + j;
      }
    }
  }
  for (int mask = full; mask; ) {
    const int i = choice[mask] / n, j = choice[mask] % n;
    partner[i] = j;
    partner[j] = i;
    mask &= ~((1 << i) | (1 << j));
  }
  if (total) *total = best[full];
  return SAGA_OK;
}

saga_status saga_merge_keys(const saga_merge_shape* s, const void* w_k, const int32_t* partner, float* w_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !w_k || !partner || !w_out || !workspace) return SAGA_ERR_NULL;
  const saga_status st = check_merge_shape(s);
  if (st != SAGA_OK) return st;
  const MergeLayout m = merge_layout(s);
  if (workspace_bytes < m.total) return SAGA_ERR_WORKSPACE;
  MergeArgs a{};
  int i = 0;
  bool seen[kMaxMergeHeads] = {};
  for (int h = 0; h < s->h_k; ++h) {
    const int p = partner[h];
    if (p < 0 || p >= s->h_k || p == h || partner[p] != h) return SAGA_ERR_SHAPE;
    if (seen[h]) continue;
    seen[h] = seen[p] = true;
    a.pa[i] = h;  // h < p: heads are visited in increasing order
    a.pb[i] = p;
    ++i;
  }
  a.wk = reinterpret_cast<const bf16_t*>(w_k);
  a.coef = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) + m.coef);
  a.out = w_out;
  a.D = s->d_model;
  a.d = s->d;
  a.h_k = s->h_k;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_merge, dim3((s->d_model + kBlock - 1) / kBlock, s->h_k / 2 * s->d), dim3(kBlock), 0,
                     (hipStream_t)stream, a);
  return launched();
}

}  // extern "C"
