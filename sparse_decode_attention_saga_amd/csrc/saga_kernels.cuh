// Kernels of the SAGA + Atop-N decode step and of the dense GQA baseline (gfx950).
//
// Stale-threshold step:  k_qk_select<gather> -> k_split_combine
// Refresh step:          k_scores_hist -> k_cand_collect -> k_select_finish
//                        -> k_qk_select<from stored logits, gather> -> k_split_combine
// Separate stages:       k_qk_select -> k_chunk_gather -> k_split_combine
// Dense GQA baseline:    k_dense_partial -> k_dense_combine
//
// No kernel waits on another workgroup and none needs a device-scope fence: every
// exchange between workgroups goes through a kernel boundary (the threshold
// histograms are accumulated with device atomics and read by the next kernel).
//
// Paper: "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
// (summary page picx.dev DRD92V): eq. (2) logits, section "Methodology > Atop-N
// Attention" (threshold = N-th largest logit, elementwise comparison, exact
// threshold refreshed every n steps), eq. (7) sparse softmax-PV, section "SAGA
// Architecture" (h_k key heads, h_v value heads).
#pragma once

#include "saga_device.cuh"

namespace saga {

// Keys per block of the key-streaming kernels: 4 waves x TPW tiles x 16 keys. The
// launch picks W = TPW from 2, 4 and 8 (the kept mask of a lane holds 32 entries);
// W = 0 is the base form used by the dense kernels and the exact row pass: 16 KiB of
// keys per wave, at most 8 tiles.
template <typename T, int D, int W = 0> struct StreamCfg {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kBase = 16384 / (16 * kRowBytes) > 0 ? 16384 / (16 * kRowBytes) : 1;
  static constexpr int kTPW = W > 0 ? W : (kBase > 8 ? 8 : kBase);  // 16-key tiles per wave
  static_assert(kTPW >= 1 && kTPW <= 8, "one to eight tiles per wave");
  static constexpr int kChunk = 16 * kTPW * kWaves;
};

// Summary of one chunk of one row (b, j), written by the select kernels: the number
// of kept entries, the largest kept logit m and, once gathered, sum_i exp(A_i - m).
struct __align__(16) ChunkHdr {
  int32_t cnt;
  float mx;
  float z;
  int32_t unused;
};

// ----------------------------------------------------------------------------
// Shared argument blocks (passed by value).

struct StreamArgs {
  // pointers first: the compiler may merge neighbouring field loads into one vector
  // load, and a pointer rebuilt from a merged integer loses its global address space
  // (its loads become flat loads, which the LDS waits of a thread also wait for)
  const void* q;           // [B, h_q, DK]
  const void* k;           // [B, h_k, l_max, DK]
  const void* v;           // [B, h_v, l_max, DV] (gathering kernels)
  const int32_t* l_kv;     // [B]
  const float* tau;        // [B*h_q] threshold (select kernels)
  float* scores;           // [B*h_q, lpad] fp32 logits (refresh steps and forced refresh)
  int32_t* surv_idx;       // [B*h_q, lpad] kept indices, one CH-segment per chunk
  float* surv_val;         // [B*h_q, lpad] kept logits; also the threshold candidates
  ChunkHdr* chunk_hdr;     // [B*h_q, nch] per chunk: kept count, largest kept logit, sum w
  float* part;             // [B*h_q, DV/16, nch, 16] chunk records: sum w*v, 16 columns per slice
  unsigned* hist;          // [8, B*h_q, 256] top-digit histogram copies (zero between calls)
  unsigned* cand_cnt;      // [B*h_q] candidates of the threshold select (zero between calls)
  const int32_t* ptab;     // paged caches: [B, ptab_stride] page ids (the kernels' PAGED form)
  long long lpad;
  int h_q, h_k, h_v, g_k, g_v, htiles, l_max, nch, N;  // g_k = h_q/h_k, g_v = h_q/h_v
  int max_l_kv;            // host bound of l_kv[]; larger device values are clamped
  int hsplit;              // blocks sharing one chunk in k_qk_select (heads split among them)
  float scale;
  int ptab_stride, page_shift;  // paged caches: page table row stride, log2(tokens per page)
  int num_pages;           // paged caches: pages per pool (page ids are clamped below it)
};

// Token rows of one (sequence, head) of a key or value cache. Contiguous caches hold
// [B, heads, l_max, D]. Paged caches (PAGED) hold pages of 2^shift tokens (at least
// 16, so a 16-key tile never straddles two pages), each page [heads, 2^shift, D];
// sequence b's page table row lists the page of its tokens [p 2^shift, (p+1) 2^shift).
template <typename T, int D, bool PAGED> struct CacheRows;

template <typename T, int D> struct CacheRows<T, D, false> {
  static constexpr bool kPaged = false;
  const T* p;
  __device__ __forceinline__ CacheRows(const void* base, const int32_t*, int, int, int, int b, int head,
                                       int heads, int l_max)
      : p(reinterpret_cast<const T*>(base) + (size_t)(b * heads + head) * l_max * D) {}
  __device__ __forceinline__ const T* row(int i) const { return p + (size_t)i * D; }
  // first row of the 16-key tile starting at t0 (a multiple of 16, wave-uniform)
  __device__ __forceinline__ const T* tile(int t0) const { return p + (size_t)t0 * D; }
};

// Page ids are clamped into the pool, so a table entry that is never meant to be
// used (a page past the sequence's length, read by a speculative load) still
// addresses memory inside the pool.
template <typename T, int D> struct CacheRows<T, D, true> {
  static constexpr bool kPaged = true;
  const T* p;            // this head's rows in page 0
  const int32_t* tab;    // this sequence's page table row
  size_t page_elems;     // elements per page (all heads)
  int shift;
  unsigned last_page;
  __device__ __forceinline__ CacheRows(const void* base, const int32_t* ptab, int stride, int shift_,
                                       int num_pages, int b, int head, int heads, int)
      : p(reinterpret_cast<const T*>(base) + ((size_t)head * D << shift_)),
        tab(ptab + (size_t)b * stride),
        page_elems((size_t)heads * D << shift_),
        shift(shift_),
        last_page((unsigned)num_pages - 1u) {}
  __device__ __forceinline__ const T* in_page(int page, int i) const {
    const unsigned pg = min((unsigned)page, last_page);
    return p + (size_t)pg * page_elems + (size_t)(i & ((1 << shift) - 1)) * D;
  }
  __device__ __forceinline__ const T* row(int i) const { return in_page(tab[i >> shift], i); }
  __device__ __forceinline__ const T* tile(int t0) const {
    const int tu = __builtin_amdgcn_readfirstlane(t0);  // one page-table read per wave
    return in_page(tab[tu >> shift], tu);
  }
};

template <typename T, int D, bool PAGED>
__device__ __forceinline__ CacheRows<T, D, PAGED> key_rows(const StreamArgs& a, int b, int g) {
  return CacheRows<T, D, PAGED>(a.k, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, g, a.h_k, a.l_max);
}
template <typename T, int D, bool PAGED>
__device__ __forceinline__ CacheRows<T, D, PAGED> value_rows(const StreamArgs& a, int b, int vh) {
  return CacheRows<T, D, PAGED>(a.v, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, vh, a.h_v, a.l_max);
}

// Kept entries of one chunk, per head of the tile, staged in LDS: offset of the key
// inside the chunk and its logit; plus the count and the largest kept logit (as an
// order key) per head; with paged caches also the pages of the chunk's tokens.
template <int CH> struct KeptLds {
  uint16_t off[16][CH];
  float val[16][CH];
  int cnt[16];
  unsigned mx[16];
  int32_t pg[CH >= 16 ? CH / 16 : 1];
};

// Paged caches: the page ids of the tokens [base, base + CH) of sequence b into
// kl.pg (one page when pages hold at least CH tokens, else CH / 2^shift pages; ids
// past the table row read as page 0 and are never used). Threads 0..CH/16-1.
template <int CH>
__device__ __forceinline__ void stage_pages(KeptLds<CH>& kl, const StreamArgs& a, int b, int base) {
  const int np = (CH >> a.page_shift) > 0 ? (CH >> a.page_shift) : 1;
  const int t = threadIdx.x;
  if (t < np) {
    const int pi = (base >> a.page_shift) + t;
    kl.pg[t] = pi < a.ptab_stride ? a.ptab[(size_t)b * a.ptab_stride + pi] : 0;
  }
}

// Eq. (7) split over chunks of keys: the chunk record of row (b, j) for every head j
// of the tile that this block owns (heads j0 + h with h mod hsplit == hs): the value
// rows of its kept entries, gathered from value head v(j), summed as
// sum_i w_i V[i,:] into the D/16 column slices and sum_i w_i into the chunk header,
// w_i = exp(A_i - m), m = the chunk's largest kept logit of the row (every w_i <= 1).
// The block's 16 groups of 16 lanes are spread over the owned heads (16 / owned
// groups each, taking alternate kept entries); the groups of one head add their sums
// in LDS. Rows without kept entries in the chunk write nothing. Called by every
// thread of the block. D is the value head dimension.
template <typename T, int D, int CH, bool PAGED>
__device__ __forceinline__ void chunk_records(const KeptLds<CH>& kl, const StreamArgs& a, int b, int j0, int nh,
                                              int c, int hs, int hsplit) {
  constexpr int EPL = Unpack<T>::kN;                    // columns per 16-byte piece
  constexpr int PIECES = D / EPL;                       // pieces per value row
  constexpr int RPG = PIECES >= 16 ? 1 : 16 / PIECES;  // rows one group load covers
  constexpr int PPL = PIECES >= 16 ? PIECES / 16 : 1;   // pieces per lane per row
  constexpr int U = 4;                                  // loads in flight per lane
  constexpr int NG = kBlock / 16;                       // groups of 16 lanes
  __shared__ float s_part[NG][D + 1];
  const int nown = hsplit == 1 ? nh : (nh - hs + hsplit - 1) / hsplit;  // owned heads (uniform)
  if (nown <= 0) return;
  const int gph = NG / nown;                            // groups per owned head
  const int tid = threadIdx.x, grp = tid >> 4, gl = tid & 15;
  const int oh = gph == 1 ? grp : grp % nown, sg = gph == 1 ? 0 : grp / nown;
  const bool act = gph == 1 ? grp < nown : sg < gph;
  const int h = hs + (act ? oh : 0) * hsplit;
  const int n = act ? kl.cnt[h] : 0;
  if (gph == 1 && n == 0) return;                       // one group per head: no LDS merge follows
  const int sub = RPG > 1 ? gl / PIECES : 0;
  const int pc = RPG > 1 ? gl % PIECES : gl;
  const int j = j0 + h;
  const int vh = j / a.g_v;
  const int base = c * CH;
  const T* vrow = reinterpret_cast<const T*>(a.v) + ((size_t)(b * a.h_v + vh) * a.l_max + base) * D + pc * EPL;
  const CacheRows<T, D, true> vpg(a.v, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, vh, a.h_v, 0);
  const int pbase = base & ((1 << a.page_shift) - 1);  // offset of the chunk in its first page
  const float m = act ? order_key_to_f32(kl.mx[h]) : 0.f;
  float acc[PPL][EPL];
#pragma unroll
  for (int p = 0; p < PPL; ++p)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[p][e] = 0.f;
  float z = 0.f;
  // row slots k = sg, sg + gph, ... ; slot k holds entries k*RPG .. k*RPG + RPG-1
  for (int k0 = sg; k0 * RPG < n; k0 += gph * U) {
    uint4 x[U][PPL];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (k0 + u * gph) * RPG + sub;
      w[u] = 0.f;
#pragma unroll
      for (int p = 0; p < PPL; ++p) x[u][p] = make_uint4(0, 0, 0, 0);
      if (e < n) {
        const int off = kl.off[h][e];
        const T* r = PAGED ? vpg.in_page(kl.pg[(pbase + off) >> a.page_shift], base + off) + pc * EPL
                           : vrow + (size_t)off * D;
#pragma unroll
        for (int p = 0; p < PPL; ++p) x[u][p] = ld16(r + 16 * p * EPL);
        w[u] = expf(kl.val[h][e] - m);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        float f[EPL];
        Unpack<T>::run(x[u][p], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[p][e] += w[u] * f[e];
      }
      z += w[u];
    }
  }
  if constexpr (RPG == 2) {  // the two rows of a group load: lanes l and l ^ 8
    auto add = [](float u, float v) { return u + v; };
#pragma unroll
    for (int p = 0; p < PPL; ++p)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[p][e] = xor_lanes<8>(acc[p][e], add);
    z = xor_lanes<8>(z, add);
  }
  static_assert(RPG <= 2, "value rows of at least 8 pieces");
  const long long nch16 = (long long)a.nch * 16;
  if (gph == 1) {
    // one group per head: it writes the record itself
    if (sub != 0) return;
    const long long row = (long long)b * a.h_q + j;
    float* rec = a.part + row * (D / 16) * nch16 + (long long)c * 16;
#pragma unroll
    for (int p = 0; p < PPL; ++p)
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const int col = (pc + 16 * p) * EPL + e;
        *reinterpret_cast<float4*>(rec + (long long)(col >> 4) * nch16 + (col & 15)) =
            make_float4(acc[p][e], acc[p][e + 1], acc[p][e + 2], acc[p][e + 3]);
      }
    if (gl == 0) a.chunk_hdr[row * a.nch + c].z = z;
    return;
  }
  if (act && sub == 0) {
#pragma unroll
    for (int p = 0; p < PPL; ++p)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_part[grp][(pc + 16 * p) * EPL + e] = acc[p][e];
    if (gl == 0) s_part[grp][D] = z;
  }
  __syncthreads();
  for (int t = tid; t < nown * (D + 1); t += kBlock) {
    const int o = t / (D + 1), col = t - o * (D + 1);
    const int hh = hs + o * hsplit;
    if (kl.cnt[hh] == 0) continue;
    float sum = 0.f;
    for (int q = 0; q < gph; ++q) sum += s_part[o + q * nown][col];
    const long long row = (long long)b * a.h_q + j0 + hh;
    if (col < D) a.part[row * (D / 16) * nch16 + (long long)(col >> 4) * nch16 + (long long)c * 16 + (col & 15)] = sum;
    else a.chunk_hdr[row * a.nch + c].z = sum;
  }
}

// Source of the logits of k_qk_select.
enum SelectMode { kFromKeys = 0, kFromKeysSpeculative = 1, kFromScores = 2 };

// ----------------------------------------------------------------------------
// Logits of one chunk of keys for the (up to) 16 query heads of one head tile, then
// the Atop-N comparison against each head's threshold. Kept (index, logit) pairs go
// to the chunk's segment of the row's kept list; the chunk's count and largest kept
// logit are recorded. MODE kFromScores reads the logits stored by k_scores_hist (a
// refresh step: the fp32 values the threshold was selected from); MODE
// kFromKeysSpeculative (one sequence) issues the key loads before l_kv arrives.
// With GATHER the block also writes the chunk records of eq. (7) (chunk_records).
// When hsplit > 1, hsplit blocks share each chunk: block hs compares and gathers only
// the heads h of the tile with h mod hsplit == hs (every block computes all the
// tile's logits; its duplicate key reads hit the cache).
// DK and DV are the key and value head dimensions.
// grid = (nch, h_k * htiles * hsplit, B), block = 256.
template <typename T, int DK, int DV, int MODE, bool GATHER, bool PAGED, int W>
__global__ __launch_bounds__(kBlock) void k_qk_select(const StreamArgs a) {
  constexpr int TPW = StreamCfg<T, DK, W>::kTPW;
  constexpr int CH = StreamCfg<T, DK, W>::kChunk;
  // every argument the key stream needs is read in one batch, before any arithmetic
  // on them (otherwise the pointers' reads may wait behind the index arithmetic)
  const T* const kbase = reinterpret_cast<const T*>(a.k);
  const T* const qbase = reinterpret_cast<const T*>(a.q);
  const int hsplit = a.hsplit, htiles = a.htiles, g_k = a.g_k, h_k = a.h_k, h_q = a.h_q;
  const int l_max = a.l_max, max_l_kv = a.max_l_kv;
  const float scale = a.scale;
  __builtin_amdgcn_sched_barrier(0);
  const int c = blockIdx.x, b = blockIdx.z;
  const int gt = hsplit == 1 ? (int)blockIdx.y : (int)blockIdx.y / hsplit;
  const int hs = blockIdx.y - gt * hsplit;
  const int g = htiles == 1 ? gt : gt / htiles, ht = gt - g * htiles;
  const int j0 = g * g_k + ht * 16;
  const int nh = min(16, g_k - ht * 16);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * h_q + j0;
  const int base = c * CH;
  const int wbase = base + wv * 16 * TPW;
  const bool live = hh < nh && (hsplit == 1 || hh % hsplit == hs);

  floatx4 sc[TPW];
  QK<T, DK> qk;
  const CacheRows<T, DK, PAGED> kh(kbase, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, g, h_k, l_max);
  if constexpr (MODE == kFromKeysSpeculative) {
    qk.load_q(qbase + (size_t)row0 * DK, nh, lane);
    score_tiles<T, DK, TPW>(sc, qk, kh, wbase, max_l_kv, lane, scale);
  }
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (base >= L) return;

  __shared__ KeptLds<GATHER ? CH : 1> kl;
  if (tid < 16) {
    kl.cnt[tid] = 0;
    kl.mx[tid] = 0u;
  }
  if constexpr (PAGED && GATHER) stage_pages<CH>(kl, a, b, base);
  const float tau_l = live ? a.tau[row0 + hh] : 0.f;
  if constexpr (MODE == kFromScores) {
    const float* srow = a.scores + (long long)(row0 + (live ? hh : 0)) * a.lpad;
#pragma unroll
    for (int t = 0; t < TPW; ++t) sc[t] = *reinterpret_cast<const floatx4*>(srow + wbase + 16 * t + 4 * kq);
  } else if constexpr (MODE == kFromKeys) {
    qk.load_q(qbase + (size_t)row0 * DK, nh, lane);
    score_tiles<T, DK, TPW>(sc, qk, kh, wbase, L, lane, scale);
  }
  __syncthreads();

  // this lane's kept entries as a bit mask (bit 4t+r: key wbase+16t+4kq+r), one LDS
  // atomic per lane for their slots, then one short loop over the set bits
  static_assert(TPW * 4 <= 32, "kept mask holds 32 entries");
  unsigned pm = 0u;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = wbase + 16 * t + 4 * kq + r;
      if (live && key < L && sc[t][r] >= tau_l) pm |= 1u << (4 * t + r);
    }
  if (pm) {
    const long long seg = (long long)(row0 + hh) * a.lpad + base;
    int slot = atomicAdd(&kl.cnt[hh], __popc(pm));
    float vmax = -INFINITY;
    do {
      const int bit = __builtin_ctz(pm);
      pm &= pm - 1u;
      float v = sc[0][0];
#pragma unroll
      for (int e = 1; e < TPW * 4; ++e) v = (bit == e) ? sc[e >> 2][e & 3] : v;
      const int key = wbase + 16 * (bit >> 2) + 4 * kq + (bit & 3);
      a.surv_idx[seg + slot] = key;
      a.surv_val[seg + slot] = v;
      if constexpr (GATHER) {
        kl.off[hh][slot] = (uint16_t)(key - base);
        kl.val[hh][slot] = v;
      }
      vmax = fmaxf(vmax, v);
      ++slot;
    } while (pm);
    atomicMax(&kl.mx[hh], order_key(vmax));
  }
  __syncthreads();
  if (tid < nh && (hsplit == 1 || tid % hsplit == hs)) {
    const long long o = (long long)(row0 + tid) * a.nch + c;
    *reinterpret_cast<int2*>(a.chunk_hdr + o) = make_int2(kl.cnt[tid], __float_as_int(order_key_to_f32(kl.mx[tid])));
  }
  if constexpr (GATHER) chunk_records<T, DV, CH, PAGED>(kl, a, b, j0, nh, c, hs, hsplit);
}

// The chunk records of eq. (7) from kept lists already in the workspace (the
// separately callable gather stage): stages each head's kept entries of the chunk
// in LDS, then chunk_records. grid = (nch, h_k * htiles, B), block = 256.
template <typename T, int DK, int DV, bool PAGED, int W>
__global__ __launch_bounds__(kBlock) void k_chunk_gather(const StreamArgs a) {
  constexpr int CH = StreamCfg<T, DK, W>::kChunk;
  const int c = blockIdx.x, gy = blockIdx.y, b = blockIdx.z;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int base = c * CH;
  if (base >= L) return;
  const int g = gy / a.htiles, ht = gy - g * a.htiles;
  const int j0 = g * a.g_k + ht * 16;
  const int nh = min(16, a.g_k - ht * 16);
  const int tid = threadIdx.x;
  const int row0 = b * a.h_q + j0;
  __shared__ KeptLds<CH> kl;
  if (tid < nh) {
    const ChunkHdr h = a.chunk_hdr[(long long)(row0 + tid) * a.nch + c];
    kl.cnt[tid] = h.cnt;
    kl.mx[tid] = order_key(h.mx);
  }
  if constexpr (PAGED) stage_pages<CH>(kl, a, b, base);
  __syncthreads();
  for (int e = tid; e < nh * CH; e += kBlock) {
    const int h = e / CH, i = e - h * CH;
    if (i < kl.cnt[h]) {
      const long long at = (long long)(row0 + h) * a.lpad + base + i;
      kl.off[h][i] = (uint16_t)(a.surv_idx[at] - base);
      kl.val[h][i] = a.surv_val[at];
    }
  }
  __syncthreads();
  chunk_records<T, DV, CH, PAGED>(kl, a, b, j0, nh, c, 0, 1);
}

// ----------------------------------------------------------------------------
// Refresh, pass 1: logits of every cached key stored as fp32, plus a histogram of
// the top 8 bits of their order keys per query head, accumulated into copy
// (chunk mod kHistCopies) of a.hist: the logits of a row fall into a few bins, and
// the copies spread the device atomics of the row's blocks over more addresses.
// D is the key head dimension. grid = (nch, h_k * htiles, B), block = 256.
constexpr int kHistCopies = 8;

template <typename T, int D, bool PAGED, int W>
__global__ __launch_bounds__(kBlock) void k_scores_hist(const StreamArgs a) {
  constexpr int TPW = StreamCfg<T, D, W>::kTPW;
  constexpr int CH = StreamCfg<T, D, W>::kChunk;
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
  const auto kh = key_rows<T, D, PAGED>(a, b, g);
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
    if (h) {
      const long long rows = (long long)gridDim.z * a.h_q;
      atomicAdd(&a.hist[((c % kHistCopies) * rows + row0 + e / 256) * 256 + (e & 255)], h);
    }
  }
}

// ----------------------------------------------------------------------------
// Refresh, pass 2: candidates for the exact threshold. The sum of the row's
// histogram copies gives the 8-bit bin that holds its N-th largest logit; each block
// copies the logits of its slice that fall in that bin to the row's candidate list
// (stored in the row's kept-logit buffer, free at this point of a refresh step).
// grid = (P, h_q, B) with P = ceil(max_l_kv / kSelSlice), block = 256.
constexpr int kSelSlice = 4096;   // logits scanned per block
constexpr int kCandLds = 8192;    // candidates the finishing block stages in LDS
constexpr int kRowThreads = 1024; // threads of the one-block-per-row kernels

// Sum of the kHistCopies copies of bin `bin` of row `row`; with `clear`, the copies
// are returned to zero.
__device__ __forceinline__ unsigned hist_sum(unsigned* hist, long long rows, long long row, int bin, bool clear) {
  unsigned v[kHistCopies];
#pragma unroll
  for (int cp = 0; cp < kHistCopies; ++cp) v[cp] = hist[(cp * rows + row) * 256 + bin];
  unsigned h = 0u;
#pragma unroll
  for (int cp = 0; cp < kHistCopies; ++cp) {
    h += v[cp];
    if (clear) hist[(cp * rows + row) * 256 + bin] = 0u;
  }
  return h;
}

__global__ __launch_bounds__(kBlock) void k_cand_collect(const StreamArgs a) {
  const int p = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const long long rows = (long long)gridDim.z * a.h_q;
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

  // the slice's logits are loaded with the histogram, before the bin is known
  const int hi = min(lo + kSelSlice, L);
  constexpr int PER = kSelSlice / kBlock;
  float vals[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = lo + u * kBlock + tid;
    vals[u] = (i < hi) ? a.scores[rbase + i] : 0.f;
  }
  s_hist[tid] = hist_sum(a.hist, rows, row, tid, false);
  if (tid == 0) s_cc = 0;
  __syncthreads();
  digit_of_kth_largest(s_hist, (unsigned)N, s_itmp, s_res);
  const unsigned d1 = s_res[0];
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
// l_kv == 0) and returns the row's histogram copies and candidate count to zero.
// grid = (h_q, B), block = 1024.
__global__ __launch_bounds__(kRowThreads) void k_select_finish(const StreamArgs a, float* tau_out) {
  constexpr int NT = kRowThreads;
  const int j = blockIdx.x, b = blockIdx.y;
  const long long rows = (long long)gridDim.y * a.h_q;
  const long long row = (long long)b * a.h_q + j;
  const int L = min(a.l_kv[b], a.max_l_kv);
  const int N = a.N;
  const int tid = threadIdx.x;
  if (L <= 0) return;  // no block added to this row's histograms

  __shared__ unsigned s_hist[256];
  __shared__ int s_itmp[NT / kWave];
  __shared__ unsigned s_res[2];
  __shared__ float s_cand[kCandLds];

  const unsigned C = a.cand_cnt[row];
  if (tid < 256) s_hist[tid] = hist_sum(a.hist, rows, row, tid, true);
  if (N >= L) {
    if (tid == 0) tau_out[row] = -INFINITY;
    return;
  }
  __syncthreads();
  digit_of_kth_largest<NT>(s_hist, (unsigned)N, s_itmp, s_res);
  const unsigned d1 = s_res[0], k1 = s_res[1];
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
  }
  // one call per source, so that each reads through a pointer of known kind (LDS or global)
  const uint32_t key =
      C <= (unsigned)kCandLds
          ? radix_select_block<NT>(s_cand, (long long)C, d1 << 24, 0xff000000u, 16, k1, s_hist, s_itmp, s_res)
          : radix_select_block<NT>(cand, (long long)C, d1 << 24, 0xff000000u, 16, k1, s_hist, s_itmp, s_res);
  if (tid == 0) {
    tau_out[row] = order_key_to_f32(key);
    a.cand_cnt[row] = 0u;
  }
}

// ----------------------------------------------------------------------------
// Sparse softmax and value gather (eq. (7)) over the kept entries of one row.

struct GatherArgs {
  // own pointers before the embedded block (no pointer right after a scalar field:
  // see StreamArgs)
  float* tau;             // [B*h_q] (written only where a row is refreshed)
  void* out;              // [B*h_q, DV]
  int32_t* sel_count;     // [B*h_q] or null
  int32_t* sel_idx;       // [B*h_q, sel_cap] or null
  int32_t* flags;         // [B*h_q] or null
  StreamArgs s;           // q, k, v, l_kv, logit buffer, kept lists and counts
  int sel_cap, out_bf16, refreshed;
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
  for (int e = 0; e < RG::EPL; ++e) acc[e] = strided_lane_sum<RG::G>(acc[e]);
  z = strided_lane_sum<RG::G>(z);
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
// and the sparse softmax-PV. Used for a stale threshold that keeps nothing (the
// forced refresh). Writes out, tau (refresh only), sel_count, sel_idx and flags.
template <typename T, int DK, int DV, int NT, bool PAGED>
__device__ void exact_row(const GatherArgs& a, int b, int j, int L, bool refresh_tau, float (*s_red)[DV],
                          float* s_z) {
  constexpr int NW = NT / kWave;
  constexpr int TPW = StreamCfg<T, DK>::kTPW;
  using RG = RowGather<T, DV, NT>;
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
    QK<T, DK> qk;
    qk.load_q(reinterpret_cast<const T*>(s.q) + (size_t)(b * s.h_q + j0) * DK, nh, lane);
    const auto kh = key_rows<T, DK, PAGED>(s, b, g);
    const int kq = lane >> 4;
    for (int base = 0; base < L; base += NW * 16 * TPW) {
      const int wbase = base + wv * 16 * TPW;
      if (wbase < L) {
        floatx4 sc[TPW];
        score_tiles<T, DK, TPW>(sc, qk, kh, wbase, L, lane, s.scale);
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

  const int vh = j / s.g_v;
  const int grp = tid / RG::G, gl = tid - grp * RG::G;
  const auto vr = value_rows<T, DV, PAGED>(s, b, vh);
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
      Unpack<T>::run(ld16(vr.row(idx) + gl * RG::EPL), x);
#pragma unroll
      for (int e = 0; e < RG::EPL; ++e) acc[e] += w * x[e];
      z += w;
      if (gl == 0 && a.sel_idx && kept + p < a.sel_cap) a.sel_idx[row * a.sel_cap + kept + p] = idx;
    }
    kept += n;
    __syncthreads();
  }
  reduce_rows<T, DV, NT>(acc, z, s_red, s_z);
  for (int d = tid; d < DV; d += NT) store_out<DV>(a, row, d, kept > 0 ? s_red[0][d] / s_z[0] : 0.f);
  if (tid == 0) {
    if (refresh_tau) a.tau[row] = tau;
    if (a.sel_count) a.sel_count[row] = kept;
    if (a.flags) a.flags[row] = refresh_tau ? 3 : (a.refreshed ? 1 : 0);
  }
  __syncthreads();
}

// Merge of the chunk records of each row (b, j) (eq. (7) reassembled from its
// chunks): M = the row's largest kept logit (the maximum of the chunk maxima),
// O = sum_c e_c o_c / sum_c e_c z_c with e_c = exp(m_c - M) over the chunks that kept
// something. Block x takes output columns [16x, 16x+16) (column slice x of the
// records, contiguous over chunks); lane quarter q = t mod 4 of thread t takes
// columns 16x+4q..16x+4q+3 of chunks t/4, t/4+64, ..., so each wave load reads 1 KB
// of consecutive records. Headers, slices and the first kept indices of the first
// kCombRegs*64 chunks are read in one round of independent loads, issued with l_kv
// and whether or not a chunk kept anything; values of chunks past l_kv or without
// kept entries are never used. The kept indices are exported in the same pass
// (chunk c by block c mod gridDim.x). A row that kept nothing is recomputed exactly
// by block 0 (forced refresh). DK and DV are the key and value head dimensions.
// grid = (DV / 16, h_q, B), block = 256.
constexpr int kCombRegs = 8;  // chunk slots per thread read speculatively

template <typename T, int DK, int DV, bool PAGED, int W>
__global__ __launch_bounds__(kBlock) void k_split_combine(const GatherArgs a) {
  constexpr int CH = StreamCfg<T, DK, W>::kChunk;
  constexpr int CB = DV / 16;
  constexpr int kSlots = kBlock / 4;  // chunks per pass of the block
  const StreamArgs& sa = a.s;
  const int cb = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const long long row = (long long)b * sa.h_q + j;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int qd = tid & 3, r0 = tid >> 2;
  const int col = cb * 16;

  __shared__ int s_itmp[kWaves];
  __shared__ float s_ftmp[kWaves];
  __shared__ float s_acc[kWaves][4][17];
  __shared__ float s_red[kWaves][DV];
  __shared__ float s_z[kWaves];

  const ChunkHdr* hdr = sa.chunk_hdr + row * sa.nch;
  const float4* sl = reinterpret_cast<const float4*>(sa.part + (row * CB + cb) * (long long)sa.nch * 16) + qd;
  const int32_t* kept = sa.surv_idx + row * sa.lpad;
  int32_t* exp_idx = a.sel_idx ? a.sel_idx + row * a.sel_cap : nullptr;
  const bool exporter = exp_idx != nullptr && qd == 0;

  float4 hreg[kCombRegs], xreg[kCombRegs];
  int4 ireg[kCombRegs];
#pragma unroll
  for (int k = 0; k < kCombRegs; ++k) {
    const int c = k * kSlots + r0;
    if (c < sa.nch) {
      hreg[k] = *reinterpret_cast<const float4*>(hdr + c);
      xreg[k] = sl[(long long)c * 4];
      if (exporter && c % CB == cb) ireg[k] = *reinterpret_cast<const int4*>(kept + (long long)c * CH);
    }
  }
  const int L = min(sa.l_kv[b], sa.max_l_kv);
  if (L <= 0) {
    if (tid < 16) store_out<DV>(a, row, col + tid, 0.f);
    if (cb == 0 && tid == 0) {
      if (a.sel_count) a.sel_count[row] = 0;
      if (a.flags) a.flags[row] = 0;
    }
    return;
  }
  const int nch_b = (L + CH - 1) / CH;
  int nreg[kCombRegs];
  float m = -INFINITY;
  int tsum = 0;
#pragma unroll
  for (int k = 0; k < kCombRegs; ++k) {
    nreg[k] = (k * kSlots + r0 < nch_b) ? __float_as_int(hreg[k].x) : 0;
    if (nreg[k] > 0) m = fmaxf(m, hreg[k].y);
    tsum += nreg[k];
  }
  for (int c = kCombRegs * kSlots + r0; c < nch_b; c += kSlots) {
    const ChunkHdr h = hdr[c];
    if (h.cnt > 0) m = fmaxf(m, h.mx);
    tsum += h.cnt;
  }
  float M;
  int total;
  int pos = block_max_excl_scan(m, qd == 0 ? tsum : 0, s_ftmp, s_itmp, M, total);
  if (total == 0) {
    if (cb == 0) exact_row<T, DK, DV, kBlock, PAGED>(a, b, j, L, true, s_red, s_z);
    return;
  }

  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  auto add = [&](const float4& x, float mc, float zc) {
    const float e = expf(mc - M);
    o[0] += e * x.x;
    o[1] += e * x.y;
    o[2] += e * x.z;
    o[3] += e * x.w;
    if (qd == 0) z += e * zc;
  };
  auto export_rest = [&](int c, int n, int from) {
    for (int i = from; i < n && pos + i < a.sel_cap; ++i) exp_idx[pos + i] = kept[(long long)c * CH + i];
  };
#pragma unroll
  for (int k = 0; k < kCombRegs; ++k) {
    const int c = k * kSlots + r0, n = nreg[k];
    if (n > 0) {
      add(xreg[k], hreg[k].y, hreg[k].z);
      if (exporter && c % CB == cb) {
        const int first[4] = {ireg[k].x, ireg[k].y, ireg[k].z, ireg[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < n && pos + i < a.sel_cap) exp_idx[pos + i] = first[i];
        export_rest(c, n, 4);
      }
      pos += n;
    }
  }
  for (int c = kCombRegs * kSlots + r0; c < nch_b; c += kSlots) {
    const ChunkHdr h = hdr[c];
    if (h.cnt > 0) {
      add(sl[(long long)c * 4], h.mx, h.z);
      if (exporter && c % CB == cb) export_rest(c, h.cnt, 0);
      pos += h.cnt;
    }
  }
  // lanes of one quarter within each row of 16 lanes, then rows and waves via LDS
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = row_stride4_sum(o[e]);
  z = row_stride4_sum(z);
  if ((lane & 15) < 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s_acc[wv][lane >> 4][4 * qd + e] = o[e];
    if (qd == 0) s_acc[wv][lane >> 4][16] = z;
  }
  __syncthreads();
  if (tid < 16) {
    float oo = 0.f, zz = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        oo += s_acc[w][r][tid];
        zz += s_acc[w][r][16];
      }
    store_out<DV>(a, row, col + tid, oo / zz);
  }
  if (cb == 0 && tid == 0) {
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
  float* part;     // [B*h_q, nchd, DV+4] per-chunk (m, Z, -, -, o[DV])
  void* out;
  const int32_t* ptab;  // paged caches: [B, ptab_stride] page ids
  int h_q, h_k, h_v, g, l_max, nchd, out_bf16;  // g = h_q / h_v query heads per value head
  int max_l_kv;
  float scale;
  int ptab_stride, page_shift, num_pages;     // paged caches (see StreamArgs)
};

// DK and DV are the key and value head dimensions.
// grid = (nchd, h_v, B), block = 256. Each block takes one chunk of CHD keys and one
// value head v: the logits of its g query heads against their key head (h_k divides
// h_v, so the g heads share one; MFMA), the chunk's softmax numerator relative to the
// chunk maximum, and its product with the chunk's rows of value head v (VALU). The
// key tiles are loaded first; the value tiles follow in two halves (see below).
template <typename T, int DK, int DV, int GH, bool PAGED>
__global__ __launch_bounds__(kBlock) void k_dense_partial(const DenseArgs a) {
  constexpr int TPW = StreamCfg<T, DK>::kTPW;
  constexpr int CHD = StreamCfg<T, DK>::kChunk;
  constexpr int EPL = Unpack<T>::kN;
  constexpr int G = DV / EPL;                        // lanes per value row
  constexpr int VL = (16 * DV) / (EPL * kWave);      // 16-byte value loads per lane per tile
  const T* const kbase = reinterpret_cast<const T*>(a.k);
  const T* const vbase = reinterpret_cast<const T*>(a.v);
  const T* const qbase = reinterpret_cast<const T*>(a.q);
  const int h_k = a.h_k, h_v = a.h_v, l_max = a.l_max, gq = a.g, h_q = a.h_q, max_l_kv = a.max_l_kv;
  const float scale = a.scale;
  __builtin_amdgcn_sched_barrier(0);
  const int c = blockIdx.x, vg = blockIdx.y, b = blockIdx.z;
  const int kg = h_k == h_v ? vg : vg / (h_v / h_k);  // key head of this value head's query heads
  const int L = min(a.l_kv[b], max_l_kv);
  const int base = c * CHD;
  if (base >= L) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * h_q + vg * gq;

  __shared__ float s_p[kWaves][TPW][16][GH];
  __shared__ float s_m[kWaves][GH], s_z[kWaves][GH];
  __shared__ float s_o[kWaves][GH][DV];

  const CacheRows<T, DK, PAGED> kh(kbase, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, kg, h_k, l_max);
  const CacheRows<T, DV, PAGED> vh(vbase, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, vg, h_v, l_max);
  const int wbase = base + wv * 16 * TPW;

  QK<T, DK> qk;
  qk.load_q(qbase + (size_t)row0 * DK, gq, lane);
  floatx4 sc[TPW];
  score_tiles<T, DK, TPW>(sc, qk, kh, wbase, L, lane, scale);
  // The value tiles are loaded once the key tiles are consumed, in two halves: the
  // first half before the softmax, the second after the first half's products, so
  // that key tiles, value tiles and the accumulators never all hold registers at
  // once and four blocks fit on a compute unit. Load latency is covered by the
  // softmax and by the other resident blocks.
  constexpr int VH = TPW >= 2 ? 2 : 1;  // value-tile halves
  constexpr int TPH = TPW / VH;         // tiles per half
  // load r of tile t covers flat element (r*64 + lane) of the 16 x G grid
  auto load_values = [&](uint4 (&vb)[TPH][VL], int t_first) {
#pragma unroll
    for (int tt = 0; tt < TPH; ++tt) {
      const int t = t_first + tt;
      const int t0 = min(wbase + 16 * t, (L - 1) & ~15);  // a clamped tile lies inside one page
      const T* vt = PAGED ? vh.tile(t0) : vh.row(0);
#pragma unroll
      for (int r = 0; r < VL; ++r) {
        const int e = r * kWave + lane;
        if constexpr (PAGED) {
          const int key = min(t0 + e / G, L - 1);
          vb[tt][r] = ld16(vt + (size_t)(key - t0) * DV + (e % G) * EPL);
        } else {
          const int key = min(wbase + 16 * t + e / G, L - 1);
          vb[tt][r] = ld16(vt + (size_t)key * DV + (e % G) * EPL);
        }
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  uint4 vb[TPH][VL];
  load_values(vb, 0);

  float mh = -INFINITY;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = wbase + 16 * t + 4 * kq + r;
      if (key >= L) sc[t][r] = -INFINITY;
      mh = fmaxf(mh, sc[t][r]);
    }
  mh = strided_lane_max<16>(mh);
  float zh = 0.f;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = (mh == -INFINITY) ? 0.f : expf(sc[t][r] - mh);
      zh += p;
      if (hh < GH) s_p[wv][t][4 * kq + r][hh] = p;
    }
  zh = strided_lane_sum<16>(zh);
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
  for (int hv = 0; hv < VH; ++hv) {
    if (hv > 0) {
      __builtin_amdgcn_sched_barrier(0);
      load_values(vb, hv * TPH);
    }
#pragma unroll
    for (int tt = 0; tt < TPH; ++tt)
#pragma unroll
      for (int r = 0; r < VL; ++r) {
        const int t = hv * TPH + tt;
        const int e = r * kWave + lane;
        const int k16 = e / G;
        float x[EPL];
        Unpack<T>::run(vb[tt][r], x);
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float p = s_p[wv][t][k16][h];
#pragma unroll
          for (int q = 0; q < EPL; ++q) o[h][q] += p * x[q];
        }
      }
  }
  // lanes with the same column group (lane % G) hold partial sums over different keys
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int q = 0; q < EPL; ++q) o[h][q] = strided_lane_sum<G>(o[h][q]);
  if (lane < G) {
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int q = 0; q < EPL; ++q) s_o[wv][h][lane * EPL + q] = o[h][q];
  }
  __syncthreads();

  // merge the 4 waves (each relative to its own maximum) and write the chunk partial
  for (int idx = tid; idx < gq * (DV + 1); idx += kBlock) {
    const int h = idx / (DV + 1), d = idx - h * (DV + 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][h];
      const float sw = (mw == -INFINITY) ? 0.f : expf(mw - M);
      acc += sw * (d < DV ? s_o[w][h][d] : s_z[w][h]);
    }
    float* pp = a.part + ((long long)(row0 + h) * a.nchd + c) * (DV + 4);
    if (d < DV) pp[4 + d] = acc;
    else {
      pp[0] = M;
      pp[1] = acc;
    }
  }
}

// Log-sum-exp merge of the chunk partials of each row (b, j). Thread t takes chunks
// t, t+256, ... and 16 columns (four 16-byte loads per chunk). D is the value head
// dimension. grid = (D / 16, h_q, B), block = 256.
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
