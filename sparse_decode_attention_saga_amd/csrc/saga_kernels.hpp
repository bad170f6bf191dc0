// Kernels of the SAGA + Atop-N decode step and of the dense GQA baseline (gfx950).
//
// Stale-threshold step:  k_qk_select<slot records> -> k_sparse_pv          (late value gather)
//                        k_qk_select<chunk records> -> k_split_combine      (early value gather)
// Refresh step:          k_scores_hist [-> k_cand_collect] -> k_select_finish
//                        -> k_qk_select<from stored logits, ...> -> the same combining kernel
// Separate stages:       k_qk_select<kept list> -> k_chunk_gather -> k_split_combine
// Dense GQA baseline:    k_dense_partial -> k_dense_combine
// The host picks the value-gather form per call (late: 256-byte value rows, about one
// kept entry per head and chunk, at least two select blocks per compute unit).
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

#include <type_traits>

#include "saga_device.hpp"

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

// Keys per block of the dense kernel: 4 waves x TPW tiles x 16 keys, TPW the power of
// two (1..8) that keeps a wave's key and value rows within 16 KiB, or 32 KiB where the
// value products run on the matrix cores (bf16, d_v = 128; the VALU form needs the
// registers for its sums); every load of a wave is in flight at once, in registers.
// Measured at the Qwen-shaped 128K layer (h_kv = 2): 36.5 us with 16 KiB, 32.7 us with
// 32 KiB per wave; the Llama-shaped 32K layer (h_kv = 8): 19.5 against 20.4 us.
template <typename T, int DK, int DV> struct DenseCfg {
  static constexpr int kBytes = 16 * (DK + DV) * (int)sizeof(T);  // one tile's keys and values
  static constexpr int kBudget = std::is_same<T, bf16_t>::value && DV == 128 ? 32768 : 16384;
  static constexpr int kFit = kBudget / kBytes;
  static constexpr int kTPW = kFit >= 8 ? 8 : kFit >= 4 ? 4 : kFit >= 2 ? 2 : 1;
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

// Kept entries of one chunk of one row (b, j) for the late value gather: the number
// of kept entries, the largest kept logit and the first kSlotE kept (index, logit)
// pairs in key order. 16-byte piece p of the record holds entries 2p-1 and 2p (piece
// 0: the count, the maximum and entry 0), so four lanes read a record in one load
// each. Entries past kSlotE stay in the chunk's segment of the kept list, at their
// place in it.
constexpr int kSlotE = 7;
struct __align__(16) ChunkSlots {
  int32_t cnt;
  float mx;
  int2 e[kSlotE];  // (key index, logit bits)
};
static_assert(sizeof(ChunkSlots) == 64, "four 16-byte pieces");

// What k_qk_select leaves for the next kernel: the kept list in the chunk's segment
// (the separate stages), chunk records of eq. (7) with the value rows gathered (the
// early gather), or slot records whose value rows the combining kernel gathers (the
// late gather).
enum SelectOut { kOutList = 0, kOutRecords = 1, kOutSlots = 2 };

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
  float* part;             // [B*h_q, DV/16, nch, 16] chunk records: sum w*v, 16 columns per slice;
                           // the late gather's slot records [B*h_q, nch] ChunkSlots use the same region
  unsigned* hist;          // [8, B*h_q, 256] top-digit histogram copies (zero between calls)
  unsigned* cand_cnt;      // [B*h_q, nsel] threshold candidates of each slice of cand_slice logits
  const int32_t* ptab;     // paged caches: [B, ptab_stride] page ids (the kernels' PAGED form)
  long long lpad;
  int h_q, h_k, h_v, g_k, g_v, htiles, l_max, nch, N;  // g_k = h_q/h_k, g_v = h_q/h_v
  int max_l_kv;            // host bound of l_kv[]; larger device values are clamped
  int hsplit;              // blocks sharing one chunk in k_qk_select (heads split among them)
  float scale;
  int nsel;                // candidate slices per row (cand_cnt's row stride)
  int cand_slice;          // logits per candidate slice: the chunk width (cand_chunk) or kSelSlice
  int cand_chunk;          // 1: k_scores_hist collects each chunk's candidates in the bin of the
                           // previous threshold; 0: k_cand_collect collects them
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
// Kept entries of one chunk, per head of the tile, staged in LDS in increasing key
// order: off[h][e] is the offset inside the chunk of head h's e-th kept key; its logit
// is val[h][off] (indexed by key offset). Plus the count and the largest kept logit
// (as an order key) per head; with paged caches also the pages of the chunk's tokens.
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
// s_part: LDS scratch of the block, [kBlock / 16][D + 1] floats.
template <typename T, int D, int CH, bool PAGED>
__device__ __forceinline__ void chunk_records(const KeptLds<CH>& kl, const StreamArgs& a, int b, int j0, int nh,
                                              int c, int hs, int hsplit, float (*s_part)[D + 1]) {
  constexpr int EPL = Unpack<T>::kN;                    // columns per 16-byte piece
  constexpr int PIECES = D / EPL;                       // pieces per value row
  constexpr int RPG = PIECES >= 16 ? 1 : 16 / PIECES;  // rows one group load covers
  constexpr int PPL = PIECES >= 16 ? PIECES / 16 : 1;   // pieces per lane per row
  constexpr int U = 4;                                  // loads in flight per lane
  constexpr int NG = kBlock / 16;                       // groups of 16 lanes
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
        w[u] = expf(kl.val[h][off] - m);
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
// OUT (SelectOut) chooses what is left for the next kernel: the kept list only, also
// the chunk records of eq. (7) (chunk_records, the early gather), or slot records
// (ChunkSlots, the late gather: the first kSlotE entries in the record, the rest in
// the segment).
// When hsplit > 1, hsplit blocks share each chunk: block hs compares and gathers only
// the heads h of the tile with h mod hsplit == hs (every block computes all the
// tile's logits; its duplicate key reads hit the cache).
// DK and DV are the key and value head dimensions.
// grid = (nch, h_k * htiles * hsplit, B), block = 256.
template <typename T, int DK, int DV, int MODE, int OUT, bool PAGED, int W>
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
  } else if constexpr (MODE == kFromScores) {
    // the stored logits lie in the workspace (rows padded to whole chunks): loaded
    // before l_kv arrives, at any batch size; keys past l_kv are masked below
    const float* srow = a.scores + (long long)(row0 + (live ? hh : 0)) * a.lpad;
#pragma unroll
    for (int t = 0; t < TPW; ++t) sc[t] = *reinterpret_cast<const floatx4*>(srow + wbase + 16 * t + 4 * kq);
  }
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (base >= L) return;

  __shared__ KeptLds<CH> kl;
  // the kept bitmap of each head (bit i of word w: chunk offset 32 w + i), dead once the
  // kept lists are built; the value gather's partial sums reuse its LDS
  constexpr int kWords = CH / 32;
  __shared__ union {
    unsigned bits[16][kWords];
    float part[kBlock / 16][DV + 1];
  } s_bp;
  if (tid < 16) {
    kl.cnt[tid] = 0;
    kl.mx[tid] = 0u;
  }
  for (int e = tid; e < 16 * kWords; e += kBlock) (&s_bp.bits[0][0])[e] = 0u;
  if constexpr (PAGED && OUT == kOutRecords) stage_pages<CH>(kl, a, b, base);
  const float tau_l = live ? a.tau[row0 + hh] : 0.f;
  if constexpr (MODE == kFromKeys) {
    qk.load_q(qbase + (size_t)row0 * DK, nh, lane);
    score_tiles<T, DK, TPW>(sc, qk, kh, wbase, L, lane, scale);
  }
  __syncthreads();

  // This lane's kept entries as a bit mask (bit 4t+r: key wbase+16t+4kq+r). They are
  // marked in the head's bitmap (order-free atomic ORs) and their logits stored at
  // their key offsets; after the barrier the kept list is read off the bitmap in key
  // order, so the lists, and every sum over them, are the same on every run.
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
    const int wo = wbase - base;  // offset of the wave's keys in the chunk (a multiple of 32)
    float vmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const unsigned nib = (pm >> (4 * t)) & 15u;
      if (nib) {
        const int pos = wo + 16 * t + 4 * kq;  // 4 consecutive offsets inside one word
        atomicOr(&s_bp.bits[hh][pos >> 5], nib << (pos & 31));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((nib >> r) & 1u) {
            kl.val[hh][pos + r] = sc[t][r];
            vmax = fmaxf(vmax, sc[t][r]);
          }
      }
    }
    atomicAdd(&kl.cnt[hh], __popc(pm));
    atomicMax(&kl.mx[hh], order_key(vmax));
  }
  __syncthreads();
  // 16 threads per head, thread s16 takes the BPT bitmap bits from offset s16 BPT on:
  // its kept keys follow those of the threads before it (a prefix over the row of 16
  // lanes). The list goes to LDS for the value gather first; its copy in memory is
  // written after the gather has issued its loads.
  constexpr int BPT = CH / 16;  // 8, 16 or 32 bits, inside one word
  static_assert(BPT == 8 || BPT == 16 || BPT == 32, "a thread's bits lie in one word");
  const int lh = tid >> 4, s16 = tid & 15;
  const int boff = s16 * BPT;
  const unsigned wb =
      lh < nh ? (s_bp.bits[lh][boff >> 5] >> (boff & 31)) & (BPT == 32 ? ~0u : (1u << BPT) - 1u) : 0u;
  const int first = row_incl_scan(__popc(wb)) - __popc(wb);
  if constexpr (OUT == kOutRecords) {
    int at = first;
    for (unsigned m = wb; m; m &= m - 1u) kl.off[lh][at++] = (uint16_t)(boff + __builtin_ctz(m));
    __syncthreads();
  }
  ChunkSlots* const slots = reinterpret_cast<ChunkSlots*>(a.part);
  if (tid < nh && (hsplit == 1 || tid % hsplit == hs)) {
    const long long o = (long long)(row0 + tid) * a.nch + c;
    const int2 h = make_int2(kl.cnt[tid], __float_as_int(order_key_to_f32(kl.mx[tid])));
    if constexpr (OUT == kOutSlots) *reinterpret_cast<int2*>(slots + o) = h;
    else *reinterpret_cast<int2*>(a.chunk_hdr + o) = h;
  }
  if constexpr (OUT == kOutRecords) chunk_records<T, DV, CH, PAGED>(kl, a, b, j0, nh, c, hs, hsplit, s_bp.part);
  if (wb) {
    const long long seg = (long long)(row0 + lh) * a.lpad + base;
    ChunkSlots* const rec = slots + (long long)(row0 + lh) * a.nch + c;
    int at = first;
    for (unsigned m = wb; m; m &= m - 1u) {
      const int off = boff + __builtin_ctz(m);
      if (OUT == kOutSlots && at < kSlotE) {
        rec->e[at] = make_int2(base + off, __float_as_int(kl.val[lh][off]));
      } else {
        a.surv_idx[seg + at] = base + off;
        a.surv_val[seg + at] = kl.val[lh][off];
      }
      ++at;
    }
  }
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
  __shared__ float s_part[kBlock / 16][DV + 1];
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
      const int off = a.surv_idx[at] - base;
      kl.off[h][i] = (uint16_t)off;
      kl.val[h][off] = a.surv_val[at];
    }
  }
  __syncthreads();
  chunk_records<T, DV, CH, PAGED>(kl, a, b, j0, nh, c, 0, 1, s_part);
}

// ----------------------------------------------------------------------------
// The refresh's guess of where the new threshold lies: the order keys within
// kGuessHalf of the key of the threshold passed in, [lo, hi] (a quarter octave either
// way for logits of either sign: a threshold that moved by less than about 19% since
// the last refresh lies inside, wherever it lies on the float scale). Empty (lo > hi,
// false) for a threshold that is not finite.
constexpr uint32_t kGuessHalf = 1u << 21;
__device__ __forceinline__ bool guess_window(float tprev, uint32_t& lo, uint32_t& hi) {
  if (!__builtin_isfinite(tprev)) {
    lo = 1u;
    hi = 0u;
    return false;
  }
  const uint32_t k = order_key(tprev);
  lo = k > kGuessHalf ? k - kGuessHalf : 0u;
  hi = k < 0xffffffffu - kGuessHalf ? k + kGuessHalf : 0xffffffffu;
  return true;
}

// ----------------------------------------------------------------------------
// Refresh, pass 1: logits of every cached key stored as fp32, plus a histogram of
// the top 8 bits of their order keys per query head, accumulated into copy
// (chunk mod kHistCopies) of a.hist: the logits of a row fall into a few bins, and
// the copies spread the device atomics of the row's blocks over more addresses.
// With a.cand_chunk, also the threshold candidates on a guess: the logits inside the
// window around the row's previous threshold (guess_window; the N-th largest logit
// of a decoding sequence moves little between refreshes) go to the chunk's segment
// of the row's kept-logit buffer; cand_cnt[row, chunk] = their number plus, in the
// upper 16 bits, the number of logits above the window. k_select_finish checks the
// guess with those counts.
// SPEC (one sequence) issues the key loads before l_kv arrives, for rows below
// max_l_kv (inside the cache); keys past l_kv are masked.
// D is the key head dimension. grid = (nch, h_k * htiles, B), block = 256.
constexpr int kHistCopies = 8;

template <typename T, int D, bool PAGED, int W, bool SPEC>
__global__ __launch_bounds__(kBlock) void k_scores_hist(const StreamArgs a) {
  constexpr int TPW = StreamCfg<T, D, W>::kTPW;
  constexpr int CH = StreamCfg<T, D, W>::kChunk;
  const int c = blockIdx.x, gy = blockIdx.y, b = blockIdx.z;
  const int base = c * CH;
  const int g = gy / a.htiles, ht = gy - g * a.htiles;
  const int j0 = g * a.g_k + ht * 16;
  const int nh = min(16, a.g_k - ht * 16);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * a.h_q + j0;
  const int wbase = base + wv * 16 * TPW;
  const auto kh = key_rows<T, D, PAGED>(a, b, g);
  QK<T, D> qk;
  floatx4 sc[TPW];
  if constexpr (SPEC) {
    qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, nh, lane);
    score_tiles<T, D, TPW>(sc, qk, kh, wbase, a.max_l_kv, lane, a.scale);
  }
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (base >= L) return;

  __shared__ unsigned s_hist[16 * 256];
  __shared__ float s_cv[16][CH];  // candidates of the chunk per head (cand_chunk)
  __shared__ int s_cc[16], s_ac[16];
  for (int e = tid; e < 16 * 256; e += kBlock) s_hist[e] = 0u;
  if (tid < 16) {
    s_cc[tid] = 0;
    s_ac[tid] = 0;
  }

  const bool live = hh < nh;
  uint32_t wlo = 1u, whi = 0u;  // the guessed window (empty: none)
  const bool wok = a.cand_chunk && a.tau && live && guess_window(a.tau[row0 + hh], wlo, whi);
  if constexpr (!SPEC) {
    qk.load_q(reinterpret_cast<const T*>(a.q) + (size_t)row0 * D, nh, lane);
    score_tiles<T, D, TPW>(sc, qk, kh, wbase, L, lane, a.scale);
  }
  __syncthreads();

  if (live) {
    float* srow = a.scores + (long long)(row0 + hh) * a.lpad;
    int above = 0;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      floatx4 v = sc[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = wbase + 16 * t + 4 * kq + r;
        if (key < L) {
          const uint32_t ok = order_key(v[r]);
          atomicAdd(&s_hist[hh * 256 + (ok >> 24)], 1u);
          if (ok >= wlo && ok <= whi) s_cv[hh][atomicAdd(&s_cc[hh], 1)] = v[r];
          else if (wok && ok > whi) ++above;
        } else {
          v[r] = -INFINITY;
        }
      }
      *reinterpret_cast<floatx4*>(srow + wbase + 16 * t + 4 * kq) = v;
    }
    if (above) atomicAdd(&s_ac[hh], above);
  }
  __syncthreads();
  for (int e = tid; e < nh * 256; e += kBlock) {
    const unsigned h = s_hist[e];
    if (h) {
      const long long rows = (long long)gridDim.z * a.h_q;
      atomicAdd(&a.hist[((c % kHistCopies) * rows + row0 + e / 256) * 256 + (e & 255)], h);
    }
  }
  if (a.cand_chunk) {  // 16 threads per head
    const int h = tid >> 4, sub = tid & 15;
    if (h < nh) {
      const int n = s_cc[h];
      const long long r = row0 + h;
      if (sub == 0) a.cand_cnt[r * a.nsel + c] = (unsigned)n | ((unsigned)s_ac[h] << 16);
      float* dst = a.surv_val + r * a.lpad + (long long)c * CH;
      for (int i = sub; i < n; i += 16) dst[i] = s_cv[h][i];
    }
  }
}

// ----------------------------------------------------------------------------
// Refresh, pass 2 for rows of more than kMaxSel chunks (shorter rows get their
// candidates from k_scores_hist): candidates for the exact threshold. The sum of the
// row's histogram copies gives the 8-bit bin that holds its N-th largest logit; each block
// copies the logits of its slice that fall in that bin to the slice's own segment of
// the row's kept-logit buffer (free at this point of a refresh step; a slice's
// candidates fit in the slice's kSelSlice places) and their number to
// cand_cnt[row, slice]. No block waits on another and there are no device atomics.
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
  __shared__ int s_cc;

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
  if (tid == 0) a.cand_cnt[row * a.nsel + p] = (unsigned)cnt;
  for (int i = tid; i < cnt; i += kBlock) a.surv_val[rbase + lo + i] = s_cand[i];
}

// Refresh, pass 3: the N-th largest logit (counting repeats) resolved on the
// candidates. The slices' candidate counts give each slice's place in the row's
// candidate list (a block scan); a group of threads per slice copies the candidates
// into LDS, or, past kCandLds of them, first finds the next digit on the candidates in
// place and stages only that digit's; a radix select resolves the remaining bits. The
// counts, the first round of candidate loads, the histogram and the threshold passed
// in are all requested at once. When k_scores_hist guessed a window (cand_chunk) that
// does not hold the N-th largest, the block collects the logits of its histogram bin
// from the row's stored logits instead. Writes tau (-inf when N >= l_kv, unchanged
// when l_kv == 0) and returns the row's histogram copies to zero.
// grid = (h_q, B), block = 1024.
constexpr int kMaxSel = 4096;  // candidate slices of a row at most

__global__ __launch_bounds__(kRowThreads) void k_select_finish(const StreamArgs a, float* tau_out) {
  constexpr int NT = kRowThreads;
  constexpr int PER = kMaxSel / NT;
  constexpr int kQ = 2;  // 16-byte candidate loads of a thread in flight per round
  const int j = blockIdx.x, b = blockIdx.y;
  const long long rows = (long long)gridDim.y * a.h_q;
  const long long row = (long long)b * a.h_q + j;
  const int N = a.N;
  const int tid = threadIdx.x;

  __shared__ unsigned s_hist[256];
  __shared__ int s_itmp[NT / kWave];
  __shared__ int s_itmp2[2 * (NT / kWave)];
  __shared__ unsigned s_res[2];
  __shared__ unsigned s_stage;
  __shared__ float s_cand[kCandLds];
  __shared__ int s_off[kMaxSel + 1];

  // The first round of loads is addressed from the host bound max_l_kv, so that none
  // waits for l_kv: the slices' candidate counts, the first 4 kQ candidates of each
  // thread's slice (a slice's candidates never outnumber its logits, so these stay
  // inside the row), the row's histogram copies and the threshold passed in (the
  // refresh callers always pass one). Slices past the row's own length are dropped
  // once it is known.
  const int S = a.cand_slice;
  const int nsl_max = (a.max_l_kv + S - 1) / S;
  // the candidate copies: one group of NT / nsl_max threads per slice (one thread per
  // slice, taking every NT-th, when there are more slices than threads)
  const int tps = nsl_max <= NT ? NT / nsl_max : 1;
  const int gsl = tid / tps, sub = tid - gsl * tps, gstep = NT / tps;
  const float* seg = a.surv_val + row * a.lpad;
  int c[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int sl = tid * PER + u;
    c[u] = sl < nsl_max ? (int)a.cand_cnt[row * a.nsel + sl] : 0;
  }
  // thread sub of a slice's group takes the candidates 4 (sub + u tps) .. +3, u < kQ
  // (16-byte loads: a slice segment starts 16-byte aligned and holds a multiple of 4
  // places, and a row's padded length covers its logits rounded up to 4)
  float4 pre[kQ];
  {
    const int cap = gsl < nsl_max ? min(S, a.max_l_kv - gsl * S) : 0;
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const int i = 4 * (sub + u * tps);
      pre[u] = i < cap ? *reinterpret_cast<const float4*>(seg + (long long)gsl * S + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // (relaxed atomic loads: plain vector loads that the compiler neither turns into
  // scalar loads nor sinks past the l_kv check to their first use)
  unsigned hv[kHistCopies] = {};
  if (tid < 256) {
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp)
      hv[cp] = __hip_atomic_load(a.hist + (cp * rows + row) * 256 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  const float tprev = __hip_atomic_load(a.tau + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (L <= 0) return;  // no block added to this row's histograms
  const int nsl = (L + S - 1) / S;  // slices holding candidates
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (tid * PER + u >= nsl) c[u] = 0;
  if (tid < 256) {  // the row's histogram, and its copies back to zero
    unsigned h = 0u;
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) {
      h += hv[cp];
      a.hist[(cp * rows + row) * 256 + tid] = 0u;
    }
    s_hist[tid] = h;
  }
  if (N >= L) {
    if (tid == 0) tau_out[row] = -INFINITY;
    return;
  }
  // a slice's count word: its candidates, and with cand_chunk in the upper 16 bits the
  // logits above the guessed window
  int above = 0;
  if (a.cand_chunk) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      above += (int)((unsigned)c[u] >> 16);
      c[u] &= 0xffff;
    }
  }
  // places of the slices in the candidate list (thread t holds slices t*PER ..), the
  // row's candidates C and its logits above the window A
  int mine = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) mine += c[u];
  int C, A;
  int off = block_excl_scan2<NT>(mine, above, s_itmp2, C, A).x;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int sl = tid * PER + u;
    if (sl < nsl) s_off[sl] = off;
    off += c[u];
  }
  if (tid == 0) s_off[nsl] = C;
  __syncthreads();
  digit_of_kth_largest<NT>(s_hist, (unsigned)N, s_itmp, s_res);
  const unsigned d1 = s_res[0], k1 = s_res[1];
  const unsigned c1 = s_hist[d1];  // the row's logits in bin d1
  // Where the select starts: the candidates of top byte d1 (the bin of the N-th
  // largest), resolving the lower 24 bits. Candidates per slice are that bin: rank k1.
  // Candidates in the guessed window: the guess holds when the window holds the N-th
  // largest (A < N <= A + C). The window then spans d1 and at most one neighbour
  // byte. If it reaches above d1, all of bin d1 lies below its top: every logit
  // above the N-th largest in bin d1 is in the window, rank k1. Otherwise the
  // logits above the window are exactly those above the window's part of bin d1:
  // rank N - A.
  uint32_t lo = 1u, hi = 0u;
  const bool wok = a.cand_chunk && guess_window(tprev, lo, hi);
  const bool hit = !a.cand_chunk || (wok && A < N && N <= A + C);
  const uint32_t p0 = d1 << 24, m0 = 0xff000000u;
  const unsigned k0 = (a.cand_chunk && (hi >> 24) == d1) ? (unsigned)(N - A) : k1;
  float* gcand = reinterpret_cast<float*>(a.surv_idx) + row * a.lpad;  // free at this point
  // f(place, logit) for every candidate of the slices, kQ 16-byte loads of a thread
  // at once (the places past a slice's count that they cover are skipped)
  auto each_cand = [&](auto&& f) {
    for (int sl = gsl; sl < nsl; sl += gstep) {
      const int o = s_off[sl], n = s_off[sl + 1] - o;
      const float* src = seg + (long long)sl * S;
      for (int q0 = sub; 4 * q0 < n; q0 += kQ * tps) {
        const bool first = sl == gsl && q0 == sub;
        float4 v[kQ];
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
          const int i = 4 * (q0 + u * tps);
          v[u] = first ? pre[u] : (i < n ? *reinterpret_cast<const float4*>(src + i) : make_float4(0.f, 0.f, 0.f, 0.f));
        }
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
          const int i = 4 * (q0 + u * tps);
          const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i + e < n) f(o + i + e, x4[e]);
        }
      }
    }
  };
  uint32_t key;
  if (!hit) {
    // the guess missed: the bin's logits, c1 of them, from the row's stored logits
    if (tid == 0) s_stage = 0u;
    __syncthreads();
    const bool in_lds = c1 <= (unsigned)kCandLds;
    const float* lg = a.scores + row * a.lpad;
    constexpr int V4 = 16;  // 16-byte loads per thread per round (256 KiB per block)
    for (int i0 = 4 * tid; i0 < L; i0 += 4 * NT * V4) {
      float4 v[V4];
#pragma unroll
      for (int u = 0; u < V4; ++u) {
        const int i = i0 + u * 4 * NT;  // a multiple of 4 below L: inside the padded row
        v[u] = i < L ? *reinterpret_cast<const float4*>(lg + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < V4; ++u) {
        const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (i0 + u * 4 * NT + e < L && (order_key(x4[e]) >> 24) == d1) {
            const unsigned at = atomicAdd(&s_stage, 1u);
            if (in_lds) s_cand[at] = x4[e];
            else gcand[at] = x4[e];
          }
        }
      }
    }
    __syncthreads();
    key = in_lds ? radix_select_block<NT>(s_cand, (long long)c1, d1 << 24, 0xff000000u, 16, k1, s_hist, s_itmp, s_res)
                 : radix_select_block<NT>(gcand, (long long)c1, d1 << 24, 0xff000000u, 16, k1, s_hist, s_itmp, s_res);
  } else if (C <= kCandLds) {
    each_cand([&](int i, float x) { s_cand[i] = x; });
    __syncthreads();
    key = radix_select_block<NT>(s_cand, (long long)C, p0, m0, 16, k0, s_hist, s_itmp, s_res);
  } else {
    // Too many for LDS: the next digit is found on the candidates where they lie, and
    // only that digit's candidates are staged (in LDS, or past kCandLds of them, as
    // with many equal logits, in the row's kept-index buffer) for the rest.
    __syncthreads();  // every thread has read s_hist[d1]
    if (tid < 256) s_hist[tid] = 0u;
    __syncthreads();
    each_cand([&](int, float x) {
      const uint32_t ok = order_key(x);
      if ((ok & m0) == p0) atomicAdd(&s_hist[(ok >> 16) & 255u], 1u);
    });
    __syncthreads();
    digit_of_kth_largest<NT>(s_hist, k0, s_itmp, s_res);
    const unsigned d2 = s_res[0], k2 = s_res[1];
    const unsigned c2 = s_hist[d2];
    const uint32_t p2 = p0 | (d2 << 16), m2 = m0 | (255u << 16);
    if (tid == 0) s_stage = 0u;
    __syncthreads();  // every thread has read s_res and s_hist; the counter is zero
    const bool in_lds = c2 <= (unsigned)kCandLds;
    each_cand([&](int, float x) {
      if ((order_key(x) & m2) == p2) {
        const unsigned at = atomicAdd(&s_stage, 1u);
        if (in_lds) s_cand[at] = x;
        else gcand[at] = x;
      }
    });
    __syncthreads();
    key = in_lds ? radix_select_block<NT>(s_cand, (long long)c2, p2, m2, 8, k2, s_hist, s_itmp, s_res)
                 : radix_select_block<NT>(gcand, (long long)c2, p2, m2, 8, k2, s_hist, s_itmp, s_res);
  }
  if (tid == 0) tau_out[row] = order_key_to_f32(key);
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
  int rows;               // B * h_q
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
  __shared__ int s_scan[NW];

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
    // the kept entries of these NT keys in key order (a block prefix sum of the flags)
    const int i = base + tid;
    const float v = i < L ? srow[i] : 0.f;
    const bool keep = i < L && v >= tau;
    int n;
    const int slot = block_excl_scan<NT>(keep ? 1 : 0, s_scan, n);
    if (keep) {
      s_list_i[slot] = i;
      s_list_v[slot] = v;
    }
    __syncthreads();
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

// The late value gather: eq. (7) over the kept entries of one row (b, j), from the
// slot records of k_qk_select<kOutSlots>. M = the row's largest kept logit (the
// maximum of the records' maxima), O = sum_i w_i V[v(j), i, :] / sum_i w_i with
// w_i = exp(A_i - M), summed in a fixed order. Each block takes one 16-byte piece of
// the value rows (EPL output columns) of one row; the P = DV * sizeof(T) / 16 blocks
// of a row are placed on one XCD (blocks are dealt to the 8 XCDs in turn), so the
// row's records and value lines are fetched into one L2.
//   - Group g of 4 threads takes records g KR .. g KR + KR - 1, thread p of the group
//     piece p of each: one round of 16-byte loads, issued together with l_kv.
//   - The group lists its records' inline entries in key order in its own LDS rows
//     (written and read by the group's wave only, so no block barrier); lane p of the
//     group loads the block's piece of the value rows of entries p, p + 4, ...
//   - While those loads are in flight, one block pass finds M and each group's place
//     in the row's kept list (the export of the kept indices, in key order, by the
//     row's first block).
//   - Entries past a record's kSlotE inline ones are read from the chunk's segment of
//     the kept list afterwards (a record keeps that many only at dense selections).
// A row that kept nothing is recomputed exactly by its first block (the forced
// refresh). DK and DV are the key and value head dimensions.
// grid = 8 ceil(B h_q / 8) P blocks, block = 256; a row has at most kPvGroupRecs * 64 chunks.
constexpr int kPvGroupRecs = 8;  // slot records per group of 4 threads
constexpr int kPvLoads = 8;      // value rows in flight per lane (32 per group)

// x of the first lane of each quad of lanes, in all four (DPP quad_perm [0,0,0,0]).
__device__ __forceinline__ int quad_first(int x) { return __builtin_amdgcn_update_dpp(0, x, 0x00, 0xf, 0xf, false); }

template <typename T, int DK, int DV, bool PAGED, int W>
__global__ __launch_bounds__(kBlock) void k_sparse_pv(const GatherArgs a) {
  constexpr int CH = StreamCfg<T, DK, W>::kChunk;
  constexpr int EPL = Unpack<T>::kN;  // columns per 16-byte piece
  constexpr int P = DV / EPL;         // blocks per row
  constexpr int KR = kPvGroupRecs;
  constexpr int NGR = kBlock / 4;     // groups of 4 threads
  constexpr int U = kPvLoads;
  constexpr int GE = KR * kSlotE;     // inline entries of a group's records
  const StreamArgs& sa = a.s;
  // block -> (row, piece): XCD x = id mod 8 holds rows x, x + 8, ..., P blocks each
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const long long row = xcd + 8LL * (slot / P);
  const int cp = slot - (slot / P) * P;
  if (row >= a.rows) return;
  const int b = (int)(row / sa.h_q), j = (int)(row - (long long)b * sa.h_q);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int grp = tid >> 2, pc = tid & 3;
  const int nch = sa.nch;

  __shared__ int s_itmp[kWaves];
  __shared__ float s_ftmp[kWaves];
  __shared__ int2 s_ent[NGR][GE];
  __shared__ float s_red[kWaves][DV];
  __shared__ float s_z[kWaves];

  // records past the row's last chunk load the last one (never used): no branches, so
  // every load of the round is in flight at once
  const int4* rec = reinterpret_cast<const int4*>(reinterpret_cast<const ChunkSlots*>(sa.part) + row * nch) + pc;
  int4 x[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) x[k] = rec[4 * min(grp * KR + k, nch - 1)];
  const int L = min(sa.l_kv[b], sa.max_l_kv);
  if (L <= 0) {
    if (tid < EPL) store_out<DV>(a, row, cp * EPL + tid, 0.f);
    if (cp == 0 && tid == 0) {
      if (a.sel_count) a.sel_count[row] = 0;
      if (a.flags) a.flags[row] = 0;
    }
    return;
  }
  const int nch_b = (L + CH - 1) / CH;
  int cnt[KR];
  float m = -INFINITY;
  int gsum = 0, gin = 0;
  const int ea = 2 * pc - 1, eb = 2 * pc;  // the entries in this thread's piece (none at -1)
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    // the count and the maximum are in piece 0: the group's first thread has them
    const int n0 = quad_first(x[k].x);
    const float m0 = __int_as_float(quad_first(x[k].y));
    cnt[k] = grp * KR + k < nch_b ? n0 : 0;
    if (cnt[k] > 0) m = fmaxf(m, m0);
    gsum += cnt[k];
    const int ni = min(cnt[k], kSlotE);
    if (ea >= 0 && ea < ni) s_ent[grp][gin + ea] = make_int2(x[k].x, x[k].y);
    if (eb < ni) s_ent[grp][gin + eb] = make_int2(x[k].z, x[k].w);
    gin += ni;
  }
  // the group's LDS rows are written and read by its own wave: the wave executes its
  // LDS instructions in order, so only the compiler must keep them in order
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const auto vr = value_rows<T, DV, PAGED>(sa, b, j / sa.g_v);
  const int col0 = cp * EPL;
  uint4 xv[U];
  float lg[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = pc + 4 * u;
    xv[u] = make_uint4(0, 0, 0, 0);
    lg[u] = -INFINITY;
    if (e < gin) {
      const int2 en = s_ent[grp][e];
      xv[u] = ld16(vr.row(en.x) + col0);
      lg[u] = __int_as_float(en.y);
    }
  }

  float M;
  int total;
  const int gbase = quad_first(block_max_excl_scan(m, pc == 0 ? gsum : 0, s_ftmp, s_itmp, M, total));
  if (total == 0) {
    if (cp == 0) exact_row<T, DK, DV, kBlock, PAGED>(a, b, j, L, true, s_red, s_z);
    return;
  }
  const long long sbase = row * sa.lpad;
  if (cp == 0 && a.sel_idx) {
    // kept indices in key order: entry e of record k at gbase + (counts before k) + e
    int32_t* const exp_idx = a.sel_idx + row * a.sel_cap;
    int p = gbase;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const int n = cnt[k], ni = min(n, kSlotE);
      if (ea >= 0 && ea < ni && p + ea < a.sel_cap) exp_idx[p + ea] = x[k].x;
      if (eb < ni && p + eb < a.sel_cap) exp_idx[p + eb] = x[k].z;
      const long long cb = sbase + (long long)(grp * KR + k) * CH;
      for (int e = kSlotE + pc; e < n && p + e < a.sel_cap; e += 4) exp_idx[p + e] = sa.surv_idx[cb + e];
      p += n;
    }
  }

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
  auto add = [&](const uint4& v, float logit) {
    const float w = expf(logit - M);  // 0 for an unused slot (logit -inf)
    float f[EPL];
    Unpack<T>::run(v, f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += w * f[e];
    z += w;
  };
#pragma unroll
  for (int u = 0; u < U; ++u) add(xv[u], lg[u]);
  // a group with more than 4 U inline entries
  for (int u0 = 4 * U; u0 < gin; u0 += 4 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = u0 + pc + 4 * u;
      xv[u] = make_uint4(0, 0, 0, 0);
      lg[u] = -INFINITY;
      if (e < gin) {
        const int2 en = s_ent[grp][e];
        xv[u] = ld16(vr.row(en.x) + col0);
        lg[u] = __int_as_float(en.y);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) add(xv[u], lg[u]);
  }
  // entries past the inline ones, from the chunks' segments of the kept list: lane p of
  // the group takes entries kSlotE + p, kSlotE + p + 4, ...
#pragma unroll 1
  for (int k = 0; k < KR; ++k) {
    const int n = cnt[k];
    const long long cb = sbase + (long long)(grp * KR + k) * CH;
    for (int e0 = kSlotE + pc; e0 < n; e0 += 4 * U) {
      int idx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + 4 * u;
        idx[u] = e < n ? sa.surv_idx[cb + e] : -1;
        lg[u] = e < n ? sa.surv_val[cb + e] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) xv[u] = idx[u] >= 0 ? ld16(vr.row(idx[u]) + col0) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) add(xv[u], lg[u]);
    }
  }
  // every lane holds sums over its own entries: the wave sums, then the waves
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = wave_sum(acc[e]);
  z = wave_sum(z);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_red[wv][e] = acc[e];
    s_z[wv] = z;
  }
  __syncthreads();
  if (tid < EPL) {
    float o = 0.f, zz = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      o += s_red[w][tid];
      zz += s_z[w];
    }
    store_out<DV>(a, row, cp * EPL + tid, o / zz);
  }
  if (cp == 0 && tid == 0) {
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
  int rows;                                   // B * h_q
};

// DK and DV are the key and value head dimensions; TPW tiles of 16 keys per wave.
// grid = (nchd, h_v, B), block = 256. Each block takes one chunk of 4 * 16 * TPW keys
// and one value head v: the logits of its g query heads against their key head (h_k
// divides h_v, so the g heads share one; MFMA), the chunk's softmax numerator
// relative to the chunk maximum, and its product with the chunk's rows of value head
// v (VALU, GH >= g heads). Every key and value load of a wave is issued at once, so a
// block waits for one memory round trip. SPEC (one sequence): the loads are issued
// before l_kv arrives, for rows up to max_l_kv - 1 (inside the caches); logits of rows
// at or past l_kv are masked and their value registers zeroed before use.
//
// P.V on the matrix cores (bf16 caches, d_v = 128 or 64, an even number of tiles): lane
// (x, kq) = (lane & 15, lane >> 4) loads row 16t + 4kq + r of tile t at columns
// c x .. c x + c - 1, c = d_v / 16 (8 or 4). The score tile leaves p(head x, key
// 16t + 4kq + r) in that same lane, so over a pair of tiles a lane holds, for the same
// 8 keys, the 8 weights of head x and 8 values of each of its c columns: exactly the
// K-slice of a 16x16x32 bf16 MFMA's A operand (rows = heads) and, taking element i of
// each value load, of its B operand (columns c n + i for n = 0..15). The fp32 weights
// enter as three bf16 terms (each the rounding of what the previous ones leave, so
// their sum is the weight to within 2^-24 of it); values are exact in bf16 and
// products accumulate in fp32.
template <typename T, int DK, int DV, int GH, bool PAGED, int TPW, bool SPEC>
__global__ __launch_bounds__(kBlock) void k_dense_partial(const DenseArgs a) {
  constexpr bool kMfmaPV = std::is_same<T, bf16_t>::value && (DV == 128 || DV == 64) && TPW % 2 == 0;
  constexpr int CHD = 16 * TPW * kWaves;
  constexpr int EPL = Unpack<T>::kN;
  constexpr int G = DV / EPL;                        // lanes per value row
  // MFMA form: 4 value rows per lane and tile, DV / 16 columns each (a 16- or 8-byte
  // load); VALU form: 16-byte loads spread over the tile
  constexpr int NCOL = DV / 16;
  using VLoad = typename std::conditional<kMfmaPV && DV == 64, uint2, uint4>::type;
  constexpr int VL = kMfmaPV ? 4 : (16 * DV) / (EPL * kWave);  // value loads per lane per tile
  constexpr int KL = QK<T, DK>::kLoads;
  const T* const kbase = reinterpret_cast<const T*>(a.k);
  const T* const vbase = reinterpret_cast<const T*>(a.v);
  const T* const qbase = reinterpret_cast<const T*>(a.q);
  const int h_k = a.h_k, h_v = a.h_v, l_max = a.l_max, gq = a.g, h_q = a.h_q, max_l_kv = a.max_l_kv;
  const float scale = a.scale;
  __builtin_amdgcn_sched_barrier(0);
  const int c = blockIdx.x, vg = blockIdx.y, b = blockIdx.z;
  const int kg = h_k == h_v ? vg : vg / (h_v / h_k);  // key head of this value head's query heads
  const int base = c * CHD;
  int L = max_l_kv;  // rows the loads may touch (SPEC), else the sequence's length
  if constexpr (!SPEC) {
    L = min(a.l_kv[b], max_l_kv);
    if (base >= L) return;
  }
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int hh = lane & 15, kq = lane >> 4;
  const int row0 = b * h_q + vg * gq;

  __shared__ float s_p[kMfmaPV ? 1 : kWaves][kMfmaPV ? 1 : TPW][16][GH];
  __shared__ float s_m[kWaves][GH], s_z[kWaves][GH];
  __shared__ __align__(16) float s_o[kWaves][GH][DV];

  const CacheRows<T, DK, PAGED> kh(kbase, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, kg, h_k, l_max);
  const CacheRows<T, DV, PAGED> vh(vbase, a.ptab, a.ptab_stride, a.page_shift, a.num_pages, b, vg, h_v, l_max);
  const int wbase = base + wv * 16 * TPW;

  QK<T, DK> qk;
  qk.load_q(qbase + (size_t)row0 * DK, gq, lane);
  // every key and value load of the wave, rows past L clamped to L - 1 (in bounds;
  // their logits are masked); a clamped tile lies inside one page
  uint4 kb[TPW][KL];
  VLoad vb[TPW][VL];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int t0 = min(wbase + 16 * t, (L - 1) & ~15);
    if constexpr (PAGED) {
      const int key = min(t0 + (lane & 15), L - 1);
      QK<T, DK>::load_k(kb[t], kh.tile(t0) + (size_t)(key - t0) * DK, lane);
    } else {
      QK<T, DK>::load_k(kb[t], kh.row(min(wbase + 16 * t + (lane & 15), L - 1)), lane);
    }
  }
  // value row of load r of tile t (the MFMA form: row 4kq + r of the tile, columns
  // NCOL hh ..; the VALU form: flat element r*64 + lane of the tile's 16 x G grid)
  auto vrow = [&](int t, int r) {
    return wbase + 16 * t + (kMfmaPV ? 4 * kq + r : (r * kWave + lane) / G);
  };
  const int vcol = kMfmaPV ? NCOL * hh : ((lane % G) * EPL);
  auto ldv = [](const T* p) { return *reinterpret_cast<const VLoad*>(p); };
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int t0 = min(wbase + 16 * t, (L - 1) & ~15);
    const T* vt = PAGED ? vh.tile(t0) : vh.row(0);
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      if constexpr (PAGED) {
        const int key = min(t0 + (vrow(t, r) - wbase - 16 * t), L - 1);
        vb[t][r] = ldv(vt + (size_t)(key - t0) * DV + vcol);
      } else {
        const int key = min(vrow(t, r), L - 1);
        vb[t][r] = ldv(vt + (size_t)key * DV + vcol);
      }
    }
  }
  // every load of the wave is issued before the first MFMA waits on one
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SPEC) {
    L = min(a.l_kv[b], max_l_kv);
    if (base >= L) return;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < VL; ++r)
        if (vrow(t, r) >= L) vb[t][r] = VLoad{};
  }
  floatx4 sc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) sc[t] = qk.mma(kb[t]) * scale;

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
      if constexpr (kMfmaPV) sc[t][r] = p;  // the weights stay in the score registers
      else if (hh < GH) s_p[wv][t][4 * kq + r][hh] = p;
    }
  zh = strided_lane_sum<16>(zh);
  if (lane < GH) {
    s_m[wv][lane] = mh;
    s_z[wv][lane] = zh;
  }

  if constexpr (kMfmaPV) {
    floatx4 acc[NCOL];
#pragma unroll
    for (int i = 0; i < NCOL; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tp = 0; tp < TPW; tp += 2) {
      // element e of a K-slice: key 16 (tp + e/4) + 4kq + e%4
      bf16x8 w1, w2, w3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = sc[tp + e / 4][e % 4];
        const __bf16 h1 = (__bf16)p;
        const float r1 = p - (float)h1;
        const __bf16 h2 = (__bf16)r1;
        const float r2 = r1 - (float)h2;
        w1[e] = h1;
        w2[e] = h2;
        w3[e] = (__bf16)r2;
      }
      const VLoad* v0 = vb[tp];
      const VLoad* v1 = vb[tp + 1];
#pragma unroll
      for (int i = 0; i < NCOL; ++i) {
        // element i of each of the 8 value loads: word i/2, half i%2
        const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
        auto word = [&](const VLoad& u) {
          if constexpr (NCOL == 4) {
            return (i >> 1) == 0 ? u.x : u.y;
          } else {
            return (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
          }
        };
        V16 bw;
        bw.u.x = __builtin_amdgcn_perm(word(v0[1]), word(v0[0]), sel);
        bw.u.y = __builtin_amdgcn_perm(word(v0[3]), word(v0[2]), sel);
        bw.u.z = __builtin_amdgcn_perm(word(v1[1]), word(v1[0]), sel);
        bw.u.w = __builtin_amdgcn_perm(word(v1[3]), word(v1[2]), sel);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, bw.h, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, bw.h, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, bw.h, acc[i], 0, 0, 0);
      }
    }
    // lane (x, kq) holds the wave's sum for head 4kq + j, column NCOL x + i in acc[i][j]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * kq + j;
      if (h < GH) {
        *reinterpret_cast<float4*>(&s_o[wv][h][NCOL * hh]) = make_float4(acc[0][j], acc[1][j], acc[2][j], acc[3][j]);
        if constexpr (NCOL == 8)
          *reinterpret_cast<float4*>(&s_o[wv][h][8 * hh + 4]) =
              make_float4(acc[4][j], acc[5][j], acc[6][j], acc[7][j]);
      }
    }
    __syncthreads();
  } else {
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
      const int k16 = (r * kWave + lane) / G;
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
  }

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

// Log-sum-exp merge of the chunk partials of each row (b, j), in one pass: thread t
// takes chunks t, t+256, ... and 16 columns, loads every one of its chunks' partials in
// one round, keeps its own maximum m_t and its sums relative to it, then the block
// rescales each thread's sums by exp(m_t - M) with M the row's maximum. D is the value
// head dimension. Block x of a row takes columns [16x, 16x + 16).
//   - D = 128 (kDenseCombXcd): a row's D / 16 blocks are placed on one XCD (block i goes
//     to XCD i mod 8), since they read interleaved 64-byte pieces of the same 528-byte
//     chunk partials; grid = 8 ceil(B h_q / 8) D / 16. Measured against row-major order:
//     31.6 against 31.9 us per dense step at the Qwen-shaped 128K layer, 405 against
//     419 us for 16 such sequences.
//   - D = 64: grid = (D / 16, h_q, B); placement on one XCD was slower there (Llama-
//     shaped 32K layer with 8 value heads: 19.1 against 18.8 us).
// block = 256.
constexpr int kDenseCombRegs = 4;  // chunks per thread whose partials are loaded together
template <int D> constexpr bool kDenseCombXcd = D >= 128;

template <int D>
__global__ __launch_bounds__(kBlock) void k_dense_combine(const DenseArgs a, int chd) {
  constexpr int CB = D / 16;
  int cg, b;
  long long row;
  if constexpr (kDenseCombXcd<D>) {
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    row = xcd + 8LL * (slot / CB);
    cg = slot - (slot / CB) * CB;
    if (row >= a.rows) return;
    b = (int)(row / a.h_q);
  } else {
    cg = blockIdx.x;
    b = blockIdx.z;
    row = (long long)b * a.h_q + blockIdx.y;
  }
  const float* rp = a.part + row * a.nchd * (D + 4);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  __shared__ float s_ftmp[kWaves];
  __shared__ float s_acc[kWaves][17];
  // the first round of loads is issued with l_kv (chunks past the length are not used)
  float2 mz[kDenseCombRegs];
  float4 x[kDenseCombRegs][4];
#pragma unroll
  for (int k = 0; k < kDenseCombRegs; ++k) {
    const int c = tid + k * kBlock;
    if (c < a.nchd) {
      const float* pc = rp + (long long)c * (D + 4);
      mz[k] = *reinterpret_cast<const float2*>(pc);
      const float4* p4 = reinterpret_cast<const float4*>(pc + 4 + cg * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) x[k][q] = p4[q];
    }
  }
  const int L = min(a.l_kv[b], a.max_l_kv);
  if (L <= 0) {
    if (tid < 16) {
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[row * D + cg * 16 + tid] = 0;
      else reinterpret_cast<float*>(a.out)[row * D + cg * 16 + tid] = 0.f;
    }
    return;
  }
  const int nch_b = (L + chd - 1) / chd;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kDenseCombRegs; ++k)
    if (tid + k * kBlock < nch_b) m = fmaxf(m, mz[k].x);
  for (int c = tid + kDenseCombRegs * kBlock; c < nch_b; c += kBlock) m = fmaxf(m, rp[(long long)c * (D + 4)]);
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  float z = 0.f;
  auto add = [&](float mc, float zc, const float4 (&xc)[4]) {
    const float w = expf(mc - m);
    z += w * zc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[4 * q] += w * xc[q].x;
      o[4 * q + 1] += w * xc[q].y;
      o[4 * q + 2] += w * xc[q].z;
      o[4 * q + 3] += w * xc[q].w;
    }
  };
#pragma unroll
  for (int k = 0; k < kDenseCombRegs; ++k)
    if (tid + k * kBlock < nch_b) add(mz[k].x, mz[k].y, x[k]);
  for (int c = tid + kDenseCombRegs * kBlock; c < nch_b; c += kBlock) {
    const float* pc = rp + (long long)c * (D + 4);
    const float4* p4 = reinterpret_cast<const float4*>(pc + 4 + cg * 16);
    const float4 xc[4] = {p4[0], p4[1], p4[2], p4[3]};
    add(pc[0], pc[1], xc);
  }
  // every chunk has at least one key, so a thread with chunks has a finite maximum
  const float M = block_max(m, s_ftmp);
  const float sc = m == -INFINITY ? 0.f : expf(m - M);
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = wave_sum(o[e] * sc);
  z = wave_sum(z * sc);
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
    const float y = oo / zz;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[row * D + cg * 16 + tid] = f32_to_bf16(y);
    else reinterpret_cast<float*>(a.out)[row * D + cg * 16 + tid] = y;
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
