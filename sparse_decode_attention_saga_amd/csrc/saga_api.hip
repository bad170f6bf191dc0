// Host side of the C ABI declared in include/saga.h: argument checks, workspace
// layout and kernel launches. Nothing here allocates, synchronises or prints.
#include "saga.h"

#include <cmath>
#include <cstddef>
#include <mutex>

#include "saga_kernels.hpp"

using namespace saga;

// Scratch of saga_decode_attn_noalloc: the decode step's workspace for callers that
// cannot allocate. One copy per GPU, set up by the runtime when the library's code
// is loaded on that GPU and held until the process ends. Host code never passes
// this name to a kernel or a copy: on the host it is only a stand-in for the
// symbol; the device address of a GPU's copy comes from hipGetSymbolAddress
// (noalloc_scratch below) and only that address is used.
static __device__ __align__(256) uint8_t scratch[SAGA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxContext = 1 << 24;   // longest supported l_kv
constexpr int kMaxWaveKeyBytes = 32768;  // keys one wave of a streaming kernel has in flight
constexpr long long kMaxRows = 1 << 24;  // most (sequence, query head) rows of one call

// Runs the statement with P = the page flag as a compile-time constant.
#define SAGA_PAGED(FLAG, ...)          \
  do {                                 \
    if (FLAG) {                        \
      constexpr bool P = true;         \
      __VA_ARGS__                      \
    } else {                           \
      constexpr bool P = false;        \
      __VA_ARGS__                      \
    }                                  \
  } while (0)

// Runs the statement with W = the tiles per wave of the key-streaming kernels (2, 4 or
// 8) as a compile-time constant. Needs T and DK: forms over kMaxWaveKeyBytes are never
// chosen (stream_tiles) and are not instantiated.
#define SAGA_TILES(TILES, ...)                                                        \
  do {                                                                                \
    if ((TILES) == 8) {                                                               \
      constexpr int W = 16 * 8 * DK * (int)sizeof(T) <= kMaxWaveKeyBytes ? 8 : 4;    \
      __VA_ARGS__                                                                     \
    } else if ((TILES) == 4) {                                                        \
      constexpr int W = 4;                                                            \
      __VA_ARGS__                                                                     \
    } else {                                                                          \
      constexpr int W = 2;                                                            \
      __VA_ARGS__                                                                     \
    }                                                                                 \
  } while (0)

// Runs the statement with T = the element type, DK and DV = the key and value head
// dimensions as compile-time constants (the built combinations; check_shape refuses
// the others).
#define SAGA_DIMS(DKV, DVV, ...)                                      \
  do {                                                                \
    if ((DKV) == 128 && (DVV) == 128) {                               \
      constexpr int DK = 128, DV = 128;                               \
      __VA_ARGS__                                                     \
    } else if ((DKV) == 64 && (DVV) == 64) {                          \
      constexpr int DK = 64, DV = 64;                                 \
      __VA_ARGS__                                                     \
    } else if ((DKV) == 64 && (DVV) == 128) {                         \
      constexpr int DK = 64, DV = 128;                                \
      __VA_ARGS__                                                     \
    } else {                                                          \
      constexpr int DK = 32, DV = 64;                                 \
      __VA_ARGS__                                                     \
    }                                                                 \
  } while (0)

// fp32 caches: the same without (64, 128)
#define SAGA_DIMS_F32(DKV, DVV, ...)                                  \
  do {                                                                \
    if ((DKV) == 128 && (DVV) == 128) {                               \
      constexpr int DK = 128, DV = 128;                               \
      __VA_ARGS__                                                     \
    } else if ((DKV) == 64 && (DVV) == 64) {                          \
      constexpr int DK = 64, DV = 64;                                 \
      __VA_ARGS__                                                     \
    } else {                                                          \
      constexpr int DK = 32, DV = 64;                                 \
      __VA_ARGS__                                                     \
    }                                                                 \
  } while (0)

#define SAGA_DISPATCH(DT, DKV, DVV, ...)                              \
  do {                                                                \
    if ((DT) == SAGA_BF16) {                                          \
      using T = bf16_t;                                               \
      SAGA_DIMS(DKV, DVV, __VA_ARGS__);                               \
    } else {                                                          \
      using T = float;                                                \
      SAGA_DIMS_F32(DKV, DVV, __VA_ARGS__);                           \
    }                                                                 \
  } while (0)

// Value head dimension of a shape (0 in the struct means d).
int value_dim(const saga_shape* s) { return s->d_v > 0 ? s->d_v : s->d; }

// Tiles per wave of the key-streaming kernels (8, 4 or 2 tiles of 16 keys). The widest
// chunks that still give the launch two blocks per compute unit, unless twice as wide
// chunks give every unit a block and every wave a full 16 KiB of keys. Measured at
// batch 1: the 32K Llama-shaped layer (2 key heads of 64) takes 13.5 us per step with
// 128 blocks of 512 keys and 11.6 us with 512 blocks of 128; the 64K Qwen-shaped layer
// (1 key head of 128) is faster with 256 blocks of 256 keys (16 KiB per wave) than with
// 512 of 128. Narrower chunks than that only add chunk records. A wave holds at most
// kMaxWaveKeyBytes of keys in flight (its registers).
constexpr long long kMinStreamBlocks = 2 * 256;
constexpr int kFullWaveKeyBytes = 16384;

int stream_tiles(const saga_shape* s, int max_l_kv) {
  const int row_bytes = s->d * (s->dtype == SAGA_BF16 ? 2 : 4);
  int t_max = 8;
  while (t_max > 2 && 16 * t_max * row_bytes > kMaxWaveKeyBytes) t_max /= 2;
  if (max_l_kv <= 0) return t_max;
  const int g_k = s->h_q / s->h_k;
  const long long groups = (long long)s->h_k * ((g_k + 15) / 16) * s->batch;
  auto blocks = [&](int t) {
    const long long ch = 16LL * t * kWaves;
    return groups * ((max_l_kv + ch - 1) / ch);
  };
  int t = t_max;
  while (t > 2 && blocks(t) < kMinStreamBlocks) t /= 2;
  if (t < t_max && 16 * t * row_bytes < kFullWaveKeyBytes && 16 * 2 * t * row_bytes >= kFullWaveKeyBytes &&
      blocks(2 * t) >= kMinStreamBlocks / 2)
    t *= 2;
  return t;
}

saga_status check_shape(const saga_shape* s) {
  if (!s) return SAGA_ERR_NULL;
  if (s->batch < 1 || s->h_q < 1 || s->h_k < 1 || s->h_v < 1 || s->d < 1 || s->l_max < 1)
    return SAGA_ERR_SHAPE;
  if (s->h_q % s->h_k || s->h_q % s->h_v) return SAGA_ERR_SHAPE;
  if (!(s->scale >= 0.f) || !std::isfinite(s->scale)) return SAGA_ERR_SHAPE;
  if ((s->dtype != SAGA_F32 && s->dtype != SAGA_BF16) || (s->out_dtype != SAGA_F32 && s->out_dtype != SAGA_BF16))
    return SAGA_ERR_UNSUPPORTED;
  // head dimensions: d_k == d_v in {64, 128}, or the reduced key dimensions
  // (d_k, d_v) = (64, 128) in bf16 and (32, 64) (section "Training from Scratch":
  // a key head dimension below the value head dimension)
  if (s->d_v < 0) return SAGA_ERR_SHAPE;
  const int dv = value_dim(s);
  const bool same = s->d == dv && (s->d == 64 || s->d == 128);
  const bool reduced = (s->d == 32 && dv == 64) || (s->d == 64 && dv == 128 && s->dtype == SAGA_BF16);
  if (!same && !reduced) return SAGA_ERR_UNSUPPORTED;
  if (s->batch > 65535 || s->h_q > 65535 || s->l_max > kMaxContext) return SAGA_ERR_UNSUPPORTED;
  // rows (sequence, query head) are indexed with 32-bit integers in the kernels
  if ((long long)s->batch * s->h_q > kMaxRows) return SAGA_ERR_UNSUPPORTED;
  return SAGA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int rows, W, ch, nch, P;  // W: tiles per wave of the stream kernels; P: threshold-candidate blocks per row
  bool cand_chunk;          // threshold candidates per chunk (k_scores_hist), else per slice (k_cand_collect)
  int nsel;                 // candidate slices per row
  int nchd;                 // chunks of the dense kernels (DenseCfg: 16 KiB of keys and values per wave)
  long long lpad;
  size_t hist, cand_cnt;
  size_t scores, surv_idx, surv_val, chunk_hdr, part, total;
};

Layout layout(const saga_shape* s, int max_l_kv) {
  Layout w{};
  w.rows = s->batch * s->h_q;
  w.W = stream_tiles(s, max_l_kv);
  w.ch = 16 * w.W * kWaves;
  w.nch = max_l_kv > 0 ? (max_l_kv + w.ch - 1) / w.ch : 1;
  int chd = 0;
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), chd = (DenseCfg<T, DK, DV>::kChunk););
  w.nchd = max_l_kv > 0 ? (max_l_kv + chd - 1) / chd : 1;
  w.lpad = (long long)w.nch * w.ch;
  w.P = max_l_kv > 0 ? (max_l_kv + kSelSlice - 1) / kSelSlice : 1;
  const size_t rows = (size_t)w.rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  // sized for every chunk width (the narrowest chunks have the most records; lpad is at
  // most max_l_kv rounded up to the widest chunk), so that the size only grows with
  // max_l_kv whatever width a launch takes
  const int ch_min = 16 * 2 * kWaves, ch_max = 16 * 8 * kWaves;
  const size_t lpad_max = max_l_kv > 0 ? (size_t)(max_l_kv + ch_max - 1) / ch_max * ch_max : (size_t)ch_max;
  const size_t nch_max = max_l_kv > 0 ? (size_t)(max_l_kv + ch_min - 1) / ch_min : 1;
  // threshold candidates per chunk while a row has at most kMaxSel chunks, else per
  // slice of kSelSlice logits (collected by k_cand_collect)
  w.cand_chunk = w.nch <= kMaxSel;
  w.nsel = w.cand_chunk ? w.nch : w.P;
  const size_t nsel_max = nch_max < (size_t)kMaxSel ? nch_max : (size_t)kMaxSel;  // >= nch here, >= P
  // counters first: they must be zero before the first call and every call leaves them at zero
  w.hist = take((size_t)kHistCopies * rows * 256 * 4);
  w.cand_cnt = take(rows * nsel_max * 4);
  w.scores = take(rows * lpad_max * 4);
  w.surv_idx = take(rows * lpad_max * 4);
  w.surv_val = take(rows * lpad_max * 4);
  w.chunk_hdr = take(rows * nch_max * sizeof(ChunkHdr));
  // chunk records (sparse: d_v floats, dense: d_v + 4)
  w.part = take(rows * (nch_max > (size_t)w.nchd ? nch_max : (size_t)w.nchd) * (value_dim(s) + 4) * 4);
  w.total = off;
  return w;
}

// Blocks per chunk of the select kernel. Each kept entry costs one value-row load and
// a block gathers with 16 groups of 16 lanes, 4 rows in flight per lane; a head with
// about CH * N / l_kv kept entries per chunk is worth more than one group once that
// exceeds two rounds of loads. The heads of a tile are then split over hsplit blocks
// (each re-reads the chunk's keys, so no split where one group suffices).
int head_split(const saga_shape* s, const Layout& w, int N, int max_l_kv) {
  if (max_l_kv <= 0) return 1;
  const int g_k = s->h_q / s->h_k;
  const int heads = g_k < 16 ? g_k : 16;
  const int elem = s->dtype == SAGA_BF16 ? 2 : 4;
  const int pieces = value_dim(s) * elem / 16;         // 16-byte pieces per value row
  const int rows_per_group_load = pieces >= 16 ? 1 : 16 / pieces;
  const long long kept = (long long)w.ch * (N < max_l_kv ? N : max_l_kv) / max_l_kv;
  const long long per_group = 2LL * rows_per_group_load * 4;  // two rounds of 4 loads
  const long long groups = (kept + per_group - 1) / per_group;
  const int owned = groups <= 1 ? 16 : (int)(16 / groups > 0 ? 16 / groups : 1);
  int hsplit = (heads + owned - 1) / owned;
  return hsplit < 1 ? 1 : hsplit;
}

// The late value gather (k_qk_select<kOutSlots> -> k_sparse_pv): the select kernel
// leaves each chunk's kept (index, logit) pairs in a slot record and the combining
// kernel gathers the kept value rows. Taken when
//   - value rows hold at least kLateMinRowBytes bytes,
//   - the caches are contiguous (with pages, each kept row's page lookup would add a
//     dependent load to the combining kernel: 18.26 against 17.13 us per step),
//   - a row has at most kPvGroupRecs * 64 chunks (one slot record per thread piece),
//   - the select kernel has at least two blocks per compute unit (kMinStreamBlocks), and
//   - a head is expected to keep at most 1 entry per chunk (CH N / max_l_kv), or at most
//     2 when the select kernel has at least kLateManyBlocks blocks.
// Otherwise the early gather (k_qk_select<kOutRecords> -> k_split_combine), which
// spreads the value rows over the select kernel's blocks. Measured on MI355X,
// amortized step, late against early gather:
//   - taken: the Qwen-shaped 128K layer (256-byte value rows, 512 blocks, 1 kept per
//     chunk) 15.78 against 16.03 us; 16 such sequences (4096 blocks, 2 per chunk) 124.4
//     against 129.2 us;
//   - not taken: at 512 blocks and 2 kept per chunk, the Qwen-shaped layer with 64-wide
//     keys 17.60 against 16.82 us and with two key heads (GQA) 23.64 against 22.12 us; the
//     Qwen-shaped layer forced to 256 blocks of 512 keys 18.6 against 16.0 us; the
//     Llama-shaped 32K layer (128-byte rows) 12.13 against 11.45 us and the ragged batch
//     of 8 with the same heads 59.2 against 55.2 us.
constexpr int kLateMinRowBytes = 256;
constexpr long long kLateManyBlocks = 2048;

bool late_gather(const saga_shape* s, const Layout& w, int N, int max_l_kv, bool paged = false) {
  if (paged || max_l_kv <= 0 || w.nch > kPvGroupRecs * (kBlock / 4)) return false;
  if (value_dim(s) * (s->dtype == SAGA_BF16 ? 2 : 4) < kLateMinRowBytes) return false;
  const int g_k = s->h_q / s->h_k;
  const long long blocks = (long long)w.nch * s->h_k * ((g_k + 15) / 16) * s->batch;
  if (blocks < kMinStreamBlocks) return false;
  const long long n = N < max_l_kv ? N : max_l_kv;
  const long long max_kept = blocks >= kLateManyBlocks ? 2 : 1;
  return (long long)w.ch * n <= max_kept * max_l_kv;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off);
}

int log2_exact(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Paged caches: the table must cover max_l_kv tokens; pages hold a power of two
// tokens, at least 16 (a 16-key tile then lies inside one page).
saga_status check_pages(const saga_pages* pg, int32_t max_l_kv) {
  if (!pg) return SAGA_ERR_NULL;
  if (!pg->table) return SAGA_ERR_NULL;
  const int pt = pg->page_tokens;
  if (pt < 16 || pt > kMaxContext || (pt & (pt - 1)) != 0) return SAGA_ERR_SHAPE;
  if (pg->max_pages < 1 || pg->num_pages < 1) return SAGA_ERR_SHAPE;
  if ((long long)pg->max_pages * pt < max_l_kv) return SAGA_ERR_SHAPE;
  return SAGA_OK;
}

StreamArgs stream_args(const saga_shape* s, const Layout& w, void* ws, const void* q, const void* k,
                       const void* v, const int32_t* l_kv, int32_t max_l_kv, const float* tau, int N,
                       const saga_pages* pg = nullptr) {
  StreamArgs a{};
  if (pg) {
    a.ptab = pg->table;
    a.ptab_stride = pg->max_pages;
    a.page_shift = log2_exact(pg->page_tokens);
    a.num_pages = pg->num_pages;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.part = at<float>(ws, w.part);
  a.h_v = s->h_v;
  a.l_kv = l_kv;
  a.tau = tau;
  a.scores = at<float>(ws, w.scores);
  a.surv_idx = at<int32_t>(ws, w.surv_idx);
  a.surv_val = at<float>(ws, w.surv_val);
  a.chunk_hdr = at<ChunkHdr>(ws, w.chunk_hdr);
  a.hist = at<unsigned>(ws, w.hist);
  a.cand_cnt = at<unsigned>(ws, w.cand_cnt);
  a.nsel = w.nsel;
  a.cand_slice = w.cand_chunk ? w.ch : kSelSlice;
  a.cand_chunk = w.cand_chunk ? 1 : 0;
  a.h_q = s->h_q;
  a.h_k = s->h_k;
  a.g_k = s->h_q / s->h_k;
  a.g_v = s->h_q / s->h_v;
  a.htiles = (a.g_k + 15) / 16;
  a.l_max = s->l_max;
  a.nch = w.nch;
  a.N = N;
  a.max_l_kv = max_l_kv;
  a.lpad = w.lpad;
  a.scale = s->scale > 0.f ? s->scale : (float)(1.0 / std::sqrt((double)s->d));
  a.hsplit = late_gather(s, w, N, max_l_kv, pg != nullptr) ? 1 : head_split(s, w, N, max_l_kv);
  return a;
}

saga_status check_common(const saga_shape* s, int32_t max_l_kv, void* ws, size_t ws_bytes, int32_t N) {
  const saga_status st = check_shape(s);
  if (st != SAGA_OK) return st;
  if (max_l_kv < 0 || max_l_kv > s->l_max) return SAGA_ERR_SHAPE;
  if (N < 1) return SAGA_ERR_SHAPE;
  if (!ws) return SAGA_ERR_NULL;
  if (ws_bytes < layout(s, max_l_kv).total) return SAGA_ERR_WORKSPACE;
  return SAGA_OK;
}

saga_status launched() { return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP; }

dim3 stream_grid(const saga_shape* s, const Layout& w) {
  const int g_k = s->h_q / s->h_k;
  return dim3(w.nch, s->h_k * ((g_k + 15) / 16), s->batch);
}

void launch_refresh(const saga_shape* s, const Layout& w, const StreamArgs& a, float* tau, hipStream_t st) {
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), SAGA_PAGED(a.ptab != nullptr, SAGA_TILES(w.W, {
    if (s->batch == 1)  // one sequence: its chunks reach max_l_kv, key loads need not wait for l_kv
      hipLaunchKernelGGL((k_scores_hist<T, DK, P, W, true>), stream_grid(s, w), dim3(kBlock), 0, st, a);
    else
      hipLaunchKernelGGL((k_scores_hist<T, DK, P, W, false>), stream_grid(s, w), dim3(kBlock), 0, st, a);
  });););
  if (!a.cand_chunk) hipLaunchKernelGGL(k_cand_collect, dim3(w.P, s->h_q, s->batch), dim3(kBlock), 0, st, a);
  hipLaunchKernelGGL(k_select_finish, dim3(s->h_q, s->batch), dim3(kRowThreads), 0, st, a, tau);
}

// Scores and Atop-N comparison, leaving `out` (SelectOut): the kept lists only, the
// chunk records of eq. (7) (early gather) or the slot records (late gather).
template <int OUT, typename T, int DK, int DV, bool P, int W>
void launch_select_out(const saga_shape* s, dim3 grid, const StreamArgs& a, bool from_scores, hipStream_t st) {
  if (from_scores)
    hipLaunchKernelGGL((k_qk_select<T, DK, DV, kFromScores, OUT, P, W>), grid, dim3(kBlock), 0, st, a);
  else if (s->batch == 1)  // one sequence: its chunks reach max_l_kv, key loads need not wait for l_kv
    hipLaunchKernelGGL((k_qk_select<T, DK, DV, kFromKeysSpeculative, OUT, P, W>), grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL((k_qk_select<T, DK, DV, kFromKeys, OUT, P, W>), grid, dim3(kBlock), 0, st, a);
}

void launch_select(const saga_shape* s, const Layout& w, const StreamArgs& a, bool from_scores, int out,
                   hipStream_t st) {
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), SAGA_PAGED(a.ptab != nullptr, SAGA_TILES(w.W, {
    dim3 grid = stream_grid(s, w);
    grid.y *= a.hsplit;
    if (out == kOutList)
      hipLaunchKernelGGL((k_qk_select<T, DK, DV, kFromKeys, kOutList, P, W>), grid, dim3(kBlock), 0, st, a);
    else if (out == kOutSlots)
      launch_select_out<kOutSlots, T, DK, DV, P, W>(s, grid, a, from_scores, st);
    else
      launch_select_out<kOutRecords, T, DK, DV, P, W>(s, grid, a, from_scores, st);
  });););
}

// Chunk records from the kept lists (only for the separate gather stage).
void launch_chunk_gather(const saga_shape* s, const Layout& w, const StreamArgs& a, hipStream_t st) {
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), SAGA_PAGED(a.ptab != nullptr, SAGA_TILES(w.W, {
    hipLaunchKernelGGL((k_chunk_gather<T, DK, DV, P, W>), stream_grid(s, w), dim3(kBlock), 0, st, a);
  });););
}

// The merge of eq. (7): of the chunk records (early gather) or, with `late`, the value
// gather over the slot records.
void launch_combine(const saga_shape* s, const Layout& w, const GatherArgs& g, bool late, hipStream_t st) {
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), SAGA_PAGED(g.s.ptab != nullptr, SAGA_TILES(w.W, {
    if (late) {
      // P blocks per row, a row's blocks on one XCD (k_sparse_pv)
      const int per_row = DV * (int)sizeof(T) / 16;
      hipLaunchKernelGGL((k_sparse_pv<T, DK, DV, P, W>), dim3(8 * ((g.rows + 7) / 8) * per_row), dim3(kBlock), 0, st,
                         g);
    }
    else
      hipLaunchKernelGGL((k_split_combine<T, DK, DV, P, W>), dim3(DV / 16, s->h_q, s->batch), dim3(kBlock), 0, st,
                         g);
  });););
}

GatherArgs gather_args(const saga_shape* s, const StreamArgs& sa, float* tau, void* out, int32_t* sel_count,
                       int32_t* sel_idx, int32_t sel_cap, int32_t* flags, bool refreshed) {
  GatherArgs g{};
  g.s = sa;
  g.tau = tau;
  g.out = out;
  g.sel_count = sel_count;
  g.sel_idx = sel_idx;
  g.flags = flags;
  g.sel_cap = sel_idx ? sel_cap : 0;
  g.out_bf16 = s->out_dtype == SAGA_BF16;
  g.refreshed = refreshed ? 1 : 0;
  g.rows = s->batch * s->h_q;
  return g;
}

saga_status decode_impl(const saga_shape* s, const saga_pages* pg, const void* q, const void* k, const void* v,
                        const int32_t* l_kv, int32_t max_l_kv, int32_t N, int32_t refresh_period, int64_t step,
                        float* tau, void* out, int32_t* sel_count, int32_t* sel_idx, int32_t sel_cap,
                        int32_t* flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !q || !k || !v || !l_kv || !tau || !out) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, N);
  if (st != SAGA_OK) return st;
  if (refresh_period < 1 || step < 0 || (sel_idx && sel_cap < 1)) return SAGA_ERR_SHAPE;
  const Layout w = layout(s, max_l_kv);
  const hipStream_t hs = (hipStream_t)stream;
  const bool refresh = (step % refresh_period) == 0;
  (void)hipGetLastError();
  const StreamArgs a = stream_args(s, w, workspace, q, k, v, l_kv, max_l_kv, tau, N, pg);
  const bool late = late_gather(s, w, N, max_l_kv, pg != nullptr);
  if (max_l_kv > 0) {
    if (refresh) launch_refresh(s, w, a, tau, hs);
    launch_select(s, w, a, refresh, late ? kOutSlots : kOutRecords, hs);
  }
  launch_combine(s, w, gather_args(s, a, tau, out, sel_count, sel_idx, sel_cap, flags, refresh), late, hs);
  return launched();
}

// Device address of the current GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept; null if the lookup fails.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

saga_status dense_impl(const saga_shape* s, const saga_pages* pg, const void* q, const void* k, const void* v,
                       const int32_t* l_kv, int32_t max_l_kv, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!s || !q || !k || !v || !l_kv || !out) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, 1);
  if (st != SAGA_OK) return st;
  // the query heads of one value head must share one key head: h_k divides h_v
  if (s->h_k > s->h_v || s->h_v % s->h_k) return SAGA_ERR_UNSUPPORTED;
  const int g = s->h_q / s->h_v;
  if (g > 16) return SAGA_ERR_UNSUPPORTED;
  const Layout w = layout(s, max_l_kv);
  const hipStream_t hs = (hipStream_t)stream;
  DenseArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.l_kv = l_kv;
  a.part = at<float>(workspace, w.part);
  a.out = out;
  a.h_q = s->h_q;
  a.h_k = s->h_k;
  a.h_v = s->h_v;
  a.g = g;
  a.l_max = s->l_max;
  a.nchd = w.nchd;
  a.max_l_kv = max_l_kv;
  a.out_bf16 = s->out_dtype == SAGA_BF16;
  a.scale = s->scale > 0.f ? s->scale : (float)(1.0 / std::sqrt((double)s->d));
  a.rows = s->batch * s->h_q;
  if (pg) {
    a.ptab = pg->table;
    a.ptab_stride = pg->max_pages;
    a.page_shift = log2_exact(pg->page_tokens);
    a.num_pages = pg->num_pages;
  }
  (void)hipGetLastError();
  SAGA_DISPATCH(s->dtype, s->d, value_dim(s), SAGA_PAGED(pg != nullptr, {
    if (max_l_kv > 0) {
      const dim3 grid(w.nchd, s->h_v, s->batch);
      constexpr int TD = DenseCfg<T, DK, DV>::kTPW;
      // one sequence: its chunks reach max_l_kv, loads need not wait for l_kv
      if (s->batch == 1) {
        if (g <= 4) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 4, P, TD, true>), grid, dim3(kBlock), 0, hs, a);
        else if (g <= 6) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 6, P, TD, true>), grid, dim3(kBlock), 0, hs, a);
        else if (g <= 8) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 8, P, TD, true>), grid, dim3(kBlock), 0, hs, a);
        else hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 16, P, TD, true>), grid, dim3(kBlock), 0, hs, a);
      } else {
        if (g <= 4) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 4, P, TD, false>), grid, dim3(kBlock), 0, hs, a);
        else if (g <= 6) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 6, P, TD, false>), grid, dim3(kBlock), 0, hs, a);
        else if (g <= 8) hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 8, P, TD, false>), grid, dim3(kBlock), 0, hs, a);
        else hipLaunchKernelGGL((k_dense_partial<T, DK, DV, 16, P, TD, false>), grid, dim3(kBlock), 0, hs, a);
      }
    }
    const dim3 cgrid = kDenseCombXcd<DV> ? dim3(8 * ((a.rows + 7) / 8) * (DV / 16)) : dim3(DV / 16, s->h_q, s->batch);
    hipLaunchKernelGGL((k_dense_combine<DV>), cgrid, dim3(kBlock), 0, hs, a, (int)DenseCfg<T, DK, DV>::kChunk);
  }););
  return launched();
}

}  // namespace

extern "C" {

const char* saga_status_str(int32_t status) {
  switch (status) {
    case SAGA_OK: return "SAGA_OK";
    case SAGA_ERR_NULL: return "SAGA_ERR_NULL";
    case SAGA_ERR_SHAPE: return "SAGA_ERR_SHAPE";
    case SAGA_ERR_UNSUPPORTED: return "SAGA_ERR_UNSUPPORTED";
    case SAGA_ERR_WORKSPACE: return "SAGA_ERR_WORKSPACE";
    case SAGA_ERR_HIP: return "SAGA_ERR_HIP";
    default: return "SAGA_ERR_UNKNOWN";
  }
}

size_t saga_workspace_bytes(const saga_shape* s, int32_t N, int32_t max_l_kv) {
  if (check_shape(s) != SAGA_OK || N < 1 || max_l_kv < 0 || max_l_kv > s->l_max) return 0;
  return layout(s, max_l_kv).total;
}

int32_t saga_gather_form(const saga_shape* s, int32_t N, int32_t max_l_kv) {
  if (check_shape(s) != SAGA_OK || N < 1 || max_l_kv < 0 || max_l_kv > s->l_max) return -1;
  return late_gather(s, layout(s, max_l_kv), N, max_l_kv) ? 1 : 0;
}

saga_status saga_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return SAGA_ERR_NULL;
  if (bytes == 0) return SAGA_OK;
  (void)hipGetLastError();
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + kBlock - 1) / kBlock;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)stream,
                     (uint8_t*)workspace, bytes);
  return launched();
}

saga_status saga_decode_attn(const saga_shape* s, const void* q, const void* k, const void* v,
                             const int32_t* l_kv, int32_t max_l_kv, int32_t N, int32_t refresh_period,
                             int64_t step, float* tau, void* out, int32_t* sel_count, int32_t* sel_idx,
                             int32_t sel_cap, int32_t* flags, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode_impl(s, nullptr, q, k, v, l_kv, max_l_kv, N, refresh_period, step, tau, out, sel_count, sel_idx,
                     sel_cap, flags, workspace, workspace_bytes, stream);
}

saga_status saga_decode_attn_paged(const saga_shape* s, const saga_pages* pages, const void* q,
                                   const void* k_pages, const void* v_pages, const int32_t* l_kv,
                                   int32_t max_l_kv, int32_t N, int32_t refresh_period, int64_t step,
                                   float* tau, void* out, int32_t* sel_count, int32_t* sel_idx,
                                   int32_t sel_cap, int32_t* flags, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const saga_status st = check_pages(pages, max_l_kv);
  if (st != SAGA_OK) return st;
  return decode_impl(s, pages, q, k_pages, v_pages, l_kv, max_l_kv, N, refresh_period, step, tau, out, sel_count,
                     sel_idx, sel_cap, flags, workspace, workspace_bytes, stream);
}

saga_status saga_decode_attn_noalloc(const saga_shape* s, const void* q, const void* k, const void* v,
                                     const int32_t* l_kv, int32_t max_l_kv, int32_t N, int32_t refresh_period,
                                     int64_t step, float* tau, void* out, int32_t* sel_count, int32_t* sel_idx,
                                     int32_t sel_cap, int32_t* flags, void* stream) {
  // every argument check of saga_decode_attn, before the scratch is touched
  if (!s || !q || !k || !v || !l_kv || !tau || !out) return SAGA_ERR_NULL;
  saga_status st = check_shape(s);
  if (st != SAGA_OK) return st;
  if (max_l_kv < 0 || max_l_kv > s->l_max || N < 1) return SAGA_ERR_SHAPE;
  if (refresh_period < 1 || step < 0 || (sel_idx && sel_cap < 1)) return SAGA_ERR_SHAPE;
  const Layout w = layout(s, max_l_kv);
  if (w.total > (size_t)SAGA_NOALLOC_SCRATCH_BYTES) return SAGA_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return SAGA_ERR_HIP;
  const hipStream_t hs = (hipStream_t)stream;
  (void)hipGetLastError();
  // The threshold counters must be zero when a refresh starts. Every refresh leaves
  // them at zero, but the scratch is shared by every call on this GPU and its first
  // contents are not the library's, so each refresh step clears them first (a fill
  // kernel, which a graph capture records as an ordinary kernel node).
  if (max_l_kv > 0 && step % refresh_period == 0)
    hipLaunchKernelGGL(k_zero_fill, dim3(32), dim3(kBlock), 0, hs, reinterpret_cast<uint8_t*>(ws), w.scores);
  return decode_impl(s, nullptr, q, k, v, l_kv, max_l_kv, N, refresh_period, step, tau, out, sel_count, sel_idx,
                     sel_cap, flags, ws, (size_t)SAGA_NOALLOC_SCRATCH_BYTES, stream);
}

saga_status saga_refresh_threshold(const saga_shape* s, const void* q, const void* k, const int32_t* l_kv,
                                   int32_t max_l_kv, int32_t N, float* tau, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!s || !q || !k || !l_kv || !tau) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, N);
  if (st != SAGA_OK) return st;
  const Layout w = layout(s, max_l_kv);
  (void)hipGetLastError();
  if (max_l_kv > 0)
    launch_refresh(s, w, stream_args(s, w, workspace, q, k, nullptr, l_kv, max_l_kv, tau, N), tau, (hipStream_t)stream);
  return launched();
}

saga_status saga_qk_select(const saga_shape* s, const void* q, const void* k, const int32_t* l_kv,
                           int32_t max_l_kv, const float* tau, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!s || !q || !k || !l_kv || !tau) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, 1);
  if (st != SAGA_OK) return st;
  const Layout w = layout(s, max_l_kv);
  (void)hipGetLastError();
  if (max_l_kv > 0)
    launch_select(s, w, stream_args(s, w, workspace, q, k, nullptr, l_kv, max_l_kv, tau, 1), false, kOutList,
                  (hipStream_t)stream);
  return launched();
}

saga_status saga_sparse_gather(const saga_shape* s, const void* q, const void* k, const void* v,
                               const int32_t* l_kv, int32_t max_l_kv, int32_t N, float* tau, void* out,
                               int32_t* sel_count, int32_t* sel_idx, int32_t sel_cap, int32_t* flags,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !q || !k || !v || !l_kv || !tau || !out) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, N);
  if (st != SAGA_OK) return st;
  if (sel_idx && sel_cap < 1) return SAGA_ERR_SHAPE;
  const Layout w = layout(s, max_l_kv);
  const hipStream_t hs = (hipStream_t)stream;
  (void)hipGetLastError();
  const StreamArgs a = stream_args(s, w, workspace, q, k, v, l_kv, max_l_kv, tau, N);
  if (max_l_kv > 0) launch_chunk_gather(s, w, a, hs);
  launch_combine(s, w, gather_args(s, a, tau, out, sel_count, sel_idx, sel_cap, flags, false), false, hs);
  return launched();
}

saga_status saga_select_gather(const saga_shape* s, const void* q, const void* k, const void* v,
                               const int32_t* l_kv, int32_t max_l_kv, int32_t N, const float* tau,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !q || !k || !v || !l_kv || !tau) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, N);
  if (st != SAGA_OK) return st;
  const Layout w = layout(s, max_l_kv);
  (void)hipGetLastError();
  if (max_l_kv > 0)
    launch_select(s, w, stream_args(s, w, workspace, q, k, v, l_kv, max_l_kv, tau, N), false,
                  late_gather(s, w, N, max_l_kv) ? kOutSlots : kOutRecords, (hipStream_t)stream);
  return launched();
}

saga_status saga_split_combine(const saga_shape* s, const void* q, const void* k, const void* v,
                               const int32_t* l_kv, int32_t max_l_kv, int32_t N, float* tau, void* out,
                               int32_t* sel_count, int32_t* sel_idx, int32_t sel_cap, int32_t* flags,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!s || !q || !k || !v || !l_kv || !tau || !out) return SAGA_ERR_NULL;
  saga_status st = check_common(s, max_l_kv, workspace, workspace_bytes, N);
  if (st != SAGA_OK) return st;
  if (sel_idx && sel_cap < 1) return SAGA_ERR_SHAPE;
  const Layout w = layout(s, max_l_kv);
  (void)hipGetLastError();
  const StreamArgs a = stream_args(s, w, workspace, q, k, v, l_kv, max_l_kv, tau, N);
  launch_combine(s, w, gather_args(s, a, tau, out, sel_count, sel_idx, sel_cap, flags, false),
                 late_gather(s, w, N, max_l_kv), (hipStream_t)stream);
  return launched();
}

saga_status saga_dense_gqa_attn(const saga_shape* s, const void* q, const void* k, const void* v,
                                const int32_t* l_kv, int32_t max_l_kv, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return dense_impl(s, nullptr, q, k, v, l_kv, max_l_kv, out, workspace, workspace_bytes, stream);
}

saga_status saga_dense_gqa_attn_paged(const saga_shape* s, const saga_pages* pages, const void* q,
                                      const void* k_pages, const void* v_pages, const int32_t* l_kv,
                                      int32_t max_l_kv, void* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  const saga_status st = check_pages(pages, max_l_kv);
  if (st != SAGA_OK) return st;
  return dense_impl(s, pages, q, k_pages, v_pages, l_kv, max_l_kv, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
