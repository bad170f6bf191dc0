// A decode layer around the SAGA attention step, for one new token per sequence:
// the projections of eq. (1) (paper "More Value per Key: Asymmetric Sparse Attention
// for Faster LLM Decoding", summary page picx.dev DRD92V, "Attention Mechanism
// Formalization": Q = X W_Q, K = X W_K, V = X W_V, with h_k key heads and h_v value
// heads as in its section "SAGA Architecture"), the append of the new key and value
// rows to the caches, the attention step (SAGA + Atop-N, or dense) and the output
// projection W_O. Host side of the layer entry points of include/saga.h.
//
// The projections are skinny products (one row of X per sequence): y = x W^T with
// W stored as [n_out, n_in] rows. One block of 16 waves owns 16 output rows; its
// waves split the n_in dimension into 32-column steps and multiply 16 weight rows
// by up to 16 activation rows on the matrix cores (bf16 MFMA 16x16x32, weight rows
// as the A operand exactly as key rows are in the score tiles), then add their
// partial tiles in LDS. The kernels are bound by the weight bytes they stream.
#include "saga.h"

#include <cstddef>

#include "saga_device.hpp"

using namespace saga;

namespace {

constexpr int kLinWaves = 16;                  // waves per block: one 16-row output tile
constexpr int kLinThreads = kLinWaves * kWave;
constexpr int kLinInFlight = 4;                // 32-column steps in flight per wave
constexpr int kMaxModel = 1 << 16;             // largest supported n_in / n_out

struct LinearArgs {
  // pointers first (no pointer right after a scalar field: the compiler may merge
  // neighbouring fields into one vector load and rebuild the pointer from an integer)
  const bf16_t* x;        // [B, n_in]
  const bf16_t* w;        // [n_out, n_in]
  void* y;                // plain product: [B, n_out] (bf16 or fp32)
  bf16_t* q;              // projection: [B, n_q]
  bf16_t* kc;             // projection: key cache [B, h_k, l_max, d]
  bf16_t* vc;             // projection: value cache [B, h_v, l_max, d]
  const int32_t* l_kv;    // projection: rows cached before this token [B]
  int32_t* l_next;        // projection: rows cached after it [B]
  int B, n_in, n_out, n_q, n_k, d, h_k, h_v, l_max, out_bf16;
};

// y[b, o] = sum_i x[b, i] w[o, i] for the 16 rows o of tile blockIdx.x and the
// batch rows b of tile blockIdx.y (16 per tile). QKV: row o of the stacked
// [W_Q; W_K; W_V] goes to q (o < n_q), to the key cache row l_kv[b] of head
// (o - n_q) / d, or to the value cache row l_kv[b] of head (o - n_q - n_k) / d, as
// bf16; block (0, 0) also writes l_next = l_kv + 1. A full cache (l_kv[b] >= l_max)
// gets no row and keeps its length. grid = (ceil(n_out/16), ceil(B/16)),
// block = 1024.
template <bool QKV>
__global__ __launch_bounds__(kLinThreads) void k_linear(const LinearArgs a) {
  const bf16_t* const wbase = a.w;
  const bf16_t* const xbase = a.x;
  const int n_in = a.n_in, n_out = a.n_out, B = a.B;
  __builtin_amdgcn_sched_barrier(0);
  const int tile = blockIdx.x, bt = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int r = lane & 15, kq = lane >> 4;
  const int row = min(tile * 16 + r, n_out - 1);  // this lane's weight row (clamped, never stored)
  const int bx = bt * 16 + r;                     // this lane's activation row
  const bool xv = bx < B;
  const bf16_t* wr = wbase + (size_t)row * n_in + 8 * kq;
  const bf16_t* xr = xbase + (size_t)(xv ? bx : 0) * n_in + 8 * kq;
  const int steps = n_in / 32;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wv; s0 < steps; s0 += kLinWaves * kLinInFlight) {
    V16 wb[kLinInFlight], xb[kLinInFlight];
#pragma unroll
    for (int u = 0; u < kLinInFlight; ++u) {
      const int s = s0 + u * kLinWaves;
      wb[u].u = make_uint4(0, 0, 0, 0);
      xb[u].u = make_uint4(0, 0, 0, 0);
      if (s < steps) {
        wb[u].u = ld16(wr + 32 * s);
        if (xv) xb[u].u = ld16(xr + 32 * s);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kLinInFlight; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[u].h, xb[u].h, acc, 0, 0, 0);
  }

  // lane l holds rows 4*(l>>4) + i of the tile for activation row l & 15
  __shared__ float s_red[kLinWaves][16][17];
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wv][4 * kq + i][r] = acc[i];
  __syncthreads();
  if (tid >= 256) return;
  const int orow = tid >> 4, col = tid & 15;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kLinWaves; ++w) sum += s_red[w][orow][col];
  const int o = tile * 16 + orow, b = bt * 16 + col;
  if constexpr (QKV) {
    if (tile == 0 && bt == 0) {
      for (int i = tid; i < B; i += 256) a.l_next[i] = min(a.l_kv[i], a.l_max - 1) + 1;
    }
    if (o >= n_out || b >= B) return;
    const uint16_t v = f32_to_bf16(sum);
    if (o < a.n_q) {
      a.q[(size_t)b * a.n_q + o] = v;
      return;
    }
    const int L = a.l_kv[b];
    if (L < 0 || L >= a.l_max) return;
    const bool is_k = o < a.n_q + a.n_k;
    const int f = o - a.n_q - (is_k ? 0 : a.n_k);
    const int head = f / a.d, c = f - head * a.d;
    const int heads = is_k ? a.h_k : a.h_v;
    bf16_t* cache = is_k ? a.kc : a.vc;
    cache[(((size_t)b * heads + head) * a.l_max + L) * a.d + c] = v;
  } else {
    if (o >= n_out || b >= B) return;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.y)[(size_t)b * n_out + o] = f32_to_bf16(sum);
    else reinterpret_cast<float*>(a.y)[(size_t)b * n_out + o] = sum;
  }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool linear_dims_ok(long long B, long long n_in, long long n_out) {
  return B >= 1 && B <= 65535 * 16 && n_in >= 32 && n_in % 32 == 0 && n_in <= kMaxModel && n_out >= 1 &&
         n_out <= kMaxModel;
}

dim3 linear_grid(int B, int n_out) { return dim3((n_out + 15) / 16, (B + 15) / 16); }

saga_status launched() { return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP; }

// The attention shape of a layer with a bf16 output (the input of W_O).
saga_shape attn_shape(const saga_layer* L) {
  saga_shape s = L->attn;
  s.out_dtype = SAGA_BF16;
  return s;
}

// Checks shared by the layer entry points; `attn_bytes` receives the attention
// workspace size (0 if the shape is invalid).
saga_status check_layer(const saga_layer* L, int32_t N, int32_t max_l_kv, size_t* attn_bytes) {
  if (!L) return SAGA_ERR_NULL;
  const saga_shape s = attn_shape(L);
  const size_t n = saga_workspace_bytes(&s, N, max_l_kv);
  if (n == 0) return SAGA_ERR_SHAPE;
  if (s.dtype != SAGA_BF16 || (s.d_v != 0 && s.d_v != s.d)) return SAGA_ERR_UNSUPPORTED;
  if (!linear_dims_ok(s.batch, L->d_model, (long long)(s.h_q + s.h_k + s.h_v) * s.d) ||
      !linear_dims_ok(s.batch, (long long)s.h_q * s.d, L->d_model))
    return L->d_model % 32 != 0 || L->d_model < 32 ? SAGA_ERR_SHAPE : SAGA_ERR_UNSUPPORTED;
  if (attn_bytes) *attn_bytes = n;
  return SAGA_OK;
}

LinearArgs qkv_args(const saga_layer* L, const void* x, const void* w_qkv, void* k_cache, void* v_cache,
                    const int32_t* l_kv, int32_t* l_next, void* q) {
  const saga_shape& s = L->attn;
  LinearArgs a{};
  a.x = reinterpret_cast<const bf16_t*>(x);
  a.w = reinterpret_cast<const bf16_t*>(w_qkv);
  a.q = reinterpret_cast<bf16_t*>(q);
  a.kc = reinterpret_cast<bf16_t*>(k_cache);
  a.vc = reinterpret_cast<bf16_t*>(v_cache);
  a.l_kv = l_kv;
  a.l_next = l_next;
  a.B = s.batch;
  a.n_in = L->d_model;
  a.n_q = s.h_q * s.d;
  a.n_k = s.h_k * s.d;
  a.n_out = (s.h_q + s.h_k + s.h_v) * s.d;
  a.d = s.d;
  a.h_k = s.h_k;
  a.h_v = s.h_v;
  a.l_max = s.l_max;
  return a;
}

}  // namespace

extern "C" {

saga_status saga_linear(int32_t batch, int32_t n_in, int32_t n_out, const void* x, const void* w, void* y,
                        int32_t out_dtype, void* stream) {
  if (!x || !w || !y) return SAGA_ERR_NULL;
  if (batch < 1 || n_in < 32 || n_in % 32 != 0 || n_out < 1) return SAGA_ERR_SHAPE;
  if (!linear_dims_ok(batch, n_in, n_out)) return SAGA_ERR_UNSUPPORTED;
  if (out_dtype != SAGA_F32 && out_dtype != SAGA_BF16) return SAGA_ERR_UNSUPPORTED;
  LinearArgs a{};
  a.x = reinterpret_cast<const bf16_t*>(x);
  a.w = reinterpret_cast<const bf16_t*>(w);
  a.y = y;
  a.B = batch;
  a.n_in = n_in;
  a.n_out = n_out;
  a.out_bf16 = out_dtype == SAGA_BF16;
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_linear<false>), linear_grid(batch, n_out), dim3(kLinThreads), 0, (hipStream_t)stream, a);
  return launched();
}

saga_status saga_qkv_append(const saga_layer* L, const void* x, const void* w_qkv, void* k_cache, void* v_cache,
                            const int32_t* l_kv, int32_t* l_kv_next, void* q, void* stream) {
  if (!L || !x || !w_qkv || !k_cache || !v_cache || !l_kv || !l_kv_next || !q) return SAGA_ERR_NULL;
  const saga_status st = check_layer(L, 1, 0, nullptr);
  if (st != SAGA_OK) return st;
  if (l_kv == l_kv_next) return SAGA_ERR_SHAPE;
  const LinearArgs a = qkv_args(L, x, w_qkv, k_cache, v_cache, l_kv, l_kv_next, q);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_linear<true>), linear_grid(a.B, a.n_out), dim3(kLinThreads), 0, (hipStream_t)stream, a);
  return launched();
}

size_t saga_layer_workspace_bytes(const saga_layer* L, int32_t N, int32_t max_l_kv) {
  size_t attn = 0;
  if (check_layer(L, N, max_l_kv, &attn) != SAGA_OK) return 0;
  const size_t act = align_up((size_t)L->attn.batch * L->attn.h_q * L->attn.d * sizeof(bf16_t));
  return align_up(attn) + 2 * act;
}

saga_status saga_decode_layer(const saga_layer* L, int32_t attention, const void* x, const void* w_qkv,
                              const void* w_o, void* k_cache, void* v_cache, const int32_t* l_kv,
                              int32_t* l_kv_next, int32_t max_l_kv, int32_t N, int32_t refresh_period,
                              int64_t step, float* tau, void* y, int32_t* sel_count, int32_t* flags,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!L || !x || !w_qkv || !w_o || !k_cache || !v_cache || !l_kv || !l_kv_next || !y || !workspace)
    return SAGA_ERR_NULL;
  if (attention != SAGA_ATTN_ATOPN && attention != SAGA_ATTN_DENSE) return SAGA_ERR_UNSUPPORTED;
  if (attention == SAGA_ATTN_ATOPN && !tau) return SAGA_ERR_NULL;
  size_t attn_bytes = 0;
  const saga_status st = check_layer(L, attention == SAGA_ATTN_ATOPN ? N : 1, max_l_kv, &attn_bytes);
  if (st != SAGA_OK) return st;
  if (l_kv == l_kv_next) return SAGA_ERR_SHAPE;
  if (L->attn.out_dtype != SAGA_F32 && L->attn.out_dtype != SAGA_BF16) return SAGA_ERR_UNSUPPORTED;
  const saga_shape s = attn_shape(L);
  if (attention == SAGA_ATTN_ATOPN) {
    if (refresh_period < 1 || step < 0) return SAGA_ERR_SHAPE;
  } else if (s.h_k > s.h_v || s.h_v % s.h_k || s.h_q / s.h_v > 16) {
    return SAGA_ERR_UNSUPPORTED;
  }
  if (workspace_bytes < saga_layer_workspace_bytes(L, attention == SAGA_ATTN_ATOPN ? N : 1, max_l_kv))
    return SAGA_ERR_WORKSPACE;

  const size_t act = align_up((size_t)s.batch * s.h_q * s.d * sizeof(bf16_t));
  char* ws = reinterpret_cast<char*>(workspace);
  void* q = ws + align_up(attn_bytes);
  void* o = ws + align_up(attn_bytes) + act;
  const hipStream_t hs = (hipStream_t)stream;

  // eq. (1) for the new token, and its key and value rows appended to the caches
  const LinearArgs a = qkv_args(L, x, w_qkv, k_cache, v_cache, l_kv, l_kv_next, q);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_linear<true>), linear_grid(a.B, a.n_out), dim3(kLinThreads), 0, hs, a);
  if (hipGetLastError() != hipSuccess) return SAGA_ERR_HIP;

  // attention over the l_kv + 1 cached rows (every argument was checked above)
  saga_status at;
  if (attention == SAGA_ATTN_ATOPN)
    at = saga_decode_attn(&s, q, k_cache, v_cache, l_kv_next, max_l_kv, N, refresh_period, step, tau, o,
                          sel_count, nullptr, 0, flags, workspace, attn_bytes, stream);
  else
    at = saga_dense_gqa_attn(&s, q, k_cache, v_cache, l_kv_next, max_l_kv, o, workspace, attn_bytes, stream);
  if (at != SAGA_OK) return at;

  // output projection
  LinearArgs p{};
  p.x = reinterpret_cast<const bf16_t*>(o);
  p.w = reinterpret_cast<const bf16_t*>(w_o);
  p.y = y;
  p.B = s.batch;
  p.n_in = s.h_q * s.d;
  p.n_out = L->d_model;
  p.out_bf16 = L->attn.out_dtype == SAGA_BF16;
  hipLaunchKernelGGL((k_linear<false>), linear_grid(p.B, p.n_out), dim3(kLinThreads), 0, hs, p);
  return launched();
}

}  // extern "C"
