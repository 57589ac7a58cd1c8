// C ABI of the sparse-attention library: argument checks, workspace carving
// and dispatch to the kernels.  Every check runs on the host before any
// launch; nothing here allocates device memory or synchronises the host.
#include "../../include/sa.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "sa_internal.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(sa_dtype t) { return t == SA_F32 || t == SA_BF16; }
bool block_ok(int b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

sa_status launched(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

// Device address of a buffer that may be pinned host memory (host placement
// of the non-dominant keys and the values, FASA sec. 2.C).  Device memory is
// used as it is; pinned host memory is replaced by its device mapping; host
// memory the device cannot reach (pageable, not registered with HIP) is
// refused, so no kernel ever dereferences it.
static bool device_view(const void* p, const void** out) {
  *out = p;
  if (!p) return true;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeHost) {
    if (!a.devicePointer) return false;
    *out = a.devicePointer;
    return true;
  }
  return a.type != hipMemoryTypeUnregistered;
}

extern "C" {

sa_status sa_rope_apply(const void* x, void* out, sa_dtype dtype, int B, int H, int S, int d,
                        const int32_t* pos, int pos0, double theta, void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!x || !out) return SA_ERR_NULL;
  if (B < 1 || H < 1 || S < 1 || !head_dim_ok(d)) return SA_ERR_SHAPE;
  if (!(theta > 1.0) || pos0 < 0) return SA_ERR_RANGE;
  const sa::RopeFreq fr = sa::make_rope_freq(d, theta);
  return launched(sa::launch_rope(x, out, dtype, B, H, S, d, pos, pos0, fr, as_stream(stream)));
}

sa_status sa_kv_cache_append(const void* k_new, const void* v_new, sa_dtype dtype, int B,
                             int Hkv, int S, int d, int Lmax, const int32_t* start, double theta,
                             int slab, const int32_t* dom_pairs, int n_dom, void* k_cache,
                             void* k_rest, void* v_cache, void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!k_new || !v_new || !start || !k_cache || !v_cache) return SA_ERR_NULL;
  if (B < 1 || Hkv < 1 || S < 1 || Lmax < 1 || !head_dim_ok(d)) return SA_ERR_SHAPE;
  if (!(theta > 1.0) || slab < 0 || slab > 2) return SA_ERR_RANGE;
  if (slab) {
    if (!dom_pairs) return SA_ERR_NULL;
    if (n_dom < 1 || 2 * n_dom > d) return SA_ERR_RANGE;
    if ((slab == 2 || 2 * n_dom < d) && !k_rest) return SA_ERR_NULL;
  }
  const void* kr = nullptr;
  const void* vc = nullptr;
  if (!device_view(k_rest, &kr) || !device_view(v_cache, &vc)) return SA_ERR_ACCESS;
  const sa::RopeFreq fr = sa::make_rope_freq(d, theta);
  return launched(sa::launch_kv_append(k_new, v_new, dtype, B, Hkv, S, d, Lmax, start, fr,
                                       slab, dom_pairs, slab ? n_dom : 0, k_cache,
                                       const_cast<void*>(kr), const_cast<void*>(vc),
                                       as_stream(stream)));
}

sa_status sa_block_score(const void* q, const void* k, sa_dtype dtype, int B, int Hq, int Hkv,
                         int S, int d, double theta, int block, int band_split_pair,
                         int calibrate, float sm_scale, int causal, void* q_rope_out,
                         float q_rope_scale, void* k_rope_out, float* pooled_q_out,
                         float* pooled_k_out, float* scores, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q || !k || !scores) return SA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || !head_dim_ok(d) ||
      !block_ok(block) || S % block != 0)
    return SA_ERR_SHAPE;
  if (!(theta > 1.0) || band_split_pair < 0 || band_split_pair > d / 2 ||
      !std::isfinite(q_rope_scale))
    return SA_ERR_RANGE;
  const int N = S / block;
  const size_t pq_bytes = static_cast<size_t>(B) * Hq * N * d * sizeof(float);
  const size_t pk_bytes = static_cast<size_t>(B) * Hkv * N * d * sizeof(float);
  size_t need = 0;
  if (!pooled_q_out) need += align_up(pq_bytes);
  if (!pooled_k_out) need += align_up(pk_bytes);
  if (need > 0 && (!ws || ws_bytes < need)) return SA_ERR_WORKSPACE;
  char* wp = static_cast<char*>(ws);
  float* pq = pooled_q_out;
  float* pk = pooled_k_out;
  if (!pq) { pq = reinterpret_cast<float*>(wp); wp += align_up(pq_bytes); }
  if (!pk) { pk = reinterpret_cast<float*>(wp); }
  const sa::RopeFreq fr = sa::make_rope_freq(d, theta);
  hipStream_t st = as_stream(stream);
  hipError_t e = sa::launch_rope_pool(q, k, dtype, B, Hq, Hkv, S, d, block, band_split_pair,
                                      calibrate ? 1 : 0, fr, q_rope_out, q_rope_scale, k_rope_out,
                                      pq, pk, st);
  if (e != hipSuccess) return SA_ERR_HIP;
  return launched(sa::launch_block_gemm(pq, pk, B, Hq, Hkv, N, d, sm_scale, causal ? 1 : 0,
                                        scores, st));
}

sa_status sa_token_score(const void* q_rope, const void* k, const void* k_rest, sa_dtype dtype,
                         int B, int Hq, int Hkv, int Lmax, int d, const int32_t* cache_len,
                         const int32_t* dom_pairs, int n_dom, int slab, float sm_scale,
                         float* scores, void* stream) {
  (void)k_rest;  // scoring reads the dominant slab only
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q_rope || !k || !cache_len || !dom_pairs || !scores) return SA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lmax < 1 || !head_dim_ok(d)) return SA_ERR_SHAPE;
  const int grp = Hq / Hkv;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return SA_ERR_UNSUPPORTED;
  if (n_dom < 1 || n_dom > d / 2) return SA_ERR_RANGE;
  if (slab) {
    const int w = 2 * n_dom;
    if (w != 8 && w != 16 && w != 32 && w != 64 && w != 128) return SA_ERR_UNSUPPORTED;
  }
  return launched(sa::launch_token_score(q_rope, k, dtype, B, Hq, Hkv, Lmax, d, cache_len,
                                         dom_pairs, n_dom, slab ? 1 : 0, sm_scale, scores,
                                         as_stream(stream)));
}

sa_status sa_token_topk(const void* q_rope, const void* k, sa_dtype dtype, int B, int Hq,
                        int Hkv, int Lmax, int d, const int32_t* cache_len,
                        const int32_t* dom_pairs, int n_dom, int slab, float sm_scale, int k_top,
                        int32_t* idx_out, int max_out, int32_t* count_out, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q_rope || !k || !cache_len || !dom_pairs || !idx_out || !count_out) return SA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lmax < 1 || Lmax > 262144 ||
      !head_dim_ok(d))
    return SA_ERR_SHAPE;
  const int grp = Hq / Hkv;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return SA_ERR_UNSUPPORTED;
  if (n_dom < 1 || n_dom > d / 2 || k_top < 0 || max_out < 1 || max_out < k_top) return SA_ERR_RANGE;
  if (slab) {
    // slab rows of 8 to 64 channels in a power of two, at most 128 bytes
    const int w = 2 * n_dom;
    const int row_bytes = w * (dtype == SA_BF16 ? 2 : 4);
    if (w < 8 || row_bytes > 128 || (w & (w - 1)) != 0) return SA_ERR_UNSUPPORTED;
  }
  const int64_t rows = static_cast<int64_t>(B) * Hq;
  if (!ws || ws_bytes < sa::token_topk_ws_bytes(rows, Lmax)) return SA_ERR_WORKSPACE;
  return launched(sa::launch_token_topk(q_rope, k, dtype, B, Hq, Hkv, Lmax, d, cache_len,
                                        dom_pairs, n_dom, slab ? 1 : 0, sm_scale, k_top, idx_out,
                                        max_out, count_out, ws, as_stream(stream)));
}

sa_status sa_topk_select(const float* scores, int64_t rows, int cols, const int32_t* valid_len,
                         const int32_t* k_per_row, int k_const, int n_sink, int n_local,
                         int32_t* idx_out, int max_out, int32_t* count_out, void* ws,
                         size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (rows < 0 || cols < 1 || cols > 262144) return SA_ERR_SHAPE;
  if (k_const < 0 || n_sink < 0 || n_local < 0) return SA_ERR_RANGE;
  if (max_out < 1 || static_cast<int64_t>(max_out) <
                         static_cast<int64_t>(n_sink) + n_local + k_const)
    return SA_ERR_RANGE;
  if (rows == 0) return SA_OK;
  if (!scores || !idx_out || !count_out) return SA_ERR_NULL;
  if (rows > 0x7fffffffLL) return SA_ERR_SHAPE;
  return launched(sa::launch_topk(scores, rows, cols, valid_len, k_per_row, k_const, n_sink,
                                  n_local, idx_out, max_out, count_out, as_stream(stream)));
}

int sa_prefill_row_params(int N, int64_t heads, int causal, int keep_const, int keep_percent,
                          int32_t* valid_len_out, int32_t* k_per_row_out) {
  if (N < 1 || heads < 1 || heads > 0x7fffffffLL / N) return -SA_ERR_SHAPE;
  if (keep_const < 0 || keep_percent < 0 || keep_percent > 100 || (!keep_const && !keep_percent))
    return -SA_ERR_RANGE;
  int kmax = 0;
  for (int I = 0; I < N; ++I) {
    const int64_t vis = causal ? I + 1 : N;
    const int64_t k = keep_const ? keep_const : (keep_percent * vis + 99) / 100;
    kmax = k > kmax ? static_cast<int>(k) : kmax;
    for (int64_t h = 0; h < heads; ++h) {
      const int64_t r = h * N + I;
      if (valid_len_out) valid_len_out[r] = static_cast<int32_t>(vis);
      if (k_per_row_out) k_per_row_out[r] = static_cast<int32_t>(k);
    }
  }
  return kmax;
}

sa_status sa_sparse_attn_prefill(const void* q_rope, const void* k_rope, const void* v,
                                 sa_dtype dtype, int B, int Hq, int Hkv, int S, int d, int block,
                                 const int32_t* blk_idx, const int32_t* blk_cnt, int max_sel,
                                 int causal, float sm_scale, void* out, float* lse, void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q_rope || !k_rope || !v || !blk_idx || !blk_cnt || !out) return SA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || !head_dim_ok(d) ||
      !block_ok(block) || S % block != 0)
    return SA_ERR_SHAPE;
  if (max_sel < 1) return SA_ERR_RANGE;
  if (static_cast<int64_t>(B) * Hq * (S / block) > 0x7fffffffLL) return SA_ERR_SHAPE;
  return launched(sa::launch_prefill(q_rope, k_rope, v, dtype, B, Hq, Hkv, S, d, block, blk_idx,
                                     blk_cnt, max_sel, causal ? 1 : 0, sm_scale, out, lse,
                                     as_stream(stream)));
}

// checks shared by both decode entry points
static sa_status decode_args(const void* q_rope, const void* k, const void*& k_rest, const void*& v,
                             sa_dtype dtype, int B, int Hq, int Hkv, int Lmax, int d,
                             const int32_t* dom_pairs, int n_dom, int slab, const int32_t* tok_idx,
                             const int32_t* tok_cnt, int max_k, const void* out) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q_rope || !k || !v || !tok_idx || !tok_cnt || !out) return SA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lmax < 1 || !head_dim_ok(d)) return SA_ERR_SHAPE;
  if (max_k < 1) return SA_ERR_RANGE;
  if (static_cast<int64_t>(B) * Hq > 0x7fffffffLL) return SA_ERR_SHAPE;
  if (slab) {
    if (!dom_pairs) return SA_ERR_NULL;
    if (n_dom < 1 || 2 * n_dom > d) return SA_ERR_RANGE;
    if (n_dom % 4 != 0) return SA_ERR_UNSUPPORTED;
    if (2 * n_dom < d && !k_rest) return SA_ERR_NULL;
  }
  return SA_OK;
}

sa_status sa_sparse_attn_decode(const void* q_rope, const void* k, const void* k_rest,
                                const void* v, sa_dtype dtype, int B, int Hq, int Hkv, int Lmax,
                                int d, const int32_t* cache_len, const int32_t* dom_pairs,
                                int n_dom, int slab, const int32_t* tok_idx,
                                const int32_t* tok_cnt, int max_k, float sm_scale, void* out,
                                float* lse, void* ws, size_t ws_bytes, void* stream) {
  const sa_status a = decode_args(q_rope, k, k_rest, v, dtype, B, Hq, Hkv, Lmax, d, dom_pairs,
                                  n_dom, slab, tok_idx, tok_cnt, max_k, out);
  if (a != SA_OK) return a;
  const size_t need = sa::decode_ws_bytes(B, Hq, max_k);
  if (!ws || ws_bytes < need) return SA_ERR_WORKSPACE;
  if (!device_view(k_rest, &k_rest) || !device_view(v, &v)) return SA_ERR_ACCESS;
  return launched(sa::launch_decode(q_rope, k, k_rest, v, dtype, B, Hq, Hkv, Lmax, d, cache_len,
                                    dom_pairs, n_dom, slab ? 1 : 0, tok_idx, tok_cnt, max_k,
                                    sm_scale, out, lse, ws, as_stream(stream)));
}

sa_status sa_sparse_attn_decode_static(const void* q_rope, const void* k, const void* k_rest,
                                       const void* v, sa_dtype dtype, int B, int Hq, int Hkv,
                                       int Lmax, int d, const int32_t* cache_len,
                                       const int32_t* dom_pairs, int n_dom, int slab,
                                       const int32_t* tok_idx, const int32_t* tok_cnt, int max_k,
                                       float sm_scale, void* out, float* lse, void* stream) {
  const sa_status a = decode_args(q_rope, k, k_rest, v, dtype, B, Hq, Hkv, Lmax, d, dom_pairs,
                                  n_dom, slab, tok_idx, tok_cnt, max_k, out);
  if (a != SA_OK) return a;
  if (sa::decode_scratch_bytes(B, Hq, max_k) > sa::kDecodeScratchBytes) return SA_ERR_WORKSPACE;
  if (!device_view(k_rest, &k_rest) || !device_view(v, &v)) return SA_ERR_ACCESS;
  void* scratch = nullptr;
  if (sa::decode_static_scratch(&scratch) != hipSuccess) return SA_ERR_HIP;
  return launched(sa::launch_decode(q_rope, k, k_rest, v, dtype, B, Hq, Hkv, Lmax, d, cache_len,
                                    dom_pairs, n_dom, slab ? 1 : 0, tok_idx, tok_cnt, max_k,
                                    sm_scale, out, lse, scratch, as_stream(stream)));
}

static bool calib_sizes_ok(int Hq, int Hkv, int M, int L, int d) {
  return Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && M >= 1 && L >= 1 && L <= 262144 &&
         head_dim_ok(d);
}

sa_status sa_calibrate_dominant(const void* q_rope, const void* k_rope, sa_dtype dtype, int Hq,
                                int Hkv, int M, int L, int d, int k_cal, int n_dom,
                                int32_t* dom_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (!q_rope || !k_rope || !dom_out || !counts_out) return SA_ERR_NULL;
  if (!calib_sizes_ok(Hq, Hkv, M, L, d)) return SA_ERR_SHAPE;
  if (k_cal < 1 || k_cal > L || n_dom < 1 || n_dom > d / 2) return SA_ERR_RANGE;
  if (dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < sa::calib_ws_bytes(Hq, M, L, d, Hkv, k_cal)) return SA_ERR_WORKSPACE;
  return launched(sa::launch_calibrate(q_rope, k_rope, Hq, Hkv, M, L, d, k_cal, n_dom, dom_out,
                                       counts_out, ws, as_stream(stream)));
}

sa_status sa_sfa_sparsify(const void* x, void* out, sa_dtype dtype, int64_t rows, int d,
                          int k_feat, void* stream) {
  if (!dtype_ok(dtype)) return SA_ERR_DTYPE;
  if (rows < 0 || !head_dim_ok(d)) return SA_ERR_SHAPE;
  if (k_feat < 0) return SA_ERR_RANGE;
  if (rows == 0) return SA_OK;
  if (!x || !out) return SA_ERR_NULL;
  return launched(sa::launch_sfa_sparsify(x, out, dtype, rows, d, k_feat, as_stream(stream)));
}

size_t sa_calibrate_workspace_bytes(int Hq, int Hkv, int M, int L, int d, int k_cal) {
  if (!calib_sizes_ok(Hq, Hkv, M, L, d) || k_cal < 1 || k_cal > L) return 0;
  return sa::calib_ws_bytes(Hq, M, L, d, Hkv, k_cal);
}

size_t sa_workspace_bytes(int op, int64_t rows, int cols, int B, int Hq, int max_k) {
  switch (op) {
    case SA_OP_BLOCK_SCORE:
      // rows = pooled vectors (B * (Hq + Hkv) * N), cols = d
      if (rows < 0 || cols < 0) return 0;
      return align_up(static_cast<size_t>(rows) * cols * sizeof(float)) + 2 * kAlign;
    case SA_OP_TOPK:
      return 0;
    case SA_OP_DECODE:
      if (B < 1 || Hq < 1 || max_k < 1) return 0;
      return sa::decode_ws_bytes(B, Hq, max_k);
    case SA_OP_TOKEN_TOPK:
      // rows = B * Hq, cols = Lmax
      if (rows < 1 || cols < 1) return 0;
      return sa::token_topk_ws_bytes(rows, cols);
    default:
      return 0;
  }
}

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "required pointer is NULL";
    case SA_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case SA_ERR_DTYPE: return "unknown dtype";
    case SA_ERR_RANGE: return "parameter out of range";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_HIP: return "HIP launch or runtime error";
    case SA_ERR_ACCESS: return "buffer not accessible from the device (pageable host memory)";
  }
  return "unknown status";
}

int sa_version(void) { return 200; }

}  // extern "C"
