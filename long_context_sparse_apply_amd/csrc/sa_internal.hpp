// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns the launch status; all
// argument checks have already been made by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kMaxPairs = 64;  // head_dim <= 128

// Rotation frequencies in revolutions per position: f_i = theta^(-2i/d) / (2 pi),
// fp64, computed on the host and passed by value as a kernel argument.
struct RopeFreq {
  double f[kMaxPairs];
};
RopeFreq make_rope_freq(int d, double theta);

// dtype codes match sa_dtype
enum { kF32 = 0, kBF16 = 1 };

hipError_t launch_rope(const void* x, void* out, int dtype, int B, int H, int S, int d,
                       const int32_t* pos, int pos0, const RopeFreq& fr, hipStream_t st);

// rotate new keys at their cache positions and write them (standard or slab
// layout) with their values into the decode cache
hipError_t launch_kv_append(const void* k_new, const void* v_new, int dtype, int B, int Hkv,
                            int S, int d, int Lmax, const int32_t* start, const RopeFreq& fr,
                            int slab, const int32_t* dom, int n_dom, void* k_out, void* k_rest,
                            void* v_out, hipStream_t st);

// fused rotation + calibrated dual-band block pooling of Q and K (one pass)
hipError_t launch_rope_pool(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int S,
                            int d, int block, int split, int calibrate, const RopeFreq& fr,
                            void* q_rope, float q_scale, void* k_rope, float* pq, float* pk,
                            hipStream_t st);

hipError_t launch_block_gemm(const float* pq, const float* pk, int B, int Hq, int Hkv, int N,
                             int d, float scale, int causal, float* scores, hipStream_t st);

hipError_t launch_topk(const float* scores, int64_t rows, int cols, const int32_t* valid_len,
                       const int32_t* k_per_row, int k_const, int n_sink, int n_local,
                       int32_t* idx_out, int max_out, int32_t* count_out, hipStream_t st);

hipError_t launch_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int S, int d, int block, const int32_t* blk_idx,
                          const int32_t* blk_cnt, int max_sel, int causal, float scale,
                          void* out, float* lse, hipStream_t st);

// candidate lists of the fused token top-k (defined with the selection keys)
struct TokenCollect;

// the scoring kernel in collect mode: tokens at or above their row's threshold
// key appended to the row's candidate lists (standard or dominant-slab layout)
hipError_t launch_token_collect(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                                int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                                int n_dom, int slab, float scale, const TokenCollect& col,
                                hipStream_t st);

// token scores and their top-k in one call, without a score array
size_t token_topk_ws_bytes(int64_t rows, int Lmax);
// long-row top-k: LDS of a work-group, candidate buffer of a row (plain and fused)
size_t topk_lds_bytes(int cols, int cap);
size_t token_select_lds_bytes(int cols, int cap);
int topk_cap(int k);
int token_topk_cap(int k);
hipError_t launch_token_topk(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                             int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                             int n_dom, int slab, float scale, int k_top, int32_t* idx_out,
                             int max_out, int32_t* count_out, void* ws, hipStream_t st);

hipError_t launch_token_score(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                              int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                              int n_dom, int slab, float scale, float* scores, hipStream_t st);

// decode: split-K partials in ws, then the merge.  With at least two (b, h)
// lists per CU of the chip a work-group takes a whole list (cpw = all its
// chunks, one pass, no partials); otherwise each takes one chunk and a merge
// pass combines the splits.
int decode_splits(int max_k);
size_t decode_ws_bytes(int B, int Hq, int max_k);
struct DecodePlan {
  int splits;  // work-groups per (b, h) list
  int cpw;     // 256-token chunks per work-group
};
DecodePlan decode_plan(int B, int Hq, int max_k);
// partials the launch actually writes (0 for the one-pass form)
size_t decode_scratch_bytes(int B, int Hq, int max_k);
// the allocation-free decode entry point's per-device array
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_static_scratch(void** ptr);
hipError_t launch_decode(const void* q, const void* k, const void* k_rest, const void* v,
                         int dtype, int B, int Hq, int Hkv, int Lmax, int d,
                         const int32_t* cache_len, const int32_t* dom, int n_dom, int slab,
                         const int32_t* tok_idx, const int32_t* tok_cnt, int max_k, float scale,
                         void* out, float* lse, void* ws, hipStream_t st);

// k-sparse feature codes (Sparse Feature Attention)
hipError_t launch_sfa_sparsify(const void* x, void* out, int dtype, int64_t rows, int d, int kf,
                               hipStream_t st);

// offline calibration of the dominant pairs (scores, selections, overlaps)
size_t calib_ws_bytes(int Hq, int M, int L, int d, int Hkv, int kcal);
hipError_t launch_calibrate(const void* q, const void* k, int Hq, int Hkv, int M, int L, int d,
                            int kcal, int n_dom, int32_t* dom_out, int32_t* counts_out, void* ws,
                            hipStream_t st);

}  // namespace sa
