// Host-only run of the C ABI's checks under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with good and bad
// arguments, and the kernel launchers are stand-ins (launch_stubs.cpp) that
// record what reached them.  Built and run by tests/test_abi_cpu.py.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/sa.h"
#include "launch_stubs.hpp"

static int g_pass = 0, g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (c) {                                                       \
      ++g_pass;                                                    \
    } else {                                                       \
      ++g_fail;                                                    \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);  \
    }                                                              \
  } while (0)

static void* dev(uintptr_t off = 0) { return reinterpret_cast<void*>(kDevLo + 0x1000 + off); }
static void* pin(uintptr_t off = 0) { return reinterpret_cast<void*>(kPinLo + 0x1000 + off); }
static void* pageable() { return reinterpret_cast<void*>(0x50000000); }
static const int32_t* idev(uintptr_t off = 0) { return static_cast<const int32_t*>(dev(off)); }

// call f(); check the status and whether exactly one launch named `name` happened
template <typename F>
static void expect(sa_status want, const char* name, F f) {
  const int before = g_log.launches;
  const sa_status got = f();
  CHECK(got == want);
  if (got != want) std::printf("  status %d, wanted %d (%s)\n", got, want, name ? name : "-");
  if (name) {
    CHECK(g_log.launches > before && std::strcmp(g_log.name, name) == 0);
  } else {
    CHECK(g_log.launches == before);
  }
  CHECK(g_log.last_error_set == 0);  // no runtime error left behind
}

static size_t al(size_t x) { return (x + 255) / 256 * 256; }

int main() {
  const sa_dtype BF = SA_BF16, F32 = SA_F32;
  // ---- rotation
  expect(SA_OK, "rope", [&] { return sa_rope_apply(dev(), dev(), BF, 2, 3, 40, 128, nullptr, 5, 5e5, nullptr); });
  expect(SA_ERR_NULL, nullptr, [&] { return sa_rope_apply(nullptr, dev(), BF, 2, 3, 40, 128, nullptr, 5, 5e5, nullptr); });
  expect(SA_ERR_SHAPE, nullptr, [&] { return sa_rope_apply(dev(), dev(), BF, 2, 3, 40, 96, nullptr, 5, 5e5, nullptr); });
  expect(SA_ERR_RANGE, nullptr, [&] { return sa_rope_apply(dev(), dev(), BF, 2, 3, 40, 128, nullptr, -1, 5e5, nullptr); });
  expect(SA_ERR_RANGE, nullptr, [&] { return sa_rope_apply(dev(), dev(), BF, 2, 3, 40, 128, nullptr, 0, 1.0, nullptr); });
  expect(SA_ERR_DTYPE, nullptr, [&] { return sa_rope_apply(dev(), dev(), static_cast<sa_dtype>(7), 2, 3, 40, 128, nullptr, 0, 5e5, nullptr); });
  g_log.fail = 1;
  expect(SA_ERR_HIP, "rope", [&] { return sa_rope_apply(dev(), dev(), F32, 1, 1, 1, 64, nullptr, 0, 1e4, nullptr); });
  g_log.fail = 0;

  // ---- cache append: device, pinned (device view passed on) and pageable buffers
  expect(SA_OK, "kv_append", [&] { return sa_kv_cache_append(dev(), dev(), BF, 2, 8, 4, 128, 64, idev(), 5e5, 0, nullptr, 0, dev(), nullptr, dev(0x100), nullptr); });
  CHECK(g_log.p[2] == dev(0x100));
  expect(SA_OK, "kv_append", [&] { return sa_kv_cache_append(dev(), dev(), BF, 2, 8, 4, 128, 64, idev(), 5e5, 1, idev(), 16, dev(), pin(0x40), pin(0x80), nullptr); });
  CHECK(reinterpret_cast<uintptr_t>(g_log.p[1]) == reinterpret_cast<uintptr_t>(pin(0x40)) + kPinShift);
  CHECK(reinterpret_cast<uintptr_t>(g_log.p[2]) == reinterpret_cast<uintptr_t>(pin(0x80)) + kPinShift);
  expect(SA_ERR_ACCESS, nullptr, [&] { return sa_kv_cache_append(dev(), dev(), BF, 2, 8, 4, 128, 64, idev(), 5e5, 0, nullptr, 0, dev(), nullptr, pageable(), nullptr); });
  expect(SA_ERR_NULL, nullptr, [&] { return sa_kv_cache_append(dev(), dev(), BF, 2, 8, 4, 128, 64, idev(), 5e5, 1, idev(), 16, dev(), nullptr, dev(), nullptr); });
  expect(SA_ERR_RANGE, nullptr, [&] { return sa_kv_cache_append(dev(), dev(), BF, 2, 8, 4, 128, 64, idev(), 5e5, 1, idev(), 65, dev(), dev(), dev(), nullptr); });

  // ---- block scores: workspace carving of the pooled vectors
  {
    const int B = 1, Hq = 32, Hkv = 8, S = 32768, d = 128, blk = 128, N = S / blk;
    const size_t pq = static_cast<size_t>(B) * Hq * N * d * 4, pk = static_cast<size_t>(B) * Hkv * N * d * 4;
    const size_t need = al(pq) + al(pk);
    expect(SA_OK, "block_gemm", [&] { return sa_block_score(dev(), dev(), BF, B, Hq, Hkv, S, d, 5e5, blk, 16, 1, 0.088f, 1, dev(), 1.f, dev(), nullptr, nullptr, static_cast<float*>(dev(0x8000)), dev(0x100000), need, nullptr); });
    CHECK(g_log.p[0] == dev(0x100000));
    CHECK(reinterpret_cast<uintptr_t>(g_log.p[1]) == reinterpret_cast<uintptr_t>(dev(0x100000)) + al(pq));
    CHECK(sa_workspace_bytes(SA_OP_BLOCK_SCORE, static_cast<int64_t>(B) * (Hq + Hkv) * N, d, 0, 0, 0) >= need);
    expect(SA_ERR_WORKSPACE, nullptr, [&] { return sa_block_score(dev(), dev(), BF, B, Hq, Hkv, S, d, 5e5, blk, 16, 1, 0.088f, 1, nullptr, 1.f, nullptr, nullptr, nullptr, static_cast<float*>(dev()), dev(), need - 1, nullptr); });
    expect(SA_OK, "block_gemm", [&] { return sa_block_score(dev(), dev(), BF, B, Hq, Hkv, S, d, 5e5, blk, 16, 1, 0.088f, 1, nullptr, 1.f, nullptr, static_cast<float*>(dev(1)), static_cast<float*>(dev(2)), static_cast<float*>(dev()), nullptr, 0, nullptr); });
    expect(SA_ERR_SHAPE, nullptr, [&] { return sa_block_score(dev(), dev(), BF, B, Hq, Hkv, S + 1, d, 5e5, blk, 16, 1, 0.088f, 1, nullptr, 1.f, nullptr, nullptr, nullptr, static_cast<float*>(dev()), dev(), need, nullptr); });
    expect(SA_ERR_RANGE, nullptr, [&] { return sa_block_score(dev(), dev(), BF, B, Hq, Hkv, S, d, 5e5, blk, 65, 1, 0.088f, 1, nullptr, 1.f, nullptr, nullptr, nullptr, static_cast<float*>(dev()), dev(), need, nullptr); });
  }

  // ---- selection, keep budget
  expect(SA_OK, nullptr, [&] { return sa_topk_select(nullptr, 0, 10, nullptr, nullptr, 2, 0, 0, nullptr, 4, nullptr, nullptr, 0, nullptr); });
  expect(SA_OK, "topk", [&] { return sa_topk_select(static_cast<const float*>(dev()), 8192, 256, idev(), idev(), 26, 1, 2, static_cast<int32_t*>(dev(4)), 29, static_cast<int32_t*>(dev(8)), nullptr, 0, nullptr); });
  expect(SA_ERR_SHAPE, nullptr, [&] { return sa_topk_select(static_cast<const float*>(dev()), 0x80000000LL, 256, nullptr, nullptr, 26, 1, 2, static_cast<int32_t*>(dev()), 29, static_cast<int32_t*>(dev()), nullptr, 0, nullptr); });
  expect(SA_ERR_SHAPE, nullptr, [&] { return sa_topk_select(static_cast<const float*>(dev()), 4, 262145, nullptr, nullptr, 26, 1, 2, static_cast<int32_t*>(dev()), 29, static_cast<int32_t*>(dev()), nullptr, 0, nullptr); });
  expect(SA_ERR_RANGE, nullptr, [&] { return sa_topk_select(static_cast<const float*>(dev()), 4, 256, nullptr, nullptr, 0x7fffffff, 1, 2, static_cast<int32_t*>(dev()), 0x7fffffff, static_cast<int32_t*>(dev()), nullptr, 0, nullptr); });
  {
    std::vector<int32_t> vl(2 * 256), kr(2 * 256);
    CHECK(sa_prefill_row_params(256, 2, 1, 0, 10, vl.data(), kr.data()) == 26);
    CHECK(vl[0] == 1 && vl[255] == 256 && vl[256] == 1 && kr[9] == 1 && kr[10] == 2 && kr[511] == 26);
    CHECK(sa_prefill_row_params(1 << 16, 1 << 15, 1, 0, 10, nullptr, nullptr) == -SA_ERR_SHAPE);
    CHECK(sa_prefill_row_params(0x7fffffff, 1, 1, 0, 100, nullptr, nullptr) == 0x7fffffff);
    CHECK(sa_prefill_row_params(8, 4, 0, 0, 0, nullptr, nullptr) == -SA_ERR_RANGE);
  }

  // ---- prefill attention: row count limit
  expect(SA_OK, "prefill", [&] { return sa_sparse_attn_prefill(dev(), dev(), dev(), BF, 1, 32, 8, 32768, 128, 128, idev(), idev(), 29, 1, 0.69314718f, dev(0x40), nullptr, nullptr); });
  expect(SA_ERR_SHAPE, nullptr, [&] { return sa_sparse_attn_prefill(dev(), dev(), dev(), BF, 1 << 16, 1 << 10, 1, 128 * 64, 128, 128, idev(), idev(), 29, 1, 0.1f, dev(), nullptr, nullptr); });
  expect(SA_ERR_RANGE, nullptr, [&] { return sa_sparse_attn_prefill(dev(), dev(), dev(), BF, 1, 32, 8, 32768, 128, 128, idev(), idev(), 0, 1, 0.1f, dev(), nullptr, nullptr); });

  // ---- token scores and the fused token top-k
  expect(SA_OK, "token_score", [&] { return sa_token_score(dev(), dev(), nullptr, BF, 16, 32, 8, 65536, 128, idev(), idev(), 16, 0, 0.088f, static_cast<float*>(dev(0x10)), nullptr); });
  expect(SA_ERR_UNSUPPORTED, nullptr, [&] { return sa_token_score(dev(), dev(), nullptr, BF, 16, 24, 8, 65536, 128, idev(), idev(), 16, 0, 0.088f, static_cast<float*>(dev()), nullptr); });
  {
    const int64_t rows = 64 * 32;
    const int L = 131072;
    const size_t need = sa_workspace_bytes(SA_OP_TOKEN_TOPK, rows, L, 0, 0, 0);
    CHECK(need > static_cast<size_t>(rows) * (L / 4096) * 4 * 256 * 8);
    expect(SA_OK, "token_topk", [&] { return sa_token_topk(dev(), dev(), BF, 64, 32, 8, L, 128, idev(), idev(), 16, 1, 0.088f, 4096, static_cast<int32_t*>(dev()), 4096, static_cast<int32_t*>(dev()), dev(0x200), need, nullptr); });
    CHECK(g_log.p[2] == dev(0x200));
    expect(SA_ERR_WORKSPACE, nullptr, [&] { return sa_token_topk(dev(), dev(), BF, 64, 32, 8, L, 128, idev(), idev(), 16, 1, 0.088f, 4096, static_cast<int32_t*>(dev()), 4096, static_cast<int32_t*>(dev()), dev(), need - 1, nullptr); });
    expect(SA_ERR_UNSUPPORTED, nullptr, [&] { return sa_token_topk(dev(), dev(), F32, 64, 32, 8, L, 128, idev(), idev(), 2, 1, 0.088f, 4096, static_cast<int32_t*>(dev()), 4096, static_cast<int32_t*>(dev()), dev(), need, nullptr); });
    expect(SA_ERR_SHAPE, nullptr, [&] { return sa_token_topk(dev(), dev(), BF, 64, 32, 8, 262145, 128, idev(), idev(), 16, 1, 0.088f, 4096, static_cast<int32_t*>(dev()), 4096, static_cast<int32_t*>(dev()), dev(), need, nullptr); });
  }

  // ---- decode attention: workspace, slab rules, host placement
  {
    const size_t need = sa_workspace_bytes(SA_OP_DECODE, 0, 0, 2, 8, 700);
    CHECK(need == static_cast<size_t>(2) * 8 * 3 * 130 * 4 + 256);
    expect(SA_OK, "decode", [&] { return sa_sparse_attn_decode(dev(), dev(), nullptr, dev(0x20), BF, 2, 8, 2, 3000, 128, nullptr, nullptr, 0, 0, idev(), idev(), 700, 0.088f, dev(), nullptr, dev(0x400), need, nullptr); });
    CHECK(g_log.p[2] == dev(0x20));
    expect(SA_OK, "decode", [&] { return sa_sparse_attn_decode(dev(), dev(), pin(0x10), pin(0x20), BF, 2, 8, 2, 3000, 128, nullptr, idev(), 16, 1, idev(), idev(), 700, 0.088f, dev(), nullptr, dev(0x400), need, nullptr); });
    CHECK(reinterpret_cast<uintptr_t>(g_log.p[1]) == reinterpret_cast<uintptr_t>(pin(0x10)) + kPinShift);
    CHECK(reinterpret_cast<uintptr_t>(g_log.p[2]) == reinterpret_cast<uintptr_t>(pin(0x20)) + kPinShift);
    expect(SA_ERR_ACCESS, nullptr, [&] { return sa_sparse_attn_decode(dev(), dev(), pageable(), dev(), BF, 2, 8, 2, 3000, 128, nullptr, idev(), 16, 1, idev(), idev(), 700, 0.088f, dev(), nullptr, dev(), need, nullptr); });
    expect(SA_ERR_WORKSPACE, nullptr, [&] { return sa_sparse_attn_decode(dev(), dev(), nullptr, dev(), BF, 2, 8, 2, 3000, 128, nullptr, nullptr, 0, 0, idev(), idev(), 700, 0.088f, dev(), nullptr, dev(), need - 1, nullptr); });
    expect(SA_ERR_UNSUPPORTED, nullptr, [&] { return sa_sparse_attn_decode(dev(), dev(), dev(), dev(), BF, 2, 8, 2, 3000, 128, nullptr, idev(), 6, 1, idev(), idev(), 700, 0.088f, dev(), nullptr, dev(), need, nullptr); });
  }

  // ---- the allocation-free decode: partials in the library's array
  expect(SA_OK, "decode", [&] { return sa_sparse_attn_decode_static(dev(), dev(), nullptr, dev(0x20), BF, 2, 8, 2, 3000, 128, nullptr, nullptr, 0, 0, idev(), idev(), 700, 0.088f, dev(), nullptr, nullptr); });
  // one-pass form (B * Hq >= 512) needs no partials, whatever max_k
  expect(SA_OK, "decode", [&] { return sa_sparse_attn_decode_static(dev(), dev(), nullptr, dev(), BF, 64, 32, 8, 131072, 128, nullptr, nullptr, 0, 0, idev(), idev(), 131072, 0.088f, dev(), nullptr, nullptr); });
  // 511 lists x 64 splits x 520 B > 16 MiB
  expect(SA_ERR_WORKSPACE, nullptr, [&] { return sa_sparse_attn_decode_static(dev(), dev(), nullptr, dev(), BF, 1, 511, 511, 20000, 128, nullptr, nullptr, 0, 0, idev(), idev(), 16384, 0.088f, dev(), nullptr, nullptr); });
  expect(SA_ERR_ACCESS, nullptr, [&] { return sa_sparse_attn_decode_static(dev(), dev(), nullptr, pageable(), BF, 2, 8, 2, 3000, 128, nullptr, nullptr, 0, 0, idev(), idev(), 700, 0.088f, dev(), nullptr, nullptr); });
  expect(SA_ERR_NULL, nullptr, [&] { return sa_sparse_attn_decode_static(dev(), dev(), nullptr, dev(), BF, 2, 8, 2, 3000, 128, nullptr, nullptr, 0, 0, nullptr, idev(), 700, 0.088f, dev(), nullptr, nullptr); });

  // ---- calibration, feature codes
  {
    const size_t need = sa_calibrate_workspace_bytes(32, 8, 16, 8192, 128, 256);
    CHECK(need > static_cast<size_t>(32) * 16 * 64 * 8192 * 4);
    expect(SA_OK, "calibrate", [&] { return sa_calibrate_dominant(dev(), dev(), BF, 32, 8, 16, 8192, 128, 256, 16, static_cast<int32_t*>(dev()), static_cast<int32_t*>(dev()), dev(0x800), need, nullptr); });
    expect(SA_ERR_UNSUPPORTED, nullptr, [&] { return sa_calibrate_dominant(dev(), dev(), F32, 32, 8, 16, 8192, 128, 256, 16, static_cast<int32_t*>(dev()), static_cast<int32_t*>(dev()), dev(), need, nullptr); });
    CHECK(sa_calibrate_workspace_bytes(32, 8, 16, 8192, 128, 8193) == 0);
  }
  expect(SA_OK, nullptr, [&] { return sa_sfa_sparsify(nullptr, nullptr, BF, 0, 128, 16, nullptr); });
  expect(SA_OK, "sfa", [&] { return sa_sfa_sparsify(dev(), dev(), BF, 8192 * 40, 128, 16, nullptr); });

  // ---- strings, sizes of unknown operations
  for (int s = 0; s <= 9; ++s) CHECK(sa_status_string(static_cast<sa_status>(s)) != nullptr);
  CHECK(sa_workspace_bytes(99, 1, 1, 1, 1, 1) == 0);
  CHECK(sa_version() >= 100);

  std::printf("abi host checks: %d passed, %d failed\n", g_pass, g_fail);
  return g_fail ? 1 : 0;
}
