// Drives every entry point of the C ABI on the host, built with
// AddressSanitizer and the stub launchers of launch_stubs.cpp (no GPU): the
// argument checks on bad input, and on good input the workspace layout the
// kernels would be handed -- every region inside the caller's workspace, no
// two regions overlapping.  Device pointers are fake and never dereferenced.
// Prints one line per failed check and exits non-zero if any failed.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/attn.h"
#include "../../exact_attention_36_amd/csrc/attn_kernels.h"

namespace stub {
extern attn::FwdArgs last_fwd;
extern attn::BwdArgs last_bwd;
extern attn::OrderArgs last_order[2];
extern int last_order_n;
extern int fwd_calls, combine_calls, bwd_calls, append_calls, rotary_calls, order_calls;
extern int last_tile_d;
}  // namespace stub

static int failures = 0;
#define CHECK(cond)                                                                 \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, attn_last_error()); \
      failures++;                                                                   \
    }                                                                               \
  } while (0)

static void* const F = (void*)0x1000;  // a device address that is never touched

static attn_params params(int hq, int hkv, int d) {
  attn_params p;
  std::memset(&p, 0, sizeof p);
  p.dtype = ATTN_BF16;
  p.head_dim = d;
  p.heads_q = hq;
  p.heads_kv = hkv;
  p.causal = 1;
  p.window_left = -1;
  p.window_right = -1;
  return p;
}

struct Region {
  const char* name;
  const char* lo;
  size_t bytes;
};

// every region lies in [ws, ws + n) and no two overlap
static bool regions_ok(const std::vector<Region>& r, const char* ws, size_t n) {
  for (size_t i = 0; i < r.size(); i++) {
    if (r[i].lo < ws || r[i].lo + r[i].bytes > ws + n) {
      std::printf("region %s outside the workspace\n", r[i].name);
      return false;
    }
    for (size_t j = 0; j < i; j++)
      if (r[i].lo < r[j].lo + r[j].bytes && r[j].lo < r[i].lo + r[i].bytes) {
        std::printf("regions %s and %s overlap\n", r[i].name, r[j].name);
        return false;
      }
  }
  return true;
}

static void bad_params() {
  attn_params p = params(4, 2, 128);
  CHECK(attn_fwd(nullptr, 1, 16, 16, F, F, F, F, (float*)F, nullptr, 0, nullptr) == ATTN_EINVAL);
  const int bad[][3] = {{7, 128, 0}, {ATTN_BF16, 100, 0}, {ATTN_BF16, 264, 0}, {ATTN_BF16, 0, 0}};
  for (auto& b : bad) {
    attn_params q = p;
    q.dtype = b[0];
    q.head_dim = b[1];
    CHECK(attn_fwd(&q, 1, 16, 16, F, F, F, F, (float*)F, nullptr, 0, nullptr) == ATTN_EINVAL);
    CHECK(std::strlen(attn_last_error()) > 0 && std::strlen(attn_last_error()) < 512);
  }
  attn_params q = p;
  q.heads_q = 6;
  q.heads_kv = 4;
  CHECK(attn_bwd(&q, 1, 16, 16, F, F, F, F, (float*)F, F, F, F, F, nullptr, ATTN_BF16, nullptr, 0, nullptr) ==
        ATTN_EINVAL);
  q = p;
  q.window_left = -3;
  CHECK(attn_fwd_varlen(&q, 2, 10, 10, (int32_t*)F, (int32_t*)F, 8, 8, F, F, F, F, (float*)F, nullptr, 0,
                        nullptr) == ATTN_EINVAL);
  q = p;
  q.num_sinks = 65;
  CHECK(attn_fwd_kvcache(&q, 2, 4, F, F, F, (int32_t*)F, nullptr, 0, 0, 64, F, (float*)F, nullptr, 0, nullptr) ==
        ATTN_EINVAL);
  q = p;
  q.softcap = -1.f;
  CHECK(attn_bwd_noalloc(&q, 1, 16, 16, F, F, F, F, (float*)F, F, F, F, F, nullptr, ATTN_BF16, nullptr) ==
        ATTN_EINVAL);
  CHECK(attn_kvcache_append(&p, 1, 0, F, F, F, F, (int32_t*)F, nullptr, nullptr, 0, 0, 16, nullptr, nullptr, 0, 1,
                            0, nullptr) == ATTN_EINVAL);
  CHECK(attn_rotary(&p, 1, 1, 1, F, F, (int32_t*)F, 1, (float*)F, (float*)F, 24, 0, 4, nullptr) == ATTN_EINVAL);
  // sizes past the kernels' 32-bit arithmetic
  attn_params g = params(128, 1, 8);
  CHECK(attn_fwd(&g, 1, 300000, 16, F, F, F, F, (float*)F, nullptr, 0, nullptr) == ATTN_ENOTSUP);
  attn_params big = params(64, 64, 8);
  CHECK(attn_bwd(&big, 16, 600000, 16, F, F, F, F, (float*)F, F, F, F, F, nullptr, ATTN_BF16, F, (size_t)1 << 40,
                 nullptr) == ATTN_ENOTSUP);
  attn_params nb = params(64, 64, 128);
  CHECK(attn_bwd_noalloc(&nb, 64, 8192, 8192, F, F, F, F, (float*)F, F, F, F, F, nullptr, ATTN_BF16, nullptr) ==
        ATTN_ENOTSUP);
  int64_t n = 0;
  double ms = 0;
  CHECK(attn_timing_read(ATTN_KERNEL_COUNT, &n, &ms) == ATTN_EINVAL);
  CHECK(attn_timing_select(1u << ATTN_KERNEL_COUNT) == ATTN_EINVAL);
}

static void forward_layouts() {
  // prefill: no workspace, one launch
  attn_params p = params(16, 16, 128);
  int before = stub::fwd_calls;
  CHECK(attn_fwd_workspace_size(&p, 4, 2048, 2048) == 0);
  CHECK(attn_fwd(&p, 4, 2048, 2048, F, F, F, F, (float*)F, nullptr, 0, nullptr) == ATTN_OK);
  CHECK(stub::fwd_calls == before + 1 && stub::last_fwd.n_split == 1 && stub::last_fwd.total_ctas >= 1024);
  CHECK(stub::last_fwd.kv_once == 0);  // 16 query tiles per head share its K/V tiles
  // decode: split keys, partials in the workspace
  p = params(64, 8, 128);
  const size_t n = attn_fwd_workspace_size(&p, 32, 16, 32768);
  CHECK(n > 0);
  std::vector<char> ws(n);
  CHECK(attn_fwd(&p, 32, 16, 32768, F, F, F, F, (float*)F, ws.data(), n - 1, nullptr) == ATTN_EINVAL);
  const int comb = stub::combine_calls;
  CHECK(attn_fwd(&p, 32, 16, 32768, F, F, F, F, (float*)F, ws.data(), n, nullptr) == ATTN_OK);
  const attn::FwdArgs& a = stub::last_fwd;
  CHECK(a.n_split > 1 && stub::combine_calls == comb + 1);
  const size_t rows = (size_t)a.n_split * 32 * 8 * a.nmb * a.bm;
  CHECK(regions_ok({{"o_part", (const char*)a.o_part, rows * stub::last_tile_d * 4},
                    {"lse_part", (const char*)a.lse_part, rows * 4}},
                   ws.data(), n));
  // a batched decode with enough work tiles not to split: one work tile per
  // (sequence, kv head), so each K/V tile is read once
  CHECK(attn_fwd_workspace_size(&p, 128, 1, 8192) == 0);
  CHECK(attn_fwd(&p, 128, 1, 8192, F, F, F, F, (float*)F, nullptr, 0, nullptr) == ATTN_OK);
  CHECK(stub::last_fwd.n_split == 1 && stub::last_fwd.kv_once == 1 && stub::last_fwd.nmb == 1);
  // KV cache, paged: the same split path
  const size_t nk = attn_fwd_kvcache_workspace_size(&p, 32, 16, (int32_t*)F, 128, 256, 0);
  CHECK(nk > 0);
  std::vector<char> wk(nk);
  CHECK(attn_fwd_kvcache(&p, 32, 16, F, F, F, (int32_t*)F, (int32_t*)F, 128, 256, 0, F, (float*)F, wk.data(), nk,
                         nullptr) == ATTN_OK);
  CHECK(stub::last_fwd.s.block_table == (const int32_t*)F && stub::last_fwd.s.page_rows == 256);
  // packed: no workspace; K/V read once only when every sequence fits one work tile
  CHECK(attn_fwd_varlen_workspace_size(&p, 64, 65536, 65536, 5636, 5636) == 0);
  CHECK(attn_fwd_varlen(&p, 64, 65536, 65536, (int32_t*)F, (int32_t*)F, 5636, 5636, F, F, F, F, (float*)F, nullptr, 0,
                        nullptr) == ATTN_OK);
  CHECK(stub::last_fwd.kv_once == 0);
  CHECK(attn_fwd_varlen(&p, 64, 1024, 65536, (int32_t*)F, (int32_t*)F, 16, 5636, F, F, F, F, (float*)F, nullptr, 0,
                        nullptr) == ATTN_OK);
  CHECK(stub::last_fwd.kv_once == 1);
}

static void backward_layouts(bool sinks, bool packed) {
  attn_params p = params(32, 8, 128);
  float fake_sinks = 0.f;
  if (sinks) p.sinks = &fake_sinks;  // never read on the host
  const int64_t B = 2, S = 8192, T = packed ? 65536 : B * S;
  const size_t n = packed ? attn_bwd_varlen_workspace_size(&p, 64, T, T, 5000, 5000, ATTN_BF16)
                          : attn_bwd_workspace_size(&p, B, S, S, ATTN_BF16);
  CHECK(n > 0);
  std::vector<char> ws(n);
  int st;
  if (packed)
    st = attn_bwd_varlen(&p, 64, T, T, (int32_t*)F, (int32_t*)F, 5000, 5000, F, F, F, F, (float*)F, F, F, F, F,
                         sinks ? (float*)F : nullptr, ATTN_BF16, ws.data(), n, nullptr);
  else
    st = attn_bwd(&p, B, S, S, F, F, F, F, (float*)F, F, F, F, F, sinks ? (float*)F : nullptr, ATTN_BF16, ws.data(),
                  n, nullptr);
  CHECK(st == ATTN_OK);
  const attn::BwdArgs& a = stub::last_bwd;
  const size_t rows = (size_t)T * 32;
  std::vector<Region> r = {{"delta", (const char*)a.delta, rows * 4},
                           {"lse2", (const char*)a.lse2, rows * 4},
                           {"dscale_part", (const char*)a.dscale_part, (size_t)a.nbq * 8 * 2 * 4}};
  if (sinks) r.push_back({"dsink_part", (const char*)a.dsink_part, (size_t)a.nbq * 32 * 4});
  else CHECK(a.dsink_part == nullptr);
  if (packed) {
    // a dK/dV grid of 576 blocks x 8 kv heads with sequences of up to 5000
    // queries: both grids run in the order of schedule tables, built by one
    // launch before them
    CHECK(a.order_q != nullptr && a.order_k != nullptr);
    CHECK(stub::last_order_n == 2 && stub::last_order[0].order == a.order_q && !stub::last_order[0].key_major &&
          stub::last_order[0].nblk == a.nblk_q && stub::last_order[1].order == a.order_k &&
          stub::last_order[1].key_major && stub::last_order[1].nblk == a.nblk);
    r.push_back({"order_q", (const char*)a.order_q, (size_t)a.nblk_q * 8 * 4});
    r.push_back({"order_k", (const char*)a.order_k, (size_t)a.nblk * 8 * 4});
  } else {
    CHECK(a.order_q == nullptr && a.order_k == nullptr);
  }
  CHECK(regions_ok(r, ws.data(), n));
  if (packed) {
    // sequences of at most 1000 queries: no tables, a smaller workspace
    const size_t n2 = attn_bwd_varlen_workspace_size(&p, 64, T, T, 1000, 1000, ATTN_BF16);
    CHECK(n2 < n);
    const int oc = stub::order_calls;
    CHECK(attn_bwd_varlen(&p, 64, T, T, (int32_t*)F, (int32_t*)F, 1000, 1000, F, F, F, F, (float*)F, F, F, F, F,
                          sinks ? (float*)F : nullptr, ATTN_BF16, ws.data(), n2, nullptr) == ATTN_OK);
    CHECK(stub::order_calls == oc && stub::last_bwd.order_q == nullptr && stub::last_bwd.order_k == nullptr);
  }
  // the dQ grid covers the workgroups the slots are indexed by
  CHECK(a.total_ctas_q >= a.nbq * 8 || !packed);
  // too small a workspace is refused
  if (!packed)
    CHECK(attn_bwd(&p, B, S, S, F, F, F, F, (float*)F, F, F, F, F, sinks ? (float*)F : nullptr, ATTN_BF16, ws.data(),
                   n - 1, nullptr) == ATTN_EINVAL);
}

static void other_calls() {
  attn_params p = params(16, 4, 128);
  const int a0 = stub::append_calls, r0 = stub::rotary_calls, b0 = stub::bwd_calls;
  CHECK(attn_kvcache_append(&p, 2, 3, F, F, F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, 8, 64, 0, (float*)F,
                            (float*)F, 64, 0, 4096, nullptr) == ATTN_OK);
  CHECK(attn_rotary(&p, 2, 3, 16, F, F, (int32_t*)F, 1, (float*)F, (float*)F, 128, 1, 4096, nullptr) == ATTN_OK);
  CHECK(attn_bwd_noalloc(&p, 2, 300, 300, F, F, F, F, (float*)F, F, F, F, F, nullptr, ATTN_BF16, nullptr) == ATTN_OK);
  CHECK(stub::append_calls == a0 + 1 && stub::rotary_calls == r0 + 1 && stub::bwd_calls == b0 + 1);
  CHECK(attn_version() == 100);
}

int main() {
  bad_params();
  forward_layouts();
  for (int s = 0; s < 2; s++)
    for (int k = 0; k < 2; k++) backward_layouts(s, k);
  other_calls();
  if (failures) {
    std::printf("%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}
