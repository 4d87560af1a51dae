// attn_timing.cpp -- optional per-kernel timing with HIP events on the
// caller's stream (attn_timing_enable / attn_timing_read).
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/attn.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int POOL = 16384;

struct Rec {
  hipEvent_t start, stop;
  int kid;
};

bool g_on = false;
uint32_t g_mask = (1u << K_COUNT) - 1;  // kernels to time while on
bool g_overflow = false;
std::vector<Rec> g_pool;  // events, created on first enable
int g_used = 0;
int g_open = -1;          // record whose start is recorded but not its stop

}  // namespace

void timing_begin(int kid, hipStream_t st) {
  if (!g_on || !((g_mask >> kid) & 1u)) return;
  if (g_used >= (int)g_pool.size()) {
    g_overflow = true;
    g_open = -1;
    return;
  }
  g_open = g_used++;
  g_pool[g_open].kid = kid;
  hipEventRecord(g_pool[g_open].start, st);
}

void timing_end(int kid, hipStream_t st) {
  if (!g_on || g_open < 0) return;
  (void)kid;
  hipEventRecord(g_pool[g_open].stop, st);
  g_open = -1;
}

}  // namespace attn

using namespace attn;

extern "C" attn_status attn_timing_enable(int32_t on) {
  if (on && g_pool.empty()) {
    g_pool.resize(POOL);
    for (auto& r : g_pool) {
      if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
        g_pool.clear();
        return ATTN_EHIP;
      }
    }
  }
  g_on = on != 0;
  g_used = 0;
  g_open = -1;
  g_overflow = false;
  return ATTN_OK;
}

extern "C" attn_status attn_timing_select(uint32_t kernel_mask) {
  if (kernel_mask >> K_COUNT) return ATTN_EINVAL;
  g_mask = kernel_mask;
  return ATTN_OK;
}

extern "C" attn_status attn_timing_read(int32_t kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= K_COUNT || !launches || !total_ms) return ATTN_EINVAL;
  int64_t n = 0;
  double ms = 0.0;
  for (int i = 0; i < g_used; i++) {
    if (g_pool[i].kid != kernel) continue;
    if (hipEventSynchronize(g_pool[i].stop) != hipSuccess) return ATTN_EHIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_pool[i].start, g_pool[i].stop) != hipSuccess) return ATTN_EHIP;
    ms += t;
    n++;
  }
  *launches = n;
  *total_ms = ms;
  return g_overflow ? ATTN_ENOTSUP : ATTN_OK;
}
