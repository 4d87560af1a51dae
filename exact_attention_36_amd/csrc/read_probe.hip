// read_probe.hip -- HBM read-rate reference for the benchmark; built into a
// library of its own (libattn36_probe.so), not into libattn36.
//
// It reads the K and V of a decode-shaped cache ([B, S, H, 128] 16-bit, so
// one key of one head is a 256-byte row and consecutive keys of a head are
// H * 256 bytes apart) in the order the split-KV attention forward reads
// them: workgroup (sequence, head, split) walks its key range in 64-key
// tiles.  Nothing is computed; the rates bound what the attention kernel can
// reach on the same access pattern.
//   probe_read_dma:  global -> LDS DMA (buffer_load ... lds, 16 bytes per
//                    lane) into a two-deep ring, one barrier per tile, with or
//                    without the non-temporal hint -- the forward's tile path
//                    without its arithmetic
//   probe_read_regs: 16-byte loads into registers, each lane's loads of two
//                    keys in flight, non-temporal hint, no LDS and no barrier
// Each lane xors what it read (the DMA kernel: its share of each tile's
// chunks, read back from LDS) into one 16-byte value written to `sink`, so
// the loads cannot be dropped and every byte of K and V enters the xor of all
// of sink exactly once (a test checks that); sink holds 4096 bytes per
// workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int ROW = 256;   // bytes of one key of one head
constexpr int TILE = 64;   // keys per tile
constexpr int THREADS = 256;

__device__ __forceinline__ i32x4 rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4{(int32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu),
               (int32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

template <bool NT>
__device__ __forceinline__ void dma16(i32x4 r, const void* lds, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" : : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}

// workgroup -> (sequence b, head h, split sp); its keys are [sp*per, (sp+1)*per)
struct Range {
  int b, h, k0, per;
};
__device__ __forceinline__ Range range_of(int S, int H, int ns) {
  const int id = blockIdx.x;
  Range r;
  r.per = S / ns;
  r.k0 = (id % ns) * r.per;
  r.h = (id / ns) % H;
  r.b = id / (ns * H);
  return r;
}

template <bool NT>
__global__ __launch_bounds__(THREADS) void read_dma_kernel(const char* k, const char* v, int S, int H, int ns,
                                                           u32x4* sink) {
  constexpr int TB = TILE * ROW;           // bytes of one K (or V) tile
  constexpr int SL = TB / 1024 / 4;        // 1 KB slabs per wave per tile
  __shared__ __attribute__((aligned(1024))) char ring[2][2][TB];
  const Range g = range_of(S, H, ns);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t head0 = ((int64_t)g.b * S * H + g.h) * ROW;  // key 0 of this head
  const uint32_t bytes = (uint32_t)(((int64_t)(S - 1) * H + 1) * ROW);
  const i32x4 rk = rsrc(k + head0, bytes), rv = rsrc(v + head0, bytes);
  uint32_t off[SL];
#pragma unroll
  for (int n = 0; n < SL; n++) {
    const int byte = (wave * SL + n) * 1024 + lane * 16;  // within the tile
    off[n] = (uint32_t)((byte / ROW) * H * ROW + byte % ROW);
  }
  const int nt = g.per / TILE;
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)((int64_t)(g.k0 + t * TILE) * H * ROW);
#pragma unroll
    for (int n = 0; n < SL; n++) dma16<NT>(rk, &ring[t & 1][0][(wave * SL + n) * 1024], base + off[n]);
#pragma unroll
    for (int n = 0; n < SL; n++) dma16<NT>(rv, &ring[t & 1][1][(wave * SL + n) * 1024], base + off[n]);
  };
  u32x4 acc = {0, 0, 0, 0};
  if (nt > 0) issue(0);
  for (int t = 0; t < nt; t++) {
    // tile t is in LDS, and this wave's reads of tile t-1's slot have returned
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // everyone is done with tile t-1's slot, which issue() refills
    if (t + 1 < nt) issue(t + 1);
    // every 16-byte chunk of the tile's K and V, once over the workgroup
#pragma unroll
    for (int i = 0; i < 2 * TB / 16 / THREADS; i++) {
      const int c = i * THREADS + threadIdx.x;
      acc ^= *(const u32x4*)&ring[t & 1][c / (TB / 16)][(c % (TB / 16)) * 16];
    }
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = acc;
}

__global__ __launch_bounds__(THREADS) void read_regs_kernel(const u32x4* k, const u32x4* v, int S, int H, int ns,
                                                            u32x4* sink) {
  const Range g = range_of(S, H, ns);
  // 16 lanes per key row, 16 keys per pass, two passes in flight
  const int c = threadIdx.x & 15, kk = threadIdx.x >> 4;
  u32x4 acc = {0, 0, 0, 0};
  for (int j = 0; j < g.per; j += 32) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int64_t row = ((int64_t)g.b * S + g.k0 + j + 16 * u + kk) * H + g.h;
      x[2 * u] = __builtin_nontemporal_load(k + row * (ROW / 16) + c);
      x[2 * u + 1] = __builtin_nontemporal_load(v + row * (ROW / 16) + c);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) acc ^= x[u];
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = acc;
}

// 0 on success; 1 for sizes the kernels do not cover (S a multiple of
// n_split * 64, every offset inside one head's keys below 2^32 bytes); else
// the launch's HIP error.
int check(int B, int S, int H, int ns) {
  if (B <= 0 || S <= 0 || H <= 0 || ns <= 0 || S % ns || (S / ns) % TILE) return 1;
  if ((int64_t)S * H * ROW >= ((int64_t)1 << 32)) return 1;
  if ((int64_t)B * H * ns >= ((int64_t)1 << 31)) return 1;
  return 0;
}

}  // namespace

extern "C" int probe_read_dma(const void* k, const void* v, int B, int S, int H, int n_split, int nt, void* sink,
                              void* stream) {
  if (int e = check(B, S, H, n_split)) return e;
  const dim3 grid((unsigned)(B * H * n_split)), block(THREADS);
  if (nt)
    hipLaunchKernelGGL(read_dma_kernel<true>, grid, block, 0, (hipStream_t)stream, (const char*)k, (const char*)v, S,
                       H, n_split, (u32x4*)sink);
  else
    hipLaunchKernelGGL(read_dma_kernel<false>, grid, block, 0, (hipStream_t)stream, (const char*)k, (const char*)v,
                       S, H, n_split, (u32x4*)sink);
  return (int)hipGetLastError();
}

extern "C" int probe_read_regs(const void* k, const void* v, int B, int S, int H, int n_split, void* sink,
                               void* stream) {
  if (int e = check(B, S, H, n_split)) return e;
  hipLaunchKernelGGL(read_regs_kernel, dim3((unsigned)(B * H * n_split)), dim3(THREADS), 0, (hipStream_t)stream,
                     (const u32x4*)k, (const u32x4*)v, S, H, n_split, (u32x4*)sink);
  return (int)hipGetLastError();
}
