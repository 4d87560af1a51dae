// attn_cache.hip -- KV-cache helpers for gfx950: rotary embedding of rows
// and the in-place append of new keys and values into a (paged) cache
// (vllm-project/flash-attention README on the GitHub search page,
// flash_attn_with_kvcache: k, v, cache_seqlens, rotary_cos, rotary_sin,
// rotary_interleaved, block_table).
//
// Rows of D 16-bit values, D/8 lanes per row and 64 / (D/8) rows per wave;
// lane c of a row's group owns the 16-byte chunk 8c .. 8c+7.  The first
// rotary_dim dims form rotary_dim/2 pairs: (2j, 2j+1) when interleaved --
// both in one chunk -- else (j, j + rotary_dim/2), whose partner chunk the
// lower lane reads and writes too.  rotary_dim is a
// multiple of 16, so no pair straddles chunks and rotating in place is safe.
// Pair j at position p turns by the angle whose cosine and sine are
// cos[p][j], sin[p][j]: (a, b) -> (a c - b s, a s + b c), in fp32, rounded to
// nearest even.
#include "attn_common.h"

namespace attn {
namespace {

// lanes per row and rows per workgroup for head dim D
__host__ __device__ constexpr int lanes_per_row(int D) { return D / 8; }
__host__ __device__ constexpr int rows_per_block(int D) { return (64 / lanes_per_row(D)) * (THREADS / 64); }
// this thread's row within the workgroup's rows (-1: an idle lane) and its chunk
__device__ __forceinline__ int row_slot(int D, int& chunk) {
  const int lpr = lanes_per_row(D), per_wave = 64 / lpr, lane = threadIdx.x & 63;
  chunk = lane % lpr;
  const int sub = lane / lpr;
  return sub < per_wave ? (int)(threadIdx.x >> 6) * per_wave + sub : -1;
}

template <bool F16>
__device__ __forceinline__ void unpack8(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; e++) {
    x[2 * e] = to_f32<F16>((uint16_t)(v[e] & 0xFFFFu));
    x[2 * e + 1] = to_f32<F16>((uint16_t)(v[e] >> 16));
  }
}
template <bool F16>
__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
  return u32x4{pack2<F16>(x[0], x[1]), pack2<F16>(x[2], x[3]), pack2<F16>(x[4], x[5]), pack2<F16>(x[6], x[7])};
}

// src row -> dst row (may be the same), rotated at position pos when R > 0.
template <bool F16>
__device__ __forceinline__ void rotary_row(const uint16_t* src, uint16_t* dst, int D, int pos, const RotaryArgs& r,
                                           int lane) {
  const int e0 = lane * 8;
  if (e0 >= D) return;
  const u32x4 v = *(const u32x4*)(src + e0);
  if (r.dim == 0 || e0 >= r.dim) {  // a chunk past the rotary dims
    *(u32x4*)(dst + e0) = v;
    return;
  }
  const int half = r.dim / 2;
  const int p = min(max(pos, 0), r.seqlen_ro - 1);  // positions past the table read its last row
  const float* cs = r.cos + (int64_t)p * half;
  const float* sn = r.sin + (int64_t)p * half;
  float x[8];
  unpack8<F16>(v, x);
  if (r.interleaved) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float c = cs[e0 / 2 + j], s = sn[e0 / 2 + j], a = x[2 * j], b = x[2 * j + 1];
      x[2 * j] = a * c - b * s;
      x[2 * j + 1] = a * s + b * c;
    }
    *(u32x4*)(dst + e0) = pack8<F16>(x);
  } else {
    if (e0 >= half) return;  // the lane of the lower half writes this chunk
    float y[8];
    unpack8<F16>(*(const u32x4*)(src + e0 + half), y);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float c = cs[e0 + j], s = sn[e0 + j], a = x[j], b = y[j];
      x[j] = a * c - b * s;
      y[j] = a * s + b * c;
    }
    *(u32x4*)(dst + e0) = pack8<F16>(x);
    *(u32x4*)(dst + e0 + half) = pack8<F16>(y);
  }
}

// x [B, S, H, D] -> out (may alias x): token i of batch b at position
// pos0[b] + (per_token ? i : 0).
template <bool F16>
__global__ __launch_bounds__(THREADS) void rotary_kernel(const uint16_t* x, uint16_t* out, int64_t rows, int S, int H,
                                                          int D, const int32_t* pos0, int per_token, RotaryArgs r) {
  int chunk;
  const int slot = row_slot(D, chunk);
  const int64_t row = (int64_t)blockIdx.x * rows_per_block(D) + slot;
  if (slot < 0 || row >= rows) return;
  const int64_t tok = row / H;
  const int b = (int)(tok / S), i = (int)(tok - (int64_t)b * S);
  rotary_row<F16>(x + row * D, out + row * D, D, pos0[b] + (per_token ? i : 0), r, chunk);
}

// New token i of slot b, kv head h -> key position len[b] + i of the slot;
// keys rotated there, values copied.  Rows past the slot are dropped.
template <bool F16>
__global__ __launch_bounds__(THREADS) void append_kernel(AppendArgs a) {
  int lane;  // this thread's chunk of the row
  const int slot = row_slot(a.D, lane);
  const int64_t row = (int64_t)blockIdx.x * rows_per_block(a.D) + slot;
  if (slot < 0 || row >= a.rows) return;
  const int h = (int)(row % a.hkv);
  const int64_t tok = row / a.hkv;
  const int b = (int)(tok / a.seqlen_new), i = (int)(tok - (int64_t)b * a.seqlen_new);
  const int64_t pos = (int64_t)a.seqlens[b] + i;
  int64_t crow;  // row of the cache tensor ([slot or page][rows][hkv][D])
  if (a.block_table) {
    const int64_t page = pos / a.page_rows;
    if (pos < 0 || page >= a.pages_per_seq) return;
    crow = (int64_t)a.block_table[(int64_t)b * a.pages_per_seq + page] * a.page_rows + pos % a.page_rows;
  } else {
    if (pos < 0 || pos >= a.capacity) return;
    crow = (int64_t)b * a.capacity + pos;
  }
  const int64_t dst = (crow * a.hkv + h) * a.D, src = row * a.D;
  rotary_row<F16>(a.k_new + src, a.k_cache + dst, a.D, (int)pos, a.rot, lane);
  if (lane * 8 < a.D) *(u32x4*)(a.v_cache + dst + lane * 8) = *(const u32x4*)(a.v_new + src + lane * 8);
}

__global__ void grow_lengths_kernel(const int32_t* in, int32_t* out, int n, int add) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < n) out[b] = in[b] + add;
}

}  // namespace

hipError_t launch_rotary(const void* x, void* out, int64_t rows, int S, int H, int D, const int32_t* pos0,
                         int per_token, const RotaryArgs& r, bool f16, hipStream_t st) {
  const dim3 grid((unsigned)((rows + rows_per_block(D) - 1) / rows_per_block(D)));
  if (f16)
    hipLaunchKernelGGL(rotary_kernel<true>, grid, dim3(THREADS), 0, st, (const uint16_t*)x, (uint16_t*)out, rows, S,
                       H, D, pos0, per_token, r);
  else
    hipLaunchKernelGGL(rotary_kernel<false>, grid, dim3(THREADS), 0, st, (const uint16_t*)x, (uint16_t*)out, rows, S,
                       H, D, pos0, per_token, r);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int32_t* seqlens_out, bool f16, hipStream_t st) {
  const dim3 grid((unsigned)((a.rows + rows_per_block(a.D) - 1) / rows_per_block(a.D)));
  if (f16) hipLaunchKernelGGL(append_kernel<true>, grid, dim3(THREADS), 0, st, a);
  else hipLaunchKernelGGL(append_kernel<false>, grid, dim3(THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !seqlens_out) return e;
  // after the append (stream order), so seqlens_out may be the input array
  hipLaunchKernelGGL(grow_lengths_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, st, a.seqlens, seqlens_out,
                     a.batch, a.seqlen_new);
  return hipGetLastError();
}

}  // namespace attn
