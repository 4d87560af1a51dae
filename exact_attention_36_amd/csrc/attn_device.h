// attn_device.h -- gfx950 device helpers shared by the attention kernels:
// MFMA operand types, buffer resources (hardware bounds checks: loads past
// the end return 0, stores past the end are dropped), LDS swizzle, the
// transposing LDS read, cross-half wave reductions and 16-bit conversions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_{bf16,f16}: A is 32(M) x 16(K), B is 16(K) x 32(N).
// Lane l holds A[m = l%32][k = 8*(l/32) .. +7] and B[k = 8*(l/32) .. +7][n = l%32];
// accumulator register i of lane l is C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32].
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
// Two floats -> two 16-bit values packed in one dword, round to nearest even
// (one v_cvt_pk_{bf16,f16}_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v{lo, hi};
  if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 8 bf16 values -> the same 8 values as fp16 (exact inside fp16's normal
// range; rounded to nearest even below it, +-inf above 65504).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const float lo = __builtin_bit_cast(float, x[e] << 16), hi = __builtin_bit_cast(float, x[e] & 0xFFFF0000u);
    r[e] = pack2<true>(lo, hi);
  }
  return r;
}

template <bool F16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, h);
  else return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer with `bytes` valid bytes from `base`; dword 3 is the gfx9-family
// default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
// The kernels' 16-byte stores write output rows (O, dQ, dK, dV) that no
// workgroup of the same kernel reads again: they carry the non-temporal hint
// (cache-policy bit 1), which keeps them from displacing the shared K/V and
// Q/dO tiles in L2 (the windowed GQA backward's dK/dV kernel measured 3 %
// faster with it, the other kernels unchanged or slightly faster).
__device__ __forceinline__ void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
}
// 16 bytes straight from global memory into LDS (buffer_load ... lds): lane
// l's bytes land at M0 + 16*l, M0 = the wave-uniform LDS address.  Issued
// through inline assembly so that the compiler does not track it: the compiler cannot tell which LDS buffer a DMA
// writes and would otherwise wait for every outstanding DMA before any later
// LDS read, serialising the prefetch.  Callers order these copies with
// explicit wait_vmcnt + s_barrier.  The descriptor is a raw buffer
// (base, 0 stride, size in bytes, gfx9 dword 3), bounds-checked by hardware.
// M0 is set inside the statement; the compiler does not preserve M0 across
// it, and no other instruction of these kernels uses M0 (the only M0
// references in their generated code are these writes).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4{(int32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu),
               (int32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
// LDS byte address of a pointer into a __shared__ array: a generic pointer to
// LDS carries the aperture in its high half and the LDS offset in its low half.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
// NT: the non-temporal hint, for data read once (a K/V tile that no other
// workgroup reads): it keeps the stream from being allocated in the caches
// as reusable, which measured ~15 % more read bandwidth than the default
// policy on a streaming read of the decode shape's 4.3 GB.
template <bool NT = false>
__device__ __forceinline__ void dma_lds16(i32x4 rsrc, const void* lds_base, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(off), "s"(rsrc)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(rsrc)
                 : "memory", "m0");
}

// ---------------------------------------------------------------- LDS tiles
// A [rows][D] 16-bit tile is stored with 16-byte chunk c of row r at chunk
// position c ^ swz(r).  The two access patterns of the kernels -- 16 lanes
// reading one chunk of 16 consecutive rows, and the transposing read of 4
// consecutive rows x 4 consecutive chunks by 32 lanes -- then touch every
// one of the 64 banks exactly once.  A 256-wide row (512 bytes) spans the
// banks twice, like a 128-wide row spans them once, so it takes the same
// swizzle of the low four chunk bits.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  if constexpr (D >= 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ constexpr int tile_off(int r, int chunk) {  // byte offset of a chunk
  return r * (D * 2) + ((chunk ^ swz<D>(r)) << 4);
}

// Rows held MFMA-style by a wave -- lane l32 holds row l32, register i of
// block d holds column 32 d + 8 (i/4) + 4 hh + i%4 -- scaled, rounded to 16
// bits and stored through LDS so that every store instruction writes whole
// rows: the wave's 32 rows go to `stage` (32 rows x 2D bytes, swizzled like
// the K/V tiles) and come back 16 bytes per lane.  row_off(r) is the byte
// offset of row r in the descriptor, or DROP_ROW for a row not to store (the
// chunk offsets added to it stay past any descriptor's end); only the first
// dg columns of a row are stored.  Only this wave touches `stage`.
constexpr uint32_t DROP_ROW = 0x80000000u;
// Byte offset of 16-byte chunk ch of a row that starts at row_byte, for a
// tensor whose rows hold dg (a multiple of 8) 16-bit values: a chunk past dg
// gets DROP_ROW instead, so a buffer load of it reads zero and a store of it
// is dropped (the zero columns of a tile wider than the head dim).
__device__ __forceinline__ uint32_t chunk_off(uint32_t row_byte, int ch, int dg) {
  return ch * 8 < dg ? row_byte + (uint32_t)(ch * 16) : DROP_ROW;
}
template <int D, bool F16, class RowOff>
__device__ __forceinline__ void store_rows16(const f32x16 (&v)[D / 32], float scale, char* stage,
                                             __amdgpu_buffer_rsrc_t rs, RowOff row_off, int dg);

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes every lane supplies the address of 4 consecutive 16-bit values; lane
// i receives, as its element e (e = 0..3), value i%4 of the 4 values
// addressed by lane 4e + i/4.  With lane 4e+j pointing at row kbase+e,
// columns cbase+4j .. +3 of a row-major tile, lane i therefore receives
// column cbase+i of rows kbase .. kbase+3.
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 lds_read16(const void* p) { return *LDS_PTR(const u32x4, p); }

template <int D, bool F16, class RowOff>
__device__ __forceinline__ void store_rows16(const f32x16 (&v)[D / 32], float scale, char* stage,
                                             __amdgpu_buffer_rsrc_t rs, RowOff row_off, int dg) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int d = 0; d < D / 32; d++)
#pragma unroll
    for (int j4 = 0; j4 < 4; j4++)
      *LDS_PTR(u32x2, stage + tile_off<D>(l32, 4 * d + j4) + 8 * hh) =
          u32x2{pack2<F16>(v[d][4 * j4] * scale, v[d][4 * j4 + 1] * scale),
                pack2<F16>(v[d][4 * j4 + 2] * scale, v[d][4 * j4 + 3] * scale)};
  constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < 32 / (64 / CPR); it++) {
    const int r = it * (64 / CPR) + lane / CPR, ch = lane % CPR;
    buf_store16(*LDS_PTR(const u32x4, stage + tile_off<D>(r, ch)), rs, chunk_off(row_off(r), ch, dg));
  }
}

// ---------------------------------------------------------------- wave reductions
// Lanes l and l^32 exchange a value; returns op(own, partner) on every lane.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Barrier ahead of LDS that the workgroup refills right after it.  The
// wave's own LDS reads must have returned first: the compiler may issue an
// operand read before the barrier and schedule the MFMA that consumes it
// after, and s_barrier does not wait for reads in flight, so without the
// wait the DMA that another wave issues right after the barrier could
// overwrite the buffer before such a read returns.  Loads from global memory
// in flight (the DMA prefetches) are not waited for.
__device__ __forceinline__ void barrier_reads_done() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
}

// Instruction-scheduling hints (sched_group_barrier masks): the compiler
// otherwise issues each LDS operand read right before the MFMA that consumes
// it and waits out the LDS latency on every MFMA.
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100, SG_VALU = 0x002;
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
// `steps` MFMA steps of `m` MFMAs each consuming `r` LDS reads, with the reads
// issued `ahead` steps before their MFMAs.
template <int steps, int m, int r, int ahead>
__device__ __forceinline__ void sched_reads_ahead() {
  static_assert(ahead >= 1 && ahead <= steps, "prefetch distance");
  SCHED_GROUP(SG_DS_READ, r * ahead);
#pragma unroll
  for (int i = 0; i < steps - ahead; i++) {
    SCHED_GROUP(SG_MFMA, m);
    SCHED_GROUP(SG_DS_READ, r);
  }
  SCHED_GROUP(SG_MFMA, m * ahead);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- scheduling
// Workgroups are dealt to the 8 XCDs round robin.  Renumber them so that
// each XCD receives a contiguous range of logical ids (neighbouring tiles that
// share K/V then share an L2).
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = id % 8, slot = id / 8;
  // XCDs < rem own per+1 logical ids, the others own per.
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

// Batched grids of ngroups x nranks workgroups, where rank 0 is the heaviest
// block of a group.  With at least two groups per XCD, XCD x (which receives
// workgroups x, x+8, x+16, ...) owns groups [x*gpx, (x+1)*gpx) and runs their
// blocks heaviest rank first across those groups (longest-processing-time
// order, and the blocks that share a group's K/V share an L2).  When every
// rank does the same work (no mask), by_group runs an XCD's groups one after
// the other instead, all ranks of a group side by side, so that the blocks
// reading a group's K/V (or Q and dO) run together.  With fewer groups the
// order is simply rank-major over the whole chip.  Returns false for padding
// slots.  grid_size() gives the matching launch size.
struct GroupGrid {
  int ngroups, nranks;
  bool by_group = false;
  __host__ __device__ bool grouped() const { return ngroups >= 16; }
  __host__ __device__ int gpx() const { return (ngroups + 7) / 8; }
  __host__ __device__ long long grid_size() const {
    return grouped() ? 8LL * gpx() * nranks : (long long)ngroups * nranks;
  }
  __device__ __forceinline__ bool decode(int bid, int& group, int& rank) const {
    if (!grouped()) {
      rank = bid / ngroups;
      group = bid - rank * ngroups;
      return rank < nranks;
    }
    const int per = gpx();
    const int xcd = bid & 7, slot = bid >> 3;
    const int g0 = xcd * per;
    const int cnt = min(per, ngroups - g0);
    if (cnt <= 0 || slot >= cnt * nranks) return false;
    if (by_group) {
      const int gi = slot / nranks;
      rank = slot - gi * nranks;
      group = g0 + gi;
      return true;
    }
    rank = slot / cnt;
    group = g0 + (slot - rank * cnt);
    return true;
  }
};

}  // namespace attn
