// fa_common.hpp - device-side building blocks shared by the gfx950 attention
// kernels: vector types, MFMA fragment helpers, half-wave exchanges and the
// work-group -> (batch, head, query tile) schedule.
//
// MFMA lane layouts used throughout (wave64, checked on gfx950 hardware):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane l holds row l%32, k = 8*(l/32) + [0..7]
//                             B (16 x 32): lane l holds col l%32, k = 8*(l/32) + [0..7]
//                             C (32 x 32): lane l holds col l%32, rows
//                                          8*(v/4) + 4*(l/32) + v%4 for v = 0..15
//   v_mfma_f32_32x32x2_f32    A: row l%32, k = l/32;  B: col l%32, k = l/32;  C as above.
// The kernels compute transposed score tiles S^T = K Q^T so that each lane
// owns ONE query column of the C tile: a query's keys live in that lane and
// in lane l^32 only, which makes the row max a local max plus one half-wave
// exchange, and makes the C fragment of P^T directly usable as the B
// operand of the next contraction (with the key order permuted consistently
// in the A operand).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Lambdas inside kernels must be inlined: an outlined call passes the
// captured register state through scratch memory.
#define FA_INLINE __attribute__((always_inline))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of the 32x32 C tile held in register v of lane l (see layout above).
__device__ __forceinline__ int c_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// max / sum of a value with the same value in the other half of the wave
// (lane l and lane l^32).  v_permlane32_swap(x, x) leaves (own, other) in the
// lower half and (other, own) in the upper half, so one max/add finishes it.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzling); out-of-range offsets read as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Wait until every vector-memory load issued by this wave has completed,
// including loads whose destination is LDS.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work-group barrier for LDS traffic issued by ordinary LDS instructions:
// waits for this wave's LDS reads and writes, then for every wave.  Global
// loads still in flight, including loads whose destination is LDS, stay in
// flight across it (a fence would wait for those as well); their LDS data
// may be read only after wait_vmem() and a later barrier.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Key length of sequence b clamped to [0, N] (N when no lengths are given).
__device__ __forceinline__ int key_length(const int32_t* seqlens_k, int b, int N) {
  if (seqlens_k == nullptr) return N;
  int L = seqlens_k[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

// Work-group schedule.  Work-groups are numbered so that consecutive ids
// cover all (batch, head) pairs of one query tile; query tiles are issued
// from the last (the longest under a causal mask) to the first, so the
// dispatcher starts the long tiles first and fills the tail with short ones.
// Consecutive ids are dispatched round-robin over the 8 XCDs, so when B*H is
// a multiple of 8 every query tile of one head runs on the same XCD and the
// head's K/V tiles are shared through that XCD's L2.
struct TileCoord {
  int b, h, qt;
};
__device__ __forceinline__ TileCoord tile_coord(int wg, int B, int H, int n_qtiles) {
  const int bh_count = B * H;
  const int qt_rev = wg / bh_count;
  const int bh = wg - qt_rev * bh_count;
  TileCoord t;
  t.qt = n_qtiles - 1 - qt_rev;
  t.b = bh / H;
  t.h = bh - t.b * H;
  return t;
}

}  // namespace fa
