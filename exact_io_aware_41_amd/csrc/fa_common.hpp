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
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
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

// Bits p of a 32-bit word set iff p <= rel (none for rel < 0, all for
// rel >= 31): the visible positions of a run of 32 keys.
__device__ __forceinline__ uint32_t prefix_bits(int rel) {
  const int r = min(max(rel + 1, 0), 32);
  return (uint32_t)((1ull << r) - 1ull);
}

// x where bit `pos` (a constant) of `bits` is set, `other` elsewhere, by bit
// operations only (v_bfe_i32 gives 0 or -1, then a bitwise select): unlike a
// compare per element, this holds no lane masks in scalar registers.
__device__ __forceinline__ float keep_if_bit(float x, uint32_t bits, int pos, float other) {
  const int m = __builtin_amdgcn_sbfe((int)bits, pos, 1);
  return __int_as_float((__float_as_int(x) & m) | (__float_as_int(other) & ~m));
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

// The two 16-bit element formats of the MFMA kernels: storage type, 8- and
// 4-element vectors, the 32x32x16 MFMA with fp32 accumulation, and the
// round-to-nearest-even conversion from fp32.  Both formats use the same
// tiles, swizzles and transposing reads; only these operations differ.
struct EltBf16 {
  using T = __bf16;
  using V8 = bf16x8;
  using V4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T cvt(float x) { return (T)x; }
  // the two elements packed in a 32-bit word (low half first), widened
  static __device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
  // acc + x[j] + x[j + 1] in fp32 (v_dot2c_f32_bf16 against (1, 1): the
  // products are exact, the sum is an fp32 accumulation)
  static __device__ __forceinline__ float sum2(V8 x, int j, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 v2;
    const v2 one = {(__bf16)1.0f, (__bf16)1.0f};
    const v2 pair = {x[j], x[j + 1]};
    return __builtin_amdgcn_fdot2_f32_bf16(pair, one, acc, false);
  }
};
struct EltF16 {
  using T = _Float16;
  using V8 = f16x8;
  using V4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T cvt(float x) { return (T)x; }
  static __device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // acc + x[j] + x[j + 1] in fp32 (v_dot2c_f32_f16 against (1, 1))
  static __device__ __forceinline__ float sum2(V8 x, int j, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 v2;
    const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
    const v2 pair = {x[j], x[j + 1]};
    return __builtin_amdgcn_fdot2(pair, one, acc, false);
  }
};

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzling); out-of-range offsets read as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Raw buffer descriptor of `bytes` bytes at `base` (gfx9 layout: 48-bit base,
// stride 0, num_records in bytes, word 3 as above), for inline assembly.
__device__ __forceinline__ u32x4 buffer_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = (uint32_t)kBufferRsrcWord3;
  return r;
}

// Buffer resource (pointer form) over `bytes` bytes at `base`, and the
// compiler-issued direct load of 16 bytes per lane into LDS at `lds_dst`
// (lane l writes bytes [16 l, 16 l + 16) of the wave's block).  Plain
// functions: a kernel template calls them instead of the target builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3);
}
// Debug builds (FA_LDS_POISON) fill the 16 bytes a lane's copy is about to
// write with all-ones (NaN in every element format of the library) just
// before issuing it, i.e. after the slot's last reader passed the barrier
// that frees it.  A reader that runs ahead of the copy's wait and barrier, or
// a copy issued while a slow reader still uses the slot, then sees NaN, which
// the parity tests reject.
#ifndef FA_LDS_POISON
#define FA_LDS_POISON 0
#endif
__device__ __forceinline__ void poison_lds16(uint32_t lds_base) {
#if FA_LDS_POISON
  auto* p = (__attribute__((address_space(3))) u32x4*)(uintptr_t)(lds_base + 16u * (threadIdx.x & 63));
  *p = u32x4{~0u, ~0u, ~0u, ~0u};
  // the poison must land before the copy's data
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#else
  (void)lds_base;
#endif
}

__device__ __forceinline__ void lds_dma16_tracked(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst,
                                                  int voff) {
  poison_lds16(__builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)lds_dst)));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}

// Direct load of 16 bytes per lane into LDS (buffer_load_dwordx4 ... lds):
// lane l writes bytes [16 l, 16 l + 16) after the wave-uniform LDS address
// `lds`, from byte voff + soff of the buffer; out-of-range reads give zeros.
// Issued by inline assembly: the compiler neither counts it nor orders LDS
// accesses against it, so the caller must wait_vmem() and pass a barrier
// before anything reads the destination.  (Issued through the builtin, the
// compiler makes the next LDS read wait for the whole copy.)
__device__ __forceinline__ void lds_dma16_at(const u32x4& rsrc, uint32_t lds, int voff, int soff) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  poison_lds16(base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(base), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// 32-bit LDS address of a __shared__ object.  Taken once from the object
// itself, it lets callers form slot addresses with integer arithmetic instead
// of casting generic pointers back to LDS (each such cast carries a null test).
template <class T>
__device__ __forceinline__ uint32_t lds_address(const T* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, const void* lds, int voff, int soff) {
  lds_dma16_at(rsrc, lds_address(static_cast<const char*>(lds)), voff, soff);
}

// Wait until every vector-memory load issued by this wave has completed,
// including loads whose destination is LDS.
// The builtin form is visible to the compiler's own counter tracking, which
// then knows nothing is outstanding (s_waitcnt simm16 on gfx9: vmcnt bits 3:0
// and 15:14 = 0, expcnt bits 6:4 = 7, lgkmcnt bits 11:8 = 15).
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Work-group barrier for LDS traffic issued by ordinary LDS instructions:
// waits for this wave's LDS reads and writes, then for every wave.  Global
// loads still in flight, including loads whose destination is LDS, stay in
// flight across it (a fence would wait for those as well); their LDS data
// may be read only after wait_vmem() and a later barrier.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row-major tiles read both ways - 16-row fragments by ds_read_b128 and
// column fragments by transposing reads (16 lanes: 4 consecutive rows x 32
// bytes; a wave half: 4 rows x 64 bytes, served as 32 lanes per cycle) -
// XOR their 16-byte chunk index with a linear map of the row bits that is
// one-to-one on every lane group of both access kinds (searched exhaustively
// under the measured grouping rules).  Rows of d = 96 and 192 (192 and 384
// bytes) are not whole bank periods; their maps change only the low 2 or 3
// bits of the chunk index, so a chunk stays inside its aligned group of 4 or
// 8 of the row's 12 or 24 chunks.
template <int D>
__device__ __forceinline__ int tile_swizzle(int row) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dimension");
  if constexpr (D == 128 || D == 256)
    return ((row & 3) << 2) ^ ((row >> 2) & 3) ^ (((row >> 4) & 1) * 3);
  else if constexpr (D == 192)
    return (((row >> 1) & 1) << 2) | ((row >> 3) & 3);
  else if constexpr (D == 96)
    return (row >> 3) & 3;
  else
    return (((row >> 1) & 1) << 2) ^ ((row >> 3) & 1) ^ (((row >> 4) & 1) << 1);
}

// Row-major tiles are stored unpadded with their 16-byte chunks XOR-swizzled
// by a function of the row.  On gfx950 a ds_read_b128 serves lanes 0-31 and
// 32-63 in different cycles, and within a half two groups of 16 lanes
// (split by the parity of lane bits 2..4, e.g. lanes 0-3, 12-15, 20-23,
// 24-27); LDS banks repeat every 256 bytes.  A read is conflict-free when
// the 16 lanes of a group touch 16 distinct 16-byte bank slots.  For d = 128
// (one 256-byte row per bank period) the swizzle below is a linear map of
// the row bits that is one-to-one on every such group, both for fragment
// reads (lane l reads row 32 b + l % 32) and for the transposition reads
// (16 lanes read rows 4 q + r of consecutive 4-row groups q, two chunk
// columns), so neither has conflicts.  For d = 64 the fragment reads are
// conflict-free; the transposition reads conflict two ways (two rows share
// a bank period, leaving 8 slots for 16 lanes).
template <int D>
__device__ __forceinline__ int row_swizzle(int row) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dimension");
  // d = 256: rows of 512 bytes repeat the 256-byte bank pattern, so the
  // d = 128 XOR of the low four chunk bits serves unchanged
  if constexpr (D == 128 || D == 256)
    return (row & 15) ^ (((row >> 4) & 1) * 12) ^ (((row >> 5) & 1) * 2);
  // d = 96 and 192: the map that also serves transposing reads (below) is
  // conflict-free for these fragment reads as well
  else if constexpr (D == 96 || D == 192)
    return tile_swizzle<D>(row);
  else
    return (row ^ (row >> 2)) & (D / 8 - 1);
}

// Row-major tiles read only by transposing reads (ds_read_b64_tr_b16) swizzle
// their 64-byte segments instead: 16 lanes of such a read fetch 4 consecutive
// rows x 32 bytes and a wave half 4 rows x 64 bytes; XOR-ing the segment
// index with the row's position inside its group of four rows (d = 128,
// 256-byte rows) or of two row pairs (d = 64, 128-byte rows) puts those
// 4 x 64 bytes on 4 distinct 64-byte bank ranges (measured conflict-free).
template <int D>
__device__ __forceinline__ int seg_swizzle(int row) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dimension");
  if constexpr (D == 128 || D == 256)
    return row & 3;
  else if constexpr (D == 192)   // 384-byte rows: row bit 0 already alternates bank halves
    return (row >> 1) & 1;
  else if constexpr (D == 96)    // 192-byte rows: four rows already fall on four 64-byte ranges
    return 0;
  else
    return (row >> 1) & 1;
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8-byte chunks addressed by lanes i / 4 + 4 j, j = 0..3.  With lane s
// addressing row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3, lane i receives
// column c0 + i of rows r0 .. r0 + 3.
template <typename T>
__device__ __forceinline__ s16x4 read_tr16(const T* p) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<T*>(p)));
}

// Key length of sequence b clamped to [0, N] (N when no lengths are given).
__device__ __forceinline__ int key_length(const int32_t* seqlens_k, int b, int N) {
  if (seqlens_k == nullptr) return N;
  int L = seqlens_k[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

// Work-group schedule.  A launch has n_tiles work-groups per (batch, head)
// pair, and a tile's rank orders them longest first (the last query tile
// under a causal mask, the first key tile in the dK/dV kernel), so that the
// dispatcher starts the long tiles first and fills the tail with short ones.
// Ids are dispatched round-robin over the 8 XCDs (id % 8), each with its own
// L2.  When B*H is a multiple of 8, XCD x takes heads x, x + 8, x + 16, ...
// in groups of FA_XCD_GROUP heads, one group after the other, and runs a
// group's tiles rank by rank: the XCD's CUs then work on few heads at a time,
// stream the same K and V rows at about the same time and share them
// through the XCD's L2, while each group still runs longest first.
// Otherwise consecutive ids cover every head at one rank before the next.
#ifndef FA_XCD_GROUP
#define FA_XCD_GROUP 2
#endif
struct WgOrder {
  int bh, rank;
};

// Debug builds (FA_WG_PERMUTE) visit the work-group ids in a scrambled
// order, id -> id * P mod n for a prime P (n the number of ids; the reversed
// order when P divides n).  Every kernel computes each tile independently of
// the others, so results must not change by a single bit.
#ifndef FA_WG_PERMUTE
#define FA_WG_PERMUTE 0
#endif
constexpr bool is_prime(unsigned n) {
  if (n < 2) return false;
  for (unsigned p = 2; p * p <= n; ++p)
    if (n % p == 0) return false;
  return true;
}
__device__ __forceinline__ int scheduled_wg(int wg, unsigned n) {
#if FA_WG_PERMUTE
  constexpr unsigned kP = 40009u;
  static_assert(is_prime(kP), "id -> id * P mod n is a permutation only for P coprime with n");
  if (n % kP != 0) return (int)(((unsigned long long)(unsigned)wg * kP) % n);
  return (int)(n - 1u - (unsigned)wg);
#else
  return wg;
#endif
}

__device__ __forceinline__ WgOrder wg_order(int wg_id, int bh_count, int n_tiles) {
  const int wg = scheduled_wg(wg_id, (unsigned)bh_count * (unsigned)n_tiles);
  WgOrder o;
  if (FA_XCD_GROUP > 0 && (bh_count & 7) == 0) {
    const int x = wg & 7, k = wg >> 3;
    const int heads = bh_count >> 3;                  // heads of this XCD
    const int span = FA_XCD_GROUP * n_tiles;          // ids of a full group
    const int full = heads / FA_XCD_GROUP;            // full groups
    int g = k / span;
    int size = FA_XCD_GROUP;
    if (g >= full) {                                  // the last, smaller group
      g = full;
      size = heads - full * FA_XCD_GROUP;
    }
    const int j = k - g * span;
    o.rank = j / size;
    o.bh = x + 8 * (g * FA_XCD_GROUP + (j - o.rank * size));
  } else {
    o.rank = wg / bh_count;
    o.bh = wg - o.rank * bh_count;
  }
  return o;
}

// Persistent kernels (one work-group per slot running a list of tiles) take
// their arguments as one struct, which sits at the start of the
// kernel-argument segment, and read the fields where each job needs them.
// The segment pointer goes through an opaque copy, so the compiler issues
// those scalar loads again per job instead of holding every argument in
// scalar registers across the whole job loop.
template <class A>
__device__ __forceinline__ const __attribute__((address_space(4))) A* job_args() {
  const unsigned long long u = (unsigned long long)__builtin_amdgcn_kernarg_segment_ptr();
  unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  unsigned up = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  asm volatile("" : "+s"(lo), "+s"(up));
  lo = __builtin_amdgcn_readfirstlane(lo);
  up = __builtin_amdgcn_readfirstlane(up);
  return (const __attribute__((address_space(4))) A*)(((unsigned long long)up << 32) | lo);
}
// A pointer read from that struct, marked as global memory again (pointer
// kernel arguments are; pointers loaded from memory are not)
template <typename T>
__device__ __forceinline__ T* global_ptr(T* p) {
  return (T*)(__attribute__((address_space(1))) T*)p;
}

// Job j of a persistent launch with `slots` work-groups (a multiple of 8,
// one per XCD lane): work-group w runs on XCD w % 8 and takes that XCD's ids
// k = 0, 1, ... (job k * 8 + w % 8) in passes of slots / 8, alternating the
// direction of each pass, so that with the ids ordered longest first every
// work-group's list adds up to about the same work.  Returns -1 past the end.
__device__ __forceinline__ int persistent_job(int pass, int n_jobs) {
  const int per_xcd = (int)(gridDim.x >> 3);
  const int x = (int)(blockIdx.x & 7u), i = (int)(blockIdx.x >> 3);
  const int k = pass * per_xcd + ((pass & 1) ? per_xcd - 1 - i : i);
  const long long j = (long long)k * 8 + x;
  return j < n_jobs ? (int)j : -1;
}

struct TileCoord {
  int b, h, qt;
};

// Query-tile work-groups: the longest is the last query tile.
__device__ __forceinline__ TileCoord tile_coord(int wg, int B, int H, int n_qtiles) {
  const WgOrder o = wg_order(wg, B * H, n_qtiles);
  TileCoord t;
  t.qt = n_qtiles - 1 - o.rank;
  t.b = o.bh / H;
  t.h = o.bh - t.b * H;
  return t;
}

// Where the rows of one (sequence b, head h) live.  Padded layout
// (cu_q == nullptr): [B][H][N][d] queries and [B][H][Nk][d] keys, every
// sequence N query rows and Nk key rows.  Packed layout: sequence b owns
// query rows cu_q[b] .. cu_q[b+1] of head h in [H][total_q][d] and key rows
// cu_k[b] .. cu_k[b+1] of [H][total_k][d] (lse and the row statistics
// [H][total_q]); offsets and lengths are clamped to the buffers and to
// N / Nk (the longest sequences the launch covers), so malformed offsets
// cannot move an access outside them.
struct SeqSpan {
  size_t q_row0, k_row0;   // first query / key row, in rows
  int nq, nk;              // query / key rows of this sequence
};
__device__ __forceinline__ SeqSpan seq_span(int b, int h, int H, int N, int Nk,
                                            const int32_t* cu_q, const int32_t* cu_k,
                                            int total_q, int total_k) {
  SeqSpan s;
  if (cu_q == nullptr) {
    const size_t head = (size_t)b * H + h;
    s.q_row0 = head * (size_t)N;
    s.k_row0 = head * (size_t)Nk;
    s.nq = N;
    s.nk = Nk;
    return s;
  }
  const int q_lo = min(max(cu_q[b], 0), total_q);
  const int k_lo = min(max(cu_k[b], 0), total_k);
  s.nq = min(min(max(cu_q[b + 1] - q_lo, 0), total_q - q_lo), N);
  s.nk = min(min(max(cu_k[b + 1] - k_lo, 0), total_k - k_lo), Nk);
  s.q_row0 = (size_t)h * total_q + q_lo;
  s.k_row0 = (size_t)h * total_k + k_lo;
  return s;
}

}  // namespace fa
