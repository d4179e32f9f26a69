// fa_fwd_fp8.hip - forward kernel on FP8 (OCP E4M3) queries, keys and values.
//
// The method is the forward of fa_fwd.hip: running maximum m, running sum l
// of exp(s - m) and unnormalised output o per query row, rescaled by
// exp(m_old - m_new) whenever a key tile raises the maximum and divided by l
// after the last tile ("FlashAttention", section "Why it is allowed to be
// exact"; "Explain FlashAttention and why it is IO-aware", section "Keep only
// the state needed for the final weighted average").  The pages name an FP8
// forward for the newest kernels ("What is FlashAttention?", sections
// "Trade-offs and edge cases" and "What is FlashAttention 3?") without its
// scaling rules; here each input tensor carries one fp32
// descale factor (its real values are code * descale), the scores are those
// of the real values, and the output O is bf16.
//
// gfx950 mapping:
//  * both products run on v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands
//    (32 bytes per lane, twice the rate of the 16-bit MFMA).  The dot
//    products of E4M3 values accumulate in fp32.
//  * S^T = K Q^T: Q stays in VGPRs as the B operand (lane l: query l % 32,
//    feature bytes [64 ks + 32 (l / 32), +32)); the A operand reads K rows
//    from LDS in a permuted order, so that lane half h of the accumulators
//    holds keys 16 h .. 16 h + 15 of each 32-key block in register order.
//  * P^T = exp2(x - m + 8) (the factor 256 moves P into the normal range of
//    E4M3; it cancels against the same factor in l) is converted to E4M3 and
//    packed straight into the B operand of O^T = V^T P^T: bytes 0..15 of a
//    lane are the keys of one 32-key block, bytes 16..31 those of the next.
//  * V^T fragments come from transposing LDS reads (ds_read_b64_tr_b8: a
//    16-lane group reads 8 rows x 16 bytes and lane i receives byte i of
//    each row), four per MFMA, in exactly that key order.
//  * K and V tiles (128 keys) go from HBM straight into LDS (buffer loads with
//    an LDS destination, 16 bytes per lane, 1 KiB per wave instruction), two
//    tiles ahead in a three-slot ring, so a copy has two tiles of compute to
//    land; the buffer descriptors end at the sequence's key length, so keys
//    past it read as zeros.  16-byte chunks are XOR-swizzled by row (each lane
//    fetches the chunk that belongs at its LDS position) so that both the K
//    fragment reads and the transposing V reads are free of bank conflicts.
//  * l is kept per lane over its own keys and combined with the partner lane
//    once, after the last tile; the running maximum is exchanged per tile.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kFp8NW = 8;     // waves per work-group, 32 query rows each
constexpr int kFp8BC = 128;   // keys per K/V tile

// E4M3 x E4M3 -> fp32, 32 x 32 outputs, 64-deep; format code 0 on both
// operands and no block scales (the plain MFMA).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four floats -> four E4M3 bytes (round to nearest even), first in the low byte.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Transposing read of 8 bytes: see the file header.
__device__ __forceinline__ i32x2 read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(const_cast<uint8_t*>(p)));
}

// Row-major [keys][128] byte tiles: the 16-byte chunk c of row r is stored at
// chunk c ^ swz(r).  Searched exhaustively: one-to-one on the 16-lane groups
// of the fragment reads (rows in the permuted order below, one chunk) and on
// the 32-lane halves of the transposing reads (8 consecutive rows, two
// chunks).
__device__ __forceinline__ int fp8_swz(int row) {
  return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}
__device__ __forceinline__ int fp8_off(int row, int chunk) {
  return row * 128 + ((chunk ^ fp8_swz(row)) & 7) * 16;
}

// K row read by A-operand row m of a 32-key block: accumulator lane half h
// then holds keys 16 h + v (v = register 0..15), see c_row.
__device__ __forceinline__ int key_perm(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

template <int D, int NW, int BC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                       const uint8_t* __restrict__ V, const int32_t* __restrict__ seqlens_k,
                       float qk_log2, float v_descale, int causal, __bf16* __restrict__ O,
                       float* __restrict__ LSE, int B, int H, int N, int Nk, int n_qtiles) {
  static_assert(D == 128, "FP8 tiles are laid out for 128-byte rows");
  constexpr int BR = NW * 32;
  constexpr int KS = D / 64;                      // k-steps of one S MFMA chain
  constexpr int NSB = BC / 32;                    // 32-key blocks per tile
  constexpr int NPV = BC / 64;                    // 64-key steps of O^T = V^T P^T
  constexpr int NDB = D / 32;                     // 32-feature blocks of O^T
  constexpr int TILE = BC * D;                    // bytes per K or V tile
  constexpr int SLOTS = 3;                        // ring depth: copies run two tiles ahead
  constexpr int kBlks = TILE / 1024;              // 1 KiB copy blocks per tensor and tile
  constexpr int kBlksPerWave = 2 * kBlks / NW;
  static_assert(kBlksPerWave * NW == 2 * kBlks, "whole copy blocks per wave");
  __shared__ __attribute__((aligned(16))) uint8_t Ks[SLOTS][TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[SLOTS][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_coord(blockIdx.x, B, H, n_qtiles);
  const size_t head = (size_t)tc.b * H + tc.h;
  const uint8_t* Qh = Q + head * (size_t)N * D;
  const uint8_t* Kh = K + head * (size_t)Nk * D;
  const uint8_t* Vh = V + head * (size_t)Nk * D;
  __bf16* Oh = O + head * (size_t)N * D;
  float* Lh = LSE + head * (size_t)N;

  const int kv_len = key_length(seqlens_k, tc.b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int q0 = tc.qt * BR;
  const int qw0 = q0 + wave * 32;
  const int query = qw0 + l32;
  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, max(0, min(q0 + BR + off, Nk)));
  const int n_kt = (kv_end + BC - 1) / BC;

  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (query < N) {
      const u32x4* src = reinterpret_cast<const u32x4*>(Qh + (size_t)query * D + 64 * ks + 32 * hi);
      const u32x4 a = src[0], b = src[1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        qf[ks][w] = (int)a[w];
        qf[ks][4 + w] = (int)b[w];
      }
    } else {
      qf[ks] = i32x8{};
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = kNegInf;   // running maximum of x = score * log2(e), this lane's query
  float l = 0.f;       // this lane's share of the running sum of 2^(x - m + 8)

  // The Q fragments must have landed before the loop: the tile copies are
  // issued outside the compiler's counter tracking, so a wait it placed for Q
  // inside the loop would also wait for copies in flight.
  wait_vmem();

  // Copies: wave w fills 1 KiB blocks w * kBlksPerWave + j (K blocks first,
  // then V) of each tile; lane l writes bytes [16 l, 16 l + 16) of a block,
  // row 8 b + l / 8, LDS chunk l % 8, so it fetches global chunk
  // (l % 8) ^ swz(row).  Keys at or past the key length read as zeros (the
  // descriptors end there), which also keeps whatever lies past it out of
  // 0 * x products.
  const u32x4 k_rsrc = buffer_rsrc_words(Kh, (uint32_t)(kv_len * D));
  const u32x4 v_rsrc = buffer_rsrc_words(Vh, (uint32_t)(kv_len * D));
  int voff[kBlksPerWave];
#pragma unroll
  for (int j = 0; j < kBlksPerWave; ++j) {
    const int rb = (wave * kBlksPerWave + j) % kBlks;
    const int row = rb * 8 + lane / 8;
    voff[j] = row * D + ((lane % 8) ^ fp8_swz(row)) * 16;
  }
  auto issue_tile = [&](int kt) FA_INLINE {
    const int slot = kt % SLOTS;
#pragma unroll
    for (int j = 0; j < kBlksPerWave; ++j) {
      const int blk = wave * kBlksPerWave + j;
      const bool is_k = blk < kBlks;
      uint8_t* dst = (is_k ? Ks[slot] : Vs[slot]) + (blk % kBlks) * 1024;
      lds_dma16(is_k ? k_rsrc : v_rsrc, dst, voff[j], kt * BC * D);
    }
  };
  if (n_kt > 0) issue_tile(0);
  if (n_kt > 1) issue_tile(1);

  // Loop-invariant parts of the LDS addresses.  K fragments: row
  // 32 sb + key_perm(l32), chunks 4 ks + 2 hi + e; the swizzle only sees row
  // bits 1..3, which key_perm fixes per lane, so 32 sb enters as an offset.
  const int krow = key_perm(l32);
  int k_at[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) k_at[ks][e] = fp8_off(krow, 4 * ks + 2 * hi + e);
  // Transposing reads: lane i of a 16-lane group addresses row i / 2 of an
  // 8-row slab, bytes 8 (i % 2) .. of the 16-byte chunk of its feature half.
  // Slab t of a 64-key step starts at row 32 (t / 2) + 16 hi + 8 (t % 2); the
  // swizzle sees row bits 1..3, i.e. the lane's row in the slab and t % 2.
  const int tr_row = (lane & 15) >> 1;
  int v_at[2][NDB];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      v_at[par][db] = fp8_off(16 * hi + 8 * par + tr_row, 2 * db + ((lane >> 4) & 1)) +
                      (lane & 1) * 8;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt % SLOTS;
    // this wave's copies of tile kt have landed once at most those of tile
    // kt + 1 are outstanding (loads complete in order); after the barrier
    // every wave's have, and every wave has finished reading the slot that
    // tile kt + 2 goes to (tile kt - 1's)
    if (kt + 1 < n_kt)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kBlksPerWave);   // vmcnt(kBlksPerWave)
    else
      wait_vmem();
    asm volatile("" ::: "memory");
    lds_barrier();
    if (kt + 2 < n_kt) issue_tile(kt + 2);
    const int key0 = kt * BC;
    const bool active = qw0 < N && (!causal || key0 <= qw0 + 31 + off);
    if (active) {
      const uint8_t* Kt = Ks[buf];
      const uint8_t* Vt = Vs[buf];
      f32x16 s[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(Kt + 32 * sb * D + k_at[ks][0]);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(Kt + 32 * sb * D + k_at[ks][1]);
          i32x8 a;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            a[w] = (int)a0[w];
            a[4 + w] = (int)a1[w];
          }
          s[sb] = mfma_fp8(a, qf[ks], s[sb]);
        }
      }

      // mask on absolute positions where the tile crosses the key length or
      // this wave's causal limit: key key0 + 32 sb + 16 hi + v is visible iff
      // it is at most lim, bit v of a per-lane prefix mask
      const bool need_mask =
          key0 + BC > kv_len || (causal && key0 + BC - 1 > qw0 + off);
      if (need_mask) {
        const int lim = (causal ? min(kv_len - 1, query + off) : kv_len - 1) - key0 - 16 * hi;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
          const uint32_t vis = prefix_bits(lim - 32 * sb);
#pragma unroll
          for (int v = 0; v < 16; ++v) s[sb][v] = keep_if_bit(s[sb][v], vis, v, kNegInf);
        }
      }
      // the maximum of the raw scores (qk_log2 > 0), then x = s * qk_log2
      float mr = kNegInf;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mr = fmaxf(mr, s[sb][v]);
      const float m_new = fmaxf(m, halfwave_max(mr) * qk_log2);
      // rescale l and o only when some lane's maximum moved
      if (__builtin_amdgcn_ballot_w64(m_new != m) != 0) {
        const float alpha = fast_exp2(m - (m_new == kNegInf ? 0.f : m_new));
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        m = m_new;
      }
      // p = 2^(x - m + 8), one fma and one exp per score
      const float nb = 8.f - (m == kNegInf ? 0.f : m);
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(s[sb][v], qk_log2, nb));
          s[sb][v] = p;
          rs += p;
        }
      l += rs;

#pragma unroll
      for (int u = 0; u < NPV; ++u) {
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pb[w] = pack_fp8x4(s[2 * u][4 * w], s[2 * u][4 * w + 1], s[2 * u][4 * w + 2],
                             s[2 * u][4 * w + 3]);
          pb[4 + w] = pack_fp8x4(s[2 * u + 1][4 * w], s[2 * u + 1][4 * w + 1],
                                 s[2 * u + 1][4 * w + 2], s[2 * u + 1][4 * w + 3]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          i32x8 a;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            // bytes 8t.. of the operand: keys 64 u + 32 (t / 2) + 16 hi + 8 (t % 2) + 0..7
            const i32x2 r = read_tr8(Vt + (64 * u + 32 * (t >> 1)) * D + v_at[t & 1][db]);
            a[2 * t] = r[0];
            a[2 * t + 1] = r[1];
          }
          o[db] = mfma_fp8(a, pb, o[db]);
        }
      }
    }
  }

  // epilogue: each lane holds its query's features 32 db + c_row(v, lane)
  l = halfwave_sum(l);
  if (query < N) {
    const float inv = l > 0.f ? v_descale / l : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hi;
        EltBf16::V4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = EltBf16::cvt(o[db][4 * g + e] * inv);
        *reinterpret_cast<EltBf16::V4*>(Oh + (size_t)query * D + d0) = w;
      }
    if (hi == 0)
      Lh[query] = l > 0.f ? (m + __builtin_amdgcn_logf(l) - 8.f) * kLn2 : kNegInf;
  }
}

}  // namespace

long long fwd_fp8_grid(int B, int H, int N, int d) {
  (void)d;
  constexpr int BR = kFp8NW * 32;
  return (long long)((N + BR - 1) / BR) * B * H;
}

hipError_t launch_fwd_fp8(const FwdArgs& a, float q_descale, float k_descale, float v_descale) {
  if (a.d != 128) return hipErrorInvalidValue;
  constexpr int BR = kFp8NW * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const dim3 grid((unsigned)((long long)n_qtiles * a.B * a.H));
  const float qk_log2 = a.scale * q_descale * k_descale * kLog2e;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, kFp8NW, kFp8BC>), grid, dim3(kFp8NW * 64), 0,
                     a.stream, static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v), a.seqlens_k, qk_log2, v_descale, a.causal,
                     static_cast<__bf16*>(a.o), a.lse, a.B, a.H, a.N, a.Nk, n_qtiles);
  return hipGetLastError();
}

}  // namespace fa
