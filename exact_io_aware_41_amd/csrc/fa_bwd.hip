// fa_bwd.hip - backward kernels: gradients of <dO, O> by recomputation.
//
// Method ("What is FlashAttention?", Step 4; "FlashAttention", section "What
// it does not do"; "Explain FlashAttention and why it is IO-aware", section
// "Exact attention, finite precision and backward"): the forward keeps only
// O and one statistic per row (here LSE); the backward rebuilds the score
// and probability tiles on chip, P_ij = exp(s_ij - LSE_i), and never writes
// an N x N matrix.  With D_i = sum_t dO_it O_it and dS = P * (dP - D):
//   dV = P^T dO,  dP = dO V^T,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three launches on the caller's stream, no atomics (deterministic):
//  1. row dot products D (memory-bound, one pass over O and dO);
//  2. dK/dV: a work-group owns 128 keys of one (batch, head); a pair of waves
//     keeps 32 keys' K and V rows in VGPRs (B operands) and their dK/dV
//     accumulators resident, and loops over 64-row query tiles held row-major
//     in LDS: 16-row fragments are the A operands of S and dP, and
//     transposing reads (ds_read_b64_tr_b16) of the same tile give the B
//     operands of dV and dK with the rows in the order of the P fragment.  S
//     and dP come out with one key per lane, so P and dS feed the next MFMA
//     straight from registers.  Up to d = 128 the two waves of a pair run
//     half a tile apart (one computes exponentials while the other issues
//     MFMAs, section 2b); at d = 192 and 256 four waves run in step;
//  3. dQ: a work-group owns query rows (like the forward) and loops over key
//     tiles; S^T and dP^T come out with one query per lane, so LSE_i and D_i
//     are one register each, and dS^T feeds dQ^T = K^T dS^T from registers,
//     with K^T read transposed from the row-major K tile.
// Tiles go from global memory straight into LDS (buffer loads with an LDS
// destination) one tile ahead, so no staging registers and no transposed
// copies exist; barriers inside the loops wait only for LDS traffic.
// Kernels 2 and 3 recompute S and P each, so the backward executes 14 N^2 d
// flops per head (7 contractions) for the 10 N^2 d it is credited with.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.h"

// Tile choices (compile-time).
#ifndef FA_DQ_NW
#define FA_DQ_NW 8
#endif
#ifndef FA_DQ_BC
#define FA_DQ_BC 64
#endif
// dK/dV with the two waves of each pair half a tile apart (d <= 128)
#ifndef FA_DKDV_PINGPONG
#define FA_DKDV_PINGPONG 1
#endif

namespace fa {

namespace {

// ---------------------------------------------------------------------------
// 1. D_i = sum_t dO_it O_it (fp32): a row's D/8 16-byte chunks on the next
//    power of two of threads (the spare ones of d = 96 and 192 add zero), so
//    the row sum is a butterfly
// ---------------------------------------------------------------------------
template <int D>
struct RowdotThreads {
  static constexpr int value = D / 8 <= 8 ? 8 : D / 8 <= 16 ? 16 : 32;
  static_assert(D / 8 <= 32, "head dimension");
};
template <class E, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_bwd_rowdot_kernel(const typename E::T* __restrict__ O, const typename E::T* __restrict__ dO,
                          float* __restrict__ Dout, long long rows) {
  using elt = typename E::T;
  using elt8 = typename E::V8;
  using elt4 = typename E::V4;
  constexpr int TPR = RowdotThreads<D>::value;  // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows && part < D / 8) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0, a1, b0, b1;
      E::unpack2(a[w], a0, a1);
      E::unpack2(b[w], b0, b1);
      acc += a0 * b0;
      acc += a1 * b1;
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) Dout[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK / dV with paired waves (two waves per SIMD)
//
// Eight waves; waves w and w+4 (a pair, same SIMD) share 32 keys of the
// work-group's 128.  For each 64-query tile, wave w computes S and dP for
// query rows 0..31 and wave w+4 for rows 32..63 (full head dimension), both
// turn them into bf16 P and dS, and swap them through a small LDS exchange
// area.  Then each wave accumulates dV = P^T dO and dK = dS^T Q for all 64
// rows but only its half of the head dimension.  Per wave this halves the
// dK/dV accumulators, so a wave fits in 256 VGPRs and two waves share each
// SIMD, without any duplicated MFMA work.  (Running the pairs' two halves of
// the work half a tile apart, so that one wave's exponentials overlap the
// other's MFMAs, measured slower: the accumulators held across the extra
// barrier did not fit without spills.)
// ---------------------------------------------------------------------------
template <int D, int BQ, int NW_>
struct DkdvPairCfg {
  static constexpr int NW = NW_;           // 8 up to d = 128 (two waves per SIMD), 4 at d = 256
  static constexpr int NP = NW / 2;        // pairs; waves w and w + NP share 32 keys
  static constexpr int BK = NP * 32;       // keys per work-group
  static constexpr int NT = NW * 64;
  static constexpr int KS = D / 16;
  static constexpr int NG = BQ / 16;       // 16-query groups per tile
  static constexpr int NDB = D / 32;
  // 32-feature blocks per wave (its half; at d = 96 the first wave of a pair
  // takes two blocks and the second one)
  static constexpr int HDB = (NDB + 1) / 2;
  static_assert(BQ == 64, "two 32-row halves per tile");
};

// LDS operand reads of the in-step dK/dV and the dQ kernels run this many
// MFMAs ahead of their use
#ifndef FA_BWD_PREFETCH
#define FA_BWD_PREFETCH 4
#endif
constexpr int kPre = FA_BWD_PREFETCH;

template <class E, int D, int BQ, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1, NW >= 8 ? 2 : 1)))
void fa_bwd_dkdv_pair_kernel(const typename E::T* __restrict__ Q,
                             const typename E::T* __restrict__ K,
                             const typename E::T* __restrict__ V,
                             const typename E::T* __restrict__ dO,
                             const float* __restrict__ LSE, const float* __restrict__ Dlt,
                             const int32_t* __restrict__ seqlens_k, float scale,
                             float scale_log2, int causal, typename E::T* __restrict__ dK,
                             typename E::T* __restrict__ dV, int B, int H, int n_q, int n_k,
                             int n_ktiles,
                             const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                             int total_q, int total_k) {
  using elt = typename E::T;
  using elt8 = typename E::V8;
  using elt4 = typename E::V4;
  using C = DkdvPairCfg<D, BQ, NW>;
  __shared__ __attribute__((aligned(16))) elt Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) elt dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];
  // P and dS fragments handed to the partner wave: [wave][slot][lane]
  __shared__ __attribute__((aligned(16))) elt8 Xs[C::NW][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int pr = wave % C::NP;   // key block of the pair
  const int half = wave / C::NP; // query half for S/dP, feature half for dK/dV

  // key tiles longest first: the first key tile is seen by the most queries
  const WgOrder wo = wg_order(blockIdx.x, B * H, n_ktiles);
  const int kt = wo.rank;
  const int bh = wo.bh;
  const int b = bh / H;
  const int h = bh - b * H;
  const SeqSpan sp = seq_span(b, h, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (kt * C::BK >= Nk) return;      // a key tile past a shorter sequence
  const elt* Qh = Q + sp.q_row0 * D;
  const elt* Kh = K + sp.k_row0 * D;
  const elt* Vh = V + sp.k_row0 * D;
  const elt* dOh = dO + sp.q_row0 * D;
  const float* Lh = LSE + sp.q_row0;
  const float* Dh = Dlt + sp.q_row0;
  elt* dKh = dK + sp.k_row0 * D;
  elt* dVh = dV + sp.k_row0 * D;

  const int kv_len = key_length(seqlens_k, b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int k0 = kt * C::BK;
  const int kw0 = k0 + pr * 32;
  const int my_key = kw0 + l32;
  // the first query tile that sees key k0: query k0 - off, causally
  const int q_begin = causal ? (max(0, k0 - off) / BQ) * BQ : 0;
  const int n_qt = (k0 < kv_len && q_begin < N) ? (N - q_begin + BQ - 1) / BQ : 0;

  // the pair's K and V rows (B operands of S = Q K^T and dP = dO V^T)
  elt8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (my_key < kv_len) {   // keys past the length never enter a product
      kf[ks] = *reinterpret_cast<const elt8*>(Kh + (size_t)my_key * D + ks * 16 + hi * 8);
      vf[ks] = *reinterpret_cast<const elt8*>(Vh + (size_t)my_key * D + ks * 16 + hi * 8);
    } else {
      kf[ks] = elt8{};
      vf[ks] = elt8{};
    }
  }
  f32x16 dkacc[C::HDB], dvacc[C::HDB];
#pragma unroll
  for (int j = 0; j < C::HDB; ++j) {
    dkacc[j] = f32x16{};
    dvacc[j] = f32x16{};
  }

  // Staging.  The row-major Q and dO tiles are copied straight from global
  // memory into LDS (buffer loads with an LDS destination: lane l of a wave
  // fills bytes [16 l, 16 l + 16) of a 1 KiB block), issued one tile ahead so
  // that the copy has a whole iteration to land.  The buffer descriptors
  // cover exactly one head, so rows at or past N read as zeros.  Each lane
  // fetches the global 16-byte chunk that the XOR swizzle places at its LDS
  // position; the tile is read both as 16-row fragments and by transposing
  // reads, so it takes the swizzle that serves both.
  auto kSwz = [](int row) FA_INLINE { return tile_swizzle<D>(row); };
  // B fragment of dO (or Q) for query rows {16g + 4hi + 0..3, 16g + 8 + 4hi
  // + 0..3} (the order of the P^T fragment) and features 32 db + l32
  const int ts = lane & 15;
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (ts & 3);
  auto colfrag = [&](const elt* tile, int g, int db) FA_INLINE {
    const int r0 = 16 * g + 4 * hi + (ts >> 2);
    const int r1 = r0 + 8;
    const int col = db * 32 + tcol;
    const s16x4 lo = read_tr16(tile + r0 * D + ((col >> 3) ^ tile_swizzle<D>(r0)) * 8 + (col & 7));
    const s16x4 up = read_tr16(tile + r1 * D + ((col >> 3) ^ tile_swizzle<D>(r1)) * 8 + (col & 7));
    return __builtin_bit_cast(elt8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // 1 KiB block rb of a tile holds its 16-byte chunk positions 64 rb .. 64 rb
  // + 63 (rows straddle blocks at d = 96 and 192)
  constexpr int kChunksPerRow = D / 8;
  constexpr int kBlksPerTensor = BQ * D * 2 / 1024;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / C::NW;
  static_assert(BQ * D * 2 % 1024 == 0 && 2 * kBlksPerTensor % C::NW == 0,
                "whole 1 KiB blocks per wave");
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(Qh, head_bytes);
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(dOh, head_bytes);
  float lreg = 0.f, dreg = 0.f;
  auto issue_tile = [&](int qi, int buf) FA_INLINE {
    const int qt0 = q_begin + qi * BQ;
    // statistics first: vector-memory counters retire in order, so waiting
    // for them later does not wait for the tile copy issued after them
    if (tid < BQ) {
      const int row = qt0 + tid;
      lreg = row < N ? Lh[row] : __builtin_huge_valf();
      dreg = row < N ? Dh[row] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBlksPerWave; ++j) {
      const int blk = wave * kBlksPerWave + j;
      const bool is_q = blk < kBlksPerTensor;
      const int rb = is_q ? blk : blk - kBlksPerTensor;
      const int pos = rb * 64 + lane;
      const int row = pos / kChunksPerRow;
      const int chunk = (pos % kChunksPerRow) ^ kSwz(row);
      const int voff = (qt0 + row) * (D * 2) + chunk * 16;
      elt* dst = (is_q ? Qs[buf] : dOs[buf]) + rb * 512;
      lds_dma16_tracked(is_q ? q_rsrc : o_rsrc, dst, voff);
    }
  };
  auto store_stats = [&](int buf) FA_INLINE {
    if (tid < BQ) {
      // rows past N, and rows that see no key, get +inf so that P = 0
      Ls[buf][tid] = (lreg == kNegInf) ? __builtin_huge_valf() : lreg * kLog2e;
      Ds[buf][tid] = dreg;
    }
  };


  if (n_qt > 0) {
    issue_tile(0, 0);
    store_stats(0);
    wait_vmem();
    __syncthreads();
    __syncthreads();
  }

  const bool pair_keys_valid = kw0 < kv_len;
  for (int qi = 0; qi < n_qt; ++qi) {
    const int buf = qi & 1;
    const int qt0 = q_begin + qi * BQ;
    const bool more = qi + 1 < n_qt;
    if (more) issue_tile(qi + 1, buf ^ 1);
    const bool pair_active = pair_keys_valid && (!causal || qt0 + BQ - 1 + off >= kw0);

    elt8 pa[2], dsa[2];
    if (pair_active) {
      // ---- phase 1: S and dP for this wave's 32 query rows (one key per lane);
      // fragments in MFMA order f = (ks, tensor), read kPre MFMAs ahead (with
      // one wave per SIMD, d > 128, nothing else hides their latency)
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const int arow = 32 * half + l32;
      const int asw = kSwz(arow);
      {
        constexpr int NF = 2 * C::KS;
        auto frag = [&](int f) FA_INLINE {
          const int ro = arow * D + ((2 * (f >> 1) + hi) ^ asw) * 8;
          return *reinterpret_cast<const elt8*>((f & 1) ? &dOs[buf][ro] : &Qs[buf][ro]);
        };
        elt8 ring[kPre];
#pragma unroll
        for (int f = 0; f < kPre; ++f) ring[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const elt8 fr = ring[f % kPre];
          if (f + kPre < NF) ring[f % kPre] = frag(f + kPre);
          if (f & 1)
            pacc = E::mfma(fr, vf[f >> 1], pacc);
          else
            sacc = E::mfma(fr, kf[f >> 1], sacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
        for (int f = 0; f < NF - kPre; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
      }
      // this lane's key is visible from tile row 32 half + 8 a4 + 4 hi + e iff
      // 32 half + 8 a4 + e >= first_vis
      const int first_vis =
          my_key >= kv_len ? BQ : (causal ? my_key - off - qt0 - 4 * hi : -BQ);
      auto p_and_ds = [&](auto masked_tag) FA_INLINE {
        constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int r0 = 32 * half + 8 * a4 + 4 * hi;
          const f32x4 lq = *reinterpret_cast<const f32x4*>(&Ls[buf][r0]);
          const f32x4 dq = *reinterpret_cast<const f32x4*>(&Ds[buf][r0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * a4 + e;
            float p = fast_exp2(__builtin_fmaf(sacc[v], scale_log2, -lq[e]));
            if (kMasked) p = (32 * half + 8 * a4 + e >= first_vis) ? p : 0.f;
            pa[v >> 3][v & 7] = E::cvt(p);
            dsa[v >> 3][v & 7] = E::cvt(p * (pacc[v] - dq[e]));
          }
        }
      };
      if ((kw0 + 31 >= kv_len) || (causal && qt0 + 32 * half + off < kw0 + 31))
        p_and_ds(std::true_type{});
      else
        p_and_ds(std::false_type{});
      Xs[wave][0][lane] = pa[0];
      Xs[wave][1][lane] = pa[1];
      Xs[wave][2][lane] = dsa[0];
      Xs[wave][3][lane] = dsa[1];
    }
    lds_barrier();
    if (more) store_stats(buf ^ 1);
    if (pair_active) {
      // ---- phase 2: dV += P^T dO, dK += dS^T Q over all 64 rows, own feature half
      const int partner = wave ^ C::NP;
      elt8 po[2], dso[2];
      po[0] = Xs[partner][0][lane];
      po[1] = Xs[partner][1][lane];
      dso[0] = Xs[partner][2][lane];
      dso[1] = Xs[partner][3][lane];
      // NB feature blocks from db0 (a compile-time count, so that at d = 96,
      // where the pair's waves take two blocks and one, each wave still runs
      // one straight-line schedule); column fragments in MFMA order (g, j,
      // tensor), read kPre MFMAs ahead.  (Splitting this per half, so that the
      // own/partner choice is static, crashed the compiler at d = 256.)
      auto accumulate = [&](auto nb_tag, int db0) FA_INLINE {
        constexpr int NB = decltype(nb_tag)::value;
        constexpr int NF = C::NG * NB * 2;
        auto frag = [&](int f) FA_INLINE {
          const int g = f / (2 * NB), j = (f / 2) % NB;
          return colfrag((f & 1) ? Qs[buf] : dOs[buf], g, db0 + j);
        };
        elt8 ring[kPre];
#pragma unroll
        for (int f = 0; f < kPre; ++f) ring[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int g = f / (2 * NB), j = (f / 2) % NB;
          const elt8 fr = ring[f % kPre];
          if (f + kPre < NF) ring[f % kPre] = frag(f + kPre);
          const bool own = (g >> 1) == half;
          if (f & 1)
            dkacc[j] = E::mfma(own ? dsa[g & 1] : dso[g & 1], fr, dkacc[j]);
          else
            dvacc[j] = E::mfma(own ? pa[g & 1] : po[g & 1], fr, dvacc[j]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
#pragma unroll
        for (int f = 0; f < NF - kPre; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
      };
      if constexpr (C::NDB % 2 == 0)
        accumulate(std::integral_constant<int, C::HDB>{}, half * C::HDB);
      else if (half == 0)
        accumulate(std::integral_constant<int, C::HDB>{}, 0);
      else
        accumulate(std::integral_constant<int, C::NDB - C::HDB>{}, C::HDB);
    }
    // the next tile's row-major copy has landed once every wave passes here
    wait_vmem();
    lds_barrier();
  }

  // ---- write dK = scale * acc, dV = acc for this wave's feature half
#pragma unroll
  for (int j = 0; j < C::HDB; ++j) {
    const int db = half * C::HDB + j;
    if (C::NDB % 2 != 0 && db >= C::NDB) break;   // the second wave's single block at d = 96
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kw0 + c_row(v, lane);
      if (key < Nk) {
        dKh[(size_t)key * D + db * 32 + l32] = E::cvt(dkacc[j][v] * scale);
        dVh[(size_t)key * D + db * 32 + l32] = E::cvt(dvacc[j][v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. dK / dV with the pairs' waves out of phase (eight waves, d <= 128)
//
// The same pairs, work split and LDS exchange as above, but the second wave
// of every pair runs half a tile behind the first, so that on each SIMD one
// wave issues MFMAs while its partner computes exponentials (the in-step
// schedule leaves the matrix cores idle while both do).  With M1(t) = S and
// dP of query tile t, V(t) = P and dS, and M2(t) = dV and dK, each stage
// ends at a work-group barrier:
//   stage X(t): leading wave  M2(t-1), M1(t)       lagging wave  V(t)
//   stage Y(t): leading wave  V(t)                 lagging wave  M2(t-1), M1(t+1)
// A leading wave hands its P and dS over at the end of its V stage, into
// one of two exchange planes (by tile parity).  A lagging wave writes its dS
// there too (two planes by parity) but its P at the start of the stage after
// its V stage, into a single plane, after reading back its own P of the tile
// before: the 160 KiB of LDS hold the tiles and all but one of the second
// planes.  Exchange writes inside an MFMA stage cost that stage several
// hundred cycles.  Tile t is read from stage Y(t-1) to Y(t+1), so
// the Q/dO tiles take three LDS slots, and the lagging group copies tile t+1
// (and stores its statistics) during stage X(t).  Each MFMA stage is one
// wave's: its operand reads run four MFMAs ahead of their use.
// ---------------------------------------------------------------------------
template <class E, int D, int BQ>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_pp_kernel(const typename E::T* __restrict__ Q,
                           const typename E::T* __restrict__ K,
                           const typename E::T* __restrict__ V,
                           const typename E::T* __restrict__ dO,
                           const float* __restrict__ LSE, const float* __restrict__ Dlt,
                           const int32_t* __restrict__ seqlens_k, float scale,
                           float scale_log2, int causal, typename E::T* __restrict__ dK,
                           typename E::T* __restrict__ dV, int B, int H, int n_q, int n_k,
                           int n_ktiles,
                           const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                           int total_q, int total_k) {
  using elt = typename E::T;
  using elt8 = typename E::V8;
  using C = DkdvPairCfg<D, BQ, 8>;
  __shared__ __attribute__((aligned(16))) elt Qs[3][BQ * D];
  __shared__ __attribute__((aligned(16))) elt dOs[3][BQ * D];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];
  // P and dS fragments handed to the partner wave, [plane][pair][fragment][lane]
  // (fragments 0-1: P, 2-3: dS): for tile t the leading waves write plane t % 2;
  // the lagging waves write their P to XP and their dS to XD[t % 2]
  __shared__ __attribute__((aligned(16))) elt8 Xs[2][C::NP][4][64];
  __shared__ __attribute__((aligned(16))) elt8 XP[C::NP][2][64];
  __shared__ __attribute__((aligned(16))) elt8 XD[2][C::NP][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int pr = wave % C::NP;   // key block of the pair
  const int half = wave / C::NP; // query half for S/dP, feature half for dK/dV
  const bool lead = half == 0;   // the leading wave of the pair

  const WgOrder wo = wg_order(blockIdx.x, B * H, n_ktiles);
  const int kt = wo.rank;
  const int bh = wo.bh;
  const int b = bh / H;
  const int h = bh - b * H;
  const SeqSpan sp = seq_span(b, h, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;
  if (kt * C::BK >= Nk) return;
  const elt* Qh = Q + sp.q_row0 * D;
  const elt* Kh = K + sp.k_row0 * D;
  const elt* Vh = V + sp.k_row0 * D;
  const elt* dOh = dO + sp.q_row0 * D;
  const float* Lh = LSE + sp.q_row0;
  const float* Dh = Dlt + sp.q_row0;
  elt* dKh = dK + sp.k_row0 * D;
  elt* dVh = dV + sp.k_row0 * D;

  const int kv_len = key_length(seqlens_k, b, Nk);
  const int off = Nk - N;
  const int k0 = kt * C::BK;
  const int kw0 = k0 + pr * 32;
  const int my_key = kw0 + l32;
  const int q_begin = causal ? (max(0, k0 - off) / BQ) * BQ : 0;
  const int n_qt = (k0 < kv_len && q_begin < N) ? (N - q_begin + BQ - 1) / BQ : 0;

  // this pair's K and V rows as MFMA fragments (one key per lane), read from
  // LDS in the prologue (see copy_kv)
  elt8 kf[C::KS], vf[C::KS];
  f32x16 dkacc[C::HDB], dvacc[C::HDB];
#pragma unroll
  for (int j = 0; j < C::HDB; ++j) {
    dkacc[j] = f32x16{};
    dvacc[j] = f32x16{};
  }

  // Staging as in the kernel above, but only the lagging group copies (its
  // vector stage is the shorter one), into slot t % 3; its first wave loads
  // the tile's statistics (one row per lane) ahead of the copies.
  auto kSwz = [](int row) FA_INLINE { return tile_swizzle<D>(row); };
  const int ts = lane & 15;
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (ts & 3);
  constexpr int kChunksPerRow = D / 8;
  constexpr int kBlksPerTensor = BQ * D * 2 / 1024;
  constexpr int kCopyWaves = C::NW / 2;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / kCopyWaves;
  static_assert(BQ * D * 2 % 1024 == 0 && 2 * kBlksPerTensor % kCopyWaves == 0,
                "whole 1 KiB blocks per copying wave");
  static_assert(BQ == 64, "one statistics row per lane");
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(Qh, head_bytes);
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(dOh, head_bytes);
  const bool stat_wave = wave == C::NP;
  float lreg = 0.f, dreg = 0.f;
  auto issue_tile = [&](int t, int slot) FA_INLINE {
    const int qt0 = q_begin + t * BQ;
    if (stat_wave) {
      const int row = qt0 + lane;
      lreg = row < N ? Lh[row] : __builtin_huge_valf();
      dreg = row < N ? Dh[row] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBlksPerWave; ++j) {
      const int blk = (wave - C::NP) * kBlksPerWave + j;
      const bool is_q = blk < kBlksPerTensor;
      const int rb = is_q ? blk : blk - kBlksPerTensor;
      const int pos = rb * 64 + lane;
      const int row = pos / kChunksPerRow;
      const int chunk = (pos % kChunksPerRow) ^ kSwz(row);
      const int voff = (qt0 + row) * (D * 2) + chunk * 16;
      elt* dst = (is_q ? Qs[slot] : dOs[slot]) + rb * 512;
      lds_dma16_tracked(is_q ? q_rsrc : o_rsrc, dst, voff);
    }
  };

  // The work-group's K and V blocks (128 keys) go to LDS with the tiles'
  // coalesced, swizzled direct loads, into the ring slots 1 and 2 of Qs and
  // dOs that no tile uses before the second prologue barrier (one block
  // fills exactly two slots), and each wave then reads its pair's fragments
  // from there.  Loaded straight into registers, each load instruction took
  // 32 rows x 32 bytes and the fragments landed about 10,700 cycles after
  // the work-group started, against 1,900 for a tile copy.  Keys at or past
  // the key length read as zeros (the descriptors end there).
  static_assert(C::BK == 2 * BQ, "a key block fills two ring slots");
  constexpr int kKvBlks = C::BK * D * 2 / 1024;            // 1 KiB blocks per tensor
  constexpr int kKvBlksPerWave = 2 * kKvBlks / C::NW;
  static_assert(2 * kKvBlks % C::NW == 0, "whole 1 KiB blocks per wave");
  elt* const kblk = &Qs[1][0];
  elt* const vblk = &dOs[1][0];
  auto copy_kv = [&]() FA_INLINE {
    const int kv_bytes = max(0, min(kv_len - k0, C::BK)) * D * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(Kh + (size_t)k0 * D, kv_bytes);
    const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(Vh + (size_t)k0 * D, kv_bytes);
#pragma unroll
    for (int j = 0; j < kKvBlksPerWave; ++j) {
      const int blk = wave * kKvBlksPerWave + j;
      const bool is_k = blk < kKvBlks;
      const int rb = is_k ? blk : blk - kKvBlks;
      const int pos = rb * 64 + lane;
      const int row = pos / kChunksPerRow;
      const int chunk = (pos % kChunksPerRow) ^ kSwz(row);
      lds_dma16_tracked(is_k ? k_rsrc : v_rsrc, (is_k ? kblk : vblk) + rb * 512,
                        row * (D * 2) + chunk * 16);
    }
  };
  auto read_kv = [&]() FA_INLINE {
    const int row = pr * 32 + l32;
    const int sw = kSwz(row);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int at = row * D + ((2 * ks + hi) ^ sw) * 8;
      kf[ks] = *reinterpret_cast<const elt8*>(&kblk[at]);
      vf[ks] = *reinterpret_cast<const elt8*>(&vblk[at]);
    }
  };

  auto store_stats = [&](int t) FA_INLINE {
    if (stat_wave) {
      Ls[t & 1][lane] = (lreg == kNegInf) ? __builtin_huge_valf() : lreg * kLog2e;
      Ds[t & 1][lane] = dreg;
    }
  };

  const bool pair_keys_valid = kw0 < kv_len;
  auto active = [&](int t) FA_INLINE {
    return pair_keys_valid && (!causal || q_begin + t * BQ + BQ - 1 + off >= kw0);
  };
  // The leading waves are the pairs' first halves and the lagging waves the
  // second, so each loop below passes its half as a compile-time constant.
  // M1: S and dP for this wave's 32 query rows (one key per lane)
  constexpr int kM1Pre = 4;
  auto m1 = [&](auto half_tag, int slot, f32x16& sacc, f32x16& pacc) FA_INLINE {
    constexpr int HF = decltype(half_tag)::value;
    sacc = f32x16{};
    pacc = f32x16{};
    const int arow = 32 * HF + l32;
    const int asw = kSwz(arow);
    // fragments in MFMA order f = (ks, tensor), read kM1Pre MFMAs ahead
    constexpr int NF = 2 * C::KS;
    auto frag = [&](int f) FA_INLINE {
      const int ro = arow * D + ((2 * (f >> 1) + hi) ^ asw) * 8;
      return *reinterpret_cast<const elt8*>((f & 1) ? &dOs[slot][ro] : &Qs[slot][ro]);
    };
    elt8 ring[kM1Pre];
#pragma unroll
    for (int f = 0; f < kM1Pre; ++f) ring[f] = frag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const elt8 fr = ring[f % kM1Pre];
      if (f + kM1Pre < NF) ring[f % kM1Pre] = frag(f + kM1Pre);
      if (f & 1)
        pacc = E::mfma(fr, vf[f >> 1], pacc);
      else
        sacc = E::mfma(fr, kf[f >> 1], sacc);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kM1Pre, 0);
#pragma unroll
    for (int f = 0; f < NF - kM1Pre; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kM1Pre, 0);
  };
  // V: P = exp(S - LSE) and dS = P (dP - D), rounded to the element format
  auto vstage = [&](auto half_tag, int t, const f32x16& sacc, const f32x16& pacc,
                    elt8 (&pa)[2], elt8 (&dsa)[2]) FA_INLINE {
    constexpr int HF = decltype(half_tag)::value;
    const int qt0 = q_begin + t * BQ;
    const int sb = t & 1;
    const int first_vis =
        my_key >= kv_len ? BQ : (causal ? my_key - off - qt0 - 4 * hi : -BQ);
    auto p_and_ds = [&](auto masked_tag) FA_INLINE {
      constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int r0 = 32 * HF + 8 * a4 + 4 * hi;
        const f32x4 lq = *reinterpret_cast<const f32x4*>(&Ls[sb][r0]);
        const f32x4 dq = *reinterpret_cast<const f32x4*>(&Ds[sb][r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * a4 + e;
          float p = fast_exp2(__builtin_fmaf(sacc[v], scale_log2, -lq[e]));
          if (kMasked) p = (32 * HF + 8 * a4 + e >= first_vis) ? p : 0.f;
          pa[v >> 3][v & 7] = E::cvt(p);
          dsa[v >> 3][v & 7] = E::cvt(p * (pacc[v] - dq[e]));
        }
      }
    };
    if ((kw0 + 31 >= kv_len) || (causal && qt0 + 32 * HF + off < kw0 + 31))
      p_and_ds(std::true_type{});
    else
      p_and_ds(std::false_type{});
  };
  // two fragments at [2][64] elt8 (fragment-major, one 16-byte piece per lane)
  auto put2 = [&](elt8* dst, const elt8 (&v)[2]) FA_INLINE {
    dst[lane] = v[0];
    dst[64 + lane] = v[1];
  };
  auto get2 = [&](const elt8* src, elt8 (&v)[2]) FA_INLINE {
    v[0] = src[lane];
    v[1] = src[64 + lane];
  };
  // Element offsets of this lane's two transposing reads (rows r and r + 8,
  // r = 16 g + 4 hi + ts / 4) for each of its feature blocks, for even and odd
  // 16-row groups g: the swizzles of d <= 128 see no row bit above 4, so
  // groups g and g + 2 differ by 32 rows, an immediate offset.
  int tr_at[C::HDB][2][2];
#pragma unroll
  for (int j = 0; j < C::HDB; ++j)
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 16 * par + 4 * hi + (ts >> 2) + 8 * u;
        const int col = (half * C::HDB + j) * 32 + tcol;
        tr_at[j][par][u] = row * D + ((col >> 3) ^ tile_swizzle<D>(row)) * 8 + (col & 7);
      }
  // M2: dV += P^T dO, dK += dS^T Q over all 64 rows, own feature half.  The
  // column fragments are read kM2Pre MFMAs ahead of their use: in this stage
  // the wave's partner runs vector work, so no second wave hides the reads.
  constexpr int kM2Pre = 4;
  auto m2 = [&](auto half_tag, int slot, const elt8 (&pa)[2], const elt8 (&dsa)[2],
                const elt8* po_src, const elt8* dso_src) FA_INLINE {
    constexpr int HF = decltype(half_tag)::value;
    // feature blocks of this half (at d = 96 the first half takes two, the second one)
    constexpr int NB = (C::NDB % 2 == 0 || HF == 0) ? C::HDB : C::NDB - C::HDB;
    elt8 po[2], dso[2];
    get2(po_src, po);
    get2(dso_src, dso);
    const elt* qt = Qs[slot];
    const elt* ot = dOs[slot];
    // fragments in MFMA order f = (g, j, tensor); tensor 0: dO (for dV), 1: Q (for dK)
    constexpr int NF = C::NG * NB * 2;
    auto frag = [&](int f) FA_INLINE {
      const int g = f / (2 * NB), j = (f / 2) % NB;
      const elt* base = ((f & 1) ? qt : ot) + (g >> 1) * 32 * D;
      const s16x4 lo = read_tr16(base + tr_at[j][g & 1][0]);
      const s16x4 up = read_tr16(base + tr_at[j][g & 1][1]);
      return __builtin_bit_cast(elt8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    elt8 ring[kM2Pre];
#pragma unroll
    for (int f = 0; f < kM2Pre; ++f) ring[f] = frag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int g = f / (2 * NB), j = (f / 2) % NB;
      const elt8 fr = ring[f % kM2Pre];
      if (f + kM2Pre < NF) ring[f % kM2Pre] = frag(f + kM2Pre);
      // row groups 2 HF and 2 HF + 1 are this wave's, the others its partner's
      const bool own = (g >> 1) == HF;
      if (f & 1)
        dkacc[j] = E::mfma(own ? dsa[g & 1] : dso[g & 1], fr, dkacc[j]);
      else
        dvacc[j] = E::mfma(own ? pa[g & 1] : po[g & 1], fr, dvacc[j]);
    }
    // keep the fragment reads kM2Pre MFMAs ahead of their consumers
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + 2 * kM2Pre, 0);
#pragma unroll
    for (int f = 0; f < NF - kM2Pre; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kM2Pre, 0);
  };

  // Each group runs its own loop (2 n + 3 barriers in both).  M1 runs for
  // every tile, also where the pair sees none of it (its values then go
  // unused), so S and dP are never carried across the dV/dK stage.
  constexpr std::integral_constant<int, 0> kLeadHalf{};
  constexpr std::integral_constant<int, 1> kLagHalf{};
  if (n_qt > 0) {
    f32x16 sacc, pacc;
    elt8 pa[2] = {}, dsa[2] = {};   // this wave's P and dS of its latest V stage
    if (lead) {
      copy_kv();
      wait_vmem();
      lds_barrier();   // the K/V block, tile 0 and its statistics
      read_kv();
      lds_barrier();   // stage P (the lagging group's M1(0)); the K/V block's slots are free again
      int slot = 0;  // tile t's slot, t % 3
      for (int t = 0; t < n_qt; ++t) {
        const int prev = slot == 0 ? 2 : slot - 1;
        // ---- stage X(t): M2(t - 1), M1(t)
        if (t >= 1 && active(t - 1))
          m2(kLeadHalf, prev, pa, dsa, &XP[pr][0][0], &XD[(t - 1) & 1][pr][0][0]);
        m1(kLeadHalf, slot, sacc, pacc);
        lds_barrier();
        // ---- stage Y(t): V(t), then hand P and dS over
        if (active(t)) {
          vstage(kLeadHalf, t, sacc, pacc, pa, dsa);
          put2(&Xs[t & 1][pr][0][0], pa);
          put2(&Xs[t & 1][pr][2][0], dsa);
        }
        lds_barrier();
        slot = slot == 2 ? 0 : slot + 1;
      }
      // ---- stage X(n): M2(n - 1)
      if (active(n_qt - 1))
        m2(kLeadHalf, slot == 0 ? 2 : slot - 1, pa, dsa, &XP[pr][0][0],
           &XD[(n_qt - 1) & 1][pr][0][0]);
      lds_barrier();
    } else {
      copy_kv();
      issue_tile(0, 0);
      wait_vmem();
      store_stats(0);
      lds_barrier();
      read_kv();
      // ---- stage P: M1(0)
      m1(kLagHalf, 0, sacc, pacc);
      lds_barrier();
      int slot = 0;
      for (int t = 0; t < n_qt; ++t) {
        const int prev = slot == 0 ? 2 : slot - 1;
        const int next = slot == 2 ? 0 : slot + 1;
        // ---- stage X(t): copy tile t + 1, V(t)
        if (t + 1 < n_qt) issue_tile(t + 1, next);
        if (active(t)) {
          vstage(kLagHalf, t, sacc, pacc, pa, dsa);
          put2(&XD[t & 1][pr][0][0], dsa);
        }
        // tile t + 1 has landed once every wave passes the barrier
        wait_vmem();
        if (t + 1 < n_qt) store_stats(t + 1);
        lds_barrier();
        // ---- stage Y(t): M2(t - 1), M1(t + 1) (after the last tile, M1 of a
        // stale slot, unused).  This wave's own P of tile t - 1 is read back
        // from XP before tile t's overwrites it, its dS from XD[(t - 1) % 2].
        elt8 pb[2], dsb[2];
        get2(&XP[pr][0][0], pb);
        get2(&XD[(t - 1) & 1][pr][0][0], dsb);
        if (active(t)) put2(&XP[pr][0][0], pa);
        if (t >= 1 && active(t - 1))
          m2(kLagHalf, prev, pb, dsb, &Xs[(t - 1) & 1][pr][0][0], &Xs[(t - 1) & 1][pr][2][0]);
        m1(kLagHalf, next, sacc, pacc);
        lds_barrier();
        slot = next;
      }
      // ---- stage X(n): nothing; stage Y(n): M2(n - 1)
      lds_barrier();
      if (active(n_qt - 1))
        m2(kLagHalf, slot == 0 ? 2 : slot - 1, pa, dsa, &Xs[(n_qt - 1) & 1][pr][0][0],
           &Xs[(n_qt - 1) & 1][pr][2][0]);
    }
  }

  // ---- write dK = scale * acc, dV = acc for this wave's feature half
#pragma unroll
  for (int j = 0; j < C::HDB; ++j) {
    const int db = half * C::HDB + j;
    if (C::NDB % 2 != 0 && db >= C::NDB) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kw0 + c_row(v, lane);
      if (key < Nk) {
        dKh[(size_t)key * D + db * 32 + l32] = E::cvt(dkacc[j][v] * scale);
        dVh[(size_t)key * D + db * 32 + l32] = E::cvt(dvacc[j][v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
template <int D, int NW, int BC>
struct DqCfg {
  static constexpr int BR = NW * 32;
  static constexpr int NT = NW * 64;
  static constexpr int KS = D / 16;
  static constexpr int NCB = BC / 32;
  static constexpr int NG = BC / 16;
  static constexpr int NDB = D / 32;
};

template <class E, int D, int NW, int BC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1, NW >= 8 ? 2 : 1)))
void fa_bwd_dq_kernel(const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
                      const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
                      const float* __restrict__ LSE, const float* __restrict__ Dlt,
                      const int32_t* __restrict__ seqlens_k, float scale, float scale_log2,
                      int causal, typename E::T* __restrict__ dQ, int B, int H, int n_q, int n_k,
                      int n_qtiles, const int32_t* __restrict__ cu_q,
                      const int32_t* __restrict__ cu_k, int total_q, int total_k) {
  using elt = typename E::T;
  using elt8 = typename E::V8;
  using elt4 = typename E::V4;
  using C = DqCfg<D, NW, BC>;
  // operand prefetch depth: with one wave per SIMD (d > 128) nothing else
  // hides the LDS latency; with two, the plain in-order loops are kept (a
  // ring measured 3-5 % slower there)
  constexpr int kRing = NW >= 8 ? 1 : kPre;
  // row-major K and V tiles in two slots (one read, one being loaded)
  __shared__ __attribute__((aligned(16))) elt Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) elt Vs[2][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_coord(blockIdx.x, B, H, n_qtiles);
  const SeqSpan sp = seq_span(tc.b, tc.h, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (tc.qt * C::BR >= N) return;    // a query tile past a shorter sequence
  const elt* Qh = Q + sp.q_row0 * D;
  const elt* Kh = K + sp.k_row0 * D;
  const elt* Vh = V + sp.k_row0 * D;
  const elt* dOh = dO + sp.q_row0 * D;
  elt* dQh = dQ + sp.q_row0 * D;

  const int kv_len = key_length(seqlens_k, tc.b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int q0 = tc.qt * C::BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, max(0, min(q0 + C::BR + off, Nk)));
  const int n_kt = (kv_end + BC - 1) / BC;

  elt8 qf[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (qrow < N) {
      qf[ks] = *reinterpret_cast<const elt8*>(Qh + (size_t)qrow * D + ks * 16 + hi * 8);
      of[ks] = *reinterpret_cast<const elt8*>(dOh + (size_t)qrow * D + ks * 16 + hi * 8);
    } else {
      qf[ks] = elt8{};
      of[ks] = elt8{};
    }
  }
  float lse2 = __builtin_huge_valf(), drow = 0.f;
  if (qrow < N) {
    const float lse = LSE[sp.q_row0 + qrow];
    lse2 = (lse == kNegInf) ? __builtin_huge_valf() : lse * kLog2e;
    drow = Dlt[sp.q_row0 + qrow];
  }

  f32x16 dqacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dqacc[db] = f32x16{};

  // Staging.  Row-major K and V tiles are copied straight from global memory
  // into LDS (lane l of a wave fills bytes [16 l, 16 l + 16) of a 1 KiB
  // block; each lane fetches the global chunk that the tile's XOR swizzle
  // places there), one tile ahead.  The buffer descriptors end at the key
  // length L_b, so keys at or past it read as zeros.
  // K is read both as 16-row fragments (S^T = K Q^T) and by transposing
  // reads (the A operand of dQ^T = K^T dS^T), so no transposed copy exists.
  constexpr int kChunksPerRow = D / 8;
  constexpr int kBlksPerTensor = BC * D * 2 / 1024;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / NW;
  static_assert(BC * D * 2 % 1024 == 0, "whole 1 KiB blocks per tile");
  static_assert(2 * kBlksPerTensor % NW == 0 && kBlksPerWave >= 1, "whole 1 KiB blocks per wave");
  const int key_bytes = kv_len * D * 2;
  const u32x4 k_rsrc = buffer_rsrc_words(Kh, (uint32_t)key_bytes);
  const u32x4 v_rsrc = buffer_rsrc_words(Vh, (uint32_t)key_bytes);
  // per-lane byte offsets inside a tile, computed once; the tile's position
  // goes in the scalar offset (see fa_fwd.hip: copies issued through the
  // builtin made the next transposing read wait for the whole copy)
  int voff[kBlksPerWave];
#pragma unroll
  for (int j = 0; j < kBlksPerWave; ++j) {
    const int blk = wave * kBlksPerWave + j;
    const int rb = blk < kBlksPerTensor ? blk : blk - kBlksPerTensor;
    const int pos = rb * 64 + lane;
    const int row = pos / kChunksPerRow;
    voff[j] = row * (D * 2) + ((pos % kChunksPerRow) ^ tile_swizzle<D>(row)) * 16;
  }
  auto issue_tile = [&](int kt, int slot) FA_INLINE {
#pragma unroll
    for (int j = 0; j < kBlksPerWave; ++j) {
      const int blk = wave * kBlksPerWave + j;
      const bool is_k = blk < kBlksPerTensor;
      const int rb = is_k ? blk : blk - kBlksPerTensor;
      elt* dst = (is_k ? Ks[slot] : Vs[slot]) + rb * 512;
      lds_dma16(is_k ? k_rsrc : v_rsrc, dst, voff[j], kt * BC * D * 2);
    }
  };
  // A fragment of K^T for keys {16g + 4hi + 0..3, 16g + 8 + 4hi + 0..3} (the
  // order of the dS^T fragment) and features 32 db + l32
  const int ts = lane & 15;
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (ts & 3);
  auto colfrag = [&](const elt* tile, int g, int db) FA_INLINE {
    const int r0 = 16 * g + 4 * hi + (ts >> 2);
    const int r1 = r0 + 8;
    const int col = db * 32 + tcol;
    const s16x4 lo = read_tr16(tile + r0 * D + ((col >> 3) ^ tile_swizzle<D>(r0)) * 8 + (col & 7));
    const s16x4 up = read_tr16(tile + r1 * D + ((col >> 3) ^ tile_swizzle<D>(r1)) * 8 + (col & 7));
    return __builtin_bit_cast(elt8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  wait_vmem();   // the query rows and their statistics
  if (n_kt > 0) {
    issue_tile(0, 0);
    wait_vmem();
    __syncthreads();
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const int slot = kt & 1;
    if (kt + 1 < n_kt) issue_tile(kt + 1, slot ^ 1);
    const int key0 = kt * BC;
    const bool wave_active = (qw0 < N) && (!causal || key0 <= qw0 + 31 + off);
    if (wave_active) {
      // ---- S^T = K Q^T, dP^T = V dO^T (C: one query per lane, rows = keys)
      f32x16 sacc[C::NCB], pacc[C::NCB];
#pragma unroll
      for (int c = 0; c < C::NCB; ++c) {
        sacc[c] = f32x16{};
        pacc[c] = f32x16{};
      }
      if constexpr (kRing == 1) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int c = 0; c < C::NCB; ++c) {
            const int arow = c * 32 + l32;
            const int ro = arow * D + ((2 * ks + hi) ^ tile_swizzle<D>(arow)) * 8;
            const elt8 ka = *reinterpret_cast<const elt8*>(&Ks[slot][ro]);
            const elt8 va = *reinterpret_cast<const elt8*>(&Vs[slot][ro]);
            sacc[c] = E::mfma(ka, qf[ks], sacc[c]);
            pacc[c] = E::mfma(va, of[ks], pacc[c]);
          }
      } else {
        // fragments in MFMA order f = (ks, c, tensor), read kRing MFMAs ahead
        constexpr int NF = C::KS * C::NCB * 2;
        auto frag = [&](int f) FA_INLINE {
          const int ks = f / (2 * C::NCB), c = (f / 2) % C::NCB;
          const int arow = c * 32 + l32;
          const int ro = arow * D + ((2 * ks + hi) ^ tile_swizzle<D>(arow)) * 8;
          return *reinterpret_cast<const elt8*>((f & 1) ? &Vs[slot][ro] : &Ks[slot][ro]);
        };
        elt8 ring[kRing];
#pragma unroll
        for (int f = 0; f < kRing; ++f) ring[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int ks = f / (2 * C::NCB), c = (f / 2) % C::NCB;
          const elt8 fr = ring[f % kRing];
          if (f + kRing < NF) ring[f % kRing] = frag(f + kRing);
          if (f & 1)
            pacc[c] = E::mfma(fr, of[ks], pacc[c]);
          else
            sacc[c] = E::mfma(fr, qf[ks], sacc[c]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
        for (int f = 0; f < NF - kRing; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kRing, 0);
      }
      // only tiles crossing the key length or the wave's diagonal are masked:
      // key key0 + 32c + 4hi + p, p = 8(v/4) + v%4, is visible iff it is at
      // most min(L - 1, this lane's query); S = -inf gives P = 0
      if ((key0 + BC > kv_len) || (causal && key0 + BC - 1 > qw0 + off)) {
        const int lim = (causal ? min(kv_len - 1, qrow + off) : kv_len - 1) - key0 - 4 * hi;
#pragma unroll
        for (int c = 0; c < C::NCB; ++c) {
          const uint32_t vis = prefix_bits(lim - 32 * c);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            sacc[c][v] = keep_if_bit(sacc[c][v], vis, 8 * (v >> 2) + (v & 3), kNegInf);
        }
      }
      // dS^T = P^T o (dP^T - rowdot)
      elt8 dsb[C::NG];
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(sacc[c][v], scale_log2, -lse2));
          dsb[2 * c + (v >> 3)][v & 7] = E::cvt(p * (pacc[c][v] - drow));
        }
      // ---- dQ^T += K^T dS^T
      if constexpr (kRing == 1) {
#pragma unroll
        for (int g = 0; g < C::NG; ++g)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            dqacc[db] = E::mfma(colfrag(Ks[slot], g, db), dsb[g], dqacc[db]);
      } else {
        // K^T fragments in MFMA order (g, db), read kRing MFMAs ahead
        constexpr int NF = C::NG * C::NDB;
        auto frag = [&](int f) FA_INLINE { return colfrag(Ks[slot], f / C::NDB, f % C::NDB); };
        elt8 ring[kRing];
#pragma unroll
        for (int f = 0; f < kRing; ++f) ring[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const elt8 fr = ring[f % kRing];
          if (f + kRing < NF) ring[f % kRing] = frag(f + kRing);
          dqacc[f % C::NDB] = E::mfma(fr, dsb[f / C::NDB], dqacc[f % C::NDB]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kRing, 0);
#pragma unroll
        for (int f = 0; f < NF - kRing; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kRing, 0);
      }
    }
    // the next tile has landed once every wave passes here
    wait_vmem();
    lds_barrier();
  }

  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * hi;
        elt4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = E::cvt(dqacc[db][4 * v4 + e] * scale);
        *reinterpret_cast<elt4*>(dQh + (size_t)qrow * D + d0) = w;
      }
  }
}

constexpr int kDqBC = FA_DQ_BC;
// key tile of the dQ kernel per head dimension: at d = 64 its registers hold
// twice the S/dP tile, which halves the barriers per key
#ifndef FA_DQ_BC64
#define FA_DQ_BC64 128
#endif
template <int D>
struct DqTile {
  static constexpr int BC = D == 64 ? FA_DQ_BC64 : kDqBC;
};
// waves per work-group of the two main backward kernels: up to d = 128 two
// waves share a SIMD; at d = 256 one wave per SIMD holds the larger operands
template <int D>
struct BwdWaves {
  static constexpr int DKDV = D <= 128 ? 8 : 4;
  static constexpr int DQ = D <= 128 ? FA_DQ_NW : 4;
};

template <class E, int D>
hipError_t launch_preprocess_d(const BwdArgs& a) {
  using T = typename E::T;
  const long long rows = a.cu_q ? (long long)a.H * a.total_q : (long long)a.B * a.H * a.N;
  if (rows == 0) return hipSuccess;
  const long long threads = rows * RowdotThreads<D>::value;
  hipLaunchKernelGGL((fa_bwd_rowdot_kernel<E, D>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, a.stream, static_cast<const T*>(a.o),
                     static_cast<const T*>(a.dout), a.delta, rows);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_dkdv_d(const BwdArgs& a) {
  using CK = DkdvPairCfg<D, 64, BwdWaves<D>::DKDV>;
  using T = typename E::T;
  const int n_ktiles = (a.Nk + CK::BK - 1) / CK::BK;
  if (n_ktiles == 0) return hipSuccess;   // no keys: dK and dV have no rows
  if constexpr (FA_DKDV_PINGPONG && BwdWaves<D>::DKDV == 8) {
    hipLaunchKernelGGL((fa_bwd_dkdv_pp_kernel<E, D, 64>),
                       dim3((unsigned)((long long)n_ktiles * a.B * a.H)), dim3(CK::NT), 0,
                       a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                       a.seqlens_k, a.scale, a.scale * kLog2e, a.causal, static_cast<T*>(a.dk),
                       static_cast<T*>(a.dv), a.B, a.H, a.N, a.Nk, n_ktiles,
                       a.cu_q, a.cu_k, a.total_q, a.total_k);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<E, D, 64, BwdWaves<D>::DKDV>),
                     dim3((unsigned)((long long)n_ktiles * a.B * a.H)), dim3(CK::NT), 0, a.stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.seqlens_k, a.scale, a.scale * kLog2e, a.causal, static_cast<T*>(a.dk),
                     static_cast<T*>(a.dv), a.B, a.H, a.N, a.Nk, n_ktiles,
                     a.cu_q, a.cu_k, a.total_q, a.total_k);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_dq_d(const BwdArgs& a) {
  using CQ = DqCfg<D, BwdWaves<D>::DQ, DqTile<D>::BC>;
  using T = typename E::T;
  const int n_qtiles = (a.N + CQ::BR - 1) / CQ::BR;
  if (n_qtiles == 0) return hipSuccess;   // no queries: dQ has no rows
  hipLaunchKernelGGL((fa_bwd_dq_kernel<E, D, BwdWaves<D>::DQ, DqTile<D>::BC>),
                     dim3((unsigned)((long long)n_qtiles * a.B * a.H)), dim3(CQ::NT), 0, a.stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.seqlens_k, a.scale, a.scale * kLog2e, a.causal, static_cast<T*>(a.dq),
                     a.B, a.H, a.N, a.Nk, n_qtiles,
                     a.cu_q, a.cu_k, a.total_q, a.total_k);
  return hipGetLastError();
}

bool bwd_head_dim(int d) { return d == 64 || d == 96 || d == 128 || d == 192 || d == 256; }

}  // namespace

long long bwd_half_grid(int B, int H, int N, int d) {
  const int bk = d <= 128 ? DkdvPairCfg<128, 64, BwdWaves<128>::DKDV>::BK
                          : DkdvPairCfg<256, 64, BwdWaves<256>::DKDV>::BK;
  const int br = 32 * (d <= 128 ? BwdWaves<128>::DQ : BwdWaves<256>::DQ);
  const long long kt = (N + bk - 1) / bk;
  const long long qt = (N + br - 1) / br;
  const int tpr = d / 8 <= 8 ? 8 : d / 8 <= 16 ? 16 : 32;   // RowdotThreads
  const long long rows_wg = ((long long)B * H * N * tpr + 255) / 256;
  long long m = kt * B * H;
  if (qt * B * H > m) m = qt * B * H;
  if (rows_wg > m) m = rows_wg;
  return m;
}

hipError_t launch_bwd_preprocess_half(const BwdArgs& a, Elt e) {
  if (!bwd_head_dim(a.d)) return hipErrorInvalidValue;
  if (e == Elt::kBf16)
    return a.d == 64    ? launch_preprocess_d<EltBf16, 64>(a)
           : a.d == 96  ? launch_preprocess_d<EltBf16, 96>(a)
           : a.d == 128 ? launch_preprocess_d<EltBf16, 128>(a)
           : a.d == 192 ? launch_preprocess_d<EltBf16, 192>(a)
                        : launch_preprocess_d<EltBf16, 256>(a);
  if (e == Elt::kF16)
    return a.d == 64    ? launch_preprocess_d<EltF16, 64>(a)
           : a.d == 96  ? launch_preprocess_d<EltF16, 96>(a)
           : a.d == 128 ? launch_preprocess_d<EltF16, 128>(a)
           : a.d == 192 ? launch_preprocess_d<EltF16, 192>(a)
                        : launch_preprocess_d<EltF16, 256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_half(const BwdArgs& a, Elt e) {
  if (!bwd_head_dim(a.d)) return hipErrorInvalidValue;
  if (e == Elt::kBf16)
    return a.d == 64    ? launch_dkdv_d<EltBf16, 64>(a)
           : a.d == 96  ? launch_dkdv_d<EltBf16, 96>(a)
           : a.d == 128 ? launch_dkdv_d<EltBf16, 128>(a)
           : a.d == 192 ? launch_dkdv_d<EltBf16, 192>(a)
                        : launch_dkdv_d<EltBf16, 256>(a);
  if (e == Elt::kF16)
    return a.d == 64    ? launch_dkdv_d<EltF16, 64>(a)
           : a.d == 96  ? launch_dkdv_d<EltF16, 96>(a)
           : a.d == 128 ? launch_dkdv_d<EltF16, 128>(a)
           : a.d == 192 ? launch_dkdv_d<EltF16, 192>(a)
                        : launch_dkdv_d<EltF16, 256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_half(const BwdArgs& a, Elt e) {
  if (!bwd_head_dim(a.d)) return hipErrorInvalidValue;
  if (e == Elt::kBf16)
    return a.d == 64    ? launch_dq_d<EltBf16, 64>(a)
           : a.d == 96  ? launch_dq_d<EltBf16, 96>(a)
           : a.d == 128 ? launch_dq_d<EltBf16, 128>(a)
           : a.d == 192 ? launch_dq_d<EltBf16, 192>(a)
                        : launch_dq_d<EltBf16, 256>(a);
  if (e == Elt::kF16)
    return a.d == 64    ? launch_dq_d<EltF16, 64>(a)
           : a.d == 96  ? launch_dq_d<EltF16, 96>(a)
           : a.d == 128 ? launch_dq_d<EltF16, 128>(a)
           : a.d == 192 ? launch_dq_d<EltF16, 192>(a)
                        : launch_dq_d<EltF16, 256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_half(const BwdArgs& a, Elt e) {
  hipError_t r = launch_bwd_preprocess_half(a, e);
  if (r != hipSuccess) return r;
  r = launch_bwd_dkdv_half(a, e);
  if (r != hipSuccess) return r;
  return launch_bwd_dq_half(a, e);
}

}  // namespace fa
