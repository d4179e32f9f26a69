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
//     accumulators resident, and loops over 64-row query tiles staged in LDS
//     both row-major (A operands of S and dP) and transposed with a permuted
//     row order (B operands of dV and dK).  S and dP come out with one key per
//     lane, so P and dS feed the next MFMA straight from registers;
//  3. dQ: a work-group owns query rows (like the forward) and loops over key
//     tiles; S^T and dP^T come out with one query per lane, so LSE_i and D_i
//     are one register each, and dS^T feeds dQ^T = K^T dS^T from registers.
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

namespace fa {

namespace {

// Position of element (4*grp + r) of a 4-element group inside the permuted
// order used for transposed LDS copies: within each 16-element group the
// middle two 4-element chunks are swapped, so that the 8 elements a lane
// feeds into one 32x32x16 MFMA (rows 16u + 8*(i/4) + 4*hi + i%4 of a C tile)
// are contiguous.
// (The chunk swap exchanges the two low bits of the group index.)
__device__ __forceinline__ int perm_pos(int grp) {
  return 16 * (grp >> 2) + 4 * (((grp & 1) << 1) | ((grp >> 1) & 1));
}

// Write 4 rows x 8 features (four 16-byte row chunks) transposed into a
// [feature][row] LDS array at column `pos`.
__device__ __forceinline__ void store_transposed(__bf16* dst, int pitch, int feat0, int pos,
                                                 const u32x4 (&rows)[4]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const int sh = (j & 1) * 16;
    u32x2 pk;
    pk[0] = ((rows[0][w] >> sh) & 0xffffu) | (((rows[1][w] >> sh) & 0xffffu) << 16);
    pk[1] = ((rows[2][w] >> sh) & 0xffffu) | (((rows[3][w] >> sh) & 0xffffu) << 16);
    *reinterpret_cast<u32x2*>(dst + (feat0 + j) * pitch + pos) = pk;
  }
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_t dO_it O_it (fp32), one row per D/8 threads
// ---------------------------------------------------------------------------
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_bwd_rowdot_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                          float* __restrict__ Dout, long long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(a[w] << 16) * __uint_as_float(b[w] << 16);
      acc += __uint_as_float(a[w] & 0xffff0000u) * __uint_as_float(b[w] & 0xffff0000u);
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
// SIMD, without any duplicated MFMA work.
// ---------------------------------------------------------------------------
template <int D, int BQ>
struct DkdvPairCfg {
  static constexpr int NW = 8;
  static constexpr int BK = 128;           // keys per work-group (4 pairs x 32)
  static constexpr int NT = NW * 64;
  static constexpr int KS = D / 16;
  static constexpr int NG = BQ / 16;       // 16-query groups per tile
  static constexpr int NDB = D / 32;
  static constexpr int HDB = NDB / 2;      // 32-feature blocks per wave (its half)
  static constexpr int TPITCH = BQ + 8;
  static constexpr int UNITS = (BQ / 4) * (D / 8);  // 4-row x 8-feature units per tensor
  static_assert(BQ == 64, "two 32-row halves per tile");
  static_assert(NDB % 2 == 0, "head dimension splits in two halves of 32-feature blocks");
  static_assert(2 * UNITS <= NT, "one staging unit per thread");
};

template <int D, int BQ>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_pair_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                             const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                             const float* __restrict__ LSE, const float* __restrict__ Dlt,
                             const int32_t* __restrict__ seqlens_k, float scale,
                             float scale_log2, int causal, __bf16* __restrict__ dK,
                             __bf16* __restrict__ dV, int B, int H, int N, int n_ktiles) {
  using C = DkdvPairCfg<D, BQ>;
  __shared__ __attribute__((aligned(16))) __bf16 Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 Qt[D * C::TPITCH];
  __shared__ __attribute__((aligned(16))) __bf16 dOt[D * C::TPITCH];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];
  // P and dS fragments handed to the partner wave: [wave][slot][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 Xs[C::NW][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int pr = wave & 3;      // key block of the pair
  const int half = wave >> 2;   // query half for S/dP, feature half for dK/dV

  const int bh_count = B * H;
  const int kt = blockIdx.x / bh_count;
  const int bh = blockIdx.x - kt * bh_count;
  const int b = bh / H;
  const int h = bh - b * H;
  const size_t head = (size_t)b * H + h;
  const __bf16* Qh = Q + head * (size_t)N * D;
  const __bf16* Kh = K + head * (size_t)N * D;
  const __bf16* Vh = V + head * (size_t)N * D;
  const __bf16* dOh = dO + head * (size_t)N * D;
  const float* Lh = LSE + head * (size_t)N;
  const float* Dh = Dlt + head * (size_t)N;
  __bf16* dKh = dK + head * (size_t)N * D;
  __bf16* dVh = dV + head * (size_t)N * D;

  const int kv_len = key_length(seqlens_k, b, N);
  const int k0 = kt * C::BK;
  const int kw0 = k0 + pr * 32;
  const int my_key = kw0 + l32;
  const int q_begin = causal ? (k0 / BQ) * BQ : 0;
  const int n_qt = (k0 < kv_len) ? (N - q_begin + BQ - 1) / BQ : 0;

  // the pair's K and V rows (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (my_key < N) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)my_key * D + ks * 16 + hi * 8);
      vf[ks] = *reinterpret_cast<const bf16x8*>(Vh + (size_t)my_key * D + ks * 16 + hi * 8);
    } else {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
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
  // position.  The transposed copies are then built from the row-major ones.
  constexpr int kRowsPerBlk = 1024 / (D * 2);
  constexpr int kBlksPerTensor = BQ / kRowsPerBlk;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / C::NW;
  static_assert(2 * kBlksPerTensor % C::NW == 0, "whole 1 KiB blocks per wave");
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Qh), 0, head_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t o_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dOh), 0, head_bytes, kBufferRsrcWord3);
  const int blk_row = lane / (D / 8);
  const int blk_cpos = lane % (D / 8);
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
      const int row = rb * kRowsPerBlk + blk_row;
      const int chunk = blk_cpos ^ row_swizzle<D>(row);
      const int voff = (qt0 + row) * (D * 2) + chunk * 16;
      __bf16* dst = (is_q ? Qs[buf] : dOs[buf]) + rb * kRowsPerBlk * D;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_q ? q_rsrc : o_rsrc, dst, 16, voff, 0, 0, 0);
    }
  };
  auto store_stats = [&](int buf) FA_INLINE {
    if (tid < BQ) {
      // rows past N, and rows that see no key, get +inf so that P = 0
      Ls[buf][tid] = (lreg == kNegInf) ? __builtin_huge_valf() : lreg * kLog2e;
      Ds[buf][tid] = dreg;
    }
  };
  // transposed copies of the row-major tile in `buf`: threads [0, UNITS)
  // handle Q, [UNITS, 2 UNITS) dO, one 4-row x 8-feature unit each
  const bool stager = tid < 2 * C::UNITS;
  const bool stage_q = tid < C::UNITS;
  const int su = tid % C::UNITS;
  const int sqg = su % (BQ / 4);
  const int sdc = su / (BQ / 4);
  auto transpose_tile = [&](int buf) FA_INLINE {
    if (stager) {
      const __bf16* rm = stage_q ? Qs[buf] : dOs[buf];
      u32x4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * sqg + r;
        rows[r] = *reinterpret_cast<const u32x4*>(&rm[row * D + (sdc ^ row_swizzle<D>(row)) * 8]);
      }
      store_transposed(stage_q ? Qt : dOt, C::TPITCH, sdc * 8, perm_pos(sqg), rows);
    }
  };

  if (n_qt > 0) {
    issue_tile(0, 0);
    store_stats(0);
    wait_vmem();
    __syncthreads();
    transpose_tile(0);
    __syncthreads();
  }

  const bool pair_keys_valid = kw0 < kv_len;
  for (int qi = 0; qi < n_qt; ++qi) {
    const int buf = qi & 1;
    const int qt0 = q_begin + qi * BQ;
    const bool more = qi + 1 < n_qt;
    if (more) issue_tile(qi + 1, buf ^ 1);
    const bool pair_active = pair_keys_valid && (!causal || qt0 + BQ - 1 >= kw0);

    bf16x8 pa[2], dsa[2];
    if (pair_active) {
      // ---- phase 1: S and dP for this wave's 32 query rows (one key per lane)
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const int arow = 32 * half + l32;
      const int asw = row_swizzle<D>(arow);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int ro = arow * D + ((2 * ks + hi) ^ asw) * 8;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[buf][ro]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&dOs[buf][ro]);
        sacc = mfma_bf16(qa, kf[ks], sacc);
        pacc = mfma_bf16(oa, vf[ks], pacc);
      }
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
            if (kMasked) {
              const int query = qt0 + r0 + e;
              const bool vis = my_key < kv_len && (!causal || my_key <= query);
              p = vis ? p : 0.f;
            }
            pa[v >> 3][v & 7] = to_bf16(p);
            dsa[v >> 3][v & 7] = to_bf16(p * (pacc[v] - dq[e]));
          }
        }
      };
      if ((kw0 + 31 >= kv_len) || (causal && qt0 + 32 * half < kw0 + 31))
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
      const int partner = wave ^ 4;
      bf16x8 po[2], dso[2];
      po[0] = Xs[partner][0][lane];
      po[1] = Xs[partner][1][lane];
      dso[0] = Xs[partner][2][lane];
      dso[1] = Xs[partner][3][lane];
#pragma unroll
      for (int g = 0; g < C::NG; ++g) {
        // groups 2*half, 2*half+1 are this wave's rows; the others the partner's
        const bool own = (g >> 1) == half;
        const bf16x8 pfrag = own ? pa[g & 1] : po[g & 1];
        const bf16x8 dsfrag = own ? dsa[g & 1] : dso[g & 1];
#pragma unroll
        for (int j = 0; j < C::HDB; ++j) {
          const int db = half * C::HDB + j;
          const int to = (db * 32 + l32) * C::TPITCH + g * 16 + hi * 8;
          const bf16x8 ob = *reinterpret_cast<const bf16x8*>(&dOt[to]);
          const bf16x8 qbv = *reinterpret_cast<const bf16x8*>(&Qt[to]);
          dvacc[j] = mfma_bf16(pfrag, ob, dvacc[j]);
          dkacc[j] = mfma_bf16(dsfrag, qbv, dkacc[j]);
        }
      }
    }
    // the next tile's row-major copy has landed once every wave passes here
    wait_vmem();
    lds_barrier();
    if (more) transpose_tile(buf ^ 1);
  }

  // ---- write dK = scale * acc, dV = acc for this wave's feature half
#pragma unroll
  for (int j = 0; j < C::HDB; ++j) {
    const int db = half * C::HDB + j;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kw0 + c_row(v, lane);
      if (key < N) {
        dKh[(size_t)key * D + db * 32 + l32] = to_bf16(dkacc[j][v] * scale);
        dVh[(size_t)key * D + db * 32 + l32] = to_bf16(dvacc[j][v]);
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
  static constexpr int TPITCH = BC + 8;
  static constexpr int UNITS = (BC / 4) * (D / 8);
  static constexpr int UPT = (UNITS + NT - 1) / NT;
};

template <int D, int NW, int BC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1, NW >= 8 ? 2 : 1)))
void fa_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                      const float* __restrict__ LSE, const float* __restrict__ Dlt,
                      const int32_t* __restrict__ seqlens_k, float scale, float scale_log2,
                      int causal, __bf16* __restrict__ dQ, int B, int H, int N, int n_qtiles) {
  using C = DqCfg<D, NW, BC>;
  // row-major K and V tiles in three slots (read, being transposed, being
  // loaded), transposed K in two
  __shared__ __attribute__((aligned(16))) __bf16 Ks[3][BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[3][BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 Kt[2][D * C::TPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_coord(blockIdx.x, B, H, n_qtiles);
  const size_t head = (size_t)tc.b * H + tc.h;
  const __bf16* Qh = Q + head * (size_t)N * D;
  const __bf16* Kh = K + head * (size_t)N * D;
  const __bf16* Vh = V + head * (size_t)N * D;
  const __bf16* dOh = dO + head * (size_t)N * D;
  __bf16* dQh = dQ + head * (size_t)N * D;

  const int kv_len = key_length(seqlens_k, tc.b, N);
  const int q0 = tc.qt * C::BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, min(q0 + C::BR, N));
  const int n_kt = (kv_end + BC - 1) / BC;

  bf16x8 qf[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (qrow < N) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + ks * 16 + hi * 8);
      of[ks] = *reinterpret_cast<const bf16x8*>(dOh + (size_t)qrow * D + ks * 16 + hi * 8);
    } else {
      qf[ks] = bf16x8{};
      of[ks] = bf16x8{};
    }
  }
  float lse2 = __builtin_huge_valf(), drow = 0.f;
  if (qrow < N) {
    const float lse = LSE[head * (size_t)N + qrow];
    lse2 = (lse == kNegInf) ? __builtin_huge_valf() : lse * kLog2e;
    drow = Dlt[head * (size_t)N + qrow];
  }

  f32x16 dqacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dqacc[db] = f32x16{};

  // Staging.  Row-major K and V tiles are copied straight from global memory
  // into LDS (lane l of a wave fills bytes [16 l, 16 l + 16) of a 1 KiB
  // block; each lane fetches the global chunk that the XOR swizzle places
  // there), two tiles ahead.  The buffer descriptors cover exactly one head,
  // so keys at or past N read as zeros; keys in [L_b, N) are masked.  Tile
  // t+1's transposed K copy is built from its row-major copy during
  // iteration t, so one barrier per tile suffices.
  constexpr int kRowsPerBlk = 1024 / (D * 2);
  constexpr int kBlksPerTensor = BC / kRowsPerBlk;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / NW;
  static_assert(2 * kBlksPerTensor % NW == 0 && kBlksPerWave >= 1, "whole 1 KiB blocks per wave");
  static_assert(C::UNITS <= C::NT, "one transposition unit per thread");
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Kh), 0, head_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Vh), 0, head_bytes, kBufferRsrcWord3);
  const int blk_row = lane / (D / 8);
  const int blk_cpos = lane % (D / 8);
  auto issue_tile = [&](int kt, int slot) FA_INLINE {
#pragma unroll
    for (int j = 0; j < kBlksPerWave; ++j) {
      const int blk = wave * kBlksPerWave + j;
      const bool is_k = blk < kBlksPerTensor;
      const int rb = is_k ? blk : blk - kBlksPerTensor;
      const int row = rb * kRowsPerBlk + blk_row;
      const int chunk = blk_cpos ^ row_swizzle<D>(row);
      const int voff = (kt * BC + row) * (D * 2) + chunk * 16;
      __bf16* dst = (is_k ? Ks[slot] : Vs[slot]) + rb * kRowsPerBlk * D;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_k ? k_rsrc : v_rsrc, dst, 16, voff, 0, 0, 0);
    }
  };
  const int tkg = tid % (BC / 4);
  const int tdc = tid / (BC / 4);
  auto transpose_tile = [&](int slot, int tbuf) FA_INLINE {
    if (tid < C::UNITS) {
      u32x4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * tkg + r;
        rows[r] = *reinterpret_cast<const u32x4*>(
            &Ks[slot][row * D + (tdc ^ row_swizzle<D>(row)) * 8]);
      }
      store_transposed(Kt[tbuf], C::TPITCH, tdc * 8, perm_pos(tkg), rows);
    }
  };

  if (n_kt > 0) {
    issue_tile(0, 0);
    if (n_kt > 1) issue_tile(1, 1);
    wait_vmem();
    __syncthreads();
    transpose_tile(0, 0);
    __syncthreads();
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const int slot = kt % 3;
    const int buf = kt & 1;
    if (kt + 2 < n_kt) issue_tile(kt + 2, (kt + 2) % 3);
    if (kt + 1 < n_kt) transpose_tile((kt + 1) % 3, buf ^ 1);
    const int key0 = kt * BC;
    const bool wave_active = (qw0 < N) && (!causal || key0 <= qw0 + 31);
    if (wave_active) {
      // ---- S^T = K Q^T, dP^T = V dO^T (C: one query per lane, rows = keys)
      f32x16 sacc[C::NCB], pacc[C::NCB];
#pragma unroll
      for (int c = 0; c < C::NCB; ++c) {
        sacc[c] = f32x16{};
        pacc[c] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int c = 0; c < C::NCB; ++c) {
          const int arow = c * 32 + l32;
          const int ro = arow * D + ((2 * ks + hi) ^ row_swizzle<D>(arow)) * 8;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[slot][ro]);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[slot][ro]);
          sacc[c] = mfma_bf16(ka, qf[ks], sacc[c]);
          pacc[c] = mfma_bf16(va, of[ks], pacc[c]);
        }
      const bool need_mask = (key0 + BC > kv_len) || (causal && key0 + BC - 1 > qw0);
      bf16x8 dsb[C::NG];
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = fast_exp2(__builtin_fmaf(sacc[c][v], scale_log2, -lse2));
          if (need_mask) {
            const int key = key0 + c * 32 + c_row(v, lane);
            const bool vis = key < kv_len && (!causal || key <= qrow);
            if (!vis) p = 0.f;
          }
          dsb[2 * c + (v >> 3)][v & 7] = to_bf16(p * (pacc[c][v] - drow));
        }
      // ---- dQ^T += K^T dS^T
#pragma unroll
      for (int g = 0; g < C::NG; ++g)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
              &Kt[buf][(db * 32 + l32) * C::TPITCH + g * 16 + hi * 8]);
          dqacc[db] = mfma_bf16(ka, dsb[g], dqacc[db]);
        }
    }
    // tile t+2 has landed and tile t+1's transposed copy is complete once
    // every wave passes here
    wait_vmem();
    lds_barrier();
  }

  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * hi;
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_bf16(dqacc[db][4 * v4 + e] * scale);
        *reinterpret_cast<bf16x4*>(dQh + (size_t)qrow * D + d0) = w;
      }
  }
}

constexpr int kDqNW = FA_DQ_NW, kDqBC = FA_DQ_BC;

template <int D>
hipError_t launch_preprocess_d(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  const long long threads = rows * (D / 8);
  hipLaunchKernelGGL((fa_bwd_rowdot_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, a.stream, static_cast<const __bf16*>(a.o),
                     static_cast<const __bf16*>(a.dout), a.delta, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdArgs& a) {
  using CK = DkdvPairCfg<D, 64>;
  const int n_ktiles = (a.N + CK::BK - 1) / CK::BK;
  hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<D, 64>),
                     dim3((unsigned)((long long)n_ktiles * a.B * a.H)), dim3(CK::NT), 0, a.stream,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dout), a.lse,
                     a.delta, a.seqlens_k, a.scale, a.scale * kLog2e, a.causal,
                     static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), a.B, a.H, a.N,
                     n_ktiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const BwdArgs& a) {
  using CQ = DqCfg<D, kDqNW, kDqBC>;
  const int n_qtiles = (a.N + CQ::BR - 1) / CQ::BR;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, kDqNW, kDqBC>),
                     dim3((unsigned)((long long)n_qtiles * a.B * a.H)), dim3(CQ::NT), 0, a.stream,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dout), a.lse,
                     a.delta, a.seqlens_k, a.scale, a.scale * kLog2e, a.causal,
                     static_cast<__bf16*>(a.dq), a.B, a.H, a.N, n_qtiles);
  return hipGetLastError();
}

}  // namespace

long long bwd_bf16_grid(int B, int H, int N, int d) {
  (void)d;
  const long long kt = (N + 127) / 128;
  const long long qt = (N + kDqNW * 32 - 1) / (kDqNW * 32);
  const long long rows_wg = ((long long)B * H * N * 16 + 255) / 256;
  long long m = kt * B * H;
  if (qt * B * H > m) m = qt * B * H;
  if (rows_wg > m) m = rows_wg;
  return m;
}

hipError_t launch_bwd_preprocess_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_preprocess_d<64>(a);
    case 128: return launch_preprocess_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_dkdv_d<64>(a);
    case 128: return launch_dkdv_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_dq_d<64>(a);
    case 128: return launch_dq_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  hipError_t e = launch_bwd_preprocess_bf16(a);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv_bf16(a);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(a);
}

}  // namespace fa
