// fa_bwd_f32.hip - backward kernels for fp32 inputs and outputs.
//
// Method ("What is FlashAttention?", Step 4; "FlashAttention", section "What
// it does not do"; "Explain FlashAttention and why it is IO-aware", section
// "Exact attention, finite precision and backward"): nothing N x N is read
// back; S and P are recomputed tile by tile from Q, K and the saved
// per-row LSE, P = exp(scale * q.k - LSE), and with D_i = sum_t dO_it O_it
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = scale dS^T Q,
//   dQ = scale dS K.
// The same algorithm as the 16-bit kernels, on the fp32 MFMA
// (v_mfma_f32_32x32x2_f32: each lane supplies one fp32 of A and of B, A lane l
// holds row l % 32 and k = l / 32, B lane l holds column l % 32 and the same
// k, and the accumulator lane l holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4).  The result keeps fp32 accuracy end to end.
//
//  * rowdot: one thread per 4 features of a row, D in fp32.
//  * dK/dV: a work-group of two waves owns 64 keys (32 per wave, one key per
//    lane) whose K and V rows stay in LDS; it walks the 32-row query tiles
//    that see them.  S = Q K^T and dP = dO V^T come out with one key per
//    lane and queries in the accumulator index, which is exactly the A
//    operand of dV = P^T dO and dK = dS^T Q: the two rows a lane contributes
//    to one MFMA are its own values for queries q and q + 4.
//  * dQ: a work-group of two waves owns 64 query rows (one query per lane)
//    and walks the 32-key tiles they see, as the forward does: S^T = K Q^T and
//    dP^T = V dO^T with the query's Q and dO in registers, then
//    dQ^T += K^T dS^T, the K^T fragments read across rows of the K tile.
//  * masking on absolute positions (key j visible from row i iff j < L and,
//    when causal, j <= i), only on tiles that cross the key length or the
//    diagonal; masked entries of P are zero, so fully masked rows (LSE = -inf)
//    contribute nothing.

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// waves per work-group: two (64 keys or query rows); the dK/dV kernel uses
// one at d = 256, where K, V, Q and dO tiles of 64 rows would not fit in LDS
template <int D>
struct F32BwdWaves {
  static constexpr int DKDV = D <= 128 ? 2 : 1;   // d >= 192: the split kernel instead
  static constexpr int DQ = 2;
};

// Row pitches in floats: +2 makes the 32-row x 2-column fragment reads
// (row l % 32, column 2 ks + l / 32) hit 64 distinct banks.
template <int D>
struct F32BwdCfg {
  static constexpr int PITCH = D + 2;
  static constexpr int KS = D / 2;     // k-steps of a D-long contraction
  static constexpr int NDB = D / 32;   // 32-feature blocks
  static_assert(D % 32 == 0, "head dimension");
};

// threads per row of the row dot products: the row's D/4 16-byte chunks on
// the next power of two of threads (the spare ones of d = 96 and 192 add zero)
template <int D>
struct RowdotF32Threads {
  static constexpr int value = D / 4 <= 16 ? 16 : D / 4 <= 32 ? 32 : 64;
  static_assert(D / 4 <= 64, "head dimension");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_bwd_rowdot_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                              float* __restrict__ Dout, long long rows) {
  constexpr int TPR = RowdotF32Threads<D>::value;   // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows && part < D / 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(O + row * D + part * 4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(dO + row * D + part * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) Dout[row] = acc;
}

// Copies rows [r0, r0 + n_rows) of a [N][D] head into an LDS tile of pitch
// PITCH (rows past `valid` as zeros), all threads of the work-group.
template <int D>
__device__ __forceinline__ void load_rows(float* tile, const float* head, int r0, int n_rows,
                                          int valid, int tid, int nthreads) {
  using C = F32BwdCfg<D>;
  for (int u = tid; u < n_rows * (D / 4); u += nthreads) {
    const int r = u / (D / 4);
    const int c4 = u % (D / 4);
    const int row = r0 + r;
    const f32x4 x = row < valid ? *reinterpret_cast<const f32x4*>(head + (size_t)row * D + c4 * 4)
                                : f32x4{};
    float* dst = tile + r * C::PITCH + c4 * 4;
    dst[0] = x[0];
    dst[1] = x[1];
    dst[2] = x[2];
    dst[3] = x[3];
  }
}

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
void fa_bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                            const float* __restrict__ V, const float* __restrict__ dO,
                            const float* __restrict__ LSE, const float* __restrict__ Dlt,
                            const int32_t* __restrict__ seqlens_k, float scale, float scale_log2,
                            int causal, float* __restrict__ dK, float* __restrict__ dV, int B,
                            int H, int n_q, int n_k, int n_kblocks,
                            const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                            int total_q, int total_k) {
  using C = F32BwdCfg<D>;
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;       // keys per work-group
  constexpr int QT = 32;            // query rows per tile
  // up to d = 128 each lane keeps the K and V features of its key that it
  // supplies to the MFMAs (2 ks + hi) in registers, so LDS holds only the
  // Q and dO tiles and two work-groups share a CU; above (a path the
  // launcher no longer takes: d >= 192 runs the split kernel) K and V stay
  // in LDS
  constexpr bool kRegKV = D <= 128;
  __shared__ __attribute__((aligned(16))) float Ks[kRegKV ? 4 : BK * C::PITCH];
  __shared__ __attribute__((aligned(16))) float Vs[kRegKV ? 4 : BK * C::PITCH];
  __shared__ __attribute__((aligned(16))) float Qs[QT * C::PITCH];
  __shared__ __attribute__((aligned(16))) float dOs[QT * C::PITCH];
  __shared__ float Ls[QT], Ds[QT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // key blocks in order: under a causal mask block 0 sees every query tile
  const WgOrder wo = wg_order(blockIdx.x, B * H, (int)(gridDim.x / (unsigned)(B * H)));
  const int kb = wo.rank;
  const int bh = wo.bh;
  const int b = bh / H;
  const SeqSpan sp = seq_span(b, bh - b * H, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (kb * BK >= Nk) return;         // a key block past a shorter sequence
  const float* Qh = Q + sp.q_row0 * D;
  const float* Kh = K + sp.k_row0 * D;
  const float* Vh = V + sp.k_row0 * D;
  const float* dOh = dO + sp.q_row0 * D;
  const float* Lh = LSE + sp.q_row0;
  const float* Dh = Dlt + sp.q_row0;
  const int kv_len = key_length(seqlens_k, b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int k0 = kb * BK;
  const int kw0 = k0 + wave * 32;           // this wave's first key
  const int my_key = kw0 + l32;

  float kreg[kRegKV ? C::KS : 1], vreg[kRegKV ? C::KS : 1];
  if constexpr (kRegKV) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bool live = my_key < kv_len;   // keys past the length never enter a product
      kreg[ks] = live ? Kh[(size_t)my_key * D + 2 * ks + hi] : 0.f;
      vreg[ks] = live ? Vh[(size_t)my_key * D + 2 * ks + hi] : 0.f;
    }
  } else {
    load_rows<D>(Ks, Kh, k0, BK, kv_len, tid, NT);
    load_rows<D>(Vs, Vh, k0, BK, kv_len, tid, NT);
  }

  f32x16 dvacc[C::NDB], dkacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  // query tiles that see any key of the block: under the causal mask the
  // first is the one holding row k0; keys past the length are never visible
  const int q_begin = causal ? (max(0, k0 - off) / QT) * QT : 0;
  const bool block_live = k0 < kv_len && q_begin < N;
  const int n_qt = block_live ? (N - q_begin + QT - 1) / QT : 0;
  const bool wave_keys_live = kw0 < kv_len;
  const float* Kw = Ks + wave * 32 * C::PITCH;
  const float* Vw = Vs + wave * 32 * C::PITCH;

  for (int qi = 0; qi < n_qt; ++qi) {
    const int qt0 = q_begin + qi * QT;
    __syncthreads();   // the previous tile's readers are done
    load_rows<D>(Qs, Qh, qt0, QT, N, tid, NT);
    load_rows<D>(dOs, dOh, qt0, QT, N, tid, NT);
    if (tid < QT) {
      const int row = qt0 + tid;
      Ls[tid] = row < N ? Lh[row] : 0.f;
      Ds[tid] = row < N ? Dh[row] : 0.f;
    }
    __syncthreads();
    // causal: the tile's last row precedes this wave's first key
    const bool active = wave_keys_live && (!causal || qt0 + QT - 1 + off >= kw0);
    if (!active) continue;

    // S[q][key] = Q K^T and dP[q][key] = dO V^T: lane = key, v = query row
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    if constexpr (kRegKV) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int col = 2 * ks + hi;
        sacc = mfma_f32(Qs[l32 * C::PITCH + col], kreg[ks], sacc);
        pacc = mfma_f32(dOs[l32 * C::PITCH + col], vreg[ks], pacc);
      }
    } else {
#pragma unroll 8
      for (int ks = 0; ks < C::KS; ++ks) {
        const int col = 2 * ks + hi;
        const float kb_op = Kw[l32 * C::PITCH + col];
        const float vb_op = Vw[l32 * C::PITCH + col];
        sacc = mfma_f32(Qs[l32 * C::PITCH + col], kb_op, sacc);
        pacc = mfma_f32(dOs[l32 * C::PITCH + col], vb_op, pacc);
      }
    }
    const bool need_mask =
        (kw0 + 31 >= kv_len) || (causal && qt0 + off < kw0 + 31) || qt0 + QT > N;
    float p[16], ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = c_row(v, lane);
      float x = fast_exp2(__builtin_fmaf(sacc[v], scale_log2, -Ls[r] * kLog2e));
      if (need_mask) {
        const int q = qt0 + r;
        const bool vis = my_key < kv_len && (!causal || my_key <= q + off) && q < N;
        x = vis ? x : 0.f;
      }
      p[v] = x;
      ds[v] = x * (pacc[v] - Ds[r]);
    }
    // dV += P^T dO and dK += dS^T Q: step v contracts over rows c_row(v, .)
    // (the pair q, q + 4 of the two lane halves)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = c_row(v, lane);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        dvacc[db] = mfma_f32(p[v], dOs[r * C::PITCH + db * 32 + l32], dvacc[db]);
        dkacc[db] = mfma_f32(ds[v], Qs[r * C::PITCH + db * 32 + l32], dkacc[db]);
      }
    }
  }

  // dV[key][feature], dK = scale * acc: accumulator lane l holds feature
  // 32 db + l % 32 of keys kw0 + c_row(v, l)
  float* dKh = dK + sp.k_row0 * D;
  float* dVh = dV + sp.k_row0 * D;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kw0 + c_row(v, lane);
      if (key < Nk) {
        dVh[(size_t)key * D + db * 32 + l32] = dvacc[db][v];
        dKh[(size_t)key * D + db * 32 + l32] = dkacc[db][v] * scale;
      }
    }
}

// dK/dV at d >= 192.  A work-group of one wave per 32 keys would need K, V,
// Q and dO tiles of 32 rows in LDS (100-133 KB), so one such work-group per
// CU would leave three SIMDs idle.  Here four waves share the 32 keys and
// split the feature dimension: wave w holds the K and V features of k-steps
// w, w + 4, ... in registers and computes the partial S = Q K^T and
// dP = dO V^T over them; the four partials meet in LDS and every wave adds
// them in the same order (so all hold the same S and dP), forms P and dS,
// and accumulates dV += P^T dO and dK += dS^T Q for its feature blocks
// w, w + 4, ...  Three barriers per query tile.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_bwd_dkdv_f32_split_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                  const float* __restrict__ V, const float* __restrict__ dO,
                                  const float* __restrict__ LSE, const float* __restrict__ Dlt,
                                  const int32_t* __restrict__ seqlens_k, float scale,
                                  float scale_log2, int causal, float* __restrict__ dK,
                                  float* __restrict__ dV, int B, int H, int n_q, int n_k,
                                  int n_kblocks, const int32_t* __restrict__ cu_q,
                                  const int32_t* __restrict__ cu_k, int total_q, int total_k) {
  using C = F32BwdCfg<D>;
  constexpr int NW = 4;
  constexpr int NT = NW * 64;
  constexpr int BK = 32;              // keys per work-group
  constexpr int QT = 32;              // query rows per tile
  constexpr int KSW = C::KS / NW;     // k-steps per wave
  constexpr int NBW = (C::NDB + NW - 1) / NW;   // feature blocks per wave (at most)
  static_assert(C::KS % NW == 0, "k-steps split evenly over the waves");
  __shared__ __attribute__((aligned(16))) float Qs[QT * C::PITCH];
  __shared__ __attribute__((aligned(16))) float dOs[QT * C::PITCH];
  __shared__ float Ls[QT], Ds[QT];
  // partial S and dP of each wave, [tensor][wave][chunk][lane]
  __shared__ __attribute__((aligned(16))) f32x4 Xp[2][NW][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // key blocks in order: under a causal mask block 0 sees every query tile
  const WgOrder wo = wg_order(blockIdx.x, B * H, n_kblocks);
  const int kb = wo.rank;
  const int bh = wo.bh;
  const int b = bh / H;
  const SeqSpan sp = seq_span(b, bh - b * H, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (kb * BK >= Nk) return;         // a key block past a shorter sequence
  const float* Qh = Q + sp.q_row0 * D;
  const float* Kh = K + sp.k_row0 * D;
  const float* Vh = V + sp.k_row0 * D;
  const float* dOh = dO + sp.q_row0 * D;
  const float* Lh = LSE + sp.q_row0;
  const float* Dh = Dlt + sp.q_row0;
  const int kv_len = key_length(seqlens_k, b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int k0 = kb * BK;
  const int my_key = k0 + l32;

  // this wave's K and V features (k-steps ks = wave + 4 i) of this lane's key
  float kreg[KSW], vreg[KSW];
  {
    const bool live = my_key < kv_len;   // keys past the length never enter a product
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int col = 2 * (wave + NW * i) + hi;
      kreg[i] = live ? Kh[(size_t)my_key * D + col] : 0.f;
      vreg[i] = live ? Vh[(size_t)my_key * D + col] : 0.f;
    }
  }

  f32x16 dvacc[NBW], dkacc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    dvacc[i] = f32x16{};
    dkacc[i] = f32x16{};
  }

  // query tiles that see any key of the block: under the causal mask the
  // first is the one holding row k0; keys past the length are never visible
  const int q_begin = causal ? (max(0, k0 - off) / QT) * QT : 0;
  const bool block_live = k0 < kv_len && q_begin < N;
  const int n_qt = block_live ? (N - q_begin + QT - 1) / QT : 0;

  for (int qi = 0; qi < n_qt; ++qi) {
    const int qt0 = q_begin + qi * QT;
    __syncthreads();   // the previous tile's readers (Q, dO, partials) are done
    load_rows<D>(Qs, Qh, qt0, QT, N, tid, NT);
    load_rows<D>(dOs, dOh, qt0, QT, N, tid, NT);
    if (tid < QT) {
      const int row = qt0 + tid;
      Ls[tid] = row < N ? Lh[row] : 0.f;
      Ds[tid] = row < N ? Dh[row] : 0.f;
    }
    __syncthreads();

    // partial S[q][key] and dP[q][key] over this wave's k-steps: lane = key,
    // v = query row
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int col = 2 * (wave + NW * i) + hi;
      sacc = mfma_f32(Qs[l32 * C::PITCH + col], kreg[i], sacc);
      pacc = mfma_f32(dOs[l32 * C::PITCH + col], vreg[i], pacc);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Xp[0][wave][c][lane] = f32x4{sacc[4 * c], sacc[4 * c + 1], sacc[4 * c + 2], sacc[4 * c + 3]};
      Xp[1][wave][c][lane] = f32x4{pacc[4 * c], pacc[4 * c + 1], pacc[4 * c + 2], pacc[4 * c + 3]};
    }
    __syncthreads();
    // the full S and dP: the four partials added in wave order
    float sf[16], pf[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 s4 = Xp[0][0][c][lane], p4 = Xp[1][0][c][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        s4 += Xp[0][w][c][lane];
        p4 += Xp[1][w][c][lane];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sf[4 * c + e] = s4[e];
        pf[4 * c + e] = p4[e];
      }
    }

    const bool need_mask =
        (k0 + BK - 1 >= kv_len) || (causal && qt0 + off < k0 + BK - 1) || qt0 + QT > N;
    float p[16], ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = c_row(v, lane);
      float x = fast_exp2(__builtin_fmaf(sf[v], scale_log2, -Ls[r] * kLog2e));
      if (need_mask) {
        const int q = qt0 + r;
        const bool vis = my_key < kv_len && (!causal || my_key <= q + off) && q < N;
        x = vis ? x : 0.f;
      }
      p[v] = x;
      ds[v] = x * (pf[v] - Ds[r]);
    }
    // dV += P^T dO and dK += dS^T Q over this wave's feature blocks: step v
    // contracts over rows c_row(v, .)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = c_row(v, lane);
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int db = wave + NW * i;
        if (db < C::NDB) {
          dvacc[i] = mfma_f32(p[v], dOs[r * C::PITCH + db * 32 + l32], dvacc[i]);
          dkacc[i] = mfma_f32(ds[v], Qs[r * C::PITCH + db * 32 + l32], dkacc[i]);
        }
      }
    }
  }

  // dV[key][feature], dK = scale * acc: accumulator lane l holds feature
  // 32 db + l % 32 of keys k0 + c_row(v, l)
  float* dKh = dK + sp.k_row0 * D;
  float* dVh = dV + sp.k_row0 * D;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int db = wave + NW * i;
    if (db >= C::NDB) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + c_row(v, lane);
      if (key < Nk) {
        dVh[(size_t)key * D + db * 32 + l32] = dvacc[i][v];
        dKh[(size_t)key * D + db * 32 + l32] = dkacc[i][v] * scale;
      }
    }
  }
}

// dQ: at d >= 192 one wave per SIMD holds the query's Q and dO rows in
// registers (the loop below fully unrolled); below, two or three waves per
// SIMD read them from scratch memory (L1-resident) in a loop unrolled by 8,
// which measured faster there (d = 128: 27 against 24 TFLOP/s; d = 256: 17
// against 23 the other way round)
template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(1, D >= 192 ? 1 : 8)))
void fa_bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                          const float* __restrict__ V, const float* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dlt,
                          const int32_t* __restrict__ seqlens_k, float scale, float scale_log2,
                          int causal, float* __restrict__ dQ, int B, int H, int n_q, int n_k,
                          int n_qtiles, const int32_t* __restrict__ cu_q,
                          const int32_t* __restrict__ cu_k, int total_q, int total_k) {
  using C = F32BwdCfg<D>;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;       // query rows per work-group
  constexpr int BC = 32;            // keys per tile
  __shared__ __attribute__((aligned(16))) float Ks[BC * C::PITCH];
  __shared__ __attribute__((aligned(16))) float Vs[BC * C::PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_coord(blockIdx.x, B, H, n_qtiles);
  const SeqSpan sp = seq_span(tc.b, tc.h, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (tc.qt * BR >= N) return;       // a query tile past a shorter sequence
  const float* Qh = Q + sp.q_row0 * D;
  const float* Kh = K + sp.k_row0 * D;
  const float* Vh = V + sp.k_row0 * D;
  const float* dOh = dO + sp.q_row0 * D;
  const int kv_len = key_length(seqlens_k, tc.b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int q0 = tc.qt * BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  // this lane's query row: Q and dO as B operands, LSE and D in registers
  float qf[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = qrow < N ? Qh[(size_t)qrow * D + 2 * ks + hi] : 0.f;
    of[ks] = qrow < N ? dOh[(size_t)qrow * D + 2 * ks + hi] : 0.f;
  }
  const float lse2 = qrow < N ? LSE[sp.q_row0 + qrow] * kLog2e : 0.f;
  const float drow = qrow < N ? Dlt[sp.q_row0 + qrow] : 0.f;

  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, max(0, min(q0 + BR + off, Nk)));
  const int n_kt = (kv_end + BC - 1) / BC;

  f32x16 dqacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dqacc[db] = f32x16{};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * BC;
    __syncthreads();
    load_rows<D>(Ks, Kh, key0, BC, kv_len, tid, NT);
    load_rows<D>(Vs, Vh, key0, BC, kv_len, tid, NT);
    __syncthreads();
    const bool active = qw0 < N && (!causal || key0 <= qw0 + 31 + off);
    if (!active) continue;

    // S^T = K Q^T, dP^T = V dO^T: lane = query, v = key
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    if constexpr (D >= 192) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int col = 2 * ks + hi;
        sacc = mfma_f32(Ks[l32 * C::PITCH + col], qf[ks], sacc);
        pacc = mfma_f32(Vs[l32 * C::PITCH + col], of[ks], pacc);
      }
    } else {
#pragma unroll 8
      for (int ks = 0; ks < C::KS; ++ks) {
        const int col = 2 * ks + hi;
        sacc = mfma_f32(Ks[l32 * C::PITCH + col], qf[ks], sacc);
        pacc = mfma_f32(Vs[l32 * C::PITCH + col], of[ks], pacc);
      }
    }
    const bool need_mask = (key0 + BC > kv_len) || (causal && key0 + BC - 1 > qw0 + off);
    float ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = key0 + c_row(v, lane);
      float x = fast_exp2(__builtin_fmaf(sacc[v], scale_log2, -lse2));
      if (need_mask) {
        const bool vis = key < kv_len && (!causal || key <= qrow + off);
        x = vis ? x : 0.f;
      }
      ds[v] = x * (pacc[v] - drow);
    }
    // dQ^T += K^T dS^T: step v contracts over keys c_row(v, .)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kr = c_row(v, lane);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        dqacc[db] = mfma_f32(Ks[kr * C::PITCH + db * 32 + l32], ds[v], dqacc[db]);
    }
  }

  // dQ^T accumulator lane l holds query l % 32 and features
  // 32 db + 8 (v / 4) + 4 (l / 32) + v % 4
  if (qrow < N) {
    float* dQh = dQ + sp.q_row0 * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * hi;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = dqacc[db][4 * v4 + e] * scale;
        *reinterpret_cast<f32x4*>(dQh + (size_t)qrow * D + d0) = w;
      }
  }
}

template <int D>
hipError_t launch_preprocess_f32_d(const BwdArgs& a) {
  const long long rows = a.cu_q ? (long long)a.H * a.total_q : (long long)a.B * a.H * a.N;
  if (rows == 0) return hipSuccess;
  const long long threads = rows * RowdotF32Threads<D>::value;
  hipLaunchKernelGGL((fa_bwd_rowdot_f32_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, a.stream, static_cast<const float*>(a.o),
                     static_cast<const float*>(a.dout), a.delta, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_f32_d(const BwdArgs& a) {
  if constexpr (D >= 192) {
    const int n_kblocks = (a.Nk + 31) / 32;
    if (n_kblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((fa_bwd_dkdv_f32_split_kernel<D>),
                       dim3((unsigned)((long long)n_kblocks * a.B * a.H)), dim3(256), 0,
                       a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<const float*>(a.dout), a.lse,
                       a.delta, a.seqlens_k, a.scale, a.scale * kLog2e, a.causal,
                       static_cast<float*>(a.dk), static_cast<float*>(a.dv), a.B, a.H, a.N,
                       a.Nk, n_kblocks, a.cu_q, a.cu_k, a.total_q, a.total_k);
    return hipGetLastError();
  } else {
    constexpr int NW = F32BwdWaves<D>::DKDV;
    const int n_kblocks = (a.Nk + NW * 32 - 1) / (NW * 32);
    if (n_kblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((fa_bwd_dkdv_f32_kernel<D, NW>),
                       dim3((unsigned)((long long)n_kblocks * a.B * a.H)), dim3(NW * 64), 0,
                       a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<const float*>(a.dout), a.lse,
                       a.delta, a.seqlens_k, a.scale, a.scale * kLog2e, a.causal,
                       static_cast<float*>(a.dk), static_cast<float*>(a.dv), a.B, a.H, a.N,
                       a.Nk, n_kblocks, a.cu_q, a.cu_k, a.total_q, a.total_k);
    return hipGetLastError();
  }
}

template <int D>
hipError_t launch_dq_f32_d(const BwdArgs& a) {
  constexpr int NW = F32BwdWaves<D>::DQ;
  const int n_qtiles = (a.N + NW * 32 - 1) / (NW * 32);
  if (n_qtiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fa_bwd_dq_f32_kernel<D, NW>),
                     dim3((unsigned)((long long)n_qtiles * a.B * a.H)), dim3(NW * 64), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<const float*>(a.dout), a.lse,
                     a.delta, a.seqlens_k, a.scale, a.scale * kLog2e, a.causal,
                     static_cast<float*>(a.dq), a.B, a.H, a.N, a.Nk, n_qtiles,
                     a.cu_q, a.cu_k, a.total_q, a.total_k);
  return hipGetLastError();
}

}  // namespace

long long bwd_f32_grid(int B, int H, int N, int d) {
  (void)d;
  const long long tiles = (N + 31) / 32;   // the smallest row block of either kernel
  const int tpr = d / 4 <= 16 ? 16 : d / 4 <= 32 ? 32 : 64;   // RowdotF32Threads
  const long long rows_wg = ((long long)B * H * N * tpr + 255) / 256;
  const long long m = tiles * B * H;
  return rows_wg > m ? rows_wg : m;
}

hipError_t launch_bwd_preprocess_f32(const BwdArgs& a) {
  if (a.d == 64) return launch_preprocess_f32_d<64>(a);
  if (a.d == 96) return launch_preprocess_f32_d<96>(a);
  if (a.d == 128) return launch_preprocess_f32_d<128>(a);
  if (a.d == 192) return launch_preprocess_f32_d<192>(a);
  if (a.d == 256) return launch_preprocess_f32_d<256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_f32(const BwdArgs& a) {
  if (a.d == 64) return launch_dkdv_f32_d<64>(a);
  if (a.d == 96) return launch_dkdv_f32_d<96>(a);
  if (a.d == 128) return launch_dkdv_f32_d<128>(a);
  if (a.d == 192) return launch_dkdv_f32_d<192>(a);
  if (a.d == 256) return launch_dkdv_f32_d<256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_f32(const BwdArgs& a) {
  if (a.d == 64) return launch_dq_f32_d<64>(a);
  if (a.d == 96) return launch_dq_f32_d<96>(a);
  if (a.d == 128) return launch_dq_f32_d<128>(a);
  if (a.d == 192) return launch_dq_f32_d<192>(a);
  if (a.d == 256) return launch_dq_f32_d<256>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32(const BwdArgs& a) {
  hipError_t r = launch_bwd_preprocess_f32(a);
  if (r != hipSuccess) return r;
  r = launch_bwd_dkdv_f32(a);
  if (r != hipSuccess) return r;
  return launch_bwd_dq_f32(a);
}

}  // namespace fa
