// fa_fwd.hip - forward kernels: exact attention with the online softmax.
//
// Method ("FlashAttention", section "Why it is allowed to be exact";
// "Explain FlashAttention and why it is IO-aware", section "Keep only the
// state needed for the final weighted average"): for every query row keep
// the running maximum m, the running sum l of exp(s - m) and the unnormalised
// output o; when a key tile raises the maximum, multiply l and o by
// exp(m_old - m_new) before adding the tile; divide o by l after the last
// tile.  Query-outer loop order ("What is FlashAttention?", Step 3): a
// work-group keeps its query tile, its o accumulators and its statistics on
// chip and writes O and one LSE per row once.
//
// gfx950 mapping (bf16 kernel):
//  * a work-group of 8 waves owns 256 consecutive query rows of one (batch,
//    head); each wave owns 32 queries, one query per lane (lanes l and l^32
//    share a query).  A wave fits in 256 VGPRs, so two waves share a SIMD.
//  * Q stays in VGPRs as the B operand of S^T = K Q^T (32x32x16 bf16 MFMA).
//  * K and V tiles of 128 keys go from HBM straight into LDS (buffer loads
//    with an LDS destination, 16 bytes per lane, one tile ahead, no
//    registers): K row-major with XOR-swizzled 16-byte chunks in a two-slot
//    ring, V row-major with swizzled 64-byte segments in a three-slot ring.
//    The A fragments of V^T come from two transposing reads
//    (ds_read_b64_tr_b16) each, which also put the keys in the order of the
//    P^T fragment; no transposed copy of V is ever written.  Fragments are
//    read several MFMAs ahead of use.  The loop's barriers wait only for LDS
//    traffic, so the copy of the next tile stays in flight across them.
//  * the waves of a SIMD run out of phase: waves 4..7 take the softmax of
//    tile t-1 and multiply P(t-1) V(t-1) before computing S(t), while waves
//    0..3 compute S(t) first, so one wave's MFMAs overlap the other's softmax.
//    Waves 0..3 issue all the copies of the next tile (16 each), one every
//    two MFMAs of their S(t) stage: waves 4..7 run the longer iteration, and
//    copies issued at the start of it cost them about 560 cycles.
//  * scores are handled in the log2 domain: x = s * scale * log2(e), so the
//    exponentials are single v_exp_f32 instructions.  The reference maximum
//    only moves when a tile's maximum exceeds it by more than 2^8, so the O
//    accumulators are rescaled rarely (the result is the same function).
//  * P^T leaves the S^T accumulators as bf16 (round to nearest even) and is
//    the B operand of O^T = V^T P^T, whose accumulators hold one query per
//    lane, so the rescale by alpha is lane-local.
//  * key tiles beyond the last visible key of the work-group (causal
//    diagonal, or the sequence's key length) are never loaded; a wave skips
//    the arithmetic of tiles that lie entirely above its own diagonal; only
//    tiles that cross the diagonal or the key length apply the mask, on
//    absolute positions.

#include <atomic>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.h"

// Tile choices (compile-time; the defaults are the tuned gfx950 configuration).
// 32 queries per wave keep a wave within 256
// VGPRs, so an 8-wave work-group (256 query rows) runs two waves per SIMD and
// one wave's MFMAs overlap the other's softmax.
#ifndef FA_FWD_QB
#define FA_FWD_QB 1
#endif
#ifndef FA_FWD_NW
#define FA_FWD_NW 8
#endif
#ifndef FA_FWD_BC
#define FA_FWD_BC 128
#endif
#ifndef FA_FWD_PREFETCH
#define FA_FWD_PREFETCH 4
#endif
#ifndef FA_FWD_SCHED
#define FA_FWD_SCHED 2
#endif
// 1: with two wave groups, only the first group issues the tile copies (the
// second group's iteration is the longer one; 8 copies cost it about 560 cycles)
#ifndef FA_FWD_DMA_LEAD
#define FA_FWD_DMA_LEAD 1
#endif


namespace fa {

namespace {

template <int D, int QB, int NW, int BC>
struct FwdBf16Cfg {
  static constexpr int BR = NW * QB * 32;  // query rows per work-group
  static constexpr int NT = NW * 64;       // threads per work-group
  static constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
  static constexpr int NCB = BC / 32;      // 32-key blocks per tile
  static constexpr int NG = BC / 16;       // 16-key groups per tile
  static constexpr int NDB = D / 32;       // 32-row blocks of O^T
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
};

// Lazy rescaling threshold (log2 units).  The reference maximum m used for
// exponentiation only moves when a tile's maximum exceeds it by more than
// this, so every p = 2^(x - m) stays <= 2^8: the arithmetic is still exact
// (numerator and denominator share m), finite in fp32 and bf16, and the O
// accumulators are rescaled only when the maximum really jumps.
constexpr float kRescaleThreshold = 8.0f;

// Arguments of the 16-bit kernel, passed as one struct (see job_args).
template <typename T>
struct FwdHalfArgs {
  const T* q;
  const T* k;
  const T* v;
  const int32_t* seqlens_k;
  T* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  float scale_log2;
  int causal;
  int B, H, n_q, n_k, n_qtiles, total_q, total_k;
  int n_jobs;    // query tiles over every (sequence, head)
  int persist;   // 1: work-group w runs jobs persistent_job(0..) instead of job w
};

template <class E, int D, int QB, int NW, int BC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(QB == 1 && D <= 128 ? 2 : 1, QB == 1 && D <= 128 ? 2 : 1)))
void fa_fwd_half_kernel(const FwdHalfArgs<typename E::T> args [[maybe_unused]]) {
  using elt = typename E::T;
  using elt8 = typename E::V8;
  using elt4 = typename E::V4;
  using C = FwdBf16Cfg<D, QB, NW, BC>;
  // Two groups of NW/2 waves; the waves of a SIMD (w and w + NW/2) sit in
  // different groups.  The second group runs one stage behind: it takes the
  // softmax of tile t-1 and multiplies P(t-1) V(t-1) before computing S(t),
  // so while one wave of a SIMD is in its MFMA phase the other is in its
  // softmax phase.  V therefore lives in a three-slot ring (group 2 still
  // reads V(t-1) while V(t+1) is written).
  constexpr bool kPingPong = (NW >= 8);
  constexpr int kVSlots = kPingPong ? 3 : 2;
  // K row-major with XOR-swizzled 16-byte chunks, V row-major with swizzled
  // 64-byte segments (read transposed); both filled by direct loads
  __shared__ __attribute__((aligned(16))) elt Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) elt Vs[kVSlots][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool lagging = kPingPong && wave >= NW / 2;

  // one job (query tile) per pass; a persistent launch runs several
  for (int pass = 0;; ++pass) {
  const auto* ka = job_args<FwdHalfArgs<elt>>();
  const int job = ka->persist ? persistent_job(pass, ka->n_jobs) : (pass == 0 ? (int)blockIdx.x : -1);
  if (job < 0) break;
  // every wave is done with the previous job's tiles before this one's copies
  if (pass > 0) __syncthreads();
  const elt* __restrict__ Q = global_ptr(ka->q);
  const elt* __restrict__ K = global_ptr(ka->k);
  const elt* __restrict__ V = global_ptr(ka->v);
  const int32_t* __restrict__ seqlens_k = global_ptr(ka->seqlens_k);
  elt* __restrict__ O = global_ptr(ka->o);
  float* __restrict__ LSE = global_ptr(ka->lse);
  const float scale_log2 = ka->scale_log2;
  const int causal = ka->causal;
  const int B = ka->B, H = ka->H;
  const TileCoord tc = tile_coord(job, B, H, ka->n_qtiles);
  const SeqSpan sp = seq_span(tc.b, tc.h, H, ka->n_q, ka->n_k, global_ptr(ka->cu_q),
                              global_ptr(ka->cu_k), ka->total_q, ka->total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (tc.qt * C::BR >= N) continue;  // a query tile past a shorter sequence
  const elt* Qh = Q + sp.q_row0 * D;
  const elt* Kh = K + sp.k_row0 * D;
  const elt* Vh = V + sp.k_row0 * D;
  elt* Oh = O + sp.q_row0 * D;
  float* Lh = LSE + sp.q_row0;

  const int kv_len = key_length(seqlens_k, tc.b, Nk);
  // N queries, Nk keys: query i sits at key position i + off (the queries are
  // the last N positions), so causally it sees keys j <= i + off
  const int off = Nk - N;
  const int q0 = tc.qt * C::BR;
  const int qw0 = q0 + wave * QB * 32;
  const int qw_last = qw0 + QB * 32 - 1;
  // key tiles the work-group loads: up to its last visible key
  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, max(0, min(q0 + C::BR + off, Nk)));
  const int n_kt = (kv_end + BC - 1) / BC;
  // key tiles this wave computes (a prefix): under the causal mask a tile whose
  // first key lies past the wave's last query is skipped
  int n_act = n_kt;
  if (qw0 >= N) n_act = 0;
  else if (causal) n_act = qw_last + off < 0 ? 0 : min(n_kt, (qw_last + off) / BC + 1);

  // ---- Q fragments (B operand of S^T = K Q^T): query l32, features 8*hi + [0..7]
  elt8 qf[QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (qrow < N)
        qf[qb][ks] = *reinterpret_cast<const elt8*>(Qh + (size_t)qrow * D + ks * 16 + hi * 8);
      else
        qf[qb][ks] = elt8{};
    }
  }

  // the Q fragments must have landed before the loop: its tile copies are
  // issued outside the compiler's counter tracking, so a wait it placed for Q
  // inside the loop would also wait for the copy in flight
  wait_vmem();

  f32x16 oacc[C::NDB][QB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x16{};
  float m[QB], l[QB], alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kNegInf;
    l[qb] = 0.f;
    alpha[qb] = 1.f;
  }

  // ---- staging: K and V tiles go straight from global memory into LDS
  // (buffer loads with an LDS destination: lane l of a wave fills bytes
  // [16 l, 16 l + 16) of a 1 KiB block), one tile ahead, with no registers.
  // The buffer descriptors end at the sequence's key length L_b, so keys at
  // or past it read as zeros (masked anyway, and whatever lies there never
  // enters a 0 * x product).  Each lane fetches the global chunk
  // that the tile's swizzle places at its LDS position.
  // A tile is BC rows of D/8 16-byte chunks stored contiguously; 1 KiB block
  // rb holds chunk positions 64 rb .. 64 rb + 63 (whole rows when D/8
  // divides 64, rows straddling blocks at d = 96 and 192).
  constexpr int kChunksPerRow = D / 8;
  constexpr int kBlksPerTensor = BC * D * 2 / 1024;
  // with two groups, only the first group's waves copy (FA_FWD_DMA_LEAD):
  // the second group's iteration is the longer one
  constexpr bool kLeadCopies = FA_FWD_DMA_LEAD && kPingPong;
  constexpr int kCopyWaves = kLeadCopies ? NW / 2 : NW;
  constexpr int kBlksPerWave = 2 * kBlksPerTensor / kCopyWaves;
  const bool copier = !kLeadCopies || !lagging;
  const int cwave = copier ? wave : 0;   // keeps a non-copying wave's offsets in range
  static_assert(BC * D * 2 % 1024 == 0, "whole 1 KiB blocks per tile");
  static_assert(2 * kBlksPerTensor % kCopyWaves == 0 && kBlksPerWave >= 1,
                "whole 1 KiB blocks per wave");
  const int key_bytes = kv_len * D * 2;
  const u32x4 k_rsrc = buffer_rsrc_words(Kh, (uint32_t)key_bytes);
  const u32x4 v_rsrc = buffer_rsrc_words(Vh, (uint32_t)key_bytes);
  // per-lane byte offsets inside a tile, computed once: the loads' address
  // registers then stay untouched for the whole loop (the compiler treats
  // them as pending load results and would otherwise wait for the copy
  // before reusing them); the tile's position goes in the scalar offset
  int voff[kBlksPerWave];
#pragma unroll
  for (int j = 0; j < kBlksPerWave; ++j) {
    const int blk = cwave * kBlksPerWave + j;
    const bool is_k = blk < kBlksPerTensor;
    const int rb = is_k ? blk : blk - kBlksPerTensor;
    const int pos = rb * 64 + lane;
    const int row = pos / kChunksPerRow;
    const int cpos = pos % kChunksPerRow;
    const int chunk = is_k ? (cpos ^ row_swizzle<D>(row))
                           : ((((cpos >> 2) ^ seg_swizzle<D>(row)) << 2) | (cpos & 3));
    voff[j] = row * (D * 2) + chunk * 16;
  }
  // one of this wave's copies of tile kt (block j of its share); slot
  // addresses are formed as 32-bit LDS offsets from the rings' bases
  const uint32_t ks_lds = lds_address(&Ks[0][0]);
  const uint32_t vs_lds = lds_address(&Vs[0][0]);
  constexpr uint32_t kSlotBytes = BC * D * 2;
  auto issue_block = [&](int kt, int kbuf, int vslot, int j) FA_INLINE {
    const int blk = cwave * kBlksPerWave + j;
    const bool is_k = blk < kBlksPerTensor;
    const int rb = is_k ? blk : blk - kBlksPerTensor;
    const uint32_t dst = (is_k ? ks_lds + (uint32_t)kbuf * kSlotBytes
                               : vs_lds + (uint32_t)vslot * kSlotBytes) +
                         (uint32_t)(rb * 1024);
    lds_dma16_at(is_k ? k_rsrc : v_rsrc, dst, voff[j], kt * BC * D * 2);
  };
  auto issue_tile = [&](int kt, int kbuf, int vslot) FA_INLINE {
    if (copier) {
#pragma unroll
      for (int j = 0; j < kBlksPerWave; ++j) issue_block(kt, kbuf, vslot, j);
    }
  };
  auto no_dma = [](int) FA_INLINE {};

  // defined at every job: left undefined, the previous job's values would be
  // carried around the job loop and these registers never freed
  f32x16 sacc[C::NCB][QB];
  elt8 pf[C::NG][QB];
#pragma unroll
  for (int c = 0; c < C::NCB; ++c)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sacc[c][qb] = f32x16{};
#pragma unroll
  for (int g = 0; g < C::NG; ++g)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pf[g][qb] = elt8{};

  // S^T(t) = K(t) Q^T.  The K fragments are read from LDS kPre reads ahead of
  // the MFMA that consumes them, so LDS latency overlaps the MFMA pipeline.
  constexpr int kPre = FA_FWD_PREFETCH;
  // `dma(j)` issues this wave's copy j of the next tile; the stage spreads the
  // copies over its MFMAs, one every NF / kBlksPerWave
  constexpr int kDmaEvery = (C::KS * C::NCB) / kBlksPerWave;
  static_assert(kDmaEvery >= 1 && kDmaEvery * kBlksPerWave == C::KS * C::NCB, "copies per stage");
  auto stage_S = [&](int kbuf, auto&& dma) FA_INLINE {
    constexpr int NF = C::KS * C::NCB;   // fragments per tile, ordered (ks, c)
    auto kfrag = [&](int f) FA_INLINE {
      const int ks = f / C::NCB, c = f % C::NCB;
      const int row = c * 32 + l32;
      return *reinterpret_cast<const elt8*>(
          &Ks[kbuf][row * D + ((2 * ks + hi) ^ row_swizzle<D>(row)) * 8]);
    };
    elt8 ring[kPre];
#pragma unroll
    for (int f = 0; f < kPre && f < NF; ++f) ring[f] = kfrag(f);
#pragma unroll
    for (int c = 0; c < C::NCB; ++c)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[c][qb] = f32x16{};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int ks = f / C::NCB, c = f % C::NCB;
      const elt8 kf = ring[f % kPre];
      if (f + kPre < NF) ring[f % kPre] = kfrag(f + kPre);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[c][qb] = E::mfma(kf, qf[qb][ks], sacc[c][qb]);
      if (f % kDmaEvery == 0) dma(f / kDmaEvery);
    }
#if FA_FWD_SCHED
    // keep the fragment reads kPre ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int f = 0; f < NF - kPre; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPre * QB, 0);
#endif
  };

  // A fragment of V^T for keys {16g + 4hi + 0..3, 16g + 8 + 4hi + 0..3}
  // (the order of the P^T fragment) and features 32 db + l32: two
  // transposing reads of the row-major V tile.  The segment swizzle sees only
  // row bits 0..1, which the lane fixes (rows 4hi + ts/4, + 8, + 16g), so the
  // lane's element offset for g = 0 is computed once per feature block and the
  // key group and the second read enter as immediate offsets.
  int v_at[C::NDB];
  {
    const int ts = lane & 15;
    const int tcol = ((lane >> 4) & 1) * 16 + 4 * (ts & 3);
    const int r0 = 4 * hi + (ts >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int col = db * 32 + tcol;
      v_at[db] = r0 * D + (((col >> 5) ^ seg_swizzle<D>(r0)) << 5) + (col & 31);
    }
  }

  // O^T += V^T(t) P^T(t), V^T fragments prefetched the same way
  auto stage_PV = [&](int vbuf, auto&& dma) FA_INLINE {
    constexpr int NF = C::NG * C::NDB;   // fragments per tile, ordered (g, db)
    // the slot index is made opaque: otherwise the compiler folds the ring's
    // modulo into the addresses as negative constants, which the reads'
    // unsigned offset field cannot hold, and adds them per read instead
    asm volatile("" : "+s"(vbuf));
    auto vfrag = [&](int f) FA_INLINE {
      const int g = f / C::NDB, db = f % C::NDB;
      const elt* vb = Vs[vbuf] + v_at[db] + 16 * g * D;
      const s16x4 lo = read_tr16(vb);
      const s16x4 up = read_tr16(vb + 8 * D);
      return __builtin_bit_cast(elt8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kReadsPerFrag = 2;
    elt8 ring[kPre];
#pragma unroll
    for (int f = 0; f < kPre && f < NF; ++f) ring[f] = vfrag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int g = f / C::NDB, db = f % C::NDB;
      const elt8 vf = ring[f % kPre];
      if (f + kPre < NF) ring[f % kPre] = vfrag(f + kPre);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mfma(vf, pf[g][qb], oacc[db][qb]);
      if (f % kDmaEvery == 0) dma(f / kDmaEvery);
    }
#if FA_FWD_SCHED >= 2
    __builtin_amdgcn_sched_group_barrier(0x100, kPre * kReadsPerFrag, 0);
#pragma unroll
    for (int f = 0; f < NF - kPre; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerFrag, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPre * QB, 0);
#endif
  };

  // mask (tiles crossing the key length or the wave's diagonal only), online
  // softmax with lazy rescaling, P^T as bf16; rescales O when a maximum jumped
  auto stage_softmax = [&](int kt) FA_INLINE {
    const int key0 = kt * BC;
    const bool need_mask = (key0 + BC > kv_len) || (causal && key0 + BC - 1 > qw0 + off);
    if (need_mask) {
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // key key0 + 32c + 4hi + p, p = 8(v/4) + v%4, is visible iff it is
          // at most min(L - 1, query): bit p of a per-lane prefix mask
          const int query = qw0 + qb * 32 + l32;
          const int lim = (causal ? min(kv_len - 1, query + off) : kv_len - 1) - key0 - 4 * hi;
          const uint32_t vis = prefix_bits(lim - 32 * c);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            sacc[c][qb][v] = keep_if_bit(sacc[c][qb][v], vis, 8 * (v >> 2) + (v & 3), kNegInf);
        }
    }
    bool scale_o = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[c][qb][v]);
      mx = halfwave_max(mx) * scale_log2;
      const bool upd = mx > m[qb] + kRescaleThreshold;
      const float m_new = upd ? mx : m[qb];
      alpha[qb] = upd ? fast_exp2(m[qb] - m_new) : 1.f;
      scale_o |= upd && (m[qb] != kNegInf);
      m[qb] = m_new;
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      // P^T is rounded to the 16-bit format for the MFMA, and the row sum
      // adds exactly those rounded weights (in fp32, two per instruction), so
      // O = o / l is a combination of the values whose weights sum to one: a
      // weight's rounding then moves O only through its difference from the
      // other values, never by a common factor
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < C::NG; ++g) {
        elt8 pk;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pk[i] = E::cvt(
              fast_exp2(__builtin_fmaf(sacc[g >> 1][qb][8 * (g & 1) + i], scale_log2, -m_use)));
        pf[g][qb] = pk;
#pragma unroll
        for (int j = 0; j < 8; j += 2) rs[j / 2] = E::sum2(pk, j, rs[j / 2]);
      }
      l[qb] = l[qb] * alpha[qb] + ((rs[0] + rs[1]) + (rs[2] + rs[3]));
    }
    // the O accumulators move only when some lane's maximum jumped
    if (__builtin_amdgcn_ballot_w64(scale_o) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[db][qb] *= alpha[qb];
    }
  };

  if (n_kt > 0) {
    issue_tile(0, 0, 0);
    wait_vmem();
    __syncthreads();
  }

  // one loop per group, so each is a plain straight-line schedule
  auto run = [&](auto lag_tag) FA_INLINE {
    constexpr bool kLag = decltype(lag_tag)::value;
    for (int kt = 0; kt < n_kt; ++kt) {
      const int kbuf = kt & 1;
      // the copies of tile kt+1 ride inside this iteration's first MFMA stage
      // (S for the first group, P V for the second) instead of all leaving at
      // once after the barrier, where they queue behind each other.  They are
      // issued unconditionally (a branch between the MFMAs costs more): in the
      // last iteration they fill slots nobody reads again, from rows past the
      // head (zeros) or past the work-group's last key.
      auto dma = [&](int j) FA_INLINE { issue_block(kt + 1, kbuf ^ 1, (kt + 1) % kVSlots, j); };
      auto dma_all = [&]() FA_INLINE {
#pragma unroll
        for (int j = 0; j < kBlksPerWave; ++j) dma(j);
      };
      if (kLag) {
        // second group: softmax(t-1) and P(t-1) V(t-1), then S(t); its
        // softmax runs while the first group computes S(t)
        if constexpr (!kLeadCopies) dma_all();
        if (kt >= 1 && kt - 1 < n_act) {
          stage_softmax(kt - 1);
          stage_PV((kt - 1) % kVSlots, no_dma);
        }
        if (kt < n_act) stage_S(kbuf, no_dma);
      } else if (kt < n_act) {
        stage_S(kbuf, dma);
        stage_softmax(kt);
        stage_PV(kt % kVSlots, no_dma);
      } else {
        dma_all();
      }
      // the next tile has landed once every wave passes here
      wait_vmem();
      lds_barrier();
    }
    // the second group's last softmax and P V
    if (kLag && n_kt > 0 && n_kt - 1 < n_act) {
      stage_softmax(n_kt - 1);
      stage_PV((n_kt - 1) % kVSlots, no_dma);
    }
  };
  if (lagging)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- epilogue: O = o / l (zeros for empty rows), LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halfwave_sum(l[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int q = qw0 + qb * 32 + l32;
    if (q < N) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = db * 32 + 8 * v4 + 4 * hi;
          elt4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = E::cvt(oacc[db][qb][4 * v4 + e] * inv);
          *reinterpret_cast<elt4*>(Oh + (size_t)q * D + d0) = w;
        }
      if (hi == 0)
        Lh[q] = lt > 0.f ? (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
    }
  }
  }  // job loop
}

// ---------------------------------------------------------------------------
// fp32 kernel: the same algorithm on 32x32x2 fp32 MFMA.  Each lane supplies one
// fp32 per operand, so V needs no transposition: the A fragment of V^T is a
// plain row-major read.  Row pitches are padded so that the two half-waves hit
// disjoint LDS banks.
// ---------------------------------------------------------------------------

// LDS operand reads issued this many MFMAs ahead in the fp32 kernel
constexpr int kF32Pre = 8;

template <int D, int NW, int BC, int KSPLIT = 1>
struct FwdF32Cfg {
  static constexpr int BR = NW * 32;
  static constexpr int NT = NW * KSPLIT * 64;
  static constexpr int BCR = BC * KSPLIT;     // keys staged per round
  static constexpr int KS = D / 2;
  static constexpr int NCB = BC / 32;
  static constexpr int NDB = D / 32;
  static constexpr int KPITCH = D + 2;   // floats per K row (halves on odd/even banks)
  static constexpr int VPITCH = D + 8;   // floats per V row (key+4 rows 32 banks apart)
  static constexpr int KU = BCR * D / 4 / NT;  // 16-byte chunks per thread
  static_assert(KU * NT * 4 == BCR * D, "tile must split evenly over threads");
};

// KSPLIT > 1 (small grids): KSPLIT waves share each 32-row block, wave
// split j taking key tiles j, j + KSPLIT, ... of a round of KSPLIT tiles, and
// the partial states (m, l, o) of a row block are merged through LDS at the
// end with the same rescale, so a grid too small to fill the chip still runs
// KSPLIT times fewer dependent tiles per wave.
template <int D, int NW, int BC, int KSPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * KSPLIT * 64, NW * KSPLIT * 64)))
void fa_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const int32_t* __restrict__ seqlens_k,
                       float scale_log2, int causal, float* __restrict__ O,
                       float* __restrict__ LSE, int B, int H, int n_q, int n_k,
                       int n_qtiles, const int32_t* __restrict__ cu_q,
                       const int32_t* __restrict__ cu_k, int total_q, int total_k) {
  using C = FwdF32Cfg<D, NW, BC, KSPLIT>;
  __shared__ __attribute__((aligned(16))) float Ks[2][C::BCR * C::KPITCH];
  __shared__ __attribute__((aligned(16))) float Vs[2][C::BCR * C::VPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = (tid >> 6) % NW;     // row block
  const int split = (tid >> 6) / NW;    // key split of the row block
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_coord(blockIdx.x, B, H, n_qtiles);
  const SeqSpan sp = seq_span(tc.b, tc.h, H, n_q, n_k, cu_q, cu_k, total_q, total_k);
  const int N = sp.nq, Nk = sp.nk;   // this sequence's query and key rows
  if (tc.qt * C::BR >= N) return;    // a query tile past a shorter sequence
  const float* Qh = Q + sp.q_row0 * D;
  const float* Kh = K + sp.k_row0 * D;
  const float* Vh = V + sp.k_row0 * D;
  float* Oh = O + sp.q_row0 * D;
  float* Lh = LSE + sp.q_row0;

  const int kv_len = key_length(seqlens_k, tc.b, Nk);
  const int off = Nk - N;   // query i sits at key position i + off
  const int q0 = tc.qt * C::BR;
  const int qw0 = q0 + wave * 32;
  int kv_end = kv_len;
  if (causal) kv_end = min(kv_end, max(0, min(q0 + C::BR + off, Nk)));
  const int n_kt = (kv_end + C::BCR - 1) / C::BCR;   // rounds of KSPLIT tiles

  const int qrow = qw0 + l32;
  float qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qf[ks] = qrow < N ? Qh[(size_t)qrow * D + 2 * ks + hi] : 0.f;

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  f32x4 kreg[C::KU], vreg[C::KU];
  // up to d = 128 the next tile's K/V wait in registers during the compute;
  // at d = 256 they would not fit beside Q and O, so the tile is copied
  // after the compute instead
  constexpr bool kStage = D <= 128;
  auto load_tile = [&](int kt) FA_INLINE {
    const int key0 = kt * C::BCR;
#pragma unroll
    for (int i = 0; i < C::KU; ++i) {
      const int u = tid + i * C::NT;
      const int r = u / (D / 4);
      const int c4 = u % (D / 4);
      const int key = key0 + r;
      const bool ok = key < kv_len;
      kreg[i] = ok ? *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + c4 * 4) : f32x4{};
      vreg[i] = ok ? *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + c4 * 4) : f32x4{};
    }
  };
  auto store_tile = [&](int buf) FA_INLINE {
#pragma unroll
    for (int i = 0; i < C::KU; ++i) {
      const int u = tid + i * C::NT;
      const int r = u / (D / 4);
      const int c4 = u % (D / 4);
      float* kd = &Ks[buf][r * C::KPITCH + c4 * 4];
      kd[0] = kreg[i][0];
      kd[1] = kreg[i][1];
      kd[2] = kreg[i][2];
      kd[3] = kreg[i][3];
      *reinterpret_cast<f32x4*>(&Vs[buf][r * C::VPITCH + c4 * 4]) = vreg[i];
    }
  };

  // unstaged copy (d = 256): each 16-byte chunk goes to LDS as soon as it
  // arrives, so only a few registers are live
  auto copy_tile = [&](int kt, int buf) FA_INLINE {
    const int key0 = kt * C::BCR;
#pragma unroll 4
    for (int i = 0; i < C::KU; ++i) {
      const int u = tid + i * C::NT;
      const int r = u / (D / 4);
      const int c4 = u % (D / 4);
      const int key = key0 + r;
      const bool ok = key < kv_len;
      const size_t at = (size_t)key * D + c4 * 4;
      const f32x4 kx = ok ? *reinterpret_cast<const f32x4*>(Kh + at) : f32x4{};
      const f32x4 vx = ok ? *reinterpret_cast<const f32x4*>(Vh + at) : f32x4{};
      float* kd = &Ks[buf][r * C::KPITCH + c4 * 4];
      kd[0] = kx[0];
      kd[1] = kx[1];
      kd[2] = kx[2];
      kd[3] = kx[3];
      *reinterpret_cast<f32x4*>(&Vs[buf][r * C::VPITCH + c4 * 4]) = vx;
    }
  };

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kStage && kt + 1 < n_kt) load_tile(kt + 1);
    const int key0 = kt * C::BCR + split * BC;   // this wave's tile of the round
    const float* Kt = &Ks[buf][split * BC * C::KPITCH];
    const float* Vt = &Vs[buf][split * BC * C::VPITCH];
    const bool wave_active =
        (qw0 < N) && key0 < kv_end && (!causal || key0 <= qw0 + 31 + off);
    if (wave_active) {
      f32x16 sacc[C::NCB];
#pragma unroll
      for (int c = 0; c < C::NCB; ++c) sacc[c] = f32x16{};
      // operands are read from LDS kF32Pre MFMAs ahead of their use, so the
      // MFMAs do not each wait for their own read
      {
        constexpr int NF = C::KS * C::NCB;   // (ks, c)
        auto kval = [&](int f) FA_INLINE {
          const int ks = f / C::NCB, c = f % C::NCB;
          return Kt[(c * 32 + l32) * C::KPITCH + 2 * ks + hi];
        };
        float ring[kF32Pre];
#pragma unroll
        for (int f = 0; f < kF32Pre; ++f) ring[f] = kval(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float x = ring[f % kF32Pre];
          if (f + kF32Pre < NF) ring[f % kF32Pre] = kval(f + kF32Pre);
          sacc[f % C::NCB] = mfma_f32(x, qf[f / C::NCB], sacc[f % C::NCB]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kF32Pre, 0);
#pragma unroll
        for (int f = 0; f < NF - kF32Pre; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kF32Pre, 0);
      }

      const bool need_mask = (key0 + BC > kv_len) || (causal && key0 + BC - 1 > qw0 + off);
      if (need_mask) {
#pragma unroll
        for (int c = 0; c < C::NCB; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + c * 32 + c_row(v, lane);
            const bool vis = key < kv_len && (!causal || key <= qrow + off);
            if (!vis) sacc[c][v] = kNegInf;
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[c][v]);
      mx = halfwave_max(mx);
      const float m_new = fmaxf(m, mx * scale_log2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < C::NCB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(sacc[c][v], scale_log2, -m_use));
          sacc[c][v] = p;
          rs += p;
        }
      l = l * alpha + rs;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha;

      // O^T += V^T P^T: one MFMA per key pair (lane halves supply keys k and k+4)
      {
        constexpr int NF = C::NCB * 16 * C::NDB;   // (c, v, db)
        auto vval = [&](int f) FA_INLINE {
          const int c = f / (16 * C::NDB), v = (f / C::NDB) % 16, db = f % C::NDB;
          return Vt[(c * 32 + c_row(v, lane)) * C::VPITCH + db * 32 + l32];
        };
        float ring[kF32Pre];
#pragma unroll
        for (int f = 0; f < kF32Pre; ++f) ring[f] = vval(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int c = f / (16 * C::NDB), v = (f / C::NDB) % 16, db = f % C::NDB;
          const float x = ring[f % kF32Pre];
          if (f + kF32Pre < NF) ring[f % kF32Pre] = vval(f + kF32Pre);
          oacc[db] = mfma_f32(x, sacc[c][v], oacc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kF32Pre, 0);
#pragma unroll
        for (int f = 0; f < NF - kF32Pre; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kF32Pre, 0);
      }
    }
    if (kt + 1 < n_kt) {
      if (kStage)
        store_tile(buf ^ 1);
      else
        copy_tile(kt + 1, buf ^ 1);
    }
    __syncthreads();
  }

  if constexpr (KSPLIT > 1) {
    // merge the row block's partial states: splits 1.. leave (m, l, o) in
    // LDS (the tile buffers are free after the loop's last barrier), split
    // 0 combines them, each weighed by 2^(m_j - M) with M the largest m
    constexpr int kSlot = C::NDB * 16 + 2;   // floats per lane
    static_assert(NW * (KSPLIT - 1) * 64 * kSlot <= 2 * C::BCR * C::KPITCH,
                  "partial states fit the K tile buffers");
    float* part = &Ks[0][0];
    if (split > 0) {
      float* dst = part + ((wave * (KSPLIT - 1) + split - 1) * 64 + lane) * kSlot;
      dst[0] = m;
      dst[1] = l;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[2 + db * 16 + v] = oacc[db][v];
    }
    __syncthreads();
    if (split > 0) return;
    float mj[KSPLIT];
    mj[0] = m;
#pragma unroll
    for (int j = 1; j < KSPLIT; ++j)
      mj[j] = part[((wave * (KSPLIT - 1) + j - 1) * 64 + lane) * kSlot];
    float M = mj[0];
#pragma unroll
    for (int j = 1; j < KSPLIT; ++j) M = fmaxf(M, mj[j]);
    const float w0 = (m == kNegInf) ? 0.f : fast_exp2(m - M);
    l *= w0;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] *= w0;
#pragma unroll
    for (int j = 1; j < KSPLIT; ++j) {
      const float* src = part + ((wave * (KSPLIT - 1) + j - 1) * 64 + lane) * kSlot;
      const float w = (mj[j] == kNegInf) ? 0.f : fast_exp2(mj[j] - M);
      l = __builtin_fmaf(src[1], w, l);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = __builtin_fmaf(src[2 + db * 16 + v], w, oacc[db][v]);
    }
    m = M;
  }

  const float lt = halfwave_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * hi;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * v4 + e] * inv;
        *reinterpret_cast<f32x4*>(Oh + (size_t)qrow * D + d0) = w;
      }
    if (hi == 0) Lh[qrow] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

constexpr int kBf16QB = FA_FWD_QB;
// Up to d = 128 a wave fits 256 VGPRs: 8 waves, two per SIMD in opposite
// phases, 128-key tiles.  At d = 256 the O accumulators and Q fragments alone
// take 192 VGPRs: 4 waves, one per SIMD with up to 512 VGPRs, 64-key tiles
// (K and V two slots each: 128 KiB of LDS).
template <int D>
struct Bf16Tile {
  static constexpr int BC = D <= 128 ? FA_FWD_BC : 64;
  static constexpr int NW = D <= 128 ? FA_FWD_NW : 4;
};
// fp32: 32-key tiles; two waves per work-group, four at d >= 192, where one
// work-group's two K/V slots (100 and 133 KB) leave room for no second one on
// the CU, so two waves would leave two SIMDs idle
constexpr int kF32BC = 32;
template <int D>
struct F32Tile {
  static constexpr int NW = D >= 192 ? 4 : 2;
};

// Work-groups of `kernel` (`threads` each) resident at once on the device of
// `stream`, rounded down to a multiple of 8 (one XCD lane each); 0 when the
// runtime cannot tell.  Cached per device id in `cache` (0: not known yet,
// -1: not available).
constexpr int kSlotCacheDevices = 64;
inline int persistent_slots(const void* kernel, int threads, hipStream_t stream,
                            std::atomic<int>* cache) {
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return 0;
  const bool cached = dev >= 0 && dev < kSlotCacheDevices;
  int v = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    int n_cu = 0, per_cu = 0;
    v = (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
         hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess)
            ? (n_cu * per_cu) / 8 * 8
            : 0;
    if (v <= 0) v = -1;
    if (cached) cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

template <class E, int D>
hipError_t launch_half_d(const FwdArgs& a) {
  constexpr int BC = Bf16Tile<D>::BC;
  constexpr int NW = Bf16Tile<D>::NW;
  using C = FwdBf16Cfg<D, kBf16QB, NW, BC>;
  using T = typename E::T;
  const int n_qtiles = (a.N + C::BR - 1) / C::BR;
  const long long n_jobs = (long long)n_qtiles * a.B * a.H;
  // Sequences of one length: a persistent launch, as many work-groups as fit
  // on the chip at once, each running a fixed list of query tiles (no gaps
  // between tiles waiting for the dispatcher).  Key lengths or packed
  // sequences keep one work-group per tile, placed by the dispatcher.
  static std::atomic<int> slots_cache[kSlotCacheDevices];
  const int slots = persistent_slots(
      reinterpret_cast<const void*>(&fa_fwd_half_kernel<E, D, kBf16QB, NW, BC>), C::NT, a.stream,
      slots_cache);
  const bool persist =
      a.seqlens_k == nullptr && a.cu_q == nullptr && slots >= 8 && n_jobs > slots;
  FwdHalfArgs<T> ka;
  ka.q = static_cast<const T*>(a.q);
  ka.k = static_cast<const T*>(a.k);
  ka.v = static_cast<const T*>(a.v);
  ka.seqlens_k = a.seqlens_k;
  ka.o = static_cast<T*>(a.o);
  ka.lse = a.lse;
  ka.cu_q = a.cu_q;
  ka.cu_k = a.cu_k;
  ka.scale_log2 = a.scale * kLog2e;
  ka.causal = a.causal;
  ka.B = a.B;
  ka.H = a.H;
  ka.n_q = a.N;
  ka.n_k = a.Nk;
  ka.n_qtiles = n_qtiles;
  ka.total_q = a.total_q;
  ka.total_k = a.total_k;
  ka.n_jobs = (int)n_jobs;
  ka.persist = persist ? 1 : 0;
  const dim3 grid((unsigned)(persist ? slots : n_jobs));
  hipLaunchKernelGGL((fa_fwd_half_kernel<E, D, kBf16QB, NW, BC>), grid, dim3(C::NT), 0,
                     a.stream, ka);
  return hipGetLastError();
}

template <class E>
hipError_t launch_half_e(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_half_d<E, 64>(a);
    case 96: return launch_half_d<E, 96>(a);
    case 128: return launch_half_d<E, 128>(a);
    case 192: return launch_half_d<E, 192>(a);
    case 256: return launch_half_d<E, 256>(a);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int KSPLIT>
hipError_t launch_f32_split(const FwdArgs& a) {
  constexpr int NW = F32Tile<D>::NW;
  using C = FwdF32Cfg<D, NW, kF32BC, KSPLIT>;
  const int n_qtiles = (a.N + C::BR - 1) / C::BR;
  const dim3 grid((unsigned)((long long)n_qtiles * a.B * a.H));
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, NW, kF32BC, KSPLIT>), grid, dim3(C::NT), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.seqlens_k, a.scale * kLog2e, a.causal,
                     static_cast<float*>(a.o), a.lse, a.B, a.H, a.N, a.Nk, n_qtiles,
                     a.cu_q, a.cu_k, a.total_q, a.total_k);
  return hipGetLastError();
}

// Grids with fewer work-groups than the chip has CUs split each row block's
// keys over four waves (d = 64, where four tiles of a round fit in LDS).
constexpr long long kF32SplitBelow = 256;

template <int D>
hipError_t launch_f32_d(const FwdArgs& a) {
  if constexpr (D == 64) {
    constexpr int NW = F32Tile<D>::NW;
    const long long grid = (long long)((a.N + NW * 32 - 1) / (NW * 32)) * a.B * a.H;
    if (grid < kF32SplitBelow) return launch_f32_split<D, 4>(a);
  }
  return launch_f32_split<D, 1>(a);
}

}  // namespace

long long fwd_half_grid(int B, int H, int N, int d) {
  const int BR = (d <= 128 ? Bf16Tile<128>::NW : Bf16Tile<256>::NW) * kBf16QB * 32;
  return (long long)((N + BR - 1) / BR) * B * H;
}

long long fwd_f32_grid(int B, int H, int N, int d) {
  const int BR = (d >= 192 ? F32Tile<256>::NW : F32Tile<128>::NW) * 32;
  return (long long)((N + BR - 1) / BR) * B * H;
}

hipError_t launch_fwd_half(const FwdArgs& a, Elt e) {
  if (e == Elt::kBf16) return launch_half_e<EltBf16>(a);
  if (e == Elt::kF16) return launch_half_e<EltF16>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_f32_d<64>(a);
    case 96: return launch_f32_d<96>(a);
    case 128: return launch_f32_d<128>(a);
    case 192: return launch_f32_d<192>(a);
    case 256: return launch_f32_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
