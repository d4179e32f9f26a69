// fa_decode.hip - decoding against a key/value cache, split over the key
// dimension, and the merge of partial softmax states.
//
// Method ("FlashAttention" (deepconcepts.dev), "What it does not do"): a
// decode step has one query row per head and reads the whole cache, one score
// per key, so nothing N x N exists to avoid; what helps is parallelism across
// the sequence dimension when the batch cannot fill the GPU (flash-decoding).
// The keys of each (batch, head) are split into parts; every part yields its
// normalised output o_s and lse_s = ln sum_{j in s} exp(s_j), and the parts
// are combined with the rescale of the online recurrence applied to whole
// parts ("FlashAttention", "Why it is allowed to be exact"; "Explain
// FlashAttention and why it is IO-aware", "Keep only the state needed for
// the final weighted average"):
//   LSE = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - LSE) o_s.
//
// The work is a matrix-vector product per head and is bound by HBM traffic
// (the cache is read once), not by MFMA: a part is processed by 256 threads,
// LPK lanes per key each holding one 16-byte chunk of the key or value row,
// with several rows in flight per lane.  Scores of the part go to LDS, the
// part's maximum and sum are block reductions, and the weighted value rows
// are summed in registers and then across key slots in LDS.

#include "fa_common.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// Split plan and loop shape (compile-time choices): aim for about
// FA_DEC_TARGET_WG work-groups so the last round of them is a small fraction
// of the run, with parts of at least FA_DEC_MIN_CHUNK keys, and
// FA_DEC_UNROLL rows in flight per lane (a sweep on MI355X: 2048 work-groups
// of 1024 keys reached 4.97 TB/s; 8192 of 256 keys 5.66 TB/s).
#ifndef FA_DEC_TARGET_WG
#define FA_DEC_TARGET_WG 8192
#endif
#ifndef FA_DEC_MIN_CHUNK
#define FA_DEC_MIN_CHUNK 128
#endif
#ifndef FA_DEC_UNROLL
#define FA_DEC_UNROLL 4
#endif
constexpr int kDecThreads = 256;
constexpr int kDecMaxChunk = 4096;   // keys per part (scores in LDS)
constexpr int kDecUnroll = FA_DEC_UNROLL;  // rows in flight per lane and pass
constexpr int kMergeThreads = 128;

template <typename T>
struct ElemsPer16;
template <>
struct ElemsPer16<__bf16> {
  static constexpr int value = 8;
};
template <>
struct ElemsPer16<_Float16> {
  static constexpr int value = 8;
};
template <>
struct ElemsPer16<float> {
  static constexpr int value = 4;
};

// 16 bytes of a row, widened to fp32
__device__ __forceinline__ void load16(const __bf16* p, float (&x)[8]) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = __uint_as_float(r[w] << 16);
    x[2 * w + 1] = __uint_as_float(r[w] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load16(const _Float16* p, float (&x)[8]) {
  const f16x8 r = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)r[e];
}
__device__ __forceinline__ void load16(const float* p, float (&x)[4]) {
  const f32x4 r = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = r[e];
}

__device__ __forceinline__ void store_out(__bf16* p, float x) { *p = to_bf16(x); }
__device__ __forceinline__ void store_out(_Float16* p, float x) { *p = (_Float16)x; }
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }

// max / sum over a 256-thread block; `scratch` holds 4 floats
__device__ __forceinline__ float block_max(float x, float* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}
__device__ __forceinline__ float block_sum(float x, float* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

// One work-group per (batch, head, part): keys [part*chunk, min(part*chunk +
// chunk, L_b)).  Writes the part's normalised output and its natural-log LSE
// (-inf and zeros for an empty part).
template <typename T, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kDecThreads, kDecThreads)))
void fa_decode_split_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                            const T* __restrict__ V, const int32_t* __restrict__ seqlens_k,
                            float scale_log2, int H, int N, int chunk, int n_parts,
                            float* __restrict__ o_parts, float* __restrict__ lse_parts) {
  constexpr int E = ElemsPer16<T>::value;
  constexpr int CPR = D / E;              // 16-byte chunks per key row
  // lanes per key row: the next power of two (d = 96 and 192 leave the last
  // lanes of each row group idle), so the row's dot product is a butterfly
  constexpr int LPK = CPR <= 1 ? 1 : 1 << (32 - __builtin_clz(CPR - 1));
  constexpr int KPS = kDecThreads / LPK;  // keys per step of the work-group
  static_assert(CPR * E == D && LPK <= 64, "a key row spans whole lanes of one wave");
  __shared__ float sc[kDecMaxChunk];
  __shared__ float red[KPS * D];
  __shared__ float scratch[4];

  const int wg = scheduled_wg(blockIdx.x, gridDim.x);
  const int part = wg % n_parts;
  const int bh = wg / n_parts;
  const int b = bh / H;
  const int L = key_length(seqlens_k, b, N);
  const int k0 = part * chunk;
  const int k1 = min(k0 + chunk, L);
  float* op = o_parts + ((size_t)bh * n_parts + part) * D;
  const int tid = threadIdx.x;
  if (k0 >= k1) {
    for (int f = tid; f < D; f += kDecThreads) op[f] = 0.f;
    if (tid == 0) lse_parts[(size_t)bh * n_parts + part] = kNegInf;
    return;
  }
  const int n = k1 - k0;
  const int kg = tid / LPK;
  const int lp = tid % LPK;
  const bool live = lp < CPR;   // this lane holds a chunk of the row
  const T* Kp = K + ((size_t)bh * N + k0) * D + lp * E;
  const T* Vp = V + ((size_t)bh * N + k0) * D + lp * E;

  // the query chunk of this lane, in log2 units of the scaled score
  float qv[E];
  if (live) {
    load16(Q + (size_t)bh * D + lp * E, qv);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] *= scale_log2;

  // ---- scores of the part
  for (int j0 = 0; j0 < n; j0 += KPS * kDecUnroll) {
    float kr[kDecUnroll][E];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * KPS + kg;
      if (j < n && live) {
        load16(Kp + (size_t)j * D, kr[u]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) kr[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot = __builtin_fmaf(qv[e], kr[u][e], dot);
#pragma unroll
      for (int off = LPK / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      const int j = j0 + u * KPS + kg;
      if (lp == 0 && j < n) sc[j] = dot;
    }
  }
  __syncthreads();

  // ---- maximum, weights and their sum
  float mx = kNegInf;
  for (int j = tid; j < n; j += kDecThreads) mx = fmaxf(mx, sc[j]);
  const float m = block_max(mx, scratch);
  float sum = 0.f;
  for (int j = tid; j < n; j += kDecThreads) {
    const float p = fast_exp2(sc[j] - m);
    sc[j] = p;
    sum += p;
  }
  const float l = block_sum(sum, scratch);  // its barriers also publish the weights

  // ---- weighted sum of the value rows
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < n; j0 += KPS * kDecUnroll) {
    float vr[kDecUnroll][E];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * KPS + kg;
      if (j < n && live) {
        load16(Vp + (size_t)j * D, vr[u]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) vr[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * KPS + kg;
      const float p = j < n ? sc[j] : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(p, vr[u][e], acc[e]);
    }
  }
  if (live) {
#pragma unroll
    for (int e = 0; e < E; ++e) red[kg * D + lp * E + e] = acc[e];
  }
  __syncthreads();
  const float inv = 1.f / l;
  for (int f = tid; f < D; f += kDecThreads) {
    float s = 0.f;
#pragma unroll 8
    for (int g = 0; g < KPS; ++g) s += red[g * D + f];
    op[f] = s * inv;
  }
  if (tid == 0) lse_parts[(size_t)bh * n_parts + part] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

// One work-group per row: LSE = ln sum_s exp(lse_s), O = sum_s w_s o_s with
// w_s = exp(lse_s - LSE); parts at -inf weigh 0; a row whose parts are all
// empty gets O = 0 and LSE = -inf.
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(kMergeThreads, kMergeThreads)))
void fa_merge_kernel(int n_parts, int D, const float* __restrict__ o_parts,
                     const float* __restrict__ lse_parts, T* __restrict__ o,
                     float* __restrict__ lse) {
  __shared__ float w[kMaxMergeParts];
  __shared__ float scratch[2];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* lp = lse_parts + (size_t)row * n_parts;
  // maximum over the parts (log2 units)
  float mx = kNegInf;
  for (int s = tid; s < n_parts; s += kMergeThreads) mx = fmaxf(mx, lp[s] * kLog2e);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) scratch[tid >> 6] = mx;
  __syncthreads();
  const float m = fmaxf(scratch[0], scratch[1]);
  __syncthreads();
  float sum = 0.f;
  for (int s = tid; s < n_parts; s += kMergeThreads) {
    const float x = lp[s];
    const float ws = (m == kNegInf || x == kNegInf) ? 0.f : fast_exp2(x * kLog2e - m);
    w[s] = ws;
    sum += ws;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((tid & 63) == 0) scratch[tid >> 6] = sum;
  __syncthreads();
  const float total = scratch[0] + scratch[1];
  const float inv = total > 0.f ? 1.f / total : 0.f;
  const float* orow = o_parts + (size_t)row * n_parts * D;
  for (int f = tid; f < D; f += kMergeThreads) {
    float acc = 0.f;
    for (int s = 0; s < n_parts; ++s) acc = __builtin_fmaf(w[s], orow[(size_t)s * D + f], acc);
    store_out(o + (size_t)row * D + f, acc * inv);
  }
  if (lse != nullptr && tid == 0)
    lse[row] = total > 0.f ? (m + __builtin_amdgcn_logf(total)) * kLn2 : kNegInf;
}

template <typename T, int D>
hipError_t launch_decode_split(const DecodeArgs& a, const DecodePlan& p, float* o_parts,
                               float* lse_parts) {
  const long long grid = (long long)a.B * a.H * p.parts;
  hipLaunchKernelGGL((fa_decode_split_kernel<T, D>), dim3((unsigned)grid), dim3(kDecThreads), 0,
                     a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.seqlens_k, a.scale * kLog2e, a.H, a.N,
                     p.chunk, p.parts, o_parts, lse_parts);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_merge_t(int rows, int n_parts, int d, const float* o_parts,
                          const float* lse_parts, void* o, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((fa_merge_kernel<T>), dim3((unsigned)rows), dim3(kMergeThreads), 0, stream,
                     n_parts, d, o_parts, lse_parts, static_cast<T*>(o), lse);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int B, int H, int N) {
  // enough parts for about FA_DEC_TARGET_WG work-groups, parts of at least
  // FA_DEC_MIN_CHUNK keys and at most kDecMaxChunk; chunks are multiples of
  // 64 keys
  DecodePlan p{1, 64};
  if (B <= 0 || H <= 0 || N <= 0) return p;
  const long long bh = (long long)B * H;
  long long parts = (FA_DEC_TARGET_WG + bh - 1) / bh;
  const long long by_min = (N + FA_DEC_MIN_CHUNK - 1) / FA_DEC_MIN_CHUNK;
  if (parts > by_min) parts = by_min;
  if (parts > kMaxMergeParts) parts = kMaxMergeParts;  // the merge holds one weight per part
  const long long by_max = (N + kDecMaxChunk - 1) / kDecMaxChunk;
  if (parts < by_max) parts = by_max;
  if (parts < 1) parts = 1;
  long long chunk = (N + parts - 1) / parts;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk > kDecMaxChunk) chunk = kDecMaxChunk;
  parts = (N + chunk - 1) / chunk;
  p.parts = (int)parts;
  p.chunk = (int)chunk;
  return p;
}

template <typename T>
hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& p, float* o_parts,
                           float* lse_parts) {
  switch (a.d) {
    case 64: return launch_decode_split<T, 64>(a, p, o_parts, lse_parts);
    case 96: return launch_decode_split<T, 96>(a, p, o_parts, lse_parts);
    case 128: return launch_decode_split<T, 128>(a, p, o_parts, lse_parts);
    case 192: return launch_decode_split<T, 192>(a, p, o_parts, lse_parts);
    case 256: return launch_decode_split<T, 256>(a, p, o_parts, lse_parts);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, Elt elt) {
  const DecodePlan p = decode_plan(a.B, a.H, a.N);
  float* o_parts = a.workspace;
  float* lse_parts = a.workspace + (size_t)a.B * a.H * p.parts * a.d;
  hipError_t e;
  switch (elt) {
    case Elt::kBf16: e = launch_decode_t<__bf16>(a, p, o_parts, lse_parts); break;
    case Elt::kF16: e = launch_decode_t<_Float16>(a, p, o_parts, lse_parts); break;
    default: e = launch_decode_t<float>(a, p, o_parts, lse_parts); break;
  }
  if (e != hipSuccess) return e;
  return launch_merge(a.B * a.H, p.parts, a.d, o_parts, lse_parts, a.o, a.lse, elt, a.stream);
}

hipError_t launch_merge(int rows, int n_parts, int d, const float* o_parts,
                        const float* lse_parts, void* o, float* lse, Elt elt,
                        hipStream_t stream) {
  switch (elt) {
    case Elt::kBf16:
      return launch_merge_t<__bf16>(rows, n_parts, d, o_parts, lse_parts, o, lse, stream);
    case Elt::kF16:
      return launch_merge_t<_Float16>(rows, n_parts, d, o_parts, lse_parts, o, lse, stream);
    default: return launch_merge_t<float>(rows, n_parts, d, o_parts, lse_parts, o, lse, stream);
  }
}

}  // namespace fa
