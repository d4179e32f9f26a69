// fa_api.cpp - the C ABI declared in include/fa.h: argument validation,
// dispatch on (dtype, d), and status codes.  Every check runs before any HIP
// call, so an invalid call enqueues nothing and works without a GPU.

#include "fa.h"

#include <cmath>
#include <cstdint>

#include "fa_internal.h"

namespace {

constexpr int kAbiVersion = 5;
constexpr long long kMaxGrid = 0x7fffffffLL;
// one head's rows of one sequence must be addressable with 32-bit byte
// offsets (the kernels' buffer descriptors)
constexpr long long kMaxHeadBytes = 0x7fffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_half(fa_dtype dtype) { return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16; }

fa::Elt elt_of(fa_dtype dtype) {
  return dtype == FA_DTYPE_BF16 ? fa::Elt::kBf16
                                : dtype == FA_DTYPE_F16 ? fa::Elt::kF16 : fa::Elt::kF32;
}

// head dimensions of the kernels: multiples of 32 from 64 to 256 that the
// tile shapes and swizzles are built for
bool head_dim_supported(int d) { return d == 64 || d == 96 || d == 128 || d == 192 || d == 256; }

bool fwd_supported(fa_dtype dtype, int d) {
  return (dtype == FA_DTYPE_F32 || is_half(dtype)) && head_dim_supported(d);
}

bool bwd_supported(fa_dtype dtype, int d) {
  return (dtype == FA_DTYPE_F32 || is_half(dtype)) && head_dim_supported(d);
}

long long bwd_grid(fa_dtype dtype, int B, int H, int N, int d) {
  return is_half(dtype) ? fa::bwd_half_grid(B, H, N, d) : fa::bwd_f32_grid(B, H, N, d);
}

// backward launches by element format (16-bit kernels or the fp32 ones)
hipError_t bwd_all(fa_dtype t, const fa::BwdArgs& a) {
  return is_half(t) ? fa::launch_bwd_half(a, elt_of(t)) : fa::launch_bwd_f32(a);
}
hipError_t bwd_pre(fa_dtype t, const fa::BwdArgs& a) {
  return is_half(t) ? fa::launch_bwd_preprocess_half(a, elt_of(t))
                    : fa::launch_bwd_preprocess_f32(a);
}
hipError_t bwd_dkdv(fa_dtype t, const fa::BwdArgs& a) {
  return is_half(t) ? fa::launch_bwd_dkdv_half(a, elt_of(t)) : fa::launch_bwd_dkdv_f32(a);
}
hipError_t bwd_dq(fa_dtype t, const fa::BwdArgs& a) {
  return is_half(t) ? fa::launch_bwd_dq_half(a, elt_of(t)) : fa::launch_bwd_dq_f32(a);
}

bool decode_supported(fa_dtype dtype, int d) {
  return (dtype == FA_DTYPE_F32 || is_half(dtype)) && head_dim_supported(d);
}


// Longest cache a decode call accepts (parts of at most 4096 keys, at most
// 4096 parts per row).
constexpr int kMaxDecodeN = 4096 * 4096;

bool known_dtype(fa_dtype dtype) { return dtype == FA_DTYPE_F32 || is_half(dtype); }

bool head_fits(fa_dtype dtype, int rows, int d) {
  return (long long)rows * d * (is_half(dtype) ? 2 : 4) <= kMaxHeadBytes;
}

// Shared size/scale/flag checks.  Returns FA_SUCCESS when the problem is
// well formed; *empty is set when there is nothing to compute.
fa_status check_common(fa_dtype dtype, int B, int H, int N, int d, float scale, int causal,
                       bool* empty) {
  *empty = false;
  if (!known_dtype(dtype)) return FA_ERROR_INVALID_VALUE;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERROR_INVALID_VALUE;
  if (causal != 0 && causal != 1) return FA_ERROR_INVALID_VALUE;
  if (B == 0 || H == 0 || N == 0) *empty = true;
  return FA_SUCCESS;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return kAbiVersion; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_SUCCESS: return "FA_SUCCESS";
    case FA_ERROR_INVALID_VALUE: return "FA_ERROR_INVALID_VALUE";
    case FA_ERROR_UNSUPPORTED: return "FA_ERROR_UNSUPPORTED";
    case FA_ERROR_LAUNCH: return "FA_ERROR_LAUNCH";
    case FA_ERROR_SCRATCH_LIMIT: return "FA_ERROR_SCRATCH_LIMIT";
  }
  return "FA_ERROR_UNKNOWN";
}

fa_status fa_forward(fa_dtype dtype, int B, int H, int Nq, int Nk, int d, const void* q,
                     const void* k, const void* v, const int32_t* seqlens_k, float scale,
                     int causal, void* o, float* lse, hipStream_t stream) {
  bool empty = false;
  fa_status st = check_common(dtype, B, H, Nq, d, scale, causal, &empty);
  if (st != FA_SUCCESS) return st;
  if (Nk < 0) return FA_ERROR_INVALID_VALUE;
  if (!fwd_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (!head_fits(dtype, Nq, d) || !head_fits(dtype, Nk, d)) return FA_ERROR_UNSUPPORTED;
  if (empty) return FA_SUCCESS;   // no query rows: nothing to write
  // with no keys the rows are written empty and k, v are never read
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERROR_INVALID_VALUE;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERROR_INVALID_VALUE;
  const long long grid = is_half(dtype) ? fa::fwd_half_grid(B, H, Nq, d)
                                        : fa::fwd_f32_grid(B, H, Nq, d);
  if (grid > kMaxGrid) return FA_ERROR_INVALID_VALUE;

  fa::FwdArgs a{B, H, Nq, d, Nk, q, k, v, seqlens_k, scale, causal, o, lse, stream};
  const hipError_t e =
      is_half(dtype) ? fa::launch_fwd_half(a, elt_of(dtype)) : fa::launch_fwd_f32(a);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

fa_status fa_forward_fp8(int B, int H, int Nq, int Nk, int d, const void* q, const void* k,
                         const void* v, const int32_t* seqlens_k, float scale, float q_descale,
                         float k_descale, float v_descale, int causal, void* o, float* lse,
                         hipStream_t stream) {
  bool empty = false;
  // the format checks of the bf16 output; scale and flags as for fa_forward
  fa_status st = check_common(FA_DTYPE_BF16, B, H, Nq, d, scale, causal, &empty);
  if (st != FA_SUCCESS) return st;
  if (Nk < 0) return FA_ERROR_INVALID_VALUE;
  for (float x : {q_descale, k_descale, v_descale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale * q_descale * k_descale)) return FA_ERROR_INVALID_VALUE;
  if (d != 128) return FA_ERROR_UNSUPPORTED;
  if ((long long)Nq * d * 2 > kMaxHeadBytes || (long long)Nk * d > kMaxHeadBytes)
    return FA_ERROR_UNSUPPORTED;
  if (empty) return FA_SUCCESS;
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERROR_INVALID_VALUE;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERROR_INVALID_VALUE;
  if (fa::fwd_fp8_grid(B, H, Nq, d) > kMaxGrid) return FA_ERROR_INVALID_VALUE;
  fa::FwdArgs a{B, H, Nq, d, Nk, q, k, v, seqlens_k, scale, causal, o, lse, stream};
  return fa::launch_fwd_fp8(a, q_descale, k_descale, v_descale) == hipSuccess ? FA_SUCCESS
                                                                              : FA_ERROR_LAUNCH;
}

size_t fa_backward_workspace_size(fa_dtype dtype, int B, int H, int N, int d) {
  (void)dtype;
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

fa_status fa_backward(fa_dtype dtype, int B, int H, int Nq, int Nk, int d, const void* q,
                      const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, const int32_t* seqlens_k, float scale, int causal,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  bool empty = false;
  fa_status st = check_common(dtype, B, H, Nq, d, scale, causal, &empty);
  if (st != FA_SUCCESS) return st;
  if (Nk < 0) return FA_ERROR_INVALID_VALUE;
  if (!bwd_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (!head_fits(dtype, Nq, d) || !head_fits(dtype, Nk, d)) return FA_ERROR_UNSUPPORTED;
  // with no query rows dK and dV are still written (zeros); with no keys, dQ.
  // Buffers of a side without rows are never touched and may be NULL.
  if (B == 0 || H == 0 || (Nq == 0 && Nk == 0)) return FA_SUCCESS;
  if (Nq > 0 && (!q || !o || !dout || !lse || !dq || !workspace)) return FA_ERROR_INVALID_VALUE;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return FA_ERROR_INVALID_VALUE;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERROR_INVALID_VALUE;
  if (workspace_bytes < fa_backward_workspace_size(dtype, B, H, Nq, d))
    return FA_ERROR_INVALID_VALUE;
  if (bwd_grid(dtype, B, H, Nq > Nk ? Nq : Nk, d) > kMaxGrid) return FA_ERROR_INVALID_VALUE;

  fa::BwdArgs a{B,  H,  Nq, d,    Nk,        q,     k,      v,  o,  dout,
                lse, seqlens_k, scale, causal, dq, dk, dv, static_cast<float*>(workspace),
                stream};
  const hipError_t e = bwd_all(dtype, a);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

fa_status fa_backward_preprocess(fa_dtype dtype, int B, int H, int N, int d, const void* o,
                                 const void* dout, float* delta, hipStream_t stream) {
  bool empty = false;
  // scale and causal do not enter this step; pass valid placeholders
  fa_status st = check_common(dtype, B, H, N, d, 1.f, 0, &empty);
  if (st != FA_SUCCESS) return st;
  if (!bwd_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (empty) return FA_SUCCESS;
  if (!o || !dout || !delta) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return FA_ERROR_INVALID_VALUE;
  if (bwd_grid(dtype, B, H, N, d) > kMaxGrid) return FA_ERROR_INVALID_VALUE;
  fa::BwdArgs a{B, H, N, d, N, nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, 1.f, 0,
                nullptr, nullptr, nullptr, delta, stream};
  return bwd_pre(dtype, a) == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

namespace {
// Checks of the dK/dV and dQ launches.  `keys_out` says which outputs the
// launch writes: dk/dv (one row per key) or dq (one row per query); the
// launch has nothing to do when its output has no rows, and buffers of a
// side without rows may be NULL.
fa_status check_bwd_phase(fa_dtype dtype, int B, int H, int Nq, int Nk, int d, const void* q,
                          const void* k, const void* v, const void* dout, const float* lse,
                          const float* delta, const int32_t* seqlens_k, float scale, int causal,
                          const void* out0, const void* out1, bool keys_out, bool* empty) {
  fa_status st = check_common(dtype, B, H, Nq, d, scale, causal, empty);
  if (st != FA_SUCCESS) return st;
  if (Nk < 0) return FA_ERROR_INVALID_VALUE;
  if (!bwd_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (!head_fits(dtype, Nq, d) || !head_fits(dtype, Nk, d)) return FA_ERROR_UNSUPPORTED;
  *empty = B == 0 || H == 0 || (keys_out ? Nk == 0 : Nq == 0);
  if (*empty) return FA_SUCCESS;
  if (!out0 || !out1) return FA_ERROR_INVALID_VALUE;
  if (Nq > 0 && (!q || !dout || !lse || !delta)) return FA_ERROR_INVALID_VALUE;
  if (Nk > 0 && (!k || !v)) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(delta) || !aligned16(out0) || !aligned16(out1))
    return FA_ERROR_INVALID_VALUE;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERROR_INVALID_VALUE;
  if (bwd_grid(dtype, B, H, Nq > Nk ? Nq : Nk, d) > kMaxGrid) return FA_ERROR_INVALID_VALUE;
  return FA_SUCCESS;
}
}  // namespace

fa_status fa_backward_dkdv(fa_dtype dtype, int B, int H, int Nq, int Nk, int d, const void* q,
                           const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, const int32_t* seqlens_k, float scale, int causal,
                           void* dk, void* dv, hipStream_t stream) {
  bool empty = false;
  fa_status st = check_bwd_phase(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta, seqlens_k,
                                 scale, causal, dk, dv, true, &empty);
  if (st != FA_SUCCESS || empty) return st;
  fa::BwdArgs a{B,   H,         Nq,    d,      Nk,      q,  k,  v, nullptr, dout,
                lse, seqlens_k, scale, causal, nullptr, dk, dv, const_cast<float*>(delta),
                stream};
  return bwd_dkdv(dtype, a) == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

fa_status fa_backward_dq(fa_dtype dtype, int B, int H, int Nq, int Nk, int d, const void* q,
                         const void* k, const void* v, const void* dout, const float* lse,
                         const float* delta, const int32_t* seqlens_k, float scale, int causal,
                         void* dq, hipStream_t stream) {
  bool empty = false;
  fa_status st = check_bwd_phase(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta, seqlens_k,
                                 scale, causal, dq, dq, false, &empty);
  if (st != FA_SUCCESS || empty) return st;
  fa::BwdArgs a{B,   H,         Nq,    d,      Nk, q,       k,       v, nullptr, dout,
                lse, seqlens_k, scale, causal, dq, nullptr, nullptr, const_cast<float*>(delta),
                stream};
  return bwd_dq(dtype, a) == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

namespace {
// Checks shared by the packed-batch calls: sizes, offsets arrays, the grid.
fa_status check_varlen(fa_dtype dtype, int B, int H, int total_q, int total_k, int max_q,
                       int max_k, int d, float scale, int causal, const int32_t* cu_q,
                       const int32_t* cu_k, bool backward) {
  bool empty = false;
  fa_status st = check_common(dtype, B, H, total_q, d, scale, causal, &empty);
  if (st != FA_SUCCESS) return st;
  if (total_k < 0 || max_q < 0 || max_k < 0) return FA_ERROR_INVALID_VALUE;
  if (!(backward ? bwd_supported(dtype, d) : fwd_supported(dtype, d)))
    return FA_ERROR_UNSUPPORTED;
  if (!head_fits(dtype, max_q, d) || !head_fits(dtype, max_k, d)) return FA_ERROR_UNSUPPORTED;
  if (B == 0 || H == 0) return FA_SUCCESS;
  if (!cu_q || !cu_k) return FA_ERROR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u))
    return FA_ERROR_INVALID_VALUE;
  const long long grid =
      backward ? bwd_grid(dtype, B, H, max_q > max_k ? max_q : max_k, d)
               : (is_half(dtype) ? fa::fwd_half_grid(B, H, max_q, d)
                                 : fa::fwd_f32_grid(B, H, max_q, d));
  if (grid > kMaxGrid) return FA_ERROR_INVALID_VALUE;
  return FA_SUCCESS;
}
}  // namespace

fa_status fa_forward_varlen(fa_dtype dtype, int B, int H, int total_q, int total_k,
                            int max_seqlen_q, int max_seqlen_k, int d, const void* q,
                            const void* k, const void* v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, float scale, int causal, void* o,
                            float* lse, hipStream_t stream) {
  fa_status st = check_varlen(dtype, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k, d,
                              scale, causal, cu_seqlens_q, cu_seqlens_k, false);
  if (st != FA_SUCCESS) return st;
  if (B == 0 || H == 0 || total_q == 0 || max_seqlen_q == 0) return FA_SUCCESS;
  const bool keys = total_k > 0 && max_seqlen_k > 0;
  if (!q || !o || !lse || (keys && (!k || !v))) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERROR_INVALID_VALUE;
  fa::FwdArgs a{B, H, max_seqlen_q, d, max_seqlen_k, q, k, v, nullptr, scale, causal, o, lse,
                stream, cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  const hipError_t e =
      is_half(dtype) ? fa::launch_fwd_half(a, elt_of(dtype)) : fa::launch_fwd_f32(a);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

fa_status fa_backward_varlen(fa_dtype dtype, int B, int H, int total_q, int total_k,
                             int max_seqlen_q, int max_seqlen_k, int d, const void* q,
                             const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, float scale, int causal, void* dq,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  fa_status st = check_varlen(dtype, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k, d,
                              scale, causal, cu_seqlens_q, cu_seqlens_k, true);
  if (st != FA_SUCCESS) return st;
  const bool queries = total_q > 0 && max_seqlen_q > 0;
  const bool keys = total_k > 0 && max_seqlen_k > 0;
  if (B == 0 || H == 0 || (!queries && !keys)) return FA_SUCCESS;
  if (queries && (!q || !o || !dout || !lse || !dq || !workspace)) return FA_ERROR_INVALID_VALUE;
  if (keys && (!k || !v || !dk || !dv)) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return FA_ERROR_INVALID_VALUE;
  if (queries && workspace_bytes < fa_backward_workspace_size(dtype, 1, H, total_q, d))
    return FA_ERROR_INVALID_VALUE;
  // with no query rows the row statistics are never read: nothing to compute
  fa::BwdArgs a{B,   H,       queries ? max_seqlen_q : 0, d,  keys ? max_seqlen_k : 0,
                q,   k,       v,       o,  dout, lse, nullptr, scale, causal, dq, dk, dv,
                static_cast<float*>(workspace), stream, cu_seqlens_q, cu_seqlens_k,
                queries ? total_q : 0, keys ? total_k : 0};
  const hipError_t e = bwd_all(dtype, a);
  return e == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

size_t fa_decode_workspace_size(fa_dtype dtype, int B, int H, int N, int d) {
  (void)dtype;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  const fa::DecodePlan p = fa::decode_plan(B, H, N);
  return (size_t)B * (size_t)H * (size_t)p.parts * ((size_t)d + 1) * sizeof(float);
}

fa_status fa_decode(fa_dtype dtype, int B, int H, int N, int d, const void* q, const void* k,
                    const void* v, const int32_t* seqlens_k, float scale, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  fa_status st = check_common(dtype, B, H, N, d, scale, 0, &empty);
  if (st != FA_SUCCESS) return st;
  if (!decode_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (empty) return FA_SUCCESS;
  if (N > kMaxDecodeN) return FA_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return FA_ERROR_INVALID_VALUE;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERROR_INVALID_VALUE;
  if (workspace_bytes < fa_decode_workspace_size(dtype, B, H, N, d)) return FA_ERROR_INVALID_VALUE;
  const fa::DecodePlan p = fa::decode_plan(B, H, N);
  if ((long long)B * H * p.parts > kMaxGrid || (long long)B * H > kMaxGrid)
    return FA_ERROR_INVALID_VALUE;
  fa::DecodeArgs a{B, H, N, d, q, k, v, seqlens_k, scale, o, lse,
                   static_cast<float*>(workspace), stream};
  return fa::launch_decode(a, elt_of(dtype)) == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH;
}

fa_status fa_merge_states(fa_dtype dtype, int rows, int n_parts, int d, const float* o_parts,
                          const float* lse_parts, void* o, float* lse, hipStream_t stream) {
  if (!known_dtype(dtype)) return FA_ERROR_INVALID_VALUE;
  if (rows < 0 || n_parts < 1 || d <= 0) return FA_ERROR_INVALID_VALUE;
  if (!decode_supported(dtype, d)) return FA_ERROR_UNSUPPORTED;
  if (n_parts > fa::kMaxMergeParts) return FA_ERROR_INVALID_VALUE;
  if (rows == 0) return FA_SUCCESS;
  if (!o_parts || !lse_parts || !o) return FA_ERROR_INVALID_VALUE;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERROR_INVALID_VALUE;
  if ((long long)rows > kMaxGrid) return FA_ERROR_INVALID_VALUE;
  return fa::launch_merge(rows, n_parts, d, o_parts, lse_parts, o, lse, elt_of(dtype),
                          stream) == hipSuccess
             ? FA_SUCCESS
             : FA_ERROR_LAUNCH;
}

}  // extern "C"
