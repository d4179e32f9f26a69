// fa_internal.h - host-side declarations shared by the C ABI and the kernel
// translation units.  Launchers assume their arguments were validated by
// fa_api.cpp and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Element format of a launch's inputs and outputs.
enum class Elt { kF32, kBf16, kF16 };

struct FwdArgs {
  int B, H, N, d;   // N: query rows per head
  int Nk;           // key/value rows per head
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens_k;
  float scale;
  int causal;
  void* o;
  float* lse;
  hipStream_t stream;
  // packed batches (cu_q != nullptr): sequence b holds query rows
  // cu_q[b] .. cu_q[b+1] and key rows cu_k[b] .. cu_k[b+1] of the head-major
  // [H][total][d] tensors; N and Nk are then the longest sequence's lengths
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
};

struct BwdArgs {
  int B, H, N, d;   // N: query rows per head
  int Nk;           // key/value rows per head
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const int32_t* seqlens_k;
  float scale;
  int causal;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B][H][N] (packed: [H][total_q]) fp32 row dot products
  hipStream_t stream;
  const int32_t* cu_q;   // packed batches, as in FwdArgs
  const int32_t* cu_k;
  int total_q, total_k;
};

struct DecodeArgs {
  int B, H, N, d;
  const void* q;  // [B][H][d]
  const void* k;  // [B][H][N][d]
  const void* v;
  const int32_t* seqlens_k;
  float scale;
  void* o;     // [B][H][d]
  float* lse;  // [B][H]
  float* workspace;
  hipStream_t stream;
};

// How decoding splits the keys of one (batch, head): `parts` parts of
// `chunk` keys (the last one possibly shorter).
struct DecodePlan {
  int parts, chunk;
};
DecodePlan decode_plan(int B, int H, int N);
// Largest number of parts a merge accepts (weights are kept in LDS).
constexpr int kMaxMergeParts = 4096;

// Each launcher returns hipSuccess or the error hipGetLastError reported
// after enqueueing; it never synchronises.
// The 16-bit launchers take Elt::kBf16 or Elt::kF16.
hipError_t launch_fwd_half(const FwdArgs& a, Elt e);
hipError_t launch_fwd_f32(const FwdArgs& a);
// FP8 (E4M3) q, k, v with per-tensor descale factors, bf16 o; d = 128
hipError_t launch_fwd_fp8(const FwdArgs& a, float q_descale, float k_descale, float v_descale);
hipError_t launch_bwd_half(const BwdArgs& a, Elt e);
hipError_t launch_bwd_preprocess_half(const BwdArgs& a, Elt e);
hipError_t launch_bwd_dkdv_half(const BwdArgs& a, Elt e);
hipError_t launch_bwd_dq_half(const BwdArgs& a, Elt e);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_bwd_preprocess_f32(const BwdArgs& a);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a);
hipError_t launch_bwd_dq_f32(const BwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a, Elt e);
hipError_t launch_merge(int rows, int n_parts, int d, const float* o_parts,
                        const float* lse_parts, void* o, float* lse, Elt e,
                        hipStream_t stream);

// Number of work-groups a launch of the given geometry needs; the ABI
// rejects problems whose grid would not fit in a signed 32-bit count.
long long fwd_half_grid(int B, int H, int N, int d);
long long fwd_f32_grid(int B, int H, int N, int d);
long long fwd_fp8_grid(int B, int H, int N, int d);
long long bwd_half_grid(int B, int H, int N, int d);
long long bwd_f32_grid(int B, int H, int N, int d);

}  // namespace fa
