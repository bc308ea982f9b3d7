// fa_kernels.h — host-side launchers of the attention kernels (internal to the library).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

enum Dtype { kBF16 = 0, kF32 = 1 };

struct FwdParams {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
  Dtype dtype;
};

struct BwdParams {
  const void* q; const void* k; const void* v;
  const void* o; const void* dO; const float* lse;
  void* dq; void* dk; void* dv;
  float* delta;    // [B, H, N] workspace: D_i = sum_c dO_ic O_ic
  float* dq_acc;   // [B, H, N, d] fp32 accumulator (bf16) or dq itself (f32)
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
  Dtype dtype;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
// The three backward phases, in stream order: D and dQ-accumulator zeroing,
// the main kernel, and (bf16 only) the dQ conversion.
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_main(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t stream);

}  // namespace fa
