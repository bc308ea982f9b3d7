// fa_kernels.h — host-side launchers of the attention kernels (internal to the library).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

enum Dtype { kBF16 = 0, kF32 = 1 };

// Key rows per workgroup of the dK/dV kernel and query rows per step of its
// loop: bf16 runs the eight-wave pair kernel, float32 the four-wave one.
constexpr int kDkdvKeysBf16 = 256, kDkdvQRowsBf16 = 32;
constexpr int kDkdvKeysF32 = 128, kDkdvQRowsF32 = 64;
inline int dkdv_keys(Dtype t) { return t == kBF16 ? kDkdvKeysBf16 : kDkdvKeysF32; }
inline int dkdv_qrows(Dtype t) { return t == kBF16 ? kDkdvQRowsBf16 : kDkdvQRowsF32; }

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
  float* delta;   // [B, H, N] workspace: -D_i = -sum_c dO_ic O_ic
  float* lse2;    // [B, H, N] workspace: lse_i * log2(e)
  float* part;    // [nsplit, 2, B, Hkv, N, d] float32 partial dK / dV (nsplit > 1 only)
  int nsplit;     // query-head slices of a GQA group handled by separate workgroups
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
  Dtype dtype;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
// Backward phases, in stream order: preprocess (D and lse2), then the dK/dV
// kernel (plus the reduction of its partials when nsplit > 1) and the dQ
// kernel, which are independent of each other.
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream);

}  // namespace fa
