// fa_kernels.h — host-side launchers of the attention kernels (internal to the library).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum Dtype { kBF16 = 0, kF32 = 1 };

// Key rows per workgroup of the dK/dV kernel and query rows per step of its
// loop: bf16 runs the eight-wave pair kernel, float32 the four-wave one.
constexpr int kDkdvKeysBf16 = 256, kDkdvQRowsBf16 = 32;
constexpr int kDkdvKeysF32 = 128, kDkdvQRowsF32 = 64;
inline int dkdv_keys(Dtype t) { return t == kBF16 ? kDkdvKeysBf16 : kDkdvKeysF32; }
inline int dkdv_qrows(Dtype t) { return t == kBF16 ? kDkdvQRowsBf16 : kDkdvQRowsF32; }

// Dropout on P (inverted scaling): the seed, the fourth counter word and the
// byte threshold t (1..255) of the Philox mask; `on` false runs without it.
struct DropParams {
  bool on = false;
  uint32_t k0 = 0, k1 = 0, offset = 0, t = 0;
  float inv = 1.f;  // 256 / (256 - t)
};
struct FwdParams {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
  Dtype dtype;
  DropParams drop;
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
  Dtype dtype;  DropParams drop;
};

// Attention of Nq query rows over Nk keys split into nsplit ranges of
// split_len keys: float32 O [nsplit, B, H, Nq, d] and LSE [nsplit, B, H, Nq]
// per range (bottom-right causal alignment when causal).
struct SplitParams {
  const void* q; const void* k; const void* v;
  float* opart; float* lpart;
  void* o; float* lse;  // final outputs, written directly when nsplit == 1
  int B, H, Hkv, Nq, Nk, d;
  int nsplit, split_len;
  float scale;
  bool causal;
  Dtype dtype;
};

// Merge of nsplit per-range results of `rows` rows into o (dtype) and lse.
struct MergeParams {
  const float* opart; const float* lpart;
  void* o; float* lse;
  long rows;
  int nsplit, d;
  Dtype dtype;
};

// Forward on OCP e4m3 codes (d = 128): element value = code * tensor scale.
struct Fp8Params {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N;
  float scale, q_scale, k_scale, v_scale;
  bool causal;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream);
hipError_t launch_fwd_split(const SplitParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
// Backward phases: preprocess (D and lse2 into the workspace), the dQ kernel
// (which writes the same D and lse2 for its rows before using them) and the
// dK/dV kernel (plus the reduction of its partials when nsplit > 1), which
// reads them: preprocess or dQ must come before dK/dV on the stream.
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream);

// Size of the fixed device scratch of fa_bwd_noalloc, and its device address
// on the current device (looked up on first use per device).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa
