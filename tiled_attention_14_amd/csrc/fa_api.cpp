// fa_api.cpp — the C ABI of include/fa.h: argument validation, workspace
// layout and kernel dispatch.  Nothing here allocates, prints or throws.
#include "../../include/fa.h"

#include <cmath>
#include <cstdint>

#include "fa_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks.  Element counts must fit comfortably in 63 bits and
// every per-tensor count must stay below 2^40 elements.
fa_status_t check_shape(int B, int H, int Hkv, int N, int d, fa_dtype_t dtype, float scale) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const double elems = (double)B * H * N * d;
  if (elems >= 1099511627776.0) return FA_ERR_INVALID_ARG;
  // Grid sizes are 32-bit: (query or key tiles) x B x H must fit.
  if ((double)B * H * ((N + 31) / 32) >= 2147483647.0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

struct WorkspaceLayout {
  size_t delta_off, delta_bytes, dq_off, dq_bytes, total;
};

WorkspaceLayout layout(int B, int H, int N, int d, fa_dtype_t dtype) {
  WorkspaceLayout w;
  const size_t rows = (size_t)B * H * N;
  w.delta_off = 0;
  w.delta_bytes = rows * sizeof(float);
  w.dq_off = round_up(w.delta_bytes, kAlign);
  w.dq_bytes = dtype == FA_BF16 ? rows * d * sizeof(float) : 0;
  w.total = w.dq_off + w.dq_bytes;
  return w;
}

// Validates the shared backward arguments and fills the shape, workspace and
// accumulator fields of p.
fa_status_t bwd_params(int B, int H, int Hkv, int N, int d, float scale, int causal, fa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* dq, fa::BwdParams* p) {
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  const WorkspaceLayout wl = layout(B, H, N, d, dtype);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < wl.total)
    return FA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  *p = fa::BwdParams{};
  p->dq = dq;
  p->delta = reinterpret_cast<float*>(ws + wl.delta_off);
  p->dq_acc = dtype == FA_BF16 ? reinterpret_cast<float*>(ws + wl.dq_off) : static_cast<float*>(dq);
  p->B = B; p->H = H; p->Hkv = Hkv; p->N = N; p->d = d;
  p->scale = scale; p->causal = causal != 0;
  p->dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  fa::FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N; p.d = d;
  p.scale = scale; p.causal = causal != 0;
  p.dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  return fa::launch_fwd(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d, fa_dtype_t dtype) {
  if (check_shape(B, H, Hkv, N, d, dtype, 1.0f) != FA_OK) return 0;
  return layout(B, H, N, d, dtype).total;
}

fa_status_t fa_bwd_preprocess(const void* o, const void* dO, void* dq, int B, int H, int Hkv, int N, int d,
                              fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!o || !dO || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(dO) || !aligned16(dq)) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, 1.0f, 0, dtype, workspace, workspace_bytes, dq, &p);
  if (st != FA_OK) return st;
  p.o = o; p.dO = dO;
  return fa::launch_bwd_pre(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_main(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq,
                        void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                        fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, dq, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.dO = dO; p.lse = lse; p.dk = dk; p.dv = dv;
  return fa::launch_bwd_main(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_finalize(void* dq, int B, int H, int Hkv, int N, int d, fa_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!dq || !aligned16(dq)) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, 1.0f, 0, dtype, workspace, workspace_bytes, dq, &p);
  if (st != FA_OK) return st;
  return fa::launch_bwd_finalize(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, dq, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse; p.dk = dk; p.dv = dv;
  if (fa::launch_bwd_pre(p, stream) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_main(p, stream) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_finalize(p, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: null or misaligned pointer, or invalid sizes or scale";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension or dtype not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
  }
  return "FA_ERR_UNKNOWN";
}

}  // extern "C"
