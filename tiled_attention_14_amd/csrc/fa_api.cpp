// fa_api.cpp — the C ABI of include/fa.h: argument validation, workspace
// layout and kernel dispatch.  Nothing here allocates, prints or throws.
#include "fa.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa_kernels.h"

namespace {

constexpr size_t kAlign = 256;
// Compute units of one MI355X; only used to balance the dK/dV work split.
constexpr double kCUs = 256.0;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks.  Every per-head slab (N x d elements) must stay below
// 2^31 bytes (32-bit buffer offsets) and grids must fit 32 bits.
fa_status_t check_shape(int B, int H, int Hkv, int N, int d, fa_dtype_t dtype, float scale) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const double esize = dtype == FA_BF16 ? 2.0 : 4.0;
  if ((double)(N + 256) * d * esize >= 2147483648.0) return FA_ERR_INVALID_ARG;
  if ((double)B * H * N * d >= 1099511627776.0) return FA_ERR_INVALID_ARG;
  if ((double)B * H * ((N + 31) / 32) >= 2147483647.0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Number of workgroups a GQA group's query heads are spread over in the dK/dV
// kernel.  One workgroup per (batch, KV head, key tile) loops over all g query
// heads; when that makes the heaviest workgroup much longer than the average
// work per compute unit, or leaves compute units idle, the heads are sliced
// and the slices' float32 partial sums are reduced afterwards.
int dkdv_nsplit(int B, int H, int Hkv, int N, bool causal, fa_dtype_t dtype) {
  const int g = H / Hkv;
  if (g == 1) return 1;
  const fa::Dtype t = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  const long keys = fa::dkdv_keys(t), rows = fa::dkdv_qrows(t);
  const long nkt = (N + keys - 1) / keys;
  const long nq = (N + rows - 1) / rows;
  const long step = keys / rows;                          // query tiles per key tile
  const long first = nq;                                  // steps of key tile 0, per head
  const long sum = causal ? nkt * nq - step * nkt * (nkt - 1) / 2 : nkt * nq;
  const double avg = (double)B * Hkv * g * sum / kCUs;    // steps per compute unit
  for (int ns = 1; ns < g; ++ns) {
    if (g % ns) continue;
    const double heavy = (double)(g / ns) * first;
    const double units = (double)B * Hkv * nkt * ns;
    if (heavy <= 1.25 * avg && units >= 2.0 * kCUs) return ns;
  }
  return g;
}

struct WorkspaceLayout {
  size_t delta_off, lse2_off, part_off, total;
};

WorkspaceLayout layout(int B, int H, int Hkv, int N, int d, int nsplit) {
  WorkspaceLayout w;
  const size_t rows = (size_t)B * H * N;
  w.delta_off = 0;
  w.lse2_off = round_up(rows * sizeof(float), kAlign);
  w.part_off = w.lse2_off + round_up(rows * sizeof(float), kAlign);
  const size_t part = nsplit > 1 ? 2 * (size_t)nsplit * B * Hkv * N * d * sizeof(float) : 0;
  w.total = w.part_off + part;
  return w;
}

// Validates the shared backward arguments and fills the shape and workspace fields of p.
fa_status_t bwd_params(int B, int H, int Hkv, int N, int d, float scale, int causal, fa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, fa::BwdParams* p) {
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  *p = fa::BwdParams{};
  p->nsplit = dkdv_nsplit(B, H, Hkv, N, causal != 0, dtype);
  const WorkspaceLayout wl = layout(B, H, Hkv, N, d, p->nsplit);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < wl.total)
    return FA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  p->delta = reinterpret_cast<float*>(ws + wl.delta_off);
  p->lse2 = reinterpret_cast<float*>(ws + wl.lse2_off);
  p->part = p->nsplit > 1 ? reinterpret_cast<float*>(ws + wl.part_off) : nullptr;
  p->B = B; p->H = H; p->Hkv = Hkv; p->N = N; p->d = d;
  p->scale = scale; p->causal = causal != 0;
  p->dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  return FA_OK;
}

// Key ranges of the split forward: enough (batch, KV head, row block, range)
// workgroups to cover the compute units twice, ranges of at least 256 keys.
int splitkv_auto(int B, int H, int Hkv, int Nq, int Nk) {
  const long nrb = ((long)(H / Hkv) * Nq + 127) / 128;
  const long base = nrb * B * Hkv;
  const long want = (long)(2 * kCUs + base - 1) / base;
  const long most = std::max<long>(1, Nk / 256);
  return (int)std::max<long>(1, std::min<long>(want, std::min<long>(most, 1024)));
}

// Range length (a multiple of the 64-key tile) and the number of non-empty
// ranges for a requested count (0 = chosen by the library).
void splitkv_ranges(int B, int H, int Hkv, int Nq, int Nk, int nsplit, int* len, int* count) {
  const int want = nsplit > 0 ? nsplit : splitkv_auto(B, H, Hkv, Nq, Nk);
  const int per = (Nk + want - 1) / want;
  *len = (per + 63) / 64 * 64;
  *count = (Nk + *len - 1) / *len;
}

fa_status_t check_splitkv(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, fa_dtype_t dtype,
                          int nsplit) {
  if (Nq < 1 || nsplit < 0) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_shape(B, H, Hkv, Nk, d, dtype, scale);
  if (st != FA_OK) return st;
  if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
  int len, count;
  splitkv_ranges(B, H, Hkv, Nq, Nk, nsplit, &len, &count);
  if ((double)count * B * H * Nq >= 2147483647.0) return FA_ERR_INVALID_ARG;
  if ((double)B * H * Nq * d >= 1099511627776.0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

size_t splitkv_bytes(int B, int H, int Nq, int d, int count, size_t* lse_off) {
  const size_t rows = (size_t)count * B * H * Nq;
  *lse_off = round_up(rows * d * sizeof(float), kAlign);
  return *lse_off + round_up(rows * sizeof(float), kAlign);
}

// Byte threshold t = round(256 p_drop) (1..255 turns dropout on; 0 leaves it off)
// and the inverted-dropout scale 256 / (256 - t).
bool drop_params(float p_drop, unsigned long long seed, unsigned int offset, fa::DropParams* out) {
  if (!std::isfinite(p_drop) || p_drop < 0.f) return false;
  const double t = std::floor(256.0 * (double)p_drop + 0.5);
  if (t > 255.0) return false;
  out->on = t > 0.0;
  out->t = (uint32_t)t;
  out->k0 = (uint32_t)(seed & 0xffffffffull);
  out->k1 = (uint32_t)(seed >> 32);
  out->offset = offset;
  out->inv = (float)(256.0 / (256.0 - t));
  return true;
}

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* x : ps)
    if (!x || !aligned16(x)) return false;
  return true;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  if (!all_aligned({q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  fa::FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N; p.d = d;
  p.scale = scale; p.causal = causal != 0;
  p.dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  return fa::launch_fwd(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int N, int d, float scale, float q_scale, float k_scale, float v_scale, int causal,
                       hipStream_t stream) {
  if (!all_aligned({q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
  for (float x : {q_scale, k_scale, v_scale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  // Shape rules of the bf16 path (a one-byte slab is half a bf16 one).
  fa_status_t st = check_shape(B, H, Hkv, N, 128, FA_BF16, scale);
  if (st != FA_OK) return st;
  fa::Fp8Params p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N;
  p.scale = scale; p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  p.causal = causal != 0;
  return fa::launch_fwd_fp8(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d, fa_dtype_t dtype) {
  if (check_shape(B, H, Hkv, N, d, dtype, 1.0f) != FA_OK) return 0;
  const int ns = std::max(dkdv_nsplit(B, H, Hkv, N, false, dtype), dkdv_nsplit(B, H, Hkv, N, true, dtype));
  return layout(B, H, Hkv, N, d, ns).total;
}

fa_status_t fa_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int Hkv, int N, int d,
                              fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!all_aligned({o, dO, lse})) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, 1.0f, 0, dtype, workspace, workspace_bytes, &p);
  if (st != FA_OK) return st;
  p.o = o; p.dO = dO; p.lse = lse;
  return fa::launch_bwd_pre(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv, int B,
                        int H, int Hkv, int N, int d, float scale, int causal, fa_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (!all_aligned({q, k, v, dO, dk, dv})) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.dO = dO; p.dk = dk; p.dv = dv;
  return fa::launch_bwd_dkdv(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                      void* dq, int B, int H, int Hkv, int N, int d, float scale, int causal, fa_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!all_aligned({q, k, v, o, dO, lse, dq})) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse; p.dq = dq;
  return fa::launch_bwd_dq(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!all_aligned({q, k, v, o, dO, lse, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse; p.dq = dq; p.dk = dk; p.dv = dv;
  // The dQ kernel also writes -D and lse * log2 e, which the dK/dV kernel reads.
  if (fa::launch_bwd_dq(p, stream) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dkdv(p, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                           float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  if (!all_aligned({q, k, v, o, dO, lse, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  const int ns = dkdv_nsplit(B, H, Hkv, N, causal != 0, dtype);
  const size_t need = layout(B, H, Hkv, N, d, ns).total;
  if (need > fa::kNoallocScratchBytes) return FA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  return fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype, ws, need, stream);
}

fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                           int N, int d, float scale, int causal, float p_drop, unsigned long long seed,
                           unsigned int offset, fa_dtype_t dtype, hipStream_t stream) {
  fa::DropParams dp;
  if (!drop_params(p_drop, seed, offset, &dp)) return FA_ERR_INVALID_ARG;
  if (!dp.on) return fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dtype, stream);
  if (!all_aligned({q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_shape(B, H, Hkv, N, d, dtype, scale);
  if (st != FA_OK) return st;
  fa::FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N; p.d = d;
  p.scale = scale; p.causal = causal != 0;
  p.dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  p.drop = dp;
  return fa::launch_fwd(p, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                           float scale, int causal, float p_drop, unsigned long long seed, unsigned int offset,
                           fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::DropParams dp;
  if (!drop_params(p_drop, seed, offset, &dp)) return FA_ERR_INVALID_ARG;
  if (!dp.on)
    return fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype, workspace,
                  workspace_bytes, stream);
  if (!all_aligned({q, k, v, o, dO, lse, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  fa_status_t st = bwd_params(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes, &p);
  if (st != FA_OK) return st;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse; p.dq = dq; p.dk = dk; p.dv = dv;
  p.drop = dp;
  if (fa::launch_bwd_dq(p, stream) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dkdv(p, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype_t dtype, int nsplit) {
  if (check_splitkv(B, H, Hkv, Nq, Nk, d, 1.0f, 0, dtype, nsplit) != FA_OK) return 0;
  int len, count;
  splitkv_ranges(B, H, Hkv, Nq, Nk, nsplit, &len, &count);
  size_t lse_off;
  return splitkv_bytes(B, H, Nq, d, count, &lse_off);
}

fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                           int Nq, int Nk, int d, float scale, int causal, fa_dtype_t dtype, int nsplit,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!all_aligned({q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
  fa_status_t st = check_splitkv(B, H, Hkv, Nq, Nk, d, scale, causal, dtype, nsplit);
  if (st != FA_OK) return st;
  int len, count;
  splitkv_ranges(B, H, Hkv, Nq, Nk, nsplit, &len, &count);
  size_t lse_off;
  const size_t need = splitkv_bytes(B, H, Nq, d, count, &lse_off);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < need)
    return FA_ERR_WORKSPACE;
  fa::SplitParams p;
  p.q = q; p.k = k; p.v = v;
  p.opart = static_cast<float*>(workspace);
  p.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off);
  p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.d = d;
  p.nsplit = count; p.split_len = len;
  p.scale = scale; p.causal = causal != 0;
  p.dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  if (fa::launch_fwd_split(p, stream) != hipSuccess) return FA_ERR_HIP;
  if (count == 1) return FA_OK;  // the single range wrote o and lse itself
  fa::MergeParams mp;
  mp.opart = p.opart; mp.lpart = p.lpart; mp.o = o; mp.lse = lse;
  mp.rows = (long)B * H * Nq; mp.nsplit = count; mp.d = d; mp.dtype = p.dtype;
  return fa::launch_merge(mp, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int nsplit, long rows, int d,
                     fa_dtype_t dtype, hipStream_t stream) {
  if (!all_aligned({o_parts, lse_parts, o, lse})) return FA_ERR_INVALID_ARG;
  if (nsplit < 1 || rows < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((double)rows * (d / 4) >= 549755813888.0) return FA_ERR_INVALID_ARG;
  fa::MergeParams mp;
  mp.opart = o_parts; mp.lpart = lse_parts; mp.o = o; mp.lse = lse;
  mp.rows = rows; mp.nsplit = nsplit; mp.d = d; mp.dtype = dtype == FA_BF16 ? fa::kBF16 : fa::kF32;
  return fa::launch_merge(mp, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: null or misaligned pointer, or invalid sizes or scale";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension or dtype not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the sizes need more workspace than the fixed 32 MiB scratch of fa_bwd_noalloc holds";
  }
  return "FA_ERR_UNKNOWN";
}

}  // extern "C"

extern "C" const char* fa_build_hash(void) { return FA_SOURCE_HASH; }
