// fa_splitkv.hip — attention over a key/value cache for gfx950: Nq query rows
// against Nk keys (Nq != Nk allowed, bottom-right causal alignment), with the
// keys split into ranges that separate workgroups process, and the merge of
// the per-range results.
//
// A range's result is the attention over its keys alone, normalised over that
// range, plus the log-sum-exp over that range.  Merging rescales each range's
// output by exp(LSE_range - LSE) with LSE = log sum exp(LSE_range): the
// correction step of the incremental softmax ("FlashAttention 在昇腾NPU上到底快在哪",
// section 三、增量 Softmax), applied across workgroups instead of across the
// tiles of one workgroup.  That makes short query blocks, such as decoding one
// token against a long cache (the cache reuse of the same page, section 七),
// fill the GPU: the parallelism comes from the key dimension.
//
// Mapping:
//  * one workgroup = 4 waves = 128 rows; a row is one (query head of the GQA
//    group, query position) pair of one KV head, so the g heads that share a
//    KV head share every K/V tile (decoding with g = 8 fills 8 of a wave's
//    32 rows instead of one);
//  * grid: row block x key range x (batch, KV head); K/V tiles of 64 keys go
//    global -> LDS directly, double-buffered, as in the forward kernel, and the
//    products and the online softmax are the forward kernel's (scores S^T =
//    K Q^T on bf16 MFMA, P V in fp16 for bf16 inputs);
//  * each range writes float32 O and LSE per row; a row that sees no key of
//    the range writes O = 0 and LSE = -inf, which the merge weights by 0.
//    With a single range the kernel writes the final O (in the input dtype)
//    and LSE itself, the values the merge would produce, and no merge runs.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kSplitRows = 32 * kSplitWaves;  // rows per workgroup
constexpr int kSplitKeys = 64;                // keys per streamed tile
constexpr float kSplitSlack = 8.f;            // log2 units the running max may lag behind

struct SplitArgs {
  const void* q; const void* k; const void* v;
  float* opart; float* lpart;
  void* o; float* lse;  // nsplit == 1: the range is the whole row, written here directly
  int B, H, Hkv, Nq, Nk;
  int nrb;        // row blocks per (batch, KV head)
  int nsplit;     // key ranges
  int split_len;  // keys per range (a multiple of kSplitKeys)
  float c;        // scale * log2(e)
};

template <typename T> struct SplitPv;
template <> struct SplitPv<bf16> { typedef f16x8 type; };
template <> struct SplitPv<float> { typedef f32x8 type; };

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// ts + the eight values of a probability fragment (fp16 pairs summed with
// v_dot2c_f32_f16 into fp32; fp32 values added directly).
__device__ __forceinline__ float add_frag(float ts, const f16x8& v) {
  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
  ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), ones, ts, false);
  ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), ones, ts, false);
  ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), ones, ts, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), ones, ts, false);
}
__device__ __forceinline__ float add_frag(float ts, const f32x8& v) {
  return ts + ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Eight consecutive elements at p (16-byte aligned) as a k16 fragment.
__device__ __forceinline__ void frag_at(bf16x8& f, const bf16* p) {
  f = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void frag_at(f32x8& f, const float* p) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p), y = *reinterpret_cast<const f32x4*>(p + 4);
  f = f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads, sizeof(T) == 2 ? 2 : 1) void fa_fwd_split_kernel(SplitArgs a) {
  typedef typename Frag<T>::type F;
  typedef typename SplitPv<T>::type PF;
  typedef Lay<T, D> L;
  typedef TileCopy<T, D, kSplitKeys, kSplitWaves> TC;
  constexpr bool kConv = sizeof(T) == 2;
  constexpr int TB = kSplitKeys * L::RB;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char sK0[TB], sK1[TB], sV0[TB], sV1[TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  int bid = blockIdx.x;
  const int rb = bid % a.nrb;
  bid /= a.nrb;
  const int sp = bid % a.nsplit;
  const int unit = bid / a.nsplit;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int g = a.H / a.Hkv;
  const int R = g * a.Nq;                    // rows of this KV head
  const int r0 = rb * kSplitRows;            // first row of the workgroup
  const int r = r0 + 32 * w + l32;           // row of this lane
  const bool rvalid = r < R;
  const int rr = rvalid ? r : R - 1;
  const int h = kvh * g + rr / a.Nq, qi = rr % a.Nq;
  const long orow = ((long)b * a.H + h) * a.Nq + qi;   // row of q, o and lse

  // Keys of this range, cut at the last key any row of the workgroup sees.
  const int off = a.Nk - a.Nq;
  const int ks0 = sp * a.split_len;
  int kend = min(a.Nk, ks0 + a.split_len);
  if (CAUSAL) {
    const int cnt = min(R, r0 + kSplitRows) - r0;
    const int p0 = r0 % a.Nq;
    const int pmax = (p0 + cnt - 1 >= a.Nq) ? a.Nq - 1 : p0 + cnt - 1;
    kend = min(kend, pmax + off + 1);
  }
  const int nt = kend > ks0 ? (kend - ks0 + kSplitKeys - 1) / kSplitKeys : 0;
  // Last key of the range this lane's row sees (keys past it are masked).
  const int lastkey = CAUSAL ? min(kend - 1, qi + off) : kend - 1;

  // Row of the partial outputs.  A range with no key visible to any row of
  // the workgroup runs no tile and writes O = 0, LSE = -inf (its first key is
  // still below Nk, so the prologue's copies stay in bounds).
  const long pidx = (long)sp * a.B * a.H * a.Nq + orow;

  F qf[KS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + orow * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) frag_at(qf[s], qp + 16 * s + 8 * hf);
  }
  wait_loads();

  const size_t slab = (size_t)a.Nk * D;
  const T* Kh = reinterpret_cast<const T*>(a.k) + (size_t)unit * slab;
  const T* Vh = reinterpret_cast<const T*>(a.v) + (size_t)unit * slab;
  RowFrags<T, D> rf;
  ColFrags<T, D> cf;
  TC tc;
  rf.init();
  cf.init();
  tc.init(w);
  lds_zero<kSplitThreads>(sK0, TB); lds_zero<kSplitThreads>(sK1, TB);
  lds_zero<kSplitThreads>(sV0, TB); lds_zero<kSplitThreads>(sV1, TB);
  __syncthreads();
  u32x4 vr[TC::CPW];
  auto copy_kv = [&](char* sK, char* sV, int k0) {
    tc.issue(Kh, a.Nk, k0, sK);
    if constexpr (kConv) tc.load(Vh, a.Nk, k0, vr);
    else tc.issue(Vh, a.Nk, k0, sV);
  };
  auto finish_v = [&](char* sV) {
    if constexpr (kConv) tc.store_f16(vr, sV);
  };
  copy_kv(sK0, sV0, ks0);
  wait_copies();
  finish_v(sV0);
  __syncthreads();

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  auto tile = [&](const char* sK, const char* sV, int k0) {
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        F kf;
        rf.read(kf, sK, kb, ks);
        s[kb] = mfma_k16(kf, qf[ks], s[kb]);
      }
    }
    // Keys past lastkey (range end, ragged tail, causal limit) are masked.
    const int lim = lastkey - k0 - 4 * hf;
    if (lim < 63) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
    float mt = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(fmaxf(s[0][i], s[1][i]), mt);
    mt = fmaxf(mt, other_half(mt)) * a.c;
    if (__ballot(mt > m + kSplitSlack)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    // A row that has seen no key yet keeps m = -inf; its p are exp2(-inf) = 0.
    const float mref = (m == -INFINITY) ? 0.f : m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -mref));
    PF pfs[kSplitKeys / 16];
    float ts = 0.f;
#pragma unroll
    for (int t = 0; t < kSplitKeys / 16; ++t) {
      frag_from(pfs[t], s[t >> 1], (t & 1) * 8);
      ts = add_frag(ts, pfs[t]);  // row sums from the values the product uses
    }
    lsum += ts;
#pragma unroll
    for (int t = 0; t < kSplitKeys / 16; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        PF vf;
        cf.read(vf, sV, t, db);
        acc[db] = mfma_k16(vf, pfs[t], acc[db]);
      }
  };
  auto step = [&](int j, char* sKc, char* sVc, char* sKn, char* sVn) {
    if (j + 1 < nt) copy_kv(sKn, sVn, ks0 + (j + 1) * kSplitKeys);
    tile(sKc, sVc, ks0 + j * kSplitKeys);
    wait_copies();
    if (j + 1 < nt) finish_v(sVn);
    __syncthreads();
  };
  for (int j = 0; j < nt; j += 2) {
    step(j, sK0, sV0, sK1, sV1);
    if (j + 1 >= nt) break;
    step(j + 1, sK1, sV1, sK0, sV0);
  }

  lsum += other_half(lsum);
  const bool seen = lsum > 0.f;
  const float inv = seen ? 1.f / lsum : 0.f;
  const float lse = seen ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
  if (a.nsplit == 1) {
    store_rows<T, D>(reinterpret_cast<T*>(a.o), (int)orow, rvalid ? (int)orow + 1 : (int)orow, acc, inv);
    if (rvalid && hf == 0) a.lse[orow] = lse;
  } else {
    store_rows<float, D>(a.opart, (int)pidx, rvalid ? (int)pidx + 1 : (int)pidx, acc, inv);
    if (rvalid && hf == 0) a.lpart[pidx] = lse;
  }
}

// Variant for bf16 with at most 32 rows per KV head (decoding: g heads x a
// few positions).  There the kernel is bound by reading the cache, which each
// workgroup reads exactly once: the copies carry the non-temporal hint, which
// lifts the streaming rate on this part by about a sixth.  Tiles of 32 keys
// rotate over kRing LDS slots for K and for V, filled by global -> LDS copies
// issued kRing - 1 tiles ahead, so that kRing - 1 of them are in flight while
// one is consumed (80 KB per workgroup at d = 128: two workgroups per CU).  V is
// consumed as bf16 straight from its slot (P V on bf16 MFMA, P rounded to bf16),
// so no V passes through registers.  Only wave 0 has rows; the other waves
// issue their share of the copies and meet the barriers.
constexpr int kRingKeys = 32;
constexpr int kRing = 5;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads, 2) void fa_fwd_split_ring_kernel(SplitArgs a) {
  typedef bf16 T;
  typedef Lay<T, D> L;
  typedef TileCopy<T, D, kRingKeys, kSplitWaves> TC;
  constexpr int TB = kRingKeys * L::RB;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char sK[kRing][TB], sV[kRing][TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  int bid = blockIdx.x;
  const int sp = bid % a.nsplit;
  const int unit = bid / a.nsplit;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int g = a.H / a.Hkv;
  const int R = g * a.Nq;                    // rows of this KV head, at most 32
  const bool rvalid = l32 < R;
  const int rr = rvalid ? l32 : R - 1;
  const int h = kvh * g + rr / a.Nq, qi = rr % a.Nq;
  const long orow = ((long)b * a.H + h) * a.Nq + qi;

  const int off = a.Nk - a.Nq;
  const int ks0 = sp * a.split_len;
  int kend = min(a.Nk, ks0 + a.split_len);
  if (CAUSAL) kend = min(kend, (R >= a.Nq ? a.Nq - 1 : R - 1) + off + 1);
  const int nt = kend > ks0 ? (kend - ks0 + kRingKeys - 1) / kRingKeys : 0;
  const int lastkey = CAUSAL ? min(kend - 1, qi + off) : kend - 1;
  const long pidx = (long)sp * a.B * a.H * a.Nq + orow;

  bf16x8 qf[KS];
  if (w == 0) {
    const T* qp = reinterpret_cast<const T*>(a.q) + orow * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) frag_at(qf[s], qp + 16 * s + 8 * hf);
    wait_loads();
  }
  const size_t slab = (size_t)a.Nk * D;
  const T* Kh = reinterpret_cast<const T*>(a.k) + (size_t)unit * slab;
  const T* Vh = reinterpret_cast<const T*>(a.v) + (size_t)unit * slab;
  RowFrags<T, D> rf;
  ColFrags<T, D> cf;
  TC tc;
  rf.init();
  cf.init();
  tc.init(w);
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    lds_zero<kSplitThreads>(sK[i], TB);
    lds_zero<kSplitThreads>(sV[i], TB);
  }
  __syncthreads();
  auto issue = [&](int j, int slot) {
    tc.template issue<true>(Kh, a.Nk, ks0 + j * kRingKeys, sK[slot]);
    tc.template issue<true>(Vh, a.Nk, ks0 + j * kRingKeys, sV[slot]);
  };
  // Waits until tile j + 1 has landed: the copies of the tiles after it (at
  // most kRing - 2 of them, 2 CPW instructions each) may stay in flight.
  auto wait_next = [&](int j) {
    const int after = min(nt - 1, j + kRing - 1) - (j + 1);
    if (after >= 3) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * 2 * TC::CPW) : "memory");
    else if (after == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * 2 * TC::CPW) : "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * TC::CPW) : "memory");
    else wait_copies();
  };
  static_assert(kRing == 5, "wait_next covers up to three tiles after the next one");
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i)
    if (i < nt) issue(i, i);
  wait_next(-1);
  __syncthreads();

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  auto tile = [&](int slot, int k0) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kf;
      rf.read(kf, sK[slot], 0, ks);
      s = mfma_k16(kf, qf[ks], s);
    }
    const int lim = lastkey - k0 - 4 * hf;
    if (lim < 27) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > lim) s[i] = -INFINITY;
    }
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = fmaxf(mt, other_half(mt)) * a.c;
    if (__ballot(mt > m + kSplitSlack)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    bf16x8 pf[2];
    float ts = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16 pb = (bf16)fast_exp2(__builtin_fmaf(s[8 * t + e], a.c, -mref));
        pf[t][e] = pb;
        ts += (float)pb;  // the row sum of the values the product uses
      }
    lsum += ts;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 vf;
        cf.read(vf, sV[slot], t, db);
        acc[db] = mfma_k16(vf, pf[t], acc[db]);
      }
  };
  // Tile j sits in slot j % kRing; unrolled by kRing so that slots are fixed.
  auto step = [&](int j, int slot) {
    if (j + kRing - 1 < nt) issue(j + kRing - 1, (slot + kRing - 1) % kRing);
    if (w == 0) tile(slot, ks0 + j * kRingKeys);
    wait_next(j);
    __syncthreads();
  };
  for (int j = 0; j < nt; j += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u)
      if (j + u < nt) step(j + u, u);
  }

  if (w != 0) return;
  lsum += other_half(lsum);
  const bool seen = lsum > 0.f;
  const float inv = seen ? 1.f / lsum : 0.f;
  const float lse = seen ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
  if (a.nsplit == 1) {
    store_rows<T, D>(reinterpret_cast<T*>(a.o), (int)orow, rvalid ? (int)orow + 1 : (int)orow, acc, inv);
    if (rvalid && hf == 0) a.lse[orow] = lse;
  } else {
    store_rows<float, D>(a.opart, (int)pidx, rvalid ? (int)pidx + 1 : (int)pidx, acc, inv);
    if (rvalid && hf == 0) a.lpart[pidx] = lse;
  }
}

// Merge of the ranges: one thread per 4 columns of one row.  LSE = log sum
// exp(LSE_s) (max-subtracted), O = sum_s exp(LSE_s - LSE) O_s.
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ opart, const float* __restrict__ lpart,
                                                       T* __restrict__ o, float* __restrict__ lse, long rows,
                                                       int nsplit) {
  constexpr int TPR = D / 4;  // threads per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / TPR;
  const int c4 = (int)(t % TPR) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, lpart[(long)s * rows + row]);
  const float ms = (mx == -INFINITY) ? 0.f : mx;
  float z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = __expf(lpart[(long)s * rows + row] - ms);
    const f32x4 x = *reinterpret_cast<const f32x4*>(opart + ((long)s * rows + row) * D + c4);
    z += wgt;
    acc += wgt * x;
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  store4(o + row * D + c4, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (c4 == 0) lse[row] = (mx == -INFINITY) ? -INFINITY : ms + __logf(z);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_split_t(const SplitParams& p, hipStream_t stream) {
  SplitArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.opart = p.opart; a.lpart = p.lpart; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Nq = p.Nq; a.Nk = p.Nk;
  a.nrb = (p.H / p.Hkv * p.Nq + kSplitRows - 1) / kSplitRows;
  a.nsplit = p.nsplit;
  a.split_len = p.split_len;
  a.c = p.scale * kLog2e;
  if constexpr (sizeof(T) == 2) {
    if (p.H / p.Hkv * p.Nq <= 32) {
      const dim3 grid((unsigned)((long)a.nsplit * p.B * p.Hkv));
      hipLaunchKernelGGL((fa_fwd_split_ring_kernel<D, CAUSAL>), grid, dim3(kSplitThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)((long)a.nrb * a.nsplit * p.B * p.Hkv));
  hipLaunchKernelGGL((fa_fwd_split_kernel<T, D, CAUSAL>), grid, dim3(kSplitThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge_t(const MergeParams& p, hipStream_t stream) {
  const long threads = p.rows * (D / 4);
  hipLaunchKernelGGL((fa_merge_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     p.opart, p.lpart, reinterpret_cast<T*>(p.o), p.lse, p.rows, p.nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_split(const SplitParams& p, hipStream_t stream) {
  if (p.dtype == kBF16) {
    if (p.d == 64) return p.causal ? launch_split_t<bf16, 64, true>(p, stream) : launch_split_t<bf16, 64, false>(p, stream);
    return p.causal ? launch_split_t<bf16, 128, true>(p, stream) : launch_split_t<bf16, 128, false>(p, stream);
  }
  if (p.d == 64) return p.causal ? launch_split_t<float, 64, true>(p, stream) : launch_split_t<float, 64, false>(p, stream);
  return p.causal ? launch_split_t<float, 128, true>(p, stream) : launch_split_t<float, 128, false>(p, stream);
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.dtype == kBF16) return p.d == 64 ? launch_merge_t<bf16, 64>(p, stream) : launch_merge_t<bf16, 128>(p, stream);
  return p.d == 64 ? launch_merge_t<float, 64>(p, stream) : launch_merge_t<float, 128>(p, stream);
}

}  // namespace fa
