// fa_bwd.hip — FlashAttention-2 style backward pass for gfx950.
//
// The probabilities are never stored: the backward pass recomputes them from
// Q, K and the forward's per-row log-sum-exp, trading arithmetic for memory
// ("FlashAttention V2深度解析", section 改进1：IO感知的算子调度), so the extra
// memory is O(N).  For the loss L = sum(dO * O):
//
//   P   = exp(scale * Q K^T - LSE)          (masked entries 0)
//   dV  = P^T dO
//   dP  = dO V^T
//   dS  = P * (dP - D),  D_i = sum_c dO_ic O_ic
//   dQ  = scale * dS K,   dK = scale * dS^T Q
//
// dS = P * (dP - D) is the full softmax Jacobian applied to dP (the
// diagonal-only form printed on that page drops the off-diagonal terms); the
// row constant D equals sum_j P_ij dP_ij because O = P V.
//
// Kernels (all on the caller's stream, no host synchronisation):
//  1. fa_bwd_pre:  D = rowsum(dO * O) and lse * log2(e), one float each per
//     query row, into the workspace;
//  2. fa_bwd_dkdv: one workgroup per (batch, KV head, 128-key tile[, slice of
//     the GQA group]); K/V fragments and the dK/dV accumulators stay in
//     registers while Q/dO tiles of 64 rows stream through LDS (global -> LDS
//     copies, double-buffered), for every query head of the group and, under
//     the causal mask, only from the diagonal on.  No atomics: each key row is
//     owned by one lane.  When a GQA group is sliced over several workgroups
//     (to balance the work of very wide groups), each writes float32 partial
//     sums and fa_bwd_reduce adds them in a fixed order;
//  3. fa_bwd_dq:   one workgroup per (batch, head, 128-query tile); Q/dO
//     fragments and the dQ accumulator stay in registers while K/V tiles of 64
//     keys stream through LDS.  It recomputes S and dP instead of exchanging
//     dS with the dK/dV kernel: seven products in total instead of five, but
//     no float atomics, whose L2 throughput on this part is far below what a
//     shared dQ accumulator would need.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dO;
  const float* delta; const float* lse2;
  void* dq; void* dk; void* dv;
  float* part;
  int B, H, Hkv, N, nsplit;
  float c;      // scale * log2(e)
  float scale;
};

BwdArgs make_args(const BwdParams& p) {
  BwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.dO = p.dO;
  a.delta = p.delta; a.lse2 = p.lse2;
  a.dq = p.dq; a.dk = p.dk; a.dv = p.dv; a.part = p.part;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N; a.nsplit = p.nsplit;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  return a;
}

// ------------------------------------------------------------------ 1. preprocess
// D/8 threads share a row; each handles 8 elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                         const float* __restrict__ lse, float* __restrict__ delta,
                                                         float* __restrict__ lse2, long rows) {
  constexpr int TPR = D / 8;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / TPR;
  const int c8 = (int)(t % TPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c8 * 8;
    float o[8], g[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(O + off);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(dO + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) { o[i] = (float)x[i]; g[i] = (float)y[i]; }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) { o[i] = O[off + i]; g[i] = dO[off + i]; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(o[i], g[i], acc);
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, TPR);
  if (row < rows && c8 == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ 2. dK / dV
constexpr int kKeys = kDkdvKeys;    // keys per workgroup (32 per wave)
constexpr int kQRows = kDkdvQRows;  // query rows per step
static_assert(kKeys == 32 * kWaves, "one 32-key column block per wave");

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a) {
  typedef typename Frag<T>::type F;
  typedef Lay<T, D> L;
  constexpr int TB = kQRows * L::RB;
  constexpr int KS = D / 16, DB = D / 32, MB = kQRows / 32;
  __shared__ __attribute__((aligned(1024))) char sQ0[TB], sQ1[TB], sO0[TB], sO1[TB];
  __shared__ __attribute__((aligned(256))) float sL0[kQRows], sL1[kQRows], sD0[kQRows], sD1[kQRows];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int g = a.H / a.Hkv, gs = g / a.nsplit;
  int unit, kt;
  xcd_map(blockIdx.x, a.B * a.Hkv * a.nsplit, unit, kt);  // lowest key tiles (most work) first
  const int bkv = unit / a.nsplit, sp = unit % a.nsplit;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const int h0 = kvh * g + sp * gs;  // first query head of this slice
  const size_t slab = (size_t)N * D;
  const uint32_t slab_bytes = (uint32_t)(slab * sizeof(T));
  const int k0 = kt * kKeys;
  const int kw = k0 + 32 * w;  // first key of this wave
  const int mykey = kw + l32;  // key row owned by this lane

  // K and V rows of this lane's key, as B fragments of S = Q K^T and dP = dO V^T.
  F kf[KS], vf[KS];
  {
    const rsrc_t rK = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)bkv * slab, slab_bytes);
    const rsrc_t rV = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)bkv * slab, slab_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag_global<D>(kf[s], rK, mykey, 16 * s + 8 * hf);
      frag_global<D>(vf[s], rV, mykey, 16 * s + 8 * hf);
    }
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int nqt = (N + kQRows - 1) / kQRows;
  const int qstart = CAUSAL ? k0 / kQRows : 0;
  const int nq = nqt - qstart;
  const int total = gs * nq;

  lds_zero<kThreads>(sQ0, TB); lds_zero<kThreads>(sQ1, TB);
  lds_zero<kThreads>(sO0, TB); lds_zero<kThreads>(sO1, TB);
  lds_zero<kThreads>(reinterpret_cast<char*>(sL0), 4 * kQRows);
  lds_zero<kThreads>(reinterpret_cast<char*>(sL1), 4 * kQRows);
  lds_zero<kThreads>(reinterpret_cast<char*>(sD0), 4 * kQRows);
  lds_zero<kThreads>(reinterpret_cast<char*>(sD1), 4 * kQRows);
  __syncthreads();

  // Copies of step `it` (query head h0 + it / nq, query tile qstart + it % nq).
  auto fetch = [&](int it, char* bq, char* bo, float* bl, float* bd) {
    const int hq = h0 + it / nq;
    const int qb0 = (qstart + it % nq) * kQRows;
    const size_t head = (size_t)b * a.H + hq;
    const rsrc_t rQ = make_rsrc(reinterpret_cast<const T*>(a.q) + head * slab, slab_bytes);
    const rsrc_t rO = make_rsrc(reinterpret_cast<const T*>(a.dO) + head * slab, slab_bytes);
    tile_to_lds<T, D, kQRows, kWaves>(rQ, bq, qb0, w);
    tile_to_lds<T, D, kQRows, kWaves>(rO, bo, qb0, w);
    if (w == 0) vec64_to_lds(make_rsrc(a.lse2 + head * N, (uint32_t)N * 4u), bl, qb0);
    if (w == 1) vec64_to_lds(make_rsrc(a.delta + head * N, (uint32_t)N * 4u), bd, qb0);
  };

  auto step = [&](const char* sQ, const char* sO, const float* sL, const float* sD, int it) {
    const int qb0 = (qstart + it % nq) * kQRows;
    if (CAUSAL && qb0 + kQRows - 1 < kw) return;  // every query of the step is before every key of the wave
    f32x16 s[MB], dp[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = f32x16{};
      dp[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        F qa, oa;
        frag_row<D>(qa, sQ, mb * 32 + l32, 16 * ks + 8 * hf);
        frag_row<D>(oa, sO, mb * 32 + l32, 16 * ks + 8 * hf);
        s[mb] = mfma_k16(qa, kf[ks], s[mb]);
        dp[mb] = mfma_k16(oa, vf[ks], dp[mb]);
      }
    }
    const bool need_mask = (CAUSAL && kw + 31 > qb0) || (qb0 + kQRows > N);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql0 = mb * 32 + 8 * g4 + 4 * hf;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + ql0);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(sD + ql0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          float p = fast_exp2(__builtin_fmaf(s[mb][i], a.c, -lv[e]));
          if (need_mask) {
            const int q = qb0 + ql0 + e;
            if ((CAUSAL && mykey > q) || q >= N) p = 0.f;
          }
          s[mb][i] = p;
          dp[mb][i] = p * (dp[mb][i] - dd[e]);
        }
      }
    // dV^T += dO^T P and dK^T += Q^T dS, 16 query rows per step.
#pragma unroll
    for (int t = 0; t < 2 * MB; ++t) {
      F pf, dsf;
      frag_from(pf, s[t >> 1], (t & 1) * 8);
      frag_from(dsf, dp[t >> 1], (t & 1) * 8);
      const int rA = (t >> 1) * 32 + (t & 1) * 16 + 4 * hf;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        F oa, qa;
        frag_col<D>(oa, sO, rA, rA + 8, db * 32);
        dv[db] = mfma_k16(oa, pf, dv[db]);
        frag_col<D>(qa, sQ, rA, rA + 8, db * 32);
        dk[db] = mfma_k16(qa, dsf, dk[db]);
      }
    }
  };

  if (total > 0) fetch(0, sQ0, sO0, sL0, sD0);
  wait_copies();
  __syncthreads();
  for (int it = 0; it < total; it += 2) {
    if (it + 1 < total) fetch(it + 1, sQ1, sO1, sL1, sD1);
    step(sQ0, sO0, sL0, sD0, it);
    wait_copies();
    __syncthreads();
    if (it + 1 >= total) break;
    if (it + 2 < total) fetch(it + 2, sQ0, sO0, sL0, sD0);
    step(sQ1, sO1, sL1, sD1, it + 1);
    wait_copies();
    __syncthreads();
  }

  if (a.nsplit == 1) {
    store_rows<T, D>(reinterpret_cast<T*>(a.dk) + (size_t)bkv * slab, mykey, N, dk, a.scale);
    store_rows<T, D>(reinterpret_cast<T*>(a.dv) + (size_t)bkv * slab, mykey, N, dv, 1.f);
  } else {
    const size_t ps = (size_t)a.B * a.Hkv * slab;  // elements of one partial tensor
    store_rows<float, D>(a.part + (2 * sp) * ps + (size_t)bkv * slab, mykey, N, dk, a.scale);
    store_rows<float, D>(a.part + (2 * sp + 1) * ps + (size_t)bkv * slab, mykey, N, dv, 1.f);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dkdv_kernel_bf16(BwdArgs a) { dkdv_body<bf16, D, CAUSAL>(a); }
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dkdv_kernel_f32(BwdArgs a) { dkdv_body<float, D, CAUSAL>(a); }

// Sums the nsplit float32 partials of dK and dV (in slice order) into dk / dv.
template <typename T>
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(const float* __restrict__ part, T* __restrict__ dk,
                                                            T* __restrict__ dv, long n4, int nsplit) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= 2 * n4) return;
  const int which = t >= n4;  // 0: dK, 1: dV
  const long i = t - which * n4;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + which * n4 + i;
  f32x4 acc = p[0];
  for (int s = 1; s < nsplit; ++s) acc += p[(long)s * 2 * n4];
  store4((which ? dv : dk) + 4 * i, acc[0], acc[1], acc[2], acc[3]);
}

// ------------------------------------------------------------------ 3. dQ
constexpr int kQTile = 32 * kWaves;  // query rows per workgroup
constexpr int kKTile = 64;           // keys per streamed tile

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int nqt) {
  typedef typename Frag<T>::type F;
  typedef Lay<T, D> L;
  constexpr int TB = kKTile * L::RB;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char sK0[TB], sK1[TB], sV0[TB], sV1[TB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  int bh, qi;
  xcd_map(blockIdx.x, a.B * a.H, bh, qi);
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = h / (a.H / a.Hkv);
  const size_t slab = (size_t)N * D;
  const uint32_t slab_bytes = (uint32_t)(slab * sizeof(T));
  const rsrc_t rK = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * slab, slab_bytes);
  const rsrc_t rV = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * slab, slab_bytes);

  const int q0w = qt * kQTile + 32 * w;
  const int myq = q0w + l32;
  F qf[KS], of[KS];
  float l2, dd;
  {
    const rsrc_t rQ = make_rsrc(reinterpret_cast<const T*>(a.q) + (size_t)bh * slab, slab_bytes);
    const rsrc_t rO = make_rsrc(reinterpret_cast<const T*>(a.dO) + (size_t)bh * slab, slab_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag_global<D>(qf[s], rQ, myq, 16 * s + 8 * hf);
      frag_global<D>(of[s], rO, myq, 16 * s + 8 * hf);
    }
    l2 = load4f(make_rsrc(a.lse2 + (size_t)bh * N, (uint32_t)N * 4u), (uint32_t)myq * 4u);
    dd = load4f(make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4u), (uint32_t)myq * 4u);
  }

  const int kend = CAUSAL ? min(N, (qt + 1) * kQTile) : N;
  const int nt = (kend + kKTile - 1) / kKTile;

  lds_zero<kThreads>(sK0, TB); lds_zero<kThreads>(sK1, TB);
  lds_zero<kThreads>(sV0, TB); lds_zero<kThreads>(sV1, TB);
  __syncthreads();
  tile_to_lds<T, D, kKTile, kWaves>(rK, sK0, 0, w);
  tile_to_lds<T, D, kKTile, kWaves>(rV, sV0, 0, w);
  wait_copies();
  __syncthreads();

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  auto tile = [&](const char* sK, const char* sV, int k0) {
    if (CAUSAL && k0 > q0w + 31) return;
    // S^T = K Q^T and dP^T = V dO^T for this wave's 32 queries.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        F kf, vf;
        frag_row<D>(kf, sK, kb * 32 + l32, 16 * ks + 8 * hf);
        frag_row<D>(vf, sV, kb * 32 + l32, 16 * ks + 8 * hf);
        s[kb] = mfma_k16(kf, qf[ks], s[kb]);
        dp[kb] = mfma_k16(vf, of[ks], dp[kb]);
      }
    }
    const bool need_mask = CAUSAL ? (k0 + kKTile - 1 > q0w) : (k0 + kKTile > N);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -l2));
        if (need_mask) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (CAUSAL ? key > myq : key >= N) p = 0.f;
        }
        dp[kb][i] = p * (dp[kb][i] - dd);
      }
    // dQ^T += K^T dS^T, 16 keys per step.
#pragma unroll
    for (int t = 0; t < kKTile / 16; ++t) {
      F dsf;
      frag_from(dsf, dp[t >> 1], (t & 1) * 8);
      const int rA = (t >> 1) * 32 + (t & 1) * 16 + 4 * hf;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        F kf;
        frag_col<D>(kf, sK, rA, rA + 8, db * 32);
        acc[db] = mfma_k16(kf, dsf, acc[db]);
      }
    }
  };

  for (int j = 0; j < nt; j += 2) {
    if (j + 1 < nt) {
      tile_to_lds<T, D, kKTile, kWaves>(rK, sK1, (j + 1) * kKTile, w);
      tile_to_lds<T, D, kKTile, kWaves>(rV, sV1, (j + 1) * kKTile, w);
    }
    tile(sK0, sV0, j * kKTile);
    wait_copies();
    __syncthreads();
    if (j + 1 >= nt) break;
    if (j + 2 < nt) {
      tile_to_lds<T, D, kKTile, kWaves>(rK, sK0, (j + 2) * kKTile, w);
      tile_to_lds<T, D, kKTile, kWaves>(rV, sV0, (j + 2) * kKTile, w);
    }
    tile(sK1, sV1, (j + 1) * kKTile);
    wait_copies();
    __syncthreads();
  }

  store_rows<T, D>(reinterpret_cast<T*>(a.dq) + (size_t)bh * slab, myq, N, acc, a.scale);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_bwd_dq_kernel_bf16(BwdArgs a, int nqt) {
  dq_body<bf16, D, CAUSAL>(a, nqt);
}
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dq_kernel_f32(BwdArgs a, int nqt) {
  dq_body<float, D, CAUSAL>(a, nqt);
}

// ------------------------------------------------------------------ launchers
template <typename T, int D>
hipError_t launch_pre_t(const BwdParams& p, hipStream_t stream) {
  const long rows = (long)p.B * p.H * p.N;
  const long threads = rows * (D / 8);
  hipLaunchKernelGGL((fa_bwd_pre_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(p.o), reinterpret_cast<const T*>(p.dO), p.lse, p.delta, p.lse2, rows);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdParams& p, hipStream_t stream) {
  const BwdArgs a = make_args(p);
  const int nkt = (p.N + kKeys - 1) / kKeys;
  const dim3 grid((unsigned)((long)nkt * p.B * p.Hkv * p.nsplit));
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel_bf16<D, CAUSAL>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel_f32<D, CAUSAL>), grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const long n4 = (long)p.B * p.Hkv * p.N * D / 4;
  hipLaunchKernelGGL((fa_bwd_reduce_kernel<T>), dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0, stream,
                     p.part, reinterpret_cast<T*>(p.dk), reinterpret_cast<T*>(p.dv), n4, p.nsplit);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdParams& p, hipStream_t stream) {
  const BwdArgs a = make_args(p);
  const int nqt = (p.N + kQTile - 1) / kQTile;
  const dim3 grid((unsigned)((long)nqt * p.B * p.H));
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((fa_bwd_dq_kernel_bf16<D, CAUSAL>), grid, dim3(kThreads), 0, stream, a, nqt);
  else
    hipLaunchKernelGGL((fa_bwd_dq_kernel_f32<D, CAUSAL>), grid, dim3(kThreads), 0, stream, a, nqt);
  return hipGetLastError();
}

#define FA_DISPATCH(fn, p, s)                                                                      \
  do {                                                                                             \
    if ((p).dtype == kBF16) {                                                                      \
      if ((p).d == 64) return (p).causal ? fn<bf16, 64, true>(p, s) : fn<bf16, 64, false>(p, s);  \
      return (p).causal ? fn<bf16, 128, true>(p, s) : fn<bf16, 128, false>(p, s);                 \
    }                                                                                              \
    if ((p).d == 64) return (p).causal ? fn<float, 64, true>(p, s) : fn<float, 64, false>(p, s);  \
    return (p).causal ? fn<float, 128, true>(p, s) : fn<float, 128, false>(p, s);                 \
  } while (0)

}  // namespace

hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream) {
  if (p.dtype == kBF16) return p.d == 64 ? launch_pre_t<bf16, 64>(p, stream) : launch_pre_t<bf16, 128>(p, stream);
  return p.d == 64 ? launch_pre_t<float, 64>(p, stream) : launch_pre_t<float, 128>(p, stream);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t stream) { FA_DISPATCH(launch_dkdv_t, p, stream); }

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) { FA_DISPATCH(launch_dq_t, p, stream); }

}  // namespace fa
