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
//  1. fa_bwd_pre:  D = rowsum(dO * O) and zeroing of the fp32 dQ accumulator;
//  2. fa_bwd_main: one workgroup per (batch, KV head, 128-key tile); K/V stay
//     resident in registers, dK/dV accumulate in registers (no atomics); the
//     workgroup walks the query tiles of every query head of its GQA group
//     (only tiles at or after the diagonal under the causal mask) and adds
//     its share of dQ into the fp32 accumulator with hardware float atomics;
//  3. fa_bwd_dq_cvt: dQ accumulator -> bf16 (the f32 path accumulates into dq
//     directly and skips it).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// ------------------------------------------------------------------ 1. preprocess
// One thread per 8 elements of a row; D/8 threads share a row.
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                         float* __restrict__ delta, float* __restrict__ dq_acc,
                                                         long rows) {
  constexpr int TPR = D / 8;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / TPR;
  const int c8 = (int)(t % TPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c8 * 8;
    float o[8], g[8];
    if constexpr (sizeof(T) == 2) {
      bf16x8 a = *reinterpret_cast<const bf16x8*>(O + off);
      bf16x8 b = *reinterpret_cast<const bf16x8*>(dO + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) { o[i] = (float)a[i]; g[i] = (float)b[i]; }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) { o[i] = O[off + i]; g[i] = dO[off + i]; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(o[i], g[i], acc);
    f32x4* z = reinterpret_cast<f32x4*>(dq_acc + off);
    z[0] = f32x4{};
    z[1] = f32x4{};
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, TPR);
  if (row < rows && c8 == 0) delta[row] = acc;
}

// ------------------------------------------------------------------ 3. dQ convert
__global__ __launch_bounds__(256) void fa_bwd_dq_cvt_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                            long n8) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * t];
  const f32x4 b = reinterpret_cast<const f32x4*>(acc)[2 * t + 1];
  reinterpret_cast<bf16x8*>(dq)[t] =
      bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

// ------------------------------------------------------------------ 2. main
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdBc = 32 * kBwdWaves;  // keys per workgroup

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dO;
  const float* lse; const float* delta;
  float* dq_acc; void* dk; void* dv;
  int B, H, Hkv, N, nkt;
  float c;      // scale * log2(e)
  float scale;
};

// MB = number of 32-row query blocks per inner step (query tile = 32*MB rows).
template <typename T, int D, bool CAUSAL, int MB>
__global__ __launch_bounds__(kBwdThreads, 1) void fa_bwd_main_kernel(BwdArgs a) {
  typedef typename Frag<T>::type F;
  constexpr int BR = 32 * MB;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int QST = D + EPC;       // Q / dO tile row stride
  constexpr int KST = D + 2 * EPC;   // K tile row stride
  constexpr int SST = BR + 4;       // dS^T tile row stride (keeps 16 B alignment for f32 rows)
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) T sQ[BR * QST];
  __shared__ __attribute__((aligned(16))) T sdO[BR * QST];
  __shared__ __attribute__((aligned(16))) T sK[kBwdBc * KST];
  __shared__ __attribute__((aligned(16))) T sdS[kBwdBc * SST];
  __shared__ float sL[BR], sD[BR];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int BHkv = a.B * a.Hkv;
  const int kt = blockIdx.x / BHkv;          // lowest key tiles carry the most work: first
  const int bkv = blockIdx.x % BHkv;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const int g = a.H / a.Hkv;
  const int k0 = kt * kBwdBc;
  const int kw = k0 + 32 * w;                // first key of this wave
  const int mykey = kw + l32;                // key column owned by this lane

  const T* K = reinterpret_cast<const T*>(a.k) + (size_t)bkv * N * D;
  const T* V = reinterpret_cast<const T*>(a.v) + (size_t)bkv * N * D;

  // K and V rows of this lane's key, as B fragments of S = Q K^T and dP = dO V^T.
  F kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (mykey < N) {
      frag_rm(kf[s], K + (size_t)mykey * D + 16 * s + 8 * hf);
      frag_rm(vf[s], V + (size_t)mykey * D + 16 * s + 8 * hf);
    } else {
      frag_zero(kf[s]);
      frag_zero(vf[s]);
    }
  }
  {
    TileCopy<T, kBwdBc, D, KST, kBwdThreads> kc;
    kc.load(K, k0, N, tid);
    kc.store(sK, tid);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int nqt = (N + BR - 1) / BR;
  const int qstart = CAUSAL ? k0 / BR : 0;
  const int nq = nqt - qstart;
  const int total = g * nq;

  TileCopy<T, BR, D, QST, kBwdThreads> qc, oc;
  float stat = 0.f;  // threads [0, BR): LSE (log2 units); [BR, 2 BR): D
  auto fetch = [&](int it) {
    const int hq = kvh * g + it / nq;
    const int qb0 = (qstart + it % nq) * BR;
    const size_t base = ((size_t)b * a.H + hq) * N;
    qc.load(reinterpret_cast<const T*>(a.q) + base * D, qb0, N, tid);
    oc.load(reinterpret_cast<const T*>(a.dO) + base * D, qb0, N, tid);
    if (tid < BR) stat = (qb0 + tid < N) ? a.lse[base + qb0 + tid] * kLog2e : 0.f;
    else if (tid < 2 * BR) stat = (qb0 + tid - BR < N) ? a.delta[base + qb0 + tid - BR] : 0.f;
  };
  auto stage = [&]() {
    qc.store(sQ, tid);
    oc.store(sdO, tid);
    if (tid < BR) sL[tid] = stat;
    else if (tid < 2 * BR) sD[tid - BR] = stat;
  };

  if (total > 0) {
    fetch(0);
    stage();
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int hq = kvh * g + it / nq;
    const int qb0 = (qstart + it % nq) * BR;
    if (it + 1 < total) fetch(it + 1);

    const bool active = !CAUSAL || (kw <= qb0 + BR - 1);
    T* dsrow = sdS + (32 * w + l32) * SST;
    if (active) {
      f32x16 s[MB], dp[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = f32x16{};
        dp[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          F qa, oa;
          frag_rm(qa, sQ + (mb * 32 + l32) * QST + 16 * ks + 8 * hf);
          frag_rm(oa, sdO + (mb * 32 + l32) * QST + 16 * ks + 8 * hf);
          s[mb] = mfma_k16(qa, kf[ks], s[mb]);
          dp[mb] = mfma_k16(oa, vf[ks], dp[mb]);
        }
      }
      const bool need_mask = (kw + 31 >= N) || (qb0 + BR > N) || (CAUSAL && kw + 31 > qb0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = mb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          float p = fast_exp2(__builtin_fmaf(s[mb][i], a.c, -sL[ql]));
          if (need_mask) {
            const int q = qb0 + ql;
            if (mykey >= N || q >= N || (CAUSAL && mykey > q)) p = 0.f;
          }
          s[mb][i] = p;
          dp[mb][i] = p * (dp[mb][i] - sD[ql]);
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
          frag_tr(oa, sdO, QST, rA, rA + 8, db * 32);
          dv[db] = mfma_k16(oa, pf, dv[db]);
          frag_tr(qa, sQ, QST, rA, rA + 8, db * 32);
          dk[db] = mfma_k16(qa, dsf, dk[db]);
        }
      }
      // scale * dS^T into LDS for the dQ product.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
          store4(dsrow + mb * 32 + 8 * gi + 4 * hf, a.scale * dp[mb][4 * gi], a.scale * dp[mb][4 * gi + 1],
                 a.scale * dp[mb][4 * gi + 2], a.scale * dp[mb][4 * gi + 3]);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) store4(dsrow + mb * 32 + 8 * gi + 4 * hf, 0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // dQ[BR x D] += (scale dS)[BR x 128] K[128 x D]; 32x32 output blocks over the waves.
    {
      float* dq = a.dq_acc + ((size_t)b * a.H + hq) * N * D;
      for (int blk = w; blk < MB * DB; blk += kBwdWaves) {
        const int qb = blk % MB, db = blk / MB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < kBwdBc / 16; ++t) {
          const int rA = 16 * t + 4 * hf;
          F sa, kb;
          frag_tr(sa, sdS, SST, rA, rA + 8, qb * 32);
          frag_tr(kb, sK, KST, rA, rA + 8, db * 32);
          acc = mfma_k16(sa, kb, acc);
        }
        const int d = db * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qb0 + qb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (q < N) unsafeAtomicAdd(dq + (size_t)q * D + d, acc[i]);
        }
      }
    }
    if (it + 1 < total) stage();
    __syncthreads();
  }

  if (mykey < N) {
    T* dK = reinterpret_cast<T*>(a.dk) + (size_t)bkv * N * D + (size_t)mykey * D;
    T* dV = reinterpret_cast<T*>(a.dv) + (size_t)bkv * N * D + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = db * 32 + 8 * gi + 4 * hf;
        store4(dK + d, a.scale * dk[db][4 * gi], a.scale * dk[db][4 * gi + 1], a.scale * dk[db][4 * gi + 2],
               a.scale * dk[db][4 * gi + 3]);
        store4(dV + d, dv[db][4 * gi], dv[db][4 * gi + 1], dv[db][4 * gi + 2], dv[db][4 * gi + 3]);
      }
  }
}

template <typename T, int D>
hipError_t launch_pre_t(const BwdParams& p, hipStream_t stream) {
  const long rows = (long)p.B * p.H * p.N;
  const long threads = rows * (D / 8);
  hipLaunchKernelGGL((fa_bwd_pre_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(p.o), reinterpret_cast<const T*>(p.dO), p.delta, p.dq_acc, rows);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_main_t(const BwdParams& p, hipStream_t stream) {
  constexpr int MB = sizeof(T) == 2 ? 2 : 1;
  BwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.dO = p.dO; a.lse = p.lse; a.delta = p.delta;
  a.dq_acc = p.dq_acc; a.dk = p.dk; a.dv = p.dv;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N;
  a.nkt = (p.N + kBwdBc - 1) / kBwdBc;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  const long grid = (long)a.nkt * p.B * p.Hkv;
  hipLaunchKernelGGL((fa_bwd_main_kernel<T, D, CAUSAL, MB>), dim3((unsigned)grid), dim3(kBwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_main_d(const BwdParams& p, hipStream_t s) {
  if (p.d == 64) return p.causal ? launch_main_t<T, 64, true>(p, s) : launch_main_t<T, 64, false>(p, s);
  return p.causal ? launch_main_t<T, 128, true>(p, s) : launch_main_t<T, 128, false>(p, s);
}

}  // namespace

hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream) {
  if (p.dtype == kBF16) return p.d == 64 ? launch_pre_t<bf16, 64>(p, stream) : launch_pre_t<bf16, 128>(p, stream);
  return p.d == 64 ? launch_pre_t<float, 64>(p, stream) : launch_pre_t<float, 128>(p, stream);
}

hipError_t launch_bwd_main(const BwdParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? launch_main_d<bf16>(p, stream) : launch_main_d<float>(p, stream);
}

hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t stream) {
  if (p.dtype != kBF16) return hipSuccess;  // the f32 path accumulates into dq directly
  const long n8 = (long)p.B * p.H * p.N * p.d / 8;
  hipLaunchKernelGGL(fa_bwd_dq_cvt_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, p.dq_acc,
                     reinterpret_cast<bf16*>(p.dq), n8);
  return hipGetLastError();
}

}  // namespace fa
