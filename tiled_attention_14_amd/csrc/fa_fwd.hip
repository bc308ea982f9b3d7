// fa_fwd.hip — tiled online-softmax attention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T) V and the per-row log-sum-exp without
// materialising the score matrix.  Q, K and V are cut into tiles (the tiling
// of "【词汇专栏】FlashAttention", section 2.1 分块计算, and of
// "FlashAttention 在昇腾NPU上到底快在哪", section 二); each query row keeps a
// running maximum m and exponential sum l that are corrected whenever a new
// tile raises the maximum, and the output is normalised once at the end (the
// incremental softmax of the same page, section 三, and of the explainer,
// section 2.2).  Work is spread over batch x head x query tile, i.e. the
// sequence dimension is parallel too ("FlashAttention V2深度解析", section
// 改进2：并行化策略优化).
//
// Mapping onto the CDNA4 compute unit:
//  * one workgroup = 4 wavefronts = 128 query rows; each wave owns 32 rows;
//  * K/V tiles of 64 keys are staged through LDS with a double buffer: the
//    global loads of tile j+1 are in flight while tile j is consumed;
//  * scores are produced transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so a
//    lane owns one query column: the row max / row sum need only one exchange
//    between the two lane halves (v_permlane32_swap), and the rescale of the
//    accumulator is a per-lane scalar;
//  * O^T += V^T P^T reuses the probability registers directly as the B
//    operand; V^T comes from LDS through the gfx950 transposing read;
//  * softmax runs in the log2 domain: p = exp2(s * scale*log2(e) - m).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBr = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;              // keys per tile

struct FwdArgs {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N, nqt;
  float c;  // scale * log2(e)
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fa_fwd_kernel(FwdArgs a) {
  typedef typename Frag<T>::type F;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KST = D + EPC;      // +16 B per K row
  constexpr int VST = D + 2 * EPC;  // +32 B per V row
  constexpr int KS = D / 16;        // contraction steps over d
  constexpr int DB = D / 32;        // 32-wide blocks of d in the output
  constexpr int SB = kFwdBc / 32;   // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) T sK[2][kFwdBc * KST];
  __shared__ __attribute__((aligned(16))) T sV[2][kFwdBc * VST];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;

  // Heaviest (latest) query tiles are dispatched first under the causal mask.
  const int BH = a.B * a.H;
  const int bid = blockIdx.x;
  const int qt = a.nqt - 1 - bid / BH;
  const int bh = bid % BH;
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = h / (a.H / a.Hkv);
  const T* Q = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * D;
  const T* K = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * N * D;
  const T* V = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * N * D;

  const int q0 = qt * kFwdBr + w * 32;  // first query row of this wave
  const int myq = q0 + l32;             // query row owned by this lane

  F qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (myq < N) frag_rm(qf[s], Q + (size_t)myq * D + 16 * s + 8 * hf);
    else frag_zero(qf[s]);
  }

  const int kend = CAUSAL ? min(N, (qt + 1) * kFwdBr) : N;
  const int nt = (kend + kFwdBc - 1) / kFwdBc;

  TileCopy<T, kFwdBc, D, KST, kFwdThreads> kc;
  TileCopy<T, kFwdBc, D, VST, kFwdThreads> vc;
  kc.load(K, 0, N, tid);
  vc.load(V, 0, N, tid);
  kc.store(sK[0], tid);
  vc.store(sV[0], tid);
  __syncthreads();

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  for (int j = 0; j < nt; ++j) {
    const int cur = j & 1;
    const int k0 = j * kFwdBc;
    if (j + 1 < nt) {
      kc.load(K, k0 + kFwdBc, N, tid);
      vc.load(V, k0 + kFwdBc, N, tid);
    }
    if (!CAUSAL || k0 <= q0 + 31) {
      const T* Kt = sK[cur];
      const T* Vt = sV[cur];
      // S^T = K Q^T for this wave's 32 queries.
      f32x16 s[SB];
#pragma unroll
      for (int kb = 0; kb < SB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          F kf;
          frag_rm(kf, Kt + (kb * 32 + l32) * KST + 16 * ks + 8 * hf);
          s[kb] = mfma_k16(kf, qf[ks], s[kb]);
        }
      }
      // Mask keys beyond N and, under the causal mask, keys after the query.
      if (k0 + kFwdBc > N || (CAUSAL && k0 + kFwdBc - 1 > q0)) {
#pragma unroll
        for (int kb = 0; kb < SB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (key >= N || (CAUSAL && key > myq)) s[kb][i] = -INFINITY;
          }
      }
      // Online softmax update (log2 domain).
      float mt = s[0][0];
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      mt = fmaxf(mt, other_half(mt));
      const float mnew = fmaxf(m, mt * a.c);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -m));
          s[kb][i] = p;
          ps += p;
        }
      lsum += ps;
      // O^T += V^T P^T, 16 keys per step.
#pragma unroll
      for (int t = 0; t < kFwdBc / 16; ++t) {
        F pf;
        frag_from(pf, s[t >> 1], (t & 1) * 8);
        const int rA = (t >> 1) * 32 + (t & 1) * 16 + 4 * hf;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          F vf;
          frag_tr(vf, Vt, VST, rA, rA + 8, db * 32);
          acc[db] = mfma_k16(vf, pf, acc[db]);
        }
      }
    }
    if (j + 1 < nt) {
      kc.store(sK[cur ^ 1], tid);
      vc.store(sV[cur ^ 1], tid);
    }
    __syncthreads();
  }

  lsum += other_half(lsum);
  if (myq < N) {
    const float inv = 1.f / lsum;
    T* O = reinterpret_cast<T*>(a.o) + (size_t)bh * N * D + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hf;
        store4(O + d, acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
               acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      }
    if (hf == 0) a.lse[(size_t)bh * N + myq] = (m + __log2f(lsum)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N;
  a.nqt = (p.N + kFwdBr - 1) / kFwdBr;
  a.c = p.scale * kLog2e;
  const long grid = (long)a.nqt * p.B * p.H;
  hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd_d(const FwdParams& p, hipStream_t s) {
  if (p.d == 64) return p.causal ? launch_fwd_t<T, 64, true>(p, s) : launch_fwd_t<T, 64, false>(p, s);
  return p.causal ? launch_fwd_t<T, 128, true>(p, s) : launch_fwd_t<T, 128, false>(p, s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? launch_fwd_d<bf16>(p, stream) : launch_fwd_d<float>(p, stream);
}

}  // namespace fa
