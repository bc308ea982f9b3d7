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
//  * one workgroup = 8 wavefronts = 256 query rows (bf16 at d = 128; 4 and
//    128 for bf16 at d = 64 and for fp32); each wave owns 32 rows, whose Q
//    fragments stay in registers for the whole kernel;
//  * K/V tiles of 64 keys go global -> LDS directly (buffer loads with the LDS
//    destination), double-buffered: the copies of tile j+1 are in flight while
//    tile j is consumed; rows past N arrive as zeros;
//  * scores are produced transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so a
//    lane owns one query column: the row max / row sum need one exchange
//    between the two lane halves (v_permlane32_swap) and the rescale is a
//    per-lane scalar;
//  * O^T += V^T P^T reuses the probability registers directly as the B
//    operand; V^T comes from LDS through the gfx950 transposing read.  For
//    bf16 inputs this product runs in fp16 (P and V converted, fp32
//    accumulation): fp16 keeps 3 more significand bits than bf16, which bounds
//    the error of O before its final bf16 rounding by about 2^-12 |O| instead
//    of 2^-9 |O|, so that peaked rows of long sequences stay within 1e-2 after
//    that rounding.  Each wave loads its part of the next V tile into
//    registers at the start of a step and writes it, converted, to the fp16
//    tile before the step's barrier, so the conversion needs no extra barrier;
//  * softmax runs in the log2 domain, p = exp2(s * scale*log2(e) - m), and the
//    running maximum is only moved when a tile raises it by more than 2^8:
//    any reference point gives the same O = acc / l and lse = m + log2(l), so
//    skipping small moves saves the accumulator rescale on most tiles.  For
//    bf16, tiles after the first are exponentiated against the running max as
//    it stands and kept when no p exceeds 2^15 (inside the fp16 range); only
//    otherwise is the tile max taken and the tile redone;
//  * workgroups of one (batch, head) share an XCD (and its L2), and under the
//    causal mask the longest query tiles are dispatched first.
#include "fa_device.h"
#include "fa_kernels.h"

#include <type_traits>

namespace fa {
namespace {

// Waves per workgroup (32 query rows each).  bf16, d = 128: eight waves, two
// per SIMD, share each K/V tile, its copy and the V conversion (one workgroup
// per CU by registers).  bf16, d = 64: four waves, and the register bound asks
// for three workgroups per CU (at most 168 registers per wave), so three waves
// from different workgroups share each SIMD.  fp32 (more registers per wave):
// four.
template <int D> constexpr int waves_bf16() { return D == 64 ? 4 : 8; }
template <int D> constexpr int wgs_bf16() { return D == 64 ? 3 : 2; }
constexpr int kWavesF32 = 4;
constexpr int kBc = 64;           // keys per tile
constexpr float kSlack = 8.f;     // log2 units the running max may lag behind
// bf16: a tile is first exponentiated against the running max as it stands;
// the result is kept when every lane's share of the tile's row sum is at most
// this (so every p <= 2^15, inside fp16 range).  Otherwise the tile max is
// taken and the tile redone.
constexpr float kPLimit = 32768.f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct FwdArgs {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N, nqt;
  float c;  // scale * log2(e)
  DropArgs drop;
};

// Operand type of the P V product: fp16 for bf16 inputs, fp32 for fp32 inputs.
template <typename T> struct PvFrag;
template <> struct PvFrag<bf16> { typedef f16x8 type; };
template <> struct PvFrag<float> { typedef f32x8 type; };

template <typename T, int D, bool CAUSAL, int NW, bool DROP>
__device__ __forceinline__ void fwd_body(const FwdArgs& a) {
  constexpr int kWaves = NW, kThreads = 64 * NW, kBr = 32 * NW;
  typedef typename Frag<T>::type F;
  typedef typename PvFrag<T>::type PF;
  typedef Lay<T, D> L;
  constexpr bool kConv = sizeof(T) == 2;  // V staged as bf16, consumed as fp16
  constexpr int TB = kBc * L::RB;         // bytes of one K or V tile
  constexpr int KS = D / 16;              // contraction steps over d
  constexpr int DB = D / 32;              // 32-wide blocks of d in the output
  __shared__ __attribute__((aligned(1024))) char sK0[TB], sK1[TB], sV0[TB], sV1[TB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  int bh, qi;
  xcd_map(blockIdx.x, a.B * a.H, bh, qi);
  const int qt = CAUSAL ? a.nqt - 1 - qi : qi;
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = h / (a.H / a.Hkv);
  const size_t slab = (size_t)N * D;
  const uint32_t slab_bytes = (uint32_t)(slab * sizeof(T));
  const rsrc_t rQ = make_rsrc(reinterpret_cast<const T*>(a.q) + (size_t)bh * slab, slab_bytes);

  const int q0w = qt * kBr + 32 * w;  // first query row of this wave
  const int myq = q0w + l32;          // query row owned by this lane
  // Q rows; they land while the tiles are cleared and the first one copied.
  F qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) frag_global<D>(qf[s], rQ, myq, 16 * s + 8 * hf);

  const int kend = CAUSAL ? min(N, (qt + 1) * kBr) : N;
  const int nt = (kend + kBc - 1) / kBc;
  const T* Kh = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * slab;
  const T* Vh = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * slab;
  RowFrags<T, D> rf;
  ColFrags<T, D> cf;
  TileCopy<T, D, kBc, kWaves> tc;
  rf.init();
  cf.init();
  tc.init(w);

  // Zero the tiles once so that nothing read from LDS is ever uninitialised.
  lds_zero<kThreads>(sK0, TB); lds_zero<kThreads>(sK1, TB);
  lds_zero<kThreads>(sV0, TB); lds_zero<kThreads>(sV1, TB);
  __syncthreads();
  // K tile j+1 is copied straight into its buffer.  V tile j+1 goes the same
  // way for fp32; bf16 V is loaded into registers at the start of the step and
  // written to its buffer as fp16 at the end (no staging copy in LDS).
  u32x4 vr[TileCopy<T, D, kBc, kWaves>::CPW];
  auto copy_kv = [&](char* sK, char* sV, int k0) {
    tc.issue(Kh, N, k0, sK);
    if constexpr (kConv) tc.load(Vh, N, k0, vr);
    else tc.issue(Vh, N, k0, sV);
  };
  auto finish_v = [&](char* sV) {
    if constexpr (kConv) tc.store_f16(vr, sV);
  };
  copy_kv(sK0, sV0, 0);
  wait_loads();  // the Q rows, V's registers and the copies
  finish_v(sV0);
  __syncthreads();

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  // Dropout: the random bytes of this lane's row; byte i % 4 of word
  // [kb][i / 4] belongs to the score in register i of key block kb (key
  // k0 + 32 kb + 8 (i / 4) + 4 hf + i % 4, query myq).  The four lanes of
  // rows 4a..4a+3 share each generator block: one draw per lane and key block.
  auto keep_words = [&](int k0, u32x4 (&dw)[2]) {
    const int r = lane & 3;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t cr = (uint32_t)(k0 + 32 * kb + 8 * r + 4 * hf) >> 2;
      dw[kb] = keep_words_rows_quad(a.drop, cr, (uint32_t)myq >> 2, (uint32_t)bh, r);
    }
  };

  // One K/V tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASK selects
  // the general form (causal diagonal, ragged tail, waves with nothing to do);
  // tiles that are full for the whole workgroup take the mask-free form.
  auto tile = [&](const char* sK, const char* sV, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK && CAUSAL && k0 > q0w + 31) return;  // every key of the tile is after every query of the wave
    // Dropout keep bits, drawn before the products so that the generator's
    // integer work can issue between them.
    u32x4 dw[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if constexpr (DROP) keep_words(k0, dw);
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
    if (MASK) {
      // key > myq (causal) or key >= N: with lim = myq - k0 - 4 hf (resp. N - 1 - k0 - 4 hf)
      // the test is a compare of lim with a per-register constant.
      const int lim = (CAUSAL ? myq : N - 1) - k0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
    // Running max: moved only when a tile raises it by more than kSlack.
    auto raise_max = [&]() {
      float mt = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(fmaxf(s[0][i], s[1][i]), mt);
      mt = fmaxf(mt, other_half(mt)) * a.c;
      if (__ballot(mt > m + kSlack)) {
        const float mnew = fmaxf(m, mt);
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      }
    };
    PF pfs[kBc / 16];
    if constexpr (kConv) {
      // p against the running max, packed to fp16; returns this lane's share
      // of the tile's row sum, added from the fp16 values that the product
      // uses, two per instruction (fp32 accumulation).
      const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
      auto probs = [&]() {
        f32x16 ps[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) ps[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -m));
        float ts = 0.f;
#pragma unroll
        for (int t = 0; t < kBc / 16; ++t) {
          frag_from(pfs[t], ps[t >> 1], (t & 1) * 8);
          const PF& v = pfs[t];
          ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), ones, ts, false);
          ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), ones, ts, false);
          ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), ones, ts, false);
          ts = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), ones, ts, false);
        }
        return ts;
      };
      // After the first tile the running max is finite for every row, and a
      // tile rarely raises it by much: try it unchanged, and take the tile max
      // only when some p would exceed kPLimit (an overflow gives inf, which
      // fails the test too).
      float ts = 0.f;
      bool ok = false;
      if (k0 != 0) {
        ts = probs();
        ok = !__ballot(!(ts <= kPLimit));
      }
      if (!ok) {
        raise_max();
        ts = probs();
      }
      lsum += ts;
      if constexpr (DROP) {
        // The row sum keeps every p; the product sees the kept ones.
#pragma unroll
        for (int t = 0; t < kBc / 16; ++t)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = 8 * (t & 1) + u;  // register i of key block t / 2
            if (!byte_kept(dw[t >> 1][i >> 2], i & 3, a.drop.t)) pfs[t][u] = (_Float16)0.f;
          }
      }
    } else {
      raise_max();
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -m));
          s[kb][i] = p;
          ps[i & 3] += p;
        }
      lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      if constexpr (DROP) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!byte_kept(dw[kb][i >> 2], i & 3, a.drop.t)) s[kb][i] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < kBc / 16; ++t) frag_from(pfs[t], s[t >> 1], (t & 1) * 8);
    }
    // O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int t = 0; t < kBc / 16; ++t) {
      const PF& pf = pfs[t];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        PF vf;
        cf.read(vf, sV, t, db);
        acc[db] = mfma_k16(vf, pf, acc[db]);
      }
    }
  };
  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Any;

  // Tiles [0, jfull) are unmasked for every query of the workgroup.
  const int jfull = min(nt, CAUSAL ? (qt * kBr) / kBc : N / kBc);
  // Two tiles per iteration so that each buffer is a distinct LDS object;
  // tile j+1 is copied while tile j is consumed.
  auto step = [&](int j, char* sKc, char* sVc, char* sKn, char* sVn, auto mask_tag) {
    if (j + 1 < nt) copy_kv(sKn, sVn, (j + 1) * kBc);
    tile(sKc, sVc, j * kBc, mask_tag);
    wait_copies();
    if (j + 1 < nt) finish_v(sVn);
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < jfull; j += 2) {
    step(j, sK0, sV0, sK1, sV1, Full());
    step(j + 1, sK1, sV1, sK0, sV0, Full());
  }
  for (; j < nt; j += 2) {
    if (j < jfull) step(j, sK0, sV0, sK1, sV1, Full());
    else step(j, sK0, sV0, sK1, sV1, Any());
    if (j + 1 >= nt) break;
    step(j + 1, sK1, sV1, sK0, sV0, Any());
  }

  lsum += other_half(lsum);
  const float os = (DROP ? a.drop.inv : 1.f) / lsum;
  if constexpr (kConv) {
    // The tiles are free after the last step's barrier: wave w stages its rows
    // in 32 rows of tile w / 2.
    const int t2 = __builtin_amdgcn_readfirstlane(w) >> 1;
    char* const stage = t2 == 0 ? sK0 : t2 == 1 ? sK1 : t2 == 2 ? sV0 : sV1;
    store_rows_lds<D, true>(reinterpret_cast<bf16*>(a.o) + (size_t)bh * slab, q0w, N, acc, os,
                      stage + (w & 1) * 32 * L::RB);
  } else {
    store_rows<T, D>(reinterpret_cast<T*>(a.o) + (size_t)bh * slab, myq, N, acc, os);
  }
  if (hf == 0 && myq < N) a.lse[(size_t)bh * N + myq] = (m + __log2f(lsum)) * kLn2;
}

// With dropout the generator's registers come on top of the tile's: those
// variants ask for one workgroup per CU only (the second bound).  At d = 64
// (four waves) that is one wave per SIMD, so the compiler may use up to 512
// registers; at d = 128 the eight waves of a workgroup are two per SIMD, and
// 256 stays the limit.
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64 * waves_bf16<D>(), DROP ? 1 : wgs_bf16<D>()) void fa_fwd_kernel_bf16(FwdArgs a) {
  fwd_body<bf16, D, CAUSAL, waves_bf16<D>(), DROP>(a);
}
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64 * kWavesF32, 1) void fa_fwd_kernel_f32(FwdArgs a) {
  fwd_body<float, D, CAUSAL, kWavesF32, DROP>(a);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N;
  constexpr int waves = sizeof(T) == 2 ? waves_bf16<D>() : kWavesF32;
  a.nqt = (p.N + 32 * waves - 1) / (32 * waves);
  a.c = p.scale * kLog2e;
  a.drop = DropArgs{p.drop.k0, p.drop.k1, p.drop.offset, p.drop.t, p.drop.inv};
  const dim3 grid((unsigned)((long)a.nqt * p.B * p.H));
  if constexpr (sizeof(T) == 2) {
    if (p.drop.on) hipLaunchKernelGGL((fa_fwd_kernel_bf16<D, CAUSAL, true>), grid, dim3(64 * waves), 0, stream, a);
    else hipLaunchKernelGGL((fa_fwd_kernel_bf16<D, CAUSAL, false>), grid, dim3(64 * waves), 0, stream, a);
  } else {
    if (p.drop.on) hipLaunchKernelGGL((fa_fwd_kernel_f32<D, CAUSAL, true>), grid, dim3(64 * waves), 0, stream, a);
    else hipLaunchKernelGGL((fa_fwd_kernel_f32<D, CAUSAL, false>), grid, dim3(64 * waves), 0, stream, a);
  }
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
