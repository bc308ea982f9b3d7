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
//  1. fa_bwd_pre:  -D = -rowsum(dO * O) and lse * log2(e), one float each
//     per query row, into the workspace (dP - D is then an addition, or the
//     start value of a dP accumulator).  The dQ kernel (3) computes the same
//     two values for its own rows, with the same summation order (so the same
//     bits), and writes them too: fa_bwd runs dQ first and dK/dV second, and
//     needs no separate preprocessing launch;
//  2. fa_bwd_dkdv: one workgroup per (batch, KV head, key tile[, slice of
//     the GQA group]); K/V fragments and the dK/dV accumulators stay in
//     registers while Q/dO tiles stream through LDS (global -> LDS copies),
//     for every query head of the group and, under the causal mask, only from
//     the diagonal on.  bf16 uses 256-key tiles and pairs of waves that split
//     the step between them (2b below); float32 uses 128-key tiles, one wave
//     per 32 keys (2a).  No atomics: each key row is owned by one lane.  When
//     a GQA group is sliced over several workgroups (to balance the work of
//     very wide groups), each writes float32 partial sums and fa_bwd_reduce
//     adds them in a fixed order;
//  3. fa_bwd_dq:   one workgroup per (batch, head, query tile: 256 rows for
//     bf16 at d = 128, 128 for bf16 at d = 64 and for fp32); Q/dO fragments and the dQ accumulator stay in registers while
//     K/V tiles of 64 keys stream through LDS.  It recomputes S and dP instead of exchanging
//     dS with the dK/dV kernel: seven products in total instead of five, but
//     no float atomics, whose L2 throughput on this part is far below what a
//     shared dQ accumulator would need.
#include "fa_device.h"
#include "fa_kernels.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dO;
  const void* o; const float* lse;
  float* delta; float* lse2;
  void* dq; void* dk; void* dv;
  float* part;
  int B, H, Hkv, N, nsplit;
  float c;      // scale * log2(e)
  float scale;
  DropArgs drop;
};

BwdArgs make_args(const BwdParams& p) {
  BwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.dO = p.dO;
  a.o = p.o; a.lse = p.lse;
  a.delta = p.delta; a.lse2 = p.lse2;
  a.dq = p.dq; a.dk = p.dk; a.dv = p.dv; a.part = p.part;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N; a.nsplit = p.nsplit;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  a.drop = DropArgs{p.drop.k0, p.drop.k1, p.drop.offset, p.drop.t, p.drop.inv};
  return a;
}

// ------------------------------------------------------------------ 1. preprocess
// D_i = sum_c dO_ic O_ic in one fixed order, shared with the dQ kernel so
// that both give the same bits.  Row i is cut into chunks of 8 columns,
// chunk c = 2 s + hf holding columns 8 c .. 8 c + 7 (the columns a lane holds
// as its k16 fragment s in lane half hf).  Each chunk is summed with fused
// multiply-adds in column order; the chunks of one half (fixed hf) are added
// as a pairwise tree over s (s with s ^ 1, then ^ 2, then ^ 4); the two halves
// are added last.
template <typename T>
__device__ __forceinline__ float chunk_dot(const typename Frag<T>::type& o, const typename Frag<T>::type& g) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  return acc;
}
// Pairwise tree over the KS chunk sums of one half, in the order above.
template <int KS>
__device__ __forceinline__ float chunk_tree(float (&c)[KS]) {
#pragma unroll
  for (int m = 1; m < KS; m <<= 1)
#pragma unroll
    for (int i = 0; i < KS; i += 2 * m) c[i] = c[i] + c[i + m];
  return c[0];
}

// D/8 threads per row, one chunk each (coalesced 16-byte loads for bf16).
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                         const float* __restrict__ lse, float* __restrict__ delta,
                                                         float* __restrict__ lse2, long rows) {
  typedef typename Frag<T>::type F;
  constexpr int CPR = D / 8;  // chunks per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / CPR;
  const int c = (int)(t % CPR);
  float v = 0.f;
  if (row < rows) {
    const rsrc_t rO = make_rsrc(O + row * D, (uint32_t)(D * sizeof(T)));
    const rsrc_t rG = make_rsrc(dO + row * D, (uint32_t)(D * sizeof(T)));
    F o, g;
    frag_global<D>(o, rO, 0, 8 * c);
    frag_global<D>(g, rG, 0, 8 * c);
    v = chunk_dot<T>(o, g);
  }
  // chunk c = 2 s + hf: the tree over s pairs lanes c ^ 2, c ^ 4, c ^ 8; then the halves (c ^ 1).
#pragma unroll
  for (int m = 2; m < CPR; m <<= 1) v = v + __shfl_xor(v, m, CPR);
  v = v + __shfl_xor(v, 1, CPR);
  if (row < rows && c == 0) {
    delta[row] = -v;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ 2a. dK / dV, float32
constexpr int kKeys = kDkdvKeysF32;    // keys per workgroup (32 per wave)
constexpr int kQRows = kDkdvQRowsF32;  // query rows per step
static_assert(kKeys == 32 * kWaves, "one 32-key column block per wave");

template <typename T, int D, bool CAUSAL, bool DROP>
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
    wait_loads();
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int nqt = (N + kQRows - 1) / kQRows;
  const int qstart = CAUSAL ? k0 / kQRows : 0;
  const int nq = nqt - qstart;
  const int total = gs * nq;

  RowFrags<T, D> rf;
  ColFrags<T, D> cf;
  TileCopy<T, D, kQRows, kWaves> tc;
  rf.init();
  cf.init();
  tc.init(w);

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
    tc.issue(reinterpret_cast<const T*>(a.q) + head * slab, N, qb0, bq);
    tc.issue(reinterpret_cast<const T*>(a.dO) + head * slab, N, qb0, bo);
    if (w == 0) vec_to_lds<64>(buffer_desc(a.lse2 + head * N, (uint32_t)N * 4u), bl, qb0);
    if (w == 1) vec_to_lds<64>(buffer_desc(a.delta + head * N, (uint32_t)N * 4u), bd, qb0);
  };
  // Steps that touch the causal diagonal or the ragged end of the sequence.
  auto masked = [&](int it) {
    const int qi = it % nq;
    return (CAUSAL && qi < kKeys / kQRows) || (qstart + qi + 1) * kQRows > N;
  };

  // One step: S = Q K^T, dP = dO V^T, P and dS, then dV^T += dO^T P and
  // dK^T += Q^T dS, in two 32-row halves (mb) so that the vector work of one
  // half runs between the matrix products of the other:
  //   products S/dP(0), S/dP(1) | softmax(0) ; products dV/dK(0) | softmax(1) ;
  //   products dV/dK(1).
  // MASK selects the general form; other steps take the mask-free form.
  auto step = [&](const char* sQ, const char* sO, const float* sL, const float* sD, int it, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int qb0 = (qstart + it % nq) * kQRows;
    if (MASK && CAUSAL && qb0 + kQRows - 1 < kw) return;  // every query of the step is before every key of the wave
    const uint32_t bhq = (uint32_t)(b * a.H + h0 + it / nq);
    f32x16 s[MB], dp[MB];
    auto sdp = [&](int mb) {
      s[mb] = f32x16{};
      dp[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        F qa, oa;
        rf.read(qa, sQ, mb, ks);
        rf.read(oa, sO, mb, ks);
        s[mb] = mfma_k16(qa, kf[ks], s[mb]);
        dp[mb] = mfma_k16(oa, vf[ks], dp[mb]);
      }
    };
    // Masked when key > q (causal) or q >= N: q - key = ql - lim.
    const int lim = mykey - qb0 - 4 * hf;
    const int qlim = N - 1 - qb0 - 4 * hf;
    auto softmax = [&](int mb) {
      // Dropout: byte e of word g4 for query qb0 + 32 mb + 8 g4 + 4 hf + e and
      // this lane's key (the lanes of keys 4c..4c+3 share each generator block).
      u32x4 dw = u32x4{0u, 0u, 0u, 0u};
      if constexpr (DROP) {
        const int r = lane & 3;  // == mykey % 4
        dw = keep_words_cols_quad(a.drop, (uint32_t)mykey >> 2, (uint32_t)(qb0 + mb * 32 + 8 * r + 4 * hf) >> 2,
                                  bhq, r);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql0 = mb * 32 + 8 * g4 + 4 * hf;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + ql0);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(sD + ql0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          float p = fast_exp2(__builtin_fmaf(s[mb][i], a.c, -lv[e]));
          if (MASK) {
            const int c = mb * 32 + 8 * g4 + e;  // ql - 4 hf
            if ((CAUSAL && c < lim) || c > qlim) p = 0.f;
          }
          if constexpr (DROP) {
            const bool keep = byte_kept(dw[g4], e, a.drop.t);
            s[mb][i] = keep ? p : 0.f;
            dp[mb][i] = p * __builtin_fmaf(dp[mb][i], keep ? a.drop.inv : 0.f, dd[e]);
          } else {
            s[mb][i] = p;
            dp[mb][i] = p * (dp[mb][i] + dd[e]);
          }
        }
      }
    };
    // dV^T += dO^T P and dK^T += Q^T dS for the 32 query rows of half mb.
    auto dvdk = [&](int mb) {
#pragma unroll
      for (int t = 2 * mb; t < 2 * mb + 2; ++t) {
        F pf, dsf;
        frag_from(pf, s[t >> 1], (t & 1) * 8);
        frag_from(dsf, dp[t >> 1], (t & 1) * 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          F oa, qa;
          cf.read(oa, sO, t, db);
          dv[db] = mfma_k16(oa, pf, dv[db]);
          cf.read(qa, sQ, t, db);
          dk[db] = mfma_k16(qa, dsf, dk[db]);
        }
      }
    };
    static_assert(MB == 2, "two query halves per step");
    sdp(0);
    sdp(1);
    softmax(0);
    dvdk(0);
    softmax(1);
    dvdk(1);
  };

  // The mask-free step, software-pipelined by hand: LDS reads are issued two
  // slots ahead of their products, and each slot pairs two matrix products
  // with a share of the softmax of the half whose scores are already done.
  // sched_barrier(0) closes every slot, so the compiler keeps this order.
  //   phase 1: S/dP of both halves; softmax(0) in the last slots
  //   phase 2: dV/dK of half 0; softmax(1)
  //   phase 3: dV/dK of half 1
  auto step_full = [&](const char* sQ, const char* sO, const float* sL, const float* sD) {
    constexpr int NX = MB * KS;      // slots of phase 1
    constexpr int NY = 2 * MB * DB;  // slots of phases 2 and 3
    constexpr int AH = 2;            // read-ahead in slots
    f32x16 s[MB], dp[MB];
    F qa[NX], oa[NX], oT[NY], qT[NY];
    f32x4 lv[MB][4], dd[MB][4];
    auto rd = [&](int x) {
      rf.read(qa[x], sQ, x / KS, x % KS);
      rf.read(oa[x], sO, x / KS, x % KS);
    };
    auto rdT = [&](int y) {
      cf.read(oT[y], sO, y / DB, y % DB);
      cf.read(qT[y], sQ, y / DB, y % DB);
    };
    auto sm = [&](int mb, int i) {
      const float p = fast_exp2(__builtin_fmaf(s[mb][i], a.c, -lv[mb][i >> 2][i & 3]));
      s[mb][i] = p;
      dp[mb][i] = p * (dp[mb][i] + dd[mb][i >> 2][i & 3]);
    };
    F pf[2 * MB], dsf[2 * MB];
    auto cvt = [&](int t) {
      frag_from(pf[t], s[t >> 1], (t & 1) * 8);
      frag_from(dsf[t], dp[t >> 1], (t & 1) * 8);
    };
#pragma unroll
    for (int x = 0; x < AH; ++x) rd(x);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        lv[mb][g4] = *reinterpret_cast<const f32x4*>(sL + mb * 32 + 8 * g4 + 4 * hf);
        dd[mb][g4] = *reinterpret_cast<const f32x4*>(sD + mb * 32 + 8 * g4 + 4 * hf);
      }
    __builtin_amdgcn_sched_barrier(0);
    // phase 1
    constexpr int S0 = KS + 2;  // first slot with softmax(0) work
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (x + AH < NX) rd(x + AH);
      const int mb = x / KS, ks = x % KS;
      s[mb] = mfma_k16(qa[x], kf[ks], ks == 0 ? f32x16{} : s[mb]);
      dp[mb] = mfma_k16(oa[x], vf[ks], ks == 0 ? f32x16{} : dp[mb]);
      if (x >= S0) {
#pragma unroll
        for (int i = (x - S0) * 16 / (NX - S0); i < (x - S0 + 1) * 16 / (NX - S0); ++i) sm(0, i);
      }
      if (x == NX - 1) { cvt(0); cvt(1); }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phases 2 and 3
#pragma unroll
    for (int y = 0; y < AH; ++y) rdT(y);
    constexpr int NY2 = NY / 2;  // slots of phase 2
#pragma unroll
    for (int y = 0; y < NY; ++y) {
      if (y + AH < NY) rdT(y + AH);
      const int t = y / DB, db = y % DB;
      dv[db] = mfma_k16(oT[y], pf[t], dv[db]);
      dk[db] = mfma_k16(qT[y], dsf[t], dk[db]);
      if (y >= 1 && y < NY2) {
#pragma unroll
        for (int i = (y - 1) * 16 / (NY2 - 1); i < y * 16 / (NY2 - 1); ++i) sm(1, i);
      }
      if (y == NY2 - 1) { cvt(2); cvt(3); }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Any;
  auto run = [&](const char* sQ, const char* sO, const float* sL, const float* sD, int it) {
    if (masked(it)) step(sQ, sO, sL, sD, it, Any());
    else if constexpr (DROP) step(sQ, sO, sL, sD, it, Full());
    else step_full(sQ, sO, sL, sD);
  };

  if (total > 0) fetch(0, sQ0, sO0, sL0, sD0);
  wait_copies();
  __syncthreads();
  for (int it = 0; it < total; it += 2) {
    if (it + 1 < total) fetch(it + 1, sQ1, sO1, sL1, sD1);
    run(sQ0, sO0, sL0, sD0, it);
    wait_copies();
    __syncthreads();
    if (it + 1 >= total) break;
    if (it + 2 < total) fetch(it + 2, sQ0, sO0, sL0, sD0);
    run(sQ1, sO1, sL1, sD1, it + 1);
    wait_copies();
    __syncthreads();
  }

  if (a.nsplit == 1) {
    store_rows<T, D>(reinterpret_cast<T*>(a.dk) + (size_t)bkv * slab, mykey, N, dk, a.scale);
    store_rows<T, D>(reinterpret_cast<T*>(a.dv) + (size_t)bkv * slab, mykey, N, dv, DROP ? a.drop.inv : 1.f);
  } else {
    const size_t ps = (size_t)a.B * a.Hkv * slab;  // elements of one partial tensor
    store_rows<float, D>(a.part + (2 * sp) * ps + (size_t)bkv * slab, mykey, N, dk, a.scale);
    store_rows<float, D>(a.part + (2 * sp + 1) * ps + (size_t)bkv * slab, mykey, N, dv, DROP ? a.drop.inv : 1.f);
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dkdv_kernel_f32(BwdArgs a) {
  dkdv_body<float, D, CAUSAL, DROP>(a);
}

// ------------------------------------------------------------------ 2b. dK / dV, bf16: wave pairs
// Eight waves and 256 keys per workgroup; the four wave pairs own 64 keys
// each.  In a pair, the P wave holds the pair's K rows and computes S = Q K^T,
// P and dV^T += dO^T P; the dS wave holds its V rows and computes dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^T dS, with P passed through LDS (in fp16).
// Waves w and w + 4 share a SIMD, so the exponentials of one overlap the
// products of the other, and owning 64 keys per wave lets every Q or dO
// fragment read from LDS feed two products (half the LDS traffic per product
// of one 32-key block per wave).  One barrier per step: while the P wave
// handles step i, the dS wave forms dP and dS of step i - 1 and adds the dK
// of step i - 2 (its dS kept in registers), and the copies of step i + 1
// land; the Q, dO, lse and D tiles rotate over four buffers and P over two.
// K/V fragments (64 registers) and the accumulators (128) of a wave fill most
// of its 256 registers at d = 128; the P-wave loop is split into dead,
// diagonal and mask-free parts so that no step carries a branch.
constexpr int kPairWaves = 8;
constexpr int kPairThreads = 64 * kPairWaves;
constexpr int kPairKeys = kDkdvKeysBf16;
constexpr int kPairRows = kDkdvQRowsBf16;
static_assert(kPairKeys == 64 * (kPairWaves / 2) && kPairRows == 32, "64 keys per pair, 32-row steps");
constexpr int kPairAhead = 2;  // fragment reads in flight ahead of their products

template <int D, bool CAUSAL, bool DROP>
__device__ __forceinline__ void dkdv_pair_body(const BwdArgs& a) {
  typedef bf16x8 F;
  typedef Lay<bf16, D> L;
  constexpr int TQ = kPairRows * L::RB;  // bytes of one 32-row tile
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int NCW = TQ / 1024 < kPairWaves ? TQ / 1024 : kPairWaves;  // waves that issue tile copies
  constexpr int PB = 2 * 2 * 1024;  // P of one pair and step: 2 key blocks x 2 row groups x 1 KB
  __shared__ __attribute__((aligned(1024))) char sQ[4][TQ], sO[4][TQ], sP[2][kPairWaves / 2][PB];
  __shared__ __attribute__((aligned(256))) float sL[4][kPairRows], sD[4][kPairRows];
  // Dropout: the P wave's random bytes of a step (per key block and lane, as
  // drawn: 16 queries x this lane's key), handed to the dS wave beside P.
  __shared__ __attribute__((aligned(256))) u32x4 sM[2][kPairWaves / 2][2][DROP ? 64 : 1];

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int pr = w & 3;  // pair
  const int N = a.N;
  const int g = a.H / a.Hkv, gs = g / a.nsplit;
  int unit, kt;
  xcd_map(blockIdx.x, a.B * a.Hkv * a.nsplit, unit, kt);  // lowest key tiles (most work) first
  const int bkv = unit / a.nsplit, sp = unit % a.nsplit;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const int h0 = kvh * g + sp * gs;  // first query head of this slice
  const size_t slab = (size_t)N * D;
  const int k0 = kt * kPairKeys;
  const int kp = k0 + 64 * pr;  // first key of the pair

  TileCopy<bf16, D, kPairRows, NCW> tc;
  if (w < NCW) tc.init(w);

  const int nqt = (N + kPairRows - 1) / kPairRows;
  const int qstart = CAUSAL ? k0 / kPairRows : 0;
  const int nq = nqt - qstart;
  const int total = gs * nq;
  auto qbase = [&](int it) { return (qstart + it % nq) * kPairRows; };
  // Per query head, steps [0, ndead) have every query before every key of
  // the pair (query tile qi ends at k0 + 32 qi + 31) and steps [ndead, lo)
  // touch the causal diagonal of the workgroup.
  const int ndead = CAUSAL ? min(nq, 2 * pr) : 0;
  const int lo = CAUSAL ? min(nq, kPairKeys / kPairRows) : 0;

  auto fetch = [&](int it, int buf) {
    const int hq = h0 + it / nq;
    const int qb0 = qbase(it);
    const size_t head = (size_t)b * a.H + hq;
    if (w < NCW) {
      tc.issue(reinterpret_cast<const bf16*>(a.q) + head * slab, N, qb0, sQ[buf]);
      tc.issue(reinterpret_cast<const bf16*>(a.dO) + head * slab, N, qb0, sO[buf]);
    }
    if (w == kPairWaves - 2) vec_to_lds<kPairRows>(buffer_desc(a.lse2 + head * N, (uint32_t)N * 4u), sL[buf], qb0);
    if (w == kPairWaves - 1) vec_to_lds<kPairRows>(buffer_desc(a.delta + head * N, (uint32_t)N * 4u), sD[buf], qb0);
  };

  // This wave's 64 keys of K (P wave) or V (dS wave) as B fragments; they
  // land while the first tiles are copied.
  F kv[2][KS];
  {
    const bf16* src = reinterpret_cast<const bf16*>(w < 4 ? a.k : a.v) + (size_t)bkv * slab;
    const rsrc_t r = make_rsrc(src, (uint32_t)(slab * sizeof(bf16)));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < KS; ++s) frag_global<D>(kv[kb][s], r, kp + 32 * kb + l32, 16 * s + 8 * hf);
  }
  // dV^T (P wave) or dK^T (dS wave) of the pair's two 32-key blocks.
  f32x16 acc[2][DB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[kb][i] = f32x16{};

  // The dS wave's first dK multiplies a zero dS with buffer 3; keep it finite.
  lds_zero<kPairThreads>(sQ[3], TQ);
  if (total > 0) fetch(0, 0);
  wait_loads();  // the K or V rows and the copies
  __syncthreads();

  constexpr int R = kPairAhead + 1;
  // Per-lane fragment addressing.  A row fragment (ks) of a 32-row tile sits
  // at rbase + ((32 ks) ^ rx); a column fragment (t, db) reads its two 4-row
  // groups at cbase[b] + 16 t RB + ((64 db) ^ cx), b = 0, 1.  The lane terms
  // are re-derived every step (the empty asm hides their loop invariance), so
  // that the compiler does not keep one offset register per fragment alive.
  const int rbase0 = l32 * L::RB;
  const int rx0 = (hf ^ L::sw(l32)) << 4;
  const int e4 = (lane & 15) >> 2, gl = ((lane & 16) >> 3) + ((lane & 3) >> 1);
  int cb0[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int row = 4 * hf + e4 + 8 * bb;
    cb0[bb] = row * L::RB + ((gl ^ (L::sw(row) & 3)) << 4) + (lane & 1) * 8;
  }
  const int cx0 = (D == 128 ? e4 : ((e4 >> 1) & 1)) << 6;
  // Row-fragment product of a 32-row tile with both key blocks:
  // out[kb] += tile(rows 0..31, all of d) * kv[kb]^T.
  auto rows_x_kv = [&](f32x16 (&out)[2], const char* tile, const f32x16& init) {
    int rx = rx0;
    asm volatile("" : "+v"(rx));
    const char* rt = tile + rbase0;
    auto rd = [&](F& f, int ks) { f = *reinterpret_cast<const F*>(rt + ((32 * ks) ^ rx)); };
    F fa_[R];
#pragma unroll
    for (int x = 0; x < kPairAhead; ++x) rd(fa_[x], x);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + kPairAhead < KS) rd(fa_[(ks + kPairAhead) % R], ks + kPairAhead);
      // The first product of each chain takes `init` as its addend, so the
      // start value needs no copy into the accumulators.
      out[0] = mfma_k16(fa_[ks % R], kv[0][ks], ks == 0 ? init : out[0]);
      out[1] = mfma_k16(fa_[ks % R], kv[1][ks], ks == 0 ? init : out[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc[kb]^T += tile^T * frag[kb]: column fragments of a 32-row tile times
  // the B fragments of both key blocks (16 rows per k-step).
  auto cols_x_frag = [&](const char* tile, const F (&fr)[2][2]) {
    constexpr int NY = 2 * DB;
    int cx = cx0;
    asm volatile("" : "+v"(cx));
    const char* c0 = tile + cb0[0];
    const char* c1 = tile + cb0[1];
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto rd = [&](F& f, int y) {
      const int t = y / DB, db = y % DB;
      const int o = 16 * t * L::RB + ((64 * db) ^ cx);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(c0 + o));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(c1 + o));
      f = __builtin_bit_cast(F, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    F ct[R];
#pragma unroll
    for (int y = 0; y < kPairAhead; ++y) rd(ct[y], y);
#pragma unroll
    for (int y = 0; y < NY; ++y) {
      if (y + kPairAhead < NY) rd(ct[(y + kPairAhead) % R], y + kPairAhead);
      const int t = y / DB, db = y % DB;
      acc[0][db] = mfma_k16(ct[y % R], fr[0][t], acc[0][db]);
      acc[1][db] = mfma_k16(ct[y % R], fr[1][t], acc[1][db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Dropout random bytes of one 32-key block kb of the pair at step `step`
  // (query rows qb0..qb0+31): byte i % 4 of word i / 4 for register i, i.e.
  // query qb0 + 8 (i / 4) + 4 hf + i % 4 and key kp + 32 kb + l32.  The P wave
  // draws them (the lanes of keys 4c..4c+3 share each generator block) and
  // hands them on in sM.
  auto pair_keep_words = [&](int kb, int qb0, int step) {
    const int key = kp + 32 * kb + l32;
    const int r = lane & 3;  // == key % 4
    const uint32_t bhq = (uint32_t)(b * a.H + h0 + step / nq);
    return keep_words_cols_quad(a.drop, (uint32_t)key >> 2, (uint32_t)(qb0 + 8 * r + 4 * hf) >> 2, bhq, r);
  };

  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Any;
  if (w < 4) {
    const float nic = -1.f / a.c;
    // ---- P wave: S = Q K^T, P = exp2(S c - lse2), P -> LDS, dV^T += dO^T P.
    // The two key blocks are staggered so that the exponentials of one run
    // between the products of the other:
    //   S0 | S1 + exp(S0) | dV0 + exp(S1) | dV1
    // (Q and dO^T fragments are read once per key block.)
    auto step = [&](int it, const char* tq, const char* to, const float* tl, char* tp, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int qb0 = qbase(it);
      // The accumulators start at -lse2 / c, so that S c - lse2 is one multiply.
      f32x16 s0, s1, si;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(tl + 8 * g4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) si[4 * g4 + e] = lv[e] * nic;
      }
      // Masked when key > q, i.e. when q - qb0 - 4 hf < key - qb0 - 4 hf.
      const int lim0 = kp + l32 - qb0 - 4 * hf, lim1 = lim0 + 32;
      auto pexp = [&](f32x16& sv, int i, int lim) {
        float p = fast_exp2(sv[i] * a.c);
        if (MASK && 8 * (i >> 2) + (i & 3) < lim) p = 0.f;
        sv[i] = p;
      };
      auto emit = [&](f32x16& sv, F (&pf)[2], int kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f16x8 ph;  // P goes to the dS wave in fp16 (P is in [0, 1]; 11-bit significand)
          frag_from(ph, sv, 8 * t);
          *reinterpret_cast<f16x8*>(tp + (2 * kb + t) * 1024 + lane * 16) = ph;
        }
        // Dropout: dV takes the kept p; the random bytes go to the dS wave too.
        if constexpr (DROP) {
          const u32x4 dw = pair_keep_words(kb, qb0, it);
          sM[it & 1][pr][kb][lane] = dw;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!byte_kept(dw[i >> 2], i & 3, a.drop.t)) sv[i] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) frag_from(pf[t], sv, 8 * t);
      };
      int rx = rx0;
      asm volatile("" : "+v"(rx));
      const char* rt = tq + rbase0;
      auto rdq = [&](F& f, int ks) { f = *reinterpret_cast<const F*>(rt + ((32 * ks) ^ rx)); };
      int cx = cx0;
      asm volatile("" : "+v"(cx));
      const char* c0 = to + cb0[0];
      const char* c1 = to + cb0[1];
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      auto rdo = [&](F& f, int y) {
        const int t = y / DB, db = y % DB;
        const int o = 16 * t * L::RB + ((64 * db) ^ cx);
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(c0 + o));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(c1 + o));
        f = __builtin_bit_cast(F, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int NY = 2 * DB;
      constexpr int EPS = 16 / KS, EPY = 16 / NY;  // exponentials per slot
      F fr[2];
      // S0
      __builtin_amdgcn_s_setprio(1);
      rdq(fr[0], 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        rdq(fr[(ks + 1) & 1], (ks + 1) % KS);  // the last read starts S1
        s0 = mfma_k16(fr[ks & 1], kv[0][ks], ks == 0 ? si : s0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // S1, exp(S0)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) rdq(fr[(KS + ks + 1) & 1], ks + 1);
        s1 = mfma_k16(fr[(KS + ks) & 1], kv[1][ks], ks == 0 ? si : s1);
#pragma unroll
        for (int e = 0; e < EPS; ++e) pexp(s0, EPS * ks + e, lim0);
        __builtin_amdgcn_sched_barrier(0);
      }
      F pf0[2], pf1[2];
      emit(s0, pf0, 0);
      // dV0, exp(S1)
      rdo(fr[0], 0);
#pragma unroll
      for (int y = 0; y < NY; ++y) {
        rdo(fr[(y + 1) & 1], (y + 1) % NY);  // the last read starts dV1
        acc[0][y % DB] = mfma_k16(fr[y & 1], pf0[y / DB], acc[0][y % DB]);
#pragma unroll
        for (int e = 0; e < EPY; ++e) pexp(s1, EPY * y + e, lim1);
        __builtin_amdgcn_sched_barrier(0);
      }
      emit(s1, pf1, 1);
      // dV1
#pragma unroll
      for (int y = 0; y < NY; ++y) {
        if (y + 1 < NY) rdo(fr[(NY + y + 1) & 1], y + 1);
        acc[1][y % DB] = mfma_k16(fr[(NY + y) & 1], pf1[y / DB], acc[1][y % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    int it = 0;
    // One step; a null mask_tag only copies and synchronises (dead steps).
    auto iter = [&](auto mask_tag) {
      const int qc = it & 3;
      if (it + 1 < total) fetch(it + 1, (it + 1) & 3);
      if constexpr (!std::is_same<decltype(mask_tag), std::nullptr_t>::value) {
        step(it, sQ[qc], sO[qc], sL[qc], sP[it & 1][pr], mask_tag);
      } else {
        // P = 0 for the dS wave, which handles every step alike.
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<u32x4*>(sP[it & 1][pr] + c * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      wait_copies();
      __syncthreads();
      ++it;
    };
    // Per query head: steps entirely above the diagonal for this pair, the
    // other steps on the causal diagonal, then the mask-free ones.  Rows past
    // N need no mask: their dO rows are zero, so they add nothing to dV, and
    // the dS wave's dP and D for them are zero too.
    for (int h = 0; h < gs; ++h) {
      for (int qi = 0; qi < ndead; ++qi) iter(nullptr);
      for (int qi = ndead; qi < lo; ++qi) iter(Any());
      for (int qi = lo; qi < nq; ++qi) iter(Full());
    }
  } else {
    // ---- dS wave, two steps behind the P wave: while the P wave handles
    // step j + 1, dK^T += Q^T dS for step j - 1 (dS kept in registers from
    // the previous interval), then dP = dO V^T - D and dS = P (dP - D) for
    // step j.  The products of this wave thus run while the P wave computes
    // exponentials, and its vector work while the P wave runs products.
    F ds[2][2];
    auto dk = [&](const char* tq) { cols_x_frag(tq, ds); };
    auto dpds = [&](const char* to, const float* td, const char* tp, const u32x4 (*tm)[DROP ? 64 : 1]) {
      f32x16 dp[2], nd;
      // The accumulators start at -D (the workspace holds -D per query row).
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(td + 8 * g4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) nd[4 * g4 + e] = v[e];
      }
      rows_x_kv(dp, to, DROP ? f32x16{} : nd);
      // dS = P * (dP - D) as fma(P, dP - D, z) with an addend z = 0 that the
      // compiler cannot fold away: that form selects v_fma_mix_f32, which
      // reads the fp16 P directly (no separate conversion).
      float z = 0.f;
      asm volatile("" : "+v"(z));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 dw = u32x4{0u, 0u, 0u, 0u};
        if constexpr (DROP) dw = tm[kb][lane];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f16x8 pv = *reinterpret_cast<const f16x8*>(tp + (2 * kb + t) * 1024 + lane * 16);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (DROP) {
              // dS = P (dP keep/(1 - rate) - D)
              const float k = byte_kept(dw[(8 * t + j) >> 2], j & 3, a.drop.t) ? a.drop.inv : 0.f;
              ds[kb][t][j] = (bf16)((float)pv[j] * __builtin_fmaf(dp[kb][8 * t + j], k, nd[8 * t + j]));
            } else {
              ds[kb][t][j] = (bf16)__builtin_fmaf((float)pv[j], dp[kb][8 * t + j], z);
            }
          }
        }
      }
    };
    // Interval 0: copies of step 1 only.
    if (1 < total) fetch(1, 1);
    wait_copies();
    __syncthreads();
    // Every interval runs dK for step j - 1 and dP / dS for step j; steps the
    // pair skips arrive with P = 0 (and so dS = 0), and the first dK adds the
    // zero dS set here.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) ds[kb][t] = F{};
    for (int j = 0; j < total; ++j) {
      if (j + 2 < total) fetch(j + 2, (j + 2) & 3);
      dk(sQ[(j - 1) & 3]);
      dpds(sO[j & 3], sD[j & 3], sP[j & 1][pr], sM[j & 1][pr]);
      if (j + 1 < total) {
        wait_copies();
        __syncthreads();
      }
    }
    dk(sQ[(total - 1) & 3]);
  }

  // Lane l32 of key block kb owns key kp + 32 kb + l32.  The final rows go
  // out through LDS (tile sQ[w] or sO[w - 4], free once every wave is past
  // its last step).
  __syncthreads();
  const int which = w < 4 ? 1 : 0;  // 0: dK, 1: dV
  const float sc = w < 4 ? (DROP ? a.drop.inv : 1.f) : a.scale;
  char* const stage = w < 4 ? sQ[w] : sO[w - 4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kp + 32 * kb + l32;
    if (a.nsplit == 1) {
      bf16* dst = reinterpret_cast<bf16*>(which ? a.dv : a.dk) + (size_t)bkv * slab;
      store_rows_lds<D, true>(dst, kp + 32 * kb, N, acc[kb], sc, stage);
    } else {
      const size_t ps = (size_t)a.B * a.Hkv * slab;  // elements of one partial tensor
      store_rows<float, D>(a.part + (2 * sp + which) * ps + (size_t)bkv * slab, key, N, acc[kb], sc);
    }
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kPairThreads, DROP ? 1 : 2) void fa_bwd_dkdv_kernel_bf16(BwdArgs a) {
  dkdv_pair_body<D, CAUSAL, DROP>(a);
}

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
// Waves (32 query rows each) per dQ workgroup: bf16 at d = 128 eight, two per
// SIMD, so that each K/V tile copy serves 256 query rows; bf16 at d = 64 four,
// with three workgroups per CU (at most 168 registers per wave), so that three
// waves share each SIMD; fp32 kWaves.
template <int D> constexpr int dq_waves_bf16() { return D == 64 ? 4 : 8; }
template <int D> constexpr int dq_wgs_bf16() { return D == 64 ? 3 : 2; }
constexpr int kKTile = 64;           // keys per streamed tile

template <typename T, int D, bool CAUSAL, int NW, bool DROP>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int nqt) {
  constexpr int kQTile = 32 * NW, kThreads = 64 * NW;
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
  const int q0w = qt * kQTile + 32 * w;
  const int myq = q0w + l32;
  F qf[KS], of[KS], ofw[KS];
  float l2, dd, lse;
  {
    // Q, dO and O rows of this lane and its LSE; the row terms are formed
    // once these and the first K/V tile have arrived.
    const rsrc_t rQ = make_rsrc(reinterpret_cast<const T*>(a.q) + (size_t)bh * slab, slab_bytes);
    const rsrc_t rG = make_rsrc(reinterpret_cast<const T*>(a.dO) + (size_t)bh * slab, slab_bytes);
    const rsrc_t rO = make_rsrc(reinterpret_cast<const T*>(a.o) + (size_t)bh * slab, slab_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag_global<D>(qf[s], rQ, myq, 16 * s + 8 * hf);
      frag_global<D>(of[s], rG, myq, 16 * s + 8 * hf);
      frag_global<D>(ofw[s], rO, myq, 16 * s + 8 * hf);
    }
    lse = load4f(make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4u), (uint32_t)myq * 4u);
  }

  const int kend = CAUSAL ? min(N, (qt + 1) * kQTile) : N;
  const int nt = (kend + kKTile - 1) / kKTile;
  const T* Kh = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * slab;
  const T* Vh = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * slab;
  RowFrags<T, D> rf;
  ColFrags<T, D> cf;
  TileCopy<T, D, kKTile, NW> tc;
  rf.init();
  cf.init();
  tc.init(w);

  lds_zero<kThreads>(sK0, TB); lds_zero<kThreads>(sK1, TB);
  lds_zero<kThreads>(sV0, TB); lds_zero<kThreads>(sV1, TB);
  __syncthreads();
  auto copy_kv = [&](char* sK, char* sV, int k0) {
    tc.issue(Kh, N, k0, sK);
    tc.issue(Vh, N, k0, sV);
  };
  copy_kv(sK0, sV0, 0);
  __builtin_amdgcn_sched_barrier(0);  // the row terms after the copies are issued
  wait_loads();  // the row fragments, the LSE and the copies
  {
    // The backward preprocessing of this lane's row (-D and lse * log2 e,
    // also written for the dK/dV kernel): D from the O and dO fragments in the
    // order of fa_bwd_pre_kernel (fragment s of lane half hf is chunk 2 s + hf
    // there).
    float cs[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) cs[s2] = chunk_dot<T>(ofw[s2], of[s2]);
    const float part = chunk_tree<KS>(cs);
    dd = -(part + other_half(part));
    l2 = lse * kLog2e;
    if (hf == 0 && myq < N) {
      a.delta[(size_t)bh * N + myq] = dd;
      a.lse2[(size_t)bh * N + myq] = l2;
    }
  }
  __syncthreads();

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  // One K/V tile: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.  MASK
  // selects the general form (causal diagonal, keys past N, waves with
  // nothing to do); tiles full for the whole workgroup take the mask-free form.
  auto tile = [&](const char* sK, const char* sV, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK && CAUSAL && k0 > q0w + 31) return;
    // key > myq (causal) or key >= N: with lim = myq - k0 - 4 hf (resp. N - 1 - k0 - 4 hf)
    // the test is a compare of lim with a per-register constant.
    const int lim = (CAUSAL ? myq : N - 1) - k0 - 4 * hf;
    // Two 32-key halves, so that only one half's S and dP are live at a time.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // Dropout: byte e of word g for the key k0 + 32 kb + 8 g + 4 hf + e
      // (one generator draw per lane, shared by the lanes of rows 4a..4a+3),
      // drawn before the products so that its integer work can issue between
      // them.
      u32x4 dw = u32x4{0u, 0u, 0u, 0u};
      if constexpr (DROP) {
        const int r = lane & 3;
        dw = keep_words_rows_quad(a.drop, (uint32_t)(k0 + 32 * kb + 8 * r + 4 * hf) >> 2, (uint32_t)myq >> 2,
                                  (uint32_t)bh, r);
      }
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        F kf, vf;
        rf.read(kf, sK, kb, ks);
        rf.read(vf, sV, kb, ks);
        s = mfma_k16(kf, qf[ks], s);
        dp = mfma_k16(vf, of[ks], dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(s[i], a.c, -l2));
        if (MASK && kb * 32 + 8 * (i >> 2) + (i & 3) > lim) p = 0.f;
        if constexpr (DROP) dp[i] = p * __builtin_fmaf(dp[i], byte_kept(dw[i >> 2], i & 3, a.drop.t) ? a.drop.inv : 0.f, dd);
        else dp[i] = p * (dp[i] + dd);
      }
      // dQ^T += K^T dS^T, 16 keys per step.
#pragma unroll
      for (int t = 2 * kb; t < 2 * kb + 2; ++t) {
        F dsf;
        frag_from(dsf, dp, (t & 1) * 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          F kf;
          cf.read(kf, sK, t, db);
          acc[db] = mfma_k16(kf, dsf, acc[db]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the halves apart: bounds register pressure
    }
  };
  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Any;

  // Tiles [0, jfull) are unmasked for every query of the workgroup.
  const int jfull = min(nt, CAUSAL ? (qt * kQTile) / kKTile : N / kKTile);
  auto step = [&](int j, char* sKc, char* sVc, char* sKn, char* sVn, auto mask_tag) {
    if (j + 1 < nt) copy_kv(sKn, sVn, (j + 1) * kKTile);
    tile(sKc, sVc, j * kKTile, mask_tag);
    wait_copies();
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

  if constexpr (sizeof(T) == 2) {
    // The tiles are free after the last step's barrier: wave w stages its rows
    // in 32 rows of tile w / 2.
    const int t2 = __builtin_amdgcn_readfirstlane(w) >> 1;
    char* const stage = t2 == 0 ? sK0 : t2 == 1 ? sK1 : t2 == 2 ? sV0 : sV1;
    store_rows_lds<D, true>(reinterpret_cast<bf16*>(a.dq) + (size_t)bh * slab, q0w, N, acc, a.scale,
                      stage + (w & 1) * 32 * L::RB);
  } else {
    store_rows<T, D>(reinterpret_cast<T*>(a.dq) + (size_t)bh * slab, myq, N, acc, a.scale);
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64 * dq_waves_bf16<D>(), DROP ? 1 : dq_wgs_bf16<D>()) void fa_bwd_dq_kernel_bf16(BwdArgs a, int nqt) {
  dq_body<bf16, D, CAUSAL, dq_waves_bf16<D>(), DROP>(a, nqt);
}
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dq_kernel_f32(BwdArgs a, int nqt) {
  dq_body<float, D, CAUSAL, kWaves, DROP>(a, nqt);
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
  constexpr int keys = sizeof(T) == 2 ? kPairKeys : kKeys;
  const int nkt = (p.N + keys - 1) / keys;
  const dim3 grid((unsigned)((long)nkt * p.B * p.Hkv * p.nsplit));
  if constexpr (sizeof(T) == 2) {
    if (p.drop.on) hipLaunchKernelGGL((fa_bwd_dkdv_kernel_bf16<D, CAUSAL, true>), grid, dim3(kPairThreads), 0, stream, a);
    else hipLaunchKernelGGL((fa_bwd_dkdv_kernel_bf16<D, CAUSAL, false>), grid, dim3(kPairThreads), 0, stream, a);
  } else {
    if (p.drop.on) hipLaunchKernelGGL((fa_bwd_dkdv_kernel_f32<D, CAUSAL, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((fa_bwd_dkdv_kernel_f32<D, CAUSAL, false>), grid, dim3(kThreads), 0, stream, a);
  }
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
  const int qtile = 32 * (sizeof(T) == 2 ? dq_waves_bf16<D>() : kWaves);
  const int nqt = (p.N + qtile - 1) / qtile;
  const dim3 grid((unsigned)((long)nqt * p.B * p.H));
  if constexpr (sizeof(T) == 2) {
    if (p.drop.on)
      hipLaunchKernelGGL((fa_bwd_dq_kernel_bf16<D, CAUSAL, true>), grid, dim3(64 * dq_waves_bf16<D>()), 0, stream, a, nqt);
    else
      hipLaunchKernelGGL((fa_bwd_dq_kernel_bf16<D, CAUSAL, false>), grid, dim3(64 * dq_waves_bf16<D>()), 0, stream, a, nqt);
  } else {
    if (p.drop.on) hipLaunchKernelGGL((fa_bwd_dq_kernel_f32<D, CAUSAL, true>), grid, dim3(kThreads), 0, stream, a, nqt);
    else hipLaunchKernelGGL((fa_bwd_dq_kernel_f32<D, CAUSAL, false>), grid, dim3(kThreads), 0, stream, a, nqt);
  }
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
