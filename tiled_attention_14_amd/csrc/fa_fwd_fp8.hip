// fa_fwd_fp8.hip — attention forward on 8-bit float inputs for gfx950.
//
// Q, K and V arrive as OCP e4m3 codes (1 byte each) with one float scale per
// tensor: the value of an element is code * scale.  The method is the forward
// of fa_fwd.hip (tiles, online softmax with a running max and sum, one
// normalisation at the end; "【词汇专栏】FlashAttention", section 2.2, and
// "FlashAttention 在昇腾NPU上到底快在哪", section 三), with both products on the
// 8-bit matrix instruction v_mfma_f32_32x32x64_f8f6f4 (64-deep contraction,
// fp32 accumulation), twice the bf16 rate:
//
//  * S^T = K Q^T: the scale product q_scale * k_scale folds into the softmax
//    constant, so the codes enter the product unchanged;
//  * P is rounded to e4m3 after multiplying by 2^7 (P <= 2^kSlack8 after the
//    lazy running max, so 2^7 P stays below the format's 448); the row sum
//    and the log-sum-exp take the fp32 P, so only the P V product sees the
//    rounding (relative error at most 2^-4 per probability);
//  * O^T += V^T P^T: a 32-byte operand fragment holds one column of V over
//    the 32 keys that the lane's P registers hold, in the order of those
//    registers.  V tiles are copied global -> LDS like K tiles (row-major),
//    and the gfx950 transposing read ds_read_b64_tr_b8 gathers the column:
//    within each 16-lane group, byte e of result lane j is byte j % 8 of the
//    8 bytes that lane 2 e + j / 8 addresses, so source lanes 2 e and 2 e + 1
//    address the same key row at columns C and C + 8, and four reads (keys
//    16 apart) give the 32 keys.
//
// d = 128 only.  O is written in bf16, LSE in fp32, as for fa_fwd.
#include "fa_device.h"
#include "fa_kernels.h"

#include <type_traits>

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kW8 = 8;              // waves (32 query rows each)
constexpr int kBr8 = 32 * kW8;      // query rows per workgroup
constexpr int kBc8 = 64;            // keys per tile
constexpr int kD8 = 128;            // head size (bytes per row of Q, K, V)
constexpr float kSlack8 = 1.f;      // log2 units the running max may lag behind
constexpr float kPExp = 7.f;        // P is stored as e4m3(2^kPExp p)

struct Fp8Args {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, Hkv, N, nqt;
  float c;       // scale * q_scale * k_scale * log2(e)
  float vscale;  // v_scale
};

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// K tiles and Q rows are 128-byte rows: the same geometry as bf16 rows of 64
// elements, so the bf16 d = 64 tile layout, copy and row-fragment reads serve.
typedef Lay<bf16, 64> KL;

template <bool CAUSAL>
__global__ __launch_bounds__(64 * kW8, 2) void fa_fwd_fp8_kernel(Fp8Args a) {
  constexpr int TBK = kBc8 * KL::RB;        // 8 KB K or V tile
  constexpr int DB = kD8 / 32;
  __shared__ __attribute__((aligned(1024))) char sK0[TBK], sK1[TBK], sV0[TBK], sV1[TBK];
  // Staging of the output rows of waves 4..7 (waves 0..3 use the tiles).
  __shared__ __attribute__((aligned(1024))) char sX[4 * TBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  int bh, qi;
  xcd_map(blockIdx.x, a.B * a.H, bh, qi);
  const int qt = CAUSAL ? a.nqt - 1 - qi : qi;
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = h / (a.H / a.Hkv);
  const size_t slab = (size_t)N * kD8;       // bytes per head
  const int q0w = qt * kBr8 + 32 * w;
  const int myq = q0w + l32;

  // Q fragments of the two 64-deep steps: bytes 64 s + 16 hf .. +15 and
  // 64 s + 32 + 16 hf .. +15 of the row (the K fragments use the same bytes).
  i32x8 qf[2];
  {
    const rsrc_t rQ = make_rsrc(reinterpret_cast<const char*>(a.q) + (size_t)bh * slab, (uint32_t)slab);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 lo = load16(rQ, (uint32_t)(myq * kD8 + 64 * s + 16 * hf));
      const u32x4 hi = load16(rQ, (uint32_t)(myq * kD8 + 64 * s + 32 + 16 * hf));
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  const int kend = CAUSAL ? min(N, (qt + 1) * kBr8) : N;
  const int nt = (kend + kBc8 - 1) / kBc8;
  const char* Kh = reinterpret_cast<const char*>(a.k) + (size_t)(b * a.Hkv + kvh) * slab;
  const char* Vh = reinterpret_cast<const char*>(a.v) + (size_t)(b * a.Hkv + kvh) * slab;
  RowFrags<bf16, 64> rf;
  TileCopy<bf16, 64, kBc8, kW8> tc;
  rf.init();
  tc.init(w);
  // Transposing reads of V: source lane 16 G + s addresses key row
  // 8 (e / 4) + 4 hf + e % 4 (+ 16 r for read r), e = s / 2, at columns
  // 32 db + 16 (G % 2) + 8 (s % 2) .. + 7; result lane l then holds column
  // 32 db + l % 32 over the keys of P register slots 8 r .. 8 r + 7.  The
  // tile's granule permutation depends on row bits 1-3 only, so read r is an
  // immediate offset of 16 r rows.
  int voff[DB];
  {
    const int s16 = lane & 15, e = s16 >> 1;
    const int vkey = 8 * (e >> 2) + 4 * hf + (e & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db] = KL::off(vkey, (32 * db + 16 * ((lane >> 4) & 1) + 8 * (s16 & 1)) / 2);
  }
  auto copy_kv = [&](char* sK, char* sV, int k0) {
    tc.issue(reinterpret_cast<const bf16*>(Kh), N, k0, sK);
    tc.issue(reinterpret_cast<const bf16*>(Vh), N, k0, sV);
  };

  lds_zero<64 * kW8>(sK0, TBK); lds_zero<64 * kW8>(sK1, TBK);
  lds_zero<64 * kW8>(sV0, TBK); lds_zero<64 * kW8>(sV1, TBK);
  __syncthreads();
  copy_kv(sK0, sV0, 0);
  wait_loads();  // the Q rows and the copies
  __syncthreads();

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  // The e4m3 P operand.  Each word is rewritten in two halves every tile; the
  // first conversion takes the word's previous value as the half it keeps, so
  // no register has to be cleared first.
  i32x8 pf = {};

  auto tile = [&](const char* sK, const char* sV, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK && CAUSAL && k0 > q0w + 31) return;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 lo, hi;
        rf.read(lo, sK, kb, 2 * st);
        rf.read(hi, sK, kb, 2 * st + 1);
        const u32x4 l4 = __builtin_bit_cast(u32x4, lo), h4 = __builtin_bit_cast(u32x4, hi);
        const i32x8 kf = {(int)l4[0], (int)l4[1], (int)l4[2], (int)l4[3], (int)h4[0], (int)h4[1], (int)h4[2], (int)h4[3]};
        s[kb] = mfma8(kf, qf[st], s[kb]);
      }
    }
    if (MASK) {
      const int lim = (CAUSAL ? myq : N - 1) - k0 - 4 * hf;
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
    if (__ballot(mt > m + kSlack8)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    // 2^kPExp p, summed in fp32 and packed to e4m3 in register order (byte
    // 16 kb + i of the operand = register i of key block kb).
    const float mb = m - kPExp;
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -mb));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], a.c, -mb));
        const float p2 = fast_exp2(__builtin_fmaf(s[kb][i + 2], a.c, -mb));
        const float p3 = fast_exp2(__builtin_fmaf(s[kb][i + 3], a.c, -mb));
        ts += (p0 + p1) + (p2 + p3);
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[(16 * kb + i) >> 2], false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
        pf[(16 * kb + i) >> 2] = wd;
      }
    lsum += ts;
    // O^T += V^T P^T: one 64-deep product per 32 columns of V.
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x2 c[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        c[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((lds_void*)(sV + voff[db] + 16 * r * KL::RB)));
      const i32x8 vf = {c[0][0], c[0][1], c[1][0], c[1][1], c[2][0], c[2][1], c[3][0], c[3][1]};
      acc[db] = mfma8(vf, pf, acc[db]);
    }
  };
  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Any;

  const int jfull = min(nt, CAUSAL ? (qt * kBr8) / kBc8 : N / kBc8);
  auto step = [&](int j, char* sKc, char* sVc, char* sKn, char* sVn, auto mask_tag) {
    if (j + 1 < nt) copy_kv(sKn, sVn, (j + 1) * kBc8);
    tile(sKc, sVc, j * kBc8, mask_tag);
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

  lsum += other_half(lsum);
  // The tiles are free after the last step's barrier; each wave stages its 32
  // output rows (8 KB) in one of them or in sX.
  char* const stage = w == 0 ? sK0 : w == 1 ? sK1 : w == 2 ? sV0 : w == 3 ? sV1 : sX + (w - 4) * TBK;
  store_rows_lds<kD8, true>(reinterpret_cast<bf16*>(a.o) + (size_t)bh * N * kD8, q0w, N, acc, a.vscale / lsum, stage);
  if (hf == 0 && myq < N) a.lse[(size_t)bh * N + myq] = (m - kPExp + __log2f(lsum)) * kLn2;
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream) {
  Fp8Args a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.N = p.N;
  a.nqt = (p.N + kBr8 - 1) / kBr8;
  a.c = p.scale * p.q_scale * p.k_scale * kLog2e;
  a.vscale = p.v_scale;
  const dim3 grid((unsigned)((long)a.nqt * p.B * p.H));
  if (p.causal)
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<true>), grid, dim3(64 * kW8), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<false>), grid, dim3(64 * kW8), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
