// fa_device.h — gfx950 device helpers shared by the attention kernels.
//
// Matrix-core conventions used throughout (checked on gfx950 hardware):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row (l % 32), k = 8*(l / 32) + 0..7       (8 bf16)
//     B: lane l holds col (l % 32), k = 8*(l / 32) + 0..7       (8 bf16)
//     D: lane l holds col (l % 32), register i holds
//        row 8*(i / 4) + 4*(l / 32) + (i % 4)                    (16 fp32)
//   v_mfma_f32_32x32x2_f32 has the same D layout; A/B hold k = l / 32.
//   ds_read_b64_tr_b16: within each group of 16 lanes, result lane j element e
//     is element (j % 4) of the 8 bytes addressed by lane 4*e + j/4.
//
// A "k16 fragment" is one lane's 8 operand values for a 16-deep step of the
// contraction.  Any fixed assignment of contraction indices to (lane half,
// register) is valid as long as the A and B fragments of one product use the
// same one; the kernels rely on that freedom to feed softmax results straight
// from D registers into the next product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------- products
__device__ __forceinline__ f32x16 mfma_k16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_k16(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------- fragments
// Eight consecutive elements starting at p (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ void frag_rm(bf16x8& f, const bf16* p) { f = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void frag_rm(f32x8& f, const float* p) {
  f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
  f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void frag_zero(bf16x8& f) { f = bf16x8{}; }
__device__ __forceinline__ void frag_zero(f32x8& f) { f = f32x8{}; }

// Column fragment from a row-major LDS matrix M (row stride `st` elements):
// the lane owning column c0 + (lane % 32) receives M[rA + 0..3][col] in
// registers 0..3 and M[rB + 0..3][col] in registers 4..7.  rA and rB may
// differ between the two lane halves.
__device__ __forceinline__ void frag_tr(bf16x8& f, const bf16* M, int st, int rA, int rB, int c0) {
  const int l = lane_id();
  const int e = (l & 15) >> 2, c = l & 3, g = (l >> 4) & 1;
  const int col = c0 + g * 16 + 4 * c;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(M + (rA + e) * st + col));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(M + (rB + e) * st + col));
  f = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ void frag_tr(f32x8& f, const float* M, int st, int rA, int rB, int c0) {
  const int col = c0 + (lane_id() & 31);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = M[(rA + e) * st + col]; f[4 + e] = M[(rB + e) * st + col]; }
}

// Eight fp32 values of a D-register block, taken as a k16 fragment.
__device__ __forceinline__ void frag_from(bf16x8& f, const f32x16& s, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)s[base + j];
}
__device__ __forceinline__ void frag_from(f32x8& f, const f32x16& s, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = s[base + j];
}

// ---------------------------------------------------------------- lane exchange
// Value held by lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane_id() < 32) ? r[1] : r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- stores
// Four consecutive elements at p (8-byte aligned for bf16, 16 for f32).
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// ---------------------------------------------------------------- tile staging
// A [ROWS x D] tile of a row-major [N x D] matrix staged through registers into
// LDS (row stride ST elements).  Rows at or beyond n are filled with zeros, so
// nothing outside the tensor is read.  NT threads cooperate; each moves CH
// 16-byte chunks.
template <typename T, int ROWS, int D, int ST, int NT>
struct TileCopy {
  static constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                    // chunks per row
  static constexpr int CH = ROWS * CPR / NT;             // chunks per thread
  static_assert(ROWS * CPR % NT == 0, "tile must split evenly over the threads");
  uint4 r[CH];
  __device__ __forceinline__ void load(const T* g, int row0, int n, int tid) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = tid + c * NT, row = id / CPR, ch = id % CPR;
      if (row0 + row < n)
        r[c] = *reinterpret_cast<const uint4*>(g + (size_t)(row0 + row) * D + ch * EPC);
      else
        r[c] = uint4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = tid + c * NT, row = id / CPR, ch = id % CPR;
      *reinterpret_cast<uint4*>(s + row * ST + ch * EPC) = r[c];
    }
  }
};

}  // namespace fa
