// fa_device.h — gfx950 device building blocks shared by the attention kernels.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, D[32x32] += A[32x16] B[16x32]):
//   A: lane l holds row (l % 32), k = 8*(l / 32) + 0..7             (8 bf16)
//   B: lane l holds col (l % 32), k = 8*(l / 32) + 0..7             (8 bf16)
//   D: lane l holds col (l % 32); register i holds
//      row 8*(i / 4) + 4*(l / 32) + (i % 4)                          (16 fp32)
// v_mfma_f32_32x32x2_f32 has the same D layout; eight of them make one
// 16-deep step with A/B lane l holding k = l / 32 in each.
//
// A "k16 fragment" is one lane's 8 operand values of a 16-deep step of the
// contraction.  Any fixed assignment of contraction indices to (lane half,
// register) is valid as long as the A and B fragments of one product use the
// same one.  The kernels use that freedom to feed the fp32 D registers of one
// product (after conversion) straight into the next product as its B operand:
// register block j of a D tile covers the rows {8j' + 4*(l/32) + 0..3}, which
// the transposing LDS read below reproduces for the other operand.
//
// LDS tiles are stored without padding.  A bf16 row of D elements is D/8
// granules of 16 bytes; granule g of row r sits at position g ^ sw(r).  The
// permutation makes both access patterns the kernels use conflict-free on the
// 64-bank LDS: a 16-lane group reading one granule of 16 consecutive rows
// (row fragments, ds_read_b128), and a 32-lane group reading four whole
// granules of four consecutive rows (column fragments, ds_read_b64_tr_b16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

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
__device__ __forceinline__ f32x16 mfma_k16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_k16(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------- global memory
// Buffer resource over `bytes` bytes at `base`.  Loads at or beyond `bytes`
// return zero instead of touching memory, which masks ragged tails for free.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float load4f(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Eight consecutive elements of row `row`, starting at column c0, of a row-major
// [*, D] tensor behind `r` (zero past its end) as a k16 fragment.
template <int D>
__device__ __forceinline__ void frag_global(bf16x8& f, rsrc_t r, int row, int c0) {
  f = __builtin_bit_cast(bf16x8, load16(r, (uint32_t)(row * D + c0) * 2u));
}
template <int D>
__device__ __forceinline__ void frag_global(f32x8& f, rsrc_t r, int row, int c0) {
  const uint32_t o = (uint32_t)(row * D + c0) * 4u;
  const f32x4 a = __builtin_bit_cast(f32x4, load16(r, o)), b = __builtin_bit_cast(f32x4, load16(r, o + 16));
  f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---------------------------------------------------------------- LDS tiles
template <typename T, int D>
struct Lay {
  static constexpr int RB = D * (int)sizeof(T);  // bytes per row
  static constexpr int G = RB / 16;              // 16-byte granules per row
  static constexpr int EPG = 16 / (int)sizeof(T);
  // Position permutation of the granules of row r (float tiles are unpermuted).
  __device__ static __forceinline__ int sw(int r) {
    if constexpr (sizeof(T) == 4) {
      return 0;
    } else if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      const int s = r >> 1;  // two 128-byte rows share one 256-byte bank line
      return ((s & 1) << 2) | ((s >> 1) & 3);
    }
  }
  // Byte offset of element (r, c) in the tile.
  __device__ static __forceinline__ int off(int r, int c) {
    return r * RB + (((c / EPG) ^ sw(r)) << 4) + (c % EPG) * (int)sizeof(T);
  }
};

// Global -> LDS copies (buffer_load ... lds): lane i's 4 or 16 bytes at
// `voff` in the buffer land at lds + 4 i or lds + 16 i.  They are issued as
// inline assembly so that the compiler does not track them: it cannot tell the
// slots of a tile ring apart and would otherwise wait for every copy in flight
// before the next read of any slot.  Each kernel waits explicitly
// (wait_copies) and then synchronises before it reads what it copied.
// Both operands are wave-uniform by construction; readfirstlane moves them to
// scalar registers where the compiler computed them in vector registers.
// The LDS destination goes through m0, a register the compiler reserves: each
// copy saves m0, sets it, issues the load (which latches m0 at issue; the
// compiler's own LDS-DMA sequences rewrite m0 right after the load the same
// way) and restores it, so the asm changes no register the compiler owns.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}
__device__ __forceinline__ void copy16_to_lds(const u32x4& desc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(desc));
}
// The same copy with the non-temporal hint, for data that one workgroup reads
// exactly once (a key/value cache streamed during decoding).  Measured on
// MI355X, streams of such loads reach about 7 TB/s, plain ones about 6.1.
__device__ __forceinline__ void copy16_to_lds_nt(const u32x4& desc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(desc));
}
__device__ __forceinline__ void copy4_to_lds(const u32x4& desc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(desc));
}

// NF (32 or 64) consecutive floats [row0, row0 + NF) of the vector behind
// `desc` into LDS, issued by one wave (lanes past NF copy nothing).
template <int NF>
__device__ __forceinline__ void vec_to_lds(const u32x4& desc, float* dst, int row0) {
  static_assert(NF == 32 || NF == 64, "one copy instruction per vector");
  if (NF == 64 || lane_id() < NF) copy4_to_lds(desc, (uint32_t)(row0 + lane_id()) * 4u, lds_addr(dst));
}

// Waits until this wave's outstanding global -> LDS copies have landed.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits for this wave's global loads to registers.  Called after the loads a
// kernel keeps for its whole life, before its loop: the compiler's own waits
// count only the memory operations it can see, so one left inside the loop
// would also wait for the copies issued in the same step.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// ---------------------------------------------------------------- precomputed addressing
// The granule permutation of a row depends only on the row index modulo 16, so
// the per-lane part of every fragment address can be computed once per kernel;
// what varies per fragment (row block, k-step, tile buffer) is then a
// compile-time constant that the LDS instructions take as an immediate offset.
template <typename T, int D>
struct RowFrags {
  // Row fragment (rb, ks): row 32 rb + lane % 32, columns 16 ks + 8 (lane / 32) .. + 7.
  int off[D / 16];
  __device__ __forceinline__ void init() {
    const int l = lane_id();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) off[ks] = Lay<T, D>::off(l & 31, 16 * ks + 8 * (l >> 5));
  }
  __device__ __forceinline__ void read(bf16x8& f, const char* tile, int rb, int ks) const {
    f = *reinterpret_cast<const bf16x8*>(tile + rb * 32 * Lay<T, D>::RB + off[ks]);
  }
  __device__ __forceinline__ void read(f32x8& f, const char* tile, int rb, int ks) const {
    const char* p = tile + rb * 32 * Lay<T, D>::RB + off[ks];
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 16);
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// Column fragments use the gfx950 transposing read ds_read_b64_tr_b16: within
// each 16-lane group, result lane j, element e is element j % 4 of the 8 bytes
// addressed by lane 4 e + j / 4.  Each lane therefore addresses row
// (base + (lane % 16) / 4) at the 4-column group of its result lanes, and two
// reads (rows r and r + 8) give one k16 fragment.
template <typename T, int D>
struct ColFrags {
  // Column fragment (t, db): rows 32 (t / 2) + 16 (t % 2) + 4 (lane / 32) + e (registers
  // e = 0..3) and the same + 8 (registers 4..7), column 32 db + lane % 32.  This is the
  // row set of register block t % 2 of a D tile's rows 32 (t / 2) .. + 31.
  int off[2][D / 32];
  __device__ __forceinline__ void init() {
    const int l = lane_id();
    const int hf = l >> 5;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        if constexpr (sizeof(T) == 2)
          off[b][db] = Lay<T, D>::off(4 * hf + ((l & 15) >> 2) + 8 * b, 32 * db + (l & 16) + 4 * (l & 3));
        else
          off[b][db] = Lay<T, D>::off(4 * hf + 8 * b, 32 * db + (l & 31));
      }
  }
  __device__ static __forceinline__ int row0(int t) { return (32 * (t >> 1) + 16 * (t & 1)) * Lay<T, D>::RB; }
  template <typename V8>
  __device__ __forceinline__ void read(V8& f, const char* tile, int t, int db) const {
    static_assert(sizeof(T) == 2, "16-bit tiles");
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* p = tile + row0(t);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + off[0][db]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + off[1][db]));
    f = __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  __device__ __forceinline__ void read(f32x8& f, const char* tile, int t, int db) const {
    const char* p = tile + row0(t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = *reinterpret_cast<const float*>(p + off[0][db] + e * Lay<T, D>::RB);
      f[4 + e] = *reinterpret_cast<const float*>(p + off[1][db] + e * Lay<T, D>::RB);
    }
  }
};

// Global -> LDS copy of a [ROWS x D] tile split over NW waves, with the per-lane
// source offsets precomputed.  `issue` copies rows [row0, row0 + ROWS) of the
// [n x D] tensor at `base`; rows at or past n arrive as zeros (the buffer
// resource of each copy starts at row0 and ends at row n).
template <typename T, int D, int ROWS, int NW>
struct TileCopy {
  typedef Lay<T, D> L;
  static constexpr int CPW = ROWS * L::RB / 1024 / NW;  // 1 KB chunks per wave
  static_assert(CPW * NW * 1024 == ROWS * L::RB, "tile must split evenly over the waves");
  uint32_t voff[CPW];
  int chunk0;
  __device__ __forceinline__ void init(int w) {
    const int lane = lane_id();
    constexpr int RPC = 64 / L::G;
    chunk0 = __builtin_amdgcn_readfirstlane(w * CPW);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int rr = (chunk0 + i) * RPC + lane / L::G;
      voff[i] = (uint32_t)rr * L::RB + (uint32_t)(((lane % L::G) ^ L::sw(rr)) * 16);
    }
  }
  // NT: with the non-temporal hint (rows that no other workgroup reads again).
  template <bool NT = false>
  __device__ __forceinline__ void issue(const T* base, int n, int row0, char* dst) const {
    const u32x4 desc = buffer_desc(base + (size_t)row0 * D, (uint32_t)(n - row0) * (uint32_t)L::RB);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if constexpr (NT) copy16_to_lds_nt(desc, voff[i], lds_addr(dst) + (uint32_t)(chunk0 + i) * 1024u);
      else copy16_to_lds(desc, voff[i], lds_addr(dst) + (uint32_t)(chunk0 + i) * 1024u);
    }
  }
  // Register path for bf16 tiles consumed as fp16: `load` fetches this wave's
  // chunks of the same rows into registers (zero past n); `store_f16` converts
  // them and writes them to the same tile positions that `issue` fills.  The
  // conversion is exact for |x| in [2^-14, 65504]; smaller magnitudes keep an
  // absolute error below 2^-25.
  __device__ __forceinline__ void load(const T* base, int n, int row0, u32x4 (&r)[CPW]) const {
    const rsrc_t rs = make_rsrc(base + (size_t)row0 * D, (uint32_t)(n - row0) * (uint32_t)L::RB);
#pragma unroll
    for (int i = 0; i < CPW; ++i) r[i] = load16(rs, voff[i]);
  }
  __device__ __forceinline__ void store_f16(const u32x4 (&r)[CPW], char* dst) const {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, r[i]);
      f16x8 y;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (f16)(float)x[j];
      *reinterpret_cast<f16x8*>(dst + (chunk0 + i) * 1024 + lane * 16) = y;
    }
  }
};

// Eight fp32 values of a D-register block as a k16 fragment.
__device__ __forceinline__ void frag_from(bf16x8& f, const f32x16& s, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)s[base + j];
}
__device__ __forceinline__ void frag_from(f16x8& f, const f32x16& s, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (f16)s[base + j];
}
__device__ __forceinline__ void frag_from(f32x8& f, const f32x16& s, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = s[base + j];
}

// Zero-fills `bytes` (a multiple of 16) of LDS with NT threads.
template <int NT>
__device__ __forceinline__ void lds_zero(char* p, int bytes) {
  for (int o = threadIdx.x * 16; o < bytes; o += NT * 16) *reinterpret_cast<u32x4*>(p + o) = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------- instruction scheduling
// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier: the groups
// placed after a block of code order that block's instructions (matching
// instructions fill the groups in order; the rest are scheduled freely).
enum : int { kSgValu = 0x2, kSgMfma = 0x8, kSgDsRead = 0x100, kSgDsWrite = 0x200 };
#define FA_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

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
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Stores a transposed accumulator tile: acc[db] holds X^T[d, row] for the
// 32 rows of this wave (lane = row); writes s * X[row, :] for row < n.
template <typename T, int D>
__device__ __forceinline__ void store_rows(T* base, int row, int n, const f32x16* acc, float s) {
  if (row >= n) return;
  const int hf = lane_id() >> 5;
  T* p = base + (size_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(p + db * 32 + 8 * g + 4 * hf, s * acc[db][4 * g], s * acc[db][4 * g + 1], s * acc[db][4 * g + 2],
             s * acc[db][4 * g + 3]);
}

// The same for bf16 rows, through `lds`, a private region of the wave of 32
// rows x 2 D bytes: each lane first writes its row's values there, then every
// lane reads one 16-byte granule of a row, so that 2 D / 16 consecutive lanes
// store one whole row (full cache lines instead of 8-byte pieces of 32 rows).
// The 16-byte granules of row r are XOR-permuted by r so that the 32 rows of
// a column group fall on different banks.  Called after the wave's last read
// of the tiles that `lds` overlaps.  NT: with the non-temporal hint (rows
// written once; measured on MI355X, the hint also suits O, which the backward
// reads again).
template <int D, bool NT = false>
__device__ __forceinline__ void store_rows_lds(bf16* base, int row0, int n, const f32x16* acc, float s, char* lds) {
  constexpr int RB = 2 * D, G = RB / 16;  // bytes and 16-byte granules per row
  const int lane = lane_id(), hf = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = db * 32 + 8 * g + 4 * hf;  // first of the four elements
      char* p = lds + l32 * RB + (((col >> 3) ^ (l32 & (G - 1))) << 4) + (col & 7) * 2;
      *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)(s * acc[db][4 * g]), (bf16)(s * acc[db][4 * g + 1]),
                                             (bf16)(s * acc[db][4 * g + 2]), (bf16)(s * acc[db][4 * g + 3])};
    }
  constexpr int RPI = 64 / G;  // rows per store instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / G, gr = lane % G;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * RB + ((gr ^ (r & (G - 1))) << 4));
    u32x4* dst = reinterpret_cast<u32x4*>(base + (size_t)(row0 + r) * D + gr * 8);
    if (row0 + r < n) {
      if constexpr (NT) __builtin_nontemporal_store(v, dst);
      else *dst = v;
    }
  }
}

// ---------------------------------------------------------------- work order
// Maps a linear workgroup index onto (unit, slice) with `units` units per
// slice-step such that all workgroups of one unit land on the same XCD:
// workgroups are dealt round-robin over the 8 XCDs, so when `units` is a
// multiple of 8 the units are split into 8 contiguous ranges, one per XCD.
// `slot` counts up in dispatch order within an XCD.
__device__ __forceinline__ void xcd_map(int bid, int units, int& unit, int& slot) {
  if ((units & 7) == 0) {
    const int per = units >> 3, x = bid & 7, y = bid >> 3;
    unit = x * per + y % per;
    slot = y / per;
  } else {
    unit = bid % units;
    slot = bid / units;
  }
}

// ---------------------------------------------------------------- dropout
// Randomness of the dropout on P: Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).  One call
// covers a 4 x 4 block of one head's score matrix, query rows 4a..4a+3 and keys
// 4c..4c+3: counter (c, a, b*H + h, offset) under the 64-bit seed.  Word r of
// the result belongs to query 4a + r and its byte e (little-endian) to key
// 4c + e; an element is kept when its byte is >= t, so the drop rate is t/256.
struct DropArgs {
  uint32_t k0, k1;  // seed: low and high word
  uint32_t offset;  // fourth counter word
  uint32_t t;       // byte threshold, 1..255
  float inv;        // 256 / (256 - t): the inverted-dropout scale
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// Value of lane (lane ^ X) within each group of four lanes (DPP quad_perm).
template <int X>
__device__ __forceinline__ uint32_t quad_xor(uint32_t v) {
  if constexpr (X == 0) return v;
  constexpr int ctrl = X == 1 ? 0xB1 : X == 2 ? 0x4E : 0x1B;  // [1,0,3,2], [2,3,0,1], [3,2,1,0]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}

// x[i] for a lane-dependent i in 0..3, as two levels of selects on the bits
// of i (with i = lane % 4 ^ constant, the two conditions are the same for
// every call, so no compares are repeated).
__device__ __forceinline__ uint32_t pick4(const u32x4& x, int i) {
  const uint32_t lo = (i & 1) ? x[1] : x[0];
  const uint32_t hi = (i & 1) ? x[3] : x[2];
  return (i & 2) ? hi : lo;
}

// The four lanes of a quad (r = lane % 4) share four generator blocks: lane r
// draws block r, then three exchanges (lane r reads lane r ^ X) hand each
// lane its share of all four.  The whole wave must be active.
//
// keep_words_rows_quad: lane r holds query row 4a + r and needs, of block g
// (key block cr - 2 (r - g), i.e. keys 8 apart between blocks), word r: the
// bytes of its row for keys 4 c_g .. 4 c_g + 3.  `cr` is the key block of
// block r.
// Round X brings block r ^ X; one more pass of selects puts them in block
// order (element g of the result), so each byte is tested where it is used.
__device__ __forceinline__ u32x4 keep_words_rows_quad(const DropArgs& d, uint32_t cr, uint32_t a, uint32_t bh,
                                                      int r) {
  const u32x4 x = philox4x32_10(cr, a, bh, d.offset, d.k0, d.k1);
  const u32x4 z = u32x4{pick4(x, r), quad_xor<1>(pick4(x, r ^ 1)), quad_xor<2>(pick4(x, r ^ 2)),
                        quad_xor<3>(pick4(x, r ^ 3))};
  return u32x4{pick4(z, r), pick4(z, r ^ 1), pick4(z, r ^ 2), pick4(z, r ^ 3)};
}

__device__ __forceinline__ bool byte_kept(uint32_t w, int e, uint32_t t) { return ((w >> (8 * e)) & 0xffu) >= t; }

// Byte j of each word of x, packed: byte e of the result is byte j of x[e].
__device__ __forceinline__ uint32_t bytes_at(const u32x4& x, int j) {
  const uint32_t sh = 8u * (uint32_t)j;
  return ((x[0] >> sh) & 0xffu) | (((x[1] >> sh) & 0xffu) << 8) | (((x[2] >> sh) & 0xffu) << 16) |
         (((x[3] >> sh) & 0xffu) << 24);
}

// keep_words_cols_quad: lane r holds key 4c + r and needs, of block g (query
// block ar - 2 (r - g)), byte r of each word: the four queries of that block.
// `ar` is the query block of block r.  Element g of the result packs them:
// byte e is the byte of query 4 a_g + e.
__device__ __forceinline__ u32x4 keep_words_cols_quad(const DropArgs& d, uint32_t c, uint32_t ar, uint32_t bh,
                                                      int r) {
  const u32x4 x = philox4x32_10(c, ar, bh, d.offset, d.k0, d.k1);
  const u32x4 z = u32x4{bytes_at(x, r), quad_xor<1>(bytes_at(x, r ^ 1)), quad_xor<2>(bytes_at(x, r ^ 2)),
                        quad_xor<3>(bytes_at(x, r ^ 3))};
  return u32x4{pick4(z, r), pick4(z, r ^ 1), pick4(z, r ^ 2), pick4(z, r ^ 3)};
}

}  // namespace fa
