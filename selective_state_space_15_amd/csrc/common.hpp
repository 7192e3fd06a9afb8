// Device-side building blocks shared by the gfx950 kernels of the mixer hot path.
//
//  * I/O element traits (bf16 stored as raw uint16 bits, or fp32).
//  * bf16 <-> fp32 conversion (round to nearest even).
//  * A wave-level MFMA tile product reading both operands from LDS, in either
//    orientation, for the two instantiations the library supports:
//      bf16 I/O: v_mfma_f32_16x16x32_bf16 (gfx950), 8 K-values per lane;
//      fp32 I/O: v_mfma_f32_16x16x4_f32, 1 K-value per lane.
//    Both accumulate a 16x16 fp32 tile; lane l holds rows 4*(l/16)+r (r = 0..3)
//    of column l%16.  Each lane feeds row l%16 of A and column l%16 of B with the
//    K-slice owned by its lane group l/16; A and B use the same slice mapping, so
//    the product does not depend on how the hardware orders K inside an
//    instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssd {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {
  uint16_t bits;
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed bf16 pair (low half = a), one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 -> packed fp16 pair (low half = a), each rounded to nearest even; and back.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2h2(float a, float b) {
  const f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float h2f_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2, w).x);
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2, w).y);
}

// ---------------------------------------------------------------- I/O traits
template <typename IO>
struct io_traits;

template <>
struct io_traits<bf16_t> {
  using elem = uint16_t;   // global element
  using lds = uint16_t;    // LDS operand element (bf16 bits)
  static constexpr int kstep = 32;  // K per MFMA
  static constexpr int kpl = 8;     // K-values per lane
  static constexpr int vec = 8;     // elements per 16-byte vector
  __device__ static __forceinline__ float to_f(elem v) { return bf2f(v); }
  __device__ static __forceinline__ elem from_f(float v) { return f2bf(v); }
  __device__ static __forceinline__ lds to_lds(float v) { return f2bf(v); }
  __device__ static __forceinline__ float lds_to_f(lds v) { return bf2f(v); }
};

template <>
struct io_traits<float> {
  using elem = float;
  using lds = float;
  static constexpr int kstep = 4;
  static constexpr int kpl = 1;
  static constexpr int vec = 4;
  __device__ static __forceinline__ float to_f(elem v) { return v; }
  __device__ static __forceinline__ elem from_f(float v) { return v; }
  __device__ static __forceinline__ lds to_lds(float v) { return v; }
  __device__ static __forceinline__ float lds_to_f(lds v) { return v; }
};

// 16-byte vector of I/O elements held as floats.
template <typename IO>
struct vec16 {
  static constexpr int n = io_traits<IO>::vec;
  float v[n];
};

template <typename IO>
__device__ __forceinline__ void load_vec16(vec16<IO>& out, const typename io_traits<IO>::elem* p) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  if constexpr (io_traits<IO>::vec == 8) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out.v[2 * i] = __uint_as_float(w[i] << 16);
      out.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    out.v[0] = __uint_as_float(raw.x);
    out.v[1] = __uint_as_float(raw.y);
    out.v[2] = __uint_as_float(raw.z);
    out.v[3] = __uint_as_float(raw.w);
  }
}

// Element v of a raw 16-byte vector of I/O elements, as float (v is a
// compile-time constant after unrolling, so this is a register select).
template <typename IO>
__device__ __forceinline__ float raw_elem(const uint4& raw, int v) {
  constexpr int per_word = io_traits<IO>::vec / 4;  // 2 (bf16) or 1 (fp32)
  const int wi = v / per_word;
  const uint32_t w = wi == 0 ? raw.x : wi == 1 ? raw.y : wi == 2 ? raw.z : raw.w;
  if constexpr (per_word == 2)
    return __uint_as_float((v & 1) ? (w & 0xffff0000u) : (w << 16));
  else
    return __uint_as_float(w);
}

// v if keep, else zeros.  Selects the four words separately: a select between two
// uint4 structs is lowered through scratch memory.
__device__ __forceinline__ uint4 keep_if(bool keep, const uint4& v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}
__device__ __forceinline__ uint2 keep_if(bool keep, const uint2& v) {
  return make_uint2(keep ? v.x : 0u, keep ? v.y : 0u);
}

template <typename IO>
__device__ __forceinline__ void zero_vec16(vec16<IO>& out) {
#pragma unroll
  for (int i = 0; i < vec16<IO>::n; ++i) out.v[i] = 0.f;
}

template <typename IO>
__device__ __forceinline__ void store_vec16(typename io_traits<IO>::elem* p, const float* v) {
  uint4 raw;
  if constexpr (io_traits<IO>::vec == 8) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f2bf2(v[2 * i], v[2 * i + 1]);
    raw = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    raw = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3]));
  }
  *reinterpret_cast<uint4*>(p) = raw;
}

// ---------------------------------------------------------------- math
// Logistic function with the hardware reciprocal (about 1 ulp) instead of an IEEE
// division: exp, add, rcp.
__device__ __forceinline__ float sigmoidf_(float u) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-u));
}
__device__ __forceinline__ float siluf_(float u) { return u * sigmoidf_(u); }
__device__ __forceinline__ float softplusf_(float u) {
  return fmaxf(u, 0.f) + log1pf(__expf(-fabsf(u)));
}
__device__ __forceinline__ float dsiluf_(float u) {
  const float s = sigmoidf_(u);
  return s * (1.f + u * (1.f - s));
}

// ---------------------------------------------------------------- cross-lane (DPP)
// Cross-lane moves within the VALU (data-parallel primitives of the gfx9 family),
// instead of LDS-routed permutes.  update_dpp(old, src, ctrl, row_mask, bank_mask,
// bound_ctrl): each lane takes src from the lane the control selects; lanes whose
// source is outside its 16-lane row get 0 when bound_ctrl is set, and lanes of rows
// masked off keep `old`.
template <int CTRL, int ROW_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, BOUND_CTRL));
}
constexpr int kDppQuad1032 = 0xB1;     // quad_perm: lane i ^ 1
constexpr int kDppQuad2301 = 0x4E;     // quad_perm: lane i ^ 2
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowShr = 0x110;      // + shift (1 .. 15)
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3

// Sum over the 16 lanes of each row (lanes 16r .. 16r+15); every lane of the row
// receives it.  Pairs, quads, half rows, rows.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuad1032>(0.f, v);
  v += dpp_f<kDppQuad2301>(0.f, v);
  v += dpp_f<kDppRowHalfMirror>(0.f, v);
  v += dpp_f<kDppRowMirror>(0.f, v);
  return v;
}

// Maximum over the 64 lanes of a wave, in every lane (row maxima, then the four rows).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuad1032>(0.f, v));
  v = fmaxf(v, dpp_f<kDppQuad2301>(0.f, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(0.f, v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(0.f, v));
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48))));
}

// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele inside each
// row (shifts 1, 2, 4, 8), then the totals of the rows before are added.
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_f<kDppRowShr + 1, 0xf, true>(0.f, v);
  v += dpp_f<kDppRowShr + 2, 0xf, true>(0.f, v);
  v += dpp_f<kDppRowShr + 4, 0xf, true>(0.f, v);
  v += dpp_f<kDppRowShr + 8, 0xf, true>(0.f, v);
  v += dpp_f<kDppRowBcast15, 0xa>(0.f, v);  // rows 1, 3 += totals of rows 0, 2
  v += dpp_f<kDppRowBcast31, 0xc>(0.f, v);  // rows 2, 3 += total of rows 0..1
  return v;
}

// Value of lane `src` (a wave-uniform lane index), in every lane.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

// Sum over the 64 lanes of a wave, in every lane: row sums, then the four rows in order.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}

// ---------------------------------------------------------------- MFMA tiles
__device__ __forceinline__ f32x4 mfma_step(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand fetch for one MFMA step.  `kc` (K-contiguous): element (row, k) at
// base[row * ld + k]; otherwise at base[k * ld + row].
template <typename L, bool kc>
struct frag;

template <bool kc>
struct frag<uint16_t, kc> {
  using type = bf16x8;
  __device__ static __forceinline__ type zero() { return __builtin_bit_cast(bf16x8, u16x8{}); }
  __device__ static __forceinline__ type get(const uint16_t* base, int ld, int row, int k) {
    if constexpr (kc) {
      const uint4 raw = *reinterpret_cast<const uint4*>(base + row * ld + k);
      return __builtin_bit_cast(bf16x8, raw);
    } else {
      // Two gfx950 LDS transpose reads (ds_read_b64_tr_b16).  Inside each group of 16
      // lanes, lane i receives element i % 4 of the 8-byte chunks that lanes i / 4,
      // i / 4 + 4, i / 4 + 8 and i / 4 + 12 address.  So lane s of the group points at
      // row k + s / 4, columns row0 + 4 (s % 4) .. + 3 (row0 = row - s, the tile's
      // first column) and gets back column `row` at k .. k + 3; the second read adds 4
      // to k.  Needs ld and row0 to be multiples of 4 elements (8-byte chunks).
      const int s = threadIdx.x & 15;
      const uint16_t* p = base + (k + (s >> 2)) * ld + (row - s) + 4 * (s & 3);
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * ld));
      const u16x8 u = {static_cast<uint16_t>(lo[0]), static_cast<uint16_t>(lo[1]),
                       static_cast<uint16_t>(lo[2]), static_cast<uint16_t>(lo[3]),
                       static_cast<uint16_t>(hi[0]), static_cast<uint16_t>(hi[1]),
                       static_cast<uint16_t>(hi[2]), static_cast<uint16_t>(hi[3])};
      return __builtin_bit_cast(bf16x8, u);
    }
  }
};

template <bool kc>
struct frag<float, kc> {
  using type = float;
  __device__ static __forceinline__ type zero() { return 0.f; }
  __device__ static __forceinline__ type get(const float* base, int ld, int row, int k) {
    return kc ? base[row * ld + k] : base[k * ld + row];
  }
};

// acc[j] += A(16 x K) * B_j(K x 16) for NJ column tiles sharing one 16-row A strip.
//   A rows m0..m0+15 of an operand stored per `akc`;
//   B tile j: columns n0 + 16*j .. +15, stored per `bkc`.
// K must be a multiple of the per-lane K-slice (8 for bf16); when it is not a
// multiple of the MFMA K-step, lanes whose slice lies at or past K feed zeros.
// Executed by one full wave.  UNROLL > 1 unrolls the K loop so the operand reads of
// later K-steps issue ahead of the MFMAs (for kernels with registers to spare).
template <typename L, bool akc, bool bkc, int NJ, int UNROLL = 1>
__device__ __forceinline__ void mma_strip(f32x4 (&acc)[NJ], const L* A, int lda, int m0, const L* B,
                                          int ldb, int n0, int K) {
  constexpr int kstep = sizeof(L) == 2 ? 32 : 4;
  constexpr int kpl = sizeof(L) == 2 ? 8 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  const int kg = lane >> 4;
  // one K-step at a time by default: a fully unrolled K loop lets the scheduler
  // hoist every fragment read of every tile ahead of the MFMAs, which costs more
  // registers than two waves per SIMD have
#pragma unroll UNROLL
  for (int k0 = 0; k0 < K; k0 += kstep) {
    const int kr = k0 + kpl * kg;
    const bool kin = kr < K;
    const int k = kin ? kr : 0;  // every lane reads (transpose reads are cooperative)
    const auto av = frag<L, akc>::get(A, lda, m0 + r, k);
    const auto a = kin ? av : frag<L, akc>::zero();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const auto bv = frag<L, bkc>::get(B, ldb, n0 + 16 * j + r, k);
      const auto b = kin ? bv : frag<L, bkc>::zero();
      acc[j] = mfma_step(a, b, acc[j]);
    }
  }
}

// acc[j] += (A1 + A2)(16 x K) * B_j(K x 16), A1 and A2 stored alike (the two parts of
// a split operand): each B fragment is read once for both products.  The A1 products
// of all tiles issue before the A2 ones, so no MFMA waits on the one before it.
template <typename L, bool akc, bool bkc, int NJ, int UNROLL = 1>
__device__ __forceinline__ void mma_strip2(f32x4 (&acc)[NJ], const L* A1, const L* A2, int lda, int m0,
                                           const L* B, int ldb, int n0, int K) {
  constexpr int kstep = sizeof(L) == 2 ? 32 : 4;
  constexpr int kpl = sizeof(L) == 2 ? 8 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  const int kg = lane >> 4;
#pragma unroll UNROLL
  for (int k0 = 0; k0 < K; k0 += kstep) {
    const int kr = k0 + kpl * kg;
    const bool kin = kr < K;
    const int k = kin ? kr : 0;
    const auto a1v = frag<L, akc>::get(A1, lda, m0 + r, k);
    const auto a2v = frag<L, akc>::get(A2, lda, m0 + r, k);
    const auto a1 = kin ? a1v : frag<L, akc>::zero();
    const auto a2 = kin ? a2v : frag<L, akc>::zero();
    typename frag<L, bkc>::type b[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const auto bv = frag<L, bkc>::get(B, ldb, n0 + 16 * j + r, k);
      b[j] = kin ? bv : frag<L, bkc>::zero();
      acc[j] = mfma_step(a1, b[j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = mfma_step(a2, b[j], acc[j]);
  }
}

// acc1[j] += A * B1_j and acc2[j] += A * B2_j with one 16-row A strip: each A fragment
// is read once for both products, and their MFMAs interleave.
template <typename L, bool akc, bool bkc, int NJ1, int NJ2>
__device__ __forceinline__ void mma_strip_ab(f32x4 (&acc1)[NJ1], f32x4 (&acc2)[NJ2], const L* A, int lda,
                                             int m0, const L* B1, int ldb1, int n01, const L* B2,
                                             int ldb2, int n02, int K) {
  constexpr int kstep = sizeof(L) == 2 ? 32 : 4;
  constexpr int kpl = sizeof(L) == 2 ? 8 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  const int kg = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += kstep) {
    const int kr = k0 + kpl * kg;
    const bool kin = kr < K;
    const int k = kin ? kr : 0;
    const auto av = frag<L, akc>::get(A, lda, m0 + r, k);
    const auto a = kin ? av : frag<L, akc>::zero();
#pragma unroll
    for (int j = 0; j < (NJ1 > NJ2 ? NJ1 : NJ2); ++j) {
      if (j < NJ1) {
        const auto bv = frag<L, bkc>::get(B1, ldb1, n01 + 16 * j + r, k);
        acc1[j] = mfma_step(a, kin ? bv : frag<L, bkc>::zero(), acc1[j]);
      }
      if (j < NJ2) {
        const auto bv = frag<L, bkc>::get(B2, ldb2, n02 + 16 * j + r, k);
        acc2[j] = mfma_step(a, kin ? bv : frag<L, bkc>::zero(), acc2[j]);
      }
    }
  }
}

// Ordered column sums of a row-major [rows][cols] fp32 matrix, 64 columns per
// 256-thread block (column blockIdx.x * 64 + lane).  Wave w adds rows w, w + 4,
// w + 8, ... with 16 loads in flight; the four wave partials are then added in
// wave order, so the result is the same on every run.  Valid on wave 0.
__device__ __forceinline__ float block_colsum(const float* m, int64_t rows, int64_t cols) {
  __shared__ float s_part[4][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t col = blockIdx.x * static_cast<int64_t>(kWave) + lane;
  float acc = 0.f;
  if (col < cols) {
    int64_t q = wave;
    for (; q + 4 * 15 < rows; q += 4 * 16) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = m[(q + 4 * i) * cols + col];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += v[i];
    }
    for (; q < rows; q += 4) acc += m[q * cols + col];
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  return s_part[0][lane] + s_part[1][lane] + s_part[2][lane] + s_part[3][lane];
}

// base + `bytes`, with the byte offset held as an opaque 32-bit vector value: the
// address is then formed at the access as a scalar base plus a 32-bit offset (one
// vector register), instead of a 64-bit per-thread pointer that the compiler would
// hoist out of a loop (two registers each, spilled under register pressure).
template <typename Ptr>
__device__ __forceinline__ Ptr byte_off(Ptr base, uint32_t bytes) {
  asm volatile("" : "+v"(bytes));
  using C = std::conditional_t<std::is_const_v<std::remove_pointer_t<Ptr>>, const char*, char*>;
  return reinterpret_cast<Ptr>(reinterpret_cast<C>(base) + bytes);
}

// Row / column of accumulator element e (0..3) of this lane inside a 16x16 tile.
__device__ __forceinline__ int acc_row(int e) { return 4 * ((threadIdx.x & 63) >> 4) + e; }
__device__ __forceinline__ int acc_col() { return threadIdx.x & 15; }

// The four values T[m0 + acc_row(e)][c0 + acc_col()], e = 0..3, of a row-major LDS tile
// (element (r, c) at base[r * ld + c]) as floats: the accumulator layout of one 16x16
// tile.  bf16 tiles take one gfx950 transpose read (ds_read_b64_tr_b16): inside each
// 16-lane group, lane a points at row m0 + 4 (lane / 16) + a / 4, columns
// c0 + 4 (a % 4) .. + 3, and lane i gets back element i % 4 of the chunks of lanes
// i / 4 + 4 e, which is column c0 + i of row m0 + 4 (lane / 16) + e.  Needs ld and c0 to
// be multiples of 4 elements.  fp32 tiles read the four values one by one.
template <typename L>
__device__ __forceinline__ void acc_gather(float (&v)[4], const L* base, int ld, int m0, int c0) {
  const int lane = threadIdx.x & 63;
  if constexpr (sizeof(L) == 2) {
    const int a = lane & 15;
    const L* p = base + (m0 + 4 * (lane >> 4) + (a >> 2)) * ld + c0 + 4 * (a & 3);
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(r[e])) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = base[(m0 + acc_row(e)) * ld + c0 + (lane & 15)];
  }
}

// Sum of v over the four lanes l % 16 + 16 k (k = 0..3), in each of them: two gfx950
// row swaps (v_permlane32_swap, v_permlane16_swap), no LDS round trip.
__device__ __forceinline__ float col_sum4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float s2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const uint32_t u2 = __float_as_uint(s2);
  const auto q = __builtin_amdgcn_permlane16_swap(u2, u2, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Map a hardware workgroup id to a logical id so that consecutive logical ids
// run on the same XCD (dispatch places workgroup i on XCD i % 8).  Bijective for
// any grid size.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t total) {
  constexpr int64_t kXcd = 8;
  const int64_t xcd = i % kXcd, slot = i / kXcd;
  const int64_t per = total / kXcd, rem = total % kXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace ssd
