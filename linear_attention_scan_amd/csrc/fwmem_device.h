// Device building blocks shared by the libfwmem kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand conventions. A 16x16 fp32 accumulator tile ("C layout") is held by
// one wave: lane l owns rows 4*(l/16)+i, i = 0..3, of column l%16. The kernels keep
// every intermediate matrix that feeds a later product in this layout and turn it
// straight into the next product's B operand, with no LDS round trip, by choosing
// which K index each operand slot carries:
//   * fp16 policy (PolF16, v_mfma_f32_16x16x32_f16): within a K block of 32, lane
//     group g = l/16 carries K = 4g+i (slots 0..3) and 16+4g+i (slots 4..7), i.e.
//     exactly the rows lane l owns in the two 16-row C tiles of that block.
//   * fp32 policy (PolF32, v_mfma_f32_16x16x4_f32): a K block of 16 is four
//     instructions; instruction i takes K = 4g+i, again the lane's own rows.
// A operands are read from LDS with the same K mapping. Since the A and B slots of
// one lane refer to the same K, the contraction is exact whatever order the
// hardware sums the slots in. For the fp16 policy, LDS rows store each K block of
// 32 in the permuted order p(16h + 4g + i) = 8g + 4h + i, so that the eight
// operands of lane group g are one contiguous 16-byte read (kpos() maps logical K
// to the stored position).
//
// fp16 operands carry a power-of-two scale so that any finite fp32 value range
// maps into fp16 without overflow: a block of values with max |x| = m is stored
// as x * 2^s with m * 2^s in [2^14, 2^15), and products are unscaled in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwmem {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
// 16-byte raw words as a native vector (HIP's uint4 is a struct that SROA keeps in memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// elu(x) + 1: x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Max over the four lanes that hold one column of an MFMA C tile (lanes l, l^16,
// l^32, l^48): per-column operand scales need only this two-step exchange.
__device__ __forceinline__ float col_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Reduction over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Power-of-two factor 2^s with m * 2^s in [2^14, 2^15) for finite m > 0; 1 otherwise.
__device__ __forceinline__ float pow2_scale(float m) {
  if (!(m > 0.f) || !(m <= 3.4028234e38f)) return 1.f;
  int e;
  (void)frexpf(m, &e);  // m in [2^(e-1), 2^e)
  int s = 15 - e;
  s = s < -126 ? -126 : (s > 126 ? 126 : s);
  return ldexpf(1.f, s);
}
// The same factor and its exact inverse (both powers of two, no division).
__device__ __forceinline__ void pow2_scale2(float m, float& sc, float& inv) {
  int s = 0;
  if (m > 0.f && m <= 3.4028234e38f) {
    int e;
    (void)frexpf(m, &e);
    s = 15 - e;
    s = s < -126 ? -126 : (s > 126 ? 126 : s);
  }
  sc = ldexpf(1.f, s);
  inv = ldexpf(1.f, -s);
}

// ---------------------------------------------------------------------------
// Precision policies.

struct PolF16 {
  using op_t = _Float16;
  using frag_t = h8;
  static constexpr int KB = 32;          // K extent of one operand block
  static constexpr bool kScaled = true;  // operands carry power-of-two scales
  static constexpr int kPad = 8;         // LDS row padding, elements

  __device__ static __forceinline__ op_t cvt(float x) { return (op_t)x; }

  // Stored position of logical K index k within an LDS row (see the header comment).
  __device__ static __forceinline__ int kpos(int k) {
    const int o = k & 31;
    return (k & ~31) + 8 * ((o >> 2) & 3) + 4 * (o >> 4) + (o & 3);
  }
  // Operand fragment of lane group g for K block kb: one 16-byte read.
  __device__ static __forceinline__ frag_t lds_row(const op_t* row, int kb, int g) {
    return *reinterpret_cast<const frag_t*>(row + kb * 32 + 8 * g);
  }
  // Store 8 operands of logical K k0..k0+7 (k0 a multiple of 8) into a row.
  __device__ static __forceinline__ void store_run(op_t* row, int k0, const frag_t& v) {
    const int p = kpos(k0);  // k0+4..k0+7 sit 8 positions further
    *reinterpret_cast<h4*>(row + p) = h4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<h4*>(row + p + 8) = h4{v[4], v[5], v[6], v[7]};
  }
  // Store 4 operands of logical K k0..k0+3 (k0 a multiple of 4).
  __device__ static __forceinline__ void store4(op_t* row, int k0, float a, float b, float c, float d) {
    *reinterpret_cast<h4*>(row + kpos(k0)) = h4{(op_t)a, (op_t)b, (op_t)c, (op_t)d};
  }
  // Operand fragment from C-layout tiles c[2kb], c[2kb+1], each value times s.
  __device__ static __forceinline__ frag_t from_c(const f4* c, int kb, float s) {
    frag_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (op_t)(c[2 * kb][i] * s);
      r[4 + i] = (op_t)(c[2 * kb + 1][i] * s);
    }
    return r;
  }
  __device__ static __forceinline__ void mma(f4& acc, const frag_t& a, const frag_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
};

struct PolF32 {
  using op_t = float;
  using frag_t = f4;
  static constexpr int KB = 16;
  static constexpr bool kScaled = false;
  static constexpr int kPad = 4;

  __device__ static __forceinline__ op_t cvt(float x) { return x; }

  __device__ static __forceinline__ int kpos(int k) { return k; }
  __device__ static __forceinline__ frag_t lds_row(const op_t* row, int kb, int g) {
    return *reinterpret_cast<const f4*>(row + kb * 16 + 4 * g);
  }
  __device__ static __forceinline__ void store_run(op_t* row, int k0, const frag_t& v) {
    *reinterpret_cast<f4*>(row + k0) = v;
  }
  __device__ static __forceinline__ void store4(op_t* row, int k0, float a, float b, float c, float d) {
    *reinterpret_cast<f4*>(row + k0) = f4{a, b, c, d};
  }
  // Fragment whose K runs down a column: element (k, m) at base[k * ld + m].
  __device__ static __forceinline__ frag_t lds_col(const op_t* base, int ld, int m, int kb, int g) {
    frag_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = base[(kb * 16 + 4 * g + i) * ld + m];
    return r;
  }
  __device__ static __forceinline__ frag_t from_c(const f4* c, int kb, float s) {
    return c[kb] * s;
  }
  __device__ static __forceinline__ void mma(f4& acc, const frag_t& a, const frag_t& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
  }
};

// Input element access: bf16 (stored as uint16_t) or float.
template <typename InT>
struct In;

template <>
struct In<uint16_t> {
  static constexpr int VW = 8;  // elements per 16-byte load
  using Pol = PolF16;
  __device__ static __forceinline__ void load(const uint16_t* p, float (&x)[VW]) {
    decode(*reinterpret_cast<const u32x4*>(p), x);
  }
  __device__ static __forceinline__ void decode(const u32x4& w, float (&x)[VW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};

template <>
struct In<float> {
  static constexpr int VW = 4;
  using Pol = PolF32;
  __device__ static __forceinline__ void load(const float* p, float (&x)[VW]) {
    decode(*reinterpret_cast<const u32x4*>(p), x);
  }
  __device__ static __forceinline__ void decode(const u32x4& w, float (&x)[VW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
};

// log|a| (floored so that an exact zero gives a large negative finite value) and
// whether a < 0; decay products are carried as (sum of logs, sign parity).
__device__ __forceinline__ float log_abs_floor(float a) { return __logf(fmaxf(fabsf(a), 1e-30f)); }

// Inclusive prefix over the 64 lanes of a wave of (log|a|, count of negative a).
__device__ __forceinline__ void wave_prefix(float& la, int& ng) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(la, o);
    const int z = __shfl_up(ng, o);
    if (lane >= o) { la += y; ng += z; }
  }
}

}  // namespace fwmem
