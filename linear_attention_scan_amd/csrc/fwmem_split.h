// bf16 split-operand scheme of the chunked scan (bf16 inputs, identity feature map,
// scalar decay): the operands shared by the prep kernel, which writes them, and the
// split propagate kernel, which consumes them.
//
// Exact and split operands. Raw bf16 keys and queries are exact bf16 MFMA operands.
// Every computed matrix (the state S, the residual R, the writes U, the solve T and
// the read mask M) is carried as an unevaluated sum hi + lo of two bf16 values
// (hi = bf16(x), lo = bf16(x - hi): 16 significant bits, the full fp32 exponent
// range, no scaling). A product A B with both operands split is evaluated as
// Ah Bh + Ah Bl + Al Bh in fp32 accumulation (the Al Bl term is below fp32 rounding
// of the result's bf16 part); with A exact it is A Bh + A Bl.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, wave64). A 16x16 fp32 accumulator tile
// ("C layout") puts rows 4g+i, i = 0..3, of column n in lane 16g+n. Operand slots
// s = 0..7 of lane 16g+n carry K index 8g+s of a 32-wide K block (A: row n, B:
// column n). So that the rows a lane owns in the two C tiles of a K block are
// exactly its eight K slots, every token-indexed (and d_k-indexed) C tile m holds the
// permuted rows
//   tok_of(m, r) = 32 (m / 2) + 8 (r / 4) + 4 (m % 2) + r % 4,   r = 0..15,
// i.e. tiles 2kb and 2kb+1 hold K block kb interleaved in groups of four. A
// accumulator tile pair then converts to the next product's B operand in registers,
// and A operands are 16 contiguous bytes of a row in natural order.
#pragma once

#include "fwmem_device.h"

namespace fwmem {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));

constexpr int kSplitTiles = 2;                  // 16-column value tiles of a propagate workgroup
constexpr int kSplitCols = 16 * kSplitTiles;    // value columns of a propagate workgroup
constexpr int kTriFrags = 6;                    // nonzero (m, kb) blocks of a 64x64 lower-triangular operand

__host__ __device__ constexpr int tok_of(int m, int r) {
  return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3);
}
// Lower-triangular fragment list: f -> (row tile m, K block kb), kb <= m / 2.
__host__ __device__ constexpr int tri_m(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__host__ __device__ constexpr int tri_kb(int f) { return f < 2 ? 0 : (f & 1); }

// Workspace record of one (head, chunk) for the split path.
template <int DK>
struct RecSplit {
  // T and M as A fragments, fragment f = 0..5: hi at 2f, lo at 2f+1, 1 KiB each
  // (lane-major, 16 bytes per lane).
  static constexpr size_t kT = 0;
  static constexpr size_t kM = kT + 2 * kTriFrags * 1024;
  // float [5][64]: per token fP, fV, fO, fU (the row factors of
  //   R = fV V - fP (X S),  O = fO (Q S) + M U,  S' = Gamma_C S + X^T (fU U)),
  // then [Gamma_C, has_prev, Gamma_C of the next chunk (1 after the last), 0...].
  static constexpr size_t kFac = kM + 2 * kTriFrags * 1024;
  static constexpr size_t kFacBytes = 5 * 64 * 4;
  // bf16 [DK]: the key feature that precedes the chunk's first token (chunk 0 only).
  static constexpr size_t kX0 = kFac + kFacBytes;
  static constexpr size_t kBytes = (kX0 + 2 * DK + 255) / 256 * 256;
};

// hi/lo split of eight fp32 values into two bf16 operand fragments.
__device__ __forceinline__ void split8(const float (&x)[8], bf8& hi, bf8& lo) {
  bf8 h;
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (__bf16)x[j];
  const u32x4 w = __builtin_bit_cast(u32x4, h);
  bf8 l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    l[2 * k] = (__bf16)(x[2 * k] - __uint_as_float(w[k] << 16));
    l[2 * k + 1] = (__bf16)(x[2 * k + 1] - __uint_as_float(w[k] & 0xffff0000u));
  }
  hi = h;
  lo = l;
}

// Operand fragment of K block kb from the C tiles c[2kb], c[2kb+1], split.
__device__ __forceinline__ void split_c(const f4* c, int kb, bf8& hi, bf8& lo) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = c[2 * kb][i];
    x[4 + i] = c[2 * kb + 1][i];
  }
  split8(x, hi, lo);
}

__device__ __forceinline__ void mma_bf16(f4& acc, const bf8& a, const bf8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// ---- LDS tiles and direct loads

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(3))) s4* lds_s4ptr;

// Granule slot of 16-byte granule cg in row `row` of a [CH][DK] bf16 tile is
// cg ^ xswz(row): conflict-free for both the row-fragment and the transpose reads.
template <int DK>
__device__ __forceinline__ int xswz(int row) {
  if constexpr (DK == 128) return ((row & 3) << 2) | ((row >> 3) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 3) & 3);
}
// Value tile [CH][32] bf16: four granules per row.
__device__ __forceinline__ int vswz(int row) { return (row >> 3) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct 16-byte-per-lane load into LDS. The destination is passed to the instruction
// as its 32-bit LDS offset (the low half of the generic address of an LDS object), which
// avoids a generic-to-local conversion with a null check for the object at offset 0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(uintptr_t)a, 16, voff, soff, 0, 0);
}

// ---- operand fragments in the K-slot order of split_c

// 16-byte buffer load: the hardware range check of the resource turns offsets past its
// end into zeros.
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Sign of a parity bit applied to x.
__device__ __forceinline__ float with_sign(float x, int parity) {
  return __int_as_float(__float_as_int(x) ^ (parity << 31));
}

// 8 bf16 values of an A fragment whose K slots are 4g..4g+3 and 16+4g..16+4g+3 of a 32-wide
// K block (the order split_c gives the B side): two 8-byte LDS reads at p and p + 16.
__device__ __forceinline__ bf8 frag_pair(const uint16_t* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
  return __builtin_bit_cast(bf8, u32x4{a.x, a.y, b.x, b.y});
}

// The same A fragment (K slots 4g..4g+3 and 16+4g..16+4g+3) of X^T, rows d_k 16 rt + n,
// K = tokens, from row-major token rows X by two LDS transpose reads. Within each group of
// 16 lanes, lane 4r + c points at 4 values of token row r, columns 4c..4c+3, and lane
// 4c + e receives column 4c + e of the four rows. `p` is this lane's address for the first
// four K slots (token 32 kq + 4g + (n >> 2), column 16 rt + 4 (n & 3)); the other four are
// 16 rows further on.
__device__ __forceinline__ bf8 xt_frag(const uint16_t* p, int ld) {
  typedef short s8v __attribute__((ext_vector_type(8)));
  const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(const void*)p);
  const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(const void*)(p + 16 * ld));
  const s8v r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf8, r);
}


}  // namespace fwmem
