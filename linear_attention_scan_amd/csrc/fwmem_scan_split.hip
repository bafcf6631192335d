// Split-operand propagate kernel of the chunked scan: bf16 inputs, identity feature
// map, scalar decay, delta or additive rule.
//
// Per chunk (the chunk algebra of fwmem_scan.hip, "Fast Weight Attention for
// Continual Learning" reading notes, sections 3.2 and 4.1-4.4):
//   R = diag(fV) V - diag(fP) (X S),   U = T R            (delta rule)
//   U = diag(fV) V                                        (additive rule)
//   O = diag(fO) (Q S) + M U,   S' = Gamma_C S + X^T diag(fU) U.
// One workgroup = 2 waves = one head and 32 value columns; each wave keeps a 16-column
// slice of S (d_k x 16, fp32, MFMA C layout) in registers and walks the chunks in
// order. X, Q, T, M, V and the row factors of a chunk are brought into LDS by direct
// global-to-LDS loads, double-buffered: the loads of chunk c+1 are in flight while
// chunk c computes, and one barrier per chunk separates the two. X is stored once,
// row-major with an XOR swizzle; X^T operands are read from it with the LDS transpose
// read. All products run on bf16 MFMA with the split operands of fwmem_split.h.
#include "fwmem_internal.h"
#include "fwmem_split.h"

namespace fwmem {
namespace {

constexpr int CH = kChunk;
constexpr int NTS = 64 * kSplitWaves;

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

template <int DK, bool DELTA>
struct SplitBuf {
  static constexpr int NGR = DK / 8;  // granules per X / Q row
  u32x4 x[CH * NGR];
  u32x4 q[CH * NGR];
  u32x4 t[DELTA ? 2 * kTriFrags * 64 : 1];
  u32x4 m[2 * kTriFrags * 64];
  u32x4 v[CH * kSplitCols / 8];
  float fac[5 * CH];
};

struct Lane {
  int lane, wave, g, n;  // wave is wave-uniform (an SGPR)
};

// Buffer resources of one head's inputs and workspace records. Every direct load goes
// through one, with a loop-invariant lane offset and a per-chunk offset in an SGPR;
// the hardware range check turns rows past the sequence end into zeros in LDS.
struct Srcs {
  __amdgpu_buffer_rsrc_t x, q, v, w;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds, 16, voff, soff, 0, 0);
}

// Loop-invariant lane offsets of the direct loads (bytes from the chunk's first row).
template <int DK>
struct LoadOffs {
  static constexpr int NGR = DK / 8;
  static constexpr int NXI = CH * NGR / 64 / kSplitWaves;  // X (and Q) loads per wave
  static constexpr int NVI = CH * kSplitCols / 8 / 64 / kSplitWaves;
  uint32_t x[NXI];  // row * DK * 2 + 16 * granule
  uint32_t v[NVI];  // row * dv * 2 + 2 * (first column of the granule)
  uint32_t lane16;  // 16 * lane
};

template <int DK>
__device__ __forceinline__ LoadOffs<DK> load_offsets(const Lane& L, int dv, int grp) {
  using LO = LoadOffs<DK>;
  constexpr int NGR = LO::NGR;
  LO o;
#pragma unroll
  for (int ii = 0; ii < LO::NXI; ++ii) {
    const int pos = 64 * (ii * kSplitWaves + L.wave) + L.lane;
    const int row = pos / NGR;
    o.x[ii] = (uint32_t)(row * DK + 8 * ((pos % NGR) ^ xswz<DK>(row))) * 2u;
  }
#pragma unroll
  for (int ii = 0; ii < LO::NVI; ++ii) {
    const int pos = 64 * (ii * kSplitWaves + L.wave) + L.lane;
    const int row = pos >> 2;
    o.v[ii] = (uint32_t)(row * dv + grp * kSplitCols + 8 * ((pos & 3) ^ vswz(row))) * 2u;
  }
  o.lane16 = (uint32_t)L.lane * 16u;
  return o;
}

// Enqueue the direct loads of chunk c into B (every thread of the workgroup). For the
// delta rule the X resource starts one row early (x_t is the key before token t); the
// row before token 0 is forced out of range and patched from the record later.
template <int DK, bool DELTA>
__device__ __forceinline__ void issue_chunk(SplitBuf<DK, DELTA>& B, const ScanParams& p, int c,
                                            const Lane& L, const LoadOffs<DK>& o, const Srcs& src) {
  using LO = LoadOffs<DK>;
  using RC = RecSplit<DK>;
  const uint32_t sx = (uint32_t)(c * CH * DK * 2);
#pragma unroll
  for (int ii = 0; ii < LO::NXI; ++ii) {
    const int i = ii * kSplitWaves + L.wave;
    uint32_t xo = o.x[ii];
    if (DELTA && c == 0 && 64 * i + L.lane < LO::NGR) xo = 0x80000000u;  // row 0 of chunk 0
    dma16(src.x, xo, sx, &B.x[64 * i]);
    dma16(src.q, o.x[ii], sx, &B.q[64 * i]);
  }
  const uint32_t sw = (uint32_t)((size_t)c * RC::kBytes);
  if constexpr (DELTA) {
#pragma unroll
    for (int jj = 0; jj < 2 * kTriFrags / kSplitWaves; ++jj) {
      const int j = jj * kSplitWaves + L.wave;
      dma16(src.w, o.lane16, sw + (uint32_t)(RC::kT + j * 1024), &B.t[64 * j]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < 2 * kTriFrags / kSplitWaves; ++jj) {
    const int j = jj * kSplitWaves + L.wave;
    dma16(src.w, o.lane16, sw + (uint32_t)(RC::kM + j * 1024), &B.m[64 * j]);
  }
  const uint32_t sv = (uint32_t)(c * CH * p.dv * 2);
#pragma unroll
  for (int ii = 0; ii < LO::NVI; ++ii) {
    const int i = ii * kSplitWaves + L.wave;
    dma16(src.v, o.v[ii], sv, &B.v[64 * i]);
  }
  // row factors: 1280 bytes
  if (L.wave == 0) dma16(src.w, o.lane16, sw + (uint32_t)RC::kFac, &B.fac[0]);
  else if (L.lane < 16) dma16(src.w, o.lane16, sw + (uint32_t)(RC::kFac + 1024), &B.fac[256]);
}

// One chunk for one wave: updates the state slice s and produces the outputs O.
template <int DK, bool DELTA>
__device__ __forceinline__ void compute_chunk(const SplitBuf<DK, DELTA>& B, const Lane& L,
                                              f4 (&s)[DK / 16], f4 (&O)[4]) {
  using Buf = SplitBuf<DK, DELTA>;
  constexpr int NGR = Buf::NGR;
  constexpr int NKD = DK / 32;
  constexpr int NRT = DK / 16;
  const int g = L.g, n = L.n;

  auto fac4 = [&](int k, int m) -> f4 {
    return *reinterpret_cast<const f4*>(&B.fac[k * CH + tok_of(m, 4 * g)]);
  };
  auto xfrag = [&](const u32x4* X, int m, int kb) -> bf8 {
    const int row = tok_of(m, n);
    return __builtin_bit_cast(bf8, X[row * NGR + ((4 * kb + g) ^ xswz<DK>(row))]);
  };
  // X^T fragment: rows d_k tok_of(rt, n), K = tokens 32kb + 8g + s, from the row-major X
  // tile; each transpose read gives four consecutive K slots.
  auto xtfrag = [&](int rt, int kb) -> bf8 {
    s4 h[2];
    const int dk0 = 32 * (rt >> 1) + 8 * (n & 3) + 4 * (rt & 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 32 * kb + 8 * g + (n >> 2) + 4 * hh;
      const char* a = reinterpret_cast<const char*>(&B.x[row * NGR + ((dk0 >> 3) ^ xswz<DK>(row))]) +
                      (dk0 & 7) * 2;
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)a);
    }
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 r = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf8, r);
  };
  auto vval = [&](int m, int i) -> float {
    const int row = tok_of(m, 4 * g + i);
    const int vc = L.wave * 16 + n;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(&B.v[row * 4 + ((vc >> 3) ^ vswz(row))]);
    return bf16_bits_to_f32(vp[vc & 7]);
  };

  bf8 Sh[NKD], Sl[NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb) split_c(s, kb, Sh[kb], Sl[kb]);

  f4 U[4];
  if constexpr (DELTA) {
    f4 P[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      P[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        const bf8 a = xfrag(B.x, m, kb);
        mma_bf16(P[m], a, Sh[kb]);
        mma_bf16(P[m], a, Sl[kb]);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f4 fv = fac4(1, m), fp = fac4(0, m);
#pragma unroll
      for (int i = 0; i < 4; ++i) P[m][i] = fv[i] * vval(m, i) - fp[i] * P[m][i];
    }
    bf8 Rh[2], Rl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_c(P, kb, Rh[kb], Rl[kb]);
#pragma unroll
    for (int m = 0; m < 4; ++m) U[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) {
      const int m = tri_m(f), kb = tri_kb(f);
      const bf8 th = __builtin_bit_cast(bf8, B.t[(2 * f) * 64 + L.lane]);
      const bf8 tl = __builtin_bit_cast(bf8, B.t[(2 * f + 1) * 64 + L.lane]);
      mma_bf16(U[m], th, Rh[kb]);
      mma_bf16(U[m], th, Rl[kb]);
      mma_bf16(U[m], tl, Rh[kb]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f4 fv = fac4(1, m);
#pragma unroll
      for (int i = 0; i < 4; ++i) U[m][i] = fv[i] * vval(m, i);
    }
  }

  // O = diag(fO) Q S + M U
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
      const bf8 a = xfrag(B.q, m, kb);
      mma_bf16(acc, a, Sh[kb]);
      mma_bf16(acc, a, Sl[kb]);
    }
    O[m] = acc * fac4(2, m);
  }
  {
    bf8 Uh[2], Ul[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_c(U, kb, Uh[kb], Ul[kb]);
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) {
      const int m = tri_m(f), kb = tri_kb(f);
      const bf8 mh = __builtin_bit_cast(bf8, B.m[(2 * f) * 64 + L.lane]);
      const bf8 ml = __builtin_bit_cast(bf8, B.m[(2 * f + 1) * 64 + L.lane]);
      mma_bf16(O[m], mh, Uh[kb]);
      mma_bf16(O[m], mh, Ul[kb]);
      mma_bf16(O[m], ml, Uh[kb]);
    }
  }

  // S' = Gamma_C S + X^T diag(fU) U
#pragma unroll
  for (int m = 0; m < 4; ++m) U[m] *= fac4(3, m);
  bf8 Wh[2], Wl[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) split_c(U, kb, Wh[kb], Wl[kb]);
  const float gC = B.fac[4 * CH];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    f4 acc = s[rt] * gC;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf8 a = xtfrag(rt, kb);
      mma_bf16(acc, a, Wh[kb]);
      mma_bf16(acc, a, Wl[kb]);
    }
    s[rt] = acc;
  }
}

// Outputs of chunk c: lane rows tok_of(m, 4g+i) of column col, through a buffer resource
// over the head's output rows (stores past the sequence end fall outside its range).
template <bool BF>
__device__ __forceinline__ void store_rows(int dv, const f4 (&O)[4], int c, __amdgpu_buffer_rsrc_t ro,
                                           uint32_t olofs) {
  constexpr uint32_t es = BF ? 2u : 4u;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = c * CH + 32 * (m >> 1) + 4 * (m & 1) + i;  // uniform part of the row
      const uint32_t so = (uint32_t)(r * dv) * es;
      if constexpr (BF) {
        const __bf16 h = (__bf16)O[m][i];
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), ro, olofs * es, so, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[m][i]), ro, olofs * es, so, 0);
      }
    }
}

__device__ __forceinline__ void store_out(const ScanParams& p, const f4 (&O)[4], int c,
                                          __amdgpu_buffer_rsrc_t ro, uint32_t olofs) {
  if ((p.flags & kFlagOutBf16) != 0) store_rows<true>(p.dv, O, c, ro, olofs);
  else store_rows<false>(p.dv, O, c, ro, olofs);
}

template <int DK, bool DELTA>
__device__ __forceinline__ void run_chunk(SplitBuf<DK, DELTA>& cur, SplitBuf<DK, DELTA>& nxt,
                                          const ScanParams& p, int c, const Lane& L, f4 (&s)[DK / 16],
                                          f4 (&O)[4], const LoadOffs<DK>& lo, const Srcs& src,
                                          const char* rec0, __amdgpu_buffer_rsrc_t ro, uint32_t olofs) {
  // this chunk's loads (and the previous chunk's output stores) have completed in
  // every wave once all waves pass the barrier; the other buffer is free again
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (DELTA && c == 0) {
    // x_0 is the carried key (zero without one): overwrite row 0 of the first X tile
    constexpr int NGR = SplitBuf<DK, DELTA>::NGR;
    if (threadIdx.x < NGR) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(rec0 + RecSplit<DK>::kX0 + 16 * threadIdx.x);
      cur.x[threadIdx.x ^ xswz<DK>(0)] = w;
    }
    __syncthreads();
  }
  if (c + 1 < p.nchunks) issue_chunk<DK, DELTA>(nxt, p, c + 1, L, lo, src);
  if (c > 0) store_out(p, O, c - 1, ro, olofs);
  compute_chunk<DK, DELTA>(cur, L, s, O);
}

template <int DK, bool DELTA>
__global__ __launch_bounds__(NTS) void prop_split_kernel(ScanParams p) {
  using Buf = SplitBuf<DK, DELTA>;
  constexpr int NRT = DK / 16;
  __shared__ Buf B0, B1;

  // workgroup -> (head, column group); the groups of a head share an XCD and its L2
  const int ngrp = p.dv / kSplitCols;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int grp = __builtin_amdgcn_readfirstlane(slot % ngrp);
  const int bh = __builtin_amdgcn_readfirstlane((slot / ngrp) * 8 + xcd);
  if (bh >= p.BH) return;

  Lane L;
  L.lane = threadIdx.x & 63;
  L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  L.g = L.lane >> 4;
  L.n = L.lane & 15;
  const int dv = p.dv;
  const size_t rowbase = (size_t)bh * p.T;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q) + rowbase * DK;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v) + rowbase * dv;
  const char* rec0 = p.ws + (size_t)bh * p.nchunks * RecSplit<DK>::kBytes;
  const uint32_t oes = (p.flags & kFlagOutBf16) != 0 ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(static_cast<const char*>(p.out) + rowbase * dv * oes, (uint32_t)(p.T * dv) * oes);
  const int col = grp * kSplitCols + L.wave * 16 + L.n;  // this lane's value column
  const uint32_t olofs = (uint32_t)(8 * L.g * dv + col);  // lane part of an output offset
  const LoadOffs<DK> lo = load_offsets<DK>(L, dv, grp);
  Srcs src;
  src.x = rsrc(DELTA ? kb - DK : kb, (uint32_t)(p.T * DK * 2));
  src.q = rsrc(qb, (uint32_t)(p.T * DK * 2));
  src.v = rsrc(vb, (uint32_t)(p.T * dv * 2));
  src.w = rsrc(rec0, (uint32_t)((size_t)p.nchunks * RecSplit<DK>::kBytes));

  f4 s[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] : 0.f;

  f4 O[4];
  issue_chunk<DK, DELTA>(B0, p, 0, L, lo, src);
  for (int c = 0; c < p.nchunks; c += 2) {
    run_chunk<DK, DELTA>(B0, B1, p, c, L, s, O, lo, src, rec0, ro, olofs);
    if (c + 1 < p.nchunks) run_chunk<DK, DELTA>(B1, B0, p, c + 1, L, s, O, lo, src, rec0, ro, olofs);
  }
  store_out(p, O, p.nchunks - 1, ro, olofs);

  if (p.S_out != nullptr) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.S_out[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] = s[rt][i];
    if (grp == 0) {
      for (int i = threadIdx.x; i < DK; i += NTS)
        p.xprev_out[(size_t)bh * DK + i] = bf16_bits_to_f32(kb[(uint32_t)((p.T - 1) * DK + i)]);
      if (threadIdx.x == 0) p.has_out[bh] = 1;
    }
  }
}

template <int DK, bool DELTA>
hipError_t launch_t(const ScanParams& p, hipStream_t st) {
  const int ngrp = p.dv / kSplitCols;
  const unsigned grid = (unsigned)(8 * ngrp * ((p.BH + 7) / 8));
  hipLaunchKernelGGL((prop_split_kernel<DK, DELTA>), dim3(grid), dim3(NTS), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prop_split(const ScanParams& p, hipStream_t st) {
  if (p.dk == 64) return p.delta ? launch_t<64, true>(p, st) : launch_t<64, false>(p, st);
  return p.delta ? launch_t<128, true>(p, st) : launch_t<128, false>(p, st);
}

}  // namespace fwmem
