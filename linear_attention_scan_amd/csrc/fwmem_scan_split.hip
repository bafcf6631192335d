// Split-operand propagate kernel of the chunked scan: bf16 inputs, identity feature
// map, scalar decay, delta or additive rule.
//
// Per chunk (the chunk algebra of fwmem_scan.hip, "Fast Weight Attention for
// Continual Learning" reading notes, sections 3.2 and 4.1-4.4):
//   R = diag(fV) V - diag(fP) (X S),   U = T R            (delta rule)
//   U = diag(fV) V                                        (additive rule)
//   O = diag(fO) (Q S) + M U,   S' = Gamma_C S + X^T diag(fU) U.
// One workgroup = one head and 32 value columns, in three waves. Each of the two compute
// waves keeps a 16-column slice of S (d_k x 16, fp32, MFMA C layout) in registers and
// walks the chunks in order. The third wave moves data: it brings X, Q, T, M, V and the
// row factors of chunk c+1 into LDS by direct global-to-LDS loads while chunk c computes
// (double-buffered), and stores chunk c-1's outputs, which the compute waves stage in
// LDS. One barrier per chunk separates the phases. X is stored once, row-major with an
// XOR swizzle; X^T operands are read from it with the LDS transpose read. All products
// run on bf16 MFMA with the split operands of fwmem_split.h.
#include "fwmem_internal.h"
#include "fwmem_split.h"

#include <type_traits>

namespace fwmem {
namespace {

constexpr int CH = kChunk;
constexpr int kLoader = kSplitWaves;          // index of the loader wave
constexpr int NTS = 64 * (kSplitWaves + 1);    // compute waves + one loader wave

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
  uint32_t neg0, neg1;   // the packed bf16 pairs (-1, 0) and (0, -1), in SGPRs (see split2)
};

// Buffer resources of one head's inputs and workspace records. Every direct load goes
// through one, with a loop-invariant lane offset and a per-chunk offset in an SGPR;
// the hardware range check turns rows past the sequence end into zeros in LDS.
struct Srcs {
  __amdgpu_buffer_rsrc_t x, q, v, w;
};

// Loop-invariant lane offsets of the loader wave's direct loads (bytes from the chunk's
// first row).
template <int DK>
struct LoadOffs {
  static constexpr int NGR = DK / 8;
  static constexpr int NXI = CH * NGR / 64;             // X (and Q) loads per chunk
  static constexpr int NVI = CH * kSplitCols / 8 / 64;  // value-tile loads per chunk
  uint32_t x[NXI];  // row * DK * 2 + 16 * granule
  uint32_t v[NVI];  // row * dv * 2 + 2 * (first column of the granule)
  uint32_t lane16;  // 16 * lane
};

template <int DK>
__device__ __forceinline__ LoadOffs<DK> load_offsets(int lane, int dv, int grp) {
  using LO = LoadOffs<DK>;
  constexpr int NGR = LO::NGR;
  LO o;
#pragma unroll
  for (int ii = 0; ii < LO::NXI; ++ii) {
    const int pos = 64 * ii + lane;
    const int row = pos / NGR;
    o.x[ii] = (uint32_t)(row * DK + 8 * ((pos % NGR) ^ xswz<DK>(row))) * 2u;
  }
#pragma unroll
  for (int ii = 0; ii < LO::NVI; ++ii) {
    const int pos = 64 * ii + lane;
    const int row = pos >> 2;
    o.v[ii] = (uint32_t)(row * dv + grp * kSplitCols + 8 * ((pos & 3) ^ vswz(row))) * 2u;
  }
  o.lane16 = (uint32_t)lane * 16u;
  return o;
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Output tiles of a chunk, staged in LDS by the compute waves for the loader wave:
// [chunk parity][compute wave][tile m][lane], in the MFMA C layout.
struct OutStage {
  f4 o[2][kSplitWaves][4][64];
};

// The loader's stores of chunk c's outputs from the stage: lane (g, n) writes rows
// tok_of(m, 4g+i) of column 16w + n of each compute wave w, through a buffer resource
// over the head's output rows (rows past the sequence end fall outside its range).
template <bool OBF>
__device__ __forceinline__ void store_staged(const OutStage& st, int c, int lane, int dv, int grp,
                                             __amdgpu_buffer_rsrc_t ro) {
  constexpr uint32_t es = OBF ? 2u : 4u;
  const int g = lane >> 4, n = lane & 15;
  static_for<0, kSplitWaves>([&](auto W) {
    const uint32_t vo = (uint32_t)(8 * g * dv + grp * kSplitCols + 16 * W + n) * es;
    static_for<0, 4>([&](auto M) {
      constexpr int m = M;
      const f4 v = st.o[c & 1][W][m][lane];
      static_for<0, 4>([&](auto I) {
        constexpr int i = I;
        const int r = c * CH + 32 * (m >> 1) + 4 * (m & 1) + i;
        const uint32_t so = (uint32_t)(r * dv) * es;
        if constexpr (OBF) {
          const __bf16 h = (__bf16)v[i];
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), ro, vo, so, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i]), ro, vo, so, 0);
        }
      });
    });
  });
}

// Direct loads of chunk c into B by the loader wave. For the delta rule the X resource
// starts one row early (x_t is the key before token t); the row before token 0 is
// forced out of range and patched from the record afterwards. Rows past the sequence
// end read as zeros.
template <int DK, bool DELTA>
__device__ __forceinline__ void issue_chunk(SplitBuf<DK, DELTA>& B, const ScanParams& p, int c, int lane,
                                            const LoadOffs<DK>& o, const Srcs& src) {
  using LO = LoadOffs<DK>;
  using RC = RecSplit<DK>;
  const uint32_t sx = (uint32_t)(c * CH * DK * 2);
  static_for<0, LO::NXI>([&](auto I) {
    constexpr int i = I;
    uint32_t xo = o.x[i];
    if (DELTA && c == 0 && 64 * i + lane < LO::NGR) xo = 0x80000000u;  // row 0 of chunk 0
    dma16(src.x, xo, sx, &B.x[64 * i]);
    dma16(src.q, o.x[i], sx, &B.q[64 * i]);
  });
  const uint32_t sw = (uint32_t)((size_t)c * RC::kBytes);
  if constexpr (DELTA) {
    static_for<0, 2 * kTriFrags>([&](auto J) {
      dma16(src.w, o.lane16, sw + (uint32_t)(RC::kT + J * 1024), &B.t[64 * J]);
    });
  }
  static_for<0, 2 * kTriFrags>([&](auto J) {
    dma16(src.w, o.lane16, sw + (uint32_t)(RC::kM + J * 1024), &B.m[64 * J]);
  });
  const uint32_t sv = (uint32_t)(c * CH * p.dv * 2);
  static_for<0, LO::NVI>([&](auto I) { dma16(src.v, o.v[I], sv, &B.v[64 * I]); });
  // row factors: 1280 bytes
  dma16(src.w, o.lane16, sw + (uint32_t)RC::kFac, &B.fac[0]);
  if (lane < 16) dma16(src.w, o.lane16, sw + (uint32_t)(RC::kFac + 1024), &B.fac[256]);
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations are
// complete before it arrives, and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One chunk for the loader wave: once the loads of chunk c (in B) have landed, patch in
// the carried key and release the chunk to the compute waves; then enqueue chunk c+1
// into N (free again: the compute waves finished chunk c-1 before the barrier) and
// store chunk c-1's outputs from the stage.
template <int DK, bool DELTA, bool OBF>
__device__ __forceinline__ void loader_step(SplitBuf<DK, DELTA>& B, SplitBuf<DK, DELTA>& N, const OutStage& st,
                                            const ScanParams& p, int c, int lane, const LoadOffs<DK>& o,
                                            const Srcs& src, const char* rec0, int grp,
                                            __amdgpu_buffer_rsrc_t ro) {
  constexpr int NGR = SplitBuf<DK, DELTA>::NGR;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (DELTA && c == 0 && lane < NGR) {
    // x_0 is the carried key (zero without one): row 0 of the first X tile
    B.x[lane ^ xswz<DK>(0)] = *reinterpret_cast<const u32x4*>(rec0 + RecSplit<DK>::kX0 + 16 * lane);
  }
  lds_barrier();
  if (c + 1 < p.nchunks) issue_chunk<DK, DELTA>(N, p, c + 1, lane, o, src);
  // chunk c-1's outputs were staged before the barrier
  if (c > 0) store_staged<OBF>(st, c - 1, lane, p.dv, grp, ro);
}

// ---------------------------------------------------------------- chunk step
// Scheduling. A single wave issues in order, so its matrix unit and its VALU only run
// at the same time if the instruction stream alternates between them. The chunk is
// therefore written as a sequence of micro-regions fenced by sched_barrier: each holds
// one MFMA plus a fixed share of the independent work (operand splits, row factors,
// LDS reads for later MFMAs, the next chunk's direct loads, the previous chunk's output
// stores), in the order given here.
#define FW_FENCE() __builtin_amdgcn_sched_barrier(0)


typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// hi/lo split of two fp32 values into one packed bf16 word each. hi is the packed
// rounding of the pair; each residual x - hi is one v_dot2c_f32_bf16 of the packed hi with
// the pair (-1, 0) or (0, -1), accumulated onto x: the products are exact and x - hi is
// representable in fp32, so the residual is exact, as a subtraction would give it, in two
// instructions instead of four. The two pairs must reach the instruction as registers:
// gfx950 reads an inline constant in a packed bf16 operand as a 32-bit float pattern, so
// -1.0 would arrive as the pair (0, -1), while the compiler assumes (-1, 0).
__device__ __forceinline__ void split2(float x0, float x1, const Lane& L, uint32_t& hi, uint32_t& lo) {
  const bf2 h = {(__bf16)x0, (__bf16)x1};
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2, L.neg0), x0, false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2, L.neg1), x1, false);
  const bf2 l = {(__bf16)r0, (__bf16)r1};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Word j (slots 2j, 2j+1) of the B fragment of K block kb from C tiles c[2kb], c[2kb+1].
template <int KB, int J>
__device__ __forceinline__ void split_word(const f4* c, const Lane& L, u32x4& hi, u32x4& lo) {
  constexpr int t = 2 * KB + (J >> 1), r = 2 * (J & 1);
  uint32_t h, l;
  split2(c[t][r], c[t][r + 1], L, h, l);
  hi[J] = h;
  lo[J] = l;
}
__device__ __forceinline__ void mma_w(f4& acc, const bf8& a, const u32x4& b) {
  mma_bf16(acc, a, __builtin_bit_cast(bf8, b));
}

// Even share [lo, hi) of N items for slot I of S slots.
template <int N, int S, int I>
struct Share {
  static constexpr int lo = N * I / S, hi = N * (I + 1) / S;
};

// One chunk for one compute wave: waits for chunk c in B, updates the state slice s and
// stages chunk c's outputs in st for the loader wave.
template <int DK, bool DELTA>
__device__ __forceinline__ void chunk_step(const SplitBuf<DK, DELTA>& B, OutStage& st, int c, const Lane& L,
                                           f4 (&s)[DK / 16]) {
  using Buf = SplitBuf<DK, DELTA>;
  constexpr int NGR = Buf::NGR;
  constexpr int NKD = DK / 32;       // K blocks over d_k
  constexpr int NRT = DK / 16;       // row tiles of S
  constexpr int NKH = NKD / 2;       // K blocks of the first half of Q S
  constexpr int NRH = NRT / 2;
  const int g = L.g, n = L.n;

  // the loader wave releases chunk c once its loads have landed; the compute waves have
  // finished with chunk c-1, so the loader may refill that buffer
  lds_barrier();

  auto fac4 = [&](int k, int m) -> f4 {
    return *reinterpret_cast<const f4*>(&B.fac[k * CH + tok_of(m, 4 * g)]);
  };
  auto xfrag = [&](const u32x4* X, int m, int kb) -> bf8 {
    const int row = tok_of(m, n);
    return __builtin_bit_cast(bf8, X[row * NGR + ((4 * kb + g) ^ xswz<DK>(row))]);
  };
  // Half hh of the X^T fragment (rt, kb): rows d_k tok_of(rt, n), K slots 4hh..4hh+3 =
  // tokens 32kb + 8g + 4hh + j, by one transpose read of the row-major X tile.
  auto xthalf = [&](int rt, int kb, int hh) -> s4 {
    const int dk0 = 32 * (rt >> 1) + 8 * (n & 3) + 4 * (rt & 1);
    const int row = 32 * kb + 8 * g + (n >> 2) + 4 * hh;
    const char* a = reinterpret_cast<const char*>(&B.x[row * NGR + ((dk0 >> 3) ^ xswz<DK>(row))]) +
                    (dk0 & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)a);
  };
  auto xtjoin = [](const s4& a, const s4& b) -> bf8 {
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf8, r);
  };
  // Values of the lane's four rows tok_of(m, 4g+i), i = 0..3 (consecutive tokens), in its
  // column: one transpose read, in which lane 4i+q of the group supplies columns
  // 4q..4q+3 of token row i.
  auto vrows = [&](int m) -> s4 {
    const int row = tok_of(m, 4 * g) + (n >> 2);
    const int c0 = L.wave * 16 + 4 * (n & 3);
    const char* a = reinterpret_cast<const char*>(&B.v[row * 4 + ((c0 >> 3) ^ vswz(row))]) + (c0 & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)a);
  };
  auto vf = [](const s4& h, int i) { return bf16_bits_to_f32((uint32_t)(uint16_t)h[i]); };
  auto tfrag = [&](const u32x4* T, int f, int part) -> bf8 {
    return __builtin_bit_cast(bf8, T[(2 * f + part) * 64 + L.lane]);
  };

  // ---- A: X fragments, value rows and their factors; split of S's first K block
  bf8 xf[4][NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
    for (int m = 0; m < 4; ++m) xf[m][kb] = xfrag(B.x, m, kb);
  s4 vv[4];
  f4 fvr[4], fpr[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    vv[m] = vrows(m);
    fvr[m] = fac4(1, m);
    if (DELTA) fpr[m] = fac4(0, m);
  }
  // The split of S also forms acc = Gamma_C S, the accumulator of the state update, so
  // that the split may overwrite S.
  const float gC = B.fac[4 * CH];
  f4 acc[NRT];
  u32x4 Sh[NKD], Sl[NKD];
  auto split_s = [&](auto KB, auto J) {
    constexpr int kb = KB, j = J, t = 2 * kb + (j >> 1), r = 2 * (j & 1);
    acc[t][r] = s[t][r] * gC;
    acc[t][r + 1] = s[t][r + 1] * gC;
    split_word<kb, j>(s, L, Sh[kb], Sl[kb]);
  };
  static_for<0, 4>([&](auto J) { split_s(std::integral_constant<int, 0>{}, J); });
  FW_FENCE();

  // ---- B: P = X S (8 NKD MFMAs; the additive rule has none and keeps only the side
  // work). Alongside: the split of S's K blocks 1.., the next chunk's X and Q loads, the
  // previous chunk's output stores, the first half of the Q fragments.
  f4 P[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) P[m] = f4{0.f, 0.f, 0.f, 0.f};
  bf8 qf[4][NKD];
  constexpr int NB = 8 * NKD;
  constexpr int NC = 8 * NKH;
  constexpr int ND = DELTA ? 3 * kTriFrags : 1;
  static_for<0, NB>([&](auto I) {
    constexpr int i = I, kb = i / 8, m = (i % 8) / 2, part = i % 2;
    if constexpr (DELTA) mma_w(P[m], xf[m][kb], part ? Sl[kb] : Sh[kb]);
    FW_FENCE();
    if constexpr (kb + 1 < NKD && part == 0)
      split_s(std::integral_constant<int, kb + 1>{}, std::integral_constant<int, m>{});
    static_for<Share<4 * NKH, NB, i>::lo, Share<4 * NKH, NB, i>::hi>([&](auto K) {
      qf[K % 4][K / 4] = xfrag(B.q, K % 4, K / 4);
    });
    FW_FENCE();
  });

  // ---- C: first half of Q S. Alongside: R = fV V - fP P and its split (delta rule) or
  // U = fV V (additive); the second half of the Q fragments and the T fragments.
  f4 Oq[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) Oq[m] = f4{0.f, 0.f, 0.f, 0.f};
  f4 U[4];
  u32x4 Rh[2], Rl[2];
  bf8 th[kTriFrags], tl[kTriFrags];
  // side work items: 16 row values (4 per tile) interleaved with the 8 split words, in
  // dependency order (tiles 0,1 -> words of K block 0 -> tiles 2,3 -> words of block 1)
  constexpr int NCV = DELTA ? 24 : 16;
  constexpr int NCD = 4 * (NKD - NKH) + (DELTA ? 2 * kTriFrags : 0);
  static_for<0, NC>([&](auto I) {
    constexpr int i = I, kb = i / 8, m = (i % 8) / 2, part = i % 2;
    mma_w(Oq[m], qf[m][kb], part ? Sl[kb] : Sh[kb]);
    FW_FENCE();
    static_for<Share<NCV, NC, i>::lo, Share<NCV, NC, i>::hi>([&](auto K) {
      constexpr int k = K;
      if constexpr (DELTA) {
        constexpr int grp = k / 12, w = k % 12;  // 12 items per K block: 8 values, 4 words
        if constexpr (w < 8) {
          constexpr int t = 2 * grp + w / 4, r = w % 4;
          P[t][r] = fvr[t][r] * vf(vv[t], r) - fpr[t][r] * P[t][r];
        } else {
          split_word<grp, w - 8>(P, L, Rh[grp], Rl[grp]);
        }
      } else {
        constexpr int t = k / 4, r = k % 4;
        U[t][r] = fvr[t][r] * vf(vv[t], r);
      }
    });
    static_for<Share<NCD, NC, i>::lo, Share<NCD, NC, i>::hi>([&](auto K) {
      constexpr int k = K;
      if constexpr (k < 4 * (NKD - NKH)) {
        qf[k % 4][NKH + k / 4] = xfrag(B.q, k % 4, NKH + k / 4);
      } else {
        constexpr int f = (k - 4 * (NKD - NKH)) / 2, part = (k - 4 * (NKD - NKH)) % 2;
        if constexpr (part == 0) th[f] = tfrag(B.t, f, 0);
        else tl[f] = tfrag(B.t, f, 1);
      }
    });
    FW_FENCE();
  });

  // ---- D: U = T R (delta rule: 18 MFMAs). Alongside: the next chunk's other loads, the
  // factors of O and W, the M fragments.
  f4 for_[4], fur[4];
  bf8 mh[kTriFrags], ml[kTriFrags];
  constexpr int NDD = 8 + 2 * kTriFrags;
  if constexpr (DELTA) {
#pragma unroll
    for (int m = 0; m < 4; ++m) U[m] = f4{0.f, 0.f, 0.f, 0.f};
  }
  static_for<0, ND>([&](auto I) {
    constexpr int i = I, f = i / 3, part = i % 3;
    if constexpr (DELTA) {
      constexpr int m = tri_m(f), kb = tri_kb(f);
      if constexpr (part == 0) mma_w(U[m], th[f], Rh[kb]);
      else if constexpr (part == 1) mma_w(U[m], th[f], Rl[kb]);
      else mma_w(U[m], tl[f], Rh[kb]);
    }
    FW_FENCE();
    static_for<Share<NDD, ND, i>::lo, Share<NDD, ND, i>::hi>([&](auto K) {
      constexpr int k = K;
      if constexpr (k < 4) for_[k] = fac4(2, k);
      else if constexpr (k < 8) fur[k - 4] = fac4(3, k - 4);
      else {
        constexpr int f = (k - 8) / 2, part = (k - 8) % 2;
        if constexpr (part == 0) mh[f] = tfrag(B.m, f, 0);
        else ml[f] = tfrag(B.m, f, 1);
      }
    });
    FW_FENCE();
  });

  // ---- E: second half of Q S. Alongside: W = fU U, then the split of U (which may then
  // overwrite U); O's Q S part scaled by fO as each tile completes; the first half of the
  // X^T fragments.
  u32x4 Uh[2], Ul[2];
  f4 Wt[4];
  f4 Om[4];
  s4 xth[NRT][2][2];
  constexpr int NE = 8 * (NKD - NKH);
  constexpr int NED = 4 * NRH;  // transpose reads
  static_for<0, NE>([&](auto I) {
    constexpr int i = I, kb = NKH + i / 8, m = (i % 8) / 2, part = i % 2;
    mma_w(Oq[m], qf[m][kb], part ? Sl[kb] : Sh[kb]);
    FW_FENCE();
    static_for<Share<8, NE, i>::lo, Share<8, NE, i>::hi>([&](auto K) {
      constexpr int t = 2 * (K / 4) + ((K % 4) >> 1), r = 2 * ((K % 4) & 1);
      Wt[t][r] = U[t][r] * fur[t][r];
      Wt[t][r + 1] = U[t][r + 1] * fur[t][r + 1];
      split_word<K / 4, K % 4>(U, L, Uh[K / 4], Ul[K / 4]);
    });
    // the last K block's MFMAs for tile m are i = NE - 8 + 2m, +1; scale two slots later
    if constexpr (i >= NE - 8 + 3 && ((i - (NE - 8 + 3)) % 2) == 0) {
      constexpr int mm = (i - (NE - 8 + 3)) / 2;
      Om[mm] = Oq[mm] * for_[mm];
    }
    static_for<Share<NED, NE, i>::lo, Share<NED, NE, i>::hi>([&](auto K) {
      constexpr int k = K, rt = k / 4, kb = (k / 2) % 2, hh = k % 2;
      xth[rt][kb][hh] = xthalf(rt, kb, hh);
    });
    FW_FENCE();
  });
  Om[3] = Oq[3] * for_[3];

  // ---- F: O += M U (18 MFMAs). Alongside: the split of W; the second half of the X^T
  // fragments.
  u32x4 Wh[2], Wl[2];
  constexpr int NF = 3 * kTriFrags;
  constexpr int NFD = 4 * (NRT - NRH);
  static_for<0, NF>([&](auto I) {
    constexpr int i = I, f = i / 3, part = i % 3;
    constexpr int m = tri_m(f), kb = tri_kb(f);
    if constexpr (part == 0) mma_w(Om[m], mh[f], Uh[kb]);
    else if constexpr (part == 1) mma_w(Om[m], mh[f], Ul[kb]);
    else mma_w(Om[m], ml[f], Uh[kb]);
    FW_FENCE();
    static_for<Share<8, NF, i>::lo, Share<8, NF, i>::hi>([&](auto K) {
      split_word<K / 4, K % 4>(Wt, L, Wh[K / 4], Wl[K / 4]);
    });
    static_for<Share<NFD, NF, i>::lo, Share<NFD, NF, i>::hi>([&](auto K) {
      constexpr int k = K, rt = NRH + k / 4, kb = (k / 2) % 2, hh = k % 2;
      xth[rt][kb][hh] = xthalf(rt, kb, hh);
    });
    FW_FENCE();
  });

  // ---- G: S' = Gamma_C S + X^T W (4 NRT MFMAs onto acc)
  constexpr int NG = 4 * NRT;
  static_for<0, NG>([&](auto I) {
    constexpr int i = I, rt = i / 4, kb = (i % 4) / 2, part = i % 2;
    mma_w(acc[rt], xtjoin(xth[rt][kb][0], xth[rt][kb][1]), part ? Wl[kb] : Wh[kb]);
    FW_FENCE();
  });
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) s[rt] = acc[rt];
#pragma unroll
  for (int m = 0; m < 4; ++m) st.o[c & 1][L.wave][m][L.lane] = Om[m];
}

template <int DK, bool DELTA, bool OBF>
__global__ __launch_bounds__(NTS) void prop_split_kernel(ScanParams p) {
  using Buf = SplitBuf<DK, DELTA>;
  constexpr int NRT = DK / 16;
  __shared__ Buf B0, B1;
  __shared__ OutStage st;

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
  // opaque moves keep the two pairs out of inline-constant folding
  asm volatile("s_mov_b32 %0, 0xbf80" : "=s"(L.neg0));
  asm volatile("s_mov_b32 %0, 0xbf800000" : "=s"(L.neg1));
  const int dv = p.dv;
  const size_t rowbase = (size_t)bh * p.T;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q) + rowbase * DK;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v) + rowbase * dv;
  const char* rec0 = p.ws + (size_t)bh * p.nchunks * RecSplit<DK>::kBytes;
  constexpr uint32_t oes = OBF ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(static_cast<const char*>(p.out) + rowbase * dv * oes, (uint32_t)(p.T * dv) * oes);
  const int col = grp * kSplitCols + L.wave * 16 + L.n;  // this lane's value column
  if (L.wave == kLoader) {
    // loader wave: one barrier per chunk, like the compute waves
    const LoadOffs<DK> lo = load_offsets<DK>(L.lane, dv, grp);
    Srcs src;
    src.x = rsrc(DELTA ? kb - DK : kb, (uint32_t)(p.T * DK * 2));
    src.q = rsrc(qb, (uint32_t)(p.T * DK * 2));
    src.v = rsrc(vb, (uint32_t)(p.T * dv * 2));
    src.w = rsrc(rec0, (uint32_t)((size_t)p.nchunks * RecSplit<DK>::kBytes));
    issue_chunk<DK, DELTA>(B0, p, 0, L.lane, lo, src);
    for (int c = 0; c < p.nchunks; c += 2) {
      loader_step<DK, DELTA, OBF>(B0, B1, st, p, c, L.lane, lo, src, rec0, grp, ro);
      if (c + 1 < p.nchunks) loader_step<DK, DELTA, OBF>(B1, B0, st, p, c + 1, L.lane, lo, src, rec0, grp, ro);
    }
    lds_barrier();  // the last chunk's outputs are staged
    store_staged<OBF>(st, p.nchunks - 1, L.lane, dv, grp, ro);
    if (p.S_out != nullptr && grp == 0) {
      for (int i = L.lane; i < DK; i += 64)
        p.xprev_out[(size_t)bh * DK + i] = bf16_bits_to_f32(kb[(uint32_t)((p.T - 1) * DK + i)]);
      if (L.lane == 0) p.has_out[bh] = 1;
    }
    return;
  }

  f4 s[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] : 0.f;

  for (int c = 0; c < p.nchunks; c += 2) {
    chunk_step<DK, DELTA>(B0, st, c, L, s);
    if (c + 1 < p.nchunks) chunk_step<DK, DELTA>(B1, st, c + 1, L, s);
  }
  lds_barrier();  // hand the last chunk's outputs to the loader

  if (p.S_out != nullptr) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.S_out[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] = s[rt][i];
  }
}

template <int DK, bool DELTA>
hipError_t launch_t(const ScanParams& p, hipStream_t st) {
  const int ngrp = p.dv / kSplitCols;
  const unsigned grid = (unsigned)(8 * ngrp * ((p.BH + 7) / 8));
  if (p.flags & kFlagOutBf16)
    hipLaunchKernelGGL((prop_split_kernel<DK, DELTA, true>), dim3(grid), dim3(NTS), 0, st, p);
  else
    hipLaunchKernelGGL((prop_split_kernel<DK, DELTA, false>), dim3(grid), dim3(NTS), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prop_split(const ScanParams& p, hipStream_t st) {
  if (p.dk == 64) return p.delta ? launch_t<64, true>(p, st) : launch_t<64, false>(p, st);
  return p.delta ? launch_t<128, true>(p, st) : launch_t<128, false>(p, st);
}

}  // namespace fwmem
