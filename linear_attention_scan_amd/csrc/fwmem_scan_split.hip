// Split-operand propagate kernel of the chunked scan: bf16 inputs, identity feature
// map, scalar decay; delta, additive or inner-product rule.
//
// Per chunk (the chunk algebra of fwmem_scan.hip, "Fast Weight Attention for
// Continual Learning" reading notes, sections 3.2 and 4.1-4.4):
//   R = diag(fV) V - diag(fP) (X S),   U = T R            (delta rule)
//   U = diag(fV) V                     (additive and inner-product rules; fV = eta for
//                                       the inner-product rule, the write scale beta
//                                       for the additive one)
//   O = diag(fO) (Q S) + M U,   S' = Gamma_C S + X^T diag(fU) U.
//
// One workgroup = one head and 32 value columns (two 16-column tiles), in five waves.
// For each tile, an alpha wave carries the state: it keeps the tile's slice of S
// (d_k x 16, fp32, MFMA C layout) in registers and computes X S, R, U = T R, W = fU U,
// the state update and the split of the new state. A beta wave computes the tile's
// outputs: Q S from the split state that alpha leaves in LDS, then M U from the U that
// alpha hands over in the middle of the chunk, and stores them. One CU's four SIMDs each
// run one of the four compute waves: the state chain, whose MFMAs and VALU work cannot
// overlap much within one wave, loses the output products to a wave of its own.
//
// The fifth wave moves data: it brings X, Q, T, M, V and the row factors of chunk c+1
// into LDS by direct global-to-LDS loads while chunk c computes (double-buffered). One
// barrier per chunk separates the phases. X is stored once, row-major with an XOR
// swizzle; X^T operands are read from it with the LDS transpose read. All products run
// on bf16 MFMA with the split operands of fwmem_split.h.
//
// Hand-offs inside a chunk period (LDS, one slot per tile):
//   * the split of the state that chunk c reads: written by alpha at the end of period
//     c-1 (before the barrier), read by beta at the start of period c. Beta raises
//     sflag = c+1 once it has the values, and alpha waits for that before it writes the
//     next split;
//   * U of chunk c: written by alpha in period c, then uflag = c+1; beta waits for the
//     flag. Beta has read U before the next barrier, after which alpha may write again.
// Each flag is written once per period by one wave and polled by the other, with a poll
// limit that bounds every wait.
#include "fwmem_internal.h"
#include "fwmem_split.h"

#include <mutex>
#include <type_traits>

namespace fwmem {
namespace {

constexpr int CH = kChunk;
constexpr int kLoader = 2 * kSplitTiles;       // index of the loader wave
constexpr int NTS = 64 * (2 * kSplitTiles + 1);

template <int DK, bool SOLVE>
struct SplitBuf {
  static constexpr int NGR = DK / 8;  // granules per X / Q row
  u32x4 x[CH * NGR];
  u32x4 q[CH * NGR];
  u32x4 t[SOLVE ? 2 * kTriFrags * 64 : 1];
  u32x4 m[2 * kTriFrags * 64];
  u32x4 v[CH * kSplitCols / 8];
  float fac[5 * CH];
};

// Alpha-to-beta hand-offs of one workgroup (see the file comment).
template <int DK>
struct Handoff {
  u32x4 s[kSplitTiles][2 * (DK / 32)][64];  // split state: hi K blocks, then lo K blocks
  f4 u[kSplitTiles][4][64];                 // U, C layout
  int sflag[kSplitTiles];
  int uflag[kSplitTiles];
};

struct Lane {
  int lane, tile, g, n;  // tile is wave-uniform (an SGPR)
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

// Direct loads of chunk c into B by the loader wave. For the shifted pair the X resource
// starts one row early (x_t is the key before token t); the row before token 0 is
// forced out of range and patched from the record afterwards. Rows past the sequence
// end read as zeros.
template <int DK, bool SOLVE, bool SHIFT>
__device__ __forceinline__ void issue_chunk(SplitBuf<DK, SOLVE>& B, const ScanParams& p, int c, int lane,
                                            const LoadOffs<DK>& o, const Srcs& src) {
  using LO = LoadOffs<DK>;
  using RC = RecSplit<DK>;
  const uint32_t sx = (uint32_t)(c * CH * DK * 2);
  static_for<0, LO::NXI>([&](auto I) {
    constexpr int i = I;
    uint32_t xo = o.x[i];
    if (SHIFT && c == 0 && 64 * i + lane < LO::NGR) xo = 0x80000000u;  // row 0 of chunk 0
    dma16(src.x, xo, sx, &B.x[64 * i]);
    dma16(src.q, o.x[i], sx, &B.q[64 * i]);
  });
  const uint32_t sw = (uint32_t)((size_t)c * RC::kBytes);
  if constexpr (SOLVE) {
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

// Direct loads of the X, Q and V rows of chunk c >= 1 into B (the record arrives through
// the loader's registers).
template <int DK, bool SOLVE>
__device__ __forceinline__ void issue_rows(SplitBuf<DK, SOLVE>& B, const ScanParams& p, int c,
                                           const LoadOffs<DK>& o, const Srcs& src) {
  using LO = LoadOffs<DK>;
  const uint32_t sx = (uint32_t)(c * CH * DK * 2);
  static_for<0, LO::NXI>([&](auto I) {
    dma16(src.x, o.x[I], sx, &B.x[64 * I]);
    dma16(src.q, o.x[I], sx, &B.q[64 * I]);
  });
  const uint32_t sv = (uint32_t)(c * CH * p.dv * 2);
  static_for<0, LO::NVI>([&](auto I) { dma16(src.v, o.v[I], sv, &B.v[64 * I]); });
}

// A chunk's record (T, M and the row factors), held in the loader wave's registers: it
// is loaded two chunks ahead and written to LDS one chunk ahead, so that its loads have a
// whole chunk period more to land than the row loads, which go straight to LDS one
// chunk ahead. (Register loads of the rows as well proved slower than direct loads.)
template <int DK, bool SOLVE>
struct ChunkRegs {
  static constexpr int NT = SOLVE ? 2 * kTriFrags : 0;
  static constexpr int NLOADS = NT + 2 * kTriFrags + 2;
  u32x4 t[SOLVE ? 2 * kTriFrags : 1];
  u32x4 m[2 * kTriFrags];
  u32x4 f0, f1;
};

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int DK, bool SOLVE>
__device__ __forceinline__ void load_regs(ChunkRegs<DK, SOLVE>& r, const Srcs& src, int c, const LoadOffs<DK>& o,
                                          int lane) {
  using RC = RecSplit<DK>;
  const uint32_t sw = (uint32_t)((size_t)c * RC::kBytes);
  if constexpr (SOLVE) {
    static_for<0, 2 * kTriFrags>([&](auto J) { r.t[J] = ld16(src.w, o.lane16, sw + (uint32_t)(RC::kT + J * 1024)); });
  }
  static_for<0, 2 * kTriFrags>([&](auto J) { r.m[J] = ld16(src.w, o.lane16, sw + (uint32_t)(RC::kM + J * 1024)); });
  r.f0 = ld16(src.w, o.lane16, sw + (uint32_t)RC::kFac);
  // the last 256 bytes of the factors: lanes 16.. read out of range (zeros, no traffic)
  r.f1 = ld16(src.w, lane < 16 ? o.lane16 : 0x80000000u, sw + (uint32_t)(RC::kFac + 1024));
}

template <int DK, bool SOLVE>
__device__ __forceinline__ void store_regs(SplitBuf<DK, SOLVE>& B, const ChunkRegs<DK, SOLVE>& r, int lane) {
  if constexpr (SOLVE) {
#pragma unroll
    for (int j = 0; j < 2 * kTriFrags; ++j) B.t[64 * j + lane] = r.t[j];
  }
#pragma unroll
  for (int j = 0; j < 2 * kTriFrags; ++j) B.m[64 * j + lane] = r.m[j];
  reinterpret_cast<u32x4*>(B.fac)[lane] = r.f0;
  if (lane < 16) reinterpret_cast<u32x4*>(B.fac)[64 + lane] = r.f1;
}

// s_waitcnt vmcnt(n) (n <= 63), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations are
// complete before it arrives, and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

typedef volatile __attribute__((address_space(3))) int* lds_flag_ptr;

__device__ __forceinline__ lds_flag_ptr flag_ptr(int* f) {
  return (lds_flag_ptr)(uintptr_t)(uint32_t)reinterpret_cast<uintptr_t>(f);
}

// Sticky status of this device: nonzero once a bounded wait of a propagate kernel gave
// up (fwmem_check_device reads and clears it).
__device__ int g_wait_status;

// Polls an LDS flag until it holds v. The writer sets it within the same chunk period,
// so a correct run never reaches the poll limit; the limit only bounds the wait. A wait
// that reaches it goes on (the chunk's values are then wrong, but every wave keeps to the
// same barriers and the kernel ends) and records the failure in g_wait_status, by a
// vector store from one lane. `bias` is 0, except in a test that forces every wait to
// give up after a few polls by waiting for a value no wave writes.
__device__ __forceinline__ void wait_flag(int* f, int v, const ScanParams& p) {
  lds_flag_ptr fp = flag_ptr(f);
  const int target = v + p.wait_bias;
  bool done = false;
  for (int i = 0; i < p.wait_polls; ++i) {
    if (__builtin_amdgcn_readfirstlane(*fp) == target) {
      done = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!done && (threadIdx.x & 63) == 0)
    __hip_atomic_store(&g_wait_status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void set_flag(int* f, int v) {
  *flag_ptr(f) = v;
}

// One chunk for the loader wave. Outstanding on entry: the direct row loads of chunk c
// (into B), then the register loads of chunk c+1's record (if there is a chunk c+1).
// Once the rows have landed, patch in the carried key and release chunk c to the
// compute waves; then, with B's partner N free again (the compute waves finished chunk
// c-1 before the barrier), enqueue chunk c+1's rows into N, write its record from
// registers into N, and start the register loads of chunk c+2's record.
template <int DK, bool SOLVE, bool SHIFT>
__device__ __forceinline__ void loader_step(SplitBuf<DK, SOLVE>& B, SplitBuf<DK, SOLVE>& N,
                                            ChunkRegs<DK, SOLVE>& R, const ScanParams& p, int c, int lane,
                                            const LoadOffs<DK>& o, const Srcs& src, const char* rec0) {
  constexpr int NGR = SplitBuf<DK, SOLVE>::NGR;
  if (c + 1 < p.nchunks) wait_vm<ChunkRegs<DK, SOLVE>::NLOADS>();
  else wait_vm<0>();
  if (SHIFT && c == 0 && lane < NGR) {
    // x_0 is the carried key (zero without one): row 0 of the first X tile
    B.x[lane ^ xswz<DK>(0)] = *reinterpret_cast<const u32x4*>(rec0 + RecSplit<DK>::kX0 + 16 * lane);
  }
  lds_barrier();
  if (c + 1 < p.nchunks) {
    issue_rows<DK, SOLVE>(N, p, c + 1, o, src);
    store_regs<DK, SOLVE>(N, R, lane);
    if (c + 2 < p.nchunks) load_regs<DK, SOLVE>(R, src, c + 2, o, lane);
  }
}

// ---------------------------------------------------------------- compute waves
// Scheduling. A wave issues in order, so its matrix unit and its VALU only run at the
// same time if the instruction stream alternates between them. The steps are written as
// sequences of micro-regions fenced by sched_barrier: each holds one MFMA plus a fixed
// share of the independent work (operand splits, row factors, LDS reads for later
// MFMAs), in the order given here.
#define FW_FENCE() __builtin_amdgcn_sched_barrier(0)

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// hi/lo split of two fp32 values into one packed bf16 word each. The packed hi word is
// kept opaque, so that the residuals unpack it instead of converting x again.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const bf2 h = {(__bf16)x0, (__bf16)x1};
  uint32_t w = __builtin_bit_cast(uint32_t, h);
  asm volatile("" : "+v"(w));
  const bf2 l = {(__bf16)(x0 - __uint_as_float(w << 16)), (__bf16)(x1 - __uint_as_float(w & 0xffff0000u))};
  hi = w;
  lo = __builtin_bit_cast(uint32_t, l);
}

// Word j (slots 2j, 2j+1) of the B fragment of K block kb from C tiles c[2kb], c[2kb+1].
template <int KB, int J>
__device__ __forceinline__ void split_word(const f4* c, u32x4& hi, u32x4& lo) {
  constexpr int t = 2 * KB + (J >> 1), r = 2 * (J & 1);
  uint32_t h, l;
  split2(c[t][r], c[t][r + 1], h, l);
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

// LDS operand reads shared by both roles.
template <int DK, bool SOLVE>
struct Frags {
  using Buf = SplitBuf<DK, SOLVE>;
  static constexpr int NGR = Buf::NGR;
  const Buf& B;
  const Lane& L;
  // row factors k of the lane's four rows of token tile m
  __device__ __forceinline__ f4 fac4(int k, int m) const {
    return *reinterpret_cast<const f4*>(&B.fac[k * CH + tok_of(m, 4 * L.g)]);
  }
  // A fragment (rows tok_of(m, n), K block kb) of a row-major [CH][DK] tile
  __device__ __forceinline__ bf8 xfrag(const u32x4* X, int m, int kb) const {
    const int row = tok_of(m, L.n);
    return __builtin_bit_cast(bf8, X[row * NGR + ((4 * kb + L.g) ^ xswz<DK>(row))]);
  }
  // Half hh of the X^T fragment (rt, kb): rows d_k tok_of(rt, n), K slots 4hh..4hh+3 =
  // tokens 32kb + 8g + 4hh + j, by one transpose read of the row-major X tile.
  __device__ __forceinline__ s4 xthalf(int rt, int kb, int hh) const {
    const int dk0 = 32 * (rt >> 1) + 8 * (L.n & 3) + 4 * (rt & 1);
    const int row = 32 * kb + 8 * L.g + (L.n >> 2) + 4 * hh;
    const char* a = reinterpret_cast<const char*>(&B.x[row * NGR + ((dk0 >> 3) ^ xswz<DK>(row))]) + (dk0 & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)a);
  }
  // Values of the lane's four rows tok_of(m, 4g+i), i = 0..3 (consecutive tokens), in its
  // column: one transpose read, in which lane 4i+q of the group supplies columns
  // 4q..4q+3 of token row i.
  __device__ __forceinline__ s4 vrows(int m) const {
    const int row = tok_of(m, 4 * L.g) + (L.n >> 2);
    const int c0 = L.tile * 16 + 4 * (L.n & 3);
    const char* a = reinterpret_cast<const char*>(&B.v[row * 4 + ((c0 >> 3) ^ vswz(row))]) + (c0 & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)a);
  }
  __device__ __forceinline__ bf8 tfrag(const u32x4* T, int f, int part) const {
    return __builtin_bit_cast(bf8, T[(2 * f + part) * 64 + L.lane]);
  }
};

// Order of the lower-triangular fragments in U = T R: those of K block 0 first.
__host__ __device__ constexpr int kb0_first(int k) { return k < 3 ? k : (k == 3 ? 4 : (k == 4 ? 3 : 5)); }

__device__ __forceinline__ bf8 xtjoin(const s4& a, const s4& b) {
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf8, r);
}

__device__ __forceinline__ float vf(const s4& h, int i) {
  return bf16_bits_to_f32((uint32_t)(uint16_t)h[i]);
}

// ---- alpha: the state chain of one tile for chunk c (data in B). On entry acc holds
// Gamma_C S (for c > 0; S itself for c = 0) and Sh/Sl the split of S; on exit acc holds
// Gamma_C' S' with Gamma_C' the next chunk's decay (1 after the last chunk) and Sh/Sl
// the split of S'.
template <int DK, bool SOLVE>
__device__ __forceinline__ void alpha_step(const ScanParams& p, const SplitBuf<DK, SOLVE>& B, Handoff<DK>& H,
                                           int c, bool last,
                                           const Lane& L, f4 (&acc)[DK / 16], u32x4 (&Sh)[DK / 32],
                                           u32x4 (&Sl)[DK / 32]) {
  constexpr int NKD = DK / 32;  // K blocks over d_k
  constexpr int NRT = DK / 16;  // row tiles of S
  const Frags<DK, SOLVE> F{B, L};

  // the loader wave releases chunk c once its loads have landed; the compute waves have
  // finished with chunk c-1, so the loader may refill that buffer
  lds_barrier();

  // ---- A: operand reads; the first chunk scales S by its decay here
  bf8 xf[4][NKD];
  if constexpr (SOLVE) {
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) xf[0][kb] = F.xfrag(B.x, 0, kb);
  }
  s4 vv[4];
  f4 fvr[4], fpr[4], fur[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    vv[m] = F.vrows(m);
    fvr[m] = F.fac4(1, m);
    if (SOLVE) fpr[m] = F.fac4(0, m);
  }
  if (c == 0) {
    const float g0 = B.fac[4 * CH];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc[rt] *= g0;
  }
  FW_FENCE();

  f4 U[4], Wt[4];
  u32x4 Wh[2], Wl[2];
  bf8 th[kTriFrags], tl[kTriFrags];
  s4 xth[NRT][2][2];
  float gCn;
  if constexpr (SOLVE) {
    // ---- B: P = X S by token tile (8 NKD MFMAs). Tile m completes before tile m+1
    // starts, so R = fV V - fP P and its split run one tile behind. Alongside: the X
    // fragments of the next tile, the T fragments, the remaining factors.
    f4 P[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) P[m] = f4{0.f, 0.f, 0.f, 0.f};
    u32x4 Rh[2], Rl[2];
    constexpr int NB = 8 * NKD;
    constexpr int NBR = 6 + 2 * kTriFrags;  // fur (4), gCn, spare, T fragments
    static_for<0, NB>([&](auto I) {
      constexpr int i = I, m = i / (2 * NKD), kb = (i % (2 * NKD)) / 2, part = i % 2;
      constexpr int j = i % (2 * NKD);  // slot within the tile
      mma_w(P[m], xf[m][kb], part ? Sl[kb] : Sh[kb]);
      FW_FENCE();
      // X fragments of tile m+1, one per two slots
      if constexpr (m + 1 < 4 && part == 0) xf[m + 1][kb] = F.xfrag(B.x, m + 1, kb);
      // R of tile m-1: four values, then its two split words, spread over the tile's slots
      if constexpr (m >= 1) {
        constexpr int pm = m - 1;
        constexpr int NR = 6;  // items: 4 values, 2 words
        static_for<Share<NR, 2 * NKD, j>::lo, Share<NR, 2 * NKD, j>::hi>([&](auto K) {
          constexpr int k = K;
          if constexpr (k < 4) {
            P[pm][k] = fvr[pm][k] * vf(vv[pm], k) - fpr[pm][k] * P[pm][k];
          } else {
            constexpr int kbt = pm / 2, w = 2 * (pm & 1) + (k - 4);
            split_word<kbt, w>(P, Rh[kbt], Rl[kbt]);
          }
        });
      }
      static_for<Share<NBR, NB, i>::lo, Share<NBR, NB, i>::hi>([&](auto K) {
        constexpr int k = K;
        if constexpr (k < 4) fur[k] = F.fac4(3, k);
        else if constexpr (k == 4) gCn = B.fac[4 * CH + 2];
        else if constexpr (k >= 6) {
          constexpr int f = (k - 6) / 2, pt = (k - 6) % 2;
          if constexpr (pt == 0) th[f] = F.tfrag(B.t, f, 0);
          else tl[f] = F.tfrag(B.t, f, 1);
        }
      });
      FW_FENCE();
    });

    // ---- C: U = T R (18 MFMAs): the K block 0 products first (they need only R tiles
    // 0 and 1), alongside R of tile 3 and its split; then K block 1, alongside U tiles 0
    // and 1 (complete by then): their hand-off to beta, W = fU U and W's split of K block
    // 0. Throughout: the X^T fragments of the state update.
#pragma unroll
    for (int m = 0; m < 4; ++m) U[m] = f4{0.f, 0.f, 0.f, 0.f};
    constexpr int NC = 3 * kTriFrags;
    constexpr int NCX = 4 * NRT;  // transpose reads
    static_for<0, NC>([&](auto I) {
      constexpr int i = I, f = kb0_first(i / 3), part = i % 3;
      constexpr int m = tri_m(f), kb = tri_kb(f);
      if constexpr (part == 0) mma_w(U[m], th[f], Rh[kb]);
      else if constexpr (part == 1) mma_w(U[m], th[f], Rl[kb]);
      else mma_w(U[m], tl[f], Rh[kb]);
      FW_FENCE();
      if constexpr (i < 12) {
        static_for<Share<6, 12, i>::lo, Share<6, 12, i>::hi>([&](auto K) {
          constexpr int k = K;
          if constexpr (k < 4) P[3][k] = fvr[3][k] * vf(vv[3], k) - fpr[3][k] * P[3][k];
          else split_word<1, 2 + (k - 4)>(P, Rh[1], Rl[1]);
        });
      } else {
        static_for<Share<8, NC - 12, i - 12>::lo, Share<8, NC - 12, i - 12>::hi>([&](auto K) {
          constexpr int k = K;
          if constexpr (k < 2) H.u[L.tile][k][L.lane] = U[k];
          else if constexpr (k < 4) Wt[k - 2] = U[k - 2] * fur[k - 2];
          else split_word<0, k - 4>(Wt, Wh[0], Wl[0]);
        });
      }
      static_for<Share<NCX, NC, i>::lo, Share<NCX, NC, i>::hi>([&](auto K) {
        constexpr int k = K, rt = k / 4, kbx = (k / 2) % 2, hh = k % 2;
        xth[rt][kbx][hh] = F.xthalf(rt, kbx, hh);
      });
      FW_FENCE();
    });
  } else {
    // no solve (additive and inner-product rules): U = fV V; the remaining reads
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) U[m][r] = fvr[m][r] * vf(vv[m], r);
      fur[m] = F.fac4(3, m);
    }
    gCn = B.fac[4 * CH + 2];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int kbx = 0; kbx < 2; ++kbx)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) xth[rt][kbx][hh] = F.xthalf(rt, kbx, hh);
  }

  // ---- D: the rest of the U hand-off and of W = fU U; the flag follows once every LDS
  // access of this wave so far has completed (the X^T reads are needed next anyway)
  constexpr int M0 = SOLVE ? 2 : 0;  // tiles already handed over and scaled in C
#pragma unroll
  for (int m = M0; m < 4; ++m) {
    H.u[L.tile][m][L.lane] = U[m];
    Wt[m] = U[m] * fur[m];
  }
  if constexpr (!SOLVE) static_for<0, 4>([&](auto J) { split_word<0, J>(Wt, Wh[0], Wl[0]); });
  lds_wait();
  set_flag(&H.uflag[L.tile], c + 1);
  FW_FENCE();

  // ---- E: S' = Gamma_C S + X^T W (4 NRT MFMAs onto acc), K block 0 over all row tiles
  // (alongside the split of W's K block 1), then K block 1 by row tile; as each row tile
  // completes, its next-chunk form Gamma_C' S' and its split follow two slots behind.
  constexpr int NE0 = 2 * NRT;
  static_for<0, NE0>([&](auto I) {
    constexpr int i = I, rt = i / 2, part = i % 2;
    mma_w(acc[rt], xtjoin(xth[rt][0][0], xth[rt][0][1]), part ? Wl[0] : Wh[0]);
    FW_FENCE();
    static_for<Share<4, NE0, i>::lo, Share<4, NE0, i>::hi>([&](auto J) {
      split_word<1, J>(Wt, Wh[1], Wl[1]);
    });
    FW_FENCE();
  });
  // beta raised sflag early in this period; the split state for the next chunk goes to
  // the hand-off slot K block by K block as it completes
  if (!last) wait_flag(&H.sflag[L.tile], c + 1, p);
  static_for<0, NE0 + 4>([&](auto I) {
    constexpr int i = I, rt = i / 2, part = i % 2;
    if constexpr (i < NE0) mma_w(acc[rt], xtjoin(xth[rt][1][0], xth[rt][1][1]), part ? Wl[1] : Wh[1]);
    FW_FENCE();
    // K block kb of the split is complete after slot 4 kb + 7
    if constexpr (i >= 8 && (i - 8) % 4 == 0) {
      constexpr int kb = (i - 8) / 4;
      if (!last) {
        H.s[L.tile][kb][L.lane] = Sh[kb];
        H.s[L.tile][NKD + kb][L.lane] = Sl[kb];
      }
    }
    // row tile pt completed two slots ago: scale it for the next chunk and split it,
    // one word per slot
    if constexpr (i >= 4) {
      constexpr int pt = (i - 4) / 2, w = 2 * (pt & 1) + ((i - 4) % 2);
      constexpr int r = 2 * (w & 1);
      const float s0 = acc[pt][r], s1 = acc[pt][r + 1];
      acc[pt][r] = s0 * gCn;
      acc[pt][r + 1] = s1 * gCn;
      uint32_t h, l;
      split2(s0, s1, h, l);
      Sh[pt / 2][w] = h;
      Sl[pt / 2][w] = l;
    }
    FW_FENCE();
  });

  // ---- F: the last K block of the split state
  if (!last) {
    H.s[L.tile][NKD - 1][L.lane] = Sh[NKD - 1];
    H.s[L.tile][2 * NKD - 1][L.lane] = Sl[NKD - 1];
  }
}

// ---- beta: the outputs of one tile for chunk c
template <int DK, bool SOLVE, bool OBF>
__device__ __forceinline__ void beta_step(const ScanParams& p, const SplitBuf<DK, SOLVE>& B, Handoff<DK>& H,
                                          int c, const Lane& L,
                                          int dv, uint32_t vo, __amdgpu_buffer_rsrc_t ro) {
  constexpr int NKD = DK / 32;
  const Frags<DK, SOLVE> F{B, L};
  lds_barrier();

  // ---- A: the split state of this chunk; tell alpha it may write the next one
  u32x4 Sh[NKD], Sl[NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb) {
    Sh[kb] = H.s[L.tile][kb][L.lane];
    Sl[kb] = H.s[L.tile][NKD + kb][L.lane];
  }
  bf8 qf[4][NKD];
#pragma unroll
  for (int kb = 0; kb < NKD; ++kb) qf[0][kb] = F.xfrag(B.q, 0, kb);
  lds_wait();
  set_flag(&H.sflag[L.tile], c + 1);

  // ---- B: O = fO (Q S) by token tile (8 NKD MFMAs); alongside, the Q fragments of the
  // next tile, the factors and the M fragments
  f4 Om[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) Om[m] = f4{0.f, 0.f, 0.f, 0.f};
  f4 for_[4];
  bf8 mh[kTriFrags], ml[kTriFrags];
  constexpr int NB = 8 * NKD;
  constexpr int NBR = 4 + 2 * kTriFrags;
  static_for<0, NB>([&](auto I) {
    constexpr int i = I, m = i / (2 * NKD), kb = (i % (2 * NKD)) / 2, part = i % 2;
    mma_w(Om[m], qf[m][kb], part ? Sl[kb] : Sh[kb]);
    FW_FENCE();
    if constexpr (m + 1 < 4 && part == 0) qf[m + 1][kb] = F.xfrag(B.q, m + 1, kb);
    static_for<Share<NBR, NB, i>::lo, Share<NBR, NB, i>::hi>([&](auto K) {
      constexpr int k = K;
      if constexpr (k < 4) for_[k] = F.fac4(2, k);
      else {
        constexpr int f = (k - 4) / 2, pt = (k - 4) % 2;
        if constexpr (pt == 0) mh[f] = F.tfrag(B.m, f, 0);
        else ml[f] = F.tfrag(B.m, f, 1);
      }
    });
    FW_FENCE();
  });
#pragma unroll
  for (int m = 0; m < 4; ++m) Om[m] *= for_[m];

  // ---- C: U from alpha, its split, and O += M U (18 MFMAs)
  wait_flag(&H.uflag[L.tile], c + 1, p);
  f4 U[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) U[m] = H.u[L.tile][m][L.lane];
  u32x4 Uh[2], Ul[2];
  static_for<0, 8>([&](auto K) { split_word<K / 4, K % 4>(U, Uh[K / 4], Ul[K / 4]); });
  static_for<0, 3 * kTriFrags>([&](auto I) {
    constexpr int i = I, f = i / 3, part = i % 3;
    constexpr int m = tri_m(f), kb = tri_kb(f);
    if constexpr (part == 0) mma_w(Om[m], mh[f], Uh[kb]);
    else if constexpr (part == 1) mma_w(Om[m], mh[f], Ul[kb]);
    else mma_w(Om[m], ml[f], Uh[kb]);
  });

  // ---- D: store the tile's outputs: lane (g, n) writes rows tok_of(m, 4g+i) of its
  // column through the output resource (rows past the sequence end fall outside it)
  constexpr uint32_t es = OBF ? 2u : 4u;
  static_for<0, 4>([&](auto M) {
    constexpr int m = M;
    static_for<0, 4>([&](auto I) {
      constexpr int i = I;
      const uint32_t so = (uint32_t)((c * CH + 32 * (m >> 1) + 4 * (m & 1) + i) * dv) * es;
      if constexpr (OBF) {
        const __bf16 h = (__bf16)Om[m][i];
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), ro, vo, so, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Om[m][i]), ro, vo, so, 0);
      }
    });
  });
}

template <int DK, int RULE, bool OBF>
__global__ __launch_bounds__(NTS) void prop_split_kernel(ScanParams p) {
  constexpr bool SOLVE = Rule<RULE>::solve, SHIFT = Rule<RULE>::shift;
  using Buf = SplitBuf<DK, SOLVE>;
  constexpr int NRT = DK / 16;
  constexpr int NKD = DK / 32;
  __shared__ Buf B0, B1;
  __shared__ Handoff<DK> H;

  // workgroup -> (head, column group); the groups of a head share an XCD and its L2
  const int ngrp = p.dv / kSplitCols;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int grp = __builtin_amdgcn_readfirstlane(slot % ngrp);
  const int bh = __builtin_amdgcn_readfirstlane((slot / ngrp) * 8 + xcd);
  if (bh >= p.BH) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int dv = p.dv;
  const size_t rowbase = (size_t)bh * p.T;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const char* rec0 = p.ws + (size_t)bh * p.nchunks * RecSplit<DK>::kBytes;

  if (wave == kLoader) {
    const uint16_t* qb = static_cast<const uint16_t*>(p.q) + rowbase * DK;
    const uint16_t* vb = static_cast<const uint16_t*>(p.v) + rowbase * dv;
    const LoadOffs<DK> lo = load_offsets<DK>(lane, dv, grp);
    Srcs src;
    src.x = rsrc(SHIFT ? kb - DK : kb, (uint32_t)(p.T * DK * 2));
    src.q = rsrc(qb, (uint32_t)(p.T * DK * 2));
    // a null value pointer means all-zero values (the transition pass of the segmented
    // scan): an empty resource reads zeros without touching memory
    src.v = p.v != nullptr ? rsrc(vb, (uint32_t)(p.T * dv * 2)) : rsrc(qb, 0u);
    src.w = rsrc(rec0, (uint32_t)((size_t)p.nchunks * RecSplit<DK>::kBytes));
    issue_chunk<DK, SOLVE, SHIFT>(B0, p, 0, lane, lo, src);
    ChunkRegs<DK, SOLVE> R;
    if (p.nchunks > 1) load_regs<DK, SOLVE>(R, src, 1, lo, lane);
    for (int c = 0; c < p.nchunks; c += 2) {
      loader_step<DK, SOLVE, SHIFT>(B0, B1, R, p, c, lane, lo, src, rec0);
      if (c + 1 < p.nchunks) loader_step<DK, SOLVE, SHIFT>(B1, B0, R, p, c + 1, lane, lo, src, rec0);
    }
    if (p.S_out != nullptr && grp == 0 && (p.flags & kFlagZnorm) == 0) {  // else the slot holds z
      for (int i = lane; i < DK; i += 64)
        p.xprev_out[(size_t)bh * DK + i] = bf16_bits_to_f32(kb[(uint32_t)((p.T - 1) * DK + i)]);
      if (lane == 0) p.has_out[bh] = 1;
    }
    return;
  }

  // compute waves: wave 0 beta of tile 0, 1 alpha of tile 0, 2 alpha of tile 1, 3 beta of
  // tile 1 (waves w and w + 4 share a SIMD, so the loader shares one with a beta wave)
  const bool alpha = wave == 1 || wave == 2;
  Lane L;
  L.lane = lane;
  L.tile = wave == 0 || wave == 1 ? 0 : 1;
  L.g = lane >> 4;
  L.n = lane & 15;
  const int col = grp * kSplitCols + L.tile * 16 + L.n;  // this lane's value column

  if (alpha) {
    f4 acc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] : 0.f;
    u32x4 Sh[NKD], Sl[NKD];
    static_for<0, NKD>([&](auto KB) {
      static_for<0, 4>([&](auto J) { split_word<KB, J>(acc, Sh[KB], Sl[KB]); });
    });
#pragma unroll
    for (int k = 0; k < NKD; ++k) {
      H.s[L.tile][k][L.lane] = Sh[k];
      H.s[L.tile][NKD + k][L.lane] = Sl[k];
    }
    set_flag(&H.sflag[L.tile], 0);
    set_flag(&H.uflag[L.tile], 0);

    for (int c = 0; c < p.nchunks; c += 2) {
      alpha_step<DK, SOLVE>(p, B0, H, c, c + 1 == p.nchunks, L, acc, Sh, Sl);
      if (c + 1 < p.nchunks) alpha_step<DK, SOLVE>(p, B1, H, c + 1, c + 2 == p.nchunks, L, acc, Sh, Sl);
    }
    // after the last chunk acc holds S' (its next-chunk decay is 1)
    if (p.S_out != nullptr) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p.S_out[((size_t)bh * DK + tok_of(rt, 4 * L.g + i)) * dv + col] = acc[rt][i];
    }
    return;
  }

  // A null output asks for the state alone (the segmented scan's state passes): the
  // resource is then empty, based at the keys, so every output store falls outside it and
  // is dropped.
  constexpr uint32_t oes = OBF ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t ro =
      p.out != nullptr ? rsrc(static_cast<const char*>(p.out) + rowbase * dv * oes, (uint32_t)(p.T * dv) * oes)
                       : rsrc(kb, 0u);
  const uint32_t vo = (uint32_t)(8 * L.g * dv + col) * oes;
  for (int c = 0; c < p.nchunks; c += 2) {
    beta_step<DK, SOLVE, OBF>(p, B0, H, c, L, dv, vo, ro);
    if (c + 1 < p.nchunks) beta_step<DK, SOLVE, OBF>(p, B1, H, c + 1, L, dv, vo, ro);
  }
}

template <int DK, int RULE>
hipError_t launch_t(const ScanParams& p, hipStream_t st) {
  const int ngrp = p.dv / kSplitCols;
  const unsigned grid = (unsigned)(8 * ngrp * ((p.BH + 7) / 8));
  if (p.flags & kFlagOutBf16)
    hipLaunchKernelGGL((prop_split_kernel<DK, RULE, true>), dim3(grid), dim3(NTS), 0, st, p);
  else
    hipLaunchKernelGGL((prop_split_kernel<DK, RULE, false>), dim3(grid), dim3(NTS), 0, st, p);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const ScanParams& p, hipStream_t st) {
  if (p.rule == kRuleDelta) return launch_t<DK, kRuleDelta>(p, st);
  if (p.rule == kRuleInner) return launch_t<DK, kRuleInner>(p, st);
  return launch_t<DK, kRuleAdditive>(p, st);
}

}  // namespace

hipError_t launch_prop_split(const ScanParams& p, hipStream_t st) {
  return p.dk == 64 ? launch_dk<64>(p, st) : launch_dk<128>(p, st);
}

namespace {
constexpr int kMaxDevices = 64;
struct StatusWord {
  std::once_flag once;
  int* ptr = nullptr;
};
StatusWord g_status[kMaxDevices];
}  // namespace

hipError_t read_wait_status(hipStream_t st, int* value) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  StatusWord& w = g_status[dev];
  std::call_once(w.once, [&w]() {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(g_wait_status)) == hipSuccess) w.ptr = static_cast<int*>(a);
  });
  if (w.ptr == nullptr) return hipErrorInvalidSymbol;
  int h = 0;
  e = hipMemcpyAsync(&h, w.ptr, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && h != 0) {
    static const int zero = 0;
    e = hipMemcpyAsync(w.ptr, &zero, sizeof(int), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  *value = h;
  return e;
}

}  // namespace fwmem
