// Chunk-parallel backward pass of the scan for the delta, inner and additive rules with a
// scalar decay (phi identity or elu+1, QK normalisation, pre-activated gates, the
// scale-coupled ridge), on fp32 MFMA. The pages give no backward pass; this is the
// reverse-mode derivative of the chunk form of the forward recurrence ("Fast Weight
// Attention for Continual Learning" reading notes, section 4.4: an intra-chunk
// triangular solve, a short inter-chunk recurrence, parallel outputs), laid out the
// same way: a parallel prep, one short serial recurrence per direction, and a parallel
// gradient pass.
//
// Per head, chunks of C = 64 tokens; inside a chunk Gamma_t = a_1 ... a_t (the decays,
// carried as a log-sum with a sign parity), Gamma_end the chunk's total, D_ts =
// Gamma_t / Gamma_s (s <= t), D'_ts = Gamma_{t-1} / Gamma_s (s < t), eta the step size
// (the write scale f = beta for the additive rule). With entry state S and exit S':
//   L = diag(eta) (D' o X X^T),  T = (I + L)^-1,  M = D o (Q X^T)
//   U = T diag(eta) (V - diag(Gamma_prev) X S)      (delta)    U = diag(f) V (inner, additive)
//   O = diag(Gamma) Q S + M U,   S' = Gamma_end S + X^T diag(Gamma_end / Gamma) U.
// Backward, from the exit gradient dS' and the chunk's dO:
//   dU = M^T dO + diag(Gamma_end / Gamma) X dS',   dR = T^T dU (delta)
//   dS = Gamma_end dS' + Q^T diag(Gamma) dO - X^T diag(eta Gamma_prev) dR
// and the gradients of Q, X, V, eta and of the log decays, per chunk.
//
// Kernels:
//   prep   (head, chunk): X, Q rows; token scalars; X X^T and Q X^T on MFMA; the masks;
//          T = (I + L)^-1 (blocked, 16x16 diagonal blocks by substitution) -> record;
//   state  (head, 32 value columns), serial over chunks: S at every chunk start;
//   dstate (head, 32 value columns), serial from the last chunk: every chunk's exit
//          gradient dS' and dL/dS_0;
//   grad   (head, chunk): every input gradient, streaming 32-column value blocks.
#include "fwmem_backward.h"
#include "fwmem_device.h"
#include "fwmem_internal.h"
#include "fwmem_split.h"

namespace fwmem {
namespace {

constexpr int CB = 64;        // tokens per chunk
constexpr int LDC = CB + 4;   // row stride (floats) of an LDS tile with CB columns
constexpr int NCOL = 32;      // value columns of a state workgroup and of a gradient block
constexpr int LDU = NCOL + 4;  // row stride of a [CB][NCOL] LDS tile

// Per-token scalars of a record ([kNSc][CB] floats).
enum {
  kScGam,    // Gamma_t
  kScGprev,  // Gamma_{t-1}
  kScGend,   // Gamma_end / Gamma_t
  kScE,      // eta_t (the write scale f_t for the additive rule); 0 without a write
  kScA,      // a_t, the decay
  kScDen,    // eta's denominator |x_t|^2 + lambda_used + eps
  kScLu,     // lambda_used (lambda_t, or lambda_t |x_t|^2 with the scale-coupled ridge)
  kScN,      // |x_t|^2
  kScBeta,   // beta_t (activated)
  kScLam,    // lambda_t (activated; the retention for the additive rule)
  kScKey,    // 1 where the token writes (a key exists and t < T), else 0
  kScG,      // g_t = log|Gamma_t|
  kScPar,    // sign parity of Gamma_t (0 or 1)
  kNSc
};

struct BRec {
  static constexpr size_t kT = 0;              // [CB][CB] T = (I + L)^-1 (delta rule)
  static constexpr size_t kM = kT + CB * CB;   // [CB][CB] M = D o (Q X^T)
  static constexpr size_t kLp = kM + CB * CB;  // [CB][CB] D' o (X X^T), strictly lower
  static constexpr size_t kSc = kLp + CB * CB;
  static constexpr size_t kMisc = kSc + (size_t)kNSc * CB;  // [0] Gamma_end
  static constexpr size_t kFloats = (kMisc + 64 + 63) / 64 * 64;
};

// ---- fp32 MFMA tile products (v_mfma_f32_16x16x4f32). A 16x16 accumulator tile in C
// layout holds rows 4g+i (i = 0..3) of column n in lane 16g+n. Instruction i of a K block
// of 16 gives lane group g the K index 4g+i, for A and B alike, so the four instructions
// cover the block whatever order the unit sums its K slots in.
__device__ __forceinline__ void mfma4(f4& acc, const f4& a, const f4& b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
}

// acc += A B over K in [k0, k1) (multiples of 16). A: AT == false: row r at a + r*lda with
// K contiguous; AT == true: A[r][k] = a[k*lda + r]. B: BN == false: column n at
// b + n*ldb with K contiguous (B^T row-major); BN == true: B[k][n] = b[k*ldb + n].
template <bool AT, bool BN>
__device__ __forceinline__ void mm(f4& acc, const float* a, int lda, const float* b, int ldb, int k0, int k1,
                                   int lane) {
  const int g = lane >> 4, n = lane & 15;
  for (int k = k0; k < k1; k += 16) {
    f4 av, bv;
    if constexpr (AT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = a[(k + 4 * g + i) * lda + n];
    } else {
      av = *reinterpret_cast<const f4*>(a + n * lda + k + 4 * g);
    }
    if constexpr (BN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = b[(k + 4 * g + i) * ldb + n];
    } else {
      bv = *reinterpret_cast<const f4*>(b + n * ldb + k + 4 * g);
    }
    mfma4(acc, av, bv);
  }
}

// C-layout tile -> LDS: transposed (dst[col][row], one 16-byte store) or natural.
__device__ __forceinline__ void store_t(float* dst, int ld, int r0, int c0, const f4& v, int lane) {
  *reinterpret_cast<f4*>(dst + (c0 + (lane & 15)) * ld + r0 + 4 * (lane >> 4)) = v;
}
__device__ __forceinline__ void store_n(float* dst, int ld, int r0, int c0, const f4& v, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(r0 + 4 * (lane >> 4) + i) * ld + c0 + (lane & 15)] = v[i];
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations complete
// before it arrives and the compiler moves no memory access across it, but its global loads
// stay in flight (__syncthreads would wait for them), so the prefetch of the next chunk or
// value block overlaps the barriers of the current one. Global memory is never shared
// between the threads of a workgroup in these kernels.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum over the 16 lanes of a lane group (the 16 columns of a C-layout tile).
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float sgn(int par) { return par ? -1.f : 1.f; }

// Written keys x_t and (WANT_Q) read queries phi(q_t) of chunk c as fp32 rows [CB][DK + 4]:
// the shift to the previous token's key (and the carried key before a call's first token),
// phi and QK normalisation applied; rows of tokens past T are zero. Ends with a barrier.
template <typename InT, int DK, bool SHIFT, bool WANT_X, bool WANT_Q, int NTH>
__device__ void stage_rows(const BwdParams& p, int bh, int c, float* Xs, float* Qs, bool has_in) {
  constexpr int LDX = DK + 4, VW = 16 / (int)sizeof(InT), GPR = DK / VW;
  const int tid = threadIdx.x;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const size_t rb = (size_t)bh * p.T;
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* qb = static_cast<const InT*>(p.q) + rb * DK;
  for (int idx = tid; idx < CB * GPR; idx += NTH) {
    const int t = idx / GPR, i0 = (idx % GPR) * VW, tau = c * CB + t;
    float x[VW], q[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) x[e] = q[e] = 0.f;
    if (tau < p.T) {
      if constexpr (WANT_X) {
        if (SHIFT && tau == 0) {
          if (has_in && p.xprev_in != nullptr) {
#pragma unroll
            for (int e = 0; e < VW; ++e) x[e] = p.xprev_in[(size_t)bh * DK + i0 + e];  // phi applied
          }
        } else {
          In<InT>::load(kb + (size_t)(SHIFT ? tau - 1 : tau) * DK + i0, x);
          if (elu) {
#pragma unroll
            for (int e = 0; e < VW; ++e) x[e] = phi_elu1(x[e]);
          }
        }
      }
      if constexpr (WANT_Q) {
        In<InT>::load(qb + (size_t)tau * DK + i0, q);
        if (elu) {
#pragma unroll
          for (int e = 0; e < VW; ++e) q[e] = phi_elu1(q[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VW; e += 4) {
      if (WANT_X) *reinterpret_cast<f4*>(Xs + t * LDX + i0 + e) = f4{x[e], x[e + 1], x[e + 2], x[e + 3]};
      if (WANT_Q) *reinterpret_cast<f4*>(Qs + t * LDX + i0 + e) = f4{q[e], q[e + 1], q[e + 2], q[e + 3]};
    }
  }
  __syncthreads();
  const float len = qk_length(p.flags, DK);
  if (len > 0.f) {
    // QK normalisation: each row rescaled to length len by one wave
    const int lane = tid & 63, wave = tid >> 6;
    for (int t = wave; t < CB; t += NTH / 64) {
      float nx = 0.f, nq = 0.f;
      for (int i = lane; i < DK; i += 64) {
        if (WANT_X) nx += Xs[t * LDX + i] * Xs[t * LDX + i];
        if (WANT_Q) nq += Qs[t * LDX + i] * Qs[t * LDX + i];
      }
      nx = wave_sum(nx);
      nq = wave_sum(nq);
      const float fx = rescale_factor(nx, len), fq = rescale_factor(nq, len);
      for (int i = lane; i < DK; i += 64) {
        if (WANT_X) Xs[t * LDX + i] *= fx;
        if (WANT_Q) Qs[t * LDX + i] *= fq;
      }
    }
    __syncthreads();
  }
}

// Raw rows of one chunk held in registers between their load and their use, so that a
// serial kernel loads chunk c+-1 while it computes chunk c. Thread tid holds 16-byte groups
// tid + NTH j (j < NG) of the [CB][DK] row block; a row's GPR groups sit in GPR consecutive
// lanes, so a row's squared norm is a sum over those lanes.
template <typename InT, int DK, int NTH>
struct Rows {
  static constexpr int VW = 16 / (int)sizeof(InT), GPR = DK / VW, NG = CB * GPR / NTH;
  static_assert(NG >= 1 && CB * GPR % NTH == 0, "row groups");
  u32x4 w[NG];
  uint32_t valid;
  // rows src[tau] for tokens tau = tau0 + t, t < CB; zero where tau is outside [lo, hi)
  __device__ __forceinline__ void load(const InT* src, int tau0, int lo, int hi) {
    valid = 0;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int idx = threadIdx.x + NTH * j, t = idx / GPR, i0 = (idx % GPR) * VW, tau = tau0 + t;
      w[j] = u32x4{0u, 0u, 0u, 0u};
      if (tau >= lo && tau < hi) {
        w[j] = *reinterpret_cast<const u32x4*>(src + (size_t)tau * DK + i0);
        valid |= 1u << j;
      }
    }
  }
  // fp32 rows into dst [CB][DK + 4]: phi = elu+1 on loaded rows (elu), row `patch` replaced
  // by the vector pv (the carried key, phi applied; zero when pv is null), every row then
  // rescaled to length len (QK normalisation, len > 0). Zero rows stay zero.
  __device__ __forceinline__ void commit(float* dst, bool elu, float len, int patch, const float* pv) const {
    constexpr int LDX = DK + 4;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int idx = threadIdx.x + NTH * j, t = idx / GPR, i0 = (idx % GPR) * VW;
      float x[VW];
      In<InT>::decode(w[j], x);
      if (t == patch) {
#pragma unroll
        for (int e = 0; e < VW; ++e) x[e] = pv != nullptr ? pv[i0 + e] : 0.f;
      } else if (elu && ((valid >> j) & 1u)) {
#pragma unroll
        for (int e = 0; e < VW; ++e) x[e] = phi_elu1(x[e]);
      }
      if (len > 0.f) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VW; ++e) ss += x[e] * x[e];
        ss = group_sum<GPR>(ss);
        const float f = rescale_factor(ss, len);
#pragma unroll
        for (int e = 0; e < VW; ++e) x[e] *= f;
      }
#pragma unroll
      for (int e = 0; e < VW; e += 4) *reinterpret_cast<f4*>(dst + t * LDX + i0 + e) = f4{x[e], x[e + 1], x[e + 2], x[e + 3]};
    }
  }
  // The same rows as bf16 hi/lo planes [CB][DK + 8] (hi at dst, lo a plane further on).
  __device__ __forceinline__ void commit_split(uint16_t* dst, bool elu, float len, int patch, const float* pv) const;
};

// ---- bf16 split operands of the gradient pass. A matrix formed in fp32 is held in LDS as
// two bf16 planes of one row-major layout, hi = bf16(x) and lo = bf16(x - hi): 16
// significant bits over fp32's exponent range. A product with both operands split is
// Ah Bh + Ah Bl + Al Bh on v_mfma_f32_16x16x32_bf16 with fp32 accumulation (Al Bl lies
// below the fp32 rounding of the result); an exact bf16 operand (raw bf16 keys and queries
// with the identity map and no QK rescaling) has a zero lo plane and takes two products.
// Plane rows are padded by 8 elements, so the row stride is an odd multiple of 16 bytes
// modulo 256 and the 16 rows of a fragment read fall in distinct bank groups.
//
// Fragments follow the K-slot order of frag_pair / xt_frag: slots 0..3 carry K = 4g..4g+3
// and slots 4..7 K = 16+4g..16+4g+3 of a 32-wide K block (g = lane / 16), for A and B alike.
__device__ __forceinline__ uint16_t bf_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ __forceinline__ void put_split(uint16_t* hi, int plane, int idx, float x) {
  const uint16_t h = bf_bits(x);
  hi[idx] = h;
  hi[plane + idx] = bf_bits(x - bf16_bits_to_f32(h));
}

// four consecutive elements (idx a multiple of 4): one 8-byte store per plane
__device__ __forceinline__ void put_split4(uint16_t* hi, int plane, int idx, const f4& x) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = bf_bits(x[i]);
    l[i] = bf_bits(x[i] - bf16_bits_to_f32(h[i]));
  }
  *reinterpret_cast<uint2*>(hi + idx) = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  *reinterpret_cast<uint2*>(hi + plane + idx) = uint2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
}

// the fp32 value hi + lo of element idx
__device__ __forceinline__ float get_split(const uint16_t* hi, int plane, int idx) {
  return bf16_bits_to_f32(hi[idx]) + bf16_bits_to_f32(hi[plane + idx]);
}

struct SFrag {
  bf8 h, l;
};

// Operand row r (A row, or B column) of the K block at k0, from planes stored with K
// contiguous (element [r][k] at r * ld + k).
__device__ __forceinline__ SFrag fk(const uint16_t* hi, int plane, int ld, int r, int k0, int g) {
  return SFrag{frag_pair(hi + r * ld + k0 + 4 * g), frag_pair(hi + plane + r * ld + k0 + 4 * g)};
}
// Operand rows r0..r0+15 of the K block at k0, from planes stored K-major (element [k][r]
// at k * ld + r), by the LDS transpose read.
__device__ __forceinline__ SFrag ft(const uint16_t* hi, int plane, int ld, int r0, int k0, int g, int n) {
  const int o = (k0 + 4 * g + (n >> 2)) * ld + r0 + 4 * (n & 3);
  return SFrag{xt_frag(hi + o, ld), xt_frag(hi + plane + o, ld)};
}

// acc += A B with both operands split
__device__ __forceinline__ void mma3(f4& acc, const SFrag& a, const SFrag& b) {
  mma_bf16(acc, a.l, b.h);
  mma_bf16(acc, a.h, b.l);
  mma_bf16(acc, a.h, b.h);
}
// acc += A B where B's lo plane is zero when bex (an exact bf16 operand)
__device__ __forceinline__ void mma3x(f4& acc, const SFrag& a, const SFrag& b, bool bex) {
  mma_bf16(acc, a.l, b.h);
  if (!bex) mma_bf16(acc, a.h, b.l);
  mma_bf16(acc, a.h, b.h);
}

template <typename InT, int DK, int NTH>
__device__ __forceinline__ void Rows<InT, DK, NTH>::commit_split(uint16_t* dst, bool elu, float len, int patch,
                                                                 const float* pv) const {
  constexpr int LX = DK + 8, PX = CB * LX;
  // raw bf16 rows with the identity map and no rescaling are their own hi plane
  const bool exact = sizeof(InT) == 2 && !elu && !(len > 0.f);
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int idx = threadIdx.x + NTH * j, t = idx / GPR, i0 = (idx % GPR) * VW;
    if (exact && t != patch) {
      static_assert(VW == 8 || sizeof(InT) != 2, "one 16-byte group of bf16");
      *reinterpret_cast<u32x4*>(dst + t * LX + i0) = w[j];
      *reinterpret_cast<u32x4*>(dst + PX + t * LX + i0) = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    float x[VW];
    In<InT>::decode(w[j], x);
    if (t == patch) {
#pragma unroll
      for (int e = 0; e < VW; ++e) x[e] = pv != nullptr ? pv[i0 + e] : 0.f;
    } else if (elu && ((valid >> j) & 1u)) {
#pragma unroll
      for (int e = 0; e < VW; ++e) x[e] = phi_elu1(x[e]);
    }
    if (len > 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VW; ++e) ss += x[e] * x[e];
      ss = group_sum<GPR>(ss);
      const float f = rescale_factor(ss, len);
#pragma unroll
      for (int e = 0; e < VW; ++e) x[e] *= f;
    }
#pragma unroll
    for (int e = 0; e < VW; e += 4) put_split4(dst, PX, t * LX + i0 + e, f4{x[e], x[e + 1], x[e + 2], x[e + 3]});
  }
}

// acc += A B with B split and A exact when aex (its lo plane zero)
__device__ __forceinline__ void mma3a(f4& acc, const SFrag& a, const SFrag& b, bool aex) {
  if (!aex) mma_bf16(acc, a.l, b.h);
  mma_bf16(acc, a.h, b.l);
  mma_bf16(acc, a.h, b.h);
}

// Written keys x_t (Q == false) or read queries phi(q_t) (Q == true) of chunk c as split
// planes [CB][DK + 8]: the shift to the previous token's key (and the carried key before a
// call's first token), phi and QK normalisation applied; rows of tokens past T are zero.
// A row's 16-byte groups sit in GPR consecutive lanes, so its norm is a lane-group sum.
template <typename InT, int DK, bool SHIFT, bool Q, int NTH>
__device__ void stage_split(const BwdParams& p, int bh, int c, uint16_t* hi, bool has_in) {
  constexpr int LX = DK + 8, PX = CB * LX, VW = 16 / (int)sizeof(InT), GPR = DK / VW;
  static_assert(CB * GPR % NTH == 0 && 64 % GPR == 0, "row groups");
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(p.flags, DK);
  const size_t rb = (size_t)bh * p.T;
  const InT* src = static_cast<const InT*>(Q ? p.q : p.k) + rb * DK;
#pragma unroll
  for (int j = 0; j < CB * GPR / NTH; ++j) {
    const int idx = threadIdx.x + NTH * j, t = idx / GPR, i0 = (idx % GPR) * VW, tau = c * CB + t;
    float x[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) x[e] = 0.f;
    if (tau < p.T) {
      if (!Q && SHIFT && tau == 0) {
        if (has_in && p.xprev_in != nullptr) {
#pragma unroll
          for (int e = 0; e < VW; ++e) x[e] = p.xprev_in[(size_t)bh * DK + i0 + e];  // phi applied
        }
      } else {
        In<InT>::load(src + (size_t)(!Q && SHIFT ? tau - 1 : tau) * DK + i0, x);
        if (elu) {
#pragma unroll
          for (int e = 0; e < VW; ++e) x[e] = phi_elu1(x[e]);
        }
      }
    }
    if (len > 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VW; ++e) ss += x[e] * x[e];
      ss = group_sum<GPR>(ss);
      const float f = rescale_factor(ss, len);
#pragma unroll
      for (int e = 0; e < VW; ++e) x[e] *= f;
    }
#pragma unroll
    for (int e = 0; e < VW; e += 4) put_split4(hi, PX, t * LX + i0 + e, f4{x[e], x[e + 1], x[e + 2], x[e + 3]});
  }
}

__device__ __forceinline__ bool head_has_key(const BwdParams& p, int bh) {
  return p.has_in != nullptr && p.has_in[bh] != 0;
}

// ================================================================ prep: one (head, chunk)
template <typename InT, int DK, int RULE>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, float* recs) {
  using R = Rule<RULE>;
  constexpr int LDX = DK + 4;
  // X and Q rows; after the products Lp, M, T ([CB][LDC] each) and Y ([16][LDC])
  constexpr int kRows = 2 * CB * LDX, kTiles = 3 * CB * LDC + 16 * LDC;
  __shared__ __align__(16) float sm[kRows > kTiles ? kRows : kTiles];
  __shared__ float s_g[CB], s_gp[CB], s_e[CB], s_n[CB];
  __shared__ int s_par[CB], s_parp[CB];
  float* Xs = sm;
  float* Qs = sm + CB * LDX;
  const int nch = (p.T + CB - 1) / CB;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool has_in = head_has_key(p, bh);
  float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
  float* sc = rec + BRec::kSc;
  stage_rows<InT, DK, R::shift, true, true, 256>(p, bh, c, Xs, Qs, has_in);

  {
    // |x_t|^2: four threads a row
    const int t = tid >> 2, part = tid & 3;
    float nn = 0.f;
#pragma unroll 8
    for (int i = part; i < DK; i += 4) nn += Xs[t * LDX + i] * Xs[t * LDX + i];
    nn += __shfl_xor(nn, 1);
    nn += __shfl_xor(nn, 2);
    if (part == 0) s_n[t] = nn;
  }
  __syncthreads();
  if (wave == 0) {
    const int t = lane, tau = c * CB + t;
    const bool valid = tau < p.T;
    const float n = s_n[t];
    const size_t gi = (size_t)bh * p.T + (size_t)(valid ? tau : 0);
    const float beta = (valid && p.beta != nullptr) ? act_beta(p.beta[gi], p.flags) : 1.f;
    const float lam = (valid && p.lam != nullptr) ? act_lam(p.lam[gi], p.flags, R::nlms) : (R::nlms ? 0.f : 1.f);
    float e, a, den = 1.f, lu = 0.f;
    bool key;
    if constexpr (R::nlms) {
      key = valid && (tau >= 1 || has_in);
      lu = (p.flags & kFlagLamScaled) ? lam * n : lam;
      den = n + lu + p.eps;
      e = key ? beta / den : 0.f;
      a = key ? 1.f - e * lu : 1.f;
    } else {
      key = valid;
      e = valid ? beta : 0.f;
      a = valid ? lam : 1.f;
    }
    float la = log_abs_floor(a);
    int ng = a < 0.f ? 1 : 0;
    wave_prefix(la, ng);
    const float gend = __shfl(la, 63);
    const int pend = __shfl(ng, 63) & 1;
    const int par = ng & 1;
    // shuffles on every lane (a lane left out of a shuffle gives its readers no value)
    const float lsh = __shfl_up(la, 1);
    const int nsh = __shfl_up(ng, 1);
    const float gprev = t > 0 ? lsh : 0.f;
    const int pprev = t > 0 ? (nsh & 1) : 0;
    s_g[t] = la;
    s_gp[t] = gprev;
    s_par[t] = par;
    s_parp[t] = pprev;
    s_e[t] = e;
    sc[kScGam * CB + t] = sgn(par) * __expf(la);
    sc[kScGprev * CB + t] = sgn(pprev) * __expf(gprev);
    sc[kScGend * CB + t] = sgn(pend ^ par) * __expf(gend - la);
    sc[kScE * CB + t] = e;
    sc[kScA * CB + t] = a;
    sc[kScDen * CB + t] = den;
    sc[kScLu * CB + t] = lu;
    sc[kScN * CB + t] = n;
    sc[kScBeta * CB + t] = beta;
    sc[kScLam * CB + t] = lam;
    sc[kScKey * CB + t] = key ? 1.f : 0.f;
    sc[kScG * CB + t] = la;
    sc[kScPar * CB + t] = (float)par;
    if (t == 0) rec[BRec::kMisc] = sgn(pend) * __expf(gend);
  }

  // X X^T (shifted-pair rules and the delta rule's solve) and Q X^T: the ten lower tiles of
  // each, five per wave
  constexpr int NPROD = R::solve ? 2 : 1;
  constexpr int NTILE = 10 * NPROD;
  f4 acc[5];
  int tm[5], ts[5], tp[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int id = wave * 5 + k;
    acc[k] = f4{0.f, 0.f, 0.f, 0.f};
    tp[k] = -1;
    if (id < NTILE) {
      const int prod = id / 10, tile = id % 10;
      const int m = tile < 1 ? 0 : (tile < 3 ? 1 : (tile < 6 ? 2 : 3));
      const int s = tile - m * (m + 1) / 2;
      tm[k] = m;
      ts[k] = s;
      tp[k] = (NPROD == 1) ? 1 : prod;  // 0: X X^T, 1: Q X^T
      mm<false, false>(acc[k], (tp[k] == 0 ? Xs : Qs) + 16 * m * LDX, LDX, Xs + 16 * s * LDX, LDX, 0, DK, lane);
    }
  }
  __syncthreads();  // X and Q are no longer read; the scalars are in LDS

  // masked tiles into LDS: Lp = D' o G (strictly lower), M = D o P (lower with diagonal)
  float* Lps = sm;
  float* Ms = sm + CB * LDC;
  float* Ts = sm + 2 * CB * LDC;
  float* Ys = sm + 3 * CB * LDC;  // [16][LDC]
  for (int i = tid; i < (R::solve ? 3 : 1) * CB * LDC; i += 256) (R::solve ? sm : Ms)[i] = 0.f;
  __syncthreads();
  {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (tp[k] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tm[k] + 4 * g + i, s = 16 * ts[k] + n;
        if (tp[k] == 0) {
          if (s < t) Lps[t * LDC + s] = sgn(s_parp[t] ^ s_par[s]) * __expf(s_gp[t] - s_g[s]) * acc[k][i];
        } else {
          if (s <= t) Ms[t * LDC + s] = sgn(s_par[t] ^ s_par[s]) * __expf(s_g[t] - s_g[s]) * acc[k][i];
        }
      }
    }
  }
  __syncthreads();

  if constexpr (R::solve) {
    // T = (I + L)^-1 with L_ts = eta_t Lp_ts. Diagonal 16x16 blocks: wave b, lane j < 16
    // substitutes down column j of block b, the column in registers.
    if (lane < 16) {
      const int b = wave, j = lane;
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 16 * b + r;
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < r; ++k) v += Lps[tr * LDC + 16 * b + k] * col[k];
        col[r] = r < j ? 0.f : (r == j ? 1.f : -s_e[tr] * v);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Ts[(16 * b + r) * LDC + 16 * b + j] = col[r];
    }
    __syncthreads();
    // below the diagonal, by row blocks i: Y_j = diag(eta) sum_{k<i} Lp_ik T_kj, then
    // T_ij = -T_ii Y_j, one 16x16 tile j < i per wave on MFMA
    for (int ib = 1; ib < 4; ++ib) {
      if (wave < ib) {
        f4 y = {0.f, 0.f, 0.f, 0.f};
        mm<false, true>(y, Lps + 16 * ib * LDC, LDC, Ts + 16 * wave, LDC, 16 * wave, 16 * ib, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] *= s_e[16 * ib + 4 * (lane >> 4) + i];
        store_n(Ys, LDC, 0, 16 * wave, y, lane);
      }
      __syncthreads();
      if (wave < ib) {
        f4 t = {0.f, 0.f, 0.f, 0.f};
        mm<false, true>(t, Ts + 16 * ib * LDC + 16 * ib, LDC, Ys + 16 * wave, LDC, 0, 16, lane);
        store_n(Ts, LDC, 16 * ib, 16 * wave, -t, lane);
      }
      __syncthreads();
    }
  }

  // the record: T and Lp (delta rule), M. With bf16 inputs T and M are stored as bf16 hi
  // and lo planes ([CB][CB] each, in the float region's bytes), the operands of the split
  // kernels, so that each column-group workgroup copies them instead of splitting them.
  for (int e = tid; e < CB * CB / 4; e += 256) {
    const int r = e / (CB / 4), c4 = (e % (CB / 4)) * 4;
    const f4 mv = *reinterpret_cast<const f4*>(Ms + r * LDC + c4);
    if constexpr (sizeof(InT) == 2) put_split4(reinterpret_cast<uint16_t*>(rec + BRec::kM), CB * CB, r * CB + c4, mv);
    else *reinterpret_cast<f4*>(rec + BRec::kM + r * CB + c4) = mv;
    if constexpr (R::solve) {
      const f4 tv = *reinterpret_cast<const f4*>(Ts + r * LDC + c4);
      if constexpr (sizeof(InT) == 2) put_split4(reinterpret_cast<uint16_t*>(rec + BRec::kT), CB * CB, r * CB + c4, tv);
      else *reinterpret_cast<f4*>(rec + BRec::kT + r * CB + c4) = tv;
      *reinterpret_cast<f4*>(rec + BRec::kLp + r * CB + c4) = *reinterpret_cast<const f4*>(Lps + r * LDC + c4);
    }
  }
}

// Workgroup -> (head, 32-column group) of the serial kernels: the groups of one head sit on
// one XCD (blocks are dealt round-robin over the 8 XCDs) and share its L2.
__device__ __forceinline__ bool state_block(const BwdParams& p, int ngrp, int& bh, int& grp) {
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  grp = slot % ngrp;
  bh = (slot / ngrp) * 8 + xcd;
  return bh < p.BH;
}

// ====================================================== state: S at every chunk start
// Chunk c+1's rows, record and values are loaded into registers while chunk c computes.
template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(256) void bwd_state_kernel(BwdParams p, const float* recs, float* Sch, float* Rh) {
  using R = Rule<RULE>;
  constexpr int LDX = DK + 4, NRT = DK / 16, RPW = NRT / 4;  // row tiles of S per wave
  constexpr int VWv = 16 / (int)sizeof(InT), NVG = CB * NCOL / VWv;  // value groups
  constexpr int NVJ = (NVG + 255) / 256;
  __shared__ __align__(16) float Xs[CB * LDX];
  __shared__ __align__(16) float Ts[R::solve ? CB * LDC : 4];
  __shared__ __align__(16) float Bt[NCOL * LDX];  // S^T [NCOL][DK], then W^T [NCOL][LDC]
  __shared__ __align__(16) float Rt[R::solve ? NCOL * LDC : 4];
  __shared__ __align__(16) float Vs[CB * LDU];    // the chunk's values [CB][NCOL]
  // eta Gamma_prev, eta (or f), Gamma_end / Gamma, Gamma_prev; [4][0] Gamma_end
  __shared__ float s_fac[5][CB];
  int bh, grp;
  if (!state_block(p, DV / NCOL, bh, grp)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int nch = (p.T + CB - 1) / CB;
  const bool has_in = head_has_key(p, bh);
  const int col0 = grp * NCOL;
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(p.flags, DK);
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV + col0;

  f4 S[RPW][2];
#pragma unroll
  for (int a = 0; a < RPW; ++a)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (w + 4 * a) + 4 * g + i;
        S[a][ct][i] = p.S_in != nullptr ? p.S_in[(size_t)bh * SS + (size_t)r * DV + col0 + 16 * ct + n] : 0.f;
      }

  // registers of the next chunk: rows, T (16 floats a thread), values, scalars
  Rows<InT, DK, 256> rows;
  f4 pt[4];
  u32x4 pv[NVJ];
  float pf[5];
  auto load = [&](int c) {
    // row t is the key of token c CB + t - 1 for the shifted pair (token 0's is the carried key)
    rows.load(kb - (R::shift ? DK : 0), c * CB, R::shift ? 1 : 0, p.T);
    const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pt[j] = *reinterpret_cast<const f4*>(rec + BRec::kT + 16 * tid + 4 * j);
    }
#pragma unroll
    for (int j = 0; j < NVJ; ++j) {
      const int idx = tid + 256 * j, t = idx / (NCOL / VWv), v0 = (idx % (NCOL / VWv)) * VWv, tau = c * CB + t;
      pv[j] = u32x4{0u, 0u, 0u, 0u};
      if (idx < NVG && tau < p.T) pv[j] = *reinterpret_cast<const u32x4*>(vb + (size_t)tau * DV + v0);
    }
    if (tid < CB) {
      const float* sc = rec + BRec::kSc;
      const float e = sc[kScE * CB + tid];
      pf[0] = e * sc[kScGprev * CB + tid];
      pf[1] = e;
      pf[2] = sc[kScGend * CB + tid];
      pf[3] = sc[kScGprev * CB + tid];
      pf[4] = rec[BRec::kMisc];
    }
  };
  auto commit = [&](int c) {
    // the carried key (phi applied) before the call's first token
    const float* x0 = (R::shift && has_in && p.xprev_in != nullptr) ? p.xprev_in + (size_t)bh * DK : nullptr;
    rows.commit(Xs, elu, len, (R::shift && c == 0) ? 0 : -1, x0);
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<f4*>(Ts + (tid >> 2) * LDC + 16 * (tid & 3) + 4 * j) = pt[j];
    }
#pragma unroll
    for (int j = 0; j < NVJ; ++j) {
      const int idx = tid + 256 * j, t = idx / (NCOL / VWv), v0 = (idx % (NCOL / VWv)) * VWv;
      if (idx < NVG) {
        float x[VWv];
        In<InT>::decode(pv[j], x);
#pragma unroll
        for (int e = 0; e < VWv; e += 4) *reinterpret_cast<f4*>(Vs + t * LDU + v0 + e) = f4{x[e], x[e + 1], x[e + 2], x[e + 3]};
      }
    }
    if (tid < CB) {
#pragma unroll
      for (int k = 0; k < 4; ++k) s_fac[k][tid] = pf[k];
      if (tid == 0) s_fac[4][0] = pf[4];
    }
  };
  // the delta rule needs every chunk's data (R-hat of the last chunk too), the others
  // every chunk's but the last
  if (R::solve || nch > 1) load(0);

  for (int c = 0; c < nch; ++c) {
    float* Sc = Sch + ((size_t)bh * nch + c) * SS;
#pragma unroll
    for (int a = 0; a < RPW; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Sc[(size_t)(16 * (w + 4 * a) + 4 * g + i) * DV + col0 + 16 * ct + n] = S[a][ct][i];
    if (!R::solve && c + 1 == nch) break;  // the state after the last chunk is not needed
    lds_barrier();  // the previous chunk's LDS reads are done
    commit(c);
    if constexpr (R::solve) {
#pragma unroll
      for (int a = 0; a < RPW; ++a)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) store_t(Bt, LDX, 16 * (w + 4 * a), 16 * ct, S[a][ct], lane);
    }
    lds_barrier();
    if (c + 1 < nch && (R::solve || c + 2 < nch)) load(c + 1);

    // this wave's token tile w: W = fU U with U = T R (delta) or fV V
    f4 W[2];
    if constexpr (R::solve) {
      // R-hat = V - Gamma_prev X S, kept for the gradient pass, and R = eta R-hat
      float* rh = Rh + ((size_t)bh * nch + c) * CB * DV + col0;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f4 xs = {0.f, 0.f, 0.f, 0.f};
        mm<false, false>(xs, Xs + 16 * w * LDX, LDX, Bt + 16 * ct * LDX, LDX, 0, DK, lane);
        f4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * w + 4 * g + i;
          const float rhat = Vs[t * LDU + 16 * ct + n] - s_fac[3][t] * xs[i];
          rh[(size_t)t * DV + 16 * ct + n] = rhat;
          r[i] = s_fac[1][t] * rhat;
        }
        store_t(Rt, LDC, 16 * w, 16 * ct, r, lane);
      }
      if (c + 1 == nch) break;  // the state after the last chunk is not needed
      lds_barrier();
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f4 u = {0.f, 0.f, 0.f, 0.f};
        mm<false, false>(u, Ts + 16 * w * LDC, LDC, Rt + 16 * ct * LDC, LDC, 0, 16 * w + 16, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) W[ct][i] = s_fac[2][16 * w + 4 * g + i] * u[i];
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * w + 4 * g + i;
          W[ct][i] = s_fac[2][t] * s_fac[1][t] * Vs[t * LDU + 16 * ct + n];
        }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) store_t(Bt, LDC, 16 * w, 16 * ct, W[ct], lane);
    lds_barrier();
    // S' = Gamma_end S + X^T W
    const float gend = s_fac[4][0];
#pragma unroll
    for (int a = 0; a < RPW; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        S[a][ct] *= gend;
        mm<true, false>(S[a][ct], Xs + 16 * (w + 4 * a), LDX, Bt + 16 * ct * LDC, LDC, 0, CB, lane);
      }
  }
}

// ================================================= dstate: the exit gradient of every chunk
// Chunk c-1's rows, records and dO are loaded into registers while chunk c computes.
template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(512) void bwd_dstate_kernel(BwdParams p, const float* recs, float* dSch, float* dRw) {
  using R = Rule<RULE>;
  constexpr int LDX = DK + 4, NRT = DK / 16;
  // dS tiles: 2 * NRT over 8 waves (DK 128: row tile w, both column tiles; DK 64: row tile
  // w % 4, column tile w / 4)
  constexpr int NTW = NRT / 4;
  __shared__ __align__(16) float Xs[CB * LDX];
  __shared__ __align__(16) float Qs[CB * LDX];
  __shared__ __align__(16) float Ts[R::solve ? CB * LDC : 4];
  __shared__ __align__(16) float Ms[R::solve ? CB * LDC : 4];
  __shared__ __align__(16) float dOt[NCOL * LDC];  // dO^T of the column group
  __shared__ __align__(16) float Bt[NCOL * LDX];   // dS^T, then (delta) (eta Gamma_prev dR)^T
  __shared__ __align__(16) float dUt[R::solve ? NCOL * LDC : 4];
  __shared__ __align__(16) float s_fac[4][CB];  // Gamma, eta Gamma_prev, Gamma_end / Gamma; [3][0] Gamma_end
  int bh, grp;
  if (!state_block(p, DV / NCOL, bh, grp)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int nch = (p.T + CB - 1) / CB;
  const bool has_in = head_has_key(p, bh);
  const int col0 = grp * NCOL;
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(p.flags, DK);
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* qb = static_cast<const InT*>(p.q) + rb * DK;
  const float* dob = p.dout + rb * DV + col0;
  auto tile_rt = [&](int a) { return NTW == 2 ? w : (w & 3); };
  auto tile_ct = [&](int a) { return NTW == 2 ? a : (w >> 2); };

  f4 dS[NTW];
#pragma unroll
  for (int a = 0; a < NTW; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * tile_rt(a) + 4 * g + i;
      dS[a][i] = p.dS_out != nullptr ? p.dS_out[(size_t)bh * SS + (size_t)r * DV + col0 + 16 * tile_ct(a) + n] : 0.f;
    }
  const int m = w & 3, ctw = w >> 2;  // this wave's (token tile, column tile) of dU and dR

  // registers of the next chunk: X and Q rows, T and M (8 floats a thread each), dO (4), scalars
  Rows<InT, DK, 512> xrows, qrows;
  f4 pt[2], pm[2], pd;
  float pf[4];
  auto load = [&](int c) {
    xrows.load(kb - (R::shift ? DK : 0), c * CB, R::shift ? 1 : 0, p.T);
    qrows.load(qb, c * CB, 0, p.T);
    const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        pt[j] = *reinterpret_cast<const f4*>(rec + BRec::kT + 8 * tid + 4 * j);
        pm[j] = *reinterpret_cast<const f4*>(rec + BRec::kM + 8 * tid + 4 * j);
      }
    }
    {
      const int t = tid / (NCOL / 4), v0 = (tid % (NCOL / 4)) * 4, tau = c * CB + t;
      pd = tau < p.T ? *reinterpret_cast<const f4*>(dob + (size_t)tau * DV + v0) : f4{0.f, 0.f, 0.f, 0.f};
    }
    if (tid < CB) {
      const float* sc = rec + BRec::kSc;
      pf[0] = sc[kScGam * CB + tid];
      pf[1] = sc[kScE * CB + tid] * sc[kScGprev * CB + tid];
      pf[2] = sc[kScGend * CB + tid];
      pf[3] = rec[BRec::kMisc];
    }
  };
  auto commit = [&](int c) {
    const float* x0 = (R::shift && has_in && p.xprev_in != nullptr) ? p.xprev_in + (size_t)bh * DK : nullptr;
    xrows.commit(Xs, elu, len, (R::shift && c == 0) ? 0 : -1, x0);
    qrows.commit(Qs, elu, len, -1, nullptr);
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        *reinterpret_cast<f4*>(Ts + (tid >> 3) * LDC + 8 * (tid & 7) + 4 * j) = pt[j];
        *reinterpret_cast<f4*>(Ms + (tid >> 3) * LDC + 8 * (tid & 7) + 4 * j) = pm[j];
      }
    }
    {
      const int t = tid / (NCOL / 4), v0 = (tid % (NCOL / 4)) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) dOt[(v0 + i) * LDC + t] = pd[i];
    }
    if (tid < CB) {
      s_fac[0][tid] = pf[0];
      s_fac[1][tid] = pf[1];
      s_fac[2][tid] = pf[2];
      if (tid == 0) s_fac[3][0] = pf[3];
    }
  };
  load(nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    float* dSc = dSch + ((size_t)bh * nch + c) * SS;
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dSc[(size_t)(16 * tile_rt(a) + 4 * g + i) * DV + col0 + 16 * tile_ct(a) + n] = dS[a][i];
    lds_barrier();  // the previous chunk's LDS reads are done
    commit(c);
#pragma unroll
    for (int a = 0; a < NTW; ++a) store_t(Bt, LDX, 16 * tile_rt(a), 16 * tile_ct(a), dS[a], lane);
    lds_barrier();
    if (c >= 1) load(c - 1);

    if constexpr (R::solve) {
      // dU = M^T dO + (Gamma_end / Gamma) X dS' for token tile m, column tile ctw (only the
      // delta rule's state gradient goes through the writes)
      f4 du = {0.f, 0.f, 0.f, 0.f};
      mm<false, false>(du, Xs + 16 * m * LDX, LDX, Bt + 16 * ctw * LDX, LDX, 0, DK, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] *= s_fac[2][16 * m + 4 * g + i];
      mm<true, false>(du, Ms + 16 * m, LDC, dOt + 16 * ctw * LDC, LDC, 16 * m, CB, lane);
      store_t(dUt, LDC, 16 * m, 16 * ctw, du, lane);
      lds_barrier();  // dU complete; dS^T no longer read
      f4 dr = {0.f, 0.f, 0.f, 0.f};
      mm<true, false>(dr, Ts + 16 * m, LDC, dUt + 16 * ctw * LDC, LDC, 16 * m, CB, lane);
      // dR, kept for the gradient pass
      float* drw = dRw + ((size_t)bh * nch + c) * CB * DV + col0 + 16 * ctw + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        drw[(size_t)(16 * m + 4 * g + i) * DV] = dr[i];
        dr[i] *= s_fac[1][16 * m + 4 * g + i];
      }
      store_t(Bt, LDC, 16 * m, 16 * ctw, dr, lane);
      lds_barrier();
    }
    // dS = Gamma_end dS' + Q^T diag(Gamma) dO - X^T (eta Gamma_prev dR)
    const float gend = s_fac[3][0];
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
      const int rt = tile_rt(a), ct = tile_ct(a);
      dS[a] *= gend;
      for (int k = 0; k < CB; k += 16) {
        f4 av, bv;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = Qs[(k + 4 * g + i) * LDX + 16 * rt + n];
        bv = *reinterpret_cast<const f4*>(dOt + (16 * ct + n) * LDC + k + 4 * g) *
             *reinterpret_cast<const f4*>(&s_fac[0][k + 4 * g]);
        mfma4(dS[a], av, bv);
      }
      if constexpr (R::solve) {
        f4 t = {0.f, 0.f, 0.f, 0.f};
        mm<true, false>(t, Xs + 16 * rt, LDX, Bt + 16 * ct * LDC, LDC, 0, CB, lane);
        dS[a] -= t;
      }
    }
  }
  if (p.gS0 != nullptr) {
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.gS0[(size_t)bh * SS + (size_t)(16 * tile_rt(a) + 4 * g + i) * DV + col0 + 16 * tile_ct(a) + n] = dS[a][i];
    if (grp == 0 && tid == 0 && p.gh0 != nullptr) p.gh0[bh] = 0;
  }
}

// ==================================================== grad: every gradient of one chunk
// Partial per-token sums, each slot written by one lane per token (no atomics).
enum {
  kPdQ0, kPdQ1,      // q_t . dQ1_t (two halves of the d_k tiles)
  kPdXR0, kPdXR1,    // x_t . dXR_t (to the log decay of token t-1)
  kPh0, kPh1,        // h_t = x_t . dXS_t
  kPMr,              // row sums of dMm o M
  kPMc0,             // column sums of dMm o M by the wave of row tile 0..3 (4 slots)
  kPLr = kPMc0 + 4,  // row sums of dLm o L (to token t-1)
  kPLc0,             // column sums of dLm o L (4 slots)
  kPeL = kPLc0 + 4,  // row sums of dLm o Lp (eta's gradient through L)
  kPe0, kPe1,        // eta's (or f's) gradient through the values, by column tile
  kNP
};

// Gradient pass on fp32 MFMA (float32 inputs, whose gradients are held to float32 accuracy).
template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(512) void bwd_grad_f32_kernel(BwdParams p, const float* recs, const float* Sch,
                                                        const float* dSch, const float* Rh, const float* dRw) {
  using R = Rule<RULE>;
  constexpr bool SOLVE = R::solve;
  constexpr int LDX = DK + 4, NDT = DK / 16, DPW = NDT / 2;  // d_k tiles per wave
  constexpr int NBLK = DV / NCOL;
  // LDS: X, T, M, and a region for one value block (phase 1) or Q, A1, W (phase 2). A value
  // block: S and dS' [DK][NCOL], dO and U [CB][NCOL] in natural layout (every K = d_v
  // product reads 16-byte operand runs); the delta rule adds dR [CB][NCOL] and R^T
  // [NCOL][CB] (from the state passes' R-hat and dR), the other rules dS'^T [NCOL][DK] and
  // dO^T [NCOL][CB] for dU = M^T dO + (Gamma_end / Gamma) X dS'.
  constexpr int kBlk1 = 2 * DK * LDU + 2 * CB * LDU + (SOLVE ? CB * LDU + NCOL * LDC : NCOL * LDX + NCOL * LDC);
  constexpr int kBlk2 = CB * LDX + 2 * CB * LDC;
  constexpr int kBlk = kBlk1 > kBlk2 ? kBlk1 : kBlk2;
  __shared__ __align__(16) float Xs[CB * LDX];
  __shared__ __align__(16) float Ts[SOLVE ? CB * LDC : 4];  // T, then Lp
  __shared__ __align__(16) float Ms[CB * LDC];
  __shared__ __align__(16) float blk[kBlk];
  __shared__ float s_sc[kNSc][CB];
  __shared__ float s_p[kNP][CB];
  __shared__ float s_dn[CB];
  __shared__ float s_red[8];
  float* Sn = blk;                     // S block [DK][NCOL]
  float* dSn = Sn + DK * LDU;          // dS' block
  float* dOn = dSn + DK * LDU;         // dO [CB][NCOL]
  float* Un = dOn + CB * LDU;          // U [CB][NCOL]
  float* dRn = Un + CB * LDU;          // dR [CB][NCOL] (delta)
  float* Rt = dRn + CB * LDU;          // R^T [NCOL][CB] (delta)
  float* dSt = Un + CB * LDU;          // dS'^T [NCOL][DK] (other rules)
  float* dOt = dSt + NCOL * LDX;       // dO^T [NCOL][CB] (other rules)
  float* Qs = blk;                     // phase 2: Q [CB][DK]
  float* A1 = blk + CB * LDX;          // dMm o D [CB][CB]
  float* Wn = A1 + CB * LDC;           // dLm o eta D' [CB][CB] (delta)

  const int nch = (p.T + CB - 1) / CB;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const bool has_in = head_has_key(p, bh);
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const int t0 = c * CB;
  const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
  const float* Sc = Sch + ((size_t)bh * nch + c) * SS;
  const float* dSc = dSch + ((size_t)bh * nch + c) * SS;
  const float* rhc = Rh + ((size_t)bh * nch + c) * CB * DV;
  const float* drc = dRw + ((size_t)bh * nch + c) * CB * DV;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV;

  for (int e = tid; e < CB * CB / 4; e += 512) {
    const int r = e / (CB / 4), c4 = (e % (CB / 4)) * 4;
    *reinterpret_cast<f4*>(Ms + r * LDC + c4) = *reinterpret_cast<const f4*>(rec + BRec::kM + r * CB + c4);
    if constexpr (SOLVE)
      *reinterpret_cast<f4*>(Ts + r * LDC + c4) = *reinterpret_cast<const f4*>(rec + BRec::kT + r * CB + c4);
  }
  for (int e = tid; e < kNSc * CB; e += 512) (&s_sc[0][0])[e] = rec[BRec::kSc + e];
  for (int e = tid; e < kNP * CB; e += 512) (&s_p[0][0])[e] = 0.f;
  stage_rows<InT, DK, R::shift, true, false, 512>(p, bh, c, Xs, nullptr, has_in);

  const int m = w & 3, ctw = w >> 2;  // token tile and column tile of this wave's block outputs
  // accumulators over the value blocks
  f4 aMm[4], aQ1[DPW], aXR[DPW], aXS[DPW];  // aMm: dMm (w < 4) or dLm (w >= 4) tiles (m, s <= m)
#pragma unroll
  for (int s = 0; s < 4; ++s) aMm[s] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < DPW; ++d) aQ1[d] = aXR[d] = aXS[d] = f4{0.f, 0.f, 0.f, 0.f};
  f4 pe = {0.f, 0.f, 0.f, 0.f};  // eta's gradient through the values, this lane's rows
  float sds = 0.f;               // <dS', S> partial

  auto fac = [&](int k, int t) { return s_sc[k][t]; };

  // the next value block in registers: S and dS' (NSJ f4 a thread each), dO and (delta) dR
  // (one f4 each), and this lane's four values of R-hat (delta) or V (other rules)
  constexpr int NSJ = DK * NCOL / 4 / 512;
  f4 ps[NSJ], pds[NSJ], pdo, pdr;
  float pv4[4];
  auto load_blk = [&](int jb) {
    const int col0 = jb * NCOL;
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int e = tid + 512 * j, r = e / (NCOL / 4), v4 = (e % (NCOL / 4)) * 4;
      ps[j] = *reinterpret_cast<const f4*>(Sc + (size_t)r * DV + col0 + v4);
      pds[j] = *reinterpret_cast<const f4*>(dSc + (size_t)r * DV + col0 + v4);
    }
    {
      const int t = tid / (NCOL / 4), v4 = (tid % (NCOL / 4)) * 4, tau = t0 + t;
      pdo = tau < p.T ? *reinterpret_cast<const f4*>(p.dout + (rb + tau) * DV + col0 + v4) : f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (SOLVE) pdr = *reinterpret_cast<const f4*>(drc + (size_t)t * DV + col0 + v4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * m + 4 * g + i, tau = t0 + t, cc = col0 + 16 * ctw + n;
      if constexpr (SOLVE) pv4[i] = rhc[(size_t)t * DV + cc];
      else pv4[i] = tau < p.T ? In<InT>::load1(vb + (size_t)tau * DV + cc) : 0.f;
    }
  };
  load_blk(0);

  for (int jb = 0; jb < NBLK; ++jb) {
    const int col0 = jb * NCOL;
    // the block into LDS from registers
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int e = tid + 512 * j, r = e / (NCOL / 4), v4 = (e % (NCOL / 4)) * 4;
      *reinterpret_cast<f4*>(Sn + r * LDU + v4) = ps[j];
      *reinterpret_cast<f4*>(dSn + r * LDU + v4) = pds[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sds += ps[j][i] * pds[j][i];
        if (!SOLVE) dSt[(v4 + i) * LDX + r] = pds[j][i];
      }
    }
    {
      const int t = tid / (NCOL / 4), v4 = (tid % (NCOL / 4)) * 4;
      *reinterpret_cast<f4*>(dOn + t * LDU + v4) = pdo;
      if constexpr (SOLVE) {
        *reinterpret_cast<f4*>(dRn + t * LDU + v4) = pdr;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dOt[(v4 + i) * LDC + t] = pdo[i];
      }
    }
    float v4r[4];  // R-hat (delta) or V, this lane's rows
#pragma unroll
    for (int i = 0; i < 4; ++i) v4r[i] = pv4[i];
    if constexpr (SOLVE) {
      f4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = fac(kScE, 16 * m + 4 * g + i) * v4r[i];
      store_t(Rt, LDC, 16 * m, 16 * ctw, r, lane);
    } else {
      f4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = fac(kScE, 16 * m + 4 * g + i) * v4r[i];
      store_n(Un, LDU, 16 * m, 16 * ctw, u, lane);
    }
    lds_barrier();
    if (jb + 1 < NBLK) load_blk(jb + 1);

    if constexpr (SOLVE) {
      // U = T R; dV = eta dR; eta's gradient through R-hat
      f4 u = {0.f, 0.f, 0.f, 0.f};
      mm<false, false>(u, Ts + 16 * m * LDC, LDC, Rt + 16 * ctw * LDC, LDC, 0, 16 * m + 16, lane);
      store_n(Un, LDU, 16 * m, 16 * ctw, u, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i, tau = t0 + t;
        const float dr = dRn[t * LDU + 16 * ctw + n];
        pe[i] += dr * v4r[i];
        if (tau < p.T) p.gv[(rb + tau) * DV + col0 + 16 * ctw + n] = fac(kScE, t) * dr;
      }
    } else {
      // dU = M^T dO + (Gamma_end / Gamma) X dS'; dV = f dU; f's gradient through V
      f4 du = {0.f, 0.f, 0.f, 0.f};
      mm<false, false>(du, Xs + 16 * m * LDX, LDX, dSt + 16 * ctw * LDX, LDX, 0, DK, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] *= fac(kScGend, 16 * m + 4 * g + i);
      mm<true, false>(du, Ms + 16 * m, LDC, dOt + 16 * ctw * LDC, LDC, 16 * m, CB, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i, tau = t0 + t;
        pe[i] += du[i] * v4r[i];
        if (tau < p.T) p.gv[(rb + tau) * DV + col0 + 16 * ctw + n] = fac(kScE, t) * du[i];
      }
    }
    lds_barrier();

    // accumulate over the block's columns: dMm = dO U^T (w < 4), dLm = -dR U^T (w >= 4),
    // dQ1 = dO S^T, dXR = dR S^T, dXS = U dS'^T
    if (w < 4) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s <= m) mm<false, false>(aMm[s], dOn + 16 * m * LDU, LDU, Un + 16 * s * LDU, LDU, 0, NCOL, lane);
    } else if constexpr (SOLVE) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s <= m) mm<false, false>(aMm[s], dRn + 16 * m * LDU, LDU, Un + 16 * s * LDU, LDU, 0, NCOL, lane);
    }
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dt = ctw * DPW + d;
      mm<false, false>(aQ1[d], dOn + 16 * m * LDU, LDU, Sn + 16 * dt * LDU, LDU, 0, NCOL, lane);
      if constexpr (SOLVE) mm<false, false>(aXR[d], dRn + 16 * m * LDU, LDU, Sn + 16 * dt * LDU, LDU, 0, NCOL, lane);
      mm<false, false>(aXS[d], Un + 16 * m * LDU, LDU, dSn + 16 * dt * LDU, LDU, 0, NCOL, lane);
    }
    lds_barrier();
  }

  // ---- phase 2
  // <dS', S> over the workgroup
  sds = wave_sum(sds);
  if (lane == 0) s_red[w] = sds;
  // eta's (or f's) gradient through the values: this lane's four rows, summed over columns
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = sum16(pe[i]);
    if (n == 0) s_p[kPe0 + ctw][16 * m + 4 * g + i] = v;
  }
  // row dots with the state-coupled terms, after their row factors
  {
    float pq[4] = {0.f, 0.f, 0.f, 0.f}, pr[4] = {0.f, 0.f, 0.f, 0.f}, ph[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        aQ1[d][i] *= fac(kScGam, t);
        aXR[d][i] *= -fac(kScE, t) * fac(kScGprev, t);
        aXS[d][i] *= fac(kScGend, t);
        const float x = Xs[t * LDX + dc];
        pr[i] += x * aXR[d][i];
        ph[i] += x * aXS[d][i];
      }
    }
    // q . dQ1 needs Q, staged below; keep the x dots now
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = sum16(pr[i]), h = sum16(ph[i]);
      if (n == 0) {
        s_p[kPdXR0 + ctw][16 * m + 4 * g + i] = r;
        s_p[kPh0 + ctw][16 * m + 4 * g + i] = h;
      }
      pq[i] = 0.f;
    }
    __syncthreads();  // phase-1 block buffers free
    stage_rows<InT, DK, R::shift, false, true, 512>(p, bh, c, nullptr, Qs, has_in);
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) pq[i] += Qs[(16 * m + 4 * g + i) * LDX + dc] * aQ1[d][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q = sum16(pq[i]);
      if (n == 0) s_p[kPdQ0 + ctw][16 * m + 4 * g + i] = q;
    }
  }
  // A1 = dMm o D with the row and column sums of dMm o M (waves 0-3), W = dLm o eta D' with
  // the row and column sums of dLm o L and the row sums of dLm o Lp (waves 4-7); Lp
  // replaces T in LDS
  if constexpr (SOLVE) {
    __syncthreads();  // T no longer read
    for (int e = tid; e < CB * CB / 4; e += 512) {
      const int r = e / (CB / 4), c4 = (e % (CB / 4)) * 4;
      *reinterpret_cast<f4*>(Ts + r * LDC + c4) = *reinterpret_cast<const f4*>(rec + BRec::kLp + r * CB + c4);
    }
  }
  for (int e = tid; e < CB * LDC; e += 512) {
    A1[e] = 0.f;
    if (SOLVE) Wn[e] = 0.f;
  }
  __syncthreads();
  {
    const float* gl = s_sc[kScG];
    const float* pa = s_sc[kScPar];
    float rs[4] = {0.f, 0.f, 0.f, 0.f}, rs2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s > m) continue;
      float cs = 0.f;
      const int sc = 16 * s + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        if (w < 4) {
          if (sc <= t) {
            const float d = sgn((int)pa[t] ^ (int)pa[sc]) * __expf(gl[t] - gl[sc]);
            const float v = aMm[s][i];
            A1[t * LDC + sc] = v * d;
            const float pm = v * Ms[t * LDC + sc];
            rs[i] += pm;
            cs += pm;
          }
        } else if constexpr (SOLVE) {
          if (sc < t) {
            const float dl = -aMm[s][i];  // dLm = -dR U^T (the waves accumulated dR U^T)
            const float lp = Ts[t * LDC + sc];  // D'_ts (x_t . x_s)
            const float e = fac(kScE, t);
            const float dp = sgn((int)pa[t - 1] ^ (int)pa[sc]) * __expf(gl[t - 1] - gl[sc]);  // D'_ts
            Wn[t * LDC + sc] = dl * e * dp;
            rs[i] += dl * e * lp;   // dLm o L
            rs2[i] += dl * lp;      // dLm o Lp
            cs += dl * e * lp;
          }
        }
      }
      // column sums over this tile's 16 rows: the four lane groups
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (g == 0) {
        if (w < 4) s_p[kPMc0 + m][sc] += cs;
        else if (SOLVE) s_p[kPLc0 + m][sc] += cs;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = sum16(rs[i]), b = sum16(rs2[i]);
      if (n == 0) {
        const int t = 16 * m + 4 * g + i;
        if (w < 4) s_p[kPMr][t] = a;
        else if (SOLVE) {
          s_p[kPLr][t] = a;
          s_p[kPeL][t] = b;
        }
      }
    }
  }
  __syncthreads();

  // dQ = dQ1 + A1 X;  dX = dXR + dXS + A1^T Q + W X + W^T X (this wave: token tile m, d_k
  // tiles ctw * DPW ...)
  f4 dQ[DPW], dX[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int dt = ctw * DPW + d;
    dQ[d] = aQ1[d];
    mm<false, true>(dQ[d], A1 + 16 * m * LDC, LDC, Xs + 16 * dt, LDX, 0, 16 * m + 16, lane);
    dX[d] = aXR[d] + aXS[d];
    mm<true, true>(dX[d], A1 + 16 * m, LDC, Qs + 16 * dt, LDX, 16 * m, CB, lane);
    if constexpr (SOLVE) {
      mm<false, true>(dX[d], Wn + 16 * m * LDC, LDC, Xs + 16 * dt, LDX, 0, 16 * m + 16, lane);
      mm<true, true>(dX[d], Wn + 16 * m, LDC, Xs + 16 * dt, LDX, 16 * m, CB, lane);
    }
  }

  // the log decays' gradient, its suffix sums, and the scalar chain (wave 0, lane = token)
  if (w == 0) {
    const int t = lane;
    const float hsum = wave_sum(s_p[kPh0][t] + s_p[kPh1][t]);
    float dg = s_p[kPdQ0][t] + s_p[kPdQ1][t] - s_p[kPh0][t] - s_p[kPh1][t] + s_p[kPMr][t];
#pragma unroll
    for (int k = 0; k < 4; ++k) dg -= s_p[kPMc0 + k][t];
    if (t + 1 < CB) dg += s_p[kPdXR0][t + 1] + s_p[kPdXR1][t + 1];
    if constexpr (SOLVE) {
      if (t + 1 < CB) dg += s_p[kPLr][t + 1];
#pragma unroll
      for (int k = 0; k < 4; ++k) dg -= s_p[kPLc0 + k][t];
    }
    if (t == CB - 1) {
      float sd = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) sd += s_red[k];
      dg += hsum + rec[BRec::kMisc] * sd;
    }
    // suffix sums: dl_t = sum_{t' >= t} dg_t'
    float dl = dg;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(dl, o);
      if (t + o < 64) dl += y;
    }
    const float a = fac(kScA, t);
    const float af = (a < 0.f ? -1.f : 1.f) * fmaxf(fabsf(a), 1e-30f);
    const float da = dl / af;
    const int tau = t0 + t;
    float dn = 0.f;
    if (tau < p.T) {
      const float beta = fac(kScBeta, t), lam = fac(kScLam, t);
      const bool key = fac(kScKey, t) != 0.f;
      float gb = 0.f, gl = 0.f;
      if constexpr (R::nlms) {
        if (key) {
          const float e = fac(kScE, t), den = fac(kScDen, t), lu = fac(kScLu, t), nx = fac(kScN, t);
          float de = s_p[kPe0][t] + s_p[kPe1][t];
          if (SOLVE) de += s_p[kPeL][t];
          de -= lu * da;
          gb = de / den;
          const float dden = -e * de / den;
          const float dlu = -e * da + dden;
          const bool scaled = (p.flags & kFlagLamScaled) != 0;
          dn = dden + (scaled ? lam * dlu : 0.f);
          gl = dlu * (scaled ? nx : 1.f);
        }
      } else {
        gb = s_p[kPe0][t] + s_p[kPe1][t];
        gl = da;
      }
      // with pre-activated gates: the gradient with respect to the pre-activation
      if (p.flags & kFlagBetaSig) gb *= beta * (1.f - beta);
      else if (p.flags & kFlagBetaSig2) gb *= beta * (1.f - 0.5f * beta);
      if (p.flags & kFlagLamAct) gl *= R::nlms ? -expm1f(-lam) : lam * (1.f - lam);
      if (p.gbeta != nullptr) p.gbeta[rb + tau] = gb;
      if (p.glam != nullptr) p.glam[rb + tau] = gl;
    }
    s_dn[t] = dn;
  }
  __syncthreads();

  // the feature maps' derivative from the staged values y = phi(z): 1 for the identity;
  // for elu+1, 1 where y > 1 (z > 0) and y = exp(z) elsewhere
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  auto dphi = [&](float y) { return elu ? (y > 1.f ? 1.f : y) : 1.f; };
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * m + 4 * g + i, tau = t0 + t;
      const float x = Xs[t * LDX + dc];
      const float gx = dX[d][i] + 2.f * s_dn[t] * x;
      if (tau < p.T) p.gq[(rb + tau) * DK + dc] = dQ[d][i] * dphi(Qs[t * LDX + dc]);
      if constexpr (R::shift) {
        // x_t is the key of token tau - 1 (the carried key before the first token)
        if (tau >= 1 && tau < p.T) p.gk[(rb + tau - 1) * DK + dc] = gx * dphi(x);
        else if (tau == 0 && p.gx0 != nullptr) p.gx0[(size_t)bh * DK + dc] = has_in ? gx : 0.f;
      } else {
        if (tau < p.T) p.gk[(rb + tau) * DK + dc] = gx * dphi(x);
      }
    }
  }
  if constexpr (R::shift) {
    // the last key is written by no step of this call
    if (c == nch - 1)
      for (int i = tid; i < DK; i += 512) p.gk[(rb + p.T - 1) * DK + i] = 0.f;
  } else {
    if (c == 0 && p.gx0 != nullptr)
      for (int i = tid; i < DK; i += 512) p.gx0[(size_t)bh * DK + i] = 0.f;
  }
}

// Gradient pass on bf16 MFMA with split operands (bf16 inputs).
template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(512) void bwd_grad_kernel(BwdParams p, const float* recs, const float* Sch,
                                                        const float* dSch, const float* Rh, const float* dRw) {
  using R = Rule<RULE>;
  constexpr bool SOLVE = R::solve;
  constexpr int NDT = DK / 16, DPW = NDT / 2;  // d_k tiles, and those of one wave
  constexpr int NBLK = DV / NCOL;
  // bf16 plane row strides and plane sizes (elements)
  constexpr int LX = DK + 8, LC = CB + 8, LB = NCOL + 8;
  constexpr int PX = CB * LX, PC = CB * LC, PS = DK * LB, PB = CB * LB;
  // Block region. Phase 1 (one 32-column value block): S and dS' [DK][NCOL], dO and U
  // [CB][NCOL], for the delta rule also dR and R = eta R-hat [CB][NCOL]. Phase 2: Q
  // [CB][DK], A1 = dMm o D [CB][CB], for the delta rule W = dLm o eta D' [CB][CB].
  constexpr int kBlk1 = 4 * PS + 2 * (SOLVE ? 4 : 2) * PB;
  constexpr int kBlk2 = 2 * PX + 2 * (SOLVE ? 2 : 1) * PC;
  constexpr int kBlk = kBlk1 > kBlk2 ? kBlk1 : kBlk2;
  static_assert(2 * PC * 2 >= CB * LDC * 4, "Lp fits the T planes");
  __shared__ __align__(16) uint16_t Xp[2 * PX];
  __shared__ __align__(16) uint16_t Tp[2 * PC];  // T (delta rule) or M (other rules); then Lp fp32
  __shared__ __align__(16) float Ms[CB * LDC];   // M in fp32 (the decay gradient's sums)
  __shared__ __align__(16) uint16_t blk[kBlk];
  __shared__ float s_sc[kNSc][CB];
  __shared__ float s_p[kNP][CB];
  __shared__ float s_dn[CB];
  __shared__ float s_red[8];
  uint16_t* Sp = blk;
  uint16_t* dSp = Sp + 2 * PS;
  uint16_t* dOp = dSp + 2 * PS;
  uint16_t* Up = dOp + 2 * PB;
  uint16_t* dRp = Up + 2 * PB;  // delta
  uint16_t* Rp = dRp + 2 * PB;  // delta
  uint16_t* Qp = blk;           // phase 2
  uint16_t* A1p = Qp + 2 * PX;
  uint16_t* Wp = A1p + 2 * PC;  // delta
  float* Lp = reinterpret_cast<float*>(Tp);

  const int nch = (p.T + CB - 1) / CB;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_in = head_has_key(p, bh);
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  // raw bf16 keys and queries with the identity map are exact bf16 operands; the carried key
  // (fp32, row 0 of chunk 0 for the shifted rules) need not be
  const bool xex = sizeof(InT) == 2 && !elu && !(qk_length(p.flags, DK) > 0.f) && !(R::shift && c == 0 && has_in);
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const int t0 = c * CB;
  const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
  const float* Sc = Sch + ((size_t)bh * nch + c) * SS;
  const float* dSc = dSch + ((size_t)bh * nch + c) * SS;
  const float* rhc = Rh + ((size_t)bh * nch + c) * CB * DV;
  const float* drc = dRw + ((size_t)bh * nch + c) * CB * DV;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV;

  {
    // T (delta rule) or M planes from the record; M also as fp32 hi + lo
    const uint16_t* mpl = reinterpret_cast<const uint16_t*>(rec + BRec::kM);
    const uint16_t* tpl = reinterpret_cast<const uint16_t*>(rec + (SOLVE ? BRec::kT : BRec::kM));
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // plane j: CB rows of CB / 8 16-byte groups, one group a thread
      const int r = tid / (CB / 8), c8 = (tid % (CB / 8)) * 8;
      *reinterpret_cast<u32x4*>(Tp + j * PC + r * LC + c8) =
          *reinterpret_cast<const u32x4*>(tpl + j * CB * CB + r * CB + c8);
    }
    for (int e = tid; e < CB * CB / 4; e += 512) {
      const int r = e / (CB / 4), c4 = (e % (CB / 4)) * 4;
      const uint2 h = *reinterpret_cast<const uint2*>(mpl + r * CB + c4);
      const uint2 l = *reinterpret_cast<const uint2*>(mpl + CB * CB + r * CB + c4);
      *reinterpret_cast<f4*>(Ms + r * LDC + c4) =
          f4{bf16_bits_to_f32(h.x & 0xffffu) + bf16_bits_to_f32(l.x & 0xffffu), bf16_bits_to_f32(h.x >> 16) + bf16_bits_to_f32(l.x >> 16),
             bf16_bits_to_f32(h.y & 0xffffu) + bf16_bits_to_f32(l.y & 0xffffu), bf16_bits_to_f32(h.y >> 16) + bf16_bits_to_f32(l.y >> 16)};
    }
  }
  for (int e = tid; e < kNSc * CB; e += 512) (&s_sc[0][0])[e] = rec[BRec::kSc + e];
  for (int e = tid; e < kNP * CB; e += 512) (&s_p[0][0])[e] = 0.f;
  stage_split<InT, DK, R::shift, false, 512>(p, bh, c, Xp, has_in);
  __syncthreads();

  const int m = w & 3, ctw = w >> 2;  // token tile and column tile of this wave's block outputs
  // accumulators over the value blocks
  f4 aMm[4], aQ1[DPW], aXR[DPW], aXS[DPW];  // aMm: dMm (w < 4) or dLm (w >= 4) tiles (m, s <= m)
#pragma unroll
  for (int s = 0; s < 4; ++s) aMm[s] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < DPW; ++d) aQ1[d] = aXR[d] = aXS[d] = f4{0.f, 0.f, 0.f, 0.f};
  f4 pe = {0.f, 0.f, 0.f, 0.f};  // eta's gradient through V (other rules: this lane's C-tile rows)
  float pe1 = 0.f;               // eta's gradient through R-hat (delta: this thread's row)
  float sds = 0.f;               // <dS', S> partial

  auto fac = [&](int k, int t) { return s_sc[k][t]; };

  // The next value block in registers. S and dS' (NSJ float4 a thread each) and dO: thread
  // tid holds float4 tid % 8 of row tid / 8. The delta rule adds dR and R-hat in the dO
  // layout; the other rules take this lane's four values of V in C-tile layout.
  constexpr int NSJ = DK * NCOL / 4 / 512;
  static_assert(NSJ >= 1 && CB * NCOL / 4 == 512, "value block layout");
  const int bt = tid / (NCOL / 4), bv4 = (tid % (NCOL / 4)) * 4, btau = t0 + bt;
  f4 ps[NSJ], pds[NSJ], pdo, pdr, prh;
  float pv4[4];
  auto load_blk = [&](int jb) {
    const int col0 = jb * NCOL;
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int e = tid + 512 * j, r = e / (NCOL / 4), v4 = (e % (NCOL / 4)) * 4;
      ps[j] = *reinterpret_cast<const f4*>(Sc + (size_t)r * DV + col0 + v4);
      pds[j] = *reinterpret_cast<const f4*>(dSc + (size_t)r * DV + col0 + v4);
    }
    pdo = btau < p.T ? *reinterpret_cast<const f4*>(p.dout + (rb + btau) * DV + col0 + bv4) : f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SOLVE) {
      pdr = *reinterpret_cast<const f4*>(drc + (size_t)bt * DV + col0 + bv4);
      prh = *reinterpret_cast<const f4*>(rhc + (size_t)bt * DV + col0 + bv4);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i, tau = t0 + t, cc = col0 + 16 * ctw + n;
        pv4[i] = tau < p.T ? In<InT>::load1(vb + (size_t)tau * DV + cc) : 0.f;
      }
    }
  };
  load_blk(0);

  for (int jb = 0; jb < NBLK; ++jb) {
    const int col0 = jb * NCOL;
    // the block into LDS planes from registers
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int e = tid + 512 * j, r = e / (NCOL / 4), v4 = (e % (NCOL / 4)) * 4;
      put_split4(Sp, PS, r * LB + v4, ps[j]);
      put_split4(dSp, PS, r * LB + v4, pds[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sds += ps[j][i] * pds[j][i];
    }
    put_split4(dOp, PB, bt * LB + bv4, pdo);
    if constexpr (SOLVE) {
      // R = eta R-hat; dV = eta dR; eta's gradient through R-hat
      const float e = fac(kScE, bt);
      put_split4(dRp, PB, bt * LB + bv4, pdr);
      put_split4(Rp, PB, bt * LB + bv4, f4{e * prh[0], e * prh[1], e * prh[2], e * prh[3]});
#pragma unroll
      for (int i = 0; i < 4; ++i) pe1 += pdr[i] * prh[i];
      if (btau < p.T)
        *reinterpret_cast<f4*>(p.gv + (rb + btau) * DV + col0 + bv4) = f4{e * pdr[0], e * pdr[1], e * pdr[2], e * pdr[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        put_split(Up, PB, t * LB + 16 * ctw + n, fac(kScE, t) * pv4[i]);
      }
    }
    float v4r[4];  // V, this lane's C-tile rows (other rules)
#pragma unroll
    for (int i = 0; i < 4; ++i) v4r[i] = pv4[i];
    lds_barrier();
    if (jb + 1 < NBLK) load_blk(jb + 1);

    if constexpr (SOLVE) {
      // U = T R, tile (m, ctw): K blocks 0 .. m/2 (T is lower triangular)
      f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (m >> 1)) mma3(u, fk(Tp, PC, LC, 16 * m + n, 32 * kb, g), ft(Rp, PB, LB, 16 * ctw, 32 * kb, g, n));
#pragma unroll
      for (int i = 0; i < 4; ++i) put_split(Up, PB, (16 * m + 4 * g + i) * LB + 16 * ctw + n, u[i]);
    } else {
      // dU = (Gamma_end / Gamma) X dS' + M^T dO; dV = f dU; f's gradient through V
      f4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const SFrag x = fk(Xp, PX, LX, 16 * m + n, 32 * kb, g);
        const SFrag b = ft(dSp, PS, LB, 16 * ctw, 32 * kb, g, n);
        mma_bf16(du, x.h, b.l);
        if (!xex) mma_bf16(du, x.l, b.h);
        mma_bf16(du, x.h, b.h);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] *= fac(kScGend, 16 * m + 4 * g + i);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb >= (m >> 1)) mma3(du, ft(Tp, PC, LC, 16 * m, 32 * kb, g, n), ft(dOp, PB, LB, 16 * ctw, 32 * kb, g, n));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i, tau = t0 + t;
        pe[i] += du[i] * v4r[i];
        if (tau < p.T) p.gv[(rb + tau) * DV + col0 + 16 * ctw + n] = fac(kScE, t) * du[i];
      }
    }
    lds_barrier();

    // accumulate over the block's 32 columns (one K block): dMm = dO U^T (w < 4), dLm =
    // -dR U^T (w >= 4), dQ1 = dO S^T, dXR = dR S^T, dXS = U dS'^T
    {
      const SFrag fdo = fk(dOp, PB, LB, 16 * m + n, 0, g);
      const SFrag fu = fk(Up, PB, LB, 16 * m + n, 0, g);
      SFrag fdr;
      if constexpr (SOLVE) fdr = fk(dRp, PB, LB, 16 * m + n, 0, g);
      if (w < 4) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s <= m) mma3(aMm[s], fdo, fk(Up, PB, LB, 16 * s + n, 0, g));
      } else if constexpr (SOLVE) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s <= m) mma3(aMm[s], fdr, fk(Up, PB, LB, 16 * s + n, 0, g));
      }
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int dt = ctw * DPW + d;
        const SFrag fs = fk(Sp, PS, LB, 16 * dt + n, 0, g);
        mma3(aQ1[d], fdo, fs);
        if constexpr (SOLVE) mma3(aXR[d], fdr, fs);
        mma3(aXS[d], fu, fk(dSp, PS, LB, 16 * dt + n, 0, g));
      }
    }
    lds_barrier();
  }

  // ---- phase 2
  // <dS', S> over the workgroup
  sds = wave_sum(sds);
  if (lane == 0) s_red[w] = sds;
  // eta's (or f's) gradient through the values
  if constexpr (SOLVE) {
    pe1 = group_sum<NCOL / 4>(pe1);
    if (tid % (NCOL / 4) == 0) s_p[kPe0][bt] = pe1;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = sum16(pe[i]);
      if (n == 0) s_p[kPe0 + ctw][16 * m + 4 * g + i] = v;
    }
  }
  // row dots with the state-coupled terms, after their row factors
  {
    float pq[4] = {0.f, 0.f, 0.f, 0.f}, pr[4] = {0.f, 0.f, 0.f, 0.f}, ph[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        aQ1[d][i] *= fac(kScGam, t);
        aXR[d][i] *= -fac(kScE, t) * fac(kScGprev, t);
        aXS[d][i] *= fac(kScGend, t);
        const float x = get_split(Xp, PX, t * LX + dc);
        pr[i] += x * aXR[d][i];
        ph[i] += x * aXS[d][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = sum16(pr[i]), h = sum16(ph[i]);
      if (n == 0) {
        s_p[kPdXR0 + ctw][16 * m + 4 * g + i] = r;
        s_p[kPh0 + ctw][16 * m + 4 * g + i] = h;
      }
    }
    __syncthreads();  // phase-1 block buffers and (delta rule) T free
    stage_split<InT, DK, R::shift, true, 512>(p, bh, c, Qp, has_in);
    if constexpr (SOLVE) {
      for (int e = tid; e < CB * CB / 4; e += 512) {
        const int r = e / (CB / 4), c4 = (e % (CB / 4)) * 4;
        *reinterpret_cast<f4*>(Lp + r * LDC + c4) = *reinterpret_cast<const f4*>(rec + BRec::kLp + r * CB + c4);
      }
    }
    for (int e = tid; e < 2 * (SOLVE ? 2 : 1) * PC / 8; e += 512) reinterpret_cast<u32x4*>(A1p)[e] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) pq[i] += get_split(Qp, PX, (16 * m + 4 * g + i) * LX + dc) * aQ1[d][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q = sum16(pq[i]);
      if (n == 0) s_p[kPdQ0 + ctw][16 * m + 4 * g + i] = q;
    }
  }
  // A1 = dMm o D with the row and column sums of dMm o M (waves 0-3), W = dLm o eta D' with
  // the row and column sums of dLm o L and the row sums of dLm o Lp (waves 4-7)
  {
    const float* gl = s_sc[kScG];
    const float* pa = s_sc[kScPar];
    float rs[4] = {0.f, 0.f, 0.f, 0.f}, rs2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s > m) continue;
      float cs = 0.f;
      const int sc = 16 * s + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        if (w < 4) {
          if (sc <= t) {
            const float d = sgn((int)pa[t] ^ (int)pa[sc]) * __expf(gl[t] - gl[sc]);
            const float v = aMm[s][i];
            put_split(A1p, PC, t * LC + sc, v * d);
            const float pm = v * Ms[t * LDC + sc];
            rs[i] += pm;
            cs += pm;
          }
        } else if constexpr (SOLVE) {
          if (sc < t) {
            const float dl = -aMm[s][i];  // dLm = -dR U^T (the waves accumulated dR U^T)
            const float lp = Lp[t * LDC + sc];  // D'_ts (x_t . x_s)
            const float e = fac(kScE, t);
            const float dp = sgn((int)pa[t - 1] ^ (int)pa[sc]) * __expf(gl[t - 1] - gl[sc]);  // D'_ts
            put_split(Wp, PC, t * LC + sc, dl * e * dp);
            rs[i] += dl * e * lp;   // dLm o L
            rs2[i] += dl * lp;      // dLm o Lp
            cs += dl * e * lp;
          }
        }
      }
      // column sums over this tile's 16 rows: the four lane groups
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (g == 0) {
        if (w < 4) s_p[kPMc0 + m][sc] += cs;
        else if (SOLVE) s_p[kPLc0 + m][sc] += cs;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = sum16(rs[i]), b = sum16(rs2[i]);
      if (n == 0) {
        const int t = 16 * m + 4 * g + i;
        if (w < 4) s_p[kPMr][t] = a;
        else if (SOLVE) {
          s_p[kPLr][t] = a;
          s_p[kPeL][t] = b;
        }
      }
    }
  }
  __syncthreads();

  // dQ = dQ1 + A1 X;  dX = dXR + dXS + A1^T Q + W X + W^T X (this wave: token tile m, d_k
  // tiles ctw * DPW ...). Row-tile m's K block is m / 2: A1 X and W X take K blocks up to
  // it (s <= t), A1^T Q and W^T X the blocks from it on (t >= s).
  f4 dQ[DPW], dX[DPW];
  {
    const int km = m >> 1;
    SFrag a1[2], a1t[2], wf[2], wft[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb <= km) {
        a1[kb] = fk(A1p, PC, LC, 16 * m + n, 32 * kb, g);
        if constexpr (SOLVE) wf[kb] = fk(Wp, PC, LC, 16 * m + n, 32 * kb, g);
      }
      if (kb >= km) {
        a1t[kb] = ft(A1p, PC, LC, 16 * m, 32 * kb, g, n);
        if constexpr (SOLVE) wft[kb] = ft(Wp, PC, LC, 16 * m, 32 * kb, g, n);
      }
    }
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dt = ctw * DPW + d;
      dQ[d] = aQ1[d];
      dX[d] = aXR[d] + aXS[d];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const SFrag bx = ft(Xp, PX, LX, 16 * dt, 32 * kb, g, n);
        if (kb <= km) {
          mma3x(dQ[d], a1[kb], bx, xex);
          if constexpr (SOLVE) mma3x(dX[d], wf[kb], bx, xex);
        }
        if (kb >= km) {
          mma3x(dX[d], a1t[kb], ft(Qp, PX, LX, 16 * dt, 32 * kb, g, n), xex);
          if constexpr (SOLVE) mma3x(dX[d], wft[kb], bx, xex);
        }
      }
    }
  }

  // the log decays' gradient, its suffix sums, and the scalar chain (wave 0, lane = token)
  if (w == 0) {
    const int t = lane;
    const float hsum = wave_sum(s_p[kPh0][t] + s_p[kPh1][t]);
    float dg = s_p[kPdQ0][t] + s_p[kPdQ1][t] - s_p[kPh0][t] - s_p[kPh1][t] + s_p[kPMr][t];
#pragma unroll
    for (int k = 0; k < 4; ++k) dg -= s_p[kPMc0 + k][t];
    if (t + 1 < CB) dg += s_p[kPdXR0][t + 1] + s_p[kPdXR1][t + 1];
    if constexpr (SOLVE) {
      if (t + 1 < CB) dg += s_p[kPLr][t + 1];
#pragma unroll
      for (int k = 0; k < 4; ++k) dg -= s_p[kPLc0 + k][t];
    }
    if (t == CB - 1) {
      float sd = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) sd += s_red[k];
      dg += hsum + rec[BRec::kMisc] * sd;
    }
    // suffix sums: dl_t = sum_{t' >= t} dg_t'
    float dl = dg;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(dl, o);
      if (t + o < 64) dl += y;
    }
    const float a = fac(kScA, t);
    const float af = (a < 0.f ? -1.f : 1.f) * fmaxf(fabsf(a), 1e-30f);
    const float da = dl / af;
    const int tau = t0 + t;
    float dn = 0.f;
    if (tau < p.T) {
      const float beta = fac(kScBeta, t), lam = fac(kScLam, t);
      const bool key = fac(kScKey, t) != 0.f;
      float gb = 0.f, gl = 0.f;
      if constexpr (R::nlms) {
        if (key) {
          const float e = fac(kScE, t), den = fac(kScDen, t), lu = fac(kScLu, t), nx = fac(kScN, t);
          float de = s_p[kPe0][t] + s_p[kPe1][t];
          if (SOLVE) de += s_p[kPeL][t];
          de -= lu * da;
          gb = de / den;
          const float dden = -e * de / den;
          const float dlu = -e * da + dden;
          const bool scaled = (p.flags & kFlagLamScaled) != 0;
          dn = dden + (scaled ? lam * dlu : 0.f);
          gl = dlu * (scaled ? nx : 1.f);
        }
      } else {
        gb = s_p[kPe0][t] + s_p[kPe1][t];
        gl = da;
      }
      // with pre-activated gates: the gradient with respect to the pre-activation
      if (p.flags & kFlagBetaSig) gb *= beta * (1.f - beta);
      else if (p.flags & kFlagBetaSig2) gb *= beta * (1.f - 0.5f * beta);
      if (p.flags & kFlagLamAct) gl *= R::nlms ? -expm1f(-lam) : lam * (1.f - lam);
      if (p.gbeta != nullptr) p.gbeta[rb + tau] = gb;
      if (p.glam != nullptr) p.glam[rb + tau] = gl;
    }
    s_dn[t] = dn;
  }
  __syncthreads();

  // the feature maps' derivative from the staged values y = phi(z): 1 for the identity;
  // for elu+1, 1 where y > 1 (z > 0) and y = exp(z) elsewhere
  auto dphi = [&](float y) { return elu ? (y > 1.f ? 1.f : y) : 1.f; };
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int dc = 16 * (ctw * DPW + d) + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * m + 4 * g + i, tau = t0 + t;
      const float x = get_split(Xp, PX, t * LX + dc);
      const float gx = dX[d][i] + 2.f * s_dn[t] * x;
      if (tau < p.T) p.gq[(rb + tau) * DK + dc] = dQ[d][i] * dphi(get_split(Qp, PX, t * LX + dc));
      if constexpr (R::shift) {
        // x_t is the key of token tau - 1 (the carried key before the first token)
        if (tau >= 1 && tau < p.T) p.gk[(rb + tau - 1) * DK + dc] = gx * dphi(x);
        else if (tau == 0 && p.gx0 != nullptr) p.gx0[(size_t)bh * DK + dc] = has_in ? gx : 0.f;
      } else {
        if (tau < p.T) p.gk[(rb + tau) * DK + dc] = gx * dphi(x);
      }
    }
  }
  if constexpr (R::shift) {
    // the last key is written by no step of this call
    if (c == nch - 1)
      for (int i = tid; i < DK; i += 512) p.gk[(rb + p.T - 1) * DK + i] = 0.f;
  } else {
    if (c == 0 && p.gx0 != nullptr)
      for (int i = tid; i < DK; i += 512) p.gx0[(size_t)bh * DK + i] = 0.f;
  }
}

// ====================== state and dstate on bf16 MFMA with split operands (bf16 inputs)
// The chunk steps of bwd_state_kernel and bwd_dstate_kernel with every product on
// v_mfma_f32_16x16x32_bf16: the keys and queries as split planes (exact bf16 for raw keys
// and queries with the identity map; the carried key of chunk 0 is fp32), S, R, W, T, M,
// dS, dO, dU and dR as hi/lo planes.
template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(512) void bwd_state_bf_kernel(BwdParams p, const float* recs, float* Sch, float* Rh) {
  using R = Rule<RULE>;
  constexpr int NRT = DK / 16;
  constexpr int NTW = NRT / 4;  // S tiles of a wave (DK 128: row tile w, both column tiles; DK 64: one)
  constexpr int VWv = 16 / (int)sizeof(InT), NVG = CB * NCOL / VWv;  // value groups
  static_assert(NVG <= 512, "value groups");
  constexpr int LX = DK + 8, LC = CB + 8, PX = CB * LX, PT = CB * LC, PB = NCOL * LX, PW = NCOL * LC;
  __shared__ __align__(16) uint16_t Xp[2 * PX];
  __shared__ __align__(16) uint16_t Tp[R::solve ? 2 * PT : 8];
  __shared__ __align__(16) uint16_t Bp[2 * PB];                 // S^T [NCOL][DK], then W^T [NCOL][CB]
  __shared__ __align__(16) uint16_t Rp[R::solve ? 2 * PW : 8];  // R^T [NCOL][CB]
  __shared__ __align__(16) float Vs[CB * LDU];                  // the chunk's values [CB][NCOL]
  // eta Gamma_prev, eta (or f), Gamma_end / Gamma, Gamma_prev; [4][0] Gamma_end
  __shared__ float s_fac[5][CB];
  int bh, grp;
  if (!state_block(p, DV / NCOL, bh, grp)) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = (p.T + CB - 1) / CB;
  const bool has_in = head_has_key(p, bh);
  const int col0 = grp * NCOL;
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(p.flags, DK);
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV + col0;
  auto tile_rt = [&](int a) { return NTW == 2 ? w : (w & 3); };
  auto tile_ct = [&](int a) { return NTW == 2 ? a : (w >> 2); };
  const int m = w & 3, ctw = w >> 2;  // this wave's (token tile, column tile) of X S, R and U

  f4 S[NTW];
#pragma unroll
  for (int a = 0; a < NTW; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * tile_rt(a) + 4 * g + i;
      S[a][i] = p.S_in != nullptr ? p.S_in[(size_t)bh * SS + (size_t)r * DV + col0 + 16 * tile_ct(a) + n] : 0.f;
    }

  // registers of the next chunk: rows, T (8 floats a thread), values, scalars
  Rows<InT, DK, 512> rows;
  u32x4 pt[2];  // T planes: one 16-byte group of each
  u32x4 pv;
  float pf[5];
  auto load = [&](int c) {
    // row t is the key of token c CB + t - 1 for the shifted pair (token 0's is the carried key)
    rows.load(kb - (R::shift ? DK : 0), c * CB, R::shift ? 1 : 0, p.T);
    const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        pt[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(rec + BRec::kT) + j * CB * CB + 8 * tid);
    }
    {
      const int t = tid / (NCOL / VWv), v0 = (tid % (NCOL / VWv)) * VWv, tau = c * CB + t;
      pv = u32x4{0u, 0u, 0u, 0u};
      if (tid < NVG && tau < p.T) pv = *reinterpret_cast<const u32x4*>(vb + (size_t)tau * DV + v0);
    }
    if (tid < CB) {
      const float* sc = rec + BRec::kSc;
      const float e = sc[kScE * CB + tid];
      pf[0] = e * sc[kScGprev * CB + tid];
      pf[1] = e;
      pf[2] = sc[kScGend * CB + tid];
      pf[3] = sc[kScGprev * CB + tid];
      pf[4] = rec[BRec::kMisc];
    }
  };
  auto commit = [&](int c) {
    // the carried key (phi applied) before the call's first token
    const float* x0 = (R::shift && has_in && p.xprev_in != nullptr) ? p.xprev_in + (size_t)bh * DK : nullptr;
    rows.commit_split(Xp, elu, len, (R::shift && c == 0) ? 0 : -1, x0);
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(Tp + j * PT + (tid >> 3) * LC + 8 * (tid & 7)) = pt[j];
    }
    if (tid < NVG) {
      const int t = tid / (NCOL / VWv), v0 = (tid % (NCOL / VWv)) * VWv;
      float x[VWv];
      In<InT>::decode(pv, x);
#pragma unroll
      for (int e = 0; e < VWv; e += 4) *reinterpret_cast<f4*>(Vs + t * LDU + v0 + e) = f4{x[e], x[e + 1], x[e + 2], x[e + 3]};
    }
    if (tid < CB) {
#pragma unroll
      for (int k = 0; k < 4; ++k) s_fac[k][tid] = pf[k];
      if (tid == 0) s_fac[4][0] = pf[4];
    }
  };
  // the delta rule needs every chunk's data (R-hat of the last chunk too), the others
  // every chunk's but the last
  if (R::solve || nch > 1) load(0);

  for (int c = 0; c < nch; ++c) {
    float* Sc = Sch + ((size_t)bh * nch + c) * SS;
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sc[(size_t)(16 * tile_rt(a) + 4 * g + i) * DV + col0 + 16 * tile_ct(a) + n] = S[a][i];
    if (!R::solve && c + 1 == nch) break;  // the state after the last chunk is not needed
    lds_barrier();  // the previous chunk's LDS reads are done
    commit(c);
    if constexpr (R::solve) {
#pragma unroll
      for (int a = 0; a < NTW; ++a) put_split4(Bp, PB, (16 * tile_ct(a) + n) * LX + 16 * tile_rt(a) + 4 * g, S[a]);
    }
    lds_barrier();
    if (c + 1 < nch && (R::solve || c + 2 < nch)) load(c + 1);
    const bool xex = !elu && !(len > 0.f) && !(R::shift && c == 0 && has_in);

    // this wave's tile (m, ctw): W = fU U with U = T R (delta) or fV V
    f4 W;
    if constexpr (R::solve) {
      // R-hat = V - Gamma_prev X S, kept for the gradient pass, and R = eta R-hat
      float* rh = Rh + ((size_t)bh * nch + c) * CB * DV + col0;
      f4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        mma3a(xs, fk(Xp, PX, LX, 16 * m + n, 32 * kb, g), fk(Bp, PB, LX, 16 * ctw + n, 32 * kb, g), xex);
      f4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        const float rhat = Vs[t * LDU + 16 * ctw + n] - s_fac[3][t] * xs[i];
        rh[(size_t)t * DV + 16 * ctw + n] = rhat;
        r[i] = s_fac[1][t] * rhat;
      }
      put_split4(Rp, PW, (16 * ctw + n) * LC + 16 * m + 4 * g, r);
      if (c + 1 == nch) break;  // the state after the last chunk is not needed
      lds_barrier();
      f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (m >> 1)) mma3(u, fk(Tp, PT, LC, 16 * m + n, 32 * kb, g), fk(Rp, PW, LC, 16 * ctw + n, 32 * kb, g));
#pragma unroll
      for (int i = 0; i < 4; ++i) W[i] = s_fac[2][16 * m + 4 * g + i] * u[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * m + 4 * g + i;
        W[i] = s_fac[2][t] * s_fac[1][t] * Vs[t * LDU + 16 * ctw + n];
      }
    }
    put_split4(Bp, PW, (16 * ctw + n) * LC + 16 * m + 4 * g, W);
    lds_barrier();
    // S' = Gamma_end S + X^T W
    const float gend = s_fac[4][0];
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
      S[a] *= gend;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma3a(S[a], ft(Xp, PX, LX, 16 * tile_rt(a), 32 * kb, g, n), fk(Bp, PW, LC, 16 * tile_ct(a) + n, 32 * kb, g), xex);
    }
  }
}

template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(512) void bwd_dstate_bf_kernel(BwdParams p, const float* recs, float* dSch, float* dRw) {
  using R = Rule<RULE>;
  constexpr int NRT = DK / 16;
  constexpr int NTW = NRT / 4;  // dS tiles of a wave (DK 128: row tile w, both column tiles; DK 64: one)
  constexpr int LX = DK + 8, LC = CB + 8, LB = NCOL + 8;
  constexpr int PX = CB * LX, PT = CB * LC, PB = NCOL * LX, PW = NCOL * LC, PO = CB * LB;
  __shared__ __align__(16) uint16_t Xp[2 * PX];
  __shared__ __align__(16) uint16_t Qp[2 * PX];
  __shared__ __align__(16) uint16_t Tp[R::solve ? 2 * PT : 8];
  __shared__ __align__(16) uint16_t Mp[R::solve ? 2 * PT : 8];
  __shared__ __align__(16) uint16_t dOp[2 * PO];  // dO of the column group [CB][NCOL]
  __shared__ __align__(16) uint16_t gOp[2 * PO];  // Gamma o dO
  __shared__ __align__(16) uint16_t Bp[2 * PB];   // dS^T [NCOL][DK], then (delta) -(eta Gamma_prev dR)^T [NCOL][CB]
  __shared__ __align__(16) uint16_t dUp[R::solve ? 2 * PW : 8];
  __shared__ float s_fac[4][CB];  // Gamma, eta Gamma_prev, Gamma_end / Gamma; [3][0] Gamma_end
  int bh, grp;
  if (!state_block(p, DV / NCOL, bh, grp)) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = (p.T + CB - 1) / CB;
  const bool has_in = head_has_key(p, bh);
  const int col0 = grp * NCOL;
  const size_t SS = (size_t)DK * DV, rb = (size_t)bh * p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(p.flags, DK);
  const bool qex = !elu && !(len > 0.f);
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* qb = static_cast<const InT*>(p.q) + rb * DK;
  const float* dob = p.dout + rb * DV + col0;
  auto tile_rt = [&](int a) { return NTW == 2 ? w : (w & 3); };
  auto tile_ct = [&](int a) { return NTW == 2 ? a : (w >> 2); };

  f4 dS[NTW];
#pragma unroll
  for (int a = 0; a < NTW; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * tile_rt(a) + 4 * g + i;
      dS[a][i] = p.dS_out != nullptr ? p.dS_out[(size_t)bh * SS + (size_t)r * DV + col0 + 16 * tile_ct(a) + n] : 0.f;
    }
  const int m = w & 3, ctw = w >> 2;  // this wave's (token tile, column tile) of dU and dR

  // registers of the next chunk: X and Q rows, T and M (8 floats a thread each), dO (4), scalars
  Rows<InT, DK, 512> xrows, qrows;
  u32x4 pt[2], pm[2];  // T and M planes: one 16-byte group of each
  f4 pd;
  float pf[4], pgam;
  auto load = [&](int c) {
    xrows.load(kb - (R::shift ? DK : 0), c * CB, R::shift ? 1 : 0, p.T);
    qrows.load(qb, c * CB, 0, p.T);
    const float* rec = recs + ((size_t)bh * nch + c) * BRec::kFloats;
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        pt[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(rec + BRec::kT) + j * CB * CB + 8 * tid);
        pm[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(rec + BRec::kM) + j * CB * CB + 8 * tid);
      }
    }
    {
      const int t = tid / (NCOL / 4), v0 = (tid % (NCOL / 4)) * 4, tau = c * CB + t;
      pd = tau < p.T ? *reinterpret_cast<const f4*>(dob + (size_t)tau * DV + v0) : f4{0.f, 0.f, 0.f, 0.f};
      pgam = rec[BRec::kSc + kScGam * CB + t];
    }
    if (tid < CB) {
      const float* sc = rec + BRec::kSc;
      pf[0] = sc[kScGam * CB + tid];
      pf[1] = sc[kScE * CB + tid] * sc[kScGprev * CB + tid];
      pf[2] = sc[kScGend * CB + tid];
      pf[3] = rec[BRec::kMisc];
    }
  };
  auto commit = [&](int c) {
    const float* x0 = (R::shift && has_in && p.xprev_in != nullptr) ? p.xprev_in + (size_t)bh * DK : nullptr;
    xrows.commit_split(Xp, elu, len, (R::shift && c == 0) ? 0 : -1, x0);
    qrows.commit_split(Qp, elu, len, -1, nullptr);
    if constexpr (R::solve) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        *reinterpret_cast<u32x4*>(Tp + j * PT + (tid >> 3) * LC + 8 * (tid & 7)) = pt[j];
        *reinterpret_cast<u32x4*>(Mp + j * PT + (tid >> 3) * LC + 8 * (tid & 7)) = pm[j];
      }
    }
    {
      const int t = tid / (NCOL / 4), v0 = (tid % (NCOL / 4)) * 4;
      put_split4(dOp, PO, t * LB + v0, pd);
      put_split4(gOp, PO, t * LB + v0, f4{pgam * pd[0], pgam * pd[1], pgam * pd[2], pgam * pd[3]});
    }
    if (tid < CB) {
      s_fac[0][tid] = pf[0];
      s_fac[1][tid] = pf[1];
      s_fac[2][tid] = pf[2];
      if (tid == 0) s_fac[3][0] = pf[3];
    }
  };
  load(nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    float* dSc = dSch + ((size_t)bh * nch + c) * SS;
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dSc[(size_t)(16 * tile_rt(a) + 4 * g + i) * DV + col0 + 16 * tile_ct(a) + n] = dS[a][i];
    lds_barrier();  // the previous chunk's LDS reads are done
    commit(c);
#pragma unroll
    for (int a = 0; a < NTW; ++a) put_split4(Bp, PB, (16 * tile_ct(a) + n) * LX + 16 * tile_rt(a) + 4 * g, dS[a]);
    lds_barrier();
    if (c >= 1) load(c - 1);
    const bool xex = qex && !(R::shift && c == 0 && has_in);

    if constexpr (R::solve) {
      // dU = M^T dO + (Gamma_end / Gamma) X dS' for token tile m, column tile ctw (only the
      // delta rule's state gradient goes through the writes)
      f4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        mma3a(du, fk(Xp, PX, LX, 16 * m + n, 32 * kb, g), fk(Bp, PB, LX, 16 * ctw + n, 32 * kb, g), xex);
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] *= s_fac[2][16 * m + 4 * g + i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb >= (m >> 1)) mma3(du, ft(Mp, PT, LC, 16 * m, 32 * kb, g, n), ft(dOp, PO, LB, 16 * ctw, 32 * kb, g, n));
      put_split4(dUp, PW, (16 * ctw + n) * LC + 16 * m + 4 * g, du);
      lds_barrier();  // dU complete; dS^T no longer read
      // dR = T^T dU
      f4 dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb >= (m >> 1)) mma3(dr, ft(Tp, PT, LC, 16 * m, 32 * kb, g, n), fk(dUp, PW, LC, 16 * ctw + n, 32 * kb, g));
      // dR, kept for the gradient pass
      float* drw = dRw + ((size_t)bh * nch + c) * CB * DV + col0 + 16 * ctw + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        drw[(size_t)(16 * m + 4 * g + i) * DV] = dr[i];
        dr[i] *= -s_fac[1][16 * m + 4 * g + i];
      }
      put_split4(Bp, PW, (16 * ctw + n) * LC + 16 * m + 4 * g, dr);
      lds_barrier();
    }
    // dS = Gamma_end dS' + Q^T diag(Gamma) dO - X^T (eta Gamma_prev dR)
    const float gend = s_fac[3][0];
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
      const int rt = tile_rt(a), ct = tile_ct(a);
      dS[a] *= gend;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        mma3a(dS[a], ft(Qp, PX, LX, 16 * rt, 32 * kb, g, n), ft(gOp, PO, LB, 16 * ct, 32 * kb, g, n), qex);
        if constexpr (R::solve)
          mma3a(dS[a], ft(Xp, PX, LX, 16 * rt, 32 * kb, g, n), fk(Bp, PW, LC, 16 * ct + n, 32 * kb, g), xex);
      }
    }
  }
  if (p.gS0 != nullptr) {
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.gS0[(size_t)bh * SS + (size_t)(16 * tile_rt(a) + 4 * g + i) * DV + col0 + 16 * tile_ct(a) + n] = dS[a][i];
    if (grp == 0 && tid == 0 && p.gh0 != nullptr) p.gh0[bh] = 0;
  }
}

template <typename InT, int DK, int DV, int RULE>
hipError_t launch_rule(const BwdParams& p, float* ws, hipStream_t st) {
  const int nch = (p.T + CB - 1) / CB;
  const size_t nrec = (size_t)p.BH * nch;
  float* recs = ws;
  float* Sch = recs + nrec * BRec::kFloats;
  float* dSch = Sch + nrec * (size_t)DK * DV;
  float* Rh = dSch + nrec * (size_t)DK * DV;  // R-hat of every chunk [CB][DV] (delta rule)
  float* dRw = Rh + nrec * (size_t)CB * DV;   // dR of every chunk (delta rule)
  const unsigned ngrid = (unsigned)(8 * (DV / NCOL) * ((p.BH + 7) / 8));
  hipLaunchKernelGGL((bwd_prep_kernel<InT, DK, RULE>), dim3((unsigned)nrec), dim3(256), 0, st, p, recs);
  if constexpr (sizeof(InT) == 2) {
    hipLaunchKernelGGL((bwd_state_bf_kernel<InT, DK, DV, RULE>), dim3(ngrid), dim3(512), 0, st, p, recs, Sch, Rh);
    hipLaunchKernelGGL((bwd_dstate_bf_kernel<InT, DK, DV, RULE>), dim3(ngrid), dim3(512), 0, st, p, recs, dSch, dRw);
  } else {
    hipLaunchKernelGGL((bwd_state_kernel<InT, DK, DV, RULE>), dim3(ngrid), dim3(256), 0, st, p, recs, Sch, Rh);
    hipLaunchKernelGGL((bwd_dstate_kernel<InT, DK, DV, RULE>), dim3(ngrid), dim3(512), 0, st, p, recs, dSch, dRw);
  }
  if constexpr (sizeof(InT) == 2)
    hipLaunchKernelGGL((bwd_grad_kernel<InT, DK, DV, RULE>), dim3((unsigned)nrec), dim3(512), 0, st, p, recs, Sch,
                       dSch, Rh, dRw);
  else
    hipLaunchKernelGGL((bwd_grad_f32_kernel<InT, DK, DV, RULE>), dim3((unsigned)nrec), dim3(512), 0, st, p, recs,
                       Sch, dSch, Rh, dRw);
  return hipGetLastError();
}

template <typename InT, int DK, int DV>
hipError_t launch_dims(const BwdParams& p, float* ws, hipStream_t st) {
  if (p.rule == kRuleDelta) return launch_rule<InT, DK, DV, kRuleDelta>(p, ws, st);
  if (p.rule == kRuleInner) return launch_rule<InT, DK, DV, kRuleInner>(p, ws, st);
  return launch_rule<InT, DK, DV, kRuleAdditive>(p, ws, st);
}

template <typename InT>
hipError_t launch_in(const BwdParams& p, float* ws, hipStream_t st) {
  if (p.dk == 64 && p.dv == 64) return launch_dims<InT, 64, 64>(p, ws, st);
  if (p.dk == 64 && p.dv == 128) return launch_dims<InT, 64, 128>(p, ws, st);
  if (p.dk == 128 && p.dv == 64) return launch_dims<InT, 128, 64>(p, ws, st);
  return launch_dims<InT, 128, 128>(p, ws, st);
}

}  // namespace

bool bwd_chunked(int rule, uint32_t flags, int T) {
  return T > 0 && (rule == kRuleDelta || rule == kRuleInner || rule == kRuleAdditive) &&
         (flags & (kFlagPerChannel | kFlagZnorm)) == 0;
}

size_t bwd_chunk_floats_per_head(int T, int dk, int dv) {
  const size_t nch = ((size_t)T + CB - 1) / CB;
  return nch * (BRec::kFloats + 2 * (size_t)dk * (size_t)dv + 2 * (size_t)CB * (size_t)dv);
}

hipError_t launch_bwd_chunked(const BwdParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  const hipError_t e = p.bf16 ? launch_in<uint16_t>(p, p.ws, st) : launch_in<float>(p, p.ws, st);
  if (e != hipSuccess) return e;
  return launch_qk_norm_bwd(p, st);
}

}  // namespace fwmem
