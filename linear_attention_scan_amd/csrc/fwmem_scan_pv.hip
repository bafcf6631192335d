// Chunked scan of the per-value-channel delta rule (Falcon-2, "Fast Weight Attention for
// Continual Learning" reading notes, section 4.4): value channel j steps by
// eta_{j,t} = beta_{j,t} / (|x_t|^2 + lambda_t + eps) on the shared shifted pair and
// decays its own column of S by a_{j,t} = 1 - eta_{j,t} lambda_t.
//
// Chunk algebra, per column j (the column index is dropped), with Gamma_t the product of
// a over the chunk's tokens 0..t, Gamma^_t = Gamma_t / Gamma_A its value relative to an
// anchor token A in mid-chunk, and W~ the chunk's writes w_t = eta_t r_t divided by
// Gamma^_t:
//   w~_t = c_t (v_t - Gamma_{t-1} (X S0)_t) - c_t Gamma^_{t-1} (G W~)_t,  c_t = eta_t / Gamma^_t
//   O    = Gamma o (Q S0) + Gamma^ o (P W~)
//   S'   = Gamma_C S0 + Gamma^_C X^T W~
// with G_ts = x_t . x_s (s < t) and P_ts = q_t . x_s (s <= t) shared by every column
// (the update geometry depends on the keys only, as the page notes). Every per-column
// factor is a row scaling, so all products run on MFMA over the shared X, Q, G, P; only
// the 16 x 16 diagonal blocks of the triangular system for W~ are solved row by row.
//
// Prep (one workgroup per (head, chunk)): G, P and the token scalars into a record.
// Propagate (one workgroup per (head, 64 value columns), four waves of 16 columns, the
// state slice in registers): per chunk, stage X, Q, G, P, beta and V in LDS, then the
// algebra above on MFMA: with bf16 inputs and the identity feature map, X and Q are exact
// bf16 numbers and X S0, Q S0 and X^T W~ run on bf16 MFMA against S0 and W~ split into
// bf16 hi + lo pairs (fwmem_split.h), which keeps about 16 bits of each; everything else
// (and every product for other inputs) on fp32 MFMA. The carried key then enters rounded
// to bf16, as on the split pair.
#include "fwmem_device.h"
#include "fwmem_internal.h"
#include "fwmem_split.h"

#include <type_traits>

namespace fwmem {
namespace {

constexpr int CH = kChunk;
constexpr int NT = 256;
constexpr int LDM = CH + 4;  // float stride of a [CH][CH] matrix

// Record of one (head, chunk), floats: G [CH][CH] (strictly lower), P [CH][CH] (lower; with
// bf16 inputs and the identity map, the same bytes hold P as bf16 hi and lo halves,
// [2][CH][CH], for the propagate's bf16 products),
// then per token: eta's denominator (infinite where there is no key to write), the
// ridge lambda_t, and the rescale factors of x_t and q_t (1 without QK normalisation);
// in chunk 0's record, the carried key (zero without one), so that the propagate kernel
// never reads the state's x_prev, which a state updated in place overwrites.
struct RecPV {
  static constexpr size_t kG = 0;
  static constexpr size_t kP = kG + CH * CH;
  static constexpr size_t kDen = kP + CH * CH;
  static constexpr size_t kLam = kDen + CH;
  static constexpr size_t kNx = kLam + CH;
  static constexpr size_t kMq = kNx + CH;
  static constexpr size_t kX0 = kMq + CH;  // [d_k <= 128]
  static constexpr size_t kFloats = kX0 + 128;
  static constexpr size_t kBytes = (4 * kFloats + 255) / 256 * 256;
};

// C += A B for a 16x16x16 block on fp32 MFMA: lane (g, n) supplies A[n][4g..4g+3] and
// B[4g+q][n] (the C layout of a previous product); MFMA q sums over K = 4g + q.
__device__ __forceinline__ void mma_block(f4& acc, const f4& a, const f4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], acc, 0, 0, 0);
}

// One (head, chunk) of prep: the chunk's written keys x_t (the previous token's phi(k);
// for the sequence's first token the carried key, or zero without one) and queries
// phi(q_t) arrive by 16-byte loads, each thread taking NG granules; their squared norms
// are summed over the threads of a row. With bf16 inputs and the identity map
// (EXACT) the rows stay raw bf16 in LDS and G and P run on bf16 MFMA (exact products,
// fp32 sums); otherwise the rows are staged as fp32 and the products run on fp32 MFMA.
template <typename InT, int DK, bool EXACT>
__global__ __launch_bounds__(NT) void prep_pv_kernel(ScanParams p) {
  static_assert(!EXACT || sizeof(InT) == 2, "exact operands are bf16");
  constexpr int LDX = DK + 4;  // fp32 row stride
  constexpr int LDB = DK + 8;  // bf16 row stride
  __shared__ __align__(16) float smem[EXACT ? CH * LDB : 2 * CH * LDX];
  float* Xs = smem;
  float* Qs = smem + CH * LDX;
  uint16_t* Xb = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Qb = Xb + CH * LDB;
  __shared__ float s_e[CH], s_nq[CH], s_nx[CH], s_mq[CH];
  __shared__ float s_x0[DK];
  const int c = blockIdx.x % p.nchunks, bh = blockIdx.x / p.nchunks;
  const int t0 = c * CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  float* rec = reinterpret_cast<float*>(p.ws + ((size_t)bh * p.nchunks + c) * RecPV::kBytes);
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  // the carried key is only read by the sequence's first token (chunk 0)
  const bool x0 = c == 0 && has_in && p.xprev_in != nullptr;
  // bf16 inputs with the identity map: the carried key is rounded to bf16 like the keys
  const bool round_x0 = sizeof(InT) == 2 && (p.flags & kFlagPhiElu1) == 0;
  if (x0) {
    for (int i = tid; i < DK; i += NT) {
      const float v = p.xprev_in[(size_t)bh * DK + i];
      s_x0[i] = round_x0 ? bf16_bits_to_f32(f32_to_bf16_bits(v)) : v;
    }
    __syncthreads();
  }
  if (c == 0)
    for (int i = tid; i < DK; i += NT) rec[RecPV::kX0 + i] = x0 ? s_x0[i] : 0.f;

  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  constexpr int VW = In<InT>::VW;
  constexpr int GPR = DK / VW;       // granules per row
  constexpr int NG = CH * GPR / NT;  // granules per thread
  static_assert(NG >= 1 && GPR <= 64, "granules");
  const InT* kb = static_cast<const InT*>(p.k) + (size_t)bh * p.T * DK;
  const InT* qb = static_cast<const InT*>(p.q) + (size_t)bh * p.T * DK;
#pragma unroll
  for (int r = 0; r < NG; ++r) {
    const int gi = tid + NT * r, t = gi / GPR, cc = (gi % GPR) * VW, tau = t0 + t;
    u32x4 wx = {0u, 0u, 0u, 0u}, wq = {0u, 0u, 0u, 0u};
    const bool first = tau == 0;
    if (tau < p.T) {
      if (tau >= 1) wx = *reinterpret_cast<const u32x4*>(kb + (size_t)(tau - 1) * DK + cc);
      wq = *reinterpret_cast<const u32x4*>(qb + (size_t)tau * DK + cc);
    }
    float x[VW], q[VW];
    In<InT>::decode(wx, x);
    In<InT>::decode(wq, q);
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      if (first) x[j] = x0 ? s_x0[cc + j] : 0.f;  // phi(k) already
      else if (elu && tau < p.T) x[j] = phi_elu1(x[j]);
      if (elu && tau < p.T) q[j] = phi_elu1(q[j]);
    }
    float ex = 0.f, eq = 0.f;
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      ex += x[j] * x[j];
      eq += q[j] * q[j];
    }
    if constexpr (EXACT) {
      if (first) {  // the rounded carried key, exact in bf16
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wx[j] = (uint32_t)f32_to_bf16_bits(x[2 * j]) | ((uint32_t)f32_to_bf16_bits(x[2 * j + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(Xb + t * LDB + cc) = wx;
      *reinterpret_cast<u32x4*>(Qb + t * LDB + cc) = wq;
    } else {
#pragma unroll
      for (int j = 0; j < VW; j += 4) {
        *reinterpret_cast<f4*>(Xs + t * LDX + cc + j) = f4{x[j], x[j + 1], x[j + 2], x[j + 3]};
        *reinterpret_cast<f4*>(Qs + t * LDX + cc + j) = f4{q[j], q[j + 1], q[j + 2], q[j + 3]};
      }
    }
    // the row's threads are GPR consecutive lanes
#pragma unroll
    for (int o = 1; o < GPR; o <<= 1) {
      ex += __shfl_xor(ex, o);
      eq += __shfl_xor(eq, o);
    }
    if (gi % GPR == 0) {
      s_e[t] = ex;
      s_nq[t] = eq;
    }
  }
  __syncthreads();
  // token scalars (wave 0, lane = token)
  if (wave == 0) {
    const int t = lane, tau = t0 + t;
    float e = s_e[t];
    const float nq = s_nq[t];
    const float len = qk_length(p.flags, DK);
    float nx = 1.f, mq = 1.f;
    if (len > 0.f) {
      nx = rescale_factor(e, len);
      mq = rescale_factor(nq, len);
      e *= nx * nx;
    }
    float lam = 0.f;
    if (tau < p.T && p.lam != nullptr) lam = act_lam(p.lam[(size_t)bh * p.T + tau], p.flags, true);
    if (p.flags & kFlagLamScaled) lam *= e;
    const bool key = tau < p.T && (tau >= 1 || has_in);
    rec[RecPV::kDen + t] = key ? e + lam + p.eps : __builtin_inff();
    rec[RecPV::kLam + t] = lam;
    rec[RecPV::kNx + t] = nx;
    rec[RecPV::kMq + t] = mq;
    s_nx[t] = nx;
    s_mq[t] = mq;
  }
  __syncthreads();
  // G and P: 10 lower 16x16 tiles each; wave w takes tiles w, w+4, ...
  for (int job = wave; job < 32; job += 4) {
    const int mat = job >> 4, mt = (job >> 2) & 3, nt = job & 3;  // mat 0: G, 1: P
    float* dst = rec + (mat == 0 ? RecPV::kG : RecPV::kP);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mt >= nt) {
      if constexpr (EXACT) {
        // A: rows 16 mt + n, K slots 8g..8g+7 of each 32-wide block; B likewise from X
        const uint16_t* arow = (mat == 0 ? Xb : Qb) + (16 * mt + n) * LDB + 8 * g;
        const uint16_t* brow = Xb + (16 * nt + n) * LDB + 8 * g;
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq)
          mma_bf16(acc, *reinterpret_cast<const bf8*>(arow + 32 * kq), *reinterpret_cast<const bf8*>(brow + 32 * kq));
      } else {
        const float* arow = (mat == 0 ? Xs : Qs) + (16 * mt + n) * LDX;
        const float* brow = Xs + (16 * nt + n) * LDX;
#pragma unroll 4
        for (int kq = 0; kq < DK / 16; ++kq) {
          const f4 a = *reinterpret_cast<const f4*>(arow + 16 * kq + 4 * g);
          const f4 b = *reinterpret_cast<const f4*>(brow + 16 * kq + 4 * g);
          mma_block(acc, a, b);
        }
      }
    }
    const int s2 = 16 * nt + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g + i;
      const bool keep = mat == 0 ? s2 < t : s2 <= t;
      const float f = (mat == 0 ? s_nx[t] : s_mq[t]) * s_nx[s2];
      const float v = keep ? f * acc[i] : 0.f;
      if (EXACT && mat == 1) {
        uint16_t* ph = reinterpret_cast<uint16_t*>(dst);
        const uint16_t h = f32_to_bf16_bits(v);
        ph[t * CH + s2] = h;
        ph[CH * CH + t * CH + s2] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
      } else {
        dst[t * CH + s2] = v;
      }
    }
  }
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The value of lane group gp (lanes 16 gp .. 16 gp + 15) in every lane group, lane n of
// each group taking lane n of group gp: v_permlane16_swap exchanges the odd 16-lane rows
// of its first operand with the even rows of its second, and v_permlane32_swap the upper
// 32 lanes of its first operand with the lower 32 of its second. From x in both operands,
// the first swap leaves rows (0, 0, 2, 2) in its first result and (1, 1, 3, 3) in its
// second; swapping either with itself across the halves leaves rows (0, 0, 0, 0) or
// (1, 1, 1, 1) in the first result and (2, 2, 2, 2) or (3, 3, 3, 3) in the second.
// Every lane must be active.
template <int GP>
__device__ __forceinline__ float group_bcast(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t y = (GP & 1) ? a[1] : a[0];
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float((GP & 2) ? b[1] : b[0]);
}

// Gate activation of beta with a hardware reciprocal (the fused variants of act_beta).
__device__ __forceinline__ float act_beta_pv(float z, uint32_t flags) {
  if (flags & kFlagBetaSig) return __builtin_amdgcn_rcpf(1.f + __expf(-z));
  if (flags & kFlagBetaSig2) return 2.f * __builtin_amdgcn_rcpf(1.f + __expf(-z));
  return z;
}

// Exclusive prefix over the column's four lane groups g (lanes n, n+16, n+32, n+48) of a
// lane total, and the sum over all four.
__device__ __forceinline__ void group_prefix(float v, int pv, int g, int n, float& excl, int& pexcl,
                                             float& tot, int& ptot) {
  excl = 0.f;
  tot = 0.f;
  pexcl = 0;
  ptot = 0;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    const float u = __shfl(v, 16 * gg + n);
    const int pu = __shfl(pv, 16 * gg + n);
    if (gg < g) {
      excl += u;
      pexcl ^= pu;
    }
    tot += u;
    ptot ^= pu;
  }
}

template <int DK>
constexpr size_t prop_pv_floats() {
  // X, Q; G, P (fp32, or bf16 hi and lo rows of CH + 8), beta, V; four token scalars
  return 2 * (size_t)CH * (DK + 4) + 3 * (size_t)CH * LDM + (size_t)CH * (CH + 8) + 4 * CH;
}

template <typename InT, int DK, bool EXACT>
__global__ __launch_bounds__(NT) void prop_pv_kernel(ScanParams p) {
  constexpr int LDX = DK + 4, NRT = DK / 16;
  static_assert(!EXACT || sizeof(InT) == 2, "exact operands are bf16");
  static_assert(4 * prop_pv_floats<DK>() <= 160 * 1024, "LDS");
  __shared__ __align__(16) float smem[prop_pv_floats<DK>()];
  float* Xs = smem;                 // [CH][LDX] phi(x_t) (fp32 operands)
  float* Qs = Xs + CH * LDX;        // [CH][LDX] phi(q_t)
  // exact operands in the same space: X and Q rows, raw bf16 (X^T operands are read
  // from the X rows with the LDS transpose read)
  constexpr int LDB = DK + 8;
  static_assert(2 * CH * LDB * 2 <= 2 * CH * LDX * 4, "bf16 operands fit");
  uint16_t* Xb = reinterpret_cast<uint16_t*>(smem);  // [CH][LDB]
  uint16_t* Qb = Xb + CH * LDB;                      // [CH][LDB]
  float* Gs = Qs + CH * LDX;        // [CH][LDM]
  float* Ps = Gs + CH * LDM;        // [CH][LDM] (fp32 operands)
  constexpr int LDPB = CH + 8;      // bf16 P rows (exact operands): hi [CH][LDPB], then lo
  static_assert(CH * LDM <= CH * LDPB, "P space");
  uint16_t* Pb = reinterpret_cast<uint16_t*>(Ps);
  float* Bs = Ps + CH * LDPB;       // [CH][LDM] beta of the group's 64 columns
  float* Vs = Bs + CH * LDM;        // [CH][LDM] values of the group's 64 columns
  float* s_rden = Vs + CH * LDM;    // [CH] 1 / eta's denominator (0 where no key is written)
  float* s_lam = s_rden + CH;       // [CH]
  float* s_nx = s_lam + CH;         // [CH]
  float* s_mq = s_nx + CH;          // [CH]

  const int ngrp = p.dv / 64;
  const int bh = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int dv = p.dv, cw = 16 * wave + n;  // the lane's column within the group
  const int col = 64 * grp + cw;
  const size_t rowbase = (size_t)bh * p.T;
  const InT* vb = static_cast<const InT*>(p.v) + rowbase * dv + 64 * grp;
  const float* bb = p.beta + rowbase * dv + 64 * grp;

  const float* rec0 = reinterpret_cast<const float*>(p.ws + (size_t)bh * p.nchunks * RecPV::kBytes);
  constexpr uint32_t OES = 4;  // output element bytes (fp32; bf16 output halves it)
  const bool obf = (p.flags & kFlagOutBf16) != 0;
  const __amdgpu_buffer_rsrc_t ro = rsrc(static_cast<const char*>(p.out) + rowbase * dv * (obf ? 2 : OES),
                                         (uint32_t)(p.T * dv) * (obf ? 2u : OES));
  const uint32_t olane = (uint32_t)(4 * g * dv + col);  // element offset of the lane's first row
  f4 s[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + 16 * rt + 4 * g + i) * dv + col] : 0.f;

  // Chunk c+1 is loaded into registers (16-byte loads) while chunk c computes, then
  // written to LDS at the top of the next iteration. X and Q go to LDS as phi(x), phi(q)
  // without their rescale factors, which scale the products' rows instead.
  constexpr int VW = In<InT>::VW;
  constexpr int GPR = DK / VW;             // granules per X / Q row
  constexpr int NGX = CH * GPR / NT;       // X (and Q) granules per thread
  constexpr int NGV = CH * (64 / VW) / NT; // value granules per thread
  static_assert(NGX >= 1 && NGV >= 1, "granules");
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const InT* kbase = static_cast<const InT*>(p.k) + rowbase * DK;
  const InT* qbase = static_cast<const InT*>(p.q) + rowbase * DK;
  u32x4 px[NGX], pq[NGX], pv[NGV];
  f4 pg[4], pp[4], pb[4];
  f4 psc = {0.f, 0.f, 0.f, 0.f};  // den, lambda, nx, mq of token tid (tid < CH)
  uint32_t xzero = 0;             // granules of the carried key (the sequence's first token)

  // Buffer resources of the head's rows; rows past the sequence end read as zeros. The key
  // resource starts one row early (x_t is the key before token t); the sequence's first
  // token reads out of range and takes the carried key instead.
  constexpr int ES = sizeof(InT);
  const __amdgpu_buffer_rsrc_t rk = rsrc(kbase - DK, (uint32_t)(p.T * DK * ES));
  const __amdgpu_buffer_rsrc_t rq = rsrc(qbase, (uint32_t)(p.T * DK * ES));
  const __amdgpu_buffer_rsrc_t rv = rsrc(vb, (uint32_t)((p.T * dv - 64 * grp) * ES));
  const __amdgpu_buffer_rsrc_t rb = rsrc(bb, (uint32_t)((p.T * dv - 64 * grp) * 4));
  const __amdgpu_buffer_rsrc_t rw = rsrc(rec0, (uint32_t)((size_t)p.nchunks * RecPV::kBytes));
  uint32_t ox[NGX], ob[4], ov[NGV];  // loop-invariant lane offsets (bytes from the chunk's first row)
#pragma unroll
  for (int r = 0; r < NGX; ++r) {
    const int gi = tid + NT * r;
    ox[r] = (uint32_t)(((gi / GPR) * DK + (gi % GPR) * VW) * ES);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gi = tid + NT * r;
    ob[r] = (uint32_t)(((gi / 16) * dv + (gi % 16) * 4) * 4);
  }
#pragma unroll
  for (int r = 0; r < NGV; ++r) {
    const int gi = tid + NT * r;
    ov[r] = (uint32_t)(((gi / (64 / VW)) * dv + (gi % (64 / VW)) * VW) * ES);
  }

  auto prefetch = [&](int cn) {
    const uint32_t sx = (uint32_t)(cn * CH * DK * ES), sv = (uint32_t)(cn * CH * dv);
    const uint32_t sw = (uint32_t)((size_t)cn * RecPV::kBytes);
    xzero = 0;
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const bool first = cn == 0 && tid + NT * r < GPR;  // token 0 of the sequence
      px[r] = bload16(rk, first ? 0x80000000u : ox[r], sx);
      pq[r] = bload16(rq, ox[r], sx);
      if (first) xzero |= 1u << r;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t o = (uint32_t)(16 * (tid + NT * r));
      pg[r] = __builtin_bit_cast(f4, bload16(rw, (uint32_t)(4 * RecPV::kG) + o, sw));
      pp[r] = __builtin_bit_cast(f4, bload16(rw, (uint32_t)(4 * RecPV::kP) + o, sw));
      pb[r] = __builtin_bit_cast(f4, bload16(rb, ob[r], sv * 4u));
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) pv[r] = bload16(rv, ov[r], sv * (uint32_t)ES);
    if (tid < CH) {
      const float* rec = reinterpret_cast<const float*>(p.ws + ((size_t)bh * p.nchunks + cn) * RecPV::kBytes);
      psc = f4{rec[RecPV::kDen + tid], rec[RecPV::kLam + tid], rec[RecPV::kNx + tid], rec[RecPV::kMq + tid]};
    }
  };

  prefetch(0);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * CH;
    // ---- registers -> LDS (chunk c)
    if constexpr (EXACT) {
#pragma unroll
      for (int r = 0; r < NGX; ++r) {
        const int gi = tid + NT * r, t = gi / GPR, cc = (gi % GPR) * VW;
        u32x4 w = px[r];
        if ((xzero >> r) & 1u) {  // the carried key, already bf16-exact in the record
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)f32_to_bf16_bits(rec0[RecPV::kX0 + cc + 2 * j]) |
                   ((uint32_t)f32_to_bf16_bits(rec0[RecPV::kX0 + cc + 2 * j + 1]) << 16);
        }
        *reinterpret_cast<u32x4*>(Xb + t * LDB + cc) = w;
        *reinterpret_cast<u32x4*>(Qb + t * LDB + cc) = pq[r];
      }
    }
#pragma unroll
    for (int r = 0; r < (EXACT ? 0 : NGX); ++r) {
      const int gi = tid + NT * r, t = gi / GPR, cc = (gi % GPR) * VW;
      float x[VW], q[VW];
      In<InT>::decode(px[r], x);
      In<InT>::decode(pq[r], q);
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if ((xzero >> r) & 1u) x[j] = rec0[RecPV::kX0 + cc + j];  // the carried key, phi(k) already
        else if (elu) x[j] = phi_elu1(x[j]);
        if (elu) q[j] = phi_elu1(q[j]);
      }
#pragma unroll
      for (int j = 0; j < VW; j += 4) {
        *reinterpret_cast<f4*>(Xs + t * LDX + cc + j) = f4{x[j], x[j + 1], x[j + 2], x[j + 3]};
        *reinterpret_cast<f4*>(Qs + t * LDX + cc + j) = f4{q[j], q[j + 1], q[j + 2], q[j + 3]};
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gi = tid + NT * r, t = gi / 16, u = (gi % 16) * 4;
      f4 b = pb[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = act_beta_pv(b[j], p.flags);
      *reinterpret_cast<f4*>(Gs + t * LDM + u) = pg[r];
      if constexpr (EXACT) {  // granule gi of the record's [2][CH][CH] bf16 P
        const int h = gi / (CH * CH / 8), rem = gi % (CH * CH / 8);
        *reinterpret_cast<f4*>(Pb + h * CH * LDPB + (rem / 8) * LDPB + (rem % 8) * 8) = pp[r];
      } else {
        *reinterpret_cast<f4*>(Ps + t * LDM + u) = pp[r];
      }
      *reinterpret_cast<f4*>(Bs + t * LDM + u) = b;  // rows past the end hold act(0); V is 0 there
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = tid + NT * r, t = gi / (64 / VW), u = (gi % (64 / VW)) * VW;
      float x[VW];
      In<InT>::decode(pv[r], x);
#pragma unroll
      for (int j = 0; j < VW; j += 4) *reinterpret_cast<f4*>(Vs + t * LDM + u + j) = f4{x[j], x[j + 1], x[j + 2], x[j + 3]};
    }
    if (tid < CH) {
      s_rden[tid] = 1.f / psc[0];
      s_lam[tid] = psc[1];
      s_nx[tid] = psc[2];
      s_mq[tid] = psc[3];
    }
    __syncthreads();
    if (c + 1 < p.nchunks) prefetch(c + 1);

    // ---- X S0 and Q S0 (C layout: rows 16 mt + 4 g + i, column n), rows rescaled
    f4 XS[4], QS[4];
    bf8 sh[EXACT ? DK / 32 : 1], sl[EXACT ? DK / 32 : 1];
    if constexpr (EXACT) {
#pragma unroll
      for (int kq = 0; kq < DK / 32; ++kq) split_c(s, kq, sh[kq], sl[kq]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      XS[mt] = f4{0.f, 0.f, 0.f, 0.f};
      QS[mt] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (EXACT) {
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq) {
          const bf8 ax = frag_pair(Xb + (16 * mt + n) * LDB + 32 * kq + 4 * g);
          const bf8 aq = frag_pair(Qb + (16 * mt + n) * LDB + 32 * kq + 4 * g);
          mma_bf16(XS[mt], ax, sh[kq]);
          mma_bf16(QS[mt], aq, sh[kq]);
          mma_bf16(XS[mt], ax, sl[kq]);
          mma_bf16(QS[mt], aq, sl[kq]);
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const f4 ax = *reinterpret_cast<const f4*>(Xs + (16 * mt + n) * LDX + 16 * rt + 4 * g);
          const f4 aq = *reinterpret_cast<const f4*>(Qs + (16 * mt + n) * LDX + 16 * rt + 4 * g);
          mma_block(XS[mt], ax, s[rt]);
          mma_block(QS[mt], aq, s[rt]);
        }
      }
      XS[mt] *= *reinterpret_cast<const f4*>(s_nx + 16 * mt + 4 * g);
      QS[mt] *= *reinterpret_cast<const f4*>(s_mq + 16 * mt + 4 * g);
    }

    // ---- per (token, column): eta, decay, and the in-chunk prefix of log2 |decay|
    float eta[4][4], la[4][4];
    int ng[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float e = Bs[t * LDM + cw] * s_rden[t];  // 0 where there is no key
        const float a = 1.f - e * s_lam[t];
        eta[mt][i] = e;
        la[mt][i] = __builtin_amdgcn_logf(fmaxf(fabsf(a), 1e-30f));
        ng[mt][i] = a < 0.f ? 1 : 0;
      }
    float gl[4][4];
    int pg[4][4];
    {
      float carry = 0.f;
      int pcarry = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float run = 0.f;
        int prun = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          run += la[mt][i];
          prun ^= ng[mt][i];
          gl[mt][i] = run;
          pg[mt][i] = prun;
        }
        float excl, tot;
        int pexcl, ptot;
        group_prefix(run, prun, g, n, excl, pexcl, tot, ptot);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gl[mt][i] += carry + excl;
          pg[mt][i] ^= pcarry ^ pexcl;
        }
        carry += tot;
        pcarry ^= ptot;
      }
    }
    // anchor A = token 31 (row tile 1, g = 3, i = 3); chunk end C = token 63
    const float gA = __shfl(gl[1][3], 48 + n);
    const int pA = __shfl(pg[1][3], 48 + n);
    const float gC = __shfl(gl[3][3], 48 + n);
    const int pC = __shfl(pg[3][3], 48 + n);
    const float GamC = with_sign(__builtin_amdgcn_exp2f(gC), pC);
    const float GhC = with_sign(__builtin_amdgcn_exp2f(gC - gA), pC ^ pA);

    // right-hand sides and row factors of the triangular system. The factors of token
    // t-1 are those of the lane's previous row, except in its first row, where they are
    // formed from the prefix before token t.
    float rhs[4][4], ef[4][4], Gam[4][4], Gh[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const int pa = pg[mt][i] ^ pA;
        Gam[mt][i] = with_sign(__builtin_amdgcn_exp2f(gl[mt][i]), pg[mt][i]);
        Gh[mt][i] = with_sign(__builtin_amdgcn_exp2f(gl[mt][i] - gA), pa);
        float Gprev, Ghprev;
        if (i == 0) {
          const float gprev = gl[mt][i] - la[mt][i];
          const int pprev = pg[mt][i] ^ ng[mt][i];
          Gprev = with_sign(__builtin_amdgcn_exp2f(gprev), pprev);
          Ghprev = with_sign(__builtin_amdgcn_exp2f(gprev - gA), pprev ^ pA);
        } else {
          Gprev = Gam[mt][i - 1];
          Ghprev = Gh[mt][i - 1];
        }
        const float cf = eta[mt][i] * with_sign(__builtin_amdgcn_exp2f(gA - gl[mt][i]), pa);  // eta / Gh
        rhs[mt][i] = cf * (Vs[t * LDM + cw] - Gprev * XS[mt][i]);
        ef[mt][i] = cf * Ghprev;
      }

    // ---- W~ by blocked forward substitution. The off-diagonal 16 x 16 blocks run on
    // fp32 MFMA: once block bk is solved, its product with G goes into the running sums
    // y of every later block, so a block waits only for the products of the block just
    // before it. Inside a diagonal block the rows go in four groups of four, each held
    // by one lane group (lane (g, n) owns rows 4g..4g+3 of column n): group gp solves its
    // 4 x 4 lower-triangular block in registers, lane swaps hand its four values to the
    // other groups of the column, and the later groups subtract ef (G w).
    f4 W[4], y[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) y[bi] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      f4 cv;
#pragma unroll
      for (int i = 0; i < 4; ++i) cv[i] = rhs[bi][i] - ef[bi][i] * y[bi][i];
      // this lane's rows of the diagonal block: G[16 bi + 4 g + i][16 bi + ...]; the rows
      // against group gp + 1 are read while step gp computes
      const float* gd = Gs + (16 * bi + 4 * g) * LDM + 16 * bi;
      f4 rgn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rgn[i] = *reinterpret_cast<const f4*>(gd + i * LDM);
      static_for<0, 4>([&](auto GPc) {
        constexpr int gp = GPc;
        // the rows of group gp's own block, and this lane's rows against group gp
        f4 rg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rg[i] = rgn[i];
        if constexpr (gp < 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i) rgn[i] = *reinterpret_cast<const f4*>(gd + i * LDM + 4 * (gp + 1));
        }
        if (g == gp) {
          cv[1] -= ef[bi][1] * (rg[1][0] * cv[0]);
          cv[2] -= ef[bi][2] * (rg[2][0] * cv[0] + rg[2][1] * cv[1]);
          cv[3] -= ef[bi][3] * (rg[3][0] * cv[0] + rg[3][1] * cv[1] + rg[3][2] * cv[2]);
        }
        if constexpr (gp < 3) {
          f4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = group_bcast<gp>(cv[j]);
          if (g > gp) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              cv[i] -= ef[bi][i] * (rg[i][0] * w[0] + rg[i][1] * w[1] + rg[i][2] * w[2] + rg[i][3] * w[3]);
          }
        }
      });
      W[bi] = cv;
      // this block's share of the later blocks' sums
#pragma unroll
      for (int bl = bi + 1; bl < 4; ++bl) {
        const f4 a = *reinterpret_cast<const f4*>(Gs + (16 * bl + n) * LDM + 16 * bi + 4 * g);
        mma_block(y[bl], a, W[bi]);
      }
    }

    // ---- O = Gamma o (Q S0) + Gamma^ o (P W~), stored
    // P W~ with the products of the four row tiles interleaved (independent sums): on
    // bf16 MFMA with P and W~ split into hi and lo halves (exact operands), else fp32
    f4 pws[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) pws[mt] = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (EXACT) {
      bf8 wph[2], wpl[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) split_c(W, kq, wph[kq], wpl[kq]);
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int mt = 2 * kq; mt < 4; ++mt) {  // K block kq reaches row tiles 2 kq and up
            const bf8 a = frag_pair(Pb + (part == 2 ? CH * LDPB : 0) + (16 * mt + n) * LDPB + 32 * kq + 4 * g);
            mma_bf16(pws[mt], a, part == 1 ? wpl[kq] : wph[kq]);
          }
    } else {
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) {
        f4 a[4];
#pragma unroll
        for (int mt = bk; mt < 4; ++mt) a[mt] = *reinterpret_cast<const f4*>(Ps + (16 * mt + n) * LDM + 16 * bk + 4 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int mt = bk; mt < 4; ++mt)
            pws[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt][q], W[bk][q], pws[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f4 pw = pws[mt];
      // rows past the sequence end fall outside the output resource
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = Gam[mt][i] * QS[mt][i] + Gh[mt][i] * pw[i];
        const uint32_t so = (uint32_t)((t0 + 16 * mt + i) * dv);
        if (obf) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o), ro, 2u * olane, 2u * so, 0);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ro, OES * olane, OES * so, 0);
      }
    }

    // ---- S' = Gamma_C S0 + Gamma^_C X^T W~ (W~ rows times the keys' rescale factors)
    if constexpr (EXACT) {
      f4 Wn[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Wn[kb] = W[kb] * *reinterpret_cast<const f4*>(s_nx + 16 * kb + 4 * g);
      bf8 wh[2], wl[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) split_c(Wn, kq, wh[kq], wl[kq]);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const bf8 a = xt_frag(Xb + (32 * kq + 4 * g + (n >> 2)) * LDB + 16 * rt + 4 * (n & 3), LDB);
          mma_bf16(acc, a, wh[kq]);
          mma_bf16(acc, a, wl[kq]);
        }
        s[rt] = s[rt] * GamC + acc * GhC;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          f4 a;
#pragma unroll
          for (int q = 0; q < 4; ++q) a[q] = Xs[(16 * kb + 4 * g + q) * LDX + 16 * rt + n];
          mma_block(acc, a, W[kb] * *reinterpret_cast<const f4*>(s_nx + 16 * kb + 4 * g));
        }
        s[rt] = s[rt] * GamC + acc * GhC;
      }
    }
    __syncthreads();  // LDS is restaged next chunk
  }

  if (p.S_out != nullptr) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.S_out[((size_t)bh * DK + 16 * rt + 4 * g + i) * dv + col] = s[rt][i];
    if (grp == 0) {
      const bool elu = (p.flags & kFlagPhiElu1) != 0;
      const InT* kb = static_cast<const InT*>(p.k) + (rowbase + p.T - 1) * DK;
      for (int i = tid; i < DK; i += NT) {
        float x = In<InT>::load1(kb + i);
        if (elu) x = phi_elu1(x);
        p.xprev_out[(size_t)bh * DK + i] = x;
      }
      if (tid == 0) p.has_out[bh] = 1;
    }
  }
}

// ---- the propagate with its roles split (bf16 inputs, identity map): one workgroup per
// (head, 32 value columns), so that every CU holds one and each of its four waves has a
// SIMD of its own. Waves 0 and 1 hold the state (X S, Q S, P W~, the outputs and the S
// update), waves 2 and 3 solve the triangular systems; waves w and w + 2 own value columns
// 16 w .. 16 w + 15 of the group.
// Three workgroup barriers per chunk:
//   [A] state: X S -> hand-off         solver: its per-(token, column) factors
//   [B] solver: right-hand sides and W~ -> hand-off
//       state: Q S, its own factors (Gamma, Gamma^), the previous chunk's outputs, the
//              next chunk's X into LDS
//   [C] state: the S update, the next chunk's Q and P into LDS
//       solver: the next chunk's G, V and token scalars into LDS
// so that the solve, the longest serial part of a chunk, runs beside the output work, and
// the chain from one chunk's W~ to the next chunk's X S holds only the S update. Each role
// loads the next chunk's rows into registers early in the chunk. X, P and the token
// scalars have two LDS buffers, since the state waves still read this chunk's after [C]
// (P until [C] of the next chunk); G and V are read by the solver waves alone, Q only
// between [B] and [C].
template <int DK>
struct Pv2Lds {
  static constexpr int LDB = DK + 8, LDPB = CH + 8, LDV2 = 32 + 4;
  static constexpr size_t kX = 0;                                  // uint16 [2][CH][LDB]
  static constexpr size_t kQ = kX + 2 * (size_t)CH * LDB * 2;      // uint16 [CH][LDB]
  static constexpr size_t kP = kQ + (size_t)CH * LDB * 2;          // uint16 [2][2][CH][LDPB] (buffer, hi/lo)
  static constexpr size_t kG = kP + 4 * (size_t)CH * LDPB * 2;     // float [CH][LDM]
  static constexpr size_t kV = kG + (size_t)CH * LDM * 4;          // float [CH][LDV2]
  static constexpr size_t kSc = kV + (size_t)CH * LDV2 * 4;        // float [2][4][CH]: 1/den, lambda, nx, mq
  static constexpr size_t kH1 = kSc + 2 * 4 * (size_t)CH * 4;      // f4 [2 waves][4][64 lanes]: X S
  static constexpr size_t kH2 = kH1 + 2 * 4 * 64 * 16;             // f4 [2 waves][4][64 lanes]: W~
  static constexpr size_t kBytes = kH2 + 2 * 4 * 64 * 16;
};

template <int DK>
__global__ __launch_bounds__(256) void prop_pv2_kernel(ScanParams p) {
  using L = Pv2Lds<DK>;
  constexpr int NR = 128;  // threads per role
  constexpr int NRT = DK / 16, LDB = L::LDB, LDPB = L::LDPB, LDV2 = L::LDV2;
  static_assert(L::kBytes <= 160 * 1024, "LDS");
  __shared__ __align__(16) char smem[L::kBytes];
  uint16_t* const Xb0 = reinterpret_cast<uint16_t*>(smem + L::kX);
  uint16_t* const Qb = reinterpret_cast<uint16_t*>(smem + L::kQ);
  uint16_t* const Pb0 = reinterpret_cast<uint16_t*>(smem + L::kP);
  float* const Gs = reinterpret_cast<float*>(smem + L::kG);
  float* const Vs = reinterpret_cast<float*>(smem + L::kV);
  float* const Sc0 = reinterpret_cast<float*>(smem + L::kSc);
  f4* const H1 = reinterpret_cast<f4*>(smem + L::kH1);
  f4* const H2 = reinterpret_cast<f4*>(smem + L::kH2);

  // The column groups of a head read the same rows and records. Workgroups are dealt to
  // the eight XCDs in turn, so with a multiple of eight heads, groups of one head take
  // workgroup indices eight apart and share an XCD's L2.
  const int ngrp = p.dv / 32, blk = blockIdx.x;
  const bool xcd = (p.BH & 7) == 0;
  const int bh = xcd ? (blk / (8 * ngrp)) * 8 + (blk & 7) : blk / ngrp;
  const int grp = xcd ? (blk >> 3) % ngrp : blk % ngrp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool solver = wave >= 2;
  const int w4 = wave & 1, rt_id = tid & (NR - 1);  // wave and thread index within the role
  const int g = lane >> 4, n = lane & 15;
  const int dv = p.dv, cw = 16 * w4 + n;  // the lane's column within the group
  const int col = 32 * grp + cw;
  const size_t rowbase = (size_t)bh * p.T;
  constexpr int ES = 2;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const uint16_t* qbase = static_cast<const uint16_t*>(p.q) + rowbase * DK;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v) + rowbase * dv + 32 * grp;
  const float* bb = p.beta + rowbase * dv + 32 * grp;
  const float* rec0 = reinterpret_cast<const float*>(p.ws + (size_t)bh * p.nchunks * RecPV::kBytes);
  const bool obf = (p.flags & kFlagOutBf16) != 0;
  const __amdgpu_buffer_rsrc_t ro = rsrc(static_cast<const char*>(p.out) + rowbase * dv * (obf ? 2 : 4),
                                         (uint32_t)(p.T * dv) * (obf ? 2u : 4u));
  const uint32_t olane = (uint32_t)(4 * g * dv + col);

  // Buffer resources of the head's rows; rows past the sequence end read as zeros. The key
  // resource starts one row early (x_t is the key before token t); the sequence's first
  // token reads out of range and takes the carried key from the record.
  const __amdgpu_buffer_rsrc_t rk = rsrc(kbase - DK, (uint32_t)(p.T * DK * ES));
  const __amdgpu_buffer_rsrc_t rq = rsrc(qbase, (uint32_t)(p.T * DK * ES));
  const __amdgpu_buffer_rsrc_t rv = rsrc(vb, (uint32_t)((p.T * dv - 32 * grp) * ES));
  const __amdgpu_buffer_rsrc_t rb = rsrc(bb, (uint32_t)((p.T * dv - 32 * grp) * 4));
  const __amdgpu_buffer_rsrc_t rw = rsrc(rec0, (uint32_t)((size_t)p.nchunks * RecPV::kBytes));

  // ---- registers of the next chunk's rows, and each role's raw beta of the lane's rows
  // 16 mt + 4 g + i, column col, for the next chunk
  constexpr int GPR = DK / 8;               // granules per X / Q row
  constexpr int NGX = CH * GPR / NR;        // X (and Q) granules per thread
  static_assert(NGX >= 1 && (CH * GPR) % NR == 0, "granules");
  constexpr int NGM = CH * CH / 4 / NR;  // granules of a [CH][CH] fp32 matrix (or the bf16 P pair) per thread
  constexpr int NGV = CH * 4 / NR;       // value granules per thread (four per 32-column row)
  u32x4 px[NGX], pq[NGX], pp[NGM], pg[NGM], pv[NGV];
  f4 psc = {0.f, 0.f, 0.f, 0.f};
  uint32_t xzero = 0;
  auto load_beta = [&](int cn, float (&bq)[4][4]) {
    const uint32_t sv = (uint32_t)(cn * CH * dv);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bq[mt][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rb, (uint32_t)(((16 * mt + 4 * g + i) * dv + cw) * 4), sv * 4u, 0));
  };
  // the rows of chunk cn into registers: X, Q, P (state role), G, V, token scalars (solver)
  auto prefetch_state = [&](int cn) {
    const uint32_t sx = (uint32_t)(cn * CH * DK * ES);
    const uint32_t sw = (uint32_t)((size_t)cn * RecPV::kBytes);
    xzero = 0;
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const int gi = rt_id + NR * r;
      const bool first = cn == 0 && gi < GPR;  // token 0 of the sequence
      const uint32_t o = (uint32_t)(((gi / GPR) * DK + (gi % GPR) * 8) * ES);
      px[r] = bload16(rk, first ? 0x80000000u : o, sx);
      pq[r] = bload16(rq, o, sx);
      if (first) xzero |= 1u << r;
    }
#pragma unroll
    for (int r = 0; r < NGM; ++r)
      pp[r] = bload16(rw, (uint32_t)(4 * RecPV::kP) + (uint32_t)(16 * (rt_id + NR * r)), sw);
  };
  auto prefetch_solver = [&](int cn) {
    const uint32_t sv = (uint32_t)(cn * CH * dv);
    const uint32_t sw = (uint32_t)((size_t)cn * RecPV::kBytes);
#pragma unroll
    for (int r = 0; r < NGM; ++r)
      pg[r] = bload16(rw, (uint32_t)(4 * RecPV::kG) + (uint32_t)(16 * (rt_id + NR * r)), sw);
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = rt_id + NR * r;
      pv[r] = bload16(rv, (uint32_t)(((gi / 4) * dv + (gi % 4) * 8) * ES), sv * (uint32_t)ES);
    }
    if (rt_id < CH) {
      const float* rec = reinterpret_cast<const float*>(p.ws + ((size_t)bh * p.nchunks + cn) * RecPV::kBytes);
      psc = f4{rec[RecPV::kDen + rt_id], rec[RecPV::kLam + rt_id], rec[RecPV::kNx + rt_id], rec[RecPV::kMq + rt_id]};
    }
  };
  // registers -> LDS for chunk cn (its X, P and token-scalar buffers cn & 1)
  auto stage_x = [&](int cn) {
    uint16_t* Xb = Xb0 + (cn & 1) * CH * LDB;
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const int gi = rt_id + NR * r, t = gi / GPR, cc = (gi % GPR) * 8;
      u32x4 w = px[r];
      if ((xzero >> r) & 1u) {  // the carried key, already bf16-exact in the record
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = (uint32_t)f32_to_bf16_bits(rec0[RecPV::kX0 + cc + 2 * j]) |
                 ((uint32_t)f32_to_bf16_bits(rec0[RecPV::kX0 + cc + 2 * j + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(Xb + t * LDB + cc) = w;
    }
  };
  auto stage_qp = [&](int cn) {
    uint16_t* Pb = Pb0 + (cn & 1) * 2 * CH * LDPB;
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const int gi = rt_id + NR * r;
      *reinterpret_cast<u32x4*>(Qb + (gi / GPR) * LDB + (gi % GPR) * 8) = pq[r];
    }
#pragma unroll
    for (int r = 0; r < NGM; ++r) {  // granule gi of the record's [2][CH][CH] bf16 P
      const int gi = rt_id + NR * r, h = gi / (CH * CH / 8), rem = gi % (CH * CH / 8);
      *reinterpret_cast<u32x4*>(Pb + h * CH * LDPB + (rem / 8) * LDPB + (rem % 8) * 8) = pp[r];
    }
  };
  auto stage_solver = [&](int cn) {
#pragma unroll
    for (int r = 0; r < NGM; ++r) {
      const int gi = rt_id + NR * r;
      *reinterpret_cast<u32x4*>(Gs + (gi / 16) * LDM + (gi % 16) * 4) = pg[r];
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = rt_id + NR * r, t = gi / 4, u = (gi % 4) * 8;
      float x[8];
      In<uint16_t>::decode(pv[r], x);
      *reinterpret_cast<f4*>(Vs + t * LDV2 + u) = f4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f4*>(Vs + t * LDV2 + u + 4) = f4{x[4], x[5], x[6], x[7]};
    }
    if (rt_id < CH) {
      float* sc = Sc0 + (cn & 1) * 4 * CH;
      sc[rt_id] = 1.f / psc[0];
      sc[CH + rt_id] = psc[1];
      sc[2 * CH + rt_id] = psc[2];
      sc[3 * CH + rt_id] = psc[3];
    }
  };

  // ---- per (token, column) factors of chunk cn: eta, and the in-chunk prefix of log2 |a|
  // (a sum over the lane's rows and the column's four lane groups, with a sign parity)
  float eta[4][4], gl[4][4], la[4][4];
  int pgr[4][4], ngr[4][4];
  float gA = 0.f, gC = 0.f;
  int pA = 0, pC = 0;
  auto prefix = [&](const float (&bq)[4][4], const float* sc) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float e = act_beta_pv(bq[mt][i], p.flags) * sc[t];  // 0 where there is no key
        const float a = 1.f - e * sc[CH + t];
        eta[mt][i] = e;
        la[mt][i] = __builtin_amdgcn_logf(fmaxf(fabsf(a), 1e-30f));
        ngr[mt][i] = a < 0.f ? 1 : 0;
      }
    float carry = 0.f;
    int pcarry = 0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float run = 0.f;
      int prun = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        run += la[mt][i];
        prun ^= ngr[mt][i];
        gl[mt][i] = run;
        pgr[mt][i] = prun;
      }
      float excl, tot;
      int pexcl, ptot;
      group_prefix(run, prun, g, n, excl, pexcl, tot, ptot);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gl[mt][i] += carry + excl;
        pgr[mt][i] ^= pcarry ^ pexcl;
      }
      carry += tot;
      pcarry ^= ptot;
    }
    // anchor A = token 31 (row tile 1, g = 3, i = 3); chunk end C = token 63
    gA = __shfl(gl[1][3], 48 + n);
    pA = __shfl(pgr[1][3], 48 + n);
    gC = __shfl(gl[3][3], 48 + n);
    pC = __shfl(pgr[3][3], 48 + n);
  };

  if (solver) {
    float bq[4][4];
    prefetch_solver(0);
    stage_solver(0);
    load_beta(0, bq);
    for (int c = 0; c < p.nchunks; ++c) {
      const float* sc = Sc0 + (c & 1) * 4 * CH;
      __syncthreads();  // [A] chunk c is in LDS
      if (c + 1 < p.nchunks) prefetch_solver(c + 1);
      // ---- the factors of the triangular system: rhs = cf V - gp (X S), ef = cf Gh_{t-1},
      // with cf = eta / Gh. The factors of token t-1 are those of the lane's previous row,
      // except in its first row, where they are formed from the prefix before token t.
      float cfv[4][4], gpv[4][4], ef[4][4];
      prefix(bq, sc);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pa = pgr[mt][i] ^ pA;
          float gprev;
          int pprev;
          if (i == 0) {
            gprev = gl[mt][i] - la[mt][i];
            pprev = pgr[mt][i] ^ ngr[mt][i];
          } else {
            gprev = gl[mt][i - 1];
            pprev = pgr[mt][i - 1];
          }
          const float cf = eta[mt][i] * with_sign(__builtin_amdgcn_exp2f(gA - gl[mt][i]), pa);  // eta / Gh
          cfv[mt][i] = cf;
          gpv[mt][i] = cf * with_sign(__builtin_amdgcn_exp2f(gprev), pprev);
          ef[mt][i] = cf * with_sign(__builtin_amdgcn_exp2f(gprev - gA), pprev ^ pA);
        }
      __syncthreads();  // [B] X S0 handed over
      // ---- right-hand sides, then W~ by blocked forward substitution. The off-diagonal
      // 16 x 16 blocks run on fp32 MFMA: once block bk is solved, its product with G goes
      // into the running sums y of every later block. Inside a diagonal block the rows go
      // in four groups of four, each held by one lane group (lane (g, n) owns rows
      // 4g..4g+3 of column n): group gp solves its 4 x 4 lower-triangular block in
      // registers, lane swaps hand its four values to the other groups of the column, and
      // the later groups subtract ef (G w).
      float rhs[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f4 xs = H1[(w4 * 4 + mt) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          rhs[mt][i] = cfv[mt][i] * Vs[(16 * mt + 4 * g + i) * LDV2 + cw] - gpv[mt][i] * xs[i];
      }
      f4 W[4], y[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) y[bi] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f4 cv;
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[i] = rhs[bi][i] - ef[bi][i] * y[bi][i];
        const float* gd = Gs + (16 * bi + 4 * g) * LDM + 16 * bi;
        f4 rgn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rgn[i] = *reinterpret_cast<const f4*>(gd + i * LDM);
        static_for<0, 4>([&](auto GPc) {
          constexpr int gp = GPc;
          f4 rg[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) rg[i] = rgn[i];
          if constexpr (gp < 3) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rgn[i] = *reinterpret_cast<const f4*>(gd + i * LDM + 4 * (gp + 1));
          }
          if (g == gp) {
            cv[1] -= ef[bi][1] * (rg[1][0] * cv[0]);
            cv[2] -= ef[bi][2] * (rg[2][0] * cv[0] + rg[2][1] * cv[1]);
            cv[3] -= ef[bi][3] * (rg[3][0] * cv[0] + rg[3][1] * cv[1] + rg[3][2] * cv[2]);
          }
          if constexpr (gp < 3) {
            f4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = group_bcast<gp>(cv[j]);
            if (g > gp) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                cv[i] -= ef[bi][i] * (rg[i][0] * w[0] + rg[i][1] * w[1] + rg[i][2] * w[2] + rg[i][3] * w[3]);
            }
          }
        });
        W[bi] = cv;
        H2[(w4 * 4 + bi) * 64 + lane] = cv;
#pragma unroll
        for (int bl = bi + 1; bl < 4; ++bl) {
          const f4 a = *reinterpret_cast<const f4*>(Gs + (16 * bl + n) * LDM + 16 * bi + 4 * g);
          mma_block(y[bl], a, W[bi]);
        }
      }
      __syncthreads();  // [C] W~ handed over; G and V are free
      if (c + 1 < p.nchunks) {
        stage_solver(c + 1);
        load_beta(c + 1, bq);
      }
    }
    if (grp == 0 && p.S_out != nullptr) {
      const uint16_t* kl = kbase + (size_t)(p.T - 1) * DK;
      for (int i = rt_id; i < DK; i += NR) p.xprev_out[(size_t)bh * DK + i] = In<uint16_t>::load1(kl + i);
      if (rt_id == 0) p.has_out[bh] = 1;
    }
  } else {
    f4 s[NRT];  // the state slice
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + 16 * rt + 4 * g + i) * dv + col] : 0.f;
    float bq[4][4];
    prefetch_state(0);
    stage_x(0);
    stage_qp(0);
    load_beta(0, bq);
    // The outputs of chunk c are formed while the solver works on chunk c + 1, from what
    // chunk c leaves: its W~, Q S0, factors, and P (whose LDS buffer the solver rewrites
    // only after [C] of chunk c + 1).
    f4 Wp[4], QSp[4];
    float Gamp[4][4], Ghp[4][4];
    auto outputs = [&](int cp) {
      const uint16_t* Pb = Pb0 + (cp & 1) * 2 * CH * LDPB;
      f4 pws[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) pws[mt] = f4{0.f, 0.f, 0.f, 0.f};
      bf8 wph[2], wpl[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) split_c(Wp, kq, wph[kq], wpl[kq]);
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int mt = 2 * kq; mt < 4; ++mt) {  // K block kq reaches row tiles 2 kq and up
            const bf8 a = frag_pair(Pb + (part == 2 ? CH * LDPB : 0) + (16 * mt + n) * LDPB + 32 * kq + 4 * g);
            mma_bf16(pws[mt], a, part == 1 ? wpl[kq] : wph[kq]);
          }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o = Gamp[mt][i] * QSp[mt][i] + Ghp[mt][i] * pws[mt][i];
          const uint32_t so = (uint32_t)((cp * CH + 16 * mt + i) * dv);
          if (obf) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o), ro, 2u * olane, 2u * so, 0);
          else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ro, 4u * olane, 4u * so, 0);
        }
    };
    for (int c = 0; c < p.nchunks; ++c) {
      const uint16_t* Xb = Xb0 + (c & 1) * CH * LDB;
      const float* sc = Sc0 + (c & 1) * 4 * CH;
      const float* s_nx = sc + 2 * CH;
      const float* s_mq = sc + 3 * CH;
      __syncthreads();  // [A] chunk c is in LDS
      // ---- X S0 (C layout: rows 16 mt + 4 g + i, column n), rows rescaled -> hand-off
      bf8 sh[DK / 32], sl[DK / 32];
#pragma unroll
      for (int kq = 0; kq < DK / 32; ++kq) split_c(s, kq, sh[kq], sl[kq]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq) {
          const bf8 ax = frag_pair(Xb + (16 * mt + n) * LDB + 32 * kq + 4 * g);
          mma_bf16(xs, ax, sh[kq]);
          mma_bf16(xs, ax, sl[kq]);
        }
        H1[(w4 * 4 + mt) * 64 + lane] = xs * *reinterpret_cast<const f4*>(s_nx + 16 * mt + 4 * g);
      }
      if (c + 1 < p.nchunks) prefetch_state(c + 1);
      __syncthreads();  // [B] X S0 handed over
      // ---- Q S0, rows rescaled; the decay factors Gamma and Gamma^ of the outputs and
      // the update; then the previous chunk's outputs
      f4 QS[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        QS[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < DK / 32; ++kq) {
          const bf8 aq = frag_pair(Qb + (16 * mt + n) * LDB + 32 * kq + 4 * g);
          mma_bf16(QS[mt], aq, sh[kq]);
          mma_bf16(QS[mt], aq, sl[kq]);
        }
        QS[mt] *= *reinterpret_cast<const f4*>(s_mq + 16 * mt + 4 * g);
      }
      float Gam[4][4], Gh[4][4];
      prefix(bq, sc);
      const float GamC = with_sign(__builtin_amdgcn_exp2f(gC), pC);
      const float GhC = with_sign(__builtin_amdgcn_exp2f(gC - gA), pC ^ pA);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Gam[mt][i] = with_sign(__builtin_amdgcn_exp2f(gl[mt][i]), pgr[mt][i]);
          Gh[mt][i] = with_sign(__builtin_amdgcn_exp2f(gl[mt][i] - gA), pgr[mt][i] ^ pA);
        }
      if (c + 1 < p.nchunks) load_beta(c + 1, bq);
      if (c > 0) outputs(c - 1);
      if (c + 1 < p.nchunks) stage_x(c + 1);
      __syncthreads();  // [C] W~ handed over
      f4 W[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) W[bi] = H2[(w4 * 4 + bi) * 64 + lane];
      // ---- S' = Gamma_C S0 + Gamma^_C X^T W~ (W~ rows times the keys' rescale factors)
      f4 Wn[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Wn[kb] = W[kb] * *reinterpret_cast<const f4*>(s_nx + 16 * kb + 4 * g);
      bf8 wh[2], wl[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) split_c(Wn, kq, wh[kq], wl[kq]);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const bf8 a = xt_frag(Xb + (32 * kq + 4 * g + (n >> 2)) * LDB + 16 * rt + 4 * (n & 3), LDB);
          mma_bf16(acc, a, wh[kq]);
          mma_bf16(acc, a, wl[kq]);
        }
        s[rt] = s[rt] * GamC + acc * GhC;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Wp[mt] = W[mt];
        QSp[mt] = QS[mt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Gamp[mt][i] = Gam[mt][i];
          Ghp[mt][i] = Gh[mt][i];
        }
      }
      if (c + 1 < p.nchunks) stage_qp(c + 1);
    }
    if (p.nchunks > 0) outputs(p.nchunks - 1);
    if (p.S_out != nullptr) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.S_out[((size_t)bh * DK + 16 * rt + 4 * g + i) * dv + col] = s[rt][i];
    }
  }
}

template <typename InT, int DK>
hipError_t launch_pv_t(const ScanParams& p, hipStream_t st, int phases) {
  if (phases & 1) {
    const dim3 pgrid((unsigned)((size_t)p.BH * p.nchunks));
    bool exact = false;
    if constexpr (sizeof(InT) == 2) exact = (p.flags & kFlagPhiElu1) == 0;
    if (exact) hipLaunchKernelGGL((prep_pv_kernel<InT, DK, sizeof(InT) == 2>), pgrid, dim3(NT), 0, st, p);
    else hipLaunchKernelGGL((prep_pv_kernel<InT, DK, false>), pgrid, dim3(NT), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    const dim3 grid((unsigned)((size_t)p.BH * (p.dv / 64)));
    if constexpr (sizeof(InT) == 2) {
      if ((p.flags & kFlagPhiElu1) == 0) {
        hipLaunchKernelGGL((prop_pv2_kernel<DK>), dim3((unsigned)((size_t)p.BH * (p.dv / 32))), dim3(256), 0, st, p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((prop_pv_kernel<InT, DK, false>), grid, dim3(NT), 0, st, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

size_t scan_pv_record_bytes() { return RecPV::kBytes; }

hipError_t launch_scan_pv(const ScanParams& p, hipStream_t st, int phases) {
  if (p.bf16) return p.dk == 64 ? launch_pv_t<uint16_t, 64>(p, st, phases) : launch_pv_t<uint16_t, 128>(p, st, phases);
  return p.dk == 64 ? launch_pv_t<float, 64>(p, st, phases) : launch_pv_t<float, 128>(p, st, phases);
}

}  // namespace fwmem
