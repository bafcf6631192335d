// Chunk-parallel fast-weight scan for gfx950.
//
// The recurrence (delta rule, per head, "Fast Weight Attention for Continual
// Learning" reading notes, sections 3.2 and 4.1-4.2):
//   S_t = a_t S_{t-1} + x_t u_t^T,  u_t = eta_t (y_t - S_{t-1}^T x_t),  a_t = 1 - eta_t lambda_t
// is cut into chunks of C = 64 tokens. Inside a chunk, with Gamma_t = prod_{s<=t} a_s
// (decay since the chunk start, carried as a log-sum and a sign parity) and S the
// state at chunk entry:
//   S_t = Gamma_t S + sum_{s<=t} (Gamma_t / Gamma_s) x_s u_s^T.
// Substituting this into the residual gives one unit-lower-triangular system for all
// the chunk's writes (the WY-style intra-chunk solve that section 4.4 of the notes
// describes; derived here from the recurrence):
//   (I + L) U = diag(eta) V - diag(eta Gamma_prev) X S,
//   L_ts = eta_t (Gamma_{t-1}/Gamma_s) x_t . x_s   (s < t).
// With T = (I + L)^-1 (one shared solve for every value column):
//   U   = T R,  R = diag(eta) V - diag(eta Gamma_prev) (X S)
//   O   = diag(Gamma) Q S + M U,  M_ts = (Gamma_t/Gamma_s) q_t . x_s  (s <= t)
//   S' = Gamma_C S + X^T diag(Gamma_C / Gamma) U.
// The additive rule ("attention is also an FFN", sections 2.1 and 3.2) is the same
// skeleton with U = diag(beta) V and no solve. Per-key-channel decay turns the
// Gamma ratios into d_k-vectors that are folded into the X / Q operands.
//
// Two kernels:
//   prep_kernel: one workgroup per (head, chunk), fully parallel. Builds the chunk's
//     Gram X X^T and Q X^T on MFMA, the decay masks, T = (I + L)^-1 in fp32 (blocked
//     forward substitution in LDS) and writes T, M and the token scalars to the
//     workspace.
//   prop_kernel: one workgroup per (head, group of 64 value columns); each of its
//     4 waves owns a 16-column tile of S in registers (fp32, MFMA C layout) and walks
//     the chunks in order; the only serial dependency is along T.
#include "fwmem_device.h"
#include "fwmem_internal.h"

namespace fwmem {

constexpr int CH = kChunk;
constexpr int NT = 256;
constexpr int NW = NT / kWave;

template <typename InT>
using PolOf = typename In<InT>::Pol;

// ---------------------------------------------------------------- workspace record
template <typename InT, int DK>
struct Rec {
  using op_t = typename PolOf<InT>::op_t;
  static constexpr size_t kT = 0;                                   // op_t [CH][CH]
  static constexpr size_t kM = kT + sizeof(op_t) * CH * CH;         // op_t [CH][CH]
  // per token t: (fP, fV, fO, fU), the row factors the propagate kernel applies
  static constexpr size_t kFac = kM + sizeof(op_t) * CH * CH;       // float4 [CH]
  static constexpr size_t kX0 = kFac + 16 * CH;                     // float [DK] key before token 0
  // 1/sT, 1/sM, has_prev, Gamma_C (scalar decay), sX, sQ
  static constexpr size_t kSc = kX0 + 4 * DK;                       // float [8]
  static constexpr size_t kBytes = (kSc + 32 + 255) / 256 * 256;
};

// ---------------------------------------------------------------- row staging
// Loads the chunk's x rows (shifted keys for the delta rule) and q rows, applies
// phi, and stores them scaled into LDS as MFMA operands. Also returns the row
// norms ||x_t||^2 (fp32) into s_norm when requested.
template <typename InT, int DK>
struct Rows {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  static constexpr int VW = In<InT>::VW;
  static constexpr int TPR = DK / VW;   // threads per row
  static constexpr int RPP = NT / TPR;  // rows per pass
  static constexpr int NPASS = CH / RPP;
  static_assert(CH % RPP == 0, "rows");
};

struct StageScales {
  float sX, sQ;
};

// x0: the key carried into token 0 of the sequence (fp32, phi already applied) or
// null; used by the delta rule when the chunk starts at token 0.
// XU (optional): second copy of X for the state update, transposed [DK][ldT] for
// the fp16 policy.
template <typename InT, int DK, bool DELTA, bool WRITE_XU>
__device__ StageScales stage_rows(const ScanParams& p, int bh, int t0, const float* x0,
                                  typename PolOf<InT>::op_t* Xs, typename PolOf<InT>::op_t* Qs,
                                  typename PolOf<InT>::op_t* XU, int ldX, int ldT,
                                  float* s_norm, float* s_red) {
  using R = Rows<InT, DK>;
  using Pol = typename R::Pol;
  constexpr int VW = R::VW, TPR = R::TPR, RPP = R::RPP, NPASS = R::NPASS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* qp = static_cast<const InT*>(p.q);
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const size_t rowbase = (size_t)bh * (size_t)p.T;
  const int col = (tid % TPR) * VW;

  float xr[NPASS][VW], qr[NPASS][VW];
  float mx = 0.f, mq = 0.f;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int t = ps * RPP + tid / TPR;
    const int tau = t0 + t;
#pragma unroll
    for (int j = 0; j < VW; ++j) { xr[ps][j] = 0.f; qr[ps][j] = 0.f; }
    if (tau < p.T) {
      if (DELTA) {
        if (tau >= 1) {
          In<InT>::load(kp + (rowbase + tau - 1) * DK + col, xr[ps]);
          if (elu) {
#pragma unroll
            for (int j = 0; j < VW; ++j) xr[ps][j] = phi_elu1(xr[ps][j]);
          }
        } else if (x0 != nullptr) {
#pragma unroll
          for (int j = 0; j < VW; ++j) xr[ps][j] = x0[col + j];
        }
      } else {
        In<InT>::load(kp + (rowbase + tau) * DK + col, xr[ps]);
        if (elu) {
#pragma unroll
          for (int j = 0; j < VW; ++j) xr[ps][j] = phi_elu1(xr[ps][j]);
        }
      }
      In<InT>::load(qp + (rowbase + tau) * DK + col, qr[ps]);
      if (elu) {
#pragma unroll
        for (int j = 0; j < VW; ++j) qr[ps][j] = phi_elu1(qr[ps][j]);
      }
    }
    float ns = 0.f;
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      ns += xr[ps][j] * xr[ps][j];
      mx = fmaxf(mx, fabsf(xr[ps][j]));
      mq = fmaxf(mq, fabsf(qr[ps][j]));
    }
    if (s_norm != nullptr) {
      ns = group_sum<TPR>(ns);
      if (tid % TPR == 0) s_norm[t] = ns;
    }
  }
  StageScales sc{1.f, 1.f};
  if (Pol::kScaled) {
    mx = wave_max(mx);
    mq = wave_max(mq);
    if (lane == 0) { s_red[wave] = mx; s_red[NW + wave] = mq; }
    __syncthreads();
    float a = s_red[0], b = s_red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) { a = fmaxf(a, s_red[w]); b = fmaxf(b, s_red[NW + w]); }
    sc.sX = pow2_scale(a);
    sc.sQ = pow2_scale(b);
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int t = ps * RPP + tid / TPR;
    typename Pol::frag_t xo, qo;  // VW operands = 16 bytes
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      xo[j] = Pol::cvt(xr[ps][j] * sc.sX);
      qo[j] = Pol::cvt(qr[ps][j] * sc.sQ);
    }
    *reinterpret_cast<typename Pol::frag_t*>(Xs + t * ldX + col) = xo;
    *reinterpret_cast<typename Pol::frag_t*>(Qs + t * ldX + col) = qo;
    if (WRITE_XU) {
      if constexpr (Pol::kScaled) {
#pragma unroll
        for (int j = 0; j < VW; ++j) XU[(col + j) * ldT + t] = xo[j];
      } else {
        *reinterpret_cast<typename Pol::frag_t*>(XU + t * ldX + col) = xo;
      }
    }
  }
  return sc;
}

// Block-wide max of a per-thread value (all threads must call it).
__device__ __forceinline__ float block_max(float v, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float m = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, s_red[w]);
  return m;
}

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

// ---------------------------------------------------------------- prep kernel
template <typename InT, int DK, bool DELTA, bool PC>
struct PrepLds {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  static constexpr int LDX = DK + Pol::kPad;  // op_t stride of a [CH][DK] operand
  static constexpr int LDF = CH + 4;          // float stride of a [CH][CH] matrix
  static constexpr size_t kOp = (size_t)CH * LDX * sizeof(op_t);
  static constexpr size_t kMat = (size_t)CH * LDF * 4;
  static constexpr size_t kReg = ((kOp > kMat ? kOp : kMat) + 15) / 16 * 16;
  static constexpr int kRegions = 4;
  static constexpr size_t kSmall = 4 * (5 * CH + 4 * NW + 16);
  static constexpr size_t kBytes = kRegions * kReg + kSmall;
};

template <typename InT, int DK, bool DELTA, bool PC>
__global__ __launch_bounds__(NT) void prep_kernel(ScanParams p) {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  using L = PrepLds<InT, DK, DELTA, PC>;
  using RC = Rec<InT, DK>;
  constexpr int LDX = L::LDX, LDF = L::LDF;
  __shared__ __align__(16) char smem[L::kBytes];
  char* reg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) reg[r] = smem + r * L::kReg;
  float* s_norm = reinterpret_cast<float*>(smem + L::kRegions * L::kReg);
  float* s_lam = s_norm + CH;
  float* s_eta = s_lam + CH;
  float* s_g = s_eta + CH;
  float* s_sg = s_g + CH;
  float* s_red = s_sg + CH;  // 4*NW + 16

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x % p.nchunks;
  const int bh = blockIdx.x / p.nchunks;
  const int t0 = c * CH;
  const size_t rowbase = (size_t)bh * p.T;
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  const float* x0 = (DELTA && has_in) ? p.xprev_in + (size_t)bh * DK : nullptr;

  op_t* Xs = reinterpret_cast<op_t*>(reg[0]);
  op_t* Qs = reinterpret_cast<op_t*>(reg[1]);
  const StageScales sc =
      stage_rows<InT, DK, DELTA, false>(p, bh, t0, x0, Xs, Qs, nullptr, LDX, 0, s_norm, s_red);

  // Per-channel: eta's denominator uses the channel max of lambda.
  if (DELTA && PC) {
    constexpr int TPRL = DK / 4, RPPL = NT / TPRL, NPL = CH / RPPL;
#pragma unroll
    for (int ps = 0; ps < NPL; ++ps) {
      const int t = ps * RPPL + tid / TPRL;
      const int tau = t0 + t;
      float m = 0.f;
      if (tau < p.T && p.lam != nullptr) {
        const float4 w = *reinterpret_cast<const float4*>(p.lam + (rowbase + tau) * DK + (tid % TPRL) * 4);
        m = fmaxf(fmaxf(w.x, w.y), fmaxf(w.z, w.w));
      }
      m = group_max<TPRL>(m);
      if (tid % TPRL == 0) s_lam[t] = m;
    }
  }
  __syncthreads();

  // Token scalars: eta_t, and for scalar decay the in-chunk prefix of log|a|.
  if (wave == 0) {
    const int t = lane;
    const int tau = t0 + t;
    const bool active = tau < p.T;
    float eta = 0.f, a = 1.f;
    if (DELTA) {
      const bool hasx = active && (tau >= 1 || has_in);
      float lam_t = 0.f;
      if (PC) lam_t = s_lam[t];
      else if (active && p.lam != nullptr) lam_t = p.lam[rowbase + tau];
      if (hasx) eta = p.beta[rowbase + tau] / (s_norm[t] + lam_t + p.eps);
      a = 1.f - eta * lam_t;
    } else {
      if (active) eta = p.beta != nullptr ? p.beta[rowbase + tau] : 1.f;
      if (active && p.lam != nullptr && !PC) a = p.lam[rowbase + tau];
    }
    s_eta[t] = eta;
    float la = log_abs_floor(a);
    int ng = a < 0.f ? 1 : 0;
    wave_prefix(la, ng);
    s_g[t] = la;
    s_sg[t] = (ng & 1) ? -1.f : 1.f;
  }
  __syncthreads();

  // Operand sources of the two Gram products.
  const op_t* A_L = Xs;  // rows x_t (scaled), decay applied by mask
  const op_t* A_M = Qs;
  const op_t* B_X = Xs;
  float invL = 1.f / (sc.sX * sc.sX);
  float invM = 1.f / (sc.sQ * sc.sX);
  float* Lf = reinterpret_cast<float*>(reg[2]);
  float* Mf = reinterpret_cast<float*>(reg[3]);
  float* Tf = reinterpret_cast<float*>(reg[0]);  // after the Gram, X is dead
  float* Ysc = reinterpret_cast<float*>(reg[1]); // after the Gram, Q is dead

  if (PC) {
    // Column pass, one thread per key channel: Gamma ratios per channel, anchored
    // at the chunk midpoint so the two factors of Gamma_{t-1}/Gamma_s stay in range.
    // BX and AM overwrite the raw X and Q in place (each element is read and
    // written by the same thread); AL goes to region 2.
    op_t* AL = reinterpret_cast<op_t*>(reg[2]);
    op_t* BX = Xs;
    op_t* AM = Qs;
    float gcol[CH];
    uint64_t par = 0;
    float mAL = 0.f, mBX = 0.f, mAM = 0.f;
    const int i = tid;
    if (i < DK) {
      float gs = 0.f;
      uint32_t pr = 0;
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        const int tau = t0 + t;
        float lam = DELTA ? 0.f : 1.f;
        if (tau < p.T && p.lam != nullptr) lam = p.lam[(rowbase + tau) * DK + i];
        const float a = DELTA ? 1.f - s_eta[t] * lam : lam;
        gs += log_abs_floor(a);
        pr ^= (a < 0.f) ? 1u : 0u;
        gcol[t] = gs;
        par |= (uint64_t)pr << t;
      }
    }
    constexpr int TA = CH / 2 - 1;
    // Two passes: the first finds the block maxima (for the fp16 scales), the
    // second writes the scaled operands.
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      float sAL = 1.f, sBX = 1.f, sAM = 1.f;
      if (pass == 1 && Pol::kScaled) {
        sAL = pow2_scale(block_max(mAL, s_red));
        sBX = pow2_scale(block_max(mBX, s_red + NW));
        sAM = pow2_scale(block_max(mAM, s_red + 2 * NW));
      }
      if (pass == 1) {
        invL = 1.f / (sc.sX * sAL * sc.sX * sBX);
        invM = 1.f / (sc.sQ * sAM * sc.sX * sBX);
      }
      if (i < DK) {
        const float anc = gcol[TA];
        const uint32_t apr = (uint32_t)(par >> TA) & 1u;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          const float xh = (float)Xs[t * LDX + i];
          const float qh = (float)Qs[t * LDX + i];
          const float gprev = t ? gcol[t - 1] : 0.f;
          const uint32_t pprev = t ? (uint32_t)(par >> (t - 1)) & 1u : 0u;
          const uint32_t pcur = (uint32_t)(par >> t) & 1u;
          const float fAL = ((pprev ^ apr) ? -1.f : 1.f) * __expf(gprev - anc);
          const float fBX = ((pcur ^ apr) ? -1.f : 1.f) * __expf(anc - gcol[t]);
          const float fAM = ((pcur ^ apr) ? -1.f : 1.f) * __expf(gcol[t] - anc);
          const float vAL = xh * fAL, vBX = xh * fBX, vAM = qh * fAM;
          if (pass == 0) {
            mAL = fmaxf(mAL, fabsf(vAL));
            mBX = fmaxf(mBX, fabsf(vBX));
            mAM = fmaxf(mAM, fabsf(vAM));
          } else {
            if (DELTA) AL[t * LDX + i] = Pol::cvt(vAL * sAL);
            BX[t * LDX + i] = Pol::cvt(vBX * sBX);
            AM[t * LDX + i] = Pol::cvt(vAM * sAM);
          }
        }
      }
    }
    __syncthreads();
    A_L = AL;
    A_M = AM;
    B_X = BX;
    Lf = reinterpret_cast<float*>(reg[3]);
    Mf = reinterpret_cast<float*>(reg[0]);
    Tf = reinterpret_cast<float*>(reg[2]);
    Ysc = reinterpret_cast<float*>(reg[1]);
  }

  // Gram products on MFMA: 16 tiles of each 64x64 product (upper tiles are zero).
  // All of a wave's tiles are accumulated first; the masked results are written
  // after a barrier, so the destinations may reuse the operand regions.
  {
    constexpr int JPW = 32 / NW;  // jobs per wave
    const int g = lane >> 4, n = lane & 15;
    f4 acc[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + NW * jj;
      const int mat = job >> 4;  // 0: L from X X^T, 1: M from Q X^T
      const int mt = (job >> 2) & 3, nt = job & 3;
      acc[jj] = f4{0.f, 0.f, 0.f, 0.f};
      if (mt >= nt && (mat == 1 || DELTA)) {
        const op_t* arow = (mat == 0 ? A_L : A_M) + (16 * mt + n) * LDX;
        const op_t* brow = B_X + (16 * nt + n) * LDX;
#pragma unroll
        for (int kb = 0; kb < DK / Pol::KB; ++kb)
          Pol::mma(acc[jj], Pol::lds_row(arow, kb, g), Pol::lds_row(brow, kb, g));
      }
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + NW * jj;
      const int mat = job >> 4;
      const int mt = (job >> 2) & 3, nt = job & 3;
      if (mat == 0 && !DELTA) continue;
      float* dst = mat == 0 ? Lf : Mf;
      const int s = 16 * nt + n;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = 16 * mt + 4 * g + ii;
        float val = 0.f;
        if (mat == 0) {
          if (s < t) {
            float f = s_eta[t] * invL;
            if (!PC) {
              const float gp = t ? s_g[t - 1] : 0.f;
              const float sp = t ? s_sg[t - 1] : 1.f;
              f *= sp * s_sg[s] * __expf(gp - s_g[s]);
            }
            val = f * acc[jj][ii];
          }
        } else {
          if (s <= t) {
            float f = invM;
            if (!PC) f *= s_sg[t] * s_sg[s] * __expf(s_g[t] - s_g[s]);
            val = f * acc[jj][ii];
          }
        }
        dst[t * LDF + s] = val;
      }
    }
  }
  __syncthreads();

  // T = (I + L)^-1 by blocked forward substitution (16x16 blocks, fp32).
  if (DELTA) {
    constexpr int NB = CH / 16;
    if (wave == 0) {
      const int b = lane >> 4, j = lane & 15;
      float tc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == j) ? 1.f : 0.f;
        const float* lrow = Lf + (16 * b + r) * LDF + 16 * b;
#pragma unroll
        for (int kk = 0; kk < r; ++kk) v -= lrow[kk] * tc[kk];
        tc[r] = v;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tf[(16 * b + r) * LDF + 16 * b + j] = tc[r];
    } else {
      // zero the blocks above the diagonal
      for (int e = tid - kWave; e < NB * NB * 256; e += NT - kWave) {
        const int blk = e >> 8, bi = blk / NB, bj = blk % NB;
        if (bi < bj) {
          const int r = (e >> 4) & 15, cc = e & 15;
          Tf[(16 * bi + r) * LDF + 16 * bj + cc] = 0.f;
        }
      }
    }
    __syncthreads();
    const int r = tid >> 4, cc = tid & 15;
#pragma unroll
    for (int bi = 1; bi < NB; ++bi) {
      // Y_bj = sum_{bk=bj}^{bi-1} L_{bi,bk} T_{bk,bj}
      for (int bj = 0; bj < bi; ++bj) {
        float y = 0.f;
        for (int bk = bj; bk < bi; ++bk) {
          const float* lrow = Lf + (16 * bi + r) * LDF + 16 * bk;
#pragma unroll
          for (int m = 0; m < 16; ++m) y += lrow[m] * Tf[(16 * bk + m) * LDF + 16 * bj + cc];
        }
        Ysc[bj * 256 + r * 16 + cc] = y;
      }
      __syncthreads();
      // T_{bi,bj} = -T_{bi,bi} Y_bj
      for (int bj = 0; bj < bi; ++bj) {
        float y = 0.f;
        const float* trow = Tf + (16 * bi + r) * LDF + 16 * bi;
#pragma unroll
        for (int m = 0; m < 16; ++m) y += trow[m] * Ysc[bj * 256 + m * 16 + cc];
        Tf[(16 * bi + r) * LDF + 16 * bj + cc] = -y;
      }
      __syncthreads();
    }
  }

  // Write T (delta) and M, scaled, plus the token scalars, to the record.
  char* rec = p.ws + ((size_t)bh * p.nchunks + c) * RC::kBytes;
  {
    const int t = tid >> 2, c0 = (tid & 3) * 16;
    float tv[16], mv[16];
    float mt_ = 0.f, mm_ = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      tv[j] = DELTA ? Tf[t * LDF + c0 + j] : 0.f;
      mv[j] = Mf[t * LDF + c0 + j];
      mt_ = fmaxf(mt_, fabsf(tv[j]));
      mm_ = fmaxf(mm_, fabsf(mv[j]));
    }
    float sT = 1.f, sM = 1.f;
    if (Pol::kScaled) {
      sT = pow2_scale(block_max(mt_, s_red));
      sM = pow2_scale(block_max(mm_, s_red + NW));
    }
    using frag_t = typename Pol::frag_t;
    constexpr int EV = 16 / sizeof(op_t);  // elements per 16-byte vector
    frag_t* Tg = reinterpret_cast<frag_t*>(reinterpret_cast<op_t*>(rec + RC::kT) + t * CH + c0);
    frag_t* Mg = reinterpret_cast<frag_t*>(reinterpret_cast<op_t*>(rec + RC::kM) + t * CH + c0);
#pragma unroll
    for (int j = 0; j < 16 / EV; ++j) {
      frag_t tw, mw;
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        tw[e] = Pol::cvt(tv[j * EV + e] * sT);
        mw[e] = Pol::cvt(mv[j * EV + e] * sM);
      }
      if (DELTA) Tg[j] = tw;
      Mg[j] = mw;
    }
    if (tid < CH) {
      // Row factors of the propagate step (see the header comment): with X, Q stored
      // scaled by sX, sQ,
      //   R = fV V - fP (X S),  O = fO (Q S) + M U,  S' = Gamma_C S + X^T (fU U).
      // Per-channel decay is folded into the operands instead, so only eta and the
      // scales remain.
      const int t = tid;
      const float e = s_eta[t];
      f4 fac;
      if (PC) {
        fac = f4{e / sc.sX, e, 1.f / sc.sQ, 1.f / sc.sX};
      } else {
        const float gprev = t ? s_g[t - 1] : 0.f;
        const float sprev = t ? s_sg[t - 1] : 1.f;
        const float gammaPrev = sprev * __expf(gprev);
        const float gammaT = s_sg[t] * __expf(s_g[t]);
        const float ratioC = s_sg[CH - 1] * s_sg[t] * __expf(s_g[CH - 1] - s_g[t]);
        fac = f4{e * gammaPrev / sc.sX, e, gammaT / sc.sQ, ratioC / sc.sX};
      }
      reinterpret_cast<f4*>(rec + RC::kFac)[t] = fac;
    }
    if (tid == 0) {
      float* scv = reinterpret_cast<float*>(rec + RC::kSc);
      scv[0] = 1.f / sT;
      scv[1] = 1.f / sM;
      scv[2] = has_in ? 1.f : 0.f;
      scv[3] = PC ? 1.f : s_sg[CH - 1] * __expf(s_g[CH - 1]);
      scv[4] = sc.sX;
      scv[5] = sc.sQ;
      scv[6] = 0.f;
      scv[7] = 0.f;
    }
    if (c == 0 && tid < DK) {
      reinterpret_cast<float*>(rec + RC::kX0)[tid] = x0 != nullptr ? x0[tid] : 0.f;
    }
  }
}

// ---------------------------------------------------------------- propagate kernel
template <typename InT, int DK, bool PC>
struct PropLds {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  static constexpr int LDX = DK + Pol::kPad;  // [CH][DK] operands
  static constexpr int LDT = CH + Pol::kPad;  // [DK][CH] transposed operand (fp16 policy)
  static constexpr int LDC = CH + Pol::kPad;  // [CH][CH] operands
  static constexpr int LDV = 64 + 4;          // [CH][64] fp32 value tile
  static constexpr size_t kX = (size_t)CH * LDX * sizeof(op_t);
  static constexpr size_t kXU = Pol::kScaled ? (size_t)DK * LDT * sizeof(op_t) : kX;
  static constexpr size_t kC = (size_t)CH * LDC * sizeof(op_t);
  static constexpr size_t kV = (size_t)CH * LDV * 4;
  static constexpr size_t oX = 0;
  static constexpr size_t oXU = oX + kX;
  static constexpr size_t oQ = oXU + kXU;
  static constexpr size_t oT = oQ + kX;
  static constexpr size_t oM = oT + kC;
  static constexpr size_t oV = oM + kC;
  static constexpr size_t oS = oV + kV;  // small: 5*CH + DK + 4*NW + 16 floats
  static constexpr size_t kBytes = oS + 4 * (5 * CH + DK + 4 * NW + 16);
};

template <typename InT, int DK, bool DELTA, bool PC>
__global__ __launch_bounds__(NT) void prop_kernel(ScanParams p) {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  using frag_t = typename Pol::frag_t;
  using L = PropLds<InT, DK, PC>;
  using RC = Rec<InT, DK>;
  constexpr int LDX = L::LDX, LDT = L::LDT, LDC = L::LDC, LDV = L::LDV;
  constexpr int KB = Pol::KB;
  constexpr int NKD = DK / KB;  // K blocks over d_k
  constexpr int NKC = CH / KB;  // K blocks over the chunk
  constexpr int NMT = CH / 16;  // row tiles of a chunk
  constexpr int NRT = DK / 16;  // row tiles of S

  __shared__ __align__(16) char smem[L::kBytes];
  op_t* Xs = reinterpret_cast<op_t*>(smem + L::oX);
  op_t* XU = reinterpret_cast<op_t*>(smem + L::oXU);
  op_t* Qs = reinterpret_cast<op_t*>(smem + L::oQ);
  op_t* Ts = reinterpret_cast<op_t*>(smem + L::oT);
  op_t* Ms = reinterpret_cast<op_t*>(smem + L::oM);
  float* Vs = reinterpret_cast<float*>(smem + L::oV);
  float* s_fP = reinterpret_cast<float*>(smem + L::oS);
  float* s_fV = s_fP + CH;
  float* s_fO = s_fV + CH;
  float* s_fU = s_fO + CH;
  float* s_misc = s_fU + CH;   // [0] Gamma_C (scalar decay), [1] 1/sT, [2] 1/sM
  float* s_gC = s_misc + CH;   // [DK] per-channel Gamma_C
  float* s_red = s_gC + DK;

  // Workgroup -> (head, column group); the groups of one head share an XCD (and
  // its L2), since consecutive workgroups are dealt round-robin over the 8 XCDs.
  const int NG = (p.dv + 63) / 64;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int grp = slot % NG;
  const int bh = (slot / NG) * 8 + xcd;
  if (bh >= p.BH) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int c0 = grp * 64 + wave * 16;  // this wave's first value column
  const bool wave_on = c0 < p.dv;
  const int dv = p.dv;
  const size_t rowbase = (size_t)bh * p.T;
  const bool out_bf16 = (p.flags & kFlagOutBf16) != 0;

  f4 s[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float v = 0.f;
      if (wave_on && p.S_in != nullptr)
        v = p.S_in[((size_t)bh * DK + 16 * rt + 4 * g + ii) * dv + c0 + n];
      s[rt][ii] = v;
    }
  }

  const char* rec0 = p.ws + (size_t)bh * p.nchunks * RC::kBytes;
  const bool has_in = reinterpret_cast<const float*>(rec0 + RC::kSc)[2] != 0.f;
  const float* x0 = (DELTA && has_in) ? reinterpret_cast<const float*>(rec0 + RC::kX0) : nullptr;

  // ---- software pipeline: the next chunk's global data is loaded into registers
  // while the current chunk computes; staging then only writes LDS.
  using Rw = Rows<InT, DK>;
  constexpr int VW = Rw::VW, TPR = Rw::TPR, RPP = Rw::RPP, NPASS = Rw::NPASS;
  constexpr int TPRv = 64 / VW, RPPv = NT / TPRv, NPV = CH / RPPv;  // value tile
  constexpr int EPT = CH * CH / NT, NVT = EPT * (int)sizeof(op_t) / 16;  // T and M
  const InT* kp = static_cast<const InT*>(p.k);
  const InT* qp = static_cast<const InT*>(p.q);
  const InT* vp = static_cast<const InT*>(p.v);
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const int col = (tid % TPR) * VW;           // row staging: this thread's columns
  const int vcol = (tid % TPRv) * VW;         // value tile: this thread's columns
  const int e0 = tid * EPT;                   // T / M: this thread's elements
  u32x4 px[NPASS], pq[NPASS], pv[NPV], pt[NVT], pm[NVT];
  f4 pf = {0.f, 0.f, 0.f, 0.f};
  uint32_t valid = 0;

  // Iteration c stages chunk c from registers, then issues the loads of chunk c+1
  // and computes chunk c while they are in flight (c = -1 only loads chunk 0).
  for (int c = -1; c < p.nchunks; ++c) {
    const int t0 = c * CH;
    if (c >= 0) {
      // ---- registers -> LDS (chunk c)
        const float* scv = reinterpret_cast<const float*>(rec0 + (size_t)c * RC::kBytes + RC::kSc);
        const float sX = scv[4], sQ = scv[5];
    #pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const int t = ps * RPP + tid / TPR;
          float x[VW], qv[VW];
          In<InT>::decode(px[ps], x);
          In<InT>::decode(pq[ps], qv);
          if (DELTA && t0 + t == 0) {
    #pragma unroll
            for (int j = 0; j < VW; ++j) x[j] = x0 != nullptr ? x0[col + j] : 0.f;
          } else if (elu && (valid >> ps & 1u)) {
    #pragma unroll
            for (int j = 0; j < VW; ++j) x[j] = phi_elu1(x[j]);
          }
          if (elu && (valid >> (16 + ps) & 1u)) {
    #pragma unroll
            for (int j = 0; j < VW; ++j) qv[j] = phi_elu1(qv[j]);
          }
          frag_t xo, qo;  // VW operands = 16 bytes
    #pragma unroll
          for (int j = 0; j < VW; ++j) {
            xo[j] = Pol::cvt(x[j] * sX);
            qo[j] = Pol::cvt(qv[j] * sQ);
          }
          *reinterpret_cast<frag_t*>(Xs + t * LDX + col) = xo;
          *reinterpret_cast<frag_t*>(Qs + t * LDX + col) = qo;
          if (!PC) {
            if constexpr (Pol::kScaled) {
    #pragma unroll
              for (int j = 0; j < VW; ++j) XU[(col + j) * LDT + t] = xo[j];
            } else {
              *reinterpret_cast<frag_t*>(XU + t * LDX + col) = xo;
            }
          }
        }
    #pragma unroll
        for (int ps = 0; ps < NPV; ++ps) {
          const int t = ps * RPPv + tid / TPRv;
          float x[VW];
          In<InT>::decode(pv[ps], x);
    #pragma unroll
          for (int j = 0; j < VW; ++j) Vs[t * LDV + vcol + j] = x[j];
        }
        const int rr = e0 / CH, cc2 = e0 % CH;
    #pragma unroll
        for (int j = 0; j < NVT; ++j) {
          if (DELTA) reinterpret_cast<u32x4*>(Ts + rr * LDC + cc2)[j] = pt[j];
          reinterpret_cast<u32x4*>(Ms + rr * LDC + cc2)[j] = pm[j];
        }
        if (tid < CH) {
          s_fP[tid] = pf[0];
          s_fV[tid] = pf[1];
          s_fO[tid] = pf[2];
          s_fU[tid] = pf[3];
        }
        if (tid == 0) {
          s_misc[0] = scv[3];
          s_misc[1] = scv[0];
          s_misc[2] = scv[1];
        }
      __syncthreads();
    }
    if (c + 1 < p.nchunks) {
      // ---- global -> registers (chunk c+1)
      const int cn = c + 1;
        const int t0 = cn * CH;
        const char* rec = rec0 + (size_t)cn * RC::kBytes;
        valid = 0;
    #pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const int tau = t0 + ps * RPP + tid / TPR;
          px[ps] = u32x4{0u, 0u, 0u, 0u};
          pq[ps] = u32x4{0u, 0u, 0u, 0u};
          if (tau < p.T) {
            const int src = DELTA ? tau - 1 : tau;
            if (src >= 0) {
              px[ps] = *reinterpret_cast<const u32x4*>(kp + (rowbase + src) * DK + col);
              valid |= 1u << ps;
            }
            pq[ps] = *reinterpret_cast<const u32x4*>(qp + (rowbase + tau) * DK + col);
            valid |= 1u << (16 + ps);
          }
        }
    #pragma unroll
        for (int ps = 0; ps < NPV; ++ps) {
          const int tau = t0 + ps * RPPv + tid / TPRv;
          pv[ps] = u32x4{0u, 0u, 0u, 0u};
          if (tau < p.T && grp * 64 + vcol < dv)
            pv[ps] = *reinterpret_cast<const u32x4*>(vp + (rowbase + tau) * dv + grp * 64 + vcol);
        }
        const u32x4* Tg = reinterpret_cast<const u32x4*>(reinterpret_cast<const op_t*>(rec + RC::kT) + e0);
        const u32x4* Mg = reinterpret_cast<const u32x4*>(reinterpret_cast<const op_t*>(rec + RC::kM) + e0);
    #pragma unroll
        for (int j = 0; j < NVT; ++j) {
          if (DELTA) pt[j] = Tg[j];
          pm[j] = Mg[j];
        }
        if (tid < CH) pf = reinterpret_cast<const f4*>(rec + RC::kFac)[tid];
    }
    if (c < 0) continue;

    if (PC) {
      // per-channel decay folded into the operands: X*Gamma_prev, Q*Gamma, X*Gamma_C/Gamma
      const int i = tid;
      if (i < DK) {
        float gcol[CH];
        uint64_t par = 0;
        float gsum = 0.f;
        uint32_t pr = 0;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          const int tau = t0 + t;
          float lam = DELTA ? 0.f : 1.f;
          if (tau < p.T && p.lam != nullptr) lam = p.lam[(rowbase + tau) * DK + i];
          const float a = DELTA ? 1.f - s_fV[t] * lam : lam;
          gsum += log_abs_floor(a);
          pr ^= (a < 0.f) ? 1u : 0u;
          gcol[t] = gsum;
          par |= (uint64_t)pr << t;
        }
        const float gC = gcol[CH - 1];
        const uint32_t pC = (uint32_t)(par >> (CH - 1)) & 1u;
        s_gC[i] = (pC ? -1.f : 1.f) * __expf(gC);
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          const uint32_t pcur = (uint32_t)(par >> t) & 1u;
          const uint32_t pprev = t ? (uint32_t)(par >> (t - 1)) & 1u : 0u;
          const float fprev = (pprev ? -1.f : 1.f) * __expf(t ? gcol[t - 1] : 0.f);
          const float fcur = (pcur ? -1.f : 1.f) * __expf(gcol[t]);
          const float fend = ((pC ^ pcur) ? -1.f : 1.f) * __expf(gC - gcol[t]);
          const float xh = (float)Xs[t * LDX + i];
          if constexpr (Pol::kScaled) XU[i * LDT + t] = Pol::cvt(xh * fend);
          else XU[t * LDX + i] = Pol::cvt(xh * fend);
          Xs[t * LDX + i] = Pol::cvt(xh * fprev);
          Qs[t * LDX + i] = Pol::cvt((float)Qs[t * LDX + i] * fcur);
        }
      }
      __syncthreads();
    }

    if (wave_on) {
      const float invT = s_misc[1], invM = s_misc[2];
      // S as the B operand of X S and Q S
      float ms = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) ms = fmaxf(ms, fabsf(s[rt][ii]));
      const float sS = Pol::kScaled ? pow2_scale(wave_max(ms)) : 1.f;
      const float isS = 1.f / sS;
      frag_t Sf[NKD];
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) Sf[kb] = Pol::from_c(s, kb, sS);

      f4 U[NMT];
      if (DELTA) {
        f4 P[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          P[mt] = f4{0.f, 0.f, 0.f, 0.f};
          const op_t* arow = Xs + (16 * mt + n) * LDX;
#pragma unroll
          for (int kb = 0; kb < NKD; ++kb) Pol::mma(P[mt], Pol::lds_row(arow, kb, g), Sf[kb]);
        }
        float mr = 0.f;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * mt + 4 * g + ii;
            const float r = s_fV[t] * Vs[t * LDV + wave * 16 + n] - s_fP[t] * isS * P[mt][ii];
            P[mt][ii] = r;
            mr = fmaxf(mr, fabsf(r));
          }
        const float sR = Pol::kScaled ? pow2_scale(wave_max(mr)) : 1.f;
        frag_t Rf[NKC];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) Rf[kb] = Pol::from_c(P, kb, sR);
        const float fu = invT / sR;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          f4 acc = {0.f, 0.f, 0.f, 0.f};
          const op_t* arow = Ts + (16 * mt + n) * LDC;
#pragma unroll
          for (int kb = 0; kb < (16 * mt + 16 + KB - 1) / KB; ++kb)
            Pol::mma(acc, Pol::lds_row(arow, kb, g), Rf[kb]);
          U[mt] = acc * fu;
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * mt + 4 * g + ii;
            U[mt][ii] = s_fV[t] * Vs[t * LDV + wave * 16 + n];
          }
      }

      // O = diag(Gamma) Q S + M U
      f4 O[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        O[mt] = f4{0.f, 0.f, 0.f, 0.f};
        const op_t* arow = Qs + (16 * mt + n) * LDX;
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) Pol::mma(O[mt], Pol::lds_row(arow, kb, g), Sf[kb]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) O[mt][ii] *= s_fO[16 * mt + 4 * g + ii] * isS;
      }
      float mu = 0.f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) mu = fmaxf(mu, fabsf(U[mt][ii]));
      const float sU = Pol::kScaled ? pow2_scale(wave_max(mu)) : 1.f;
      {
        frag_t Uf[NKC];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) Uf[kb] = Pol::from_c(U, kb, sU);
        const float fm = invM / sU;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          f4 acc = {0.f, 0.f, 0.f, 0.f};
          const op_t* arow = Ms + (16 * mt + n) * LDC;
#pragma unroll
          for (int kb = 0; kb < (16 * mt + 16 + KB - 1) / KB; ++kb)
            Pol::mma(acc, Pol::lds_row(arow, kb, g), Uf[kb]);
          O[mt] += acc * fm;
        }
      }
      // store the chunk's outputs
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int tau = t0 + 16 * mt + 4 * g + ii;
          if (tau < p.T) {
            const size_t o = (rowbase + tau) * dv + c0 + n;
            if (out_bf16) static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_bits(O[mt][ii]);
            else static_cast<float*>(p.out)[o] = O[mt][ii];
          }
        }

      // S' = Gamma_C S + X^T (diag(Gamma_C/Gamma) U)
      float mut = 0.f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          U[mt][ii] *= s_fU[16 * mt + 4 * g + ii];
          mut = fmaxf(mut, fabsf(U[mt][ii]));
        }
      const float sUt = Pol::kScaled ? pow2_scale(wave_max(mut)) : 1.f;
      const float iUt = 1.f / sUt;
      frag_t Utf[NKC];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) Utf[kb] = Pol::from_c(U, kb, sUt);
      const float gCs = s_misc[0];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) {
          frag_t a;
          if constexpr (Pol::kScaled) a = Pol::lds_row(XU + (16 * rt + n) * LDT, kb, g);
          else a = PolF32::lds_col(XU, LDX, 16 * rt + n, kb, g);
          Pol::mma(acc, a, Utf[kb]);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float gc = PC ? s_gC[16 * rt + 4 * g + ii] : gCs;
          s[rt][ii] = gc * s[rt][ii] + acc[ii] * iUt;
        }
      }
    }
    __syncthreads();
  }

  // final state
  if (p.S_out != nullptr) {
    if (wave_on) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          p.S_out[((size_t)bh * DK + 16 * rt + 4 * g + ii) * dv + c0 + n] = s[rt][ii];
    }
    if (grp == 0) {
      const InT* kp = static_cast<const InT*>(p.k);
      const bool elu = (p.flags & kFlagPhiElu1) != 0;
      for (int i = tid; i < DK; i += NT) {
        float x = In<InT>::load1(kp + (rowbase + p.T - 1) * DK + i);
        if (elu) x = phi_elu1(x);
        p.xprev_out[(size_t)bh * DK + i] = x;
      }
      if (tid == 0) p.has_out[bh] = 1;
    }
  }
}

// ---------------------------------------------------------------- T == 0: state copy
__global__ void state_copy_kernel(const float* S_in, const float* x_in, const int32_t* h_in,
                                  float* S_out, float* x_out, int32_t* h_out, size_t nS, size_t nX,
                                  size_t nH) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nS + nX + nH; i += stride) {
    if (i < nS) S_out[i] = S_in ? S_in[i] : 0.f;
    else if (i < nS + nX) x_out[i - nS] = x_in ? x_in[i - nS] : 0.f;
    else h_out[i - nS - nX] = h_in ? h_in[i - nS - nX] : 0;
  }
}

// ---------------------------------------------------------------- host launchers
size_t scan_record_bytes(int bf16, int dk) {
  if (bf16) return dk == 64 ? Rec<uint16_t, 64>::kBytes : Rec<uint16_t, 128>::kBytes;
  return dk == 64 ? Rec<float, 64>::kBytes : Rec<float, 128>::kBytes;
}

bool scan_supported(int dk, int dv) {
  return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

template <typename InT, int DK, bool DELTA, bool PC>
static hipError_t launch_scan_t(const ScanParams& p, hipStream_t st, int phases) {
  if (phases & 1) {
    const unsigned nprep = (unsigned)((size_t)p.BH * p.nchunks);
    hipLaunchKernelGGL((prep_kernel<InT, DK, DELTA, PC>), dim3(nprep), dim3(NT), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    const int NG = (p.dv + 63) / 64;
    const unsigned nprop = (unsigned)(8 * NG * ((p.BH + 7) / 8));
    hipLaunchKernelGGL((prop_kernel<InT, DK, DELTA, PC>), dim3(nprop), dim3(NT), 0, st, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename InT, int DK>
static hipError_t launch_scan_dk(const ScanParams& p, hipStream_t st, int ph) {
  const bool pc = (p.flags & kFlagPerChannel) != 0;
  if (p.delta)
    return pc ? launch_scan_t<InT, DK, true, true>(p, st, ph) : launch_scan_t<InT, DK, true, false>(p, st, ph);
  return pc ? launch_scan_t<InT, DK, false, true>(p, st, ph) : launch_scan_t<InT, DK, false, false>(p, st, ph);
}

hipError_t launch_scan(const ScanParams& p, hipStream_t st, int phases) {
  if (p.bf16)
    return p.dk == 64 ? launch_scan_dk<uint16_t, 64>(p, st, phases) : launch_scan_dk<uint16_t, 128>(p, st, phases);
  return p.dk == 64 ? launch_scan_dk<float, 64>(p, st, phases) : launch_scan_dk<float, 128>(p, st, phases);
}

hipError_t launch_state_copy(const float* S_in, const float* xprev_in, const int32_t* has_in,
                             float* S_out, float* xprev_out, int32_t* has_out, size_t nS, size_t nX,
                             size_t nH, hipStream_t st) {
  const size_t n = nS + nX + nH;
  unsigned blocks = (unsigned)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, st, S_in, xprev_in, has_in,
                     S_out, xprev_out, has_out, nS, nX, nH);
  return hipGetLastError();
}

}  // namespace fwmem
