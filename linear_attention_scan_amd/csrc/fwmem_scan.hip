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
// skeleton with U = diag(beta) V and no solve. The inner-product rule (section 4.3 of
// the notes) keeps the delta rule's shifted keys, eta_t and decay, and writes
// U = diag(eta) V with no solve. Per-key-channel decay turns the Gamma ratios into
// d_k-vectors that are folded into the X / Q operands.
//
// Two kernels:
//   prep_kernel: one workgroup per (head, chunk), fully parallel. Builds the chunk's
//     Gram X X^T and Q X^T on MFMA, the decay masks, T = (I + L)^-1 in fp32 (blocked
//     forward substitution in LDS) and writes T, M, the per-token row factors and
//     the operand scales to the workspace.
//   prop_kernel: one workgroup per (head, group of 64 value columns); each of its
//     4 waves owns a 16-column tile of S in registers (fp32, MFMA C layout) and walks
//     the chunks in order; the only serial dependency is along T. The next chunk's
//     global data is loaded into registers while the current chunk computes.
#include "fwmem_device.h"
#include "fwmem_internal.h"
#include "fwmem_split.h"  // record size of the split path

namespace fwmem {

constexpr int CH = kChunk;
constexpr int NT = 256;
constexpr int NW = NT / kWave;

template <typename InT>
using PolOf = typename In<InT>::Pol;

// ---------------------------------------------------------------- workspace record
template <typename InT, int DK, bool PC = false>
struct Rec {
  using op_t = typename PolOf<InT>::op_t;
  // T and M rows in the policy's LDS operand order (copied verbatim into LDS)
  static constexpr size_t kT = 0;                                   // op_t [CH][CH]
  static constexpr size_t kM = kT + sizeof(op_t) * CH * CH;         // op_t [CH][CH]
  // per token t: fP, fV, fO, fU (four arrays of CH), the row factors of the step
  //   R = fV V - fP (X S),  O = fO (Q S) + M U,  S' = Gamma_C S + X^T (fU U)
  static constexpr size_t kFac = kM + sizeof(op_t) * CH * CH;       // float [4][CH]
  static constexpr size_t kX0 = kFac + 16 * CH;                     // float [DK] key before token 0
  // 1/sT, 1/sM, has_prev, Gamma_C (scalar decay), sX, sQ
  static constexpr size_t kSc = kX0 + 4 * DK;                       // float [8]
  static constexpr size_t kBase = (kSc + 32 + 255) / 256 * 256;
  // Per-channel decay with fp16 operands (bf16 inputs): the chunk's operands with the
  // decay folded in, formed once by prep (fp16 [CH][DK], natural channel order, scaled by
  // sX or sQ like the rows they come from), then the per-channel Gamma_C:
  //   X~ = X o Gamma_prev (rows of X S),  X^ = X o Gamma_C / Gamma (the update's X^T),
  //   Q~ = Q o Gamma (the read).
  static constexpr bool kOps = PC && PolOf<InT>::kScaled;
  static constexpr size_t kPX = kBase;
  static constexpr size_t kPU = kPX + 2 * CH * DK;
  static constexpr size_t kPQ = kPU + 2 * CH * DK;
  static constexpr size_t kPG = kPQ + 2 * CH * DK;  // float [DK]
  static constexpr size_t kBytes = kOps ? (kPG + 4 * DK + 255) / 256 * 256 : kBase;
};

// Thread layout of a [CH][DK] row staging: 16-byte loads of VW elements.
template <typename InT, int DK>
struct Rows {
  static constexpr int VW = In<InT>::VW;
  static constexpr int TPR = DK / VW;   // threads per row
  static constexpr int RPP = NT / TPR;  // rows per pass
  static constexpr int NPASS = CH / RPP;
  static_assert(CH % RPP == 0, "rows");
};

// 16-byte load at a uniform base plus a 32-bit byte offset (lets the compiler use
// the scalar-base + vector-offset addressing form).
template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Workgroup barrier for LDS: waits for this wave's LDS operations only. Every barrier of
// these kernels orders LDS traffic alone (no wave reads global memory that another wave
// of the workgroup writes), and a plain __syncthreads would also wait until the wave's
// outstanding global loads have returned and its stores (record rows, outputs) have
// been acknowledged.
static __device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Block-wide max of a per-thread value (all threads must call it).
__device__ __forceinline__ float block_max(float v, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  lds_barrier();
  if (lane == 0) s_red[wave] = v;
  lds_barrier();
  float m = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, s_red[w]);
  return m;
}

// Column block J of T = (I + L)^-1 (64 x 64, fp32, row stride LD) below the diagonal, given
// its diagonal blocks D_b = T_bb in Tf: T_iJ = -D_i sum_{k=J}^{i-1} L_ik T_kJ for i = J+1..3, on
// v_mfma_f32_16x16x4f32 (lane (g, n) supplies A[n][4g..4g+3] and B[4g..4g+3][n]; a C-layout
// tile is a B operand as it stands).
template <int J, int LD>
__device__ __forceinline__ void t_column_block(const float* Lf, float* Tf, int lane) {
  const int g = lane >> 4, n = lane & 15;
  f4 Tc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) Tc[J][q] = Tf[(16 * J + 4 * g + q) * LD + 16 * J + n];
#pragma unroll
  for (int i = J + 1; i < 4; ++i) {
    f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = J; k < i; ++k) {
      const f4 a = *reinterpret_cast<const f4*>(Lf + (16 * i + n) * LD + 16 * k + 4 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], Tc[k][q], y, 0, 0, 0);
    }
    const f4 d = *reinterpret_cast<const f4*>(Tf + (16 * i + n) * LD + 16 * i + 4 * g);
    f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) t = __builtin_amdgcn_mfma_f32_16x16x4f32(d[q], y[q], t, 0, 0, 0);
    Tc[i] = -t;
#pragma unroll
    for (int q = 0; q < 4; ++q) Tf[(16 * i + 4 * g + q) * LD + 16 * J + n] = -t[q];
  }
}

// ================================================================ prep kernel
// NREG operand/matrix regions: four for the delta rule; three for the rules without a
// solve (X, Q and M; the L and T region is never written), so that three workgroups share
// a CU.
template <typename InT, int DK, int NREG>
struct PrepLds {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  static constexpr int LDX = DK + Pol::kPad;  // op_t stride of a [CH][DK] operand
  static constexpr int LDF = CH + 4;          // float stride of a [CH][CH] matrix
  static constexpr size_t kOp = (size_t)CH * LDX * sizeof(op_t);
  static constexpr size_t kMat = (size_t)CH * LDF * 4;
  static constexpr size_t kReg = ((kOp > kMat ? kOp : kMat) + 15) / 16 * 16;
  static constexpr size_t kSmall = 4 * (8 * CH + 4 * NW + 16);
  static constexpr size_t kBytes = NREG * kReg + kSmall;
};

template <typename InT, int DK, int RULE, bool PC, bool ELU>
__global__ __launch_bounds__(NT) void prep_kernel(ScanParams p) {
  using R = Rule<RULE>;
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  using frag_t = typename Pol::frag_t;
  constexpr int NREG = R::solve ? 4 : 3;
  using L = PrepLds<InT, DK, NREG>;
  using RC = Rec<InT, DK, PC>;
  using Rw = Rows<InT, DK>;
  constexpr int LDX = L::LDX, LDF = L::LDF;
  constexpr int VW = Rw::VW, TPR = Rw::TPR, RPP = Rw::RPP, NPASS = Rw::NPASS;
  __shared__ __align__(16) char smem[L::kBytes];
  // Without a solve, region 3 aliases region 2: only one of them is ever written (the
  // read mask M, or the column pass's scratch before M exists).
  char* reg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) reg[r] = smem + (r < NREG ? r : NREG - 1) * L::kReg;
  float* s_norm = reinterpret_cast<float*>(smem + NREG * L::kReg);
  float* s_lam = s_norm + CH;
  float* s_eta = s_lam + CH;
  float* s_g = s_eta + CH;
  float* s_sg = s_g + CH;
  float* s_red = s_sg + CH;  // 4*NW + 16
  float* s_qn = s_red + 4 * NW + 16;  // |q_t|^2 (normalised queries and keys only)
  float* s_nx = s_qn + CH;            // rescale factors of x_t and q_t (1 without)
  float* s_mq = s_nx + CH;
  // With normalised queries and keys the raw rows stay the operands: x_t and q_t are used
  // as nx_t x_t and mq_t q_t, folded into eta, the masks and the row factors.
  const float qk_len = qk_length(p.flags, DK);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x % p.nchunks;
  const int bh = blockIdx.x / p.nchunks;
  const int t0 = c * CH;
  const size_t rowbase = (size_t)bh * p.T;
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  const float* x0 = (R::shift && has_in) ? p.xprev_in + (size_t)bh * DK : nullptr;
  const InT* kbase = static_cast<const InT*>(p.k) + rowbase * DK;
  const InT* qbase = static_cast<const InT*>(p.q) + rowbase * DK;
  char* rec = p.ws + ((size_t)bh * p.nchunks + c) * RC::kBytes;

  // Token gates for wave 0 (lane = token), loaded first so their latency overlaps
  // the row loads.
  float g_beta = 0.f, g_lam = 0.f;
  if (wave == 0 && t0 + lane < p.T) {
    const size_t ti = rowbase + t0 + lane;
    g_beta = p.beta != nullptr ? act_beta(p.beta[ti], p.flags) : 1.f;
    if (!PC && p.lam != nullptr) g_lam = act_lam(p.lam[ti], p.flags, R::nlms);
  }
  // Per-channel lambda is loaded here too, so that its latency overlaps the row loads:
  // the rows of [CH][DK] for the channel maximum in eta's denominator (lmx), and the
  // column pass's share (lamv: channel tid % DK, SEGP tokens from (tid / DK) * SEGP).
  constexpr int TPRL = DK / 4, RPPL = NT / TPRL, NPL = CH / RPPL;
  constexpr int TPP = NT / DK, SEGP = CH / TPP;  // column pass: threads per channel, tokens each
  static_assert(SEGP <= 32, "segment parity fits 32 bits");
  f4 lmx[(R::nlms && PC) ? NPL : 1];
  float lamv[PC ? SEGP : 1];
  if constexpr (PC) {
    if constexpr (R::nlms) {
#pragma unroll
      for (int ps = 0; ps < NPL; ++ps) {
        const int tau = t0 + ps * RPPL + tid / TPRL;
        const float m0 = lam_max_init(p.flags);
        lmx[ps] = f4{m0, m0, m0, m0};
        if (tau < p.T && p.lam != nullptr)
          lmx[ps] = *reinterpret_cast<const f4*>(p.lam + (rowbase + tau) * DK + (tid % TPRL) * 4);
      }
    }
    {
      const int tb = (tid / DK) * SEGP;
#pragma unroll
      for (int u = 0; u < SEGP; ++u) {
        const int tau = t0 + tb + u;
        lamv[u] = (tau < p.T && p.lam != nullptr) ? p.lam[(rowbase + tau) * DK + tid % DK] : 0.f;
      }
    }
  }

  // ---- row staging: x rows (shifted keys for the shifted pair) and q rows, phi
  // applied, scaled by one power of two per matrix, into LDS as MFMA operands.
  op_t* Xs = reinterpret_cast<op_t*>(reg[0]);
  op_t* Qs = reinterpret_cast<op_t*>(reg[1]);
  float sX = 1.f, sQ = 1.f;
  {
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
        const int src = R::shift ? tau - 1 : tau;
        if (src >= 0) {
          In<InT>::load(kbase + (uint32_t)(src * DK + col), xr[ps]);
          if (ELU) {
#pragma unroll
            for (int j = 0; j < VW; ++j) xr[ps][j] = phi_elu1(xr[ps][j]);
          }
        } else if (x0 != nullptr) {
#pragma unroll
          for (int j = 0; j < VW; ++j) xr[ps][j] = x0[col + j];
        }
        In<InT>::load(qbase + (uint32_t)(tau * DK + col), qr[ps]);
        if (ELU) {
#pragma unroll
          for (int j = 0; j < VW; ++j) qr[ps][j] = phi_elu1(qr[ps][j]);
        }
      }
      float ns = 0.f, nq = 0.f;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        ns += xr[ps][j] * xr[ps][j];
        nq += qr[ps][j] * qr[ps][j];
        mx = fmaxf(mx, fabsf(xr[ps][j]));
        mq = fmaxf(mq, fabsf(qr[ps][j]));
      }
      ns = group_sum<TPR>(ns);
      if (qk_len > 0.f) nq = group_sum<TPR>(nq);
      if (tid % TPR == 0) {
        s_norm[t] = ns;
        s_qn[t] = nq;
      }
    }
    if (Pol::kScaled) {
      sX = pow2_scale(block_max(mx, s_red));
      sQ = pow2_scale(block_max(mq, s_red + NW));
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int t = ps * RPP + tid / TPR;
      frag_t xo, qo;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        xo[j] = Pol::cvt(xr[ps][j] * sX);
        qo[j] = Pol::cvt(qr[ps][j] * sQ);
      }
      Pol::store_run(Xs + t * LDX, col, xo);
      Pol::store_run(Qs + t * LDX, col, qo);
    }
  }

  // Per-channel: eta's denominator uses the channel max of lambda.
  if constexpr (R::nlms && PC) {
#pragma unroll
    for (int ps = 0; ps < NPL; ++ps) {
      const int t = ps * RPPL + tid / TPRL;
      const f4 w = lmx[ps];
      float m = fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3]));
      m = group_max<TPRL>(m);
      // the activation is monotonic: the max of the activated values is the activated max
      if (tid % TPRL == 0) s_lam[t] = p.lam != nullptr ? act_lam(m, p.flags, true) : 0.f;
    }
  }
  lds_barrier();

  // Token scalars: eta_t, and for scalar decay the in-chunk prefix of log|a|.
  if (wave == 0) {
    const int t = lane;
    const int tau = t0 + t;
    const bool active = tau < p.T;
    float nx = 1.f, mqf = 1.f, xx = s_norm[t];
    if (qk_len > 0.f) {
      nx = rescale_factor(s_norm[t], qk_len);
      mqf = rescale_factor(s_qn[t], qk_len);
      xx = s_norm[t] * nx * nx;
    }
    s_nx[t] = nx;
    s_mq[t] = mqf;
    float eta = 0.f, a = 1.f;
    if (R::nlms) {
      const bool hasx = active && (tau >= 1 || has_in);
      // scale-coupled ridge (scalar lambda): the base ridge times the written key's energy
      const float lam_t = PC ? s_lam[t] : ((p.flags & kFlagLamScaled) ? g_lam * xx : g_lam);
      if (hasx) eta = g_beta / (xx + lam_t + p.eps);
      a = 1.f - eta * lam_t;
    } else {
      if (active) eta = g_beta;
      if (active && p.lam != nullptr && !PC) a = g_lam;
    }
    s_eta[t] = eta;
    float la = log_abs_floor(a);
    int ng = a < 0.f ? 1 : 0;
    wave_prefix(la, ng);
    s_g[t] = la;
    s_sg[t] = (ng & 1) ? -1.f : 1.f;
  }
  lds_barrier();

  // Operand sources of the two Gram products.
  const op_t* A_L = Xs;  // rows x_t (scaled); scalar decay is applied by the mask
  const op_t* A_M = Qs;
  const op_t* B_X = Xs;
  float invL = 1.f / (sX * sX);
  float invM = 1.f / (sQ * sX);
  float* Lf = reinterpret_cast<float*>(reg[2]);  // delta rule only
  float* Mf = reinterpret_cast<float*>(reg[3]);
  float* Tf = reinterpret_cast<float*>(reg[0]);   // after the Gram, X is dead

  if (PC) {
    // Column pass: Gamma ratios per channel, anchored at the chunk midpoint so the two
    // factors of Gamma_{t-1}/Gamma_s stay in range. Each channel's 64 tokens are split over
    // TPP threads (SEGP consecutive tokens each); the segments' log-sums and sign
    // parities meet in region 3 (unused until the Gram products) to give each thread its
    // offset and the anchor. With e_t = exp(g_t - g_A) and s_t its sign, the operands
    // take AM = s_t e_t q, BX = s_t / e_t x and AL = s_{t-1} e_{t-1} x (e_{-1} = exp(-g_A)).
    // BX and AM overwrite the raw X and Q in place (each element is read and written by
    // the same thread); AL goes to region 2.
    op_t* AL = reinterpret_cast<op_t*>(reg[2]);
    op_t* BX = Xs;
    op_t* AM = Qs;
    float* x_tot = reinterpret_cast<float*>(reg[3]);           // [NT] segment log-sums
    uint32_t* x_par = reinterpret_cast<uint32_t*>(x_tot + NT);  // [NT] segment parities
    float* x_anc = reinterpret_cast<float*>(x_par + NT);        // [DK] anchor, in-segment part
    uint32_t* x_apr = reinterpret_cast<uint32_t*>(x_anc + DK);  // [DK]
    constexpr int TA = CH / 2 - 1;
    const int i = tid % DK, part = tid / DK, tb = part * SEGP;
    const int ip = Pol::kpos(i);
    float ev[SEGP];
    uint32_t pl = 0, pr = 0;
    {
      float gs = 0.f;
#pragma unroll
      for (int u = 0; u < SEGP; ++u) {
        const int t = tb + u, tau = t0 + t;
        float lam = R::nlms ? 0.f : 1.f;
        if (tau < p.T && p.lam != nullptr) lam = act_lam(lamv[u], p.flags, R::nlms);
        const float a = R::nlms ? 1.f - s_eta[t] * lam : lam;
        gs += log_abs_floor(a);
        pr ^= (a < 0.f) ? 1u : 0u;
        ev[u] = gs;  // in-segment prefix for now
        pl |= pr << u;
        if (u == TA % SEGP && part == TA / SEGP) {  // t == TA
          x_anc[i] = gs;
          x_apr[i] = pr;
        }
      }
      x_tot[tid] = gs;
      x_par[tid] = pr;
    }
    lds_barrier();
    float off = 0.f, anc, gtot = 0.f;
    uint32_t poff = 0, apr, ptot = 0;
    {
      constexpr int partA = TA / SEGP;
      float aoff = 0.f;
      uint32_t apoff = 0;
#pragma unroll
      for (int w = 0; w < TPP; ++w) {
        const float gw = x_tot[w * DK + i];
        const uint32_t pw = x_par[w * DK + i];
        if (w < part) {
          off += gw;
          poff ^= pw;
        }
        if (w < partA) {
          aoff += gw;
          apoff ^= pw;
        }
        gtot += gw;
        ptot ^= pw;
      }
      anc = aoff + x_anc[i];
      apr = apoff ^ x_apr[i];
    }
    if constexpr (RC::kOps) {
      // The propagate step's operands, from the decay since the chunk start: Gamma_t =
      // exp(off + in-segment prefix) with its sign, Gamma_prev the one before (1 before
      // the first token), Gamma_C the chunk's total. Formed from the staged rows (already
      // scaled by sX, sQ), in the same order of operations the propagate kernel would use.
      _Float16* px = reinterpret_cast<_Float16*>(rec + RC::kPX);
      _Float16* pu = reinterpret_cast<_Float16*>(rec + RC::kPU);
      _Float16* pq = reinterpret_cast<_Float16*>(rec + RC::kPQ);
      float fprev = (poff ? -1.f : 1.f) * __expf(off);
#pragma unroll
      for (int u = 0; u < SEGP; ++u) {
        const int t = tb + u;
        const float g = off + ev[u];
        const uint32_t pcur = poff ^ ((pl >> u) & 1u);
        // signs set in the sign bit of the positive exponentials
        const float fcur = __uint_as_float(__float_as_uint(__expf(g)) | (pcur << 31));
        const float fend = __uint_as_float(__float_as_uint(__expf(gtot - g)) | ((ptot ^ pcur) << 31));
        const float xh = (float)Xs[t * LDX + ip];
        px[t * DK + i] = Pol::cvt(xh * fprev);
        pu[t * DK + i] = Pol::cvt(xh * fend);
        pq[t * DK + i] = Pol::cvt((float)Qs[t * LDX + ip] * fcur);
        fprev = fcur;
      }
      if (part == 0) reinterpret_cast<float*>(rec + RC::kPG)[i] = (ptot ? -1.f : 1.f) * __expf(gtot);
    }
    // e_t with its sign (set in the sign bit of the positive exponential, so that the
    // operands below are plain products), then the block maxima (for the fp16 scales)
    const float eprev =
        __uint_as_float(__float_as_uint(__expf(off - anc)) | ((poff ^ apr) << 31));
    float mAL = 0.f, mBX = 0.f, mAM = 0.f;
#pragma unroll
    for (int u = 0; u < SEGP; ++u) {
      const int t = tb + u;
      const uint32_t sgn = poff ^ ((pl >> u) & 1u) ^ apr;
      ev[u] = __uint_as_float(__float_as_uint(__expf(off + ev[u] - anc)) | (sgn << 31));
      const float xh = (float)Xs[t * LDX + ip];
      const float qh = (float)Qs[t * LDX + ip];
      const float ep = u ? ev[u - 1] : eprev;
      mAL = fmaxf(mAL, fabsf(xh * ep));
      mBX = fmaxf(mBX, fabsf(xh * __builtin_amdgcn_rcpf(ev[u])));
      mAM = fmaxf(mAM, fabsf(qh * ev[u]));
    }
    {
      float sAL = 1.f, sBX = 1.f, sAM = 1.f;
      if (Pol::kScaled) {
        sAL = pow2_scale(block_max(mAL, s_red));
        sBX = pow2_scale(block_max(mBX, s_red + NW));
        sAM = pow2_scale(block_max(mAM, s_red + 2 * NW));
      }
      invL = 1.f / (sX * sAL * sX * sBX);
      invM = 1.f / (sQ * sAM * sX * sBX);
#pragma unroll
      for (int u = 0; u < SEGP; ++u) {
        const int t = tb + u;
        const float xh = (float)Xs[t * LDX + ip];
        const float qh = (float)Qs[t * LDX + ip];
        const float ep = u ? ev[u - 1] : eprev;
        if (R::solve) AL[t * LDX + ip] = Pol::cvt(xh * ep * sAL);
        BX[t * LDX + ip] = Pol::cvt(xh * __builtin_amdgcn_rcpf(ev[u]) * sBX);
        AM[t * LDX + ip] = Pol::cvt(qh * ev[u] * sAM);
      }
    }
    lds_barrier();
    A_L = AL;
    A_M = AM;
    B_X = BX;
    Lf = reinterpret_cast<float*>(reg[3]);
    Mf = reinterpret_cast<float*>(reg[0]);
    Tf = reinterpret_cast<float*>(reg[2]);
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
      if (mt >= nt && (mat == 1 || R::solve)) {
        const op_t* arow = (mat == 0 ? A_L : A_M) + (16 * mt + n) * LDX;
        const op_t* brow = B_X + (16 * nt + n) * LDX;
#pragma unroll
        for (int kb = 0; kb < DK / Pol::KB; ++kb)
          Pol::mma(acc[jj], Pol::lds_row(arow, kb, g), Pol::lds_row(brow, kb, g));
      }
    }
    lds_barrier();
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + NW * jj;
      const int mat = job >> 4;
      const int mt = (job >> 2) & 3, nt = job & 3;
      if (mat == 0 && !R::solve) continue;
      float* dst = mat == 0 ? Lf : Mf;
      const int s = 16 * nt + n;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = 16 * mt + 4 * g + ii;
        float val = 0.f;
        if (mat == 0) {
          if (s < t) {
            float f = s_eta[t] * invL * s_nx[t] * s_nx[s];
            if (!PC) {
              const float gp = t ? s_g[t - 1] : 0.f;
              const float sp = t ? s_sg[t - 1] : 1.f;
              f *= sp * s_sg[s] * __expf(gp - s_g[s]);
            }
            val = f * acc[jj][ii];
          }
        } else {
          if (s <= t) {
            float f = invM * s_mq[t] * s_nx[s];
            if (!PC) f *= s_sg[t] * s_sg[s] * __expf(s_g[t] - s_g[s]);
            val = f * acc[jj][ii];
          }
        }
        dst[t * LDF + s] = val;
      }
    }
  }
  lds_barrier();

  // T = (I + L)^-1 by blocked forward substitution (16x16 blocks, fp32).
  if (R::solve) {
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
    lds_barrier();
    // Below the diagonal on fp32 MFMA: wave j forms column block j top-down,
    //   T_ij = -D_i sum_{k=j}^{i-1} L_ik T_kj,
    // keeping the column's blocks in registers (C layout, which is the B operand's layout),
    // so no further synchronisation is needed.
    static_assert(NB == 4, "four 16-row blocks");
    if (wave == 0) t_column_block<0, LDF>(Lf, Tf, lane);
    else if (wave == 1) t_column_block<1, LDF>(Lf, Tf, lane);
    else if (wave == 2) t_column_block<2, LDF>(Lf, Tf, lane);
    lds_barrier();
  }

  // Write T (delta rule) and M, scaled and in operand order, plus the token factors.
  {
    const int t = tid >> 2, c0 = (tid & 3) * 16;
    float tv[16], mv[16];
    float mt_ = 0.f, mm_ = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      tv[j] = R::solve ? Tf[t * LDF + c0 + j] : 0.f;
      mv[j] = Mf[t * LDF + c0 + j];
      mt_ = fmaxf(mt_, fabsf(tv[j]));
      mm_ = fmaxf(mm_, fabsf(mv[j]));
    }
    float sT = 1.f, sM = 1.f;
    if (Pol::kScaled) {
      sT = pow2_scale(block_max(mt_, s_red));
      sM = pow2_scale(block_max(mm_, s_red + NW));
    }
    op_t* Tg = reinterpret_cast<op_t*>(rec + RC::kT) + t * CH;
    op_t* Mg = reinterpret_cast<op_t*>(rec + RC::kM) + t * CH;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int k0 = c0 + 4 * r4;
      if (R::solve)
        Pol::store4(Tg, k0, tv[4 * r4] * sT, tv[4 * r4 + 1] * sT, tv[4 * r4 + 2] * sT, tv[4 * r4 + 3] * sT);
      Pol::store4(Mg, k0, mv[4 * r4] * sM, mv[4 * r4 + 1] * sM, mv[4 * r4 + 2] * sM, mv[4 * r4 + 3] * sM);
    }
    if (tid < CH) {
      // The row factors of the propagate step: with X, Q stored scaled by sX, sQ,
      //   R = fV V - fP (X S),  O = fO (Q S) + M U,  S' = Gamma_C S + X^T (fU U).
      // Per-channel decay is folded into the operands instead, so only eta and the
      // scales remain.
      const int tt = tid;
      const float e = s_eta[tt];
      float fP, fO, fU;
      if (PC) {
        fP = e / sX;
        fO = 1.f / sQ;
        fU = 1.f / sX;
      } else {
        const float gprev = tt ? s_g[tt - 1] : 0.f;
        const float sprev = tt ? s_sg[tt - 1] : 1.f;
        fP = e * (sprev * __expf(gprev)) / sX;
        fO = (s_sg[tt] * __expf(s_g[tt])) / sQ;
        fU = (s_sg[CH - 1] * s_sg[tt] * __expf(s_g[CH - 1] - s_g[tt])) / sX;
      }
      float* fac = reinterpret_cast<float*>(rec + RC::kFac);
      fac[tt] = fP * s_nx[tt];
      fac[CH + tt] = e;
      fac[2 * CH + tt] = fO * s_mq[tt];
      fac[3 * CH + tt] = fU * s_nx[tt];
    }
    if (tid == 0) {
      float* scv = reinterpret_cast<float*>(rec + RC::kSc);
      scv[0] = 1.f / sT;
      scv[1] = 1.f / sM;
      scv[2] = has_in ? 1.f : 0.f;
      scv[3] = PC ? 1.f : s_sg[CH - 1] * __expf(s_g[CH - 1]);
      scv[4] = sX;
      scv[5] = sQ;
      scv[6] = 0.f;
      scv[7] = 0.f;
    }
    if (c == 0 && tid < DK) {
      reinterpret_cast<float*>(rec + RC::kX0)[tid] = x0 != nullptr ? x0[tid] : 0.f;
    }
  }

  // Normalised linear attention (additive rule, scalar decay): the chunk's terms of the
  // normaliser (ZRec): den_in[t] = sum_{s<=t} M_ts b_s, the factor Gamma_t mq_t of
  // q_t . z at chunk entry, Gamma_C, and the chunk's write sum_s fU_s b_s x_s.
  if (!PC && p.zrec != nullptr) {
    float* zr = p.zrec + ((size_t)bh * p.nchunks + c) * zrec_floats(DK);
    const float gC = s_g[CH - 1], sC = s_sg[CH - 1];
    if (tid < CH) {
      float d = 0.f;
      for (int s = 0; s <= tid; ++s) d += Mf[tid * LDF + s] * s_eta[s];
      zr[tid] = d;
      zr[CH + tid] = s_sg[tid] * __expf(s_g[tid]) * s_mq[tid];
      if (tid == 0) zr[2 * CH] = sC * __expf(gC);
    } else if (tid < CH + DK) {
      const int i = tid - CH, ip = Pol::kpos(i);
      float w = 0.f;
      for (int s = 0; s < CH; ++s)
        w += s_eta[s] * sC * s_sg[s] * __expf(gC - s_g[s]) * s_nx[s] * (float)Xs[s * LDX + ip];
      zr[2 * CH + 4 + i] = w / sX;  // X is held scaled by sX
    }
  }
}

// ================================================================ propagate kernel
// T only for the delta rule; per-channel Gamma_C and the column pass's exchange only with
// per-channel decay (PCX: 1 the per-channel Gamma_C, 2 also the column pass's exchange). With
// bf16 inputs the value tile holds the raw bf16 values, and a d_k = 128 workgroup stays under
// 80 KiB (two share a CU) except with the column pass.
template <typename InT, int DK, bool SOLVE, int PCX>
struct PropLds {
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  static constexpr int LDX = DK + Pol::kPad;  // [CH][DK] operands
  // [DK][CH] transposed operand (fp16 policy). A stride of 34 dwords puts the
  // 4-byte token-pair writes of 8-channel groups in distinct banks.
  static constexpr int LDT = CH + 4;
  static constexpr int LDC = CH + Pol::kPad;  // [CH][CH] operands
  static constexpr int LDV = 64 + 16 / (int)sizeof(InT);  // [CH][64] value tile, input type
  static constexpr size_t kX = (size_t)CH * LDX * sizeof(op_t);
  static constexpr size_t kXU = Pol::kScaled ? (size_t)DK * LDT * sizeof(op_t) : kX;
  static constexpr size_t kC = (size_t)CH * LDC * sizeof(op_t);
  static constexpr size_t kV = (size_t)CH * LDV * sizeof(InT);
  static constexpr size_t oX = 0;
  static constexpr size_t oXU = oX + kX;
  static constexpr size_t oQ = oXU + kXU;
  static constexpr size_t oT = oQ + kX;
  static constexpr size_t oM = oT + (SOLVE ? kC : 0);
  static constexpr size_t oV = oM + kC;
  static constexpr size_t oS = oV + kV;  // small: 5*CH (+ DK, + 2*NT) floats
  static constexpr size_t kBytes = oS + 4 * (5 * CH + (PCX >= 1 ? DK : 0) + (PCX >= 2 ? 2 * NT : 0));
};

// With bf16 inputs two workgroups share a CU where the LDS allows it (two waves per SIMD, so
// each hides the other's LDS and memory latency): the register budget is held to 256 a wave.
template <typename InT, int DK, int RULE, bool PC, bool ELU>
__global__ __launch_bounds__(NT, sizeof(InT) == 2 ? 2 : 1) void prop_kernel(ScanParams p) {
  using R = Rule<RULE>;
  using Pol = PolOf<InT>;
  using op_t = typename Pol::op_t;
  using frag_t = typename Pol::frag_t;
  using RC = Rec<InT, DK, PC>;
  using L = PropLds<InT, DK, R::solve, PC ? (RC::kOps ? 1 : 2) : 0>;
  using Rw = Rows<InT, DK>;
  constexpr int LDX = L::LDX, LDT = L::LDT, LDC = L::LDC, LDV = L::LDV;
  constexpr int KB = Pol::KB;
  constexpr int NKD = DK / KB;  // K blocks over d_k
  constexpr int NKC = CH / KB;  // K blocks over the chunk
  constexpr int NMT = CH / 16;  // row tiles of a chunk
  constexpr int NRT = DK / 16;  // row tiles of S
  constexpr int VW = Rw::VW, TPR = Rw::TPR, RPP = Rw::RPP, NPASS = Rw::NPASS;
  constexpr int TPRv = 64 / VW, RPPv = NT / TPRv, NPV = CH / RPPv;      // value tile
  constexpr int EPT = CH * CH / NT, NVT = EPT * (int)sizeof(op_t) / 16;  // T and M
  // fp16 policy: x rows are staged by (token pair, 8-channel group) tasks so that the
  // transposed copy XU is written as 4-byte token pairs.
  constexpr int NXT = Pol::kScaled ? (CH / 2) * (DK / 8) / NT : 0;  // tasks per thread
  constexpr int NPX = Pol::kScaled ? 2 * NXT : NPASS;

  __shared__ __align__(16) char smem[L::kBytes];
  op_t* Xs = reinterpret_cast<op_t*>(smem + L::oX);
  op_t* XU = reinterpret_cast<op_t*>(smem + L::oXU);
  op_t* Qs = reinterpret_cast<op_t*>(smem + L::oQ);
  op_t* Ts = reinterpret_cast<op_t*>(smem + L::oT);
  op_t* Ms = reinterpret_cast<op_t*>(smem + L::oM);
  InT* Vs = reinterpret_cast<InT*>(smem + L::oV);
  float* s_fac = reinterpret_cast<float*>(smem + L::oS);  // [4][CH]: fP, fV, fO, fU
  float* s_misc = s_fac + 4 * CH;  // [0] Gamma_C (scalar decay), [1] 1/sT, [2] 1/sM
  float* s_gC = s_misc + CH;       // [DK] per-channel Gamma_C
  float* s_pg = s_gC + DK;         // [NT] per-channel decay: each thread's segment log-sum
  uint32_t* s_pp = reinterpret_cast<uint32_t*>(s_pg + NT);  // [NT] and its sign parity
  const float* s_fP = s_fac;
  const float* s_fV = s_fac + CH;
  const float* s_fO = s_fac + 2 * CH;
  const float* s_fU = s_fac + 3 * CH;

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
  // A null output pointer asks for the state alone (the segmented scan's state passes):
  // the read (Q S + M U) and its operands are skipped.
  const bool want_out = p.out != nullptr;
  // per-head base pointers; every per-thread offset below fits in 32 bits
  const InT* kbase = static_cast<const InT*>(p.k) + rowbase * DK;
  const InT* qbase = static_cast<const InT*>(p.q) + rowbase * DK;
  const InT* vbase = static_cast<const InT*>(p.v) + rowbase * dv + grp * 64;
  float* obase32 = static_cast<float*>(p.out) + rowbase * dv + grp * 64;
  uint16_t* obase16 = static_cast<uint16_t*>(p.out) + rowbase * dv + grp * 64;
  const uint32_t olane = (uint32_t)(4 * g * dv + wave * 16 + n);  // lane's part of the offset

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
  const float* x0 = (R::shift && has_in) ? reinterpret_cast<const float*>(rec0 + RC::kX0) : nullptr;

  const int col = (tid % TPR) * VW;    // row staging: this thread's columns
  const int vcol = (tid % TPRv) * VW;  // value tile: this thread's columns
  const int e0 = tid * EPT;            // T / M: this thread's elements
  u32x4 px[NPX], pq[NPASS], pv[NPV], pt[NVT], pm[NVT];
  f4 pf = {0.f, 0.f, 0.f, 0.f};
  // Per-channel decay: thread (channel i, part) handles SEG consecutive tokens of its
  // channel. Their raw lambdas for chunk c are loaded during chunk c-1 (software
  // pipelined: consumed at the top of the column pass, then reloaded for the next chunk).
  constexpr int TPC = NT / DK, SEG = CH / TPC;
  // With fp16 operands the prep kernel has folded the per-channel decay into the chunk's
  // operands (X~, X^, Q~ and Gamma_C in the record): staging copies them, no lambda is read.
  constexpr bool OPS = RC::kOps;
  float plam[(PC && !OPS) ? SEG : 1];
  u32x4 pxu[OPS ? NPX : 1];
  float pgc = 1.f;
  auto load_lam = [&](int tbase) {
    if constexpr (PC && !OPS) {
      const int i = tid % DK, tb = (tid / DK) * SEG;
#pragma unroll
      for (int u = 0; u < SEG; ++u) {
        const int tau = tbase + tb + u;
        plam[u] = (tau < p.T && p.lam != nullptr) ? p.lam[(rowbase + tau) * DK + i] : 0.f;
      }
    }
  };
  load_lam(0);
  float psX = 1.f, psQ = 1.f, pinvT = 1.f, pinvM = 1.f, pgC = 1.f;
  uint32_t valid = 0;

  // Iteration c stages chunk c from registers, then issues the loads of chunk c+1
  // and computes chunk c while they are in flight (c = -1 only loads chunk 0).
  for (int c = -1; c < p.nchunks; ++c) {
    const int t0 = c * CH;
    if (c >= 0) {
      // ---- registers -> LDS (chunk c)
      if constexpr (Pol::kScaled) {
#pragma unroll
        for (int r = 0; r < NXT; ++r) {
          const int task = tid + NT * r;
          const int cg = (task & 3) + 4 * (task >> 7), tp = (task >> 2) & 31;
          frag_t xo[2];
          if constexpr (OPS) {
            // X~ rows into Xs; the update's operand X^ into the transposed copy
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              Pol::store_run(Xs + (2 * tp + h) * LDX, 8 * cg, __builtin_bit_cast(frag_t, px[2 * r + h]));
              xo[h] = __builtin_bit_cast(frag_t, pxu[2 * r + h]);
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int t = 2 * tp + h;
              float x[VW];
              In<InT>::decode(px[2 * r + h], x);
              if (R::shift && t0 + t == 0) {
#pragma unroll
                for (int j = 0; j < VW; ++j) x[j] = x0 != nullptr ? x0[8 * cg + j] : 0.f;
              } else if (ELU && (valid >> (2 * r + h) & 1u)) {
#pragma unroll
                for (int j = 0; j < VW; ++j) x[j] = phi_elu1(x[j]);
              }
#pragma unroll
              for (int j = 0; j < VW; ++j) xo[h][j] = Pol::cvt(x[j] * psX);
              Pol::store_run(Xs + t * LDX, 8 * cg, xo[h]);
            }
          }
          if (!PC || OPS) {
            const int tp2 = Pol::kpos(2 * tp);  // tokens 2tp, 2tp+1 are adjacent
#pragma unroll
            for (int j = 0; j < VW; ++j)
              *reinterpret_cast<h2*>(XU + (8 * cg + j) * LDT + tp2) = h2{xo[0][j], xo[1][j]};
          }
        }
      } else {
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const int t = ps * RPP + tid / TPR;
          float x[VW];
          In<InT>::decode(px[ps], x);
          if (R::shift && t0 + t == 0) {
#pragma unroll
            for (int j = 0; j < VW; ++j) x[j] = x0 != nullptr ? x0[col + j] : 0.f;
          } else if (ELU && (valid >> ps & 1u)) {
#pragma unroll
            for (int j = 0; j < VW; ++j) x[j] = phi_elu1(x[j]);
          }
          frag_t xo;
#pragma unroll
          for (int j = 0; j < VW; ++j) xo[j] = Pol::cvt(x[j] * psX);
          Pol::store_run(Xs + t * LDX, col, xo);
          if (!PC) Pol::store_run(XU + t * LDX, col, xo);
        }
      }
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int t = ps * RPP + tid / TPR;
        if (!want_out) {
        } else if constexpr (OPS) {
          Pol::store_run(Qs + t * LDX, col, __builtin_bit_cast(frag_t, pq[ps]));
        } else {
          float qv[VW];
          In<InT>::decode(pq[ps], qv);
          if (ELU && (valid >> (16 + ps) & 1u)) {
#pragma unroll
            for (int j = 0; j < VW; ++j) qv[j] = phi_elu1(qv[j]);
          }
          frag_t qo;
#pragma unroll
          for (int j = 0; j < VW; ++j) qo[j] = Pol::cvt(qv[j] * psQ);
          Pol::store_run(Qs + t * LDX, col, qo);
        }
      }
      if (OPS && tid < DK) s_gC[tid] = pgc;
#pragma unroll
      for (int ps = 0; ps < NPV; ++ps) {
        const int t = ps * RPPv + tid / TPRv;
        // the raw input values (16 bytes a thread)
        *reinterpret_cast<u32x4*>(Vs + t * LDV + vcol) = pv[ps];
      }
      const int rr = e0 / CH, cc2 = e0 % CH;
#pragma unroll
      for (int j = 0; j < NVT; ++j) {
        if (R::solve) reinterpret_cast<u32x4*>(Ts + rr * LDC + cc2)[j] = pt[j];
        if (want_out) reinterpret_cast<u32x4*>(Ms + rr * LDC + cc2)[j] = pm[j];
      }
      if (tid < CH) {
        s_fac[tid] = pf[0];
        s_fac[CH + tid] = pf[1];
        s_fac[2 * CH + tid] = pf[2];
        s_fac[3 * CH + tid] = pf[3];
      }
      if (tid == 0) {
        s_misc[0] = pgC;
        s_misc[1] = pinvT;
        s_misc[2] = pinvM;
      }
      lds_barrier();
    }
    if (c + 1 < p.nchunks) {
      // ---- global -> registers (chunk c+1)
      const int tn = t0 + CH;
      const char* rec = rec0 + (size_t)(c + 1) * RC::kBytes;
      valid = 0;
      if constexpr (OPS) {
        // the record holds every row of the chunk (zero past the sequence end)
#pragma unroll
        for (int r = 0; r < NXT; ++r) {
          const int task = tid + NT * r;
          const int cg = (task & 3) + 4 * (task >> 7), tp = (task >> 2) & 31;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t off = (uint32_t)((2 * tp + h) * DK + 8 * cg) * 2u;
            px[2 * r + h] = ld16(rec + RC::kPX, off);
            pxu[2 * r + h] = ld16(rec + RC::kPU, off);
          }
        }
        if (tid < DK) pgc = reinterpret_cast<const float*>(rec + RC::kPG)[tid];
      } else if constexpr (Pol::kScaled) {
#pragma unroll
        for (int r = 0; r < NXT; ++r) {
          const int task = tid + NT * r;
          const int cg = (task & 3) + 4 * (task >> 7), tp = (task >> 2) & 31;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int tau = tn + 2 * tp + h;
            const int src = R::shift ? tau - 1 : tau;
            px[2 * r + h] = u32x4{0u, 0u, 0u, 0u};
            if (tau < p.T && src >= 0) {
              px[2 * r + h] = ld16(kbase, (uint32_t)(src * DK + 8 * cg) * (uint32_t)sizeof(InT));
              valid |= 1u << (2 * r + h);
            }
          }
        }
      } else {
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const int tau = tn + ps * RPP + tid / TPR;
          const int src = R::shift ? tau - 1 : tau;
          px[ps] = u32x4{0u, 0u, 0u, 0u};
          if (tau < p.T && src >= 0) {
            px[ps] = ld16(kbase, (uint32_t)(src * DK + col) * (uint32_t)sizeof(InT));
            valid |= 1u << ps;
          }
        }
      }
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int tau = tn + ps * RPP + tid / TPR;
        if (!want_out) {
        } else if constexpr (OPS) {
          pq[ps] = ld16(rec + RC::kPQ, (uint32_t)((ps * RPP + tid / TPR) * DK + col) * 2u);
        } else {
          pq[ps] = u32x4{0u, 0u, 0u, 0u};
          if (tau < p.T) {
            pq[ps] = ld16(qbase, (uint32_t)(tau * DK + col) * (uint32_t)sizeof(InT));
            valid |= 1u << (16 + ps);
          }
        }
      }
#pragma unroll
      for (int ps = 0; ps < NPV; ++ps) {
        const int tau = tn + ps * RPPv + tid / TPRv;
        pv[ps] = u32x4{0u, 0u, 0u, 0u};
        // a null value pointer means all-zero values (the segmented scan's transition pass)
        if (tau < p.T && grp * 64 + vcol < dv && p.v != nullptr)
          pv[ps] = ld16(vbase, (uint32_t)(tau * dv + vcol) * (uint32_t)sizeof(InT));
      }
      const u32x4* Tg = reinterpret_cast<const u32x4*>(reinterpret_cast<const op_t*>(rec + RC::kT) + e0);
      const u32x4* Mg = reinterpret_cast<const u32x4*>(reinterpret_cast<const op_t*>(rec + RC::kM) + e0);
#pragma unroll
      for (int j = 0; j < NVT; ++j) {
        if (R::solve) pt[j] = Tg[j];
        if (want_out) pm[j] = Mg[j];
      }
      if (tid < CH) {
        const float* fac = reinterpret_cast<const float*>(rec + RC::kFac);
        pf = f4{fac[tid], fac[CH + tid], fac[2 * CH + tid], fac[3 * CH + tid]};
      }
      const float* scv = reinterpret_cast<const float*>(rec + RC::kSc);
      pinvT = scv[0];
      pinvM = scv[1];
      pgC = scv[3];
      psX = scv[4];
      psQ = scv[5];
    }
    if (c < 0) continue;

    if (PC && !OPS) {
      // per-channel decay folded into the operands: X*Gamma_prev, Q*Gamma, X*Gamma_C/Gamma.
      // Each channel's 64 tokens are split over TPC threads; the segments' log-sums and
      // sign parities are combined through LDS into each segment's offset and the chunk
      // total. Gamma_prev of a token is Gamma of the one before, carried along.
      static_assert(SEG <= 32, "segment parity fits 32 bits");
      const int i = tid % DK, part = tid / DK, tb = part * SEG;
      const int ip = Pol::kpos(i);
      float gl[SEG];
      uint32_t pl = 0, pr = 0;
      float gsum = 0.f;
#pragma unroll
      for (int u = 0; u < SEG; ++u) {
        const int tau = t0 + tb + u;
        float lam = R::nlms ? 0.f : 1.f;
        if (tau < p.T && p.lam != nullptr) lam = act_lam(plam[u], p.flags, R::nlms);
        const float a = R::nlms ? 1.f - s_fV[tb + u] * lam : lam;
        gsum += log_abs_floor(a);
        pr ^= (a < 0.f) ? 1u : 0u;
        gl[u] = gsum;
        pl |= pr << u;
      }
      if (c + 1 < p.nchunks) load_lam(t0 + CH);
      s_pg[tid] = gsum;
      s_pp[tid] = pr;
      lds_barrier();
      float off = 0.f, gC = 0.f;
      uint32_t poff = 0, pC = 0;
#pragma unroll
      for (int w = 0; w < TPC; ++w) {
        const float g = s_pg[w * DK + i];
        const uint32_t pp = s_pp[w * DK + i];
        if (w < part) {
          off += g;
          poff ^= pp;
        }
        gC += g;
        pC ^= pp;
      }
      if (part == 0) s_gC[i] = (pC ? -1.f : 1.f) * __expf(gC);
      float fprev = (poff ? -1.f : 1.f) * __expf(off);
#pragma unroll
      for (int u = 0; u < SEG; ++u) {
        const int t = tb + u;
        const float g = off + gl[u];
        const uint32_t pcur = poff ^ ((pl >> u) & 1u);
        const float fcur = (pcur ? -1.f : 1.f) * __expf(g);
        const float fend = ((pC ^ pcur) ? -1.f : 1.f) * __expf(gC - g);
        const float xh = (float)Xs[t * LDX + ip];
        if constexpr (Pol::kScaled) XU[i * LDT + Pol::kpos(t)] = Pol::cvt(xh * fend);
        else XU[t * LDX + i] = Pol::cvt(xh * fend);
        Xs[t * LDX + ip] = Pol::cvt(xh * fprev);
        Qs[t * LDX + ip] = Pol::cvt((float)Qs[t * LDX + ip] * fcur);
        fprev = fcur;
      }
      lds_barrier();
    }

    if (wave_on) {
      const float invT = s_misc[1], invM = s_misc[2];
      // row factors of the lane's rows: 4 consecutive rows per tile
      auto fac4 = [&](const float* f, int mt) { return *reinterpret_cast<const f4*>(f + 16 * mt + 4 * g); };
      // S as the B operand of X S and Q S (one power-of-two scale per column)
      float ms = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) ms = fmaxf(ms, fabsf(s[rt][ii]));
      float sS = 1.f, isS = 1.f;
      if (Pol::kScaled) pow2_scale2(col_max(ms), sS, isS);
      frag_t Sf[NKD];
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) Sf[kb] = Pol::from_c(s, kb, sS);

      f4 U[NMT];
      if (R::solve) {
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
            const float r = fac4(s_fV, mt)[ii] * In<InT>::load1(Vs + t * LDV + wave * 16 + n) -
                            fac4(s_fP, mt)[ii] * isS * P[mt][ii];
            P[mt][ii] = r;
            mr = fmaxf(mr, fabsf(r));
          }
        float sR = 1.f, isR = 1.f;
        if (Pol::kScaled) pow2_scale2(col_max(mr), sR, isR);
        frag_t Rf[NKC];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) Rf[kb] = Pol::from_c(P, kb, sR);
        const float fu = invT * isR;
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
            U[mt][ii] = fac4(s_fV, mt)[ii] * In<InT>::load1(Vs + t * LDV + wave * 16 + n);
          }
      }

      // O = diag(Gamma) Q S + M U
      if (want_out) {
      f4 O[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        O[mt] = f4{0.f, 0.f, 0.f, 0.f};
        const op_t* arow = Qs + (16 * mt + n) * LDX;
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) Pol::mma(O[mt], Pol::lds_row(arow, kb, g), Sf[kb]);
        O[mt] *= fac4(s_fO, mt) * isS;
      }
      float mu = 0.f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) mu = fmaxf(mu, fabsf(U[mt][ii]));
      float sU = 1.f, isU = 1.f;
      if (Pol::kScaled) pow2_scale2(col_max(mu), sU, isU);
      {
        frag_t Uf[NKC];
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) Uf[kb] = Pol::from_c(U, kb, sU);
        const float fm = invM * isU;
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
          const int trow = t0 + 16 * mt + ii;  // uniform part of the row
          if (trow + 4 * g < p.T) {
            const uint32_t o = (uint32_t)(trow * dv) + olane;
            if (out_bf16) obase16[o] = f32_to_bf16_bits(O[mt][ii]);
            else obase32[o] = O[mt][ii];
          }
        }
      }

      // S' = Gamma_C S + X^T (diag(Gamma_C/Gamma) U)
      float mut = 0.f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        U[mt] *= fac4(s_fU, mt);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) mut = fmaxf(mut, fabsf(U[mt][ii]));
      }
      float sUt = 1.f, iUt = 1.f;
      if (Pol::kScaled) pow2_scale2(col_max(mut), sUt, iUt);
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
        if (PC) {
          const f4 gc = *reinterpret_cast<const f4*>(s_gC + 16 * rt + 4 * g);
          s[rt] = gc * s[rt] + acc * iUt;
        } else {
          s[rt] = s[rt] * gCs + acc * iUt;
        }
      }
    }
    lds_barrier();
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
    if (grp == 0 && (p.flags & kFlagZnorm) == 0) {  // with the normaliser the slot holds z
      for (int i = tid; i < DK; i += NT) {
        float x = In<InT>::load1(kbase + (uint32_t)((p.T - 1) * DK + i));
        if (ELU) x = phi_elu1(x);
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
bool scan_split_path(int bf16, uint32_t flags) {
  return bf16 != 0 && (flags & (kFlagPhiElu1 | kFlagPerChannel)) == 0;
}

size_t scan_record_bytes(int bf16, int dk, uint32_t flags) {
  if (scan_split_path(bf16, flags)) return dk == 64 ? RecSplit<64>::kBytes : RecSplit<128>::kBytes;
  if (bf16 && (flags & kFlagPerChannel))
    return dk == 64 ? Rec<uint16_t, 64, true>::kBytes : Rec<uint16_t, 128, true>::kBytes;
  if (bf16) return dk == 64 ? Rec<uint16_t, 64>::kBytes : Rec<uint16_t, 128>::kBytes;
  return dk == 64 ? Rec<float, 64>::kBytes : Rec<float, 128>::kBytes;
}

bool scan_supported(int dk, int dv) {
  return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

template <typename InT, int DK, int RULE, bool PC, bool ELU>
static hipError_t launch_scan_t(const ScanParams& p, hipStream_t st, int phases) {
  const unsigned nprep = (unsigned)((size_t)p.BH * p.nchunks);
  if constexpr (sizeof(InT) == 2 && !PC && !ELU) {
    // bf16, identity map, scalar decay: split-operand propagate kernel
    if (phases & 1) {
      const hipError_t e = launch_prep_split(p, st);
      if (e != hipSuccess) return e;
    }
    if (phases & 2) return launch_prop_split(p, st);
    return hipSuccess;
  } else {
    if (phases & 1) {
      hipLaunchKernelGGL((prep_kernel<InT, DK, RULE, PC, ELU>), dim3(nprep), dim3(NT), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & 2) {
      const int NG = (p.dv + 63) / 64;
      const unsigned nprop = (unsigned)(8 * NG * ((p.BH + 7) / 8));
      hipLaunchKernelGGL((prop_kernel<InT, DK, RULE, PC, ELU>), dim3(nprop), dim3(NT), 0, st, p);
      return hipGetLastError();
    }
    return hipSuccess;
  }
}

template <typename InT, int DK, int RULE, bool PC>
static hipError_t launch_scan_e(const ScanParams& p, hipStream_t st, int ph) {
  return (p.flags & kFlagPhiElu1) ? launch_scan_t<InT, DK, RULE, PC, true>(p, st, ph)
                                  : launch_scan_t<InT, DK, RULE, PC, false>(p, st, ph);
}

template <typename InT, int DK, int RULE>
static hipError_t launch_scan_r(const ScanParams& p, hipStream_t st, int ph) {
  return (p.flags & kFlagPerChannel) ? launch_scan_e<InT, DK, RULE, true>(p, st, ph)
                                     : launch_scan_e<InT, DK, RULE, false>(p, st, ph);
}

template <typename InT, int DK>
static hipError_t launch_scan_dk(const ScanParams& p, hipStream_t st, int ph) {
  if (p.rule == kRuleDelta) return launch_scan_r<InT, DK, kRuleDelta>(p, st, ph);
  if (p.rule == kRuleInner) return launch_scan_r<InT, DK, kRuleInner>(p, st, ph);
  return launch_scan_r<InT, DK, kRuleAdditive>(p, st, ph);
}

hipError_t launch_scan(const ScanParams& p, hipStream_t st, int phases) {
  if (scan_add_path(p.bf16, p.rule, p.flags)) return (phases & 2) ? launch_scan_add(p, st) : hipSuccess;
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
