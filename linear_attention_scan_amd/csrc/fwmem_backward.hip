// Backward pass of the scan: the gradients of L = <dO, o> + <dS_T, S_T> with respect to
// q, k, v, beta, lambda, the initial state S0 and the carried key, for the delta, inner,
// additive and per-value-channel rules with phi identity or elu+1. The pages give no
// backward pass; this is the
// reverse-mode derivative of the recurrence as the forward pass states it ("Fast Weight
// Attention for Continual Learning" reading notes, sections 3.2, 4.1-4.3; "attention is
// also an FFN", sections 2.1, 3.2):
//   S_t = a_t S_{t-1} + eta_t x_t w_t^T,  o_t = S_t^T phi(q_t),
// with w_t = v_t - S_{t-1}^T x_t (delta) or v_t (inner, additive), and for the delta and
// inner rules a_t = 1 - eta_t lambda_t, eta_t = beta_t / (|x_t|^2 + lambda_t + eps),
// x_t = phi(k_{t-1}). Undoing step t with G = dL/dS_t:
//   dphi(q_t) = S_t dO_t;  G += phi(q_t) dO_t^T;  da = <G, S_{t-1}>;
//   delta:    deta = x^T G r, dr = eta G^T x, dx = eta G r - S_{t-1} dr, dv = dr,
//             G_{t-1} = a G - x dr^T
//   inner:    deta = x^T G v, dx = eta G v, dv = eta G^T x, G_{t-1} = a G
//   additive: dgamma = da, dbeta = k^T G v, dphi(k) = beta G v, dv = beta G^T phi(k),
//             G_{t-1} = gamma G
// and for the shifted rules the scalar chain through a, eta and the denominator.
//
// The per-value-channel rule gives column c its own step eta_c and decay 1 - eta_c lambda,
// so da, deta and the beta gradient are per column.
// Options: per channel, lambda_i scales row i's decay (1 - eta lambda_i, or the retention
// gamma_i) and eta's denominator takes the largest lambda_i, so da and the lambda gradient
// are per row. Pre-activated gates are activated as they are staged and their gradients
// taken through the activation. The scale-coupled ridge is lambda |x|^2 (scalar lambda).
// With QK normalisation, q, k and the carried key are rescaled to a fixed length as they
// are staged, and a second kernel takes their gradients back through the rescaling. With
// the normaliser (additive rule), o_t = S_t^T q_t / (z_t . q_t + eps): a gradient of z is
// carried back beside G, and the chunk's z values are recomputed into LDS.
//
// One persistent 1024-thread workgroup per head, token-serial (the chunked backward is
// future work). The state is distributed as in the decode kernel: thread (rg, cq) holds
// float4 column group cq of rows rg, rg + RG, ... A chunk here is 64 tokens, 32 with a
// per-channel lambda, a per-column beta or the normaliser. A forward pass stores the state at every chunk start in the
// workspace; then, per chunk from the last, the chunk's states after each token are
// recomputed into the workspace and the chunk's tokens are undone from the last. Each
// chunk's keys, queries, values, dO and gates are staged in LDS once; a token's column and
// scalar sums share one reduction (two LDS-only barriers), and the state before the next
// token to undo is loaded while the current one is undone.
#include "fwmem_backward.h"
#include "fwmem_device.h"
#include "fwmem_internal.h"

namespace fwmem {
namespace {

constexpr int NT = 1024;
constexpr int NWV = NT / 64;

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations are complete
// before it arrives and the compiler moves no memory access across it, but its global loads
// stay in flight (__syncthreads would wait for them), so the prefetch of the next state
// overlaps the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-token scalars of the write: step size (or write scale) eta, decay a, the
// denominator of eta, the write scale b, and whether the step writes at all.
struct Sc {
  float eta, a, den, rden, b;
  float lsc;  // the ridge's scale: |x|^2 with the scale-coupled ridge, else 1
  bool key;
};

template <typename InT, int DK, int DV, int RULE, bool PCX, bool ZN>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  using R = Rule<RULE>;
  constexpr bool PV = RULE == kRuleDeltaPV;  // one step size per value column
  // tokens staged at a time, and between stored states (a per-channel lambda or a
  // per-column beta, also staged, halves it to fit LDS)
  constexpr int CK = bwd_chunk(PCX || PV || ZN);
  static_assert(!ZN || (RULE == kRuleAdditive && !PCX), "the normaliser: additive rule, scalar decay");
  constexpr int TPRd = DV / 4;   // threads per row
  constexpr int RG = NT / TPRd;  // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(DK % RG == 0 && RPT >= 1, "shape");
  // One chunk at a time in LDS (149,536 bytes at dk = dv = 128; 100,128 with a per-channel
  // lambda).
  // (float4 accesses: s_w, s_do, s_col and s_tot rows are 16-byte aligned)
  __shared__ float s_x[CK][DK];   // written keys x_t (phi applied)
  __shared__ float s_q[CK][DK];   // phi(q_t)
  __shared__ __attribute__((aligned(16))) float s_w[CK][DV];   // v_t; delta: the residual once recomputed
  __shared__ __attribute__((aligned(16))) float s_do[CK][DV];  // dO_t
  __shared__ __attribute__((aligned(16))) float s_col[2][NWV][DV];
  __shared__ float s_sum[2][NWV][2];
  __shared__ __attribute__((aligned(16))) float s_tot[2][DV + 4];  // column totals, then the two scalars
  __shared__ float s_lc[PCX ? CK : 1][PCX ? DK : 1];  // per-channel lambda (or retention)
  __shared__ __attribute__((aligned(16))) float s_bc[PV ? CK : 1][PV ? DV : 4];  // per-column beta
  __shared__ float s_n[CK], s_bt[CK], s_lm[CK];  // |x|^2, beta, lambda (per channel: its maximum)
  __shared__ int s_im[CK];                        // per channel: the first channel at the maximum
  // the normaliser: z after each of the chunk's tokens, before its first, and z_t . q_t + eps
  __shared__ float s_z[ZN ? CK : 1][ZN ? DK : 1], s_z0[ZN ? DK : 1], s_den[ZN ? CK : 1];

  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % TPRd, rg = tid / TPRd;
  const int T = p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const float qlen = qk_length(p.flags, DK);  // > 0: q, k and the carried key are rescaled
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  const size_t rb = (size_t)bh * T;
  const InT* qb = static_cast<const InT*>(p.q) + rb * DK;
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV;
  const size_t SS = (size_t)DK * DV;
  const int nch = (T + CK - 1) / CK;
  float* ckpt = p.ws + (size_t)bh * bwd_floats_per_head(T, DK, DV, PCX || PV || ZN, ZN);
  float* cs = ckpt + (size_t)nch * SS;  // [CK] states after each token of a chunk
  float* zck = cs + (size_t)CK * SS + (size_t)CK * DV;  // ZN: [nch][DK] z at each chunk start

  auto phi = [&](float x) { return elu ? phi_elu1(x) : x; };
  // phi'(z) from y = phi(z): 1 for the identity; for elu+1, 1 where z > 0 (y > 1) and
  // exp(z) = y elsewhere
  auto dphi_of = [&](float y) { return elu ? (y > 1.f ? 1.f : y) : 1.f; };
  auto row = [&](int j) { return rg + RG * j; };

  // Sums over the workgroup: a per-thread float4 (the thread's four columns) summed over
  // the row groups, and two scalars summed over all threads. Each wave leaves its partial
  // sums in LDS; after a barrier DV + 2 threads add the waves' partials of one value each;
  // after a second barrier every thread reads the totals. The two sets of LDS buffers
  // alternate, so a buffer is rewritten only after every thread has passed the barriers
  // of the call in between.
  int par = 0;
  auto reduce = [&](f4 v, float a, float b, float& sa, float& sb) -> f4 {
#pragma unroll
    for (int o = TPRd; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], o);
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane < TPRd) *reinterpret_cast<f4*>(&s_col[par][wave][4 * cq]) = v;
    if (lane == 0) {
      s_sum[par][wave][0] = a;
      s_sum[par][wave][1] = b;
    }
    lds_barrier();
    if (tid < DV + 2) {
      float x = 0.f;
      if (tid < DV) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) x += s_col[par][w][tid];
      } else {
#pragma unroll
        for (int w = 0; w < NWV; ++w) x += s_sum[par][w][tid - DV];
      }
      s_tot[par][tid] = x;
    }
    lds_barrier();
    const f4 s = *reinterpret_cast<const f4*>(&s_tot[par][4 * cq]);
    sa = s_tot[par][DV];
    sb = s_tot[par][DV + 1];
    par ^= 1;
    return s;
  };
  // sum over a row's TPRd consecutive lanes
  auto rowsum = [&](float v) -> float {
#pragma unroll
    for (int o = 1; o < TPRd; o <<= 1) v += __shfl_xor(v, o);
    return v;
  };
  auto load_state = [&](const float* src, f4 (&S)[RPT]) {
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      S[j] = src != nullptr ? *reinterpret_cast<const f4*>(src + (size_t)row(j) * DV + 4 * cq) : f4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_state = [&](float* dst, const f4 (&S)[RPT]) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) *reinterpret_cast<f4*>(dst + (size_t)row(j) * DV + 4 * cq) = S[j];
  };
  // Tokens [t0, t1) of a chunk into LDS (rows past t1 zero): the written keys and their
  // squared norms, v and the gates; for the backward also phi(q) and dO.
  auto stage = [&](int t0, int t1, bool bwd) {
    for (int idx = tid; idx < CK * DK; idx += NT) {
      const int u = idx / DK, i = idx % DK, t = t0 + u;
      float x = 0.f, qq = 0.f;
      if (t < t1) {
        if (R::shift) {
          if (t >= 1) x = phi(In<InT>::load1(kb + (size_t)(t - 1) * DK + i));
          else if (has_in && p.xprev_in != nullptr) x = p.xprev_in[(size_t)bh * DK + i];
        } else {
          x = phi(In<InT>::load1(kb + (size_t)t * DK + i));
        }
        if (bwd) qq = phi(In<InT>::load1(qb + (size_t)t * DK + i));
      }
      s_x[u][i] = x;
      if (bwd) s_q[u][i] = qq;
      if (PCX)
        s_lc[u][i] = (t < t1 && p.lam != nullptr) ? act_lam(p.lam[(rb + t) * DK + i], p.flags, R::nlms)
                                                   : (R::nlms ? 0.f : 1.f);
    }
    for (int idx = tid; idx < CK * DV; idx += NT) {
      const int u = idx / DV, j = idx % DV, t = t0 + u;
      s_w[u][j] = t < t1 ? In<InT>::load1(vb + (size_t)t * DV + j) : 0.f;
      if (bwd) s_do[u][j] = t < t1 ? p.dout[(rb + t) * DV + j] : 0.f;
      if constexpr (PV) s_bc[u][j] = t < t1 ? act_beta(p.beta[(rb + t) * DV + j], p.flags) : 1.f;
    }
    if (tid < CK) {
      const int t = t0 + tid;
      s_bt[tid] = (!PV && t < t1 && p.beta != nullptr) ? act_beta(p.beta[rb + t], p.flags) : 1.f;
      if (!PCX)
        s_lm[tid] = (t < t1 && p.lam != nullptr) ? act_lam(p.lam[rb + t], p.flags, R::nlms) : (R::nlms ? 0.f : 1.f);
    }
    __syncthreads();
    for (int u = wave; u < CK; u += NWV) {
      float n = 0.f;
      for (int i = lane; i < DK; i += 64) n += s_x[u][i] * s_x[u][i];
      n = wave_sum(n);
      if (qlen > 0.f) {
        // QK normalisation: the row rescaled to length qlen by the wave that measured it
        float nq = 0.f;
        if (bwd) {
          for (int i = lane; i < DK; i += 64) nq += s_q[u][i] * s_q[u][i];
          nq = wave_sum(nq);
        }
        const float fx = rescale_factor(n, qlen), fq = rescale_factor(nq, qlen);
        for (int i = lane; i < DK; i += 64) {
          s_x[u][i] *= fx;
          if (bwd) s_q[u][i] *= fq;
        }
        n *= fx * fx;
      }
      if (lane == 0) s_n[u] = n;
      if (PCX && R::nlms) {
        // the largest lambda over the channels and the first channel holding it
        float best = s_lc[u][lane];
        int bi = lane;
        for (int i = lane + 64; i < DK; i += 64)
          if (s_lc[u][i] > best) {
            best = s_lc[u][i];
            bi = i;
          }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ob = __shfl_xor(best, o);
          const int oi = __shfl_xor(bi, o);
          if (ob > best || (ob == best && oi < bi)) {
            best = ob;
            bi = oi;
          }
        }
        if (lane == 0) {
          s_lm[u] = best;
          s_im[u] = bi;
        }
      }
    }
    __syncthreads();
  };
  // With pre-activated gates the gradients are taken with respect to the pre-activation
  // z: times the activation's derivative, from the activated value y: sigmoid y (1 - y),
  // 2 sigmoid y (1 - y / 2), the additive retention y (1 - y), softplus 1 - e^-y.
  auto dbeta_dz = [&](float y) {
    if (p.flags & kFlagBetaSig) return y * (1.f - y);
    if (p.flags & kFlagBetaSig2) return y * (1.f - 0.5f * y);
    return 1.f;
  };
  auto dlam_dz = [&](float y) {
    if (!(p.flags & kFlagLamAct)) return 1.f;
    return R::nlms ? -expm1f(-y) : y * (1.f - y);
  };
  // decay of row j at token u: 1 - eta lambda_i (ridge rules) or gamma_i (additive) per
  // channel, else the token's scalar decay
  auto arow = [&](const Sc& s, int u, int j) -> float {
    if (!PCX) return s.a;
    const float l = s_lc[u][row(j)];
    return R::nlms ? 1.f - s.eta * l * s.lsc : l;
  };
  auto scal = [&](int t, int u) -> Sc {
    Sc s;
    if (R::nlms) {
      s.key = t >= 1 || has_in;
      s.lsc = (p.flags & kFlagLamScaled) ? s_n[u] : 1.f;
      s.den = s_n[u] + s_lm[u] * s.lsc + p.eps;
      s.rden = __builtin_amdgcn_rcpf(s.den);
      s.eta = s.key ? s_bt[u] * s.rden : 0.f;
      s.a = 1.f - s.eta * s_lm[u] * s.lsc;
      s.b = 1.f;
    } else {
      s.key = true;
      s.lsc = 1.f;
      s.den = 1.f;
      s.rden = 1.f;
      s.b = s_bt[u];
      s.eta = s.b;
      s.a = PCX ? 1.f : s_lm[u];  // per channel the rows' retentions come from s_lc
    }
    return s;
  };
  // One forward step at token t (u within the chunk) on the registers S; for the delta
  // rule the residual replaces v in s_w[u] (read by every thread before the barrier in
  // reduce, written by row group 0 after it).
  auto fwd_tok = [&](int t, int u, f4 (&S)[RPT]) {
    const Sc s = scal(t, u);
    f4 w = *reinterpret_cast<const f4*>(&s_w[u][4 * cq]);
    if (R::solve) {
      f4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < RPT; ++j) pp += S[j] * s_x[u][row(j)];
      float d0, d1;
      w = w - reduce(pp, 0.f, 0.f, d0, d1);
      if (rg == 0) *reinterpret_cast<f4*>(&s_w[u][4 * cq]) = w;
    }
    if constexpr (PV) {  // column c decays by 1 - eta_c lambda and steps by eta_c
      const f4 e4 = s.key ? *reinterpret_cast<const f4*>(&s_bc[u][4 * cq]) * s.rden : f4{0.f, 0.f, 0.f, 0.f};
      const f4 a4 = 1.f - e4 * (s_lm[u] * s.lsc);
      const f4 ew = e4 * w;
#pragma unroll
      for (int j = 0; j < RPT; ++j) S[j] = S[j] * a4 + ew * s_x[u][row(j)];
      return;
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = S[j] * arow(s, u, j) + w * (s.eta * s_x[u][row(j)]);
  };

  // the normaliser on the thread's rows (ZN): z_t = gamma_t z_{t-1} + beta_t phi(k_t)
  float zr[RPT];
  auto zstep = [&](int u) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) zr[j] = s_lm[u] * zr[j] + s_bt[u] * s_x[u][row(j)];
  };

  // ---- forward: the state (and z) at every chunk start
  f4 S[RPT];
  load_state(p.S_in != nullptr ? p.S_in + (size_t)bh * SS : nullptr, S);
#pragma unroll
  for (int j = 0; j < RPT; ++j) zr[j] = (ZN && p.xprev_in != nullptr) ? p.xprev_in[(size_t)bh * DK + row(j)] : 0.f;
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * CK, t1 = min(T, t0 + CK);
    store_state(ckpt + (size_t)c * SS, S);
    if constexpr (ZN)
      if (cq == 0)
#pragma unroll
        for (int j = 0; j < RPT; ++j) zck[(size_t)c * DK + row(j)] = zr[j];
    stage(t0, t1, false);
    for (int t = t0; t < t1; ++t) {
      fwd_tok(t, t - t0, S);
      if constexpr (ZN) zstep(t - t0);
    }
    __syncthreads();  // LDS is restaged for the next chunk
  }

  // ---- backward
  f4 G[RPT];
  load_state(p.dS_out != nullptr ? p.dS_out + (size_t)bh * SS : nullptr, G);
  float Gz[RPT];         // ZN: dL/dz_t on the thread's rows
  float dden_pend = 0.f;  // ZN: the normaliser's gradient of the token whose read was last undone
  // the final normaliser is an output (the state's carried-key slot): its gradient starts G_z
#pragma unroll
  for (int j = 0; j < RPT; ++j) Gz[j] = (ZN && p.dz_out != nullptr) ? p.dz_out[(size_t)bh * DK + row(j)] : 0.f;
  if (R::shift && T >= 1)  // the last key is written by no step of this call
    for (int i = tid; i < DK; i += NT) p.gk[(rb + T - 1) * DK + i] = 0.f;
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * CK, t1 = min(T, t0 + CK), len = t1 - t0;
    const float* start = ckpt + (size_t)c * SS;
    // recompute the chunk's states after each token (the last one stays in S)
    stage(t0, t1, true);
    load_state(start, S);
    if constexpr (ZN) {
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        zr[j] = zck[(size_t)c * DK + row(j)];
        if (cq == 0) s_z0[row(j)] = zr[j];
      }
    }
    for (int t = t0; t < t1; ++t) {
      fwd_tok(t, t - t0, S);
      if (t + 1 < t1) store_state(cs + (size_t)(t - t0) * SS, S);
      if constexpr (ZN) {
        zstep(t - t0);
        if (cq == 0)
#pragma unroll
          for (int j = 0; j < RPT; ++j) s_z[t - t0][row(j)] = zr[j];
      }
    }
    __syncthreads();  // the residuals in s_w (and z in s_z) are read by every thread below
    if constexpr (ZN) {
      for (int u = wave; u < t1 - t0; u += NWV) {
        float d = 0.f;
        for (int i = lane; i < DK; i += 64) d += s_z[u][i] * s_q[u][i];
        d = wave_sum(d);
        if (lane == 0) s_den[u] = d + p.eps;
      }
      __syncthreads();
    }
    // the read's gradient dphi(q_t) = S_t dO_t, from the state after token t: for the
    // chunk's last token from S, for the others while token t + 1 is undone (its Sp)
    auto read_grad = [&](int t, const f4 (&St)[RPT]) {
      const int u = t - t0;
      const f4 dO = *reinterpret_cast<const f4*>(&s_do[u][4 * cq]);
      if constexpr (ZN) {
        // o = num / den with num = S_t^T q, den = z_t . q + eps: dnum = dO / den and
        // dden = -(dO . num) / den^2, so dq = S_t dnum + z_t dden
        f4 nq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) nq += St[j] * s_q[u][row(j)];
        float d0, d1;
        const f4 num = reduce(nq, 0.f, 0.f, d0, d1);
        const float rd = 1.f / s_den[u];
        const f4 m0 = dO * num;
        dden_pend = -rowsum(m0[0] + m0[1] + m0[2] + m0[3]) * rd * rd;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const f4 m = St[j] * dO;
          const float dqi = rowsum(m[0] + m[1] + m[2] + m[3]) * rd + s_z[u][row(j)] * dden_pend;
          if (cq == 0) p.gq[(rb + t) * DK + row(j)] = dqi * dphi_of(s_q[u][row(j)]);
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const f4 m = St[j] * dO;
        const float dqi = rowsum(m[0] + m[1] + m[2] + m[3]);
        if (cq == 0) p.gq[(rb + t) * DK + row(j)] = dqi * dphi_of(s_q[u][row(j)]);
      }
    };
    read_grad(t1 - 1, S);
    // Sp: the state before token t (after t - 1); nx: before t - 1
    f4 Sp[RPT];
    load_state(len >= 2 ? cs + (size_t)(len - 2) * SS : start, Sp);
    for (int t = t1 - 1; t >= t0; --t) {
      const int u = t - t0;
      const float dden_t = dden_pend;  // ZN: set when token t's read was undone
      if (u >= 1) read_grad(t - 1, Sp);
      const f4 dO = *reinterpret_cast<const f4*>(&s_do[u][4 * cq]);
      f4 nx[RPT];
      if (u >= 1) load_state(u >= 2 ? cs + (size_t)(u - 2) * SS : start, nx);
      else
#pragma unroll
        for (int j = 0; j < RPT; ++j) nx[j] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (ZN) {  // the read: G += phi(q) (dO / den)^T, G_z += phi(q) dden
        const f4 dn = dO * (1.f / s_den[u]);
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          G[j] += dn * s_q[u][row(j)];
          Gz[j] += s_q[u][row(j)] * dden_t;
        }
      } else {
#pragma unroll
        for (int j = 0; j < RPT; ++j) G[j] += dO * s_q[u][row(j)];  // the read: G += phi(q) dO^T
      }
      const Sc s = scal(t, u);
      if (!s.key) {  // no write: S_t = S_{t-1}; nothing else depends on this step
        if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = f4{0.f, 0.f, 0.f, 0.f};
        if (tid == 0) {
          if (p.gbeta != nullptr && !PV) p.gbeta[rb + t] = 0.f;
          if (p.glam != nullptr && !PCX) p.glam[rb + t] = 0.f;
        }
        if constexpr (PV)
          if (p.gbeta != nullptr && rg == 0)
            *reinterpret_cast<f4*>(p.gbeta + (rb + t) * DV + 4 * cq) = f4{0.f, 0.f, 0.f, 0.f};
        if (PCX && p.glam != nullptr)
          for (int i = tid; i < DK; i += NT) p.glam[(rb + t) * DK + i] = 0.f;
        if (p.gx0 != nullptr)
          for (int i = tid; i < DK; i += NT) p.gx0[(size_t)bh * DK + i] = 0.f;
      } else if constexpr (PV) {
        // per value column c: da_c = <G_:c, S_{t-1}:c>, deta_c = (G^T x)_c r_c - ridge da_c,
        // dr_c = eta_c (G^T x)_c; eta's shared denominator takes sum_c eta_c deta_c
        const f4 w = *reinterpret_cast<const f4*>(&s_w[u][4 * cq]);  // the residual
        f4 gx = {0.f, 0.f, 0.f, 0.f}, dap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          gx += G[j] * s_x[u][row(j)];
          dap += G[j] * Sp[j];
        }
        float d0, d1;
        const f4 gtx = reduce(gx, 0.f, 0.f, d0, d1);
        const f4 da4 = reduce(dap, 0.f, 0.f, d0, d1);
        const f4 b4 = *reinterpret_cast<const f4*>(&s_bc[u][4 * cq]);
        const f4 e4 = b4 * s.rden;
        const float ridge = s_lm[u] * s.lsc;
        const f4 a4 = 1.f - e4 * ridge;
        const f4 deta = gtx * w - da4 * ridge;
        const f4 dr = e4 * gtx;
        if (rg == 0) {
          *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = dr;
          if (p.gbeta != nullptr) {
            f4 gb;
#pragma unroll
            for (int e = 0; e < 4; ++e) gb[e] = deta[e] * s.rden * dbeta_dz(b4[e]);
            *reinterpret_cast<f4*>(p.gbeta + (rb + t) * DV + 4 * cq) = gb;
          }
        }
        const f4 ed = e4 * deta, ea = e4 * da4;
        const float dden = -rowsum(ed[0] + ed[1] + ed[2] + ed[3]) * s.rden;
        const float dlr = -rowsum(ea[0] + ea[1] + ea[2] + ea[3]) + dden;  // the ridge's gradient
        const float dxl = (p.flags & kFlagLamScaled) ? 2.f * dlr * s_lm[u] : 0.f;
        if (tid == 0 && p.glam != nullptr) p.glam[rb + t] = dlr * s.lsc * dlam_dz(s_lm[u]);
        const f4 ew = e4 * w;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const float x = s_x[u][row(j)];
          const f4 m = G[j] * ew - Sp[j] * dr;
          const float dx = rowsum(m[0] + m[1] + m[2] + m[3]) + x * (2.f * dden + dxl);
          if (cq == 0) {
            if (t >= 1) p.gk[(rb + t - 1) * DK + row(j)] = dx * dphi_of(x);
            else if (p.gx0 != nullptr) p.gx0[(size_t)bh * DK + row(j)] = dx;
          }
          G[j] = G[j] * a4 - dr * x;
        }
      } else {
        // w: the residual (delta) or the value; G w per row; <G, S_{t-1}> (per channel:
        // per row, and the ridge rules' sum of lambda_i times it), x^T G w, G^T x
        const f4 w = *reinterpret_cast<const f4*>(&s_w[u][4 * cq]);
        float gw[RPT], dar[RPT], da_p = 0.f, xgw_p = 0.f;
        f4 gx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const float x = s_x[u][row(j)];
          const f4 m = G[j] * w;
          gw[j] = rowsum(m[0] + m[1] + m[2] + m[3]);
          const f4 d = G[j] * Sp[j];
          if (PCX) {
            dar[j] = rowsum(d[0] + d[1] + d[2] + d[3]);
            if (R::nlms && cq == 0) da_p += s_lc[u][row(j)] * dar[j];
          } else {
            da_p += d[0] + d[1] + d[2] + d[3];
          }
          if (cq == 0) xgw_p += x * gw[j];
          gx += G[j] * x;
          if constexpr (ZN)  // z_t = gamma z_{t-1} + beta x: G_z joins da and x^T G w
            if (cq == 0) {
              da_p += Gz[j] * (u >= 1 ? s_z[u - 1][row(j)] : s_z0[row(j)]);
              xgw_p += Gz[j] * x;
            }
        }
        float da, xgw;  // per channel (ridge rules): da holds sum_i lambda_i da_i
        const f4 gtx = reduce(gx, da_p, xgw_p, da, xgw);
        if (R::nlms) {
          const f4 dr = gtx * s.eta;  // delta: dL/dr; inner: dL/dv
          if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = dr;
          // a = 1 - eta lambda, eta = beta / den, den = |x|^2 + lambda + eps (per channel
          // a_i = 1 - eta lambda_i and den takes the largest lambda_i, which passes the
          // denominator's gradient to the first channel holding it)
          // With the scale-coupled ridge the ridge used is lambda |x|^2 (scalar lambda): its
          // gradient dlr gives lambda's times |x|^2 and adds 2 x lambda dlr to the key's.
          const float deta = xgw - (PCX ? da : s_lm[u] * s.lsc * da);
          const float dden = -s.eta * deta * s.rden;
          const float dlr = -s.eta * da + dden;  // scalar lambda: the ridge's gradient
          const float dxl = (!PCX && (p.flags & kFlagLamScaled)) ? 2.f * dlr * s_lm[u] : 0.f;
          if (tid == 0) {
            if (p.gbeta != nullptr) p.gbeta[rb + t] = deta * s.rden * dbeta_dz(s_bt[u]);
            if (p.glam != nullptr && !PCX) p.glam[rb + t] = dlr * s.lsc * dlam_dz(s_lm[u]);
          }
          if (PCX && p.glam != nullptr && cq == 0)
#pragma unroll
            for (int j = 0; j < RPT; ++j)
              p.glam[(rb + t) * DK + row(j)] =
                  (-s.eta * dar[j] + (row(j) == s_im[u] ? dden : 0.f)) * dlam_dz(s_lc[u][row(j)]);
#pragma unroll
          for (int j = 0; j < RPT; ++j) {
            const float x = s_x[u][row(j)];
            float dx = s.eta * gw[j] + x * (2.f * dden + dxl);
            if (R::solve) {
              const f4 m = Sp[j] * dr;
              dx -= rowsum(m[0] + m[1] + m[2] + m[3]);
            }
            if (cq == 0) {
              if (t >= 1) p.gk[(rb + t - 1) * DK + row(j)] = dx * dphi_of(x);
              else if (p.gx0 != nullptr) p.gx0[(size_t)bh * DK + row(j)] = dx;
            }
            G[j] = G[j] * arow(s, u, j) - (R::solve ? dr * x : f4{0.f, 0.f, 0.f, 0.f});
          }
        } else {
          // additive: x = phi(k_t), b the write scale, a the retention
          if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = gtx * s.b;
          if (tid == 0) {
            if (p.gbeta != nullptr) p.gbeta[rb + t] = xgw * dbeta_dz(s_bt[u]);
            if (p.glam != nullptr && !PCX) p.glam[rb + t] = da * dlam_dz(s_lm[u]);
          }
#pragma unroll
          for (int j = 0; j < RPT; ++j) {
            if (cq == 0) {
              p.gk[(rb + t) * DK + row(j)] = s.b * (gw[j] + (ZN ? Gz[j] : 0.f)) * dphi_of(s_x[u][row(j)]);
              if (PCX && p.glam != nullptr) p.glam[(rb + t) * DK + row(j)] = dar[j] * dlam_dz(s_lc[u][row(j)]);
            }
            G[j] = G[j] * arow(s, u, j);
            if constexpr (ZN) Gz[j] *= s.a;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < RPT; ++j) Sp[j] = nx[j];
    }
    __syncthreads();  // LDS is restaged for the previous chunk
  }
  if (p.gS0 != nullptr) store_state(p.gS0 + (size_t)bh * SS, G);
  if (p.gh0 != nullptr && tid == 0) p.gh0[bh] = 0;
  if constexpr (ZN) {  // the initial normaliser's gradient (the carried-key slot holds z)
    if (p.gx0 != nullptr && cq == 0)
#pragma unroll
      for (int j = 0; j < RPT; ++j) p.gx0[(size_t)bh * DK + row(j)] = Gz[j];
  } else if (p.gx0 != nullptr && (!R::shift || T == 0)) {
    for (int i = tid; i < DK; i += NT) p.gx0[(size_t)bh * DK + i] = 0.f;
  }
}

// QK normalisation: the main kernel's q, k and carried-key gradients are with respect to
// the rescaled vectors y = len x / |x|; with respect to the raw x they are
// (len / |x|) (g - x (x . g) / |x|^2), zero for a zero row. One wave per vector: the q
// rows, then the k rows, then the carried keys.
template <typename InT, int DK>
__global__ __launch_bounds__(256) void qk_norm_bwd_kernel(BwdParams p, float len) {
  constexpr int E = DK / 64;
  const int lane = threadIdx.x & 63;
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t nrow = (size_t)p.BH * (size_t)p.T;
  // the carried-key slot holds z with the normaliser: no key rows then
  const size_t nkey = (p.gx0 != nullptr && p.xprev_in != nullptr && !(p.flags & kFlagZnorm)) ? (size_t)p.BH : 0;
  if (r >= 2 * nrow + nkey) return;
  float x[E], g[E];
  float* gp;
  if (r < 2 * nrow) {
    const InT* src = static_cast<const InT*>(r < nrow ? p.q : p.k) + (r % nrow) * DK;
    gp = (r < nrow ? p.gq : p.gk) + (r % nrow) * DK;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = In<InT>::load1(src + lane + 64 * e);
  } else {
    const size_t b = r - 2 * nrow;
    gp = p.gx0 + b * DK;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = p.xprev_in[b * DK + lane + 64 * e];
  }
  float xx = 0.f, xg = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    g[e] = gp[lane + 64 * e];
    xx += x[e] * x[e];
    xg += x[e] * g[e];
  }
  xx = wave_sum(xx);
  xg = wave_sum(xg);
  const float f = rescale_factor(xx, len), c = xx > 0.f ? xg / xx : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) gp[lane + 64 * e] = f * (g[e] - x[e] * c);
}

template <typename InT, int DK, int DV, bool PCX>
hipError_t launch_pc(const BwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)p.BH), block(NT);
  if (p.rule == kRuleDelta) hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleDelta, PCX, false>), grid, block, 0, st, p);
  else if (!PCX && p.rule == kRuleDeltaPV)
    hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleDeltaPV, false, false>), grid, block, 0, st, p);
  else if (p.rule == kRuleInner) hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleInner, PCX, false>), grid, block, 0, st, p);
  else if (!PCX && (p.flags & kFlagZnorm))
    hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleAdditive, false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleAdditive, PCX, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

template <typename InT, int DK>
hipError_t launch_qk(const BwdParams& p, hipStream_t st) {
  const float len = qk_length(p.flags, DK);
  if (len <= 0.f) return hipSuccess;
  const size_t rows = 2 * (size_t)p.BH * (size_t)p.T +
                      ((p.gx0 != nullptr && p.xprev_in != nullptr && !(p.flags & kFlagZnorm)) ? p.BH : 0);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((qk_norm_bwd_kernel<InT, DK>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, p, len);
  return hipGetLastError();
}

template <typename InT, int DK, int DV>
hipError_t launch_t(const BwdParams& p, hipStream_t st) {
  const hipError_t e =
      (p.flags & kFlagPerChannel) ? launch_pc<InT, DK, DV, true>(p, st) : launch_pc<InT, DK, DV, false>(p, st);
  if (e != hipSuccess) return e;
  return launch_qk<InT, DK>(p, st);
}

template <typename InT>
hipError_t launch_in(const BwdParams& p, hipStream_t st) {
  if (p.dk == 64 && p.dv == 64) return launch_t<InT, 64, 64>(p, st);
  if (p.dk == 64 && p.dv == 128) return launch_t<InT, 64, 128>(p, st);
  if (p.dk == 128 && p.dv == 64) return launch_t<InT, 128, 64>(p, st);
  return launch_t<InT, 128, 128>(p, st);
}

}  // namespace

bool bwd_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

hipError_t launch_bwd(const BwdParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  return p.bf16 ? launch_in<uint16_t>(p, st) : launch_in<float>(p, st);
}

hipError_t launch_qk_norm_bwd(const BwdParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  if (p.bf16) return p.dk == 64 ? launch_qk<uint16_t, 64>(p, st) : launch_qk<uint16_t, 128>(p, st);
  return p.dk == 64 ? launch_qk<float, 64>(p, st) : launch_qk<float, 128>(p, st);
}

}  // namespace fwmem
