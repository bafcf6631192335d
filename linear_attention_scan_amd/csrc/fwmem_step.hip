// One-token recurrent decode for gfx950: a pure stream of the fp32 state.
//
// Per head (delta rule, "Fast Weight Attention for Continual Learning" reading
// notes, sections 3.2 and 4.1):
//   x = x_prev (if a previous key exists, else 0)
//   eta = beta / (||x||^2 + lambda_hat + eps)  (0 without a previous key)
//   r = v - S^T x
//   S' = diag(a) S + eta x r^T,  a = 1 - eta lambda   (scalar or per key channel)
//   o = S'^T q~ = S^T (a o q~) + eta (x . q~) r
// so one read of S yields both column reductions (S^T x and S^T (a o q~)) and the
// state is written back from registers: exactly one read and one write of S.
// Additive rule ("attention is also an FFN", section 3.2):
//   S' = diag(gamma) S + b phi(k) v^T,  o = S^T (gamma o q~) + b (phi(k) . q~) v.
// With the normaliser (FWMEM_ZNORM, the same page, section 4.2) the state's x_prev slot
// holds z: z' = gamma o z + b phi(k), and o is divided by z' . q~ + eps.
// Inner-product rule (the reading notes above, section 4.3): x, eta and a as for the
// delta rule, with the value itself written: S' = diag(a) S + eta x v^T,
//   o = S^T (a o q~) + eta (x . q~) v.
//
// Layout: one 1024-thread workgroup per head. Thread (rg, cq) owns float4 column
// group cq (4 value columns) of rows rg, rg + RG, ... (four rows at d_k = d_v = 128);
// a wave's 16-byte loads cover whole rows of S, so every access is a coalesced
// 128-bit load or store. Sixteen waves per head keep few loads per lane in flight
// and the whole 64 KiB state of a head moving at once; measured on the
// B=256 H=32 d=128 decode, this streams about 10% faster than 256 threads.
#include "fwmem_device.h"
#include "fwmem_internal.h"

namespace fwmem {

namespace {

constexpr int NT = 1024;

template <typename InT, int DK, int DV, int RULE, bool PC>
__global__ __launch_bounds__(NT) void step_kernel(StepParams p) {
  using R = Rule<RULE>;
  constexpr int TPRd = DV / 4;       // threads per row (float4 each)
  constexpr int RG = NT / TPRd;      // row groups
  constexpr int RPT = DK / RG;       // rows per thread
  constexpr int RGW = 64 / TPRd;     // row groups per wave
  constexpr int NWV = NT / 64;
  static_assert(DK % RG == 0 && RGW >= 1, "shape");

  __shared__ float s_x[DK], s_q[DK], s_a[DK], s_k[DK], s_z[DK];
  __shared__ float s_red[2][NWV][DV];
  __shared__ float s_sc[8];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % TPRd, rg = tid / TPRd;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const bool znorm = !R::solve && !R::shift && (p.flags & kFlagZnorm) != 0;
  // per-value-channel rule: eta_j = beta_j / den and the decay 1 - eta_j lambda act on
  // the columns; the rows carry no decay
  constexpr bool PV = RULE == kRuleDeltaPV;
  const InT* qp = static_cast<const InT*>(p.q) + (size_t)bh * DK;
  const InT* kp = static_cast<const InT*>(p.k) + (size_t)bh * DK;
  const InT* vp = static_cast<const InT*>(p.v) + (size_t)bh * DV;
  const bool has = p.has_in != nullptr && p.has_in[bh] != 0;

  // Issue the state loads first: they are the whole cost of the step.
  f4 S[RPT];
  const float* Sin = p.S_in != nullptr ? p.S_in + (size_t)bh * DK * DV : nullptr;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    S[j] = Sin != nullptr
               ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(Sin + (size_t)row * DV) + cq)
               : f4{0.f, 0.f, 0.f, 0.f};
  }

  // Per-head vectors into LDS. The carried key for the next token is phi(k), stored raw
  // (before any normalisation), or with the normaliser z' (below); each thread reads its
  // own x_prev entries before it writes them, so the state may be updated in place.
  const float qk_len = qk_length(p.flags, DK);
  for (int i = tid; i < DK; i += NT) {
    float q = In<InT>::load1(qp + i);
    float k = In<InT>::load1(kp + i);
    if (elu) { q = phi_elu1(q); k = phi_elu1(k); }
    s_q[i] = q;
    s_k[i] = k;
    s_x[i] = (R::shift && has && p.xprev_in != nullptr) ? p.xprev_in[(size_t)bh * DK + i] : 0.f;
    if (znorm) s_z[i] = p.xprev_in != nullptr ? p.xprev_in[(size_t)bh * DK + i] : 0.f;
    else p.xprev_out[(size_t)bh * DK + i] = k;
  }
  __syncthreads();

  // Scalars: ||x||^2, max lambda (per channel), x.q or k.q; wave 0 reduces. With
  // normalised queries and keys, x and q are rescaled by mx and mq (to length qk_len).
  if (wave == 0) {
    float nx = 0.f, dq = 0.f, lm = lam_max_init(p.flags), nq = 0.f;
    for (int i = lane; i < DK; i += 64) {
      const float xi = R::shift ? s_x[i] : s_k[i];
      nx += xi * xi;
      dq += xi * s_q[i];
      nq += s_q[i] * s_q[i];
      if (PC && p.lam != nullptr) lm = fmaxf(lm, p.lam[(size_t)bh * DK + i]);
    }
    nx = wave_sum(nx);
    dq = wave_sum(dq);
    nq = wave_sum(nq);
    lm = wave_max(lm);
    if (PC && p.lam != nullptr) lm = act_lam(lm, p.flags, true);  // monotonic: max commutes
    float mx = 1.f, mq = 1.f;
    if (qk_len > 0.f) {
      mx = rescale_factor(nx, qk_len);
      mq = rescale_factor(nq, qk_len);
      nx *= mx * mx;
      dq *= mx * mq;
    }
    if (lane == 0) {
      float eta = 0.f, a = 1.f;
      if (R::nlms) {
        // with the scale-coupled ridge, lambda is a base ridge times the key energy nx
        const float es = (p.flags & kFlagLamScaled) ? nx : 1.f;
        const float lam = es * (PC ? (p.lam != nullptr ? lm : 0.f)
                                   : (p.lam != nullptr ? act_lam(p.lam[bh], p.flags, true) : 0.f));
        s_sc[6] = es;
        if (PV) {
          eta = has ? 1.f / (nx + lam + p.eps) : 0.f;  // times each column's beta below
          a = lam;
        } else {
          if (has) eta = act_beta(p.beta[bh], p.flags) / (nx + lam + p.eps);
          a = 1.f - eta * lam;
        }
      } else {
        eta = p.beta != nullptr ? act_beta(p.beta[bh], p.flags) : 1.f;  // write scale
        a = (!PC && p.lam != nullptr) ? act_lam(p.lam[bh], p.flags, false) : 1.f;
      }
      s_sc[0] = eta;
      s_sc[1] = a;
      s_sc[2] = dq;
      s_sc[3] = mx;
      s_sc[4] = mq;
    }
  }
  __syncthreads();
  const float eta = s_sc[0], a_sc = s_sc[1], dq = s_sc[2];
  for (int i = tid; i < DK; i += NT) {
    if (qk_len > 0.f) {
      s_q[i] *= s_sc[4];
      if (R::shift) s_x[i] *= s_sc[3];
      else s_k[i] *= s_sc[3];
    }
    float a = PV ? 1.f : a_sc;
    if (PC) {
      const float lam = p.lam != nullptr ? act_lam(p.lam[(size_t)bh * DK + i], p.flags, R::nlms) : (R::nlms ? 0.f : 1.f);
      a = R::nlms ? 1.f - eta * s_sc[6] * lam : lam;
    }
    s_a[i] = a;
    if (znorm) {
      const float zn = a * s_z[i] + eta * s_k[i];
      s_z[i] = zn;
      p.xprev_out[(size_t)bh * DK + i] = zn;
    }
  }
  __syncthreads();
  if (znorm && wave == NWV - 1) {
    float d = 0.f;
    for (int i = lane; i < DK; i += 64) d += s_z[i] * s_q[i];
    d = wave_sum(d);
    if (lane == 0) s_sc[5] = 1.f / (d + p.eps);
  }

  // Column partial sums over this thread's rows: p = S^T x, w = S^T (a o q).
  f4 pp = {0.f, 0.f, 0.f, 0.f}, ww = pp;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    const float xi = s_x[row], aq = s_a[row] * s_q[row];
    pp += S[j] * xi;
    ww += S[j] * aq;
  }
  // reduce over the row groups inside the wave (lanes cq, cq + TPRd, ...)
#pragma unroll
  for (int o = TPRd; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[e] += __shfl_xor(pp[e], o);
      ww[e] += __shfl_xor(ww[e], o);
    }
  }
  if (lane < TPRd) {
    *reinterpret_cast<f4*>(&s_red[0][wave][4 * cq]) = pp;
    *reinterpret_cast<f4*>(&s_red[1][wave][4 * cq]) = ww;
  }
  __syncthreads();
  f4 P = {0.f, 0.f, 0.f, 0.f}, W = P;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    P += *reinterpret_cast<const f4*>(&s_red[0][w][4 * cq]);
    W += *reinterpret_cast<const f4*>(&s_red[1][w][4 * cq]);
  }

  float v4[4];
  {
    const int c = 4 * cq;
#pragma unroll
    for (int e = 0; e < 4; ++e) v4[e] = In<InT>::load1(vp + c + e);
  }
  // r (delta) or the written value b*v (additive), and the output.
  const f4 vv = {v4[0], v4[1], v4[2], v4[3]};
  f4 r, o, a4 = {1.f, 1.f, 1.f, 1.f};
  if constexpr (PV) {
    f4 e4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      e4[e] = act_beta(p.beta[(size_t)bh * DV + 4 * cq + e], p.flags) * eta;
      a4[e] = 1.f - e4[e] * a_sc;
    }
    r = (vv - P) * e4;
    o = W * a4 + r * dq;  // W = S^T q here
  } else {
    r = R::solve ? (vv - P) * eta : vv * eta;  // the written value u
    o = znorm ? (W + r * dq) * s_sc[5] : W + r * dq;
  }

  // New state from registers.
  float* Sout = p.S_out + (size_t)bh * DK * DV;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    const float a = s_a[row];
    const float xi = R::shift ? s_x[row] : s_k[row];
    const f4 n4 = PV ? S[j] * a4 + r * xi : S[j] * a + r * xi;
    __builtin_nontemporal_store(n4, reinterpret_cast<f4*>(Sout + (size_t)row * DV) + cq);
  }
  if (rg == 0) {
    const size_t ob = (size_t)bh * DV + 4 * cq;
    if (p.flags & kFlagOutBf16) {
      uint16_t* op = static_cast<uint16_t*>(p.out) + ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) op[e] = f32_to_bf16_bits(o[e]);
    } else {
      *reinterpret_cast<f4*>(static_cast<float*>(p.out) + ob) = o;
    }
  }
  if (tid == 0) p.has_out[bh] = 1;
}

template <typename InT, int DK, int DV>
hipError_t launch_t(const StepParams& p, hipStream_t st) {
  const bool pc = (p.flags & kFlagPerChannel) != 0;
  const dim3 grid(p.BH), block(NT);
  if (p.rule == kRuleDelta) {
    if (pc) hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleDelta, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleDelta, false>), grid, block, 0, st, p);
  } else if (p.rule == kRuleDeltaPV) {
    hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleDeltaPV, false>), grid, block, 0, st, p);
  } else if (p.rule == kRuleInner) {
    if (pc) hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleInner, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleInner, false>), grid, block, 0, st, p);
  } else {
    if (pc) hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleAdditive, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((step_kernel<InT, DK, DV, kRuleAdditive, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

template <typename InT>
hipError_t launch_in(const StepParams& p, hipStream_t st) {
  if (p.dk == 64 && p.dv == 64) return launch_t<InT, 64, 64>(p, st);
  if (p.dk == 64 && p.dv == 128) return launch_t<InT, 64, 128>(p, st);
  if (p.dk == 128 && p.dv == 64) return launch_t<InT, 128, 64>(p, st);
  return launch_t<InT, 128, 128>(p, st);
}

}  // namespace

bool step_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

hipError_t launch_step(const StepParams& p, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  return p.bf16 ? launch_in<uint16_t>(p, st) : launch_in<float>(p, st);
}

}  // namespace fwmem
