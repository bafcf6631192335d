// Backward pass of the scan: the gradients of L = <dO, o> + <dS_T, S_T> with respect to
// q, k, v, beta, lambda, the initial state S0 and the carried key, for the delta, inner and
// additive rules with phi identity or elu+1 and a scalar lambda. The pages give no backward
// pass; this is the reverse-mode derivative of the recurrence as the forward pass states it
// ("Fast Weight Attention for Continual Learning" reading notes, sections 3.2, 4.1-4.3;
// "attention is also an FFN", sections 2.1, 3.2):
//   S_t = a_t S_{t-1} + eta_t x_t w_t^T,  o_t = S_t^T phi(q_t),
// with w_t = v_t - S_{t-1}^T x_t (delta) or v_t (inner, additive), and for the delta and inner
// rules a_t = 1 - eta_t lambda_t, eta_t = beta_t / (|x_t|^2 + lambda_t + eps), x_t = phi(k_{t-1}).
// Undoing step t with G = dL/dS_t:
//   dphi(q_t) = S_t dO_t;  G += phi(q_t) dO_t^T;  da = <G, S_{t-1}>;
//   delta:    deta = x^T G r, dr = eta G^T x, dx = eta G r - S_{t-1} dr, dv = dr,
//             G_{t-1} = a G - x dr^T
//   inner:    deta = x^T G v, dx = eta G v, dv = eta G^T x, G_{t-1} = a G
//   additive: dgamma = da, dbeta = k^T G v, dphi(k) = beta G v, dv = beta G^T phi(k),
//             G_{t-1} = gamma G
// and for the shifted rules the scalar chain through a, eta and the denominator.
//
// One persistent 1024-thread workgroup per head, token-serial (a first, simple form; the
// chunked backward is future work). The state is distributed as in the decode kernel:
// thread (rg, cq) holds float4 column group cq of rows rg, rg + RG, ... A forward pass
// stores the state at every chunk start; then, per chunk from the last, the chunk's states
// after each token are recomputed into the workspace and the chunk's tokens are undone
// from the last.
#include "fwmem_backward.h"
#include "fwmem_device.h"
#include "fwmem_internal.h"

namespace fwmem {
namespace {

constexpr int NT = 1024;
constexpr int NWV = NT / 64;
constexpr int CH = kChunk;

template <typename InT, int DK, int DV, int RULE>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  using R = Rule<RULE>;
  constexpr int TPRd = DV / 4;   // threads per row
  constexpr int RG = NT / TPRd;  // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(DK % RG == 0 && RPT >= 1, "shape");
  __shared__ float s_x[DK], s_q[DK], s_w[DV];
  __shared__ float s_col[NWV][DV];
  __shared__ float s_sum[NWV][2];
  __shared__ float s_eta[CH], s_a[CH], s_den[CH], s_b[CH];
  __shared__ float s_n;

  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % TPRd, rg = tid / TPRd;
  const int T = p.T;
  const bool elu = (p.flags & kFlagPhiElu1) != 0;
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  const size_t rb = (size_t)bh * T;
  const InT* qb = static_cast<const InT*>(p.q) + rb * DK;
  const InT* kb = static_cast<const InT*>(p.k) + rb * DK;
  const InT* vb = static_cast<const InT*>(p.v) + rb * DV;
  const size_t SS = (size_t)DK * DV;
  float* ckpt = p.ws + (size_t)bh * bwd_floats_per_head(T, DK, DV);
  float* cs = ckpt + (size_t)p.nchunks * SS;  // [CH] states after each token of a chunk
  float* rr = cs + (size_t)CH * SS;           // [CH][DV] residuals of the chunk (delta)

  auto phi = [&](float x) { return elu ? phi_elu1(x) : x; };
  auto dphi = [&](float x) { return elu ? (x > 0.f ? 1.f : __expf(x)) : 1.f; };
  auto row = [&](int j) { return rg + RG * j; };

  // sum over the row groups of a per-thread float4 (the thread's four columns)
  auto colsum = [&](f4 v) -> f4 {
#pragma unroll
    for (int o = TPRd; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], o);
    if (lane < TPRd) *reinterpret_cast<f4*>(&s_col[wave][4 * cq]) = v;
    __syncthreads();
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w) s += *reinterpret_cast<const f4*>(&s_col[w][4 * cq]);
    __syncthreads();
    return s;
  };
  // sum over a row's TPRd consecutive lanes
  auto rowsum = [&](float v) -> float {
#pragma unroll
    for (int o = 1; o < TPRd; o <<= 1) v += __shfl_xor(v, o);
    return v;
  };
  // sums over the whole workgroup of two values
  auto fullsum2 = [&](float a, float b, float& sa, float& sb) {
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
      s_sum[wave][0] = a;
      s_sum[wave][1] = b;
    }
    __syncthreads();
    sa = 0.f;
    sb = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      sa += s_sum[w][0];
      sb += s_sum[w][1];
    }
    __syncthreads();
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
  auto load_v = [&](int t) -> f4 {
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = In<InT>::load1(vb + (size_t)t * DV + 4 * cq + e);
    return v;
  };
  // x_t into s_x (the written key), then its squared norm into s_n
  auto stage_x = [&](int t) {
    for (int i = tid; i < DK; i += NT) {
      float x = 0.f;
      if (R::shift) {
        if (t >= 1) x = phi(In<InT>::load1(kb + (size_t)(t - 1) * DK + i));
        else if (has_in && p.xprev_in != nullptr) x = p.xprev_in[(size_t)bh * DK + i];
      } else {
        x = phi(In<InT>::load1(kb + (size_t)t * DK + i));
      }
      s_x[i] = x;
    }
    __syncthreads();
    if (wave == 0) {
      float n = 0.f;
      for (int i = lane; i < DK; i += 64) n += s_x[i] * s_x[i];
      n = wave_sum(n);
      if (lane == 0) s_n = n;
    }
    __syncthreads();
  };
  // one forward step at token t (u = t within its chunk), recording eta, a, den, beta
  auto fwd_step = [&](int t, int u, f4 (&S)[RPT]) {
    stage_x(t);
    float eta, a, den = 1.f, b = 1.f;
    if (R::nlms) {
      const bool key = t >= 1 || has_in;
      const float lam = p.lam != nullptr ? p.lam[rb + t] : 0.f;
      den = s_n + lam + p.eps;
      eta = key ? p.beta[rb + t] / den : 0.f;
      a = 1.f - eta * lam;
    } else {
      b = p.beta != nullptr ? p.beta[rb + t] : 1.f;
      eta = b;
      a = p.lam != nullptr ? p.lam[rb + t] : 1.f;
    }
    if (tid == 0) {
      s_eta[u] = eta;
      s_a[u] = a;
      s_den[u] = den;
      s_b[u] = b;
    }
    f4 w = load_v(t);
    if (R::solve) {
      f4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < RPT; ++j) pp += S[j] * s_x[row(j)];
      w = w - colsum(pp);
      if (rg == 0) *reinterpret_cast<f4*>(rr + (size_t)u * DV + 4 * cq) = w;
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = S[j] * a + w * (eta * s_x[row(j)]);
    __syncthreads();  // s_x is restaged by the next step
  };

  // ---- forward: the state at every chunk start
  f4 S[RPT];
  load_state(p.S_in != nullptr ? p.S_in + (size_t)bh * SS : nullptr, S);
  for (int c = 0; c < p.nchunks; ++c) {
    store_state(ckpt + (size_t)c * SS, S);
    const int t1 = min(T, (c + 1) * CH);
    for (int t = c * CH; t < t1; ++t) fwd_step(t, t - c * CH, S);
  }
  __syncthreads();

  // ---- backward
  f4 G[RPT];
  load_state(p.dS_out != nullptr ? p.dS_out + (size_t)bh * SS : nullptr, G);
  if (R::shift && T >= 1)  // the last key is written by no step of this call
    for (int i = tid; i < DK; i += NT) p.gk[(rb + T - 1) * DK + i] = 0.f;
  for (int c = p.nchunks - 1; c >= 0; --c) {
    const int t0 = c * CH, t1 = min(T, t0 + CH);
    // recompute the chunk's states after each token (and its scalars and residuals)
    load_state(ckpt + (size_t)c * SS, S);
    __threadfence_block();
    for (int t = t0; t < t1; ++t) {
      fwd_step(t, t - t0, S);
      store_state(cs + (size_t)(t - t0) * SS, S);
    }
    __threadfence_block();
    __syncthreads();
    for (int t = t1 - 1; t >= t0; --t) {
      const int u = t - t0;
      f4 St[RPT], Sp[RPT];
      load_state(cs + (size_t)u * SS, St);
      load_state(u > 0 ? cs + (size_t)(u - 1) * SS : ckpt + (size_t)c * SS, Sp);
      stage_x(t);
      for (int i = tid; i < DK; i += NT) s_q[i] = phi(In<InT>::load1(qb + (size_t)t * DK + i));
      __syncthreads();
      f4 dO;
#pragma unroll
      for (int e = 0; e < 4; ++e) dO[e] = p.dout[(rb + t) * DV + 4 * cq + e];
      // the read: dphi(q) = S_t dO, G += phi(q) dO^T
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const f4 m = St[j] * dO;
        const float dqi = rowsum(m[0] + m[1] + m[2] + m[3]);
        if (cq == 0) p.gq[(rb + t) * DK + row(j)] = dqi * dphi(In<InT>::load1(qb + (size_t)t * DK + row(j)));
        G[j] += dO * s_q[row(j)];
      }
      const float eta = s_eta[u], a = s_a[u], den = s_den[u], b = s_b[u];
      const bool key = !R::shift || t >= 1 || has_in;
      if (!key) {  // no write: S_t = S_{t-1}; nothing else depends on this step
        if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = f4{0.f, 0.f, 0.f, 0.f};
        if (tid == 0) {
          if (p.gbeta != nullptr) p.gbeta[rb + t] = 0.f;
          if (p.glam != nullptr) p.glam[rb + t] = 0.f;
        }
        for (int i = tid; i < DK; i += NT)
          if (p.gx0 != nullptr) p.gx0[(size_t)bh * DK + i] = 0.f;
        __syncthreads();
        continue;
      }
      // w: the residual (delta) or the value; G w per row; <G, S_{t-1}> and x^T G w
      const f4 w = R::solve ? *reinterpret_cast<const f4*>(rr + (size_t)u * DV + 4 * cq) : load_v(t);
      float gw[RPT], da_p = 0.f, xgw_p = 0.f;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const f4 m = G[j] * w;
        gw[j] = rowsum(m[0] + m[1] + m[2] + m[3]);
        const f4 d = G[j] * Sp[j];
        da_p += d[0] + d[1] + d[2] + d[3];
        if (cq == 0) xgw_p += s_x[row(j)] * gw[j];
      }
      float da, xgw;
      fullsum2(da_p, xgw_p, da, xgw);
      if (R::nlms) {
        // G^T x (columns), then dx per row
        f4 gx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) gx += G[j] * s_x[row(j)];
        const f4 gtx = colsum(gx);
        const f4 dr = gtx * eta;  // delta: dr; inner: dv
        float dxv[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          dxv[j] = eta * gw[j];
          if (R::solve) {
            const f4 m = Sp[j] * dr;
            dxv[j] -= rowsum(m[0] + m[1] + m[2] + m[3]);
          }
        }
        if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = dr;
        // a = 1 - eta lambda, eta = beta / den, den = |x|^2 + lambda + eps
        const float lam = p.lam != nullptr ? p.lam[rb + t] : 0.f;
        const float deta = xgw - lam * da;
        const float dden = -eta * deta / den;
        if (tid == 0) {
          if (p.gbeta != nullptr) p.gbeta[rb + t] = deta / den;
          if (p.glam != nullptr) p.glam[rb + t] = -eta * da + dden;
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          if (cq == 0) {
            const float dx = dxv[j] + 2.f * s_x[row(j)] * dden;
            if (t >= 1) p.gk[(rb + t - 1) * DK + row(j)] = dx * dphi(In<InT>::load1(kb + (size_t)(t - 1) * DK + row(j)));
            else if (p.gx0 != nullptr) p.gx0[(size_t)bh * DK + row(j)] = dx;
          }
          G[j] = G[j] * a - (R::solve ? dr * s_x[row(j)] : f4{0.f, 0.f, 0.f, 0.f});
        }
      } else {
        // additive: x is phi(k_t), b the write scale, a the retention
        f4 gx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) gx += G[j] * s_x[row(j)];
        const f4 gtx = colsum(gx);
        if (rg == 0) *reinterpret_cast<f4*>(p.gv + (rb + t) * DV + 4 * cq) = gtx * b;
        if (tid == 0) {
          if (p.gbeta != nullptr) p.gbeta[rb + t] = xgw;
          if (p.glam != nullptr) p.glam[rb + t] = da;
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          if (cq == 0) p.gk[(rb + t) * DK + row(j)] = b * gw[j] * dphi(In<InT>::load1(kb + (size_t)t * DK + row(j)));
          G[j] = G[j] * a;
        }
      }
      __syncthreads();  // s_x, s_q are restaged by the next token
    }
  }
  if (p.gS0 != nullptr) store_state(p.gS0 + (size_t)bh * SS, G);
  if (p.gh0 != nullptr && tid == 0) p.gh0[bh] = 0;
  if (!R::shift && p.gx0 != nullptr)
    for (int i = tid; i < DK; i += NT) p.gx0[(size_t)bh * DK + i] = 0.f;
  if (R::shift && T == 0 && p.gx0 != nullptr)
    for (int i = tid; i < DK; i += NT) p.gx0[(size_t)bh * DK + i] = 0.f;
}

template <typename InT, int DK, int DV>
hipError_t launch_t(const BwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)p.BH), block(NT);
  if (p.rule == kRuleDelta) hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleDelta>), grid, block, 0, st, p);
  else if (p.rule == kRuleInner) hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleInner>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((bwd_kernel<InT, DK, DV, kRuleAdditive>), grid, block, 0, st, p);
  return hipGetLastError();
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

}  // namespace fwmem
