// Segment-parallel scan: the set-up, combine and fix-up kernels (see SegParams in
// fwmem_internal.h). The split of a long sequence into segments whose maps compose
// is the scan's own linearity: the write S_t = (diag(a_t) - eta_t x_t x_t^T) S_{t-1}
// + eta_t x_t v_t^T (delta rule; "Fast Weight Attention for Continual Learning"
// reading notes, sections 3.2 and 4.2), and its additive and inner-product forms, are
// affine in S, so a segment maps its start state S to A S + B. For the additive rule
// with a scalar decay ("attention is also an FFN", section 3.2) A is the product of the
// segment's retentions times the identity.
#include "fwmem_device.h"
#include "fwmem_internal.h"
#include "fwmem_split.h"

namespace fwmem {
namespace {

constexpr int NTH = 256;

// Virtual initial states. Local pass: the caller's state for segment 0, zero for the
// others. Transition pass: the identity. Both carry the same key: the caller's for
// segment 0, the last (raw, or elu+1 of the raw) key of the previous segment for p >= 1.
template <typename InT>
__global__ __launch_bounds__(NTH) void seg_init_kernel(SegParams s) {
  const int vh = blockIdx.x, h = vh / s.P, p = vh % s.P;
  const int dk = s.dk, dv = s.dv;
  const bool elu = (s.flags & kFlagPhiElu1) != 0;
  float* B = s.B0_S + (size_t)vh * dk * dv;
  float* A = s.A0_S + (size_t)vh * dk * dk;
  const float* Sin = (p == 0 && s.S_in != nullptr) ? s.S_in + (size_t)h * dk * dv : nullptr;
  for (int e = threadIdx.x; e < dk * dv; e += NTH) B[e] = Sin != nullptr ? Sin[e] : 0.f;
  if (!s.diag)
    for (int e = threadIdx.x; e < dk * dk; e += NTH) A[e] = (e / dk == e % dk) ? 1.f : 0.f;
  const InT* kprev = static_cast<const InT*>(s.k) + ((size_t)vh * s.L - 1) * dk;  // p >= 1 only
  for (int i = threadIdx.x; i < dk; i += NTH) {
    float x = 0.f;
    if (p > 0) {
      x = In<InT>::load1(kprev + i);
      if (elu) x = phi_elu1(x);
    } else if (s.S_in != nullptr) {
      x = s.xprev_in[(size_t)h * dk + i];
    }
    s.B0_x[(size_t)vh * dk + i] = x;
    if (!s.diag) s.A0_x[(size_t)vh * dk + i] = x;
  }
  if (threadIdx.x == 0) {
    const int has = p > 0 ? 1 : (s.S_in != nullptr && s.has_in[h] != 0 ? 1 : 0);
    s.B0_h[vh] = has;
    if (!s.diag) s.A0_h[vh] = has;
  }
}

// Diagonal transitions: gam[vh][t] = product of the retentions of the segment's tokens
// 0..t, as a running product over chunks of 256 tokens (one token per thread, a prefix
// product inside each wave, then across the four waves). A product that underflows
// stands for a start state the segment has forgotten.
__global__ __launch_bounds__(NTH) void seg_decay_kernel(SegParams s) {
  const size_t vh = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float wtot[NTH / 64];
  const float* lam = s.lam != nullptr ? s.lam + vh * s.L : nullptr;
  float* gam = s.gam + vh * s.L;
  float carry = 1.f;
  for (int base = 0; base < s.L; base += NTH) {
    const int t = base + threadIdx.x;
    float g = 1.f;
    if (t < s.L && lam != nullptr) g = act_lam(lam[t], s.flags, false);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(g, o);
      if (lane >= o) g *= u;
    }
    if (lane == 63) wtot[wave] = g;
    __syncthreads();
    float pre = carry;
    for (int w = 0; w < wave; ++w) pre *= wtot[w];
    g *= pre;
    if (t < s.L) gam[t] = g;
    float tot = carry;
    for (int w = 0; w < NTH / 64; ++w) tot *= wtot[w];
    carry = tot;
    __syncthreads();  // wtot is rewritten next round
  }
}

// C += A B for a 16x16x16 block on fp32 MFMA: lane (g, n) supplies A[n][4g..4g+3] and
// B[4g+q][n] (the C layout of a previous product); MFMA q sums over K = 4g + q.
__device__ __forceinline__ void mma_f32_block(f4& acc, const f4& a, const f4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], acc, 0, 0, 0);
}

// Writes of the combine's last step: the caller's final state, carried key and flag.
__device__ __forceinline__ void combine_final_extras(const SegParams& s, int h, int j0) {
  if (j0 == 0) {
    const size_t last = (size_t)h * s.P + s.P - 1;
    if ((s.flags & kFlagZnorm) == 0)  // with the normaliser the slot holds z
      for (int i = threadIdx.x; i < s.dk; i += NTH) s.xprev_out[(size_t)h * s.dk + i] = s.B1_x[last * s.dk + i];
    if (threadIdx.x == 0) s.has_out[h] = 1;
  }
}

// Diagonal transitions: S_start(p+1) = Gamma_p S_start(p) + B_p, Gamma_p the segment's last
// gam; every element on its own, one thread per element of the 16-column tile.
__device__ void combine_diagonal(const SegParams& s, int h, int j0) {
  const int dk = s.dk, dv = s.dv;
  const int j = threadIdx.x & 15, i0 = threadIdx.x >> 4;  // rows i0, i0 + 16, ...
  const int RP = dk / 16;
  float v[8];
  const float* B0 = s.B1_S + (size_t)(h * s.P) * dk * dv;
  for (int r = 0; r < RP; ++r) v[r] = B0[(size_t)(i0 + 16 * r) * dv + j0 + j];
  for (int p = 1; p < s.P; ++p) {
    const size_t vh = (size_t)h * s.P + p;
    float* St = s.S_start + vh * dk * dv;
    const float* Bm = s.B1_S + vh * dk * dv;
    const float gp = s.gam[vh * s.L + s.L - 1];
    for (int r = 0; r < RP; ++r) {
      St[(size_t)(i0 + 16 * r) * dv + j0 + j] = v[r];
      v[r] = gp * v[r] + Bm[(size_t)(i0 + 16 * r) * dv + j0 + j];
    }
  }
  if (s.S_out != nullptr) {
    for (int r = 0; r < RP; ++r) s.S_out[((size_t)h * dk + i0 + 16 * r) * dv + j0 + j] = v[r];
    combine_final_extras(s, h, j0);
  }
}

// General transitions: S_start(p+1) = A_p S_start(p) + B_p, a [d_k x d_k] x [d_k x 16]
// product per segment on fp32 MFMA. Wave w owns row tiles w, w + 4 of the tile in C layout;
// the current start state goes through LDS so that every wave reads all of it as B
// fragments.
template <int DK>
__device__ void combine_general(const SegParams& s, int h, int j0) {
  constexpr int NRT = DK / 16, RPW = (NRT + 3) / 4;
  __shared__ float cur[DK * 16];
  const int dv = s.dv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  f4 v[RPW];
  const float* B0 = s.B1_S + (size_t)(h * s.P) * DK * dv;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rt = wave + 4 * r;
    if (rt < NRT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[r][i] = B0[(size_t)(16 * rt + 4 * g + i) * dv + j0 + n];
        cur[(16 * rt + 4 * g + i) * 16 + n] = v[r][i];
      }
    }
  }
  __syncthreads();
  for (int p = 1; p < s.P; ++p) {
    const size_t vh = (size_t)h * s.P + p;
    float* St = s.S_start + vh * DK * dv;
    const float* A = s.A1_S + vh * DK * DK;
    const float* Bm = s.B1_S + vh * DK * dv;
    f4 bfr[NRT];
#pragma unroll
    for (int kb = 0; kb < NRT; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) bfr[kb][q] = cur[(16 * kb + 4 * g + q) * 16 + n];
    f4 nv[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int rt = wave + 4 * r;
      if (rt < NRT) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NRT; ++kb) {
          const f4 a = *reinterpret_cast<const f4*>(A + (size_t)(16 * rt + n) * DK + 16 * kb + 4 * g);
          mma_f32_block(acc, a, bfr[kb]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t e = (size_t)(16 * rt + 4 * g + i) * dv + j0 + n;
          St[e] = v[r][i];
          nv[r][i] = acc[i] + Bm[e];
        }
      }
    }
    __syncthreads();  // every wave has read cur
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int rt = wave + 4 * r;
      if (rt < NRT) {
        v[r] = nv[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[(16 * rt + 4 * g + i) * 16 + n] = v[r][i];
      }
    }
    __syncthreads();
  }
  if (s.S_out != nullptr) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int rt = wave + 4 * r;
      if (rt < NRT)
#pragma unroll
        for (int i = 0; i < 4; ++i) s.S_out[((size_t)h * DK + 16 * rt + 4 * g + i) * dv + j0 + n] = v[r][i];
    }
    combine_final_extras(s, h, j0);
  }
}

// S_start(p+1) = A_p S_start(p) + B_p, serial over the segments of one head, for one
// 16-column tile per workgroup (columns evolve independently). S_start(1) is segment 0's
// final local state, which began at the caller's state. Writes S_start(p) for p >= 1, and
// the final state, carried key and flag to the caller's state.
__global__ __launch_bounds__(NTH) void seg_combine_kernel(SegParams s) {
  const int ntile = s.dv / 16;
  const int h = blockIdx.x / ntile, j0 = (blockIdx.x % ntile) * 16;
  if (s.diag) combine_diagonal(s, h, j0);
  else if (s.dk == 64) combine_general<64>(s, h, j0);
  else combine_general<128>(s, h, j0);
}

// out[vh, t, :] += S_start(vh)^T z_t for segments p >= 1, a [64 x dk] x [dk x dv] product
// per tile of 64 tokens, on bf16 MFMA with hi/lo split operands (the products hi.hi,
// hi.lo and lo.hi keep about 16 bits of each factor). One workgroup per (virtual head,
// group of up to kFixTiles token tiles); wave w owns value columns 16 NTW w ..
// 16 NTW (w + 1) - 1 and keeps their S_start fragments in registers across the tiles.
// Diagonal transitions: z_t = gam_t phi(q~_t), formed here from the queries (feature map
// and QK normalisation as in the scan); the row factor is applied to the product.
constexpr int kFixTiles = 2;

__device__ __forceinline__ void load_row8(const uint16_t* p, float (&x)[8]) { In<uint16_t>::load(p, x); }
__device__ __forceinline__ void load_row8(const float* p, float (&x)[8]) {
  float a[4], b[4];
  In<float>::load(p, a);
  In<float>::load(p + 4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

template <typename InT, int DK, int DV>
__global__ __launch_bounds__(NTH) void seg_fixup_kernel(SegParams s) {
  constexpr int NKQ = DK / 32, NTW = DV / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int ntb = s.L / 64, ngrp = (ntb + kFixTiles - 1) / kFixTiles;
  int b = blockIdx.x;
  const int tg = b % ngrp;
  b /= ngrp;
  const int nseg = s.P - 1;
  const int h = b / nseg, p = 1 + b % nseg;
  const size_t vh = (size_t)h * s.P + p;

  // B fragments: lane (g, n) holds S_start[32 kq + 8 g + e][column 16 (NTW wave + j) + n]
  bf8 bh[NTW][NKQ], bl[NTW][NKQ];
  {
    const float* St = s.S_start + vh * DK * DV;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col = 16 * (NTW * wave + j) + n;
#pragma unroll
      for (int kq = 0; kq < NKQ; ++kq) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = St[(size_t)(32 * kq + 8 * g + e) * DV + col];
        split8(x, bh[j][kq], bl[j][kq]);
      }
    }
  }
  const bool elu = (s.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(s.flags, DK);
  const int tt1 = min(ntb, (tg + 1) * kFixTiles);
  for (int tt = tg * kFixTiles; tt < tt1; ++tt) {
    const size_t row0 = vh * s.L + (size_t)tt * 64;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // A fragments: lane (g, n) holds z[token 16 mt + n][32 kq + 8 g + e]
      const size_t row = row0 + 16 * mt + n;
      f4 acc[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
      float ss = 0.f;
#pragma unroll
      for (int kq = 0; kq < NKQ; ++kq) {
        float x[8];
        if (s.diag) {
          load_row8(static_cast<const InT*>(s.q) + row * DK + 32 * kq + 8 * g, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (elu) x[e] = phi_elu1(x[e]);
            ss += x[e] * x[e];
          }
        } else {
          load_row8(s.z + row * DK + 32 * kq + 8 * g, x);
        }
        bf8 ah, al;
        split8(x, ah, al);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          mma_bf16(acc[j], ah, bh[j][kq]);
          mma_bf16(acc[j], ah, bl[j][kq]);
          mma_bf16(acc[j], al, bh[j][kq]);
        }
      }
      float f = 1.f;
      if (s.diag) {
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        f = s.gam[row] * (len > 0.f ? rescale_factor(ss, len) : 1.f);
      }
      // acc[j][i] is token 16 mt + 4 g + i, whose factor lane 4 g + i holds
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float fi = __shfl(f, 4 * g + i);
        float* o = s.out + (row0 + 16 * mt + 4 * g + i) * DV + n;
#pragma unroll
        for (int j = 0; j < NTW; ++j) o[16 * (NTW * wave + j)] += acc[j][i] * fi;
      }
    }
  }
}

template <typename InT>
hipError_t launch_fixup_in(const SegParams& s, unsigned grid, hipStream_t st) {
  if (s.dk == 64 && s.dv == 64) hipLaunchKernelGGL((seg_fixup_kernel<InT, 64, 64>), dim3(grid), dim3(NTH), 0, st, s);
  else if (s.dk == 64) hipLaunchKernelGGL((seg_fixup_kernel<InT, 64, 128>), dim3(grid), dim3(NTH), 0, st, s);
  else if (s.dv == 64) hipLaunchKernelGGL((seg_fixup_kernel<InT, 128, 64>), dim3(grid), dim3(NTH), 0, st, s);
  else hipLaunchKernelGGL((seg_fixup_kernel<InT, 128, 128>), dim3(grid), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

}  // namespace

int scan_segments(size_t BH, size_t T, int dk, int dv, int bf16, int rule, uint32_t flags) {
  (void)dk;
  if (flags & kFlagOutBf16) return 1;
  const bool split = scan_split_path(bf16, flags);
  const size_t groups = split ? (size_t)dv / kSplitCols : ((size_t)dv + 63) / 64;
  const size_t wgs = BH * groups;
  // propagate workgroups resident at once: one per CU, two for the general pair's rules
  // without a solve or per-channel decay (the diagonal ones), whose LDS fits twice
  const size_t cap = (!split && seg_diagonal(rule, flags)) ? 512 : 256;
  int P = 1;
  while (P < 16 && wgs * 2 * P <= cap && T % (64 * 2 * (size_t)P) == 0 && T / (2 * (size_t)P) >= 512) P *= 2;
  // With a transition pass the propagate work doubles, so fewer than 8 segments do not
  // pay (an additive elu+1 scan with 32 heads, T = 16384, ran no faster with 4 before
  // its transitions were made diagonal); diagonal transitions pay from 2.
  if (seg_diagonal(rule, flags)) return P;
  return P >= 8 ? P : 1;
}

hipError_t launch_seg_decay(const SegParams& s, hipStream_t st) {
  hipLaunchKernelGGL(seg_decay_kernel, dim3((unsigned)((size_t)s.BH * s.P)), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_seg_init(const SegParams& s, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)s.BH * s.P));
  if (s.bf16) hipLaunchKernelGGL((seg_init_kernel<uint16_t>), grid, dim3(NTH), 0, st, s);
  else hipLaunchKernelGGL((seg_init_kernel<float>), grid, dim3(NTH), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const SegParams& s, hipStream_t st) {
  hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(s.BH * (s.dv / 16))), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_seg_fixup(const SegParams& s, hipStream_t st) {
  const size_t ngrp = ((size_t)s.L / 64 + kFixTiles - 1) / kFixTiles;
  const size_t n = (size_t)s.BH * (s.P - 1) * ngrp;
  if (n == 0) return hipSuccess;
  // the queries (diagonal transitions) are read in the input type; z is float32
  return s.bf16 ? launch_fixup_in<uint16_t>(s, (unsigned)n, st) : launch_fixup_in<float>(s, (unsigned)n, st);
}

}  // namespace fwmem
