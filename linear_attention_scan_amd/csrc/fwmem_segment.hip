// Segment-parallel scan: the set-up, combine and fix-up kernels (see SegParams in
// fwmem_internal.h). The split of a long sequence into segments whose maps compose
// is the scan's own linearity: the write S_t = (diag(a_t) - eta_t x_t x_t^T) S_{t-1}
// + eta_t x_t v_t^T (delta rule; "Fast Weight Attention for Continual Learning"
// reading notes, sections 3.2 and 4.2), and its additive and inner-product forms, are
// affine in S, so a segment maps its start state S to A S + B.
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
    s.A0_x[(size_t)vh * dk + i] = x;
  }
  if (threadIdx.x == 0) {
    const int has = p > 0 ? 1 : (s.S_in != nullptr && s.has_in[h] != 0 ? 1 : 0);
    s.B0_h[vh] = has;
    s.A0_h[vh] = has;
  }
}

// S_start(p+1) = A_p S_start(p) + B_p, serial over the segments of one head, for one
// 16-column tile per workgroup (columns evolve independently). S_start(1) is segment 0's
// final local state, which began at the caller's state. Writes S_start(p) for p >= 1,
// and the final state, carried key and flag to the caller's state.
__global__ __launch_bounds__(NTH) void seg_combine_kernel(SegParams s) {
  const int dk = s.dk, dv = s.dv;
  const int ntile = dv / 16;
  const int h = blockIdx.x / ntile, j0 = (blockIdx.x % ntile) * 16;
  __shared__ float cur[128 * 16];
  const int j = threadIdx.x & 15, i0 = threadIdx.x >> 4;  // rows i0, i0 + 16, ...
  const int RP = dk / 16;                                  // rows per thread
  float v[8];
  // S_start(1)
  const float* B0 = s.B1_S + (size_t)(h * s.P) * dk * dv;
  for (int r = 0; r < RP; ++r) {
    v[r] = B0[(size_t)(i0 + 16 * r) * dv + j0 + j];
    cur[(i0 + 16 * r) * 16 + j] = v[r];
  }
  __syncthreads();
  for (int p = 1; p < s.P; ++p) {
    const size_t vh = (size_t)h * s.P + p;
    float* St = s.S_start + vh * dk * dv;
    for (int r = 0; r < RP; ++r) St[(size_t)(i0 + 16 * r) * dv + j0 + j] = v[r];
    const float* A = s.A1_S + vh * dk * dk;
    const float* Bm = s.B1_S + vh * dk * dv;
    float nv[8];
    for (int r = 0; r < RP; ++r) {
      const int i = i0 + 16 * r;
      const f4* Ar = reinterpret_cast<const f4*>(A + (size_t)i * dk);
      float acc0 = 0.f, acc1 = 0.f;
      for (int k4 = 0; k4 < dk / 4; ++k4) {
        const f4 a = Ar[k4];
        acc0 += a[0] * cur[(4 * k4) * 16 + j];
        acc1 += a[1] * cur[(4 * k4 + 1) * 16 + j];
        acc0 += a[2] * cur[(4 * k4 + 2) * 16 + j];
        acc1 += a[3] * cur[(4 * k4 + 3) * 16 + j];
      }
      nv[r] = acc0 + acc1 + Bm[(size_t)i * dv + j0 + j];
    }
    __syncthreads();  // every thread has read cur
    for (int r = 0; r < RP; ++r) {
      v[r] = nv[r];
      cur[(i0 + 16 * r) * 16 + j] = v[r];
    }
    __syncthreads();
  }
  if (s.S_out != nullptr) {
    for (int r = 0; r < RP; ++r) s.S_out[((size_t)h * dk + i0 + 16 * r) * dv + j0 + j] = v[r];
    if (j0 == 0) {
      const size_t last = (size_t)h * s.P + s.P - 1;
      if ((s.flags & kFlagZnorm) == 0)  // with the normaliser the slot holds z
        for (int i = threadIdx.x; i < dk; i += NTH) s.xprev_out[(size_t)h * dk + i] = s.B1_x[last * dk + i];
      if (threadIdx.x == 0) s.has_out[h] = 1;
    }
  }
}

// out[vh, t, c] += sum_k z[vh, t, k] S_start(vh)[k, c] for segments p >= 1: one
// workgroup per (virtual head, 64 tokens, 64 columns), fp32, each thread a 4 x 4 block.
__global__ __launch_bounds__(NTH) void seg_fixup_kernel(SegParams s) {
  const int dk = s.dk, dv = s.dv;
  const int ncb = dv / 64, ntb = s.L / 64;
  int b = blockIdx.x;
  const int cb = b % ncb;
  b /= ncb;
  const int tb = b % ntb;
  b /= ntb;
  const int nseg = s.P - 1;
  const int h = b / nseg, p = 1 + b % nseg;
  const size_t vh = (size_t)h * s.P + p;
  __shared__ float zt[128 * 64];  // [k][t]
  __shared__ float sc[128 * 64];  // [k][c]
  const float* z = s.z + (vh * s.L + (size_t)tb * 64) * dk;
  const float* St = s.S_start + vh * dk * dv + cb * 64;
  for (int e = threadIdx.x; e < 64 * dk; e += NTH) {
    const int t = e / dk, kk = e % dk;
    zt[kk * 64 + t] = z[(size_t)t * dk + kk];
  }
  for (int e = threadIdx.x; e < dk * 64; e += NTH) {
    const int kk = e / 64, c = e % 64;
    sc[kk * 64 + c] = St[(size_t)kk * dv + c];
  }
  __syncthreads();
  const int t0 = (threadIdx.x >> 4) * 4, c0 = (threadIdx.x & 15) * 4;
  f4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int kk = 0; kk < dk; ++kk) {
    const f4 a = *reinterpret_cast<const f4*>(&zt[kk * 64 + t0]);
    const f4 bb = *reinterpret_cast<const f4*>(&sc[kk * 64 + c0]);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += a[r] * bb;
  }
  float* o = s.out + ((vh * s.L) + (size_t)tb * 64 + t0) * dv + cb * 64 + c0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f4* dst = reinterpret_cast<f4*>(o + (size_t)r * dv);
    *dst = *dst + acc[r];
  }
}

}  // namespace

int scan_segments(size_t BH, size_t T, int dk, int dv, int bf16, uint32_t flags) {
  (void)dk;
  if (flags & kFlagOutBf16) return 1;
  const size_t groups = scan_split_path(bf16, flags) ? (size_t)dv / kSplitCols : ((size_t)dv + 63) / 64;
  const size_t wgs = BH * groups;
  // The two passes double the propagate work, so fewer than 8 segments do not pay (an
  // additive elu+1 scan with 32 heads, T = 16384, ran no faster with 4).
  int P = 1;
  while (P < 16 && wgs * 2 * P <= 256 && T % (64 * 2 * (size_t)P) == 0 && T / (2 * (size_t)P) >= 512) P *= 2;
  return P >= 8 ? P : 1;
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
  const size_t n = (size_t)s.BH * (s.P - 1) * (s.L / 64) * (s.dv / 64);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(seg_fixup_kernel, dim3((unsigned)n), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

}  // namespace fwmem
