// Normalised linear attention (FWMEM_ZNORM): the chain of the normaliser z over the
// chunks of each head and the division of the outputs. "attention is also an FFN",
// section 4.2: o_t = S_t^T phi(q_t) / (z_t . phi(q_t) + eps), z_t = gamma_t z_{t-1} +
// beta_t phi(k_t), the decay applied to z as to S. The chunk terms come from the prep
// kernels (ZRec in fwmem_internal.h).
#include "fwmem_device.h"
#include "fwmem_internal.h"

namespace fwmem {
namespace {

// z at the entry of every chunk, serially over the chunks of one head (one channel per
// thread); the final z goes to the state's carried slot. The chunk terms are loaded eight
// chunks ahead of the dependent updates.
__global__ __launch_bounds__(128) void zchain_kernel(ZParams z) {
  const int bh = blockIdx.x, i = threadIdx.x;
  if (i >= z.dk) return;
  const size_t nf = zrec_floats(z.dk);
  const float* rec = z.zrec + (size_t)bh * z.nchunks * nf;
  float* zc = z.zc + (size_t)bh * z.nchunks * z.dk;
  float zi = z.z_in != nullptr ? z.z_in[(size_t)bh * z.dk + i] : 0.f;
  constexpr int U = 8;
  for (int c0 = 0; c0 < z.nchunks; c0 += U) {
    float a[U], w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      a[u] = c < z.nchunks ? rec[(size_t)c * nf + 128] : 1.f;
      w[u] = c < z.nchunks ? rec[(size_t)c * nf + 132 + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      if (c < z.nchunks) {
        zc[(size_t)c * z.dk + i] = zi;
        zi = a[u] * zi + w[u];
      }
    }
  }
  if (z.z_out != nullptr) {
    z.z_out[(size_t)bh * z.dk + i] = zi;
    if (i == 0) z.has_out[bh] = 1;
  }
}

// out[t, :] /= den_in[t] + gq[t] (phi(q_t) . z_c) + eps for the 64 tokens of one chunk per
// workgroup: 16 lanes per token row, so that q and out move in 16-byte pieces along the
// row (four rows per wave instruction).
template <typename InT>
__global__ __launch_bounds__(256) void zfinal_kernel(ZParams z) {
  constexpr int VW = In<InT>::VW;
  const int bh = blockIdx.x / z.nchunks, c = blockIdx.x % z.nchunks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 4, l16 = lane & 15;
  const bool elu = (z.flags & kFlagPhiElu1) != 0;
  const size_t nf = zrec_floats(z.dk);
  const float* r = z.zrec + ((size_t)bh * z.nchunks + c) * nf;
  const float* zc = z.zc + ((size_t)bh * z.nchunks + c) * z.dk;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int tl = wave * 16 + rr * 4 + sub;  // token within the chunk
    const int t = c * 64 + tl;
    float dot = 0.f;
    if (t < z.T) {
      const InT* qr = static_cast<const InT*>(z.q) + ((size_t)bh * z.T + t) * z.dk;
      for (int i0 = l16 * VW; i0 < z.dk; i0 += 16 * VW) {
        float q[VW];
        In<InT>::load(qr + i0, q);
#pragma unroll
        for (int j = 0; j < VW; ++j) dot += (elu ? phi_elu1(q[j]) : q[j]) * zc[i0 + j];
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o);
    if (t < z.T) {
      const float inv = 1.f / (r[tl] + r[64 + tl] * dot + z.eps);
      f4* orow = reinterpret_cast<f4*>(z.out + ((size_t)bh * z.T + t) * z.dv);
      for (int j4 = l16; j4 < z.dv / 4; j4 += 16) orow[j4] = orow[j4] * inv;
    }
  }
}

}  // namespace

hipError_t launch_znorm(const ZParams& z, hipStream_t st) {
  if (z.BH == 0 || z.T == 0) return hipSuccess;
  hipLaunchKernelGGL(zchain_kernel, dim3((unsigned)z.BH), dim3(128), 0, st, z);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((size_t)z.nchunks * z.BH));  // below 2^31 (checked by the caller)
  if (z.bf16) hipLaunchKernelGGL((zfinal_kernel<uint16_t>), grid, dim3(256), 0, st, z);
  else hipLaunchKernelGGL((zfinal_kernel<float>), grid, dim3(256), 0, st, z);
  return hipGetLastError();
}

}  // namespace fwmem
