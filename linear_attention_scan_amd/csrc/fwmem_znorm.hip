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
// thread); the final z goes to the state's carried slot.
__global__ __launch_bounds__(128) void zchain_kernel(ZParams z) {
  const int bh = blockIdx.x, i = threadIdx.x;
  if (i >= z.dk) return;
  const size_t nf = zrec_floats(z.dk);
  float zi = z.z_in != nullptr ? z.z_in[(size_t)bh * z.dk + i] : 0.f;
  for (int c = 0; c < z.nchunks; ++c) {
    const float* r = z.zrec + ((size_t)bh * z.nchunks + c) * nf;
    z.zc[((size_t)bh * z.nchunks + c) * z.dk + i] = zi;
    zi = r[128] * zi + r[132 + i];
  }
  if (z.z_out != nullptr) {
    z.z_out[(size_t)bh * z.dk + i] = zi;
    if (i == 0) z.has_out[bh] = 1;
  }
}

// out[t, :] /= den_in[t] + gq[t] (phi(q_t) . z_c) + eps for 64 tokens of one head per
// workgroup; four threads per token.
template <typename InT>
__global__ __launch_bounds__(256) void zfinal_kernel(ZParams z) {
  const int bh = blockIdx.x / z.nchunks, c = blockIdx.x % z.nchunks;
  const int tl = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int t = c * 64 + tl;
  const bool elu = (z.flags & kFlagPhiElu1) != 0;
  const size_t nf = zrec_floats(z.dk);
  const float* r = z.zrec + ((size_t)bh * z.nchunks + c) * nf;
  const float* zc = z.zc + ((size_t)bh * z.nchunks + c) * z.dk;
  float dot = 0.f;
  if (t < z.T) {
    const InT* qr = static_cast<const InT*>(z.q) + ((size_t)bh * z.T + t) * z.dk;
    for (int i = part; i < z.dk; i += 4) {
      float q = In<InT>::load1(qr + i);
      if (elu) q = phi_elu1(q);
      dot += q * zc[i];
    }
  }
  dot += __shfl_xor(dot, 1);
  dot += __shfl_xor(dot, 2);
  if (t >= z.T) return;
  const float inv = 1.f / (r[tl] + r[64 + tl] * dot + z.eps);
  float* o = z.out + ((size_t)bh * z.T + t) * z.dv;
  for (int j = part; j < z.dv; j += 4) o[j] *= inv;
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
