// Internal interface of the scan's backward pass (fwmem_backward.hip), between the C-ABI
// layer and its launcher. Host code only sees plain structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fwmem {

// Pointers are device pointers; optional ones may be null. Gradients are float32 in the
// layout of the input they belong to.
struct BwdParams {
  const void* q;          // [BH][T][dk]
  const void* k;          // [BH][T][dk]
  const void* v;          // [BH][T][dv]
  const float* beta;      // [BH][T] ([BH][T][dv] per value channel; optional for the additive rule)
  const float* lam;       // [BH][T] ([BH][T][dk] with kFlagPerChannel) or null
  const float* S_in;      // [BH][dk][dv] or null (zeros)
  const float* xprev_in;  // [BH][dk] or null
  const int32_t* has_in;  // [BH] or null
  const float* dout;      // [BH][T][dv]
  const float* dS_out;    // [BH][dk][dv] or null (zeros)
  const float* dz_out;    // [BH][dk] the final normaliser's gradient (normaliser only), or null
  float* gq;              // [BH][T][dk]
  float* gk;              // [BH][T][dk]
  float* gv;              // [BH][T][dv]
  float* gbeta;           // beta's shape, or null (not written)
  float* glam;            // lam's shape, or null (not written)
  float* gS0;             // [BH][dk][dv] or null
  float* gx0;             // [BH][dk] or null (with gS0)
  int32_t* gh0;           // [BH] or null (with gS0): written 0
  float* ws;              // per head: chunk-start states, then one chunk's states
  int BH, T, dk, dv, nchunks;
  int rule;  // kRuleDelta, kRuleAdditive, kRuleInner or kRuleDeltaPV
  int bf16;
  uint32_t flags;
  float eps;
};

// Tokens the backward stages at a time and between the states it keeps: 64, or 32 with a
// per-channel lambda, a per-value-channel beta or the normaliser (whose staged values
// would not fit LDS with 64).
__host__ __device__ constexpr int bwd_chunk(bool small) { return small ? 32 : 64; }
// Workspace floats per head: the state at each chunk start, the states after each of a
// chunk's tokens, and a chunk's worth of d_v-vectors.
// With the normaliser (znorm), also its value at each chunk start.
__host__ __device__ inline size_t bwd_floats_per_head(int T, int dk, int dv, bool small, bool znorm) {
  const size_t ck = (size_t)bwd_chunk(small);
  const size_t nchunks = ((size_t)T + ck - 1) / ck;
  const size_t SS = (size_t)dk * (size_t)dv;
  return T > 0 ? (nchunks + ck) * SS + ck * (size_t)dv + (znorm ? nchunks * (size_t)dk : 0) : 0;
}
bool bwd_supported(int dk, int dv);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
// QK normalisation: maps the q, k and carried-key gradients, taken with respect to the
// rescaled vectors, back to the raw ones in place (nothing without the flags).
hipError_t launch_qk_norm_bwd(const BwdParams& p, hipStream_t stream);

// The chunk-parallel backward (fwmem_backward_chunk.hip): the delta, inner and additive
// rules with a scalar decay and without the normaliser, T >= 1. Its workspace per head:
// one record and two states per 64-token chunk.
bool bwd_chunked(int rule, uint32_t flags, int T);
size_t bwd_chunk_floats_per_head(int T, int dk, int dv);
hipError_t launch_bwd_chunked(const BwdParams& p, hipStream_t stream);

}  // namespace fwmem
