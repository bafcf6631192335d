// Internal interface between the C-ABI layer (fwmem_api.cpp) and the kernel
// launchers (fwmem_scan.hip, fwmem_step.hip). Host code only sees plain structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fwmem {

enum : uint32_t {
  kFlagPhiElu1 = 1u << 0,
  kFlagPerChannel = 1u << 1,
  kFlagOutBf16 = 1u << 2,
  kFlagQkL2 = 1u << 3,
  kFlagQkRms = 1u << 4,
};

constexpr int kChunk = 64;  // scan chunk length (tokens)

// Length that FWMEM_QK_L2NORM / FWMEM_QK_RMSNORM give q_t and k_t (0: not normalised).
__host__ __device__ inline float qk_length(uint32_t flags, int dk) {
  if (flags & kFlagQkL2) return 1.f;
  if (flags & kFlagQkRms) return __builtin_sqrtf((float)dk);
  return 0.f;
}
// Factor that rescales a vector with squared length ss to length len (a zero vector
// stays zero).
__host__ __device__ inline float rescale_factor(float ss, float len) {
  return ss > 0.f ? len / __builtin_sqrtf(ss) : 0.f;
}

// Write rules (the values of fwmem_rule).
enum : int { kRuleDelta = 0, kRuleAdditive = 1, kRuleInner = 2 };

// What each rule needs of the kernels:
//   shift: the written key is the previous token's (x_t = phi(k_{t-1})), with the key
//          carried across calls in the state and a no-op first step at a sequence start;
//   solve: the write is the residual, which couples the chunk's tokens through the
//          unit-lower-triangular solve (delta rule only);
//   nlms:  the step size is eta_t = beta_t / (|x_t|^2 + lambda_t + eps) and the decay
//          is 1 - eta_t lambda_t (otherwise beta is a write scale and lambda the decay).
template <int RULE>
struct Rule {
  static constexpr bool shift = RULE != kRuleAdditive;
  static constexpr bool solve = RULE == kRuleDelta;
  static constexpr bool nlms = RULE != kRuleAdditive;
};

// Pointers are device pointers; optional ones may be null.
struct ScanParams {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;     // [BH][T] (optional for the additive rule)
  const float* lam;      // [BH][T] or [BH][T][dk], optional
  const float* S_in;     // [BH][dk][dv] or null (zeros)
  const float* xprev_in; // [BH][dk] or null
  const int32_t* has_in; // [BH] or null
  void* out;             // [BH][T][dv] fp32 or bf16
  float* S_out;          // [BH][dk][dv] or null (state not written)
  float* xprev_out;      // [BH][dk] (with S_out)
  int32_t* has_out;      // [BH]     (with S_out)
  char* ws;              // workspace records
  int BH, T, dk, dv, nchunks;
  int rule;              // kRuleDelta, kRuleAdditive or kRuleInner
  int bf16;              // 1: bf16 inputs, 0: fp32
  uint32_t flags;
  float eps;
};

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;      // [BH] (optional for the additive rule)
  const float* lam;       // [BH] or [BH][dk], optional
  const float* S_in;      // [BH][dk][dv] or null
  const float* xprev_in;  // [BH][dk] or null
  const int32_t* has_in;  // [BH] or null
  void* out;              // [BH][dv]
  float* S_out;           // [BH][dk][dv] (required)
  float* xprev_out;
  int32_t* has_out;
  int BH, dk, dv;
  int rule;  // kRuleDelta, kRuleAdditive or kRuleInner
  int bf16;
  uint32_t flags;
  float eps;
};

// Bytes of one (head, chunk) workspace record.
size_t scan_record_bytes(int bf16, int dk, uint32_t flags);
// bf16 inputs with the identity feature map and scalar decay take the split-operand
// propagate kernel (fwmem_scan_split.hip).
bool scan_split_path(int bf16, uint32_t flags);
hipError_t launch_prep_split(const ScanParams& p, hipStream_t stream);
hipError_t launch_prop_split(const ScanParams& p, hipStream_t stream);
// Whether kernels exist for this size.
bool scan_supported(int dk, int dv);
bool step_supported(int dk, int dv);

// Enqueue the scan (T >= 1): phases bit 0 = prep kernel, bit 1 = propagate kernel.
// Returns hipSuccess or the launch error.
hipError_t launch_scan(const ScanParams& p, hipStream_t stream, int phases);
// Enqueue one decode step.
hipError_t launch_step(const StepParams& p, hipStream_t stream);
// S_out := S_in (or the zero state), for T == 0 scans. Bytes is the state size.
hipError_t launch_state_copy(const float* S_in, const float* xprev_in, const int32_t* has_in,
                             float* S_out, float* xprev_out, int32_t* has_out, size_t nS,
                             size_t nX, size_t nH, hipStream_t stream);

}  // namespace fwmem
