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
  kFlagBetaSig = 1u << 5,
  kFlagBetaSig2 = 1u << 6,
  kFlagLamAct = 1u << 7,
  kFlagZnorm = 1u << 8,
  kFlagLamScaled = 1u << 9,
};

constexpr int kChunk = 64;  // scan chunk length (tokens)

// Length that FWMEM_QK_L2NORM / FWMEM_QK_RMSNORM give q_t and k_t (0: not normalised).
__host__ __device__ inline float qk_length(uint32_t flags, int dk) {
  if (flags & kFlagQkL2) return 1.f;
  if (flags & kFlagQkRms) return __builtin_sqrtf((float)dk);
  return 0.f;
}
// Gate activations (FWMEM_BETA_SIGMOID / FWMEM_BETA_SIGMOID2 / FWMEM_LAMBDA_PREACT): the
// step size or write scale sigmoid(z) or 2 sigmoid(z); the ridge softplus(z) for the
// shifted-pair rules (nlms) and the retention sigmoid(z) for the additive rule. Without
// the flags the gate is used as given.
__device__ inline float act_beta(float z, uint32_t flags) {
  if (flags & kFlagBetaSig) return 1.f / (1.f + __expf(-z));
  if (flags & kFlagBetaSig2) return 2.f / (1.f + __expf(-z));
  return z;
}
__device__ inline float act_lam(float z, uint32_t flags, bool nlms) {
  if (!(flags & kFlagLamAct)) return z;
  if (!nlms) return 1.f / (1.f + __expf(-z));
  return z > 30.f ? z : log1pf(__expf(z));
}
// Start of a running maximum of lambda over channels: pre-activations may be negative.
__device__ inline float lam_max_init(uint32_t flags) { return (flags & kFlagLamAct) ? -__builtin_inff() : 0.f; }

// Factor that rescales a vector with squared length ss to length len (a zero vector
// stays zero).
__host__ __device__ inline float rescale_factor(float ss, float len) {
  return ss > 0.f ? len / __builtin_sqrtf(ss) : 0.f;
}

// Write rules (the values of fwmem_rule).
enum : int { kRuleDelta = 0, kRuleAdditive = 1, kRuleInner = 2, kRuleDeltaPV = 3 };

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
  static constexpr bool solve = RULE == kRuleDelta || RULE == kRuleDeltaPV;
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
  float* zrec;           // normalised linear attention: per (head, chunk) ZRec, or null
  int BH, T, dk, dv, nchunks;
  int rule;              // kRuleDelta, kRuleAdditive or kRuleInner
  int bf16;              // 1: bf16 inputs, 0: fp32
  uint32_t flags;
  float eps;
  // bounded waits of the split propagate kernel: polls before giving up, and an offset
  // added to the awaited value (0; a test sets it so that every wait gives up)
  int wait_polls, wait_bias;
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
// The per-value-channel rule (fwmem_scan_pv.hip): its record size and both phases.
size_t scan_pv_record_bytes();
hipError_t launch_scan_pv(const ScanParams& p, hipStream_t stream, int phases);
hipError_t launch_prop_split(const ScanParams& p, hipStream_t stream);
// The additive rule with elu + 1 features and a scalar retention on bf16 inputs
// (without the normaliser) runs as one fused kernel per head (fwmem_scan_add.hip): the
// prep phase does nothing, the propagate phase everything, and no record is written.
bool scan_add_path(int bf16, int rule, uint32_t flags);
hipError_t launch_scan_add(const ScanParams& p, hipStream_t stream);
// Polls of a bounded wait before it gives up, and the offset of the awaited value: from
// FWMEM_TEST_WAIT_TIMEOUT=n (n > 0, a test's setting: every wait gives up after n polls),
// else 2^22 and 0.
void wait_config(int* polls, int* bias);
// Synchronises `stream`, reads the current device's sticky wait status into *value and
// clears it if it was set.
hipError_t read_wait_status(hipStream_t stream, int* value);
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

// ---- segment-parallel scan (few heads, long sequences)
//
// A head's T tokens are cut into P segments of L = T / P tokens. Because q, k, v, the
// gates and out are [BH][T][...] row-major, segment p of head h is virtual head
// h * P + p of a [BH * P][L][...] problem, and the ordinary kernels run all segments at
// once. Two state passes over the virtual heads (no outputs):
//   local:      from S = 0 with the real values; gives the segment's own state B_p;
//   transition: from S = I with zero values; gives A_p (the segment's linear map
//               S -> A_p S + B_p).
// Then S_start(p+1) = A_p S_start(p) + B_p (a short serial chain over segments from
// S_start(0), the caller's state), written into B0, and one pass over the virtual heads
// from those start states writes the outputs. No pass of the propagate phase reads what
// another writes before the combine, so the phase can run again after one prep. Each segment's first token takes the previous segment's last key as its
// carried key.
struct SegParams {
  const void* k;          // [BH][T][dk] raw keys (the carried key of each segment)
  const float* S_in;      // caller's state or null
  const float* xprev_in;
  const int32_t* has_in;
  float* S_out;           // caller's state or null
  float* xprev_out;
  int32_t* has_out;
  // Virtual state buffers (S, then x_prev, then has_prev, as in the ABI's state layout):
  // the passes start from A0 (transition, S [BH*P][dk][dk]) and B0 (local, S
  // [BH*P][dk][dv]), written by the set-up kernel, and end in A1 and B1, so a propagate
  // phase never changes its own inputs.
  float* A0_S;
  float* A0_x;
  int32_t* A0_h;
  float* B0_S;
  float* B0_x;
  int32_t* B0_h;
  float* A1_S;
  float* B1_S;
  float* B1_x;
  float* S_start;         // [BH*P][dk][dv] (segment p >= 1): B0_S
  float* out;             // [BH][T][dv] float32
  // Diagonal transitions (additive rule, scalar decay): a segment maps S to
  // Gamma_p S + B_p, so there is no transition pass and no A buffer; the segments' own
  // states B_p come from seg_state (B1 holds them).
  int diag;
  const void* q;          // [BH][T][dk] raw queries
  const void* v;          // [BH][T][dv] values
  const float* beta;      // [BH][T] write scales (or pre-activations), or null (1)
  const float* lam;       // [BH][T] retention (or pre-activations), or null (1)
  float* gam;             // [BH*P] each segment's decay Gamma_p (diagonal transitions)
  // The normaliser with the fused additive pass: seg_state leaves each segment's change of
  // z in B1_x, the combine chains z into B0_x, and the pass carries it from there.
  int zfused;
  int BH, P, L, dk, dv, bf16;
  uint32_t flags;
};
// A scan whose segments compose by a scalar: the additive rule with a scalar decay.
__host__ __device__ inline bool seg_diagonal(int rule, uint32_t flags) {
  return rule == kRuleAdditive && (flags & kFlagPerChannel) == 0;
}
// Segment count for a scan of this shape: 1 (no segmentation) unless the propagate
// grid would leave most of the GPU idle and T splits into equal chunk-aligned segments.
int scan_segments(size_t BH, size_t T, int dk, int dv, int bf16, int rule, uint32_t flags);
hipError_t launch_seg_init(const SegParams& s, hipStream_t st);

// ---- normalised linear attention (FWMEM_ZNORM; additive rule, scalar decay)
//
// Per (head, chunk) the prep kernels write a ZRec of floats:
//   [0, 64)        den_in[t] = sum_{s<=t} M_ts beta_s    (the chunk's own writes)
//   [64, 128)      gq[t] = Gamma_t (times q_t's rescale factor with QK normalisation)
//   128            Gamma_C
//   [132, 132+dk)  w = sum_s (Gamma_C / Gamma_s) beta_s x_s  (the chunk's write to z)
// The normaliser at token t of chunk c is den_in[t] + gq[t] (q_t . z_c), z_c the
// normaliser at chunk entry: z_{c+1} = Gamma_C z_c + w.
__host__ __device__ inline size_t zrec_floats(int dk) { return (size_t)132 + (size_t)dk; }
struct ZParams {
  const float* zrec;       // [BH][nchunks] ZRec
  float* zc;               // [BH][nchunks][dk] z at chunk entry
  const float* z_in;       // the state's carried slot, or null (z = 0)
  float* z_out;            // the state's carried slot, or null
  int32_t* has_out;
  const void* q;           // raw q [BH][T][dk]
  float* out;              // [BH][T][dv] float32, divided in place
  int BH, T, nchunks, dk, dv, bf16;
  uint32_t flags;
  float eps;
};
hipError_t launch_znorm(const ZParams& z, hipStream_t st);
hipError_t launch_seg_combine(const SegParams& s, hipStream_t st);
hipError_t launch_seg_state(const SegParams& s, hipStream_t st);
hipError_t launch_seg_extras(const SegParams& s, hipStream_t st);

}  // namespace fwmem
