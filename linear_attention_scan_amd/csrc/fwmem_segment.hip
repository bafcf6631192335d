// Segment-parallel scan: the set-up, segment-state and combine kernels (see SegParams in
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

// Virtual initial states. Segment 0's start state: the caller's state, or zero (the
// combine and the output pass read it; the other segments' start states come from the
// combine). Transition pass: the identity. Every pass carries the same key: the caller's
// for segment 0, the last (raw, or elu+1 of the raw) key of the previous segment for p >= 1.
template <typename InT>
__global__ __launch_bounds__(NTH) void seg_init_kernel(SegParams s) {
  const int vh = blockIdx.x, h = vh / s.P, p = vh % s.P;
  const int dk = s.dk, dv = s.dv;
  const bool elu = (s.flags & kFlagPhiElu1) != 0;
  float* B = s.B0_S + (size_t)vh * dk * dv;
  float* A = s.A0_S + (size_t)vh * dk * dk;
  const float* Sin = (p == 0 && s.S_in != nullptr) ? s.S_in + (size_t)h * dk * dv : nullptr;
  // the caller's state (4-byte aligned only): eight loads in flight per thread
  if (p == 0) {
#pragma unroll 8
    for (int e = threadIdx.x; e < dk * dv; e += NTH) B[e] = Sin != nullptr ? Sin[e] : 0.f;
  }
  // the identity in 16-byte stores (A lies in the workspace, 256-byte aligned, and dk is a
  // multiple of 4)
  if (!s.diag)
    for (int e = 4 * threadIdx.x; e < dk * dk; e += 4 * NTH) {
      f4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = ((e + j) / dk == (e + j) % dk) ? 1.f : 0.f;
      *reinterpret_cast<f4*>(A + e) = a;
    }
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

// Diagonal transitions with the segment states formed first: S_start(p+1) = Gamma_p
// S_start(p) + B_p, every element on its own, four consecutive elements per thread (one
// 16-byte access per segment). Gamma_p is the segment's decay, from seg_state_kernel.
__global__ __launch_bounds__(NTH) void seg_combine_diag_kernel(SegParams s) {
  const size_t n = (size_t)s.dk * s.dv;  // a multiple of 4 NTH
  const size_t nb = n / (4 * NTH);
  const size_t h = blockIdx.x / nb;
  const size_t e = ((blockIdx.x % nb) * NTH + threadIdx.x) * 4;
  f4 v = *reinterpret_cast<const f4*>(s.B1_S + h * s.P * n + e);
  for (int p = 1; p < s.P; ++p) {
    const size_t vh = h * s.P + p;
    *reinterpret_cast<f4*>(s.S_start + vh * n + e) = v;
    const float gp = s.gam[vh];
    v = gp * v + *reinterpret_cast<const f4*>(s.B1_S + vh * n + e);
  }
  if (s.S_out != nullptr) *reinterpret_cast<f4*>(s.S_out + h * n + e) = v;
  // the normaliser's start values, chained the same way (its key slot)
  if (s.zfused && blockIdx.x % nb == 0 && (int)threadIdx.x < s.dk) {
    const size_t i = threadIdx.x;
    float vz = s.B1_x[h * s.P * s.dk + i];
    for (int p = 1; p < s.P; ++p) {
      const size_t vh = h * s.P + p;
      s.B0_x[vh * s.dk + i] = vz;
      vz = s.gam[vh] * vz + s.B1_x[vh * s.dk + i];
    }
  }
}

// General transitions: S_start(p+1) = A_p S_start(p) + B_p, a [d_k x d_k] x [d_k x 16]
// product per segment on fp32 MFMA. The local pass ran every segment from zero, so the
// chain starts at S_start(0), the caller's state (its copy in B0 made at set-up); without
// one, at S_start(1) = B_0. Wave w owns row tiles w, w + 4 of the tile in C layout; the
// current start state goes through LDS so that every wave reads all of it as B fragments.
template <int DK>
__device__ void combine_general(const SegParams& s, int h, int j0) {
  constexpr int NRT = DK / 16, RPW = (NRT + 3) / 4;
  __shared__ float cur[2][DK * 16];
  const int dv = s.dv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const bool from_in = s.S_in != nullptr;
  const int p0 = from_in ? 0 : 1;
  f4 v[RPW];
  const float* V0 = (from_in ? s.B0_S : s.B1_S) + (size_t)(h * s.P) * DK * dv;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rt = wave + 4 * r;
    if (rt < NRT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[r][i] = V0[(size_t)(16 * rt + 4 * g + i) * dv + j0 + n];
        cur[p0 & 1][(16 * rt + 4 * g + i) * 16 + n] = v[r][i];
      }
    }
  }
  // The lane's rows of A_p and its elements of B_p do not depend on the chain: they are
  // loaded one step ahead, so a step waits only for its product and one barrier (the
  // start state alternates between two LDS tiles).
  f4 an[RPW][NRT], bn[RPW];
  auto fetch = [&](int p) {
    const size_t vh = (size_t)h * s.P + p;
    const float* A = s.A1_S + vh * DK * DK;
    const float* Bm = s.B1_S + vh * DK * dv;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int rt = wave + 4 * r;
      if (rt < NRT) {
#pragma unroll
        for (int kb = 0; kb < NRT; ++kb)
          an[r][kb] = *reinterpret_cast<const f4*>(A + (size_t)(16 * rt + n) * DK + 16 * kb + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) bn[r][i] = Bm[(size_t)(16 * rt + 4 * g + i) * dv + j0 + n];
      }
    }
  };
  if (p0 < s.P) fetch(p0);
  __syncthreads();
  for (int p = p0; p < s.P; ++p) {
    f4 a[RPW][NRT], b[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      b[r] = bn[r];
#pragma unroll
      for (int kb = 0; kb < NRT; ++kb) a[r][kb] = an[r][kb];
    }
    if (p + 1 < s.P) fetch(p + 1);
    const float* cb = cur[p & 1];
    float* cn = cur[(p + 1) & 1];
    f4 bfr[NRT];
#pragma unroll
    for (int kb = 0; kb < NRT; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) bfr[kb][q] = cb[(16 * kb + 4 * g + q) * 16 + n];
    float* St = s.S_start + ((size_t)h * s.P + p) * DK * dv;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int rt = wave + 4 * r;
      if (rt < NRT) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NRT; ++kb) mma_f32_block(acc, a[r][kb], bfr[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (p > 0) St[(size_t)(16 * rt + 4 * g + i) * dv + j0 + n] = v[r][i];
          v[r][i] = acc[i] + b[r][i];
          cn[(16 * rt + 4 * g + i) * 16 + n] = v[r][i];
        }
      }
    }
    __syncthreads();  // the next start state is in cn; every wave has read cb
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
// 16-column tile per workgroup (columns evolve independently). Writes S_start(p) for
// p >= 1, and the final state, carried key and flag to the caller's state.
__global__ __launch_bounds__(NTH) void seg_combine_kernel(SegParams s) {
  const int ntile = s.dv / 16;
  const int h = blockIdx.x / ntile, j0 = (blockIdx.x % ntile) * 16;
  if (s.dk == 64) combine_general<64>(s, h, j0);
  else combine_general<128>(s, h, j0);
}

// Eight K slots of a bf16 MFMA operand from a row-major [token][column] tile by two LDS
// transpose reads: within each group of 16 lanes, lane 4r + c points at four values of
// token row r, columns 4c..4c+3, and lane 4c + e receives column 4c + e of the four rows.
// `p` is this lane's address for the first four K slots; `step` (elements) reaches the
// rows of the other four.
__device__ __forceinline__ bf8 tr_pair(const uint16_t* p, int step) {
  typedef short s8v __attribute__((ext_vector_type(8)));
  const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(const void*)p);
  const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(const void*)(p + step));
  const s8v r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf8, r);
}

// Diagonal transitions: each segment's own contribution to the state,
//   B_p = sum_t (product of the retentions after t in the segment) beta_t x_t v_t^T,
// plus Gamma_p S_in for segment 0, a [d_k x L] x [L x d_v] product per segment, so that
// the combine gives every segment its start state before any output is formed. One
// workgroup per segment walks its 64-token blocks from the end backwards, carrying the
// product of the retentions after the block. x_t = phi(k_t) (times its QK factor) and
// w_t v_t go to LDS as bf16 hi and lo rows; each of the eight waves owns a share of the
// [d_k x d_v] result's 16 x 16 tiles, on bf16 MFMA with the split products
// hi.hi, hi.lo and lo.hi, and reads the X^T and W operands with the LDS transpose read
// (two reads of four tokens give a fragment's eight K slots).
constexpr int kStateThreads = 512;

template <typename InT, int DK, int DV>
__global__ __launch_bounds__(kStateThreads) void seg_state_kernel(SegParams s) {
  constexpr int LDX = DK + 8, LDW = DV + 8;  // bf16 row strides
  constexpr int NT = kStateThreads, NW = NT / 64;
  // wave w owns NMT d_k row tiles from mt0 against NNW value tiles from nt0
  constexpr int NMTT = DK / 16;                        // d_k row tiles
  constexpr int WPM = NW >= NMTT ? NW / NMTT : 1;      // waves that share a row tile
  constexpr int NMT = NMTT >= NW ? NMTT / NW : 1;
  constexpr int NNW = DV / 16 / WPM;
  constexpr int VW = In<InT>::VW;
  constexpr int GX = DK / VW, GV = DV / VW;  // 16-byte granules per row
  constexpr int NGX = 64 * GX / NT, NGV = 64 * GV / NT;
  static_assert(NGX >= 1 && NGV >= 1 && GX <= 64 && NNW >= 1, "granules");
  __shared__ __align__(16) uint16_t xs[2][64 * LDX];  // hi, lo
  __shared__ __align__(16) uint16_t ws[2][64 * LDW];
  __shared__ float s_w[64];
  __shared__ float s_tot;
  __shared__ float s_zb[NW][DK];  // with the normaliser: each wave's part of sum_t w_t x_t
  const size_t vh = blockIdx.x;
  const int p = (int)(vh % s.P), L = s.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // with the normaliser, thread tid adds up w_t x_t over its rows for the VW columns of
  // granule tid % GX (the same granule in every row it stages)
  float zp[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) zp[j] = 0.f;
  const int g = lane >> 4, n = lane & 15;
  const int mt0 = (wave / WPM) * NMT, nt0 = (wave % WPM) * NNW;
  const bool elu = (s.flags & kFlagPhiElu1) != 0;
  const float len = qk_length(s.flags, DK);
  const InT* kb = static_cast<const InT*>(s.k) + vh * L * DK;
  const InT* vb = static_cast<const InT*>(s.v) + vh * L * DV;
  const float* lam = s.lam != nullptr ? s.lam + vh * L : nullptr;
  const float* bet = s.beta != nullptr ? s.beta + vh * L : nullptr;

  f4 acc[NMT][NNW];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NNW; ++nt) acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
  float carry = 1.f;  // product of the retentions after the current block
  u32x4 rk[NGX], rv[NGV];
  float rgm = 1.f, rbt = 1.f;  // raw gates of token lane of the block (wave 0)
  auto load_rows = [&](int t0) {
    if (wave == 0) {
      if (lam != nullptr) rgm = lam[t0 + lane];
      if (bet != nullptr) rbt = bet[t0 + lane];
    }
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const int gi = tid + NT * r;
      rk[r] = *reinterpret_cast<const u32x4*>(kb + (size_t)(t0 + gi / GX) * DK + (gi % GX) * VW);
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = tid + NT * r;
      rv[r] = *reinterpret_cast<const u32x4*>(vb + (size_t)(t0 + gi / GV) * DV + (gi % GV) * VW);
    }
  };
  const int nblk = L / 64;
  load_rows((nblk - 1) * 64);
  for (int blk = nblk - 1; blk >= 0; --blk) {
    const int t0 = blk * 64;
    // token weights: w_t = beta_t times the retentions after t (inside the block, then
    // after it); the block's product of retentions for the carry
    if (wave == 0) {
      const float gm = lam != nullptr ? act_lam(rgm, s.flags, false) : 1.f;
      const float bt = bet != nullptr ? act_beta(rbt, s.flags) : 1.f;
      float suf = gm;  // inclusive suffix product over lanes lane..63
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_down(suf, o);
        if (lane + o < 64) suf *= u;
      }
      float after = __shfl_down(suf, 1);  // tokens after this one inside the block
      if (lane == 63) after = 1.f;
      s_w[lane] = bt * after * carry;
      if (lane == 0) s_tot = suf;
    }
    __syncthreads();  // s_w; the previous block's operand reads are done
    // rows of this block into LDS: phi(k) with its QK factor, and w v, split hi / lo
#pragma unroll
    for (int r = 0; r < NGX; ++r) {
      const int gi = tid + NT * r, t = gi / GX, cc = (gi % GX) * VW;
      float x[VW];
      In<InT>::decode(rk[r], x);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if (elu) x[j] = phi_elu1(x[j]);
        ss += x[j] * x[j];
      }
      if (len > 0.f) {
        ss = group_sum<GX>(ss);
        const float f = rescale_factor(ss, len);
#pragma unroll
        for (int j = 0; j < VW; ++j) x[j] *= f;
      }
      if (s.zfused) {  // the normaliser's share: w_t x_t
        const float wt = s_w[t];
#pragma unroll
        for (int j = 0; j < VW; ++j) zp[j] += wt * x[j];
      }
#pragma unroll
      for (int j = 0; j < VW; j += 8 < VW ? 8 : VW) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (j + e < VW) ? x[j + e] : 0.f;
        bf8 hh, ll;
        split8(y, hh, ll);
        if (VW >= 8) {
          *reinterpret_cast<bf8*>(&xs[0][t * LDX + cc + j]) = hh;
          *reinterpret_cast<bf8*>(&xs[1][t * LDX + cc + j]) = ll;
        } else {
          typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<bf4*>(&xs[0][t * LDX + cc + j]) = bf4{hh[0], hh[1], hh[2], hh[3]};
          *reinterpret_cast<bf4*>(&xs[1][t * LDX + cc + j]) = bf4{ll[0], ll[1], ll[2], ll[3]};
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = tid + NT * r, t = gi / GV, cc = (gi % GV) * VW;
      float x[VW];
      In<InT>::decode(rv[r], x);
      const float wt = s_w[t];
#pragma unroll
      for (int j = 0; j < VW; ++j) x[j] *= wt;
#pragma unroll
      for (int j = 0; j < VW; j += 8 < VW ? 8 : VW) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (j + e < VW) ? x[j + e] : 0.f;
        bf8 hh, ll;
        split8(y, hh, ll);
        if (VW >= 8) {
          *reinterpret_cast<bf8*>(&ws[0][t * LDW + cc + j]) = hh;
          *reinterpret_cast<bf8*>(&ws[1][t * LDW + cc + j]) = ll;
        } else {
          typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<bf4*>(&ws[0][t * LDW + cc + j]) = bf4{hh[0], hh[1], hh[2], hh[3]};
          *reinterpret_cast<bf4*>(&ws[1][t * LDW + cc + j]) = bf4{ll[0], ll[1], ll[2], ll[3]};
        }
      }
    }
    const float tot = s_tot;
    __syncthreads();  // the block's operands are in LDS; the gates are consumed
    if (blk > 0) load_rows(t0 - 64);
    // B_p += X^T W over the block's two 32-token K blocks
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int row = 32 * kq + 8 * g + (n >> 2);  // token row of this lane's first read
      bf8 ah[NMT], al[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int col = 16 * (mt0 + mt) + 4 * (n & 3);
        ah[mt] = tr_pair(&xs[0][row * LDX + col], 4 * LDX);
        al[mt] = tr_pair(&xs[1][row * LDX + col], 4 * LDX);
      }
#pragma unroll
      for (int nt = 0; nt < NNW; ++nt) {
        const int col = 16 * (nt0 + nt) + 4 * (n & 3);
        const bf8 bhi = tr_pair(&ws[0][row * LDW + col], 4 * LDW);
        const bf8 blo = tr_pair(&ws[1][row * LDW + col], 4 * LDW);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          mma_bf16(acc[mt][nt], ah[mt], bhi);
          mma_bf16(acc[mt][nt], ah[mt], blo);
          mma_bf16(acc[mt][nt], al[mt], bhi);
        }
      }
    }
    carry *= tot;
  }
  // the segment's decay for the combine; with the normaliser, the segment's own change of z
  // (plus Gamma_0 z_in for segment 0) in its key slot
  if (tid == 0) s.gam[vh] = carry;
  if (s.zfused) {  // (uniform: every wave reaches the barrier)
    static_assert(NT % GX == 0 && GX <= 64, "one granule column per thread");
#pragma unroll
    for (int o = GX; o < 64; o <<= 1)
#pragma unroll
      for (int j = 0; j < VW; ++j) zp[j] += __shfl_xor(zp[j], o);
    if (lane < GX)
#pragma unroll
      for (int j = 0; j < VW; ++j) s_zb[wave][lane * VW + j] = zp[j];
    __syncthreads();
    if (tid < DK) {
      float zb = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) zb += s_zb[w][tid];
      s.B1_x[vh * DK + tid] = zb + (p == 0 ? carry * s.B0_x[vh * DK + tid] : 0.f);
    }
  }
  // segment 0 also carries the caller's state through the segment's decay
  float* Bo = s.B1_S + vh * DK * DV;
  const float* S0 = p == 0 ? s.B0_S + vh * DK * DV : nullptr;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NNW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t e = (size_t)(16 * (mt0 + mt) + 4 * g + i) * DV + 16 * (nt0 + nt) + n;
        Bo[e] = acc[mt][nt][i] + (S0 != nullptr ? carry * S0[e] : 0.f);
      }
}

// The caller's carried key and flag after a segmented scan whose combine ran before the
// propagate pass (diagonal transitions): the last segment's key, written by that pass.
__global__ __launch_bounds__(NTH) void seg_extras_kernel(SegParams s) {
  const int h = blockIdx.x;
  const size_t last = (size_t)h * s.P + s.P - 1;
  // the last segment's key, or with the normaliser of the fused pass its final z (without
  // the fused pass the normaliser's own kernels write z)
  if ((s.flags & kFlagZnorm) == 0 || s.zfused)
    for (int i = threadIdx.x; i < s.dk; i += NTH) s.xprev_out[(size_t)h * s.dk + i] = s.B1_x[last * s.dk + i];
  if (threadIdx.x == 0) s.has_out[h] = 1;
}

template <typename InT>
hipError_t launch_state_in(const SegParams& s, unsigned grid, hipStream_t st) {
  const dim3 blk(kStateThreads);
  if (s.dk == 64 && s.dv == 64) hipLaunchKernelGGL((seg_state_kernel<InT, 64, 64>), dim3(grid), blk, 0, st, s);
  else if (s.dk == 64) hipLaunchKernelGGL((seg_state_kernel<InT, 64, 128>), dim3(grid), blk, 0, st, s);
  else if (s.dv == 64) hipLaunchKernelGGL((seg_state_kernel<InT, 128, 64>), dim3(grid), blk, 0, st, s);
  else hipLaunchKernelGGL((seg_state_kernel<InT, 128, 128>), dim3(grid), blk, 0, st, s);
  return hipGetLastError();
}

}  // namespace

int scan_segments(size_t BH, size_t T, int dk, int dv, int bf16, int rule, uint32_t flags) {
  (void)dk;
  if (flags & kFlagOutBf16) return 1;
  const bool split = scan_split_path(bf16, flags);
  const bool fused = scan_add_path(bf16, rule, flags);
  const size_t groups = fused ? 1 : split ? (size_t)dv / kSplitCols : ((size_t)dv + 63) / 64;
  const size_t wgs = BH * groups;
  // propagate workgroups resident at once: one per CU; two for the general pair with bf16
  // inputs (and its diagonal rules), whose workgroups fit twice in a CU's LDS and registers
  const bool twice = !fused && !split && (bf16 || seg_diagonal(rule, flags));
  const size_t cap = twice ? 512 : 256;
  const int pmax = (twice && bf16) ? 32 : 16;
  int P = 1;
  while (P < pmax && wgs * 2 * P <= cap && T % (64 * 2 * (size_t)P) == 0 && T / (2 * (size_t)P) >= 512) P *= 2;
  // With a transition pass the propagate work doubles, so fewer than 8 segments do not
  // pay (an additive elu+1 scan with 32 heads, T = 16384, ran no faster with 4 before
  // its transitions were made diagonal); diagonal transitions pay from 2.
  if (seg_diagonal(rule, flags)) return P;
  return P >= 8 ? P : 1;
}

hipError_t launch_seg_init(const SegParams& s, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)s.BH * s.P));
  if (s.bf16) hipLaunchKernelGGL((seg_init_kernel<uint16_t>), grid, dim3(NTH), 0, st, s);
  else hipLaunchKernelGGL((seg_init_kernel<float>), grid, dim3(NTH), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const SegParams& s, hipStream_t st) {
  if (s.diag) {
    const size_t nb = (size_t)s.dk * s.dv / (4 * NTH);
    hipLaunchKernelGGL(seg_combine_diag_kernel, dim3((unsigned)(s.BH * nb)), dim3(NTH), 0, st, s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(s.BH * (s.dv / 16))), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_seg_state(const SegParams& s, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)s.BH * s.P);
  return s.bf16 ? launch_state_in<uint16_t>(s, grid, st) : launch_state_in<float>(s, grid, st);
}

hipError_t launch_seg_extras(const SegParams& s, hipStream_t st) {
  if (s.S_out == nullptr) return hipSuccess;
  hipLaunchKernelGGL(seg_extras_kernel, dim3((unsigned)s.BH), dim3(NTH), 0, st, s);
  return hipGetLastError();
}

}  // namespace fwmem
