// Fused chunked scan of the additive rule with a scalar retention: linear attention
// ("attention is also an FFN", sections 2.1 and 3.2) with the per-token retention gamma_t
// and write scale beta_t of the inner-product family ("Fast Weight Attention for
// Continual Learning" reading notes, sections 4.3 and 4.4):
//   S_t = gamma_t S_{t-1} + beta_t phi(k_t) v_t^T,   o_t = S_t^T phi(q_t).
// Chunks of C = 64 tokens. With g_t = prod_{u <= t} gamma_u inside the chunk (kept as a
// log2-sum and a sign parity, the chunk-local log prefix of section 4.4) and S the state
// at chunk entry:
//   O  = diag(g) Q S + (P o D) V,   P_ts = phi(q_t) . phi(k_s),  D_ts = (g_t / g_s) beta_s  (s <= t)
//   S' = g_C S + K^T diag(beta_s g_C / g_s) V.
// There is no triangular solve, so the only dependency between chunks is S -> S', a
// scaled add. One workgroup per head owns all value columns (one wave per 16 columns,
// its slice of S in registers) and forms every product of a chunk on MFMA itself: no
// prep pass and no workspace record. The Gram tile P is built once per chunk as P^T
// tiles, whose accumulator layout is already the A operand of P V (split_c's K order),
// and shared through LDS as six operand fragments.
//
// Operands (v_mfma_f32_16x16x32_bf16): raw bf16 values are exact; phi(q), phi(k) under
// elu + 1, the masked P, the state S and the scaled values are carried as bf16 hi + lo
// pairs (fwmem_split.h), and a product of two split operands is hi.hi + hi.lo + lo.hi.
//
// Per chunk and workgroup: the next chunk's rows are loaded into registers while this
// one computes; two barriers (after staging, after the P fragments).
//
// The normaliser ("attention is also an FFN", section 4.2): o_t = S_t^T phi(q_t) /
// (z_t . phi(q_t) + eps) with z_t = gamma_t z_{t-1} + beta_t phi(k_t), z carried in the
// state's key slot. In the chunk's terms, z_t . phi(q_t) = g_t (phi(q_t) . z) + the row
// sum of P o D, and z' = g_C z + sum_s w_s phi(k_s). The waves that form the P fragments
// add up their rows' sums, every wave takes a share of the dot products phi(q_t) . z and of
// the sums w_s phi(k_s) (LDS atomics), and the outputs are divided before they are stored.
#include "fwmem_device.h"
#include "fwmem_internal.h"
#include "fwmem_split.h"

namespace fwmem {
namespace {

constexpr int CH = kChunk;

template <int DK, int DV, bool ELU>
struct AddLds {
  static constexpr int LDQ = DK + 8;      // bf16 row stride of the phi(q), phi(k) tiles
  static constexpr int LDV = DV + 8;      // bf16 row stride of the value tile
  static constexpr int NPL = ELU ? 2 : 1; // planes of phi(q), phi(k): hi (or raw), lo
  static constexpr size_t kQ = 0;                                     // uint16 [NPL][CH][LDQ]
  static constexpr size_t kK = kQ + (size_t)NPL * CH * LDQ * 2;       // uint16 [NPL][CH][LDQ]
  static constexpr size_t kV = kK + (size_t)NPL * CH * LDQ * 2;       // uint16 [CH][LDV]
  static constexpr size_t kP = kV + (size_t)CH * LDV * 2;             // [kTriFrags][hi, lo][64 lanes] x 16 B
  static constexpr size_t kS = kP + (size_t)kTriFrags * 2 * 64 * 16;  // float l, beta, g, w [CH]; int parity [CH]
  // the normaliser: z at the chunk start (two buffers), the chunk's sum w_s phi(k_s),
  // phi(q_t) . z, and the row sums of P o D by fragment
  static constexpr size_t kZ = kS + 5 * CH * 4;                       // float [2][DK]
  static constexpr size_t kZn = kZ + 2 * DK * 4;                      // float [DK]
  static constexpr size_t kQz = kZn + DK * 4;                         // float [CH]
  static constexpr size_t kRs = kQz + CH * 4;                         // float [kTriFrags][16]
  // each wave's outputs, turned from the accumulator layout into rows for 16-byte stores
  static constexpr int LDO = 16 + 4;
  static constexpr size_t kO = kRs + kTriFrags * 16 * 4;              // float [DV / 16][CH][LDO]
  static constexpr size_t kBytes = kO + (size_t)(DV / 16) * CH * LDO * 4;
};

__device__ __forceinline__ float bf8_at(const bf8& v, int j) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  return bf16_bits_to_f32((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
}

// Inclusive prefix over the 64 lanes of a wave of (log2 |gamma|, count of negative gamma).
__device__ __forceinline__ void lane_prefix(float& la, int& ng) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(la, o);
    const int z = __shfl_up(ng, o);
    if (lane >= o) {
      la += y;
      ng += z;
    }
  }
}

// Workgroup barrier for LDS: waits for this wave's LDS operations only. The kernel's
// barriers order LDS traffic alone; a plain __syncthreads would also wait for the next
// chunk's rows in flight and for the previous chunk's output stores to be acknowledged.
static __device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DK, int DV, bool ELU, bool ZN>
__global__ __launch_bounds__(4 * DV) void add_kernel(ScanParams p) {
  using L = AddLds<DK, DV, ELU>;
  constexpr int NT = 4 * DV, NW = DV / 16, NRT = DK / 16, NKB = DK / 32;
  constexpr int LDQ = L::LDQ, LDV = L::LDV;
  static_assert(L::kBytes <= 160 * 1024, "LDS");
  __shared__ __align__(16) char smem[L::kBytes];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem + L::kQ);  // plane 0: hi (raw without elu); plane 1: lo
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + L::kK);
  uint16_t* Vs = reinterpret_cast<uint16_t*>(smem + L::kV);
  u32x4* Pf = reinterpret_cast<u32x4*>(smem + L::kP);
  float* s_l = reinterpret_cast<float*>(smem + L::kS);  // in-chunk inclusive prefix of log2 |gamma|
  float* s_b = s_l + CH;                                // beta (0 past the sequence end)
  float* s_g = s_b + CH;                                // g_t (signed)
  float* s_w = s_g + CH;                                // beta_t g_C / g_t (signed)
  int* s_par = reinterpret_cast<int*>(s_w + CH);        // sign parity of the prefix
  float* s_z = reinterpret_cast<float*>(smem + L::kZ);
  float* s_zn = reinterpret_cast<float*>(smem + L::kZn);
  float* s_qz = reinterpret_cast<float*>(smem + L::kQz);
  float* s_rs = reinterpret_cast<float*>(smem + L::kRs);

  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int col = 16 * wave + n;  // the lane's value column
  float* s_o = reinterpret_cast<float*>(smem + L::kO) + wave * CH * L::LDO;  // this wave's output rows
  const size_t rowbase = (size_t)bh * p.T;
  const uint16_t* qbase = static_cast<const uint16_t*>(p.q) + rowbase * DK;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + rowbase * DV;
  // rows past the sequence end read as zeros and their output stores are dropped
  const __amdgpu_buffer_rsrc_t rq = rsrc(qbase, (uint32_t)((size_t)p.T * DK * 2));
  const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, (uint32_t)((size_t)p.T * DK * 2));
  const __amdgpu_buffer_rsrc_t rv = rsrc(vbase, (uint32_t)((size_t)p.T * DV * 2));
  const bool obf = (p.flags & kFlagOutBf16) != 0;
  const uint32_t oes = obf ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(static_cast<const char*>(p.out) + rowbase * DV * oes, (uint32_t)((size_t)p.T * DV * oes));

  f4 s[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[rt][i] = p.S_in != nullptr ? p.S_in[((size_t)bh * DK + 16 * rt + 4 * g + i) * DV + col] : 0.f;

  // ---- loads of one chunk into registers: 16-byte granules of the q, k and v rows, and
  // the raw gates of token tid (tid < CH)
  constexpr int GQ = DK / 8, GV = DV / 8;  // granules per row
  constexpr int NGQ = CH * GQ / NT, NGV = CH * GV / NT;
  static_assert(NGQ >= 1 && NGV >= 1 && (CH * GQ) % NT == 0 && (CH * GV) % NT == 0, "granules");
  uint32_t oq[NGQ], ov[NGV];
#pragma unroll
  for (int r = 0; r < NGQ; ++r) {
    const int gi = tid + NT * r;
    oq[r] = (uint32_t)(((gi / GQ) * DK + (gi % GQ) * 8) * 2);
  }
#pragma unroll
  for (int r = 0; r < NGV; ++r) {
    const int gi = tid + NT * r;
    ov[r] = (uint32_t)(((gi / GV) * DV + (gi % GV) * 8) * 2);
  }
  u32x4 pq[NGQ], pk[NGQ], pv[NGV];
  float gbeta = 0.f, ggam = 1.f;
  auto prefetch = [&](int cn) {
    const uint32_t sq = (uint32_t)cn * (uint32_t)(CH * DK * 2), sv = (uint32_t)cn * (uint32_t)(CH * DV * 2);
#pragma unroll
    for (int r = 0; r < NGQ; ++r) {
      pq[r] = bload16(rq, oq[r], sq);
      pk[r] = bload16(rk, oq[r], sq);
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) pv[r] = bload16(rv, ov[r], sv);
    if (tid < CH) {
      const int tau = cn * CH + tid;
      gbeta = 0.f;  // past the end: no write and no decay
      ggam = 1.f;
      if (tau < p.T) {  // raw here; activated when staged, so the loads stay in flight
        gbeta = p.beta != nullptr ? p.beta[rowbase + tau] : 1.f;
        ggam = p.lam != nullptr ? p.lam[rowbase + tau] : 1.f;
      }
    }
  };

  // the normaliser: thread tid < DK keeps z[tid]
  float zreg = 0.f;
  if (ZN && tid < DK) {
    zreg = p.xprev_in != nullptr ? p.xprev_in[(size_t)bh * DK + tid] : 0.f;
    s_z[tid] = zreg;
    s_zn[tid] = 0.f;
  }

  prefetch(0);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * CH;
    // ---- registers -> LDS: phi(q), phi(k) (split under elu + 1), raw values, token scalars
#pragma unroll
    for (int r = 0; r < NGQ; ++r) {
      const int gi = tid + NT * r, t = gi / GQ, cc = (gi % GQ) * 8;
      if constexpr (ELU) {
        float xq[8], xk[8];
        In<uint16_t>::decode(pq[r], xq);
        In<uint16_t>::decode(pk[r], xk);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xq[j] = phi_elu1(xq[j]);
          xk[j] = phi_elu1(xk[j]);
        }
        bf8 h, l;
        split8(xq, h, l);
        *reinterpret_cast<bf8*>(Qs + t * LDQ + cc) = h;
        *reinterpret_cast<bf8*>(Qs + CH * LDQ + t * LDQ + cc) = l;
        split8(xk, h, l);
        *reinterpret_cast<bf8*>(Ks + t * LDQ + cc) = h;
        *reinterpret_cast<bf8*>(Ks + CH * LDQ + t * LDQ + cc) = l;
      } else {
        *reinterpret_cast<u32x4*>(Qs + t * LDQ + cc) = pq[r];
        *reinterpret_cast<u32x4*>(Ks + t * LDQ + cc) = pk[r];
      }
    }
#pragma unroll
    for (int r = 0; r < NGV; ++r) {
      const int gi = tid + NT * r;
      *reinterpret_cast<u32x4*>(Vs + (gi / GV) * LDV + (gi % GV) * 8) = pv[r];
    }
    if (wave == 0) {
      const bool live = c * CH + lane < p.T;
      const float gb = live && p.beta != nullptr ? act_beta(gbeta, p.flags) : gbeta;
      const float gm = live && p.lam != nullptr ? act_lam(ggam, p.flags, false) : ggam;
      float la = __builtin_amdgcn_logf(fmaxf(fabsf(gm), 1e-30f));
      int ng = gm < 0.f ? 1 : 0;
      lane_prefix(la, ng);
      const float lc = __shfl(la, CH - 1);
      const int pc = __shfl(ng, CH - 1) & 1;
      s_l[lane] = la;
      s_par[lane] = ng & 1;
      s_b[lane] = gb;
      s_g[lane] = with_sign(__builtin_amdgcn_exp2f(la), ng & 1);
      s_w[lane] = gb * with_sign(__builtin_amdgcn_exp2f(lc - la), pc ^ (ng & 1));
    }
    lds_barrier();
    if (c + 1 < p.nchunks) prefetch(c + 1);

    // ---- P^T tiles (rows s, columns t) of the lower triangle, masked: fragment f of the
    // P V operand (row tile mt, token block kq) is the tile pair (2 kq, mt), (2 kq + 1, mt)
    // fragments f = 1, 2, 4, 5 hold two tiles, 0 and 3 one; waves w and w + 4 share a SIMD
    for (int fi = wave; fi < kTriFrags; fi += NW) {
      constexpr int kOrder[kTriFrags] = {1, 2, 4, 5, 3, 0};
      const int f = kOrder[fi];
      const int mt = tri_m(f), kq = tri_kb(f);
      const int t = 16 * mt + n;
      const float lt = s_l[t];
      const int pt = s_par[t];
      float x[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nt = 2 * kq + h;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        if (nt <= mt) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const uint16_t* ka = Ks + (16 * nt + n) * LDQ + 32 * kb + 8 * g;
            const uint16_t* qb = Qs + (16 * mt + n) * LDQ + 32 * kb + 8 * g;
            const bf8 a = *reinterpret_cast<const bf8*>(ka);
            const bf8 b = *reinterpret_cast<const bf8*>(qb);
            mma_bf16(acc, a, b);
            if constexpr (ELU) {
              mma_bf16(acc, a, *reinterpret_cast<const bf8*>(qb + CH * LDQ));
              mma_bf16(acc, *reinterpret_cast<const bf8*>(ka + CH * LDQ), b);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sk = 16 * nt + 4 * g + i;
          const float d = s_b[sk] * with_sign(__builtin_amdgcn_exp2f(lt - s_l[sk]), pt ^ s_par[sk]);
          x[4 * h + i] = sk <= t ? acc[i] * d : 0.f;
        }
      }
      bf8 hi, lo;
      split8(x, hi, lo);
      Pf[(2 * f) * 64 + lane] = __builtin_bit_cast(u32x4, hi);
      Pf[(2 * f + 1) * 64 + lane] = __builtin_bit_cast(u32x4, lo);
      if constexpr (ZN) {  // this fragment's part of the row sums of P o D, rows 16 mt + n
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) rs += x[j];
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        if (g == 0) s_rs[16 * f + n] = rs;
      }
    }

    if constexpr (ZN) {
      // phi(q_t) . z: TPT threads per token, each over DK / TPT dimensions of the split rows
      constexpr int TPT = NT / CH, DPT = DK / TPT;
      const float* zc = s_z + (c & 1) * DK;
      {
        const int t = tid / TPT, d0 = (tid % TPT) * DPT;
        float a = 0.f;
#pragma unroll
        for (int d = 0; d < DPT; d += 8) {
          const u32x4 h = *reinterpret_cast<const u32x4*>(Qs + t * LDQ + d0 + d);
          const u32x4 l = *reinterpret_cast<const u32x4*>(Qs + CH * LDQ + t * LDQ + d0 + d);
          const f4 z0 = *reinterpret_cast<const f4*>(zc + d0 + d), z1 = *reinterpret_cast<const f4*>(zc + d0 + d + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t wh = h[j >> 1], wl = l[j >> 1];
            const float q = bf16_bits_to_f32((j & 1) ? wh >> 16 : wh & 0xffffu) +
                            bf16_bits_to_f32((j & 1) ? wl >> 16 : wl & 0xffffu);
            a += q * (j < 4 ? z0[j] : z1[j - 4]);
          }
        }
#pragma unroll
        for (int o = 1; o < TPT; o <<= 1) a += __shfl_xor(a, o);
        if (tid % TPT == 0) s_qz[t] = a;
      }
      // sum_s w_s phi(k_s): thread (d, part) over the part's CH * DK / NT tokens
      {
        constexpr int NPART = NT / DK, TPP = CH / NPART;
        const int d = tid % DK, t0p = (tid / DK) * TPP;
        float a = 0.f;
#pragma unroll 4
        for (int t = t0p; t < t0p + TPP; ++t)
          a += s_w[t] * (bf16_bits_to_f32(Ks[t * LDQ + d]) + bf16_bits_to_f32(Ks[CH * LDQ + t * LDQ + d]));
        atomicAdd(&s_zn[d], a);
      }
    }

    // ---- O = diag(g) (Q S) (C layout: rows 16 mt + 4 g + i, column n)
    f4 O[4];
    {
      bf8 sh[NKB], sl[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) split_c(s, kb, sh[kb], sl[kb]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        O[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint16_t* qa = Qs + (16 * mt + n) * LDQ + 32 * kb + 4 * g;
          const bf8 a = frag_pair(qa);
          mma_bf16(O[mt], a, sh[kb]);
          mma_bf16(O[mt], a, sl[kb]);
          if constexpr (ELU) mma_bf16(O[mt], frag_pair(qa + CH * LDQ), sh[kb]);
        }
        O[mt] *= *reinterpret_cast<const f4*>(s_g + 16 * mt + 4 * g);
      }
    }

    // ---- S' = g_C S + K^T (w o V), w_s = beta_s g_C / g_s. The value fragments (tokens in
    // split_c's K order, column n) serve the update scaled and split, and P V raw.
    bf8 vf[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
      vf[kq] = xt_frag(Vs + (32 * kq + 4 * g + (n >> 2)) * LDV + 16 * wave + 4 * (n & 3), LDV);
    {
      bf8 vh[2], vl[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const f4 w0 = *reinterpret_cast<const f4*>(s_w + 32 * kq + 4 * g);
        const f4 w1 = *reinterpret_cast<const f4*>(s_w + 32 * kq + 16 + 4 * g);
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = bf8_at(vf[kq], j) * w0[j];
          x[4 + j] = bf8_at(vf[kq], 4 + j) * w1[j];
        }
        split8(x, vh[kq], vl[kq]);
      }
      const float gC = s_g[CH - 1];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const uint16_t* ka = Ks + (32 * kq + 4 * g + (n >> 2)) * LDQ + 16 * rt + 4 * (n & 3);
          const bf8 a = xt_frag(ka, LDQ);
          mma_bf16(acc, a, vh[kq]);
          mma_bf16(acc, a, vl[kq]);
          if constexpr (ELU) mma_bf16(acc, xt_frag(ka + CH * LDQ, LDQ), vh[kq]);
        }
        s[rt] = s[rt] * gC + acc;
      }
    }
    lds_barrier();  // the P fragments are complete

    // ---- O += (P o D) V, stored. The next chunk's staging only begins after every wave
    // has passed this chunk's second barrier, and nothing below reads LDS except the P
    // fragments, which the next chunk rewrites after its first barrier.
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) {
      const int mt = tri_m(f), kq = tri_kb(f);
      mma_bf16(O[mt], __builtin_bit_cast(bf8, Pf[(2 * f) * 64 + lane]), vf[kq]);
      mma_bf16(O[mt], __builtin_bit_cast(bf8, Pf[(2 * f + 1) * 64 + lane]), vf[kq]);
    }
    if constexpr (ZN) {
      // z_t . phi(q_t) = g_t (phi(q_t) . z) + the row sums of P o D (fragments f of row tile mt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * mt + 4 * g + i, r = 4 * g + i;
          float den = s_g[t] * s_qz[t];
#pragma unroll
          for (int f = 0; f < kTriFrags; ++f)
            if (tri_m(f) == mt) den += s_rs[16 * f + r];
          O[mt][i] *= __builtin_amdgcn_rcpf(den + p.eps);
        }
      if (tid < DK) {  // z at the next chunk's start
        zreg = s_g[CH - 1] * zreg + s_zn[tid];
        s_z[((c + 1) & 1) * DK + tid] = zreg;
        s_zn[tid] = 0.f;
      }
    }
    // ---- the outputs through the wave's own LDS rows: lane r then stores row t0 + r of the
    // wave's 16 columns in 16-byte pieces (the wave's LDS operations complete in order)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[(16 * mt + 4 * g + i) * L::LDO + n] = O[mt][i];
    {
      f4 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = *reinterpret_cast<const f4*>(s_o + lane * L::LDO + 4 * j);
      const uint32_t so = (uint32_t)((t0 + lane) * DV + 16 * wave);  // element offset of the row piece
      if (obf) {
        u32x4 b[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j >> 1][2 * (j & 1)] = (uint32_t)f32_to_bf16_bits(r[j][0]) | ((uint32_t)f32_to_bf16_bits(r[j][1]) << 16);
          b[j >> 1][2 * (j & 1) + 1] = (uint32_t)f32_to_bf16_bits(r[j][2]) | ((uint32_t)f32_to_bf16_bits(r[j][3]) << 16);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b[h]), ro, 2u * so + 16u * h, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r[j]), ro, 4u * so + 16u * j, 0, 0);
      }
    }
  }

  if (p.S_out != nullptr) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.S_out[((size_t)bh * DK + 16 * rt + 4 * g + i) * DV + col] = s[rt][i];
    if (ZN) {  // with the normaliser the key slot holds z
      if (tid < DK) p.xprev_out[(size_t)bh * DK + tid] = zreg;
      if (tid == 0) p.has_out[bh] = 1;
    } else {
      const uint16_t* kl = kbase + (size_t)(p.T - 1) * DK;
      for (int i = tid; i < DK; i += NT) {
        float x = In<uint16_t>::load1(kl + i);
        if (ELU) x = phi_elu1(x);
        p.xprev_out[(size_t)bh * DK + i] = x;
      }
      if (tid == 0) p.has_out[bh] = 1;
    }
  }
}

template <int DK, int DV>
hipError_t launch_add_t(const ScanParams& p, hipStream_t st) {
  const dim3 grid((unsigned)p.BH), block(4 * DV);
  if (p.flags & kFlagZnorm) hipLaunchKernelGGL((add_kernel<DK, DV, true, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((add_kernel<DK, DV, true, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool scan_add_path(int bf16, int rule, uint32_t flags) {
  return bf16 != 0 && rule == kRuleAdditive && (flags & kFlagPhiElu1) != 0 && (flags & kFlagPerChannel) == 0;
}

hipError_t launch_scan_add(const ScanParams& p, hipStream_t st) {
  if (p.dk == 64) return p.dv == 64 ? launch_add_t<64, 64>(p, st) : launch_add_t<64, 128>(p, st);
  return p.dv == 64 ? launch_add_t<128, 64>(p, st) : launch_add_t<128, 128>(p, st);
}

}  // namespace fwmem
