// Prep kernel of the split path (bf16 inputs, identity feature map, scalar decay): one
// workgroup per (head, chunk) builds the chunk's record (RecSplit) from its keys,
// queries and gates.
//
// With Gamma_t the decay since the chunk start ("Fast Weight Attention for Continual
// Learning" reading notes, sections 4.1-4.4; the algebra is derived in fwmem_scan.hip):
//   L_ts = eta_t (Gamma_{t-1}/Gamma_s) x_t . x_s  (s < t),   T = (I + L)^-1  (delta rule;
//   the inner-product rule shares the shifted keys and eta_t but has no solve)
//   M_ts = (Gamma_t / Gamma_s) q_t . x_s          (s <= t)
// and the per-token row factors fP = eta Gamma_{t-1}, fV = eta, fO = Gamma_t,
// fU = Gamma_C / Gamma_t with Gamma_C the decay over the whole chunk.
// With normalised queries and keys (QKN) the raw rows stay the operands: x_t and q_t are
// used as nx_t x_t and mq_t q_t, so L_ts and M_ts take the factors nx_t nx_s and
// mq_t nx_s, fP and fU take nx_t, fO takes mq_t, and |x_t|^2 in eta becomes
// nx_t^2 |x_t|^2. The propagate kernel is unchanged.
//
// Steps (4 waves):
//   1. X and Q rows arrive in LDS by direct loads (rows past the sequence end read as
//      zeros); wave 0 loads the gates.
//   2. Gram products X X^T and Q X^T on bf16 MFMA: the products of bf16 values are exact
//      and accumulate in fp32. The diagonal of X X^T gives |x_t|^2.
//   3. Wave 0 forms eta_t, the decay prefix (log-sum and sign parity) and the row factors.
//   4. The masked L and M are written to LDS in fp32.
//   5. T = (I + L)^-1 by 16x16 blocks: wave b inverts diagonal block b by forward
//      substitution, then wave j forms column block j of T,
//        T_ij = -D_i sum_{k=j}^{i-1} L_ik T_kj,
//      on fp32 MFMA from LDS and its own registers, with no further synchronisation.
//   6. T and M are written to the record as bf16 hi/lo A fragments.
#include "fwmem_internal.h"
#include "fwmem_split.h"

namespace fwmem {
namespace {

constexpr int CH = kChunk;
constexpr int NTP = 256;

// fp32 [64][64] matrix in LDS: element (r, c) at r * 64 + (c ^ 4 (r % 16)); groups of
// four aligned columns stay contiguous.
__device__ __forceinline__ int mat_idx(int r, int c) { return r * 64 + (c ^ ((r & 15) << 2)); }

constexpr int kRegion = 16384;  // bytes of each of the two LDS regions

// Lower 16x16 tiles of a 64x64 matrix, in row order: tile -> (row tile, column tile).
__device__ constexpr int low_mt(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__device__ constexpr int low_nt(int t) { return t - (low_mt(t) * (low_mt(t) + 1)) / 2; }

// C += A B for 16x16 blocks in fp32 MFMA: lane (g, n) supplies A[n][4g..4g+3] (a) and
// B[4g+q][n] (b, the C layout of a previous product).
__device__ __forceinline__ void mma_f32_block(f4& acc, const f4& a, const f4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], acc, 0, 0, 0);
}

// Column block J of T: T_ij for i = J+1..3 (wave J), given D_J (= T_JJ, B layout) in Tc[J].
template <int J>
__device__ __forceinline__ void t_column_block(const float* Lf, float* Tf, f4 (&Tc)[4], int g, int n) {
#pragma unroll
  for (int i = J + 1; i < 4; ++i) {
    f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = J; k < i; ++k) {
      const f4 a = *reinterpret_cast<const f4*>(&Lf[mat_idx(16 * i + n, 16 * k + 4 * g)]);
      mma_f32_block(y, a, Tc[k]);
    }
    const f4 d = *reinterpret_cast<const f4*>(&Tf[mat_idx(16 * i + n, 16 * i + 4 * g)]);
    f4 t = {0.f, 0.f, 0.f, 0.f};
    mma_f32_block(t, d, y);
    Tc[i] = -t;
#pragma unroll
    for (int q = 0; q < 4; ++q) Tf[mat_idx(16 * i + 4 * g + q, 16 * J + n)] = -t[q];
  }
}

// A lower-triangular fp32 [64][64] matrix in LDS (mat_idx layout) to the record as its
// six split A fragments: fragment f, lane ln holds row tok_of(m_f, ln % 16), K columns
// 32 kb_f + 8 (ln / 16) .. +7; hi at 2f, lo at 2f+1.
template <size_t OFF>
__device__ __forceinline__ void split_to_record(const float* src, char* rec, int tid) {
#pragma unroll
  for (int r = 0; r < (kTriFrags * 64 + NTP - 1) / NTP; ++r) {
    const int task = tid + NTP * r;
    if (task < kTriFrags * 64) {
      const int f = task >> 6, ln = task & 63;
      const int row = tok_of(tri_m(f), ln & 15), k0 = 32 * tri_kb(f) + 8 * (ln >> 4);
      const f4 x0 = *reinterpret_cast<const f4*>(&src[mat_idx(row, k0)]);
      const f4 x1 = *reinterpret_cast<const f4*>(&src[mat_idx(row, k0 + 4)]);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      bf8 hi, lo;
      split8(x, hi, lo);
      u32x4* dst = reinterpret_cast<u32x4*>(rec + OFF) + (2 * f) * 64 + ln;
      dst[0] = __builtin_bit_cast(u32x4, hi);
      dst[64] = __builtin_bit_cast(u32x4, lo);
    }
  }
}

template <int DK, int RULE, bool QKN>
__global__ __launch_bounds__(NTP) void prep_split_kernel(ScanParams p) {
  using RC = RecSplit<DK>;
  using R = Rule<RULE>;
  constexpr int NGR = DK / 8;          // 16-byte granules per X / Q row
  constexpr int NKD = DK / 32;         // K blocks over d_k
  constexpr int NI = CH * NGR / 64;    // direct loads per tile
  static_assert(CH * DK * 2 <= kRegion, "tile fits a region");
  // Two regions: X, then L; Q, then M, then T (once M is in the record). 33 KiB in all,
  // so that four workgroups share a CU.
  __shared__ __align__(16) char smem[2 * kRegion + (QKN ? 7 : 4) * CH * 4];
  u32x4* Xs = reinterpret_cast<u32x4*>(smem);
  u32x4* Qs = reinterpret_cast<u32x4*>(smem + kRegion);
  float* Lf = reinterpret_cast<float*>(smem);            // after the Gram products
  float* Mf = reinterpret_cast<float*>(smem + kRegion);  // after the Gram products
  float* Tf = Mf;                                        // after M's split
  float* s_diag = reinterpret_cast<float*>(smem + 2 * kRegion);
  float* s_eta = s_diag + CH;
  float* s_g = s_eta + CH;
  float* s_sg = s_g + CH;
  float* s_qd = s_sg + CH;  // QKN: |q_t|^2, then the rescale factors of x_t and q_t
  float* s_n = s_qd + CH;
  float* s_m = s_n + CH;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int c = __builtin_amdgcn_readfirstlane(blockIdx.x % p.nchunks);
  const int bh = __builtin_amdgcn_readfirstlane(blockIdx.x / p.nchunks);
  const int t0 = c * CH, T = p.T;
  const size_t rowbase = (size_t)bh * T;
  const bool has_in = p.has_in != nullptr && p.has_in[bh] != 0;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k) + rowbase * DK;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q) + rowbase * DK;
  char* rec = p.ws + ((size_t)bh * p.nchunks + c) * RC::kBytes;

  // ---- 1. rows into LDS (X starts one row early for the shifted pair: x_t = k_{t-1})
  {
    const __amdgpu_buffer_rsrc_t rx = rsrc(R::shift ? kb - DK : kb, (uint32_t)(T * DK * 2));
    const __amdgpu_buffer_rsrc_t rq = rsrc(qb, (uint32_t)(T * DK * 2));
    const uint32_t so = (uint32_t)(t0 * DK * 2);
#pragma unroll
    for (int ii = 0; ii < NI / 4; ++ii) {
      const int i = ii * 4 + wave;
      const int pos = 64 * i + lane;
      const int row = pos / NGR;
      const uint32_t off = (uint32_t)(row * DK + 8 * ((pos % NGR) ^ xswz<DK>(row))) * 2u;
      // the row before token 0 is the carried key, written below
      dma16(rx, (R::shift && c == 0 && row == 0) ? 0x80000000u : off, so, &Xs[64 * i]);
      dma16(rq, off, so, &Qs[64 * i]);
    }
  }
  float g_beta = 0.f, g_lam = 0.f;
  if (wave == 0 && t0 + lane < T) {
    g_beta = p.beta != nullptr ? act_beta(p.beta[rowbase + t0 + lane], p.flags) : 1.f;
    if (p.lam != nullptr) g_lam = act_lam(p.lam[rowbase + t0 + lane], p.flags, R::nlms);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (R::shift && c == 0 && tid < NGR) {
    // threads tid < NGR issued the loads of row 0, so their own wait covers them
    u32x4 w = {0u, 0u, 0u, 0u};
    if (has_in) {
      const float* x0 = p.xprev_in + (size_t)bh * DK + 8 * tid;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)f32_to_bf16_bits(x0[2 * j]) | ((uint32_t)f32_to_bf16_bits(x0[2 * j + 1]) << 16);
    }
    Xs[tid ^ xswz<DK>(0)] = w;
  }
  __syncthreads();

  // ---- 2. Gram products: jobs over the 10 lower 16x16 tiles of X X^T (its diagonal
  // gives |x_t|^2, its lower part L for the delta rule; needed by the shifted pair and by
  // QKN), the 10 lower tiles of Q X^T, and with QKN the 4 diagonal tiles of Q Q^T
  // (|q_t|^2). Job kinds: 0 X X^T, 1 Q X^T, 2 Q Q^T.
  constexpr int NG = (R::shift || QKN) ? 10 : 0;
  constexpr int NJ = NG + 10 + (QKN ? 4 : 0);
  constexpr int JPW = (NJ + 3) / 4;
  auto job_kind = [&](int job) { return job < NG ? 0 : (job < NG + 10 ? 1 : 2); };
  auto job_tile = [&](int job, int& mt, int& nt) {
    if (job < NG + 10) {
      const int tile = job < NG ? job : job - NG;
      mt = low_mt(tile);
      nt = low_nt(tile);
    } else {
      mt = nt = job - NG - 10;
    }
  };
  auto rowfrag = [&](const u32x4* S, int row, int kq) -> bf8 {
    return __builtin_bit_cast(bf8, S[row * NGR + ((4 * kq + g) ^ xswz<DK>(row))]);
  };
  f4 acc[JPW];
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int job = jj * 4 + wave;
    acc[jj] = f4{0.f, 0.f, 0.f, 0.f};
    if (job < NJ) {
      const int kind = job_kind(job);  // wave-uniform
      int mt, nt;
      job_tile(job, mt, nt);
      const u32x4* A = kind == 0 ? Xs : Qs;
      const u32x4* Bm = kind == 2 ? Qs : Xs;
#pragma unroll
      for (int kq = 0; kq < NKD; ++kq)
        mma_bf16(acc[jj], rowfrag(A, 16 * mt + n, kq), rowfrag(Bm, 16 * nt + n, kq));
      if (kind != 1 && mt == nt && (n >> 2) == g) {
        const int i = n & 3;
        const float d = i == 0 ? acc[jj][0] : i == 1 ? acc[jj][1] : i == 2 ? acc[jj][2] : acc[jj][3];
        (kind == 0 ? s_diag : s_qd)[16 * mt + n] = d;
      }
    }
  }
  __syncthreads();  // diagonal complete; X and Q no longer read

  // ---- 3. token scalars and row factors (wave 0, lane = token)
  if (wave == 0) {
    const int t = lane, tau = t0 + t;
    const bool active = tau < T;
    // QKN: x_t and q_t are used rescaled by nx and mq (to length qk_length); the raw bf16
    // rows stay the MFMA operands and the factors go into the masks and row factors.
    float nx = 1.f, mq = 1.f, xx = s_diag[t];
    if (QKN) {
      const float len = qk_length(p.flags, DK);
      nx = rescale_factor(s_diag[t], len);
      mq = rescale_factor(s_qd[t], len);
      xx = s_diag[t] * nx * nx;
      s_n[t] = nx;
      s_m[t] = mq;
    }
    float eta = 0.f, a = 1.f;
    if (R::nlms) {
      const bool hasx = active && (tau >= 1 || has_in);
      // scale-coupled ridge: the base ridge times the written key's energy
      const float lam = (p.flags & kFlagLamScaled) ? g_lam * xx : g_lam;
      if (hasx) eta = g_beta / (xx + lam + p.eps);
      a = 1.f - eta * lam;
    } else {
      if (active) eta = g_beta;
      if (active && p.lam != nullptr) a = g_lam;
    }
    float la = log_abs_floor(a);
    int ng = a < 0.f ? 1 : 0;
    wave_prefix(la, ng);
    const float sg = (ng & 1) ? -1.f : 1.f;
    s_eta[t] = eta;
    s_g[t] = la;
    s_sg[t] = sg;
    float gprev = __shfl_up(la, 1), sprev = __shfl_up(sg, 1);
    if (t == 0) {
      gprev = 0.f;
      sprev = 1.f;
    }
    const float gC = __shfl(la, CH - 1), sC = __shfl(sg, CH - 1);
    float* fac = reinterpret_cast<float*>(rec + RC::kFac);
    fac[t] = eta * sprev * __expf(gprev) * nx;
    fac[CH + t] = eta;
    fac[2 * CH + t] = sg * __expf(la) * mq;
    fac[3 * CH + t] = sC * sg * __expf(gC - la) * nx;
    // row 4: [Gamma_C, has_prev, Gamma_C of the next chunk, 0...]. Slot 2 of a record is
    // written by the next chunk's workgroup (1 for the last chunk), so that the propagate
    // kernel knows the next decay one chunk early.
    const float gamma_c = sC * __expf(gC);
    const bool last = c + 1 == p.nchunks;
    if (t != 2 || last)
      fac[4 * CH + t] = t == 0 ? gamma_c : (t == 1 ? (has_in ? 1.f : 0.f) : (t == 2 ? 1.f : 0.f));
    if (t == 2 && c > 0) reinterpret_cast<float*>(rec - RC::kBytes + RC::kFac)[4 * CH + 2] = gamma_c;
  }
  __syncthreads();

  // ---- 4. masked L (delta) and M, fp32, into LDS; zero the two upper 16x16 tiles that
  // the output fragments cover (row tiles 0 / 2, column tiles 1 / 3). The token scalars
  // of every job are read before the first store (the stores could alias them).
  float sc_g[JPW][4], sc_sg[JPW][4], sc_eta[JPW][4], sc_gp[JPW][4], sc_sp[JPW][4], sc_gs[JPW], sc_ss[JPW];
  float sc_r[JPW][4], sc_ns[JPW];  // QKN: the row's and the column's rescale factors
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int job = jj * 4 + wave;
    int mt, nt;
    job_tile(job < NJ ? job : 0, mt, nt);
    const bool gram = job_kind(job) == 0;
    const int s = 16 * nt + n;
    sc_gs[jj] = s_g[s];
    sc_ss[jj] = s_sg[s];
    sc_ns[jj] = QKN ? s_n[s] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g + i;
      sc_g[jj][i] = s_g[t];
      sc_sg[jj][i] = s_sg[t];
      sc_eta[jj][i] = s_eta[t];
      sc_gp[jj][i] = t ? s_g[t - 1] : 0.f;
      sc_sp[jj][i] = t ? s_sg[t - 1] : 1.f;
      sc_r[jj][i] = QKN ? (gram ? s_n[t] : s_m[t]) : 1.f;
    }
  }
  // Branch-free per element: the decay ratio is formed for every element and the masked
  // ones are replaced by zero (a ratio that overflows there is discarded by the select).
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int job = jj * 4 + wave;
    const int kind = job < NJ ? job_kind(job) : 2;  // wave-uniform
    if (kind == 1 || (kind == 0 && R::solve)) {
      const bool gram = kind == 0;
      int mt, nt;
      job_tile(job, mt, nt);
      float* dst = gram ? Lf : Mf;
      const int s = 16 * nt + n;
      const float gs = sc_gs[jj], ss = sc_ss[jj] * sc_ns[jj];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float coef = (gram ? sc_eta[jj][i] * sc_sp[jj][i] : sc_sg[jj][i]) * sc_r[jj][i];
        const float ga = gram ? sc_gp[jj][i] : sc_g[jj][i];
        const bool keep = gram ? (s < t) : (s <= t);
        const float r = __builtin_amdgcn_exp2f((ga - gs) * 1.44269504088896341f);
        const float v = coef * ss * r * acc[jj][i];
        dst[mat_idx(t, s)] = keep ? v : 0.f;
      }
    }
  }
  if (wave < 2) {
    // wave w zeroes tile w of: M(0,1), M(2,3)
    const int r0 = (wave & 1) ? 32 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) Mf[mat_idx(r0 + 4 * g + q, r0 + 16 + n)] = 0.f;
  }
  __syncthreads();

  // ---- normalised linear attention (additive rule): the chunk's terms of the normaliser
  // (ZRec): den_in[t] = sum_{s<=t} M_ts b_s, the factor Gamma_t mq_t of q_t . z at chunk
  // entry, Gamma_C, and the chunk's write sum_s fU_s b_s x_s. Without a solve X keeps its
  // region.
  if (!R::solve && p.zrec != nullptr) {
    float* zr = p.zrec + ((size_t)bh * p.nchunks + c) * zrec_floats(DK);
    const float gC = s_g[CH - 1], sC = s_sg[CH - 1];
    if (tid < CH) {
      float d = 0.f;
      for (int s = 0; s <= tid; ++s) d += Mf[mat_idx(tid, s)] * s_eta[s];
      zr[tid] = d;
      zr[CH + tid] = s_sg[tid] * __expf(s_g[tid]) * (QKN ? s_m[tid] : 1.f);
      if (tid == 0) zr[2 * CH] = sC * __expf(gC);
    } else if (tid < CH + DK) {
      const int i = tid - CH;
      float w = 0.f;
      for (int s = 0; s < CH; ++s) {
        const u32x4 gr = Xs[s * NGR + ((i >> 3) ^ xswz<DK>(s))];
        const uint32_t word = gr[(i & 7) >> 1];
        const float x = bf16_bits_to_f32((i & 1) ? word >> 16 : word & 0xffffu);
        w += s_eta[s] * sC * s_sg[s] * __expf(gC - s_g[s]) * (QKN ? s_n[s] : 1.f) * x;
      }
      zr[2 * CH + 4 + i] = w;
    }
  }

  // ---- 5. M as split A fragments into the record (its region then holds T)
  split_to_record<RC::kM>(Mf, rec, tid);

  // ---- 6. T = (I + L)^-1
  if constexpr (R::solve) {
    __syncthreads();  // M has left its region
    if (wave >= 2) {
      // wave 2 / 3 zeroes T(0,1) / T(2,3)
      const int r0 = (wave & 1) ? 32 : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) Tf[mat_idx(r0 + 4 * g + q, r0 + 16 + n)] = 0.f;
    }
    f4 Tc[4];
    {
      // diagonal block b = wave: lane (g, n) forms column n of D_b, keeps rows 4g..4g+3
      const int b = wave;
      float d[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* lrow = &Lf[(16 * b + r) * 64];
        float s0 = (r == n) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < r; k4 += 4) {
          const f4 l = *reinterpret_cast<const f4*>(lrow + ((16 * b + k4) ^ (r << 2)));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (k4 + q < r) {
              if (q & 1) s1 -= l[q] * d[k4 + q];
              else s0 -= l[q] * d[k4 + q];
            }
          }
        }
        d[r] = s0 + s1;
      }
      f4 db;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        db[q] = g == 0 ? d[q] : g == 1 ? d[4 + q] : g == 2 ? d[8 + q] : d[12 + q];
        Tf[mat_idx(16 * b + r, 16 * b + n)] = db[q];
      }
      Tc[0] = Tc[1] = Tc[2] = Tc[3] = db;
    }
    __syncthreads();  // every D_b in LDS
    if (wave == 0) t_column_block<0>(Lf, Tf, Tc, g, n);
    else if (wave == 1) t_column_block<1>(Lf, Tf, Tc, g, n);
    else if (wave == 2) t_column_block<2>(Lf, Tf, Tc, g, n);
    __syncthreads();

    // ---- 7. T as split A fragments into the record
    split_to_record<RC::kT>(Tf, rec, tid);
  }
  if (c == 0 && tid < DK) {
    uint16_t v = 0;
    if (R::shift && has_in) v = f32_to_bf16_bits(p.xprev_in[(size_t)bh * DK + tid]);
    reinterpret_cast<uint16_t*>(rec + RC::kX0)[tid] = v;
  }
}

template <int DK, int RULE>
hipError_t launch_t(const ScanParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)p.BH * p.nchunks);
  if (p.flags & (kFlagQkL2 | kFlagQkRms))
    hipLaunchKernelGGL((prep_split_kernel<DK, RULE, true>), dim3(grid), dim3(NTP), 0, st, p);
  else
    hipLaunchKernelGGL((prep_split_kernel<DK, RULE, false>), dim3(grid), dim3(NTP), 0, st, p);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const ScanParams& p, hipStream_t st) {
  if (p.rule == kRuleDelta) return launch_t<DK, kRuleDelta>(p, st);
  if (p.rule == kRuleInner) return launch_t<DK, kRuleInner>(p, st);
  return launch_t<DK, kRuleAdditive>(p, st);
}

}  // namespace

hipError_t launch_prep_split(const ScanParams& p, hipStream_t st) {
  return p.dk == 64 ? launch_dk<64>(p, st) : launch_dk<128>(p, st);
}

}  // namespace fwmem
