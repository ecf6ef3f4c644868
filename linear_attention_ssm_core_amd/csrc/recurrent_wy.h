// Write-on-accept verify over fp32 states in the WY form, on the matrix cores.
//
// Same operation as the write-on-accept mode of recurrent_kernel.h (gdn_wy4_woa_k,
// metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page): outputs of the k
// rows of each sequence and the stash of their rank-1 updates, no state written.
// The form is the WY / UT representation of a block of delta-rule updates (Yang
// et al., NeurIPS 2024, section 3.2) with per-token decay (Gated Delta Networks,
// ICLR 2025, section 3.3), taken over the n <= 16 rows of one sequence.  Per value
// head, with start state h0 = S0^T (d_k x d_v), unit keys k_t, queries q_t and
// gates a_t, b_t:
//
//   R_ts  = a_{s+1} ... a_t  (s <= t, R_tt = 1),   Gam_t = a_0 ... a_t
//   P = K h0,  Pq = Q h0                       the only products with the state
//   A_ts  = b_t R_ts (k_t . k_s)  (s < t),     T = (I + A)^-1
//   X_t   = b_t (v_t - Gam_t P_t),             U = T X   (the update vectors u_t)
//   M_ts  = R_ts (q_t . k_s)  (s <= t),        O = scale (diag(Gam) Pq + M U)
//
// which is the token recurrence (u_t = b_t (v_t - a_t S_{t-1} k_t),
// S_t = a_t S_{t-1} + u_t k_t^T, o_t = scale S_t q_t) unrolled over the block.
//
// Why: row by row, every row costs three fp32 operations per state element (S k,
// S q and the rank-1 update) on the vector ALUs.  Here the state enters two
// products of 16 x d_k by d_k x d_v on bf16 MFMA, fp32 operands split into
// hi + lo (hi*hi + hi*lo + lo*hi, about 2^-16 relative), and is never updated in
// registers; the 16 x 16 work (Gram matrices, the unit-triangular inverse) is
// small.  The k-token decode, which must also write the advanced state, keeps the
// row loop: holding the state to the end costs it the occupancy this form needs.
//
// Layout: one workgroup per (sequence, key head) as in recurrent_kernel.h; four
// waves per value head, wave w owning the d_v / 4 columns JW w .. JW w + JW - 1.
// A lane (jn = lane % 16, lg = lane / 16) holds h0[(d / 4) lg + ks][j0 .. j0 + NE - 1]
// for every ks (j0 = JW w + NE jn, NE = JW / 16 consecutive columns, one 8-byte
// load per row at d = 128).  bf16 k-step m pairs lane group lg's 8 operand
// elements with d_k indices (d / 4) lg + 8 m .. + 7, so a lane's own state rows
// are its B operand.  P, Pq, X, U and O sit in the MFMA result layout (rows
// 4 lg .. 4 lg + 3, column j0 + e), and the fp32 products over t take their k-steps
// in the order (lg, kk) -> row 4 lg + kk, so each lane feeds its own result
// registers back as operands.  Used for fp32 states at d = 64 and 128; binary16
// states (whose rows carry the rounded state) and d = 32 take recurrent_kernel.h.
#pragma once

#include "recurrent_kernel.h"

namespace gdn {

typedef float floatx2 __attribute__((ext_vector_type(2)));

// D(16x16 fp32) += A(16x4) B(4x16) on the fp32 matrix cores: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += (ah + al)(bh + bl) without the al bl term
__device__ __forceinline__ floatx4 mma3(floatx4 acc, const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh,
                                        const bf16x8 &bl) {
  acc = mfma16(al, bh, acc);
  acc = mfma16(ah, bl, acc);
  return mfma16(ah, bh, acc);
}

// NE consecutive fp32 values
template <int NE>
struct Cols;
template <>
struct Cols<1> {
  static __device__ __forceinline__ void load(gptr<const float> p, float v[1]) { v[0] = *p; }
  static __device__ __forceinline__ void store(gptr<float> p, const float v[1]) { *p = v[0]; }
};
template <>
struct Cols<2> {
  static __device__ __forceinline__ void load(gptr<const float> p, float v[2]) {
    const floatx2 x = *reinterpret_cast<gptr<const floatx2>>(p);
    v[0] = x.x;
    v[1] = x.y;
  }
  static __device__ __forceinline__ void store(gptr<float> p, const float v[2]) {
    *reinterpret_cast<gptr<floatx2>>(p) = floatx2{v[0], v[1]};
  }
};

template <int D, int G, typename TA>
__global__ __launch_bounds__(kSlot *G) __attribute__((amdgpu_waves_per_eu(G == 1 ? 2 : 4)))
void woa_wy_kernel(RecurrentLaunch p) {
  constexpr int MAXR = 16;             // rows of a write-on-accept verify
  constexpr int NCH = (2 + G) * D;     // q, k, and G v heads
  constexpr int SQ = NCH + 4;          // LDS row stride of s_qkv
  constexpr int NT = kSlot * G;
  constexpr int JW = D / 4;            // state columns per wave
  constexpr int NE = JW / 16;          // 16-column result tiles per wave
  constexpr int NKS = D / 4;           // state rows per lane
  constexpr int NKB = D / 32;          // bf16 k-steps: 8 of a lane group's state rows each
  static_assert(NE >= 1 && NE <= 2 && JW % 16 == 0, "d = 64 or 128");

  __shared__ __align__(16) float s_qkv[MAXR][SQ];
  __shared__ __align__(16) bf16 s_qk16[4][MAXR][D + 8];  // k_hat hi, k_hat lo, q_hat hi, q_hat lo
  __shared__ __align__(16) float s_ga[G][MAXR];
  __shared__ float s_gb[G][MAXR], s_gg[G][MAXR];         // b_t, Gam_t (rows past the end: a = 1, b = 0)
  __shared__ __align__(16) float s_T[G][MAXR][MAXR + 4];  // A, then T = (I + A)^-1
  __shared__ float s_M[G][MAXR][MAXR + 1];
  __shared__ float s_ss[G][4][MAXR];                      // gated norm: per-wave sums of o^2

  const int Hk = p.geo.Hk, Hv = p.geo.Hv, K = p.geo.K, C = p.geo.conv_dim;
  const int rank = blockIdx.x / Hk;
  const int g = blockIdx.x - rank * Hk;
  const int tid = threadIdx.x;

  // Sequences in index order: the work of a workgroup hardly depends on its
  // sequence's length (one state read), so ordering by length would balance
  // nothing, while index order keeps the state reads in flight within one
  // contiguous stretch of the batch's states (about 12 % faster, measured).
  int i, r0, nrows;
  {
    i = rank;
    r0 = __builtin_amdgcn_readfirstlane(p.cu[i]);
    nrows = __builtin_amdgcn_readfirstlane(p.cu[i + 1]) - r0;
    nrows = nrows < 0 ? 0 : (nrows > MAXR ? MAXR : nrows);
  }
  if (nrows == 0) return;  // uniform over the block

  // ---- loads: conv taps, conv state, input rows, gates, then the state ---------
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  const TA *ring = static_cast<const TA *>(p.conv_state[i]);
  constexpr int NIT = (NCH + NT - 1) / NT;
  const bool has_z = p.z != nullptr;
  auto chan = [&](int cl) {
    if (cl < D) return g * D + cl;
    if (cl < 2 * D) return Hk * D + g * D + (cl - D);
    return 2 * Hk * D + g * G * D + (cl - 2 * D);
  };
  TA rw[NIT][4], rr3[NIT][3], rx[NIT][MAXR];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = chan(min(tid + it * NT, NCH - 1));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) rw[it][jj] = w[(size_t)c * K + max(jj - (4 - K), 0)];
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) rr3[it][jj] = ring[(size_t)max(K - 4 + jj, 0) * C + c];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) rx[it][r] = x[(size_t)(r0 + min(r, nrows - 1)) * C + c];
  }
  const int gr = min(tid / G, MAXR - 1), gs = tid % G;
  const float ga = p.a[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];
  const float gb = p.b[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];

  const int s = tid / kSlot, t = tid % kSlot;
  const int h = g * G + s;
  const int wv = t / kWave, lane = t % kWave, jn = lane % 16, lg = lane / 16;
  const int j0 = JW * wv + NE * jn;
  const bool solver = wv == s % 4;  // the wave that builds this value head's T and M
  const gptr<const float> S_in = to_global(static_cast<const float *>(p.states[i])) + (size_t)h * D * D;
  float hr[NKS][NE];  // h0[(D / 4) lg + ks][j0 + e]
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) Cols<NE>::load(S_in + (size_t)((D / 4) * lg + ks) * D + j0, hr[ks]);

  // ---- conv + SiLU of the group's channels for every row ---------------------
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int cl = tid + it * NT;
    if (cl >= NCH) break;
    float wt[4], win[3];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wt[jj] = (jj >= 4 - K) ? (float)rw[it][jj] : 0.0f;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) win[jj] = (K - 4 + jj >= 0) ? (float)rr3[it][jj] : 0.0f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nrows) {
        const float xv = (float)rx[it][r];
        s_qkv[r][cl] = silu(wt[0] * win[0] + wt[1] * win[1] + wt[2] * win[2] + wt[3] * xv);
        win[0] = win[1];
        win[1] = win[2];
        win[2] = xv;
      }
    }
  }
  if (tid < MAXR * G) {  // rows past the end: a = 1, b = 0, so they change nothing
    const bool live = gr < nrows;
    s_ga[gs][gr] = live ? (p.gates_raw ? decay_from_raw(ga) : ga) : 1.0f;
    s_gb[gs][gr] = live ? (p.gates_raw ? strength_from_raw(gb) : gb) : 0.0f;
  }
  __syncthreads();

  // ---- L2 norm of q and k (one wave per row), and their bf16 hi/lo splits -----
  {
    const int wave = tid / kWave, ln = tid % kWave;
    for (int r = wave; r < nrows; r += NT / kWave) {
      float sq = 0.0f, sk = 0.0f;
      for (int c = ln; c < D; c += kWave) {
        const float qv = s_qkv[r][c], kv = s_qkv[r][D + c];
        sq += qv * qv;
        sk += kv * kv;
      }
      sq = wave_sum(sq);
      sk = wave_sum(sk);
      const float iq = rsqrt_hw(sq + p.l2_eps), ik = rsqrt_hw(sk + p.l2_eps);
      for (int c = ln; c < D; c += kWave) {
        const float qn = s_qkv[r][c] * iq, kn = s_qkv[r][D + c] * ik;
        s_qkv[r][D + c] = kn;
        bf16 hv, lv;
        split_bf16(kn, hv, lv);
        s_qk16[0][r][c] = hv;
        s_qk16[1][r][c] = lv;
        split_bf16(qn, hv, lv);
        s_qk16[2][r][c] = hv;
        s_qk16[3][r][c] = lv;
      }
    }
  }
  __syncthreads();

  // ---- P = K h0 and Pq = Q h0 on the matrix cores ------------------------------
  // A operands: row jn of k_hat / q_hat (rows past the end read the last row:
  // finite, and then multiplied by b = 0 or never stored); B: this lane's state rows
  auto operand = [&](int which, int m) {
    return *reinterpret_cast<const bf16x8 *>(&s_qk16[which][min(jn, nrows - 1)][(D / 4) * lg + 8 * m]);
  };
  floatx4 P[NE], Pq[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) P[e] = Pq[e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NKB; ++m) {
    const bf16x8 kh = operand(0, m), kl = operand(1, m), qh = operand(2, m), ql = operand(3, m);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      bf16x8 hh, hl;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16 hv, lv;
        split_bf16(hr[8 * m + c][e], hv, lv);
        hh[c] = hv;
        hl[c] = lv;
      }
      P[e] = mma3(P[e], kh, kl, hh, hl);
      Pq[e] = mma3(Pq[e], qh, ql, hh, hl);
    }
  }

  // z and the norm weight of this lane's outputs (rows 4 lg + r, columns j0 + e),
  // issued now so that they arrive during the solve
  TA zr[4][NE], wn[NE];
  {
    const TA *zp = has_z ? static_cast<const TA *>(p.z) : x;
    const TA *nwp = has_z ? static_cast<const TA *>(p.norm_w) : x;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < NE; ++e)
        zr[r][e] = zp[has_z ? (size_t)(r0 + min(4 * lg + r, nrows - 1)) * Hv * D + (size_t)h * D + j0 + e : 0];
#pragma unroll
    for (int e = 0; e < NE; ++e) wn[e] = nwp[has_z ? j0 + e : 0];
  }

  // ---- solver wave: Gram matrices, decays, A, M, Gam; T = (I + A)^-1 -----------
  if (solver) {
    floatx4 KK = {0.f, 0.f, 0.f, 0.f}, KQ = {0.f, 0.f, 0.f, 0.f};  // rows 4 lg + r, column jn
#pragma unroll
    for (int m = 0; m < NKB; ++m) {
      const bf16x8 kh = operand(0, m), kl = operand(1, m), qh = operand(2, m), ql = operand(3, m);
      KK = mma3(KK, kh, kl, kh, kl);
      KQ = mma3(KQ, qh, ql, kh, kl);
    }
    float av[MAXR];
#pragma unroll
    for (int q = 0; q < MAXR; q += 4)
      *reinterpret_cast<floatx4 *>(&av[q]) = *reinterpret_cast<const floatx4 *>(&s_ga[s][q]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 4 * lg + r, sc = jn;
      float R = 1.0f;  // a_{sc+1} ... a_tr
#pragma unroll
      for (int q = 1; q < MAXR; ++q) R *= (q > sc && q <= tr) ? av[q] : 1.0f;
      s_T[s][tr][sc] = sc < tr ? s_gb[s][tr] * R * KK[r] : 0.0f;
      s_M[s][tr][sc] = sc <= tr ? R * KQ[r] : 0.0f;
      if (sc == 0) s_gg[s][tr] = R * av[0];
    }
    // column c = jn of T: x_t = [t == c] - sum_{s < t} A_ts x_s (rows past the end
    // have A = 0 and keep x_t = [t == c]); the rows of A are read as broadcasts
    float xc[MAXR];
#pragma unroll
    for (int tr = 0; tr < MAXR; ++tr) xc[tr] = tr == jn ? 1.0f : 0.0f;
#pragma unroll
    for (int tr = 1; tr < MAXR; ++tr) {
      float v = xc[tr];
#pragma unroll
      for (int sc = 0; sc < tr; ++sc) v -= s_T[s][tr][sc] * xc[sc];
      xc[tr] = v;
    }
    if (lane < 16) {
#pragma unroll
      for (int tr = 0; tr < MAXR; ++tr) s_T[s][tr][jn] = xc[tr];
    }
  }
  __syncthreads();  // T, M and Gam of every value head

  // ---- X, U = T X and O = diag(Gam) Pq + M U -----------------------------------
  // k-step (lg, kk) of the products over t is row 4 lg + kk: this lane's register kk
  const float *gb_s = s_gb[s], *gg_s = s_gg[s];
  floatx4 X[NE], U[NE], O[NE];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 4 * lg + r;
    const float bt = gb_s[tr], gt = gg_s[tr];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float v = s_qkv[min(tr, nrows - 1)][2 * D + s * D + j0 + e];
      X[e][r] = bt * (v - gt * P[e][r]);
      O[e][r] = gt * Pq[e][r];
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) U[e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float ta = s_T[s][jn][4 * lg + kk];
#pragma unroll
    for (int e = 0; e < NE; ++e) U[e] = mfma4(ta, X[e][kk], U[e]);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float ma = s_M[s][jn][4 * lg + kk];
#pragma unroll
    for (int e = 0; e < NE; ++e) O[e] = mfma4(ma, U[e][kk], O[e]);
  }

  // ---- stash: u of the value heads, k_hat of the key head, a ---------------------
  {
    const int stash_u = Hk * D + h * D, stash_a = Hk * D + Hv * D + g * G;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 4 * lg + r;
      if (tr < nrows) {
        float u[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) u[e] = U[e][r];
        Cols<NE>::store(to_global(p.stash) + (size_t)(r0 + tr) * p.stash_row + stash_u + j0, u);
      }
    }
    for (int idx = tid; idx < nrows * (D / 4); idx += NT) {
      const int r = idx / (D / 4), q4 = idx - r * (D / 4);
      *reinterpret_cast<gptr<floatx4>>(to_global(p.stash) + (size_t)(r0 + r) * p.stash_row + g * D + 4 * q4) =
          *reinterpret_cast<const floatx4 *>(&s_qkv[r][D + 4 * q4]);
    }
    for (int idx = tid; idx < nrows * G; idx += NT) {
      const int r = idx / G, s2 = idx - r * G;
      p.stash[(size_t)(r0 + r) * p.stash_row + stash_a + s2] = s_ga[s2][r];
    }
  }

  // ---- outputs, through the gated norm when z is given ---------------------------
  // o = scale O; the norm's sum over the d_v columns of a row adds the 16 lanes of a
  // lane group, then the four waves of the value head in a fixed order
  float inv[4];
  if (has_z) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float o = p.scale * O[e][r];
        ss += o * o;
      }
      ss = sum_lanes<16>(ss);
      if (jn == 0) s_ss[s][wv][4 * lg + r] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 4 * lg + r;
      const float ss = (s_ss[s][0][tr] + s_ss[s][1][tr]) + (s_ss[s][2][tr] + s_ss[s][3][tr]);
      inv[r] = rsqrt_hw(ss / D + p.norm_eps);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 4 * lg + r;
    if (tr >= nrows) continue;
    const size_t oi = (size_t)(r0 + tr) * Hv * D + (size_t)h * D + j0;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float v = p.scale * O[e][r];
      if (has_z) v *= inv[r] * (norm_gate((float)zr[r][e], p.norm_sigmoid) * (float)wn[e]);
      if (p.geo.out_bf16)
        st(static_cast<bf16 *>(p.out), oi + e, v);
      else
        st(static_cast<float *>(p.out), oi + e, v);
    }
  }
}

template <int D, int G>
hipError_t launch_woa_wy_g(const RecurrentLaunch &p, hipStream_t stream) {
  const dim3 grid(p.n * p.geo.Hk), block(kSlot * G);
  if (p.geo.act_bf16)
    hipLaunchKernelGGL((woa_wy_kernel<D, G, bf16>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((woa_wy_kernel<D, G, float>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_woa_wy_d(const RecurrentLaunch &p, hipStream_t stream) {
  switch (p.geo.Hv / p.geo.Hk) {
    case 1: return launch_woa_wy_g<D, 1>(p, stream);
    case 2: return launch_woa_wy_g<D, 2>(p, stream);
    case 4: return launch_woa_wy_g<D, 4>(p, stream);
  }
  return hipErrorInvalidValue;
}

// The write-on-accept verify: fp32 states at d = 64 or 128 in the WY form,
// everything else row by row.
inline hipError_t launch_woa(const RecurrentLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  if (!p.state_f16 && p.geo.D == 128) return launch_woa_wy_d<128>(p, stream);
  if (!p.state_f16 && p.geo.D == 64) return launch_woa_wy_d<64>(p, stream);
  return launch_rec_mode<16, kModeWoa>(p, stream);
}

}  // namespace gdn
