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
// In bf16 k-step m a lane (jn = lane % 16, lg = lane / 16) reads
// h0[(d / 4) lg + 8 m + c][j0 .. j0 + NE - 1], c < 8 (j0 = JW w + NE jn, NE = JW / 16
// consecutive columns, one 8-byte load per row at d = 128): lane group lg's 8 operand
// elements are d_k indices (d / 4) lg + 8 m .. + 7, so the rows a lane reads are its
// B operand, split into hi/lo as they arrive and dropped after the k-step.
//
// Occupancy: nothing of the state outlives its k-step, and the conv outputs of q and
// k stay in registers until their norms are known, so a workgroup of two value heads
// needs 64 VGPRs and 40 KiB of LDS and four fit on a CU: on 256 CUs the 1,024
// workgroups of 64 sequences x 16 key heads are all resident at once, and the
// state streams of one workgroup overlap the front and epilogue of the others
// (holding the whole state per lane, two fit and the batch runs in two rounds
// that each leave HBM idle while they compute: 46-47 against 36-38 us for 64
// sequences on one MI355X, with the non-temporal hint on the state loads worth
// 2-3 us of that).  P, Pq, X, U and O sit in the MFMA result layout (rows
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

// NE consecutive fp32 values; load_once carries the non-temporal hint (a value read
// once: the state, which the kernel streams through its products)
template <int NE>
struct Cols;
template <>
struct Cols<1> {
  static __device__ __forceinline__ void load_once(gptr<const float> p, float v[1]) {
    v[0] = __builtin_nontemporal_load(p);
  }
  static __device__ __forceinline__ void store(gptr<float> p, const float v[1]) { *p = v[0]; }
};
template <>
struct Cols<2> {
  static __device__ __forceinline__ void load_once(gptr<const float> p, float v[2]) {
    const floatx2 x = __builtin_nontemporal_load(reinterpret_cast<gptr<const floatx2>>(p));
    v[0] = x.x;
    v[1] = x.y;
  }
  static __device__ __forceinline__ void store(gptr<float> p, const float v[2]) {
    *reinterpret_cast<gptr<floatx2>>(p) = floatx2{v[0], v[1]};
  }
};

// Lane l of a wave ends with the sum over the wave's 64 lanes of v[(l >> 2) & 15]:
// each exchange (lane bits 5, 4, 3, 2) halves the values a lane carries, keeping the
// half its bit selects, and the last two add the four lanes that share a row.
__device__ __forceinline__ float rows16_wave_sum(const float v[16]) {
  const int lane = threadIdx.x % kWave;
  float a[8], b[4], c[2];
  const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8, h2 = lane & 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (h5 ? v[8 + i] : v[i]) + __shfl_xor(h5 ? v[i] : v[8 + i], 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (h4 ? a[4 + i] : a[i]) + __shfl_xor(h4 ? a[i] : a[4 + i], 16);
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = (h3 ? b[2 + i] : b[i]) + __shfl_xor(h3 ? b[i] : b[2 + i], 8);
  const float d = (h2 ? c[1] : c[0]) + __shfl_xor(h2 ? c[0] : c[1], 4);
  return sum_lanes<4>(d);
}

// 4 x 4 transpose within each quad of lanes: lane j of a quad holds a[0..3] as row j
// of a block and ends with its column j (element i from lane i of the quad).  The
// off-diagonal 2 x 2 blocks are swapped between lanes l and l ^ 2, then each 2 x 2
// block is transposed between lanes l and l ^ 1: four DPP moves in all.
__device__ __forceinline__ void quad_transpose(float a[4]) {
  const int l = threadIdx.x & 3;
  {
    const bool hi = l & 2;
    const float r0 = dpp_f<0x4E>(hi ? a[0] : a[2]), r1 = dpp_f<0x4E>(hi ? a[1] : a[3]);  // quad_perm [2,3,0,1]
    a[0] = hi ? r0 : a[0];
    a[1] = hi ? r1 : a[1];
    a[2] = hi ? a[2] : r0;
    a[3] = hi ? a[3] : r1;
  }
  {
    const bool odd = l & 1;
    const float r0 = dpp_f<0xB1>(odd ? a[0] : a[1]), r1 = dpp_f<0xB1>(odd ? a[2] : a[3]);  // quad_perm [1,0,3,2]
    a[0] = odd ? r0 : a[0];
    a[1] = odd ? a[1] : r0;
    a[2] = odd ? r1 : a[2];
    a[3] = odd ? a[3] : r1;
  }
}

// N consecutive activations (N = 1, 2 or 4) widened to fp32, in one load; the
// address is a multiple of N elements.
template <int N>
__device__ __forceinline__ void load_act(const bf16 *p, float v[N]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N == 4) {
    const u32x2 w = *reinterpret_cast<gptr<const u32x2>>(to_global(p));
    v[0] = __builtin_bit_cast(float, w.x << 16);
    v[1] = __builtin_bit_cast(float, w.x & 0xffff0000u);
    v[2] = __builtin_bit_cast(float, w.y << 16);
    v[3] = __builtin_bit_cast(float, w.y & 0xffff0000u);
  } else if constexpr (N == 2) {
    const uint32_t w = *reinterpret_cast<gptr<const uint32_t>>(to_global(p));
    v[0] = __builtin_bit_cast(float, w << 16);
    v[1] = __builtin_bit_cast(float, w & 0xffff0000u);
  } else {
    v[0] = (float)*to_global(p);
  }
}
template <int N>
__device__ __forceinline__ void load_act(const float *p, float v[N]) {
  if constexpr (N == 4) {
    const floatx4 w = *reinterpret_cast<gptr<const floatx4>>(to_global(p));
    v[0] = w.x, v[1] = w.y, v[2] = w.z, v[3] = w.w;
  } else if constexpr (N == 2) {
    const floatx2 w = *reinterpret_cast<gptr<const floatx2>>(to_global(p));
    v[0] = w.x, v[1] = w.y;
  } else {
    v[0] = *to_global(p);
  }
}
// N consecutive outputs (N = 1 or 2) in one store; bf16 rounds to nearest even.
template <int N>
__device__ __forceinline__ void store_out(bf16 *p, const float v[N]) {
  if constexpr (N == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<gptr<bf16x2>>(to_global(p)) = __builtin_convertvector(floatx2{v[0], v[1]}, bf16x2);
  } else {
    *to_global(p) = (bf16)v[0];
  }
}
template <int N>
__device__ __forceinline__ void store_out(float *p, const float v[N]) {
  if constexpr (N == 2)
    *reinterpret_cast<gptr<floatx2>>(to_global(p)) = floatx2{v[0], v[1]};
  else
    *to_global(p) = v[0];
}

template <int D, int G, typename TA>
__global__ __launch_bounds__(kSlot *G) __attribute__((amdgpu_waves_per_eu(8)))
void woa_wy_kernel(RecurrentLaunch p) {
  constexpr int MAXR = 16;             // rows of a write-on-accept verify
  constexpr int NCH = (2 + G) * D;     // q, k, and G v heads
  constexpr int NT = kSlot * G;
  constexpr int JW = D / 4;            // state columns per wave
  constexpr int NE = JW / 16;          // 16-column result tiles per wave
  constexpr int NKB = D / 32;          // bf16 k-steps: 8 of a lane group's state rows each
  constexpr int NRED = 2 * D / kWave;  // waves of q and k channels
  static_assert(NE >= 1 && NE <= 2 && JW % 16 == 0, "d = 64 or 128");

  __shared__ __align__(16) bf16 s_qk16[4][MAXR][D + 8];  // k_hat hi, k_hat lo, q_hat hi, q_hat lo
  __shared__ __align__(16) float s_v[G][MAXR][D + 4];     // v after the conv (rows past the end: 0)
  __shared__ __align__(16) float s_ga[G][MAXR];
  __shared__ float s_gb[G][MAXR], s_gg[G][MAXR];         // b_t, Gam_t (rows past the end: a = 1, b = 0)
  __shared__ __align__(16) float s_T[G][MAXR][MAXR + 4];  // A, then T = (I + A)^-1
  __shared__ float s_M[G][MAXR][MAXR + 1];
  __shared__ __align__(16) float s_red[NRED][MAXR];       // per-wave sums of q^2 and k^2 of a row
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

  // ---- loads: conv taps, conv state, input rows, gates ---------------------------
  // The 64 channels of a wave are contiguous in x and in the conv state (D is a
  // multiple of 64 and the q, k and v blocks start at multiples of D).  A lane reads
  // 4 channels of one row (row 4 q + lane % 4 in load q), and quad_transpose then
  // hands every lane its own channel's rows: a quarter of the load instructions of
  // one element per row, which matters while the other workgroups of the CU stream
  // their states through the same vector-memory path.
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
  const int wave_base = kWave * (tid / kWave);  // first channel of this wave (it = 0)
  const int ln = tid % kWave, l4 = ln & 3, cq = ln & ~3;
  float xr[NIT][MAXR], win4[NIT][4], wt[NIT][4];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int base = wave_base + it * NT;
    if (base >= NCH) break;  // uniform over the wave
    const int c4 = chan(base) + cq;  // the 4 channels this lane reads
#pragma unroll
    for (int q = 0; q < MAXR / 4; ++q)
      load_act<4>(x + (size_t)(r0 + min(4 * q + l4, nrows - 1)) * C + c4, &xr[it][4 * q]);
    // conv state row K - 4 + lane % 4, clamped into its K - 1 rows (rows before the
    // first are weighted 0 below)
    load_act<4>(ring + (size_t)min(max(K - 4 + l4, 0), K - 2) * C + c4, win4[it]);
    const int c = chan(base) + ln;  // this lane's own channel
    if (K == 4) {
      load_act<4>(w + (size_t)c * 4, wt[it]);
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wt[it][jj] = jj >= 4 - K ? (float)w[(size_t)c * K + jj - (4 - K)] : 0.0f;
    }
  }
  const int gr = min(tid / G, MAXR - 1), gs = tid % G;
  float ga = 1.0f, gb = 0.0f;
  if (tid < MAXR * G) {
    ga = p.a[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];
    gb = p.b[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];
  }

  // ---- conv + SiLU of the group's channels for every row, in registers -----------
  // (rows past the end are 0); v goes to LDS, q and k stay for their L2 norms, whose
  // per-row sums of squares are taken over each wave's 64 channels
  float cv[NIT][MAXR];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int cl = tid + it * NT, base = wave_base + it * NT;
    if (base >= NCH) break;  // uniform over the wave
#pragma unroll
    for (int q = 0; q < MAXR / 4; ++q) quad_transpose(&xr[it][4 * q]);
    quad_transpose(win4[it]);
    float win[3];
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) win[jj] = (K - 4 + jj >= 0) ? win4[it][jj] : 0.0f;
    const float *wk = wt[it];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const float xv = xr[it][r];
      const float y = silu(wk[0] * win[0] + wk[1] * win[1] + wk[2] * win[2] + wk[3] * xv);
      cv[it][r] = r < nrows ? y : 0.0f;
      win[0] = win[1];
      win[1] = win[2];
      win[2] = xv;
    }
    if (base < 2 * D) {
      float sq[MAXR];
#pragma unroll
      for (int r = 0; r < MAXR; ++r) sq[r] = cv[it][r] * cv[it][r];
      const float tot = rows16_wave_sum(sq);
      if (l4 == 0) s_red[base / kWave][(ln >> 2) & 15] = tot;
    } else {
      const int vc = cl - 2 * D, vs = vc / D, c = vc - vs * D;
#pragma unroll
      for (int r = 0; r < MAXR; ++r) s_v[vs][r][c] = cv[it][r];
    }
  }
  if (tid < MAXR * G) {  // rows past the end: a = 1, b = 0, so they change nothing
    const bool live = gr < nrows;
    s_ga[gs][gr] = live ? (p.gates_raw ? decay_from_raw(ga) : ga) : 1.0f;
    s_gb[gs][gr] = live ? (p.gates_raw ? strength_from_raw(gb) : gb) : 0.0f;
  }
  __syncthreads();

  // ---- L2 norm of q and k, their bf16 hi/lo splits, and k_hat into the stash -----
  // The normalized values go back through quad_transpose, so that a lane writes 4
  // channels of one row: 8 bytes of hi and of lo into LDS, 16 bytes of k_hat.
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int base = wave_base + it * NT;
    if (base >= 2 * D) break;  // uniform over the wave
    const int cls = base / D;  // 0: q, 1: k
    const int w16 = cls == 1 ? 0 : 2, c0 = base - cls * D + cq;
#pragma unroll
    for (int b4 = 0; b4 < MAXR / 4; ++b4) {
      floatx4 ss = *reinterpret_cast<const floatx4 *>(&s_red[cls * (D / kWave)][4 * b4]);
#pragma unroll
      for (int q = 1; q < D / kWave; ++q) ss += *reinterpret_cast<const floatx4 *>(&s_red[cls * (D / kWave) + q][4 * b4]);
      float nv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) nv[e] = cv[it][4 * b4 + e] * rsqrt_hw(ss[e] + p.l2_eps);
      quad_transpose(nv);  // channels c0 .. c0 + 3 of row 4 b4 + lane % 4
      const int row = 4 * b4 + l4;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const Split2 s01 = split_bf16_2(nv[0], nv[1]), s23 = split_bf16_2(nv[2], nv[3]);
      *reinterpret_cast<u32x2 *>(&s_qk16[w16][row][c0]) = u32x2{s01.hi, s23.hi};
      *reinterpret_cast<u32x2 *>(&s_qk16[w16 + 1][row][c0]) = u32x2{s01.lo, s23.lo};
      if (cls == 1 && row < nrows)
        *reinterpret_cast<gptr<floatx4>>(to_global(p.stash) + (size_t)(r0 + row) * p.stash_row + g * D + c0) =
            floatx4{nv[0], nv[1], nv[2], nv[3]};
    }
  }
  __syncthreads();

  const int s = tid / kSlot, t = tid % kSlot;
  const int h = g * G + s;
  const int wv = t / kWave, lane = t % kWave, jn = lane % 16, lg = lane / 16;
  const int j0 = JW * wv + NE * jn;
  const bool solver = wv == s % 4;  // the wave that builds this value head's T and M
  // A operands: row jn of k_hat / q_hat (rows past the end are 0)
  auto operand = [&](int which, int m) {
    return *reinterpret_cast<const bf16x8 *>(&s_qk16[which][jn][(D / 4) * lg + 8 * m]);
  };

  // ---- solver wave: Gram matrices, decays, A, M, Gam; T = (I + A)^-1 -----------
  // (before its own products; the other waves of the head start theirs at once)
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

  // ---- P = K h0 and Pq = Q h0 on the matrix cores, the state streamed -------------
  // k-step m takes this lane's state rows (D / 4) lg + 8 m .. + 7 (columns j0 ..
  // j0 + NE - 1), read once and split into bf16 hi/lo as they arrive; nothing of
  // the state is held beyond its k-step, which keeps a workgroup small enough for
  // every workgroup of a batch to be resident at once
  const gptr<const float> S_lane =
      to_global(static_cast<const float *>(p.states[i])) + (size_t)h * D * D + (size_t)((D / 4) * lg) * D + j0;
  floatx4 P[NE], Pq[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) P[e] = Pq[e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NKB; ++m) {
    float hr[8][NE];
#pragma unroll
    for (int c = 0; c < 8; ++c) Cols<NE>::load_once(S_lane + (size_t)(8 * m + c) * D, hr[c]);
    bf16x8 hh[NE], hl[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16 hv, lv;
        split_bf16(hr[c][e], hv, lv);
        hh[e][c] = hv;
        hl[e][c] = lv;
      }
    // one A operand at a time, hi * (hi + lo) then lo * hi: four of its registers
    // live instead of sixteen, within the 64 that four workgroups per CU allow
    bf16x8 a = operand(0, m);
#pragma unroll
    for (int e = 0; e < NE; ++e) P[e] = mfma16(a, hh[e], mfma16(a, hl[e], P[e]));
    a = operand(1, m);
#pragma unroll
    for (int e = 0; e < NE; ++e) P[e] = mfma16(a, hh[e], P[e]);
    a = operand(2, m);
#pragma unroll
    for (int e = 0; e < NE; ++e) Pq[e] = mfma16(a, hh[e], mfma16(a, hl[e], Pq[e]));
    a = operand(3, m);
#pragma unroll
    for (int e = 0; e < NE; ++e) Pq[e] = mfma16(a, hh[e], Pq[e]);
  }

  // The lane's coordinates again, from an opaque copy of the thread index, so that
  // nothing derived from it is held through the products (at 64 VGPRs it spills)
  {
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o;
    const int s = tid / kSlot, t = tid % kSlot;
    const int h = g * G + s;
    const int wv = t / kWave, lane = t % kWave, jn = lane % 16, lg = lane / 16;
    const int j0 = JW * wv + NE * jn;

    // z and the norm weight of this lane's outputs (rows 4 lg + r, columns j0 + e)
    float zr[4][NE], wn[NE];
    if (has_z) {
      const TA *zp = static_cast<const TA *>(p.z), *nwp = static_cast<const TA *>(p.norm_w);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_act<NE>(zp + (size_t)(r0 + min(4 * lg + r, nrows - 1)) * Hv * D + (size_t)h * D + j0, zr[r]);
      load_act<NE>(nwp + j0, wn);
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
        const float v = s_v[s][tr][j0 + e];
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

    // ---- stash: u of the value heads and a (k_hat went in with its norm) -----------
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
      float v[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        v[e] = p.scale * O[e][r];
        if (has_z) v[e] *= inv[r] * (norm_gate(zr[r][e], p.norm_sigmoid) * wn[e]);
      }
      if (p.geo.out_bf16)
        store_out<NE>(static_cast<bf16 *>(p.out) + oi, v);
      else
        store_out<NE>(static_cast<float *>(p.out) + oi, v);
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
