// Chunked WY/UT-form prefill of the gated delta rule over packed varlen batches.
//
// What is computed: the three-step chunked prefill that the pages name as the
// gdn_prefill_fla_recompute_wu_k, gdn_prefill_fla_chunk_delta_h_k and
// gdn_prefill_fla_chunk_fwd_o_k handles (metrale_model_layers/layers/qwen3_ssm/
// layer_struct.rs page), over the varlen descriptor of
// prefill_gdn_full_batched_fla_varlen (trait_layer.rs page).  The algorithm is
// the chunkwise WY / UT-transform form of the delta rule (Yang et al., NeurIPS
// 2024, section 3.2) with per-token decay (Gated Delta Networks, ICLR 2025,
// section 3.3).  For a chunk of C = 64 tokens with start state h = S^T
// (d_k x d_v), gamma_i = sum_{s<=i} ln a_s (each ln a_s clamped at -30),
// Gam_i = exp(gamma_i), D_s = exp(gamma_63 - gamma_s):
//
//   Abar_ts = b_t exp(gamma_t - gamma_s) (k_t . k_s)    (s < t)
//   T       = (I + Abar)^-1 diag(b)                      (UT transform)
//   M_ts    = exp(gamma_t - gamma_s) (q_t . k_s)         (s <= t)
//   E  = K^T diag(D) T      (d_k x C)      MT = M T      (C x C)
//   X  = V - diag(Gam) K h                               (C x d_v)
//   O  = diag(Gam) Q h + MT X                            (outputs, times scale)
//   h <- Gam_63 h + E X                                  (next chunk's state)
//
// which equals the token recurrence (U' = T X are the corrected writes u_t).
//
// MI355X design.  Three launches:
//   1. chunk_table_kernel: chunk list of the packed batch (chunks restart at each
//      sequence) and a longest-first sequence order.
//   2. prep_kernel, one workgroup per (chunk, value head), all chunks in
//      parallel: K K^T and Q K^T on bf16 MFMA, the 64x64 UT solve in fp32 (16x16
//      blocks: the four diagonal blocks by substitution, the off-diagonal blocks
//      by block substitution), then E and MT on MFMA.  E and MT go to the
//      workspace as bf16 hi/lo pairs, already in the row order the next kernel
//      loads as MFMA A operands.
//   3. spine_kernel, one workgroup per (sequence, value head, 16-column block of
//      d_v): the serial pass over the chunks.  Columns of h evolve independently,
//      so a 128-wide state splits into 8 workgroups; the block's 128x16 state
//      lives in MFMA accumulators, its bf16 hi/lo copy in LDS is the B operand of
//      K h and Q h.  Each chunk is two MFMA stages separated by one barrier, and
//      the next chunk's operands are loaded into registers while the current one
//      computes.  The eight column blocks of a head are mapped onto one XCD so
//      they share E/MT/K/Q through one L2.
// Precision: fp32-derived operands (h, X, T, E, MT, and fp32 activations) enter
// MFMA as bf16 hi + lo; a product takes hi*hi + hi*lo + lo*hi, about 2^-16
// relative, which keeps states within 1e-4 of the fp64 recurrence.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kC = 64;     // chunk length
constexpr int kLP = 72;    // padded LDS row (bf16 elements) of [*][64] tiles

__host__ __device__ constexpr size_t a256(size_t v) { return (v + 255) & ~size_t(255); }
int64_t max_chunks(int n, int64_t T) { return T / kC + n; }
__host__ __device__ constexpr size_t unit_bytes(int D) { return a256((size_t)4 * D * kC + (size_t)4 * kC * kC + 256); }

struct Tables {
  int32_t *seq_chunk0;   // [n+1] first chunk of each sequence
  int32_t *order;        // [n]   sequences, longest first
  int32_t *chunk_seq;    // [NC]  sequence of a chunk, -1 for unused slots
  int32_t *chunk_start;  // [NC]  first packed row of a chunk
  int32_t *chunk_len;    // [NC]  rows in a chunk (1..64)
};

size_t tables_bytes(int n, int64_t NC) {
  return a256(4 * (size_t)(n + 1)) + a256(4 * (size_t)n) + 3 * a256(4 * (size_t)NC);
}

Tables carve_tables(char *ws, int n, int64_t NC) {
  Tables t;
  size_t off = 0;
  t.seq_chunk0 = reinterpret_cast<int32_t *>(ws + off); off += a256(4 * (size_t)(n + 1));
  t.order = reinterpret_cast<int32_t *>(ws + off); off += a256(4 * (size_t)n);
  t.chunk_seq = reinterpret_cast<int32_t *>(ws + off); off += a256(4 * (size_t)NC);
  t.chunk_start = reinterpret_cast<int32_t *>(ws + off); off += a256(4 * (size_t)NC);
  t.chunk_len = reinterpret_cast<int32_t *>(ws + off);
  return t;
}

// ---- operand helpers ---------------------------------------------------------
__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}

// 8 consecutive activations as an MFMA operand: bf16 storage is exact (lo unused),
// fp32 storage is split into hi + lo.
__device__ __forceinline__ void frag8(const bf16 *p, bool valid, bf16x8 &hi, bf16x8 &lo) {
  hi = valid ? *reinterpret_cast<const bf16x8 *>(p) : zero8();
  lo = zero8();
}
__device__ __forceinline__ void frag8(const float *p, bool valid, bf16x8 &hi, bf16x8 &lo) {
  if (!valid) {
    hi = zero8();
    lo = zero8();
    return;
  }
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h, l;
    split_bf16(v[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// acc += (ah + al)(bh + bl) without the al*bl term; *_SPLIT = false means the
// operand is exact in bf16 and its lo part is zero.
template <bool A_SPLIT, bool B_SPLIT>
__device__ __forceinline__ floatx4 mma(floatx4 acc, const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh,
                                       const bf16x8 &bl) {
  if (A_SPLIT) acc = mfma16(al, bh, acc);
  if (B_SPLIT) acc = mfma16(ah, bl, acc);
  return mfma16(ah, bh, acc);
}

// Four consecutive fp32 values -> bf16 hi/lo, stored as two 8-byte words.
__device__ __forceinline__ void store_split4(bf16 *hi, bf16 *lo, const float v[4]) {
  union {
    bf16 b[4];
    uint2 u;
  } H, L;
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(v[e], H.b[e], L.b[e]);
  *reinterpret_cast<uint2 *>(hi) = H.u;
  *reinterpret_cast<uint2 *>(lo) = L.u;
}

// ---- 1. chunk table ----------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t *cu, int n, int64_t NC, Tables tb) {
  __shared__ int32_t s_part[256];
  __shared__ int32_t s_total;
  const int tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + kC - 1) / kC;
  s_part[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int k = 0; k < 256; ++k) {
      const int v = s_part[k];
      s_part[k] = acc;
      acc += v;
    }
    s_total = acc;
    tb.seq_chunk0[n] = acc;
  }
  __syncthreads();
  int run = s_part[tid];
  for (int s = s0; s < s1; ++s) {
    tb.seq_chunk0[s] = run;
    const int len = cu[s + 1] - cu[s];
    const int nc = (len + kC - 1) / kC;
    for (int c = 0; c < nc; ++c) {
      tb.chunk_seq[run + c] = s;
      tb.chunk_start[run + c] = cu[s] + kC * c;
      tb.chunk_len[run + c] = min(kC, len - kC * c);
    }
    run += nc;
  }
  for (int64_t idx = s_total + tid; idx < NC; idx += 256) tb.chunk_seq[idx] = -1;
  // longest sequences first (rank sort; identity order for very large batches)
  for (int s = tid; s < n; s += 256) {
    if (n <= 4096) {
      const int len = cu[s + 1] - cu[s];
      int rank = 0;
      for (int s2 = 0; s2 < n; ++s2) {
        const int l2 = cu[s2 + 1] - cu[s2];
        rank += (l2 > len) || (l2 == len && s2 < s);
      }
      tb.order[rank] = s;
    } else {
      tb.order[s] = s;
    }
  }
}

// ---- 2. per-chunk UT transform -------------------------------------------------
template <int D, typename TY>
__global__ __launch_bounds__(256) void prep_kernel(PrefillLaunch p, Tables tb, char *units) {
  constexpr bool SP = std::is_same<TY, float>::value;
  constexpr int NP = SP ? 2 : 1;
  constexpr int KS = D / 32;
  constexpr int NTI = D / 16;
  const int Hv = p.geo.Hv, Hk = p.geo.Hk, G = Hv / Hk, CD = p.geo.conv_dim;
  const int cidx = blockIdx.x / Hv, h = blockIdx.x - cidx * Hv;
  const int seq = tb.chunk_seq[cidx];
  if (seq < 0) return;
  const int t0 = tb.chunk_start[cidx], L = tb.chunk_len[cidx];
  const int g = h / G;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, lr = lane % 16, lg = lane / 16;
  const TY *y = static_cast<const TY *>(p.y);
  const TY *Qb = y + (size_t)t0 * CD + (size_t)g * D;
  const TY *Kb = y + (size_t)t0 * CD + (size_t)(Hk + g) * D;

  char *unit = units + ((size_t)cidx * Hv + h) * unit_bytes(D);
  bf16 *E_hi = reinterpret_cast<bf16 *>(unit);
  bf16 *E_lo = E_hi + D * kC;
  bf16 *MT_hi = E_lo + D * kC;
  bf16 *MT_lo = MT_hi + kC * kC;
  float *Gam = reinterpret_cast<float *>(MT_lo + kC * kC);

  __shared__ float s_gam[kC], s_bb[kC], s_dec[kC];
  __shared__ __align__(16) bf16 s_Kt[NP][D][kLP];    // K^T, B operand of E
  __shared__ __align__(16) bf16 s_M[2][kC][kLP];     // M hi/lo, row-major
  __shared__ __align__(16) float s_T[kC][kC + 1];    // T, fp32
  __shared__ __align__(16) float s_A[kC][kC + 1];    // Abar, fp32
  __shared__ float s_Li[4][16][17];                  // inverses of the diagonal blocks of I + Abar
  __shared__ float s_P[3][16][17];

  // ---- A: gates and K^T staging ----
  if (wave == 0) {
    float la = 0.0f, bb = 0.0f;
    if (lane < L) {
      la = fmaxf(logf(p.a[(size_t)(t0 + lane) * Hv + h]), -30.0f);
      bb = p.b[(size_t)(t0 + lane) * Hv + h];
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float v = __shfl_up(la, off);
      if (lane >= off) la += v;
    }
    s_gam[lane] = la;
    s_bb[lane] = bb;
    const float glast = __shfl(la, kC - 1);
    s_dec[lane] = expf(glast - la);
    Gam[lane] = expf(la);
  }
  for (int e = tid; e < kC * (D / 8); e += 256) {
    const int sr = e / (D / 8), i0 = (e % (D / 8)) * 8;
    bf16x8 hi, lo;
    frag8(Kb + (size_t)sr * CD + i0, sr < L, hi, lo);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s_Kt[0][i0 + u][sr] = hi[u];
      if (SP) s_Kt[NP - 1][i0 + u][sr] = lo[u];
    }
  }
  __syncthreads();

  // ---- B: K K^T -> Abar (strictly lower), Q K^T -> M (lower incl. diagonal) ----
#pragma unroll 1
  for (int m = 0; m < 8; ++m) {
    const int idx = wave + 4 * m;
    const int which = idx >> 4, ti = (idx >> 2) & 3, tj = idx & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) {
      const TY *Arow = (which ? Qb : Kb) + (size_t)(16 * ti + lr) * CD + 8 * lg;
      const TY *Brow = Kb + (size_t)(16 * tj + lr) * CD + 8 * lg;
      const bool va = 16 * ti + lr < L, vb = 16 * tj + lr < L;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 ah, al, bh, bl;
        frag8(Arow + 32 * ks, va, ah, al);
        frag8(Brow + 32 * ks, vb, bh, bl);
        acc = mma<SP, SP>(acc, ah, al, bh, bl);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 16 * ti + 4 * lg + rr, c = 16 * tj + lr;
      const float dec = expf(s_gam[r] - s_gam[c]);
      if (which == 0) {
        s_A[r][c] = (c < r) ? s_bb[r] * dec * acc[rr] : 0.0f;
      } else {
        const float v = (c <= r) ? dec * acc[rr] : 0.0f;
        bf16 hi, lo;
        split_bf16(v, hi, lo);
        s_M[0][r][c] = hi;
        s_M[1][r][c] = lo;
      }
    }
  }
  __syncthreads();

  // ---- C: T = (I + Abar)^-1 diag(b), blocks of 16 ----
  if (lane < 16) {  // wave w inverts diagonal block w, lane = column
    const int bk = wave, c = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc -= s_A[16 * bk + r][16 * bk + m] * x[m];
      x[r] = acc;
    }
    const float bc = s_bb[16 * bk + c];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s_Li[bk][r][c] = x[r];
      s_T[16 * bk + r][16 * bk + c] = x[r] * bc;
    }
  }
  for (int e = tid; e < kC * kC; e += 256) {
    const int r = e / kC, c = e % kC;
    if ((c >> 4) > (r >> 4)) s_T[r][c] = 0.0f;
  }
  __syncthreads();
#pragma unroll 1
  for (int bi = 1; bi < 4; ++bi) {
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e >> 8, r = (e >> 4) & 15, c = e & 15;
      float acc = 0.0f;
      for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
        for (int m = 0; m < 16; ++m) acc += s_A[16 * bi + r][16 * bk + m] * s_T[16 * bk + m][16 * bj + c];
      }
      s_P[bj][r][c] = acc;
    }
    __syncthreads();
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e >> 8, r = (e >> 4) & 15, c = e & 15;
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < 16; ++m) acc += s_Li[bi][r][m] * s_P[bj][m][c];
      s_T[16 * bi + r][16 * bj + c] = -acc;
    }
    __syncthreads();
  }

  // ---- D: MT = M T and E = K^T diag(D) T on MFMA; wave w owns rows j of T^T ----
  const int jrow = 16 * wave + lr;
  bf16x8 th[2], tl[2], dh[2], dl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 8 * lg + 32 * ks + e;
      const float tv = s_T[s][jrow];
      bf16 hi, lo;
      split_bf16(tv, hi, lo);
      th[ks][e] = hi;
      tl[ks][e] = lo;
      split_bf16(s_dec[s] * tv, hi, lo);
      dh[ks][e] = hi;
      dl[ks][e] = lo;
    }
  }
  // MT^T[j][t] = sum_s T[s][j] M[t][s]; lane holds column t, rows j..j+3 -> MT[t][j..j+3]
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 mh = *reinterpret_cast<const bf16x8 *>(&s_M[0][16 * tt + lr][8 * lg + 32 * ks]);
      const bf16x8 ml = *reinterpret_cast<const bf16x8 *>(&s_M[1][16 * tt + lr][8 * lg + 32 * ks]);
      acc = mma<true, true>(acc, th[ks], tl[ks], mh, ml);
    }
    const int t = 16 * tt + lr, j0 = 16 * wave + 4 * lg;
    const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    store_split4(MT_hi + t * kC + j0, MT_lo + t * kC + j0, v);
  }
  // E^T[j][i] = sum_s D_s T[s][j] K[s][i]; lane holds column i, rows j..j+3 -> E[i][j..j+3]
#pragma unroll
  for (int ti = 0; ti < NTI; ++ti) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kh = *reinterpret_cast<const bf16x8 *>(&s_Kt[0][16 * ti + lr][8 * lg + 32 * ks]);
      const bf16x8 kl = SP ? *reinterpret_cast<const bf16x8 *>(&s_Kt[NP - 1][16 * ti + lr][8 * lg + 32 * ks])
                           : zero8();
      acc = mma<true, SP>(acc, dh[ks], dl[ks], kh, kl);
    }
    const int i = 16 * ti + lr, j0 = 16 * wave + 4 * lg;
    const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    store_split4(E_hi + i * kC + j0, E_lo + i * kC + j0, v);
  }
}

// ---- 3. the serial pass over chunks -------------------------------------------
template <int D, typename TY>
struct ChunkOps {
  static constexpr int KS = D / 32;
  static constexpr int NRT = D / 16;
  static constexpr int TPW = (NRT + 3) / 4;
  bf16x8 kh[KS], kl[KS], qh[KS], ql[KS];   // K, Q rows of this wave's 16 tokens
  bf16x8 eh[TPW][2], el[TPW][2];          // E rows of this wave's state tiles
  bf16x8 mh[2], ml[2];                    // MT rows of this wave's 16 tokens
  float gam[4], v[4], gC;
  int t0, L;
};

template <int D, typename TY>
__device__ __forceinline__ void load_chunk(ChunkOps<D, TY> &f, const PrefillLaunch &p, const Tables &tb,
                                           const char *units, int cidx, int h, int g, int cb, int wave,
                                           int lr, int lg) {
  using F = ChunkOps<D, TY>;
  const int Hv = p.geo.Hv, Hk = p.geo.Hk, CD = p.geo.conv_dim;
  f.t0 = tb.chunk_start[cidx];
  f.L = tb.chunk_len[cidx];
  const char *unit = units + ((size_t)cidx * Hv + h) * unit_bytes(D);
  const bf16 *E_hi = reinterpret_cast<const bf16 *>(unit);
  const bf16 *E_lo = E_hi + D * kC;
  const bf16 *MT_hi = E_lo + D * kC;
  const bf16 *MT_lo = MT_hi + kC * kC;
  const float *Gam = reinterpret_cast<const float *>(MT_lo + kC * kC);
  const TY *y = static_cast<const TY *>(p.y);
  const int srow = 16 * wave + lr;
  const bool valid = srow < f.L;
  const TY *qrow = y + (size_t)(f.t0 + (valid ? srow : 0)) * CD + (size_t)g * D + 8 * lg;
  const TY *krow = qrow + (size_t)Hk * D;
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) {
    frag8(krow + 32 * ks, valid, f.kh[ks], f.kl[ks]);
    frag8(qrow + 32 * ks, valid, f.qh[ks], f.ql[ks]);
  }
#pragma unroll
  for (int k = 0; k < F::TPW; ++k) {
    const int rt = wave + 4 * k;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (rt < F::NRT) {
        f.eh[k][ks] = *reinterpret_cast<const bf16x8 *>(E_hi + (16 * rt + lr) * kC + 8 * lg + 32 * ks);
        f.el[k][ks] = *reinterpret_cast<const bf16x8 *>(E_lo + (16 * rt + lr) * kC + 8 * lg + 32 * ks);
      } else {
        f.eh[k][ks] = zero8();
        f.el[k][ks] = zero8();
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    f.mh[ks] = *reinterpret_cast<const bf16x8 *>(MT_hi + (16 * wave + lr) * kC + 8 * lg + 32 * ks);
    f.ml[ks] = *reinterpret_cast<const bf16x8 *>(MT_lo + (16 * wave + lr) * kC + 8 * lg + 32 * ks);
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int s = 16 * wave + 4 * lg + rr;
    f.gam[rr] = Gam[s];
    f.v[rr] = (s < f.L) ? ld(y, (size_t)(f.t0 + s) * CD + (size_t)2 * Hk * D + (size_t)h * D + 16 * cb + lr)
                        : 0.0f;
  }
  f.gC = Gam[kC - 1];
}

template <int D, typename TY, typename TO>
__global__ __launch_bounds__(256) void spine_kernel(PrefillLaunch p, Tables tb, const char *units) {
  constexpr bool SP = std::is_same<TY, float>::value;
  using F = ChunkOps<D, TY>;
  constexpr int NCB = D / 16;
  const int Hv = p.geo.Hv, Hk = p.geo.Hk, G = Hv / Hk;
  // Each group of 64 consecutive workgroups is dispatched round-robin over the 8
  // XCDs; remap so that every XCD receives 8 consecutive logical blocks (the
  // column blocks of one head when d = 128), keeping the longest-first order.
  int b = blockIdx.x;
  const int nb = gridDim.x;
  if (b < nb - nb % 64) b = (b & ~63) | ((b & 7) << 3) | ((b & 63) >> 3);
  const int cb = b % NCB, hq = b / NCB, h = hq % Hv, q = hq / Hv;
  const int seq = tb.order[q];
  const int c_first = tb.seq_chunk0[seq], nch = tb.seq_chunk0[seq + 1] - c_first;
  if (nch == 0) return;  // zero-length sequence: state unchanged
  const int g = h / G;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;

  __shared__ __align__(16) bf16 s_hT[2][16][D + 8];   // state block, transposed [j][i], hi/lo
  __shared__ __align__(16) bf16 s_XT[2][16][kLP];     // X block, transposed [j][s], hi/lo

  float *hs = p.h_state[seq] + (size_t)h * D * D;
  floatx4 hacc[F::TPW];
#pragma unroll
  for (int k = 0; k < F::TPW; ++k) {
    const int rt = wave + 4 * k;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      hacc[k][rr] = (rt < F::NRT) ? hs[(size_t)(16 * rt + 4 * lg + rr) * D + 16 * cb + lr] : 0.0f;
    if (rt < F::NRT) {
      const float v[4] = {hacc[k][0], hacc[k][1], hacc[k][2], hacc[k][3]};
      store_split4(&s_hT[0][lr][16 * rt + 4 * lg], &s_hT[1][lr][16 * rt + 4 * lg], v);
    }
  }
  __syncthreads();

  TO *o = static_cast<TO *>(p.o);
  F cur;
  load_chunk<D, TY>(cur, p, tb, units, c_first, h, g, cb, wave, lr, lg);
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    F nxt;
    if (c + 1 < nch) load_chunk<D, TY>(nxt, p, tb, units, c_first + c + 1, h, g, cb, wave, lr, lg);

    // stage 1: rows s of this wave -- P = K h, R = Q h, X = V - Gam P
    floatx4 P = {0.f, 0.f, 0.f, 0.f}, R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&s_hT[0][lr][8 * lg + 32 * ks]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&s_hT[1][lr][8 * lg + 32 * ks]);
      P = mma<SP, true>(P, cur.kh[ks], cur.kl[ks], bh, bl);
      R = mma<SP, true>(R, cur.qh[ks], cur.ql[ks], bh, bl);
    }
    float X[4];
    floatx4 O;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      X[rr] = cur.v[rr] - cur.gam[rr] * P[rr];
      O[rr] = cur.gam[rr] * R[rr];
    }
    store_split4(&s_XT[0][lr][16 * wave + 4 * lg], &s_XT[1][lr][16 * wave + 4 * lg], X);
    __syncthreads();

    // stage 2: h <- Gam_63 h + E X,  O = Gam Q h + MT X
    bf16x8 xh[2], xl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      xh[ks] = *reinterpret_cast<const bf16x8 *>(&s_XT[0][lr][8 * lg + 32 * ks]);
      xl[ks] = *reinterpret_cast<const bf16x8 *>(&s_XT[1][lr][8 * lg + 32 * ks]);
    }
#pragma unroll
    for (int k = 0; k < F::TPW; ++k) {
      const int rt = wave + 4 * k;
      if (rt < F::NRT) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) hacc[k][rr] *= cur.gC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) hacc[k] = mma<true, true>(hacc[k], cur.eh[k][ks], cur.el[k][ks], xh[ks], xl[ks]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) O = mma<true, true>(O, cur.mh[ks], cur.ml[ks], xh[ks], xl[ks]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int s = 16 * wave + 4 * lg + rr;
      if (s < cur.L)
        st(o, (size_t)(cur.t0 + s) * Hv * D + (size_t)h * D + 16 * cb + lr, p.scale * O[rr]);
    }
#pragma unroll
    for (int k = 0; k < F::TPW; ++k) {
      const int rt = wave + 4 * k;
      if (rt < F::NRT) {
        const float v[4] = {hacc[k][0], hacc[k][1], hacc[k][2], hacc[k][3]};
        store_split4(&s_hT[0][lr][16 * rt + 4 * lg], &s_hT[1][lr][16 * rt + 4 * lg], v);
      }
    }
    __syncthreads();
    cur = nxt;
  }
#pragma unroll
  for (int k = 0; k < F::TPW; ++k) {
    const int rt = wave + 4 * k;
    if (rt < F::NRT) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) hs[(size_t)(16 * rt + 4 * lg + rr) * D + 16 * cb + lr] = hacc[k][rr];
    }
  }
}

template <int D, typename TY, typename TO>
hipError_t launch_prefill_t(const PrefillLaunch &p, hipStream_t stream) {
  const int64_t NC = max_chunks(p.n, p.T);
  char *ws = static_cast<char *>(p.workspace);
  Tables tb = carve_tables(ws, p.n, NC);
  char *units = ws + a256(tables_bytes(p.n, NC));
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, p.cu, p.n, NC, tb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prep_kernel<D, TY>), dim3((unsigned)(NC * p.geo.Hv)), dim3(256), 0, stream, p, tb, units);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((spine_kernel<D, TY, TO>), dim3((unsigned)(p.n * p.geo.Hv * (D / 16))), dim3(256), 0,
                     stream, p, tb, static_cast<const char *>(units));
  return hipGetLastError();
}

template <int D, typename TY>
hipError_t launch_prefill_o(const PrefillLaunch &p, hipStream_t stream) {
  if (p.o_f32 || !p.geo.out_bf16) return launch_prefill_t<D, TY, float>(p, stream);
  return launch_prefill_t<D, TY, bf16>(p, stream);
}

template <int D>
hipError_t launch_prefill_y(const PrefillLaunch &p, hipStream_t stream) {
  return p.y_bf16 ? launch_prefill_o<D, bf16>(p, stream) : launch_prefill_o<D, float>(p, stream);
}

}  // namespace

size_t prefill_core_workspace(const Geometry &geo, int n, int64_t T) {
  const int64_t NC = max_chunks(n, T);
  return a256(tables_bytes(n, NC)) + (size_t)NC * geo.Hv * unit_bytes(geo.D);
}

hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  switch (p.geo.D) {
    case 32: return launch_prefill_y<32>(p, stream);
    case 64: return launch_prefill_y<64>(p, stream);
    case 128: return launch_prefill_y<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
