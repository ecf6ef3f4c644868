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
// MI355X design.  Three launches (two for a single sequence):
//   1. chunk_table_kernel: chunk list of the packed batch (chunks restart at each
//      sequence; every chunk's entry filled in parallel) and a longest-first
//      sequence order.  With one sequence the list is implicit (chunk c = rows
//      64 c ..) and this launch is skipped.
//   2. prep_kernel, one workgroup per (chunk, key head), all chunks in parallel: K K^T
//      and Q K^T on bf16 MFMA once for the key head's value heads, then per value
//      head the 64x64 UT solve in fp32 (16x16 blocks: the four diagonal blocks by
//      substitution, the off-diagonal blocks by block products) and E and MT on
//      MFMA.  E and MT go to the workspace as bf16 hi/lo pairs in MFMA fragment
//      order, so the next kernel loads each fragment as one contiguous 1 KiB block.
//   3. spine_kernel, one workgroup per (sequence, value head, 16- or 32-column block
//      of d_v): the serial pass over the chunks.  d_k / 32 "chain" waves keep the
//      state block in MFMA accumulators (one d_k k-step each) and carry
//      h -> K h -> X -> E X -> h in registers; the exchanges per chunk are the sum of
//      their partial K h and the X each of them forms for one token tile, through
//      LDS.  Four "output" waves compute O one chunk behind.  See the comment at
//      the kernel.  Columns of h evolve independently, so a 128-wide state splits
//      into 8 (or 4) workgroups; those of the value heads of one key head are
//      mapped onto one XCD so they share its operands through one L2.
// Precision: fp32-derived operands (h, X, T, E, MT, and fp32 activations) enter
// MFMA as bf16 hi + lo; a product takes hi*hi + hi*lo + lo*hi, about 2^-16
// relative, which keeps states within 1e-4 of the fp64 recurrence.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kC = 64;     // chunk length
constexpr int kLP = 72;    // padded LDS row (bf16 elements) of [*][64] tiles

__host__ __device__ constexpr size_t a256(size_t v) { return (v + 255) & ~size_t(255); }
int64_t max_chunks(int n, int64_t T) { return T / kC + n; }
// Per (chunk, value head): E and MT as bf16 hi/lo planes in MFMA A-fragment order
// ([tile][k-step][lane][8]: one wave-wide 16-byte load is one contiguous 1 KiB
// block), then Gam[64].
__host__ __device__ constexpr size_t unit_bytes(int D) { return a256((size_t)4 * D * kC + (size_t)4 * kC * kC + 256); }
// Element offset of lane `lane`'s 8 values of fragment (tile, ks) with nks k-steps.
__host__ __device__ constexpr int frag_off(int tile, int ks, int nks, int lane) { return ((tile * nks + ks) * 64 + lane) * 8; }
// Per (chunk, key head): the chunk's K and Q rows as the spine's MFMA A operands,
// bf16 in fragment order [tile][k-step][lane][8] with the tiles' rows in the order
// row_of (below), rows past the chunk's end zero: K then Q, each one plane (bf16
// activations, exact) or a hi and a lo plane (fp32 activations).  The prep writes
// them; the spine then loads every operand fragment as one contiguous 1 KiB block
// instead of 16-byte pieces of 16 rows a row stride apart.
__host__ __device__ constexpr size_t kq_bytes(int D, int planes) { return a256((size_t)planes * 2 * kC * D * 2); }

// Row order of the spine's operands.  A 16x16 MFMA result leaves lane (n, g)
// holding rows 4g .. 4g + 3 of column n; the B operand of a 16x16x32 product wants
// lane (n, g) to hold k-indices 8g .. 8g + 7.  If the rows of result tile t are the
// matrix rows
//      row_of(t, m) = 32 (t / 2) + 8 (m / 4) + 4 (t % 2) + m % 4     (m = 0..15),
// then result tiles 2s and 2s + 1 give lane (n, g) exactly the rows
// 32 s + 8 g .. 32 s + 8 g + 7 in order: they ARE the B operand of k-step s of the
// next product, with no data movement.  The spine therefore takes the rows of every
// A operand in this order -- the token rows of K and Q (loaded so) and the rows of E
// (d_k) and MT (tokens), stored so by the prep -- while k-indices stay natural.
__host__ __device__ constexpr int row_of(int t, int m) { return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3); }
// Element offset of matrix entry (row, col) of a 64-column E or MT plane in that
// order: tile t and operand row m with row_of(t, m) == row, k-step col / 32, lane
// m + 16 ((col % 32) / 8), element col % 8.
__host__ __device__ constexpr int pfrag_off(int row, int col) {
  return frag_off(2 * (row >> 5) + ((row >> 2) & 1), col >> 5, 2, 4 * ((row >> 3) & 3) + (row & 3) + 16 * ((col >> 3) & 3)) +
         (col & 7);
}

struct Tables {
  int32_t *seq_chunk0;   // [n+1] first chunk of each sequence
  int32_t *order;        // [n]   sequences, longest first
  int32_t *chunk_seq;    // [NC]  sequence of a chunk, -1 for unused slots
  int32_t *chunk_start;  // [NC]  first packed row of a chunk
  int32_t *chunk_len;    // [NC]  rows in a chunk (1..64)
  // One sequence: no table is built -- its rows are 0 .. T-1 (cu[0] = 0 and
  // cu[1] = T by contract), so chunk c starts at row 64 c.
  int implicit;
  int T;
};

size_t tables_bytes(int n, int64_t NC) {
  return a256(4 * (size_t)(n + 1)) + a256(4 * (size_t)n) + 3 * a256(4 * (size_t)NC);
}

Tables carve_tables(char *ws, int n, int64_t NC) {
  Tables t{};
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
// fp32 storage is split into hi + lo.  Loads are unconditional: callers clamp the
// row into the chunk, and rows past the chunk end only ever meet exact zeros
// (T has zero rows and columns for them), so no exec-masked load -- and no
// waitcnt that would drain the next chunk's prefetch -- is needed.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }
// Eight fp32 values -> bf16 hi and lo operands (packed conversions).
__device__ __forceinline__ void split8f(const floatx4 &a, const floatx4 &b, bf16x8 &hi, bf16x8 &lo) {
  const Split2 s0 = split_bf16_2(a[0], a[1]), s1 = split_bf16_2(a[2], a[3]);
  const Split2 s2 = split_bf16_2(b[0], b[1]), s3 = split_bf16_2(b[2], b[3]);
  hi = as_bf16x8(make_uint4(s0.hi, s1.hi, s2.hi, s3.hi));
  lo = as_bf16x8(make_uint4(s0.lo, s1.lo, s2.lo, s3.lo));
}
__device__ __forceinline__ void frag8(const bf16 *p, bf16x8 &hi, bf16x8 &lo) {
  hi = *reinterpret_cast<const bf16x8 *>(p);
  lo = zero8();
}
__device__ __forceinline__ void frag8(const float *p, bf16x8 &hi, bf16x8 &lo) {
  split8f(reinterpret_cast<const floatx4 *>(p)[0], reinterpret_cast<const floatx4 *>(p)[1], hi, lo);
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
  const Split2 a = split_bf16_2(v[0], v[1]), b = split_bf16_2(v[2], v[3]);
  *reinterpret_cast<uint2 *>(hi) = make_uint2(a.hi, b.hi);
  *reinterpret_cast<uint2 *>(lo) = make_uint2(a.lo, b.lo);
}

// ---- 1. chunk table ----------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t *cu, int n, int64_t NC, Tables tb) {
  __shared__ int32_t s_wave[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int per = (n + 255) / 256;
  const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + kC - 1) / kC;
  // block-wide exclusive scan of the per-thread chunk counts
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += (w < wave) ? s_wave[w] : 0;
    total += s_wave[w];
  }
  int run = base + incl - local;
  if (tid == 0) tb.seq_chunk0[n] = total;
  for (int s = s0; s < s1; ++s) {
    tb.seq_chunk0[s] = run;
    run += (cu[s + 1] - cu[s] + kC - 1) / kC;
  }
  __syncthreads();  // seq_chunk0 complete (workgroup-scope ordering of the global writes)
  // every chunk in parallel: its sequence is the last s with seq_chunk0[s] <= chunk
  for (int idx = tid; idx < total; idx += 256) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (tb.seq_chunk0[mid] <= idx) lo = mid; else hi = mid - 1;
    }
    const int c = idx - tb.seq_chunk0[lo];
    const int len = cu[lo + 1] - cu[lo];
    tb.chunk_seq[idx] = lo;
    tb.chunk_start[idx] = cu[lo] + kC * c;
    tb.chunk_len[idx] = min(kC, len - kC * c);
  }
  for (int64_t idx = total + tid; idx < NC; idx += 256) tb.chunk_seq[idx] = -1;
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
// acc += A(16x16) * B(16x16) with fp32 operands from LDS (row strides lda, ldb),
// as four fp32 MFMAs of k = 4.  Lane l supplies A[l%16][4kk + l/16] and
// B[4kk + l/16][l%16]; the result is in the usual 16x16 D layout.
__device__ __forceinline__ floatx4 mm16_f32(const float *A, int lda, const float *B, int ldb, floatx4 acc, int lr,
                                            int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[lr * lda + 4 * kk + lg], B[(4 * kk + lg) * ldb + lr], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ void store_tile(float *dst, int ld, const floatx4 &v, float sgn, int lr, int lg) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) dst[(4 * lg + rr) * ld + lr] = sgn * v[rr];
}

// LDS of prep_kernel, three regions reused across its phases (41 KiB, so three
// workgroups share a CU):
//   R0  L^-1 (fp32, solve and the reads of T)       -> M hi/lo (bf16, MT products)
//   R1  Abar (fp32, solve)                          -> K^T hi(/lo) (bf16, E products)
//   R2  block-product scratch (solve), gates
// With fp32 activations K^T is a hi/lo pair: it is staged half of d_k at a time
// (NPASS = 2), which keeps R1 at Abar's size and the workgroup at three per CU
// instead of two.
constexpr int kLF = 72;  // fp32 row stride of L^-1 and Abar
template <int D, int NP, int NPASS>
struct PrepLds {
  static constexpr size_t kt = (size_t)NP * (D / NPASS) * kLP * 2;
  static constexpr size_t r0 = (size_t)kC * kLF * 4 > (size_t)2 * kC * kLP * 2 ? (size_t)kC * kLF * 4 : (size_t)2 * kC * kLP * 2;
  static constexpr size_t r1 = (size_t)kC * kLF * 4 > kt ? (size_t)kC * kLF * 4 : kt;
};

// Held to three waves per SIMD (<= 168 VGPRs): with the LDS above, three workgroups
// then share a CU.
template <int D, typename TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void prep_kernel(PrefillLaunch p, Tables tb, char *units, char *kq) {
  constexpr bool SP = std::is_same<TY, float>::value;
  constexpr int NP = SP ? 2 : 1;
  constexpr int KS = D / 32;
  constexpr int NTI = D / 16;
  constexpr int NIG = D / 8 / 4;  // groups of 8 K columns staged per wave
  constexpr int NPASS = (SP && NIG % 2 == 0) ? 2 : 1;  // K^T staged in NPASS parts of d_k
  constexpr int NTP = NTI / NPASS;                      // E tiles per part
  constexpr int kMaxG = 4;                              // value heads per key head
  const int Hv = p.geo.Hv, Hk = p.geo.Hk, G = Hv / Hk, CD = p.geo.conv_dim;
  // One workgroup per (chunk, key head): the G value heads of a key head share the
  // chunk's K and Q rows and their Gram matrices Q K^T and K K^T (only the gates
  // differ), so those are loaded and formed once; the solve and the E and MT
  // products then run once per value head.
  const int cidx = blockIdx.x / Hk, g = blockIdx.x - cidx * Hk;
  const int seq = tb.implicit ? (cidx * kC < tb.T ? 0 : -1) : tb.chunk_seq[cidx];
  if (seq < 0) return;
  const int t0 = tb.implicit ? cidx * kC : tb.chunk_start[cidx];
  const int L = tb.implicit ? min(kC, tb.T - t0) : tb.chunk_len[cidx];
  const int tid = threadIdx.x, lane = tid % kWave, lr = lane % 16, lg = lane / 16;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const TY *y = static_cast<const TY *>(p.y);
  const TY *Qb = y + (size_t)t0 * CD + (size_t)g * D;
  const TY *Kb = y + (size_t)t0 * CD + (size_t)(Hk + g) * D;
  auto unit_of = [&](int hv) { return units + ((size_t)cidx * Hv + hv) * unit_bytes(D); };

  using LDS = PrepLds<D, NP, NPASS>;
  __shared__ __align__(16) char s_r0[LDS::r0];
  __shared__ __align__(16) char s_r1[LDS::r1];
  __shared__ __align__(16) float s_Y[4][16][17];  // block-product scratch
  __shared__ float s_gam[kMaxG][kC], s_bb[kMaxG][kC], s_dec[kMaxG][kC];
  float (*s_L)[kLF] = reinterpret_cast<float (*)[kLF]>(s_r0);
  bf16 (*s_M)[kC][kLP] = reinterpret_cast<bf16 (*)[kC][kLP]>(s_r0);  // [2][kC][kLP]
  float (*s_A)[kLF] = reinterpret_cast<float (*)[kLF]>(s_r1);
  bf16 (*s_Kt)[D / NPASS][kLP] = reinterpret_cast<bf16 (*)[D / NPASS][kLP]>(s_r1);  // [NP][D / NPASS][kLP]

  // ---- A: gates of the G value heads (wave s: value head G g + s); every load of
  // the shared part up front ----
  if (wave < G) {
    const int hv = g * G + wave;
    const size_t gi = (size_t)(t0 + min(lane, L - 1)) * Hv + hv;
    const float a_raw = p.a[gi], b_raw = p.b[gi];
    // ln a, clamped at -30; from raw gate inputs ln a = -softplus(g) and b = sigmoid(beta)
    const float ln_a = p.gates_raw ? -(fmaxf(a_raw, 0.0f) + log1pf(expf(-fabsf(a_raw)))) : logf(a_raw);
    float la = (lane < L) ? fmaxf(ln_a, -30.0f) : 0.0f;
    const float bb = (lane < L) ? (p.gates_raw ? 1.0f / (1.0f + expf(-b_raw)) : b_raw) : 0.0f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float v = __shfl_up(la, off);
      if (lane >= off) la += v;
    }
    s_gam[wave][lane] = la;
    s_bb[wave][lane] = bb;
    const float glast = __shfl(la, kC - 1);
    s_dec[wave][lane] = __expf(glast - la);
    float *Gam = reinterpret_cast<float *>(unit_of(hv) + (size_t)2 * (2 * D * kC + 2 * kC * kC));
    Gam[lane] = __expf(la);
  }
  // K rows for the K^T staging of phase D: lane = token, 8 consecutive columns
  // per load (columns 8 (wave + 4 m) ..), loaded again for each value head in its
  // phase D (cache hits) rather than held through the solves.  With fp32
  // activations every operand is a hi/lo pair: the K tiles of phase B are then
  // loaded one at a time.
  bf16x8 kth[NIG], ktl[NIG];
  auto load_kt = [&]() {
#pragma unroll
    for (int m = 0; m < NIG; ++m) frag8(Kb + (size_t)min(lane, L - 1) * CD + 8 * (wave + 4 * m), kth[m], ktl[m]);
  };
  // wave w owns row block w of Q K^T -> M and of K K^T -> Abar.  (Its own K rows
  // are loaded on their own: picking them out of kh by the wave index would be a
  // run-time index into a register array, i.e. scratch memory.)
  const int ti = wave;
  constexpr int NKT = SP ? 1 : 4;  // K tiles held at once
  bf16x8 qh[KS], ql[KS], kih[KS], kil[KS], kh[NKT][KS], kl[NKT][KS];
  auto load_ktile = [&](int tj, int slot) {
    const TY *krow = Kb + (size_t)min(16 * tj + lr, L - 1) * CD + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) frag8(krow + 32 * ks, kh[slot][ks], kl[slot][ks]);
  };
  if constexpr (!SP) {
    // bf16 activations: the chunk's Q and K rows go to LDS once (R0 and R1 are free
    // until the solves), 16 bytes per thread and load, and every wave reads its MFMA
    // operands there -- a quarter of the global loads of each wave fetching all the K
    // tiles it multiplies.  Row stride D + 8 elements: the 16 rows of an operand read
    // fall on distinct banks.
    constexpr int kRS = D + 8;
    constexpr int PER = kC * D / 8 / 256;  // 16-byte pieces per thread and matrix
    static_assert((size_t)kC * kRS * 2 <= LDS::r0 && (size_t)kC * kRS * 2 <= LDS::r1, "staged rows fit R0 and R1");
    bf16 *sq = reinterpret_cast<bf16 *>(s_r0), *sk = reinterpret_cast<bf16 *>(s_r1);
    uint4 rq[PER], rk[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid + 256 * q, row = idx / (D / 8), cc = 8 * (idx % (D / 8));
      rq[q] = *reinterpret_cast<const uint4 *>(Qb + (size_t)min(row, L - 1) * CD + cc);
      rk[q] = *reinterpret_cast<const uint4 *>(Kb + (size_t)min(row, L - 1) * CD + cc);
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid + 256 * q, row = idx / (D / 8), cc = 8 * (idx % (D / 8));
      *reinterpret_cast<uint4 *>(sq + row * kRS + cc) = rq[q];
      *reinterpret_cast<uint4 *>(sk + row * kRS + cc) = rk[q];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qh[ks] = *reinterpret_cast<const bf16x8 *>(sq + (16 * ti + lr) * kRS + 32 * ks + 8 * lg);
      kih[ks] = *reinterpret_cast<const bf16x8 *>(sk + (16 * ti + lr) * kRS + 32 * ks + 8 * lg);
      ql[ks] = kil[ks] = zero8();
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kh[tj][ks] = *reinterpret_cast<const bf16x8 *>(sk + (16 * tj + lr) * kRS + 32 * ks + 8 * lg);
        kl[tj][ks] = zero8();
      }
  } else {
    const TY *qrow = Qb + (size_t)min(16 * ti + lr, L - 1) * CD + 8 * lg;
    const TY *kirow = Kb + (size_t)min(16 * ti + lr, L - 1) * CD + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag8(qrow + 32 * ks, qh[ks], ql[ks]);
      frag8(kirow + 32 * ks, kih[ks], kil[ks]);
    }
  }
  // The chunk's K and Q rows of tile ti for the spine: natural row r = 16 ti + lr is
  // operand row m of spine tile tt, with row_of(tt, m) = r; rows past the chunk's end
  // are written as zeros.
  {
    bf16 *dst = reinterpret_cast<bf16 *>(kq + ((size_t)cidx * Hk + g) * kq_bytes(D, NP));
    const int r = 16 * ti + lr;
    const bool live = r < L;
    const int tt = 2 * (r >> 5) + ((r >> 2) & 1), m = 4 * ((r & 31) >> 3) + (r & 3);
    const bf16x8 z8 = zero8();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int fo = frag_off(tt, ks, KS, m + 16 * lg);
      *reinterpret_cast<bf16x8 *>(dst + fo) = live ? kih[ks] : z8;
      *reinterpret_cast<bf16x8 *>(dst + NP * kC * D + fo) = live ? qh[ks] : z8;
      if constexpr (SP) {
        *reinterpret_cast<bf16x8 *>(dst + kC * D + fo) = live ? kil[ks] : z8;
        *reinterpret_cast<bf16x8 *>(dst + 3 * kC * D + fo) = live ? ql[ks] : z8;
      }
    }
  }

  // ---- B: the Gram tiles (ti, tj <= ti) of Q K^T and K K^T, shared by the value heads ----
  floatx4 gq[4], gk[4];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    gq[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
    gk[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) {
      const int slot = SP ? 0 : tj;
      if constexpr (SP) load_ktile(tj, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        gq[tj] = mma<SP, SP>(gq[tj], qh[ks], ql[ks], kh[slot][ks], kl[slot][ks]);
        gk[tj] = mma<SP, SP>(gk[tj], kih[ks], kil[ks], kh[slot][ks], kl[slot][ks]);
      }
    }
  }
  __syncthreads();  // the gates are in LDS

#pragma unroll 1
  for (int s = 0; s < G; ++s) {
    const int hv = g * G + s;
    char *unit = unit_of(hv);
    bf16 *E_hi = reinterpret_cast<bf16 *>(unit);
    bf16 *E_lo = E_hi + D * kC;
    bf16 *MT_hi = E_lo + D * kC;
    bf16 *MT_lo = MT_hi + kC * kC;
    if (s > 0) __syncthreads();  // every wave is done with the previous value head's M and K^T
    // Abar of value head s from the Gram tiles (tiles above the diagonal are never read)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= ti) {
        const float gc = s_gam[s][16 * tj + lr];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * ti + 4 * lg + rr, c = 16 * tj + lr;
          s_A[r][c] = (c < r) ? s_bb[s][r] * __expf(s_gam[s][r] - gc) * gk[tj][rr] : 0.0f;  // c < r: argument <= 0
        }
      }
    }
    __syncthreads();

    // ---- C: L^-1 for L = I + Abar (unit lower triangular), fp32 ----
    // Level 1: the four 16x16 diagonal blocks, right-looking substitution (wave 0:
    // lane = block * 16 + column; after step m, x[m] is final and the updates of
    // the rows below it are independent).  The blocks above the diagonal are never
    // written: phase D, the only reader of those entries, masks them.
    if (wave == 0) {
      const int bk = lane / 16, c = lane % 16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < 15; ++m)
#pragma unroll
        for (int r = m + 1; r < 16; ++r) x[r] -= s_A[16 * bk + r][16 * bk + m] * x[m];
#pragma unroll
      for (int r = 0; r < 16; ++r) s_L[16 * bk + r][16 * bk + c] = x[r];
    }
    __syncthreads();
    // Level 2: [A 0; C B]^-1 = [A^-1 0; -B^-1 C A^-1  B^-1] on the two 32x32 diagonal
    // blocks (wave 0: rows 0..31, wave 1: rows 32..63).
    if (wave < 2) {
      const int o = 32 * wave;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm16_f32(&s_A[o + 16][o], kLF, &s_L[o][o], kLF, acc, lr, lg);  // C A^-1
      store_tile(&s_Y[wave][0][0], 17, acc, 1.0f, lr, lg);
    }
    __syncthreads();
    if (wave < 2) {
      const int o = 32 * wave;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm16_f32(&s_L[o + 16][o + 16], kLF, &s_Y[wave][0][0], 17, acc, lr, lg);  // B^-1 (C A^-1)
      store_tile(&s_L[o + 16][o], kLF, acc, -1.0f, lr, lg);
    }
    __syncthreads();
    // Level 3: the same identity with 32x32 blocks; wave w owns output tile (w/2, w%2).
    {
      const int yi = wave >> 1, yj = wave & 1;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      // Y = C A^-1, C = Abar[32:64, 0:32], A^-1 = L^-1[0:32, 0:32] (lower: k >= yj)
      for (int k = yj; k < 2; ++k)
        acc = mm16_f32(&s_A[32 + 16 * yi][16 * k], kLF, &s_L[16 * k][16 * yj], kLF, acc, lr, lg);
      store_tile(&s_Y[wave][0][0], 17, acc, 1.0f, lr, lg);
    }
    __syncthreads();
    {
      const int xi = wave >> 1, xj = wave & 1;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      // X = -B^-1 Y, B^-1 = L^-1[32:64, 32:64] (lower: k <= xi)
      for (int k = 0; k <= xi; ++k)
        acc = mm16_f32(&s_L[32 + 16 * xi][32 + 16 * k], kLF, &s_Y[2 * k + xj][0][0], 17, acc, lr, lg);
      store_tile(&s_L[32 + 16 * xi][16 * xj], kLF, acc, -1.0f, lr, lg);
    }
    __syncthreads();

    // ---- D: T = L^-1 diag(b); MT = M T and E = K^T diag(D) T on MFMA ----
    // Wave w owns rows j in [16w, 16w + 16) of T^T; its A operands are columns of T,
    // read now, before L^-1's region is reused for M.
    load_kt();
    const int jrow = 16 * wave + lr;
    const float bj = s_bb[s][jrow];
    bf16x8 th[2], tl[2], dh[2], dl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t wth[4], wtl[4], wdh[4], wdl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int sr = 8 * lg + 32 * ks + e;
        // L^-1 is zero above its diagonal blocks (block row 2 ks + lg / 2 < block column wave)
        const bool upper = wave > 2 * ks + (lg >> 1);
        const float t0v = upper ? 0.0f : s_L[sr][jrow] * bj, t1v = upper ? 0.0f : s_L[sr + 1][jrow] * bj;
        const Split2 ts = split_bf16_2(t0v, t1v), ds = split_bf16_2(s_dec[s][sr] * t0v, s_dec[s][sr + 1] * t1v);
        wth[e / 2] = ts.hi;
        wtl[e / 2] = ts.lo;
        wdh[e / 2] = ds.hi;
        wdl[e / 2] = ds.lo;
      }
      th[ks] = as_bf16x8(make_uint4(wth[0], wth[1], wth[2], wth[3]));
      tl[ks] = as_bf16x8(make_uint4(wtl[0], wtl[1], wtl[2], wtl[3]));
      dh[ks] = as_bf16x8(make_uint4(wdh[0], wdh[1], wdh[2], wdh[3]));
      dl[ks] = as_bf16x8(make_uint4(wdl[0], wdl[1], wdl[2], wdl[3]));
    }
    __syncthreads();
    // M of value head s (hi/lo) into R0, from the Gram tiles; the first part of K^T
    // (rows past the chunk end zero: E must see exact zeros) into R1
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const float gc = s_gam[s][16 * tj + lr];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * ti + 4 * lg + rr, c = 16 * tj + lr;
        // M[r][c] = exp(gamma_r - gamma_c) (q_r . k_c) for c <= r (the argument is <= 0), else 0
        const float mvv = (tj <= ti && c <= r) ? __expf(s_gam[s][r] - gc) * gq[tj][rr] : 0.0f;
        bf16 hi, lo;
        split_bf16(mvv, hi, lo);
        s_M[0][r][c] = hi;
        s_M[1][r][c] = lo;
      }
    }
    {
      const bool live = lane < L;
#pragma unroll
      for (int m = 0; m < NIG / NPASS; ++m)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          s_Kt[0][8 * (wave + 4 * m) + u][lane] = live ? kth[m][u] : (bf16)0.0f;
          if (SP) s_Kt[NP - 1][8 * (wave + 4 * m) + u][lane] = live ? ktl[m][u] : (bf16)0.0f;
        }
    }
    __syncthreads();
    // The lane's results below are X[r0 + lr][16 wave + 4 lg + r], r = 0..3 (X = MT or E,
    // r0 the tile's first row): four consecutive columns, one 8-byte word of the
    // spine's fragment order (pfrag_off).
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
      const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
      const int fo = pfrag_off(16 * tt + lr, 16 * wave + 4 * lg);
      store_split4(MT_hi + fo, MT_lo + fo, v);
    }
    // E^T[j][i] = sum_s D_s T[s][j] K[s][i]; lane holds column i, rows j..j+3 -> E[i][j..j+3]
#pragma unroll
    for (int part = 0; part < NPASS; ++part) {
      if (part > 0) {  // K^T rows [D/NPASS part, D/NPASS (part + 1)), once every wave is done with the last part
        __syncthreads();
        const bool live = lane < L;
#pragma unroll
        for (int m = part * (NIG / NPASS); m < (part + 1) * (NIG / NPASS); ++m)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int row = 8 * (wave + 4 * m) + u - part * (D / NPASS);
            s_Kt[0][row][lane] = live ? kth[m][u] : (bf16)0.0f;
            if (SP) s_Kt[NP - 1][row][lane] = live ? ktl[m][u] : (bf16)0.0f;
          }
        __syncthreads();
      }
#pragma unroll
      for (int tp = 0; tp < NTP; ++tp) {
        const int tix = part * NTP + tp;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 khh = *reinterpret_cast<const bf16x8 *>(&s_Kt[0][16 * tp + lr][8 * lg + 32 * ks]);
          const bf16x8 kll = SP ? *reinterpret_cast<const bf16x8 *>(&s_Kt[NP - 1][16 * tp + lr][8 * lg + 32 * ks])
                                : zero8();
          acc = mma<true, SP>(acc, dh[ks], dl[ks], khh, kll);
        }
        const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
        const int fo = pfrag_off(16 * tix + lr, 16 * wave + 4 * lg);
        store_split4(E_hi + fo, E_lo + fo, v);
      }
    }
  }
}

// ---- 3. the serial pass over chunks -------------------------------------------
// One workgroup of 8 waves per (sequence, value head, 16-column block of d_v);
// columns of h evolve independently, so a d_v-wide state splits over d_v / 16
// workgroups.
//   waves 0 .. D/32 - 1 ("chain"): wave w keeps d_k rows [32 w, 32 w + 32) of the
//     state block h (fp32) in MFMA accumulators -- one k-step of every product with
//     h.  Per chunk:
//       P_w = K[:, rows of w] h_w          partial K h for all 64 tokens (8 MFMAs)
//       -- barrier 1 --
//       wave w sums the partials of its own token tiles (fixed order), forms
//       X = V - Gam P for them and writes them, split bf16 hi/lo, as its part of
//       the B operand of the token k-steps in LDS
//       -- barrier 2 --
//       h_w <- Gam_63 h_w + E[rows of w, :] X   (X from LDS; 12 MFMAs)
//     With the operand row order of row_of(), each product's result tiles are lane
//     by lane the B operand of the next product: h, P and X only change precision
//     (bf16 hi/lo split), never lanes, and the work of forming X is split over the
//     chain waves instead of repeated in each.
//   waves 4 .. 7 ("output"): token tile w - 4; after barrier 1 of chunk c,
//     R = Gam (Q h) with h from LDS; after barrier 2, O = scale (R + MT X), stored.
// LDS: the partial products, h for the output waves (2 slots) and X (2 slots).
// Every wave loads exactly the operands it consumes (16-byte accesses but for V)
// through buffer descriptors whose extent ends at the chunk's last row, so rows
// past it read as zero and stores there are dropped; loads for a later chunk go out
// right after the last use of the registers they fill and stay raw until used.
constexpr int kCB = 16;  // state columns of one column tile
// 32-column workgroups once 16-column ones would exceed twice this many, 64-column
// ones once they would exceed four times this many
constexpr int64_t kSpineWideMinBlocks = 256;

// K or Q row fragments (bf16: one 16-byte word, fp32: two) kept raw until used.
template <typename TY>
struct Raw8;
template <>
struct Raw8<bf16> {
  uint4 w;
};
template <>
struct Raw8<float> {
  uint4 w0, w1;
};
__device__ __forceinline__ void load8(Raw8<bf16> &r, const bf16 *p) { r.w = *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void load8(Raw8<float> &r, const float *p) {
  r.w0 = reinterpret_cast<const uint4 *>(p)[0];
  r.w1 = reinterpret_cast<const uint4 *>(p)[1];
}
// as an MFMA operand: bf16 is exact (lo unused), fp32 splits into hi + lo
__device__ __forceinline__ void split8(const Raw8<bf16> &r, bf16x8 &hi, bf16x8 &lo) {
  hi = as_bf16x8(r.w);
  lo = hi;
}
__device__ __forceinline__ void split8(const Raw8<float> &r, bf16x8 &hi, bf16x8 &lo) {
  split8f(__builtin_bit_cast(floatx4, r.w0), __builtin_bit_cast(floatx4, r.w1), hi, lo);
}
// One activation kept raw: bf16 as its 16 bits, fp32 as is.
template <typename TY>
struct RawS;
template <>
struct RawS<bf16> {
  uint16_t v;
};
template <>
struct RawS<float> {
  float v;
};
__device__ __forceinline__ void loads(RawS<bf16> &r, const bf16 *p) { r.v = *reinterpret_cast<const uint16_t *>(p); }
__device__ __forceinline__ void loads(RawS<float> &r, const float *p) { r.v = *p; }
__device__ __forceinline__ float unpack(const RawS<bf16> &r) { return __builtin_bit_cast(float, (uint32_t)r.v << 16); }
__device__ __forceinline__ float unpack(const RawS<float> &r) { return r.v; }

// Buffer accesses: a descriptor (base address, extent in bytes) in scalar registers
// and a 32-bit per-lane byte offset.  Reads at or past the extent return zero and
// writes there are dropped, so rows past a chunk's end need no clamp and no branch.
// Every offset that the range check must see goes into the per-lane offset.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
  const int n = (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bload(Raw8<bf16> &v, Rsrc r, uint32_t off) { v.w = bload16(r, off); }
__device__ __forceinline__ void bload(Raw8<float> &v, Rsrc r, uint32_t off) {
  v.w0 = bload16(r, off);
  v.w1 = bload16(r, off + 16);
}
__device__ __forceinline__ void bload(RawS<bf16> &v, Rsrc r, uint32_t off) {
  v.v = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ void bload(RawS<float> &v, Rsrc r, uint32_t off) {
  v.v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void store_raw(bf16 *p, const Raw8<bf16> &v) { *reinterpret_cast<uint4 *>(p) = v.w; }
__device__ __forceinline__ void store_raw(float *p, const Raw8<float> &v) {
  reinterpret_cast<uint4 *>(p)[0] = v.w0;
  reinterpret_cast<uint4 *>(p)[1] = v.w1;
}
__device__ __forceinline__ floatx4 bloadf4(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore(Rsrc r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore(Rsrc r, uint32_t off, bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, (int)off, 0, 0);
}

template <int D, int NC, typename TY, typename TO>
__global__ __launch_bounds__(512) void spine_kernel(PrefillLaunch p, Tables tb, const char *units, const char *kq) {
  constexpr bool SP = std::is_same<TY, float>::value;
  constexpr int KS = D / 32;        // k-steps over d_k = chain waves
  constexpr int CB = kCB * NC;      // state columns per workgroup (NC tiles of 16)
  constexpr int NCB = D / CB;       // column blocks per head
  constexpr int TPW = 4 / KS;       // token tiles whose X a chain wave forms
  constexpr int NT = SP ? 3 : 2;    // terms of a product with h: hi hi, hi lo (, lo hi)
  constexpr int NP = SP ? 2 : 1;    // planes of the K and Q fragments: hi (, lo)
  const int Hv = p.geo.Hv, Hk = p.geo.Hk, G = Hv / Hk, CD = p.geo.conv_dim;
  // Consecutive workgroups are dispatched round-robin over the 8 XCDs; within
  // each group of 8 * G * NCB, remap so that one XCD receives the NCB column blocks
  // of the G value heads of one key head (they share its K and Q rows, and each
  // head's units, through one L2), keeping the longest-sequence-first order
  // between groups.
  int b = blockIdx.x;
  const int nb = gridDim.x, per_xcd = G * NCB, grp = 8 * per_xcd;
  if (b < nb - nb % grp) {
    const int r = b % grp;
    b = (b - r) + (r % 8) * per_xcd + r / 8;
  }
  const int cb = b % NCB, hq = b / NCB, h = hq % Hv, q = hq / Hv;
  const int seq = tb.implicit ? 0 : tb.order[q];
  const int c_first = tb.implicit ? 0 : tb.seq_chunk0[seq];
  const int nch = tb.implicit ? (tb.T + kC - 1) / kC : tb.seq_chunk0[seq + 1] - c_first;
  if (nch == 0) return;  // zero-length sequence: state unchanged
  // chunk c of the sequence starts at row seq_t0 + 64 c (no table loads in the loop)
  const int seq_t0 = p.cu[seq], seq_len = p.cu[seq + 1] - seq_t0;
  const int g = h / G;
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // One slot each: partials are written before barrier 1 and read before barrier 2;
  // h is written before barrier 1 and read (by the output waves) before barrier 2;
  // X is written between the barriers and read before the next chunk's barrier 1.
  __shared__ floatx4 s_P[KS][4][NC][kWave];    // partial K h: chain wave, token tile, column tile
  __shared__ bf16x8 s_H[KS][2][NC][kWave];     // h as B operands: k-step, hi/lo, column tile
  __shared__ uint2 s_X[2][2][NC][kWave][2];    // X as B operands: token k-step, hi/lo, column tile, lane, tile parity
  // V and Gam of the next chunk, from the output waves (each loads its token tile's
  // V rows, 16 bytes per lane, and the chunk's 64 Gam, 4 bytes per lane), for every
  // wave; written before barrier 1, read before barrier 2.  V rows in operand-row
  // order m of the tile; Gam by token, so a lane's 4 rows row_of(tt, 4 lg + r) are
  // 4 consecutive values.
  __shared__ __align__(16) TY s_V[4][16][CB];
  __shared__ __align__(16) float s_G[kC];

  const TY *y = static_cast<const TY *>(p.y);
  auto unit_of = [&](int c) { return units + ((size_t)(c_first + c) * Hv + h) * unit_bytes(D); };
  // K and Q fragments of chunk c (key head g)
  auto kq_of = [&](int c) { return make_rsrc(kq + ((size_t)(c_first + c) * Hk + g) * kq_bytes(D, NP), kq_bytes(D, NP)); };
  auto gam_of = [&](int c) {
    return reinterpret_cast<const float *>(reinterpret_cast<const bf16 *>(unit_of(c)) + 2 * D * kC + 2 * kC * kC);
  };
  auto chunk_t0 = [&](int c) { return seq_t0 + kC * c; };
  auto chunk_len = [&](int c) { return min(kC, seq_len - kC * c); };
  // Descriptor of the y rows of token tile tt of chunk c (row order row_of): base at
  // the tile's first row 32 (tt / 2) + 4 (tt % 2), extent up to the chunk's end, so
  // rows past it read as zero.
  auto tile_rows = [&](int c, int tt) {
    const int r0 = 32 * (tt >> 1) + 4 * (tt & 1);
    return make_rsrc(y + (size_t)(chunk_t0(c) + r0) * CD, (int64_t)(chunk_len(c) - r0) * CD * (int64_t)sizeof(TY));
  };
  constexpr uint32_t kGamOff = 2 * (2 * D * kC + 2 * kC * kC);  // byte offset of Gam in a unit
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  if (wave < 4) {
    if (wave >= KS) {  // D < 128: fewer chain waves; keep the barrier count
#pragma unroll 1
      for (int c = 0; c < nch; ++c) {
        __syncthreads();
        __syncthreads();
      }
      return;
    }
    // ---------------- chain waves ----------------
    const int cw = wave;
    // the sequence's state: fp32, or binary16 widened here and narrowed at the end;
    // result tile (i, ct) of this wave holds d_k rows row_of(2 cw + i, 4 lg + r) of
    // column 16 ct + lr of the block
    const size_t hoff = (size_t)h * D * D + CB * cb + lr;
    gptr<float> hs = to_global(static_cast<float *>(p.h_state[seq])) + hoff;
    gptr<_Float16> hs16 = to_global(static_cast<_Float16 *>(p.h_state[seq])) + hoff;
    // all of the block's state loads first (one branch on the stored width)
    floatx4 hacc[2][NC];
    if (p.state_f16) {
      _Float16 raw[2][NC][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) raw[i][ct][r] = hs16[(size_t)row_of(2 * cw + i, 4 * lg + r) * D + 16 * ct];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) hacc[i][ct][r] = (float)raw[i][ct][r];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) hacc[i][ct][r] = hs[(size_t)row_of(2 * cw + i, 4 * lg + r) * D + 16 * ct];
    }
    uint4 kf[4][NP];              // K fragments of token tile tt, this wave's k-step: hi (, lo)
    uint4 ef[2][2][2];            // E fragments: result tile, token k-step, hi / lo
    auto fetch_k = [&](int c) {
      const Rsrc rk = kq_of(c);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) kf[tt][pl] = bload16(rk, 2 * (uint32_t)(pl * kC * D + frag_off(tt, cw, KS, lane)));
    };
    auto fetch_e = [&](int c) {
      const Rsrc ru = make_rsrc(unit_of(c), unit_bytes(D));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
            ef[i][s][hl] = bload16(ru, 2 * (uint32_t)(hl * D * kC + frag_off(2 * cw + i, s, 2, lane)));
    };
    // The state first, then the operand loads in the order the loop body issues them
    // (K, then E; kept so by scheduling barriers): both paths into the loop then reach
    // its header with the same loads pending, so the compiler's waits there stay
    // partial instead of a full vmcnt(0) that would stall on the operands just issued.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): the state has arrived
    __builtin_amdgcn_sched_barrier(0);
    fetch_k(0);
    __builtin_amdgcn_sched_barrier(0);
    fetch_e(0);
    __builtin_amdgcn_sched_barrier(0);
    auto chain_chunk = [&](int c) {
      const int cn = min(c + 1, nch - 1);  // past the end: the last chunk again, unused
      // h as the B operand (hi, lo) of this wave's k-step; to LDS for the output waves
      bf16x8 hb[NC][2];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const Split2 a0 = split_bf16_2(hacc[0][ct][0], hacc[0][ct][1]), a1 = split_bf16_2(hacc[0][ct][2], hacc[0][ct][3]);
        const Split2 b0 = split_bf16_2(hacc[1][ct][0], hacc[1][ct][1]), b1 = split_bf16_2(hacc[1][ct][2], hacc[1][ct][3]);
        hb[ct][0] = __builtin_bit_cast(bf16x8, uint4{a0.hi, a1.hi, b0.hi, b1.hi});
        hb[ct][1] = __builtin_bit_cast(bf16x8, uint4{a0.lo, a1.lo, b0.lo, b1.lo});
        s_H[cw][0][ct][lane] = hb[ct][0];
        s_H[cw][1][ct][lane] = hb[ct][1];
      }
      // partial P = K h over this wave's rows; the token and column tiles are
      // independent accumulation chains, innermost
      floatx4 pp[4][NC];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) pp[tt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      {
        bf16x8 kh[4], kl[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          kh[tt] = as_bf16x8(kf[tt][0]);
          kl[tt] = as_bf16x8(kf[tt][NP - 1]);  // (bf16: unused)
        }
#pragma unroll
        for (int term = 0; term < NT; ++term)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ct = 0; ct < NC; ++ct)
              pp[tt][ct] = mfma16(term == 2 ? kl[tt] : kh[tt], term == 1 ? hb[ct][1] : hb[ct][0], pp[tt][ct]);
      }
      if (KS > 1) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) s_P[cw][tt][ct][lane] = pp[tt][ct];
      }
      fetch_k(cn);
      __syncthreads();  // barrier 1
      // Gam_63 of this chunk (read before barrier 2: the output waves overwrite s_G
      // after it)
      const float gC = s_G[kC - 1];
      // X of the own token tiles: partials summed in wave order (the own one read
      // back too: picking it out of pp by the wave-dependent tile index would put pp
      // in scratch memory), then V - Gam P, split into this wave's half of the token
      // k-step's B operand
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tt = TPW * cw + j;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          floatx4 P;
          if (KS == 1) {
            P = pp[j][ct];
          } else {
            P = s_P[0][tt][ct][lane];
#pragma unroll
            for (int w2 = 1; w2 < KS; ++w2) P += s_P[w2][tt][ct][lane];
          }
          const floatx4 gam = *reinterpret_cast<const floatx4 *>(&s_G[row_of(tt, 4 * lg)]);
          float X[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) X[r] = ld(&s_V[tt][4 * lg + r][0], 16 * ct + lr) - gam[r] * P[r];
          const Split2 x01 = split_bf16_2(X[0], X[1]), x23 = split_bf16_2(X[2], X[3]);
          s_X[tt >> 1][0][ct][lane][tt & 1] = uint2{x01.hi, x23.hi};
          s_X[tt >> 1][1][ct][lane][tt & 1] = uint2{x01.lo, x23.lo};
        }
      }
      __syncthreads();  // barrier 2
      bf16x8 xb[2][2][NC];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) xb[s][hl][ct] = *reinterpret_cast<const bf16x8 *>(&s_X[s][hl][ct][lane][0]);
      // h <- Gam_63 h + E X: hi hi, hi lo, lo hi
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) hacc[i][ct] *= gC;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int term = 0; term < 3; ++term)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ct = 0; ct < NC; ++ct)
              hacc[i][ct] = mfma16(as_bf16x8(ef[i][s][term == 2 ? 1 : 0]), term == 1 ? xb[s][1][ct] : xb[s][0][ct],
                                   hacc[i][ct]);
      fetch_e(cn);
    };
    // one chunk per iteration (no double buffer here): a single loop body keeps the
    // compiler's waits at the loop header partial
#pragma unroll 1
    for (int c = 0; c < nch; ++c) chain_chunk(c);
    if (p.state_f16) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hs16[(size_t)row_of(2 * cw + i, 4 * lg + r) * D + 16 * ct] = (_Float16)hacc[i][ct][r];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) hs[(size_t)row_of(2 * cw + i, 4 * lg + r) * D + 16 * ct] = hacc[i][ct][r];
    }
  } else {
    // ---------------- output waves ----------------
    const int tt = wave - 4;  // token tile
    TO *o = static_cast<TO *>(p.o);
    const size_t ostride = (size_t)Hv * D;
    const int ocol = h * D + CB * cb + lr;
    const uint32_t ooff = (uint32_t)((8 * lg * ostride + ocol) * sizeof(TO));
    // NB buffers, filled NB chunks ahead: two with bf16 activations; one with fp32
    // activations, whose hi/lo fragments would otherwise hold the kernel to one
    // workgroup per CU
    constexpr int NB = SP ? 1 : 2;
    uint4 qf[NB][KS][NP];  // Q fragments of the tile, all k-steps, hi (, lo); chunk parity
    uint4 mf[NB][2][2];    // MT fragments: chunk parity, token k-step, hi / lo
    float go[NB];          // Gam of token `lane` of the chunk; chunk parity
    // V of the tile's 16 rows x CB columns, 8 columns per lane, in VPS passes of the
    // wave (two at 64-column blocks).  With 16-column blocks one pass takes half the
    // wave: the other lanes read past the descriptor's extent (zeros, no memory access)
    // and write nothing.
    constexpr int LPR = CB / 8;                              // lanes per row
    constexpr int VPS = (16 * LPR + kWave - 1) / kWave;      // passes
    constexpr int RPP = 16 / VPS;                            // rows per pass
    Raw8<TY> vr[NB][VPS];  // V of the tile for the chain waves: operand rows vm[.], 8 columns from vc
    const int vc = 8 * (lane % LPR);
    const bool vlane = lane < 16 * LPR;
    int vm[VPS];
    uint32_t vof[VPS];
#pragma unroll
    for (int ps = 0; ps < VPS; ++ps) {
      vm[ps] = ((lane / LPR) & (RPP - 1)) + RPP * ps;
      vof[ps] = vlane ? ((8 * (vm[ps] >> 2) + (vm[ps] & 3)) * CD + 2 * Hk * D + h * D + CB * cb + vc) *
                            (uint32_t)sizeof(TY)
                      : 0x7fff0000u;
    }
    // the token rows of this wave's tile: the Gam it writes to LDS
    const bool grow = tt == 2 * (lane >> 5) + ((lane >> 2) & 1);
    auto fetch_q = [&](auto par, int c) {
      constexpr int PAR = decltype(par)::value;
      const Rsrc rq = kq_of(c);
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
          qf[PAR % NB][s][pl] = bload16(rq, 2 * (uint32_t)((NP + pl) * kC * D + frag_off(tt, s, KS, lane)));
#pragma unroll
      for (int ps = 0; ps < VPS; ++ps) bload(vr[PAR % NB][ps], tile_rows(c, tt), vof[ps]);
      go[PAR % NB] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(unit_of(c), unit_bytes(D)), (int)(kGamOff + 4 * lane), 0, 0));
    };
    // the chunk's V (in the activation dtype) and Gam to LDS for the chain waves
    auto put_vg = [&](auto par) {
      constexpr int PAR = decltype(par)::value;
      if (vlane) {
#pragma unroll
        for (int ps = 0; ps < VPS; ++ps) store_raw(&s_V[tt][vm[ps]][vc], vr[PAR % NB][ps]);
      }
      if (grow) s_G[lane] = go[PAR % NB];
    };
    auto fetch_mt = [&](auto par, int c) {
      constexpr int PAR = decltype(par)::value;
      const Rsrc ru = make_rsrc(unit_of(c), unit_bytes(D));
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
          mf[PAR % NB][s][hl] = bload16(ru, 2 * (uint32_t)(2 * D * kC + hl * kC * kC + frag_off(tt, s, 2, lane)));
    };
    auto out_chunk = [&](int c, auto par) {
      constexpr int PAR = decltype(par)::value;
      __syncthreads();  // barrier 1: h of chunk c is in LDS
      floatx4 O[NC];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) O[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qh = as_bf16x8(qf[PAR % NB][s][0]), ql = as_bf16x8(qf[PAR % NB][s][NP - 1]);
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const bf16x8 hh = s_H[s][0][ct][lane], hl = s_H[s][1][ct][lane];
          O[ct] = mfma16(qh, hh, O[ct]);
          O[ct] = mfma16(qh, hl, O[ct]);
          if (SP) O[ct] = mfma16(ql, hh, O[ct]);
        }
      }
      {
        const floatx4 gam = *reinterpret_cast<const floatx4 *>(&s_G[row_of(tt, 4 * lg)]);
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) O[ct] *= gam;
      }
      fetch_q(par, min(c + NB, nch - 1));  // this chunk's Q is consumed
      __syncthreads();  // barrier 2: X of chunk c is in LDS
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const bf16x8 xh = *reinterpret_cast<const bf16x8 *>(&s_X[s][0][ct][lane][0]);
          const bf16x8 xl = *reinterpret_cast<const bf16x8 *>(&s_X[s][1][ct][lane][0]);
          O[ct] = mfma16(as_bf16x8(mf[PAR % NB][s][0]), xh, O[ct]);
          O[ct] = mfma16(as_bf16x8(mf[PAR % NB][s][0]), xl, O[ct]);
          O[ct] = mfma16(as_bf16x8(mf[PAR % NB][s][1]), xh, O[ct]);
        }
      // stores through the tile's descriptor over o: rows past the chunk's end are dropped
      const int r0 = 32 * (tt >> 1) + 4 * (tt & 1);
      const Rsrc ro = make_rsrc(o + (size_t)(chunk_t0(c) + r0) * ostride,
                                (int64_t)(chunk_len(c) - r0) * (int64_t)ostride * (int64_t)sizeof(TO));
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bstore(ro, ooff + (uint32_t)((r * ostride + 16 * ct) * sizeof(TO)), (TO)(p.scale * O[ct][r]));
      fetch_mt(par, min(c + NB, nch - 1));
      // next chunk's V and Gam for the chain waves (read after barrier 1; the chain
      // waves finished reading this chunk's before barrier 2)
      // (one buffer: fetch_q above has just brought the next chunk's into it)
      if (NB == 1 || PAR == 1) put_vg(P0()); else put_vg(P1());
    };
    fetch_q(P0(), 0);
    fetch_mt(P0(), 0);
    if constexpr (NB == 2) {
      fetch_q(P1(), min(1, nch - 1));
      fetch_mt(P1(), min(1, nch - 1));
    }
    put_vg(P0());
    // pairs of chunks, then an odd last chunk after the loop: no exit from the middle
    // of the body (that exit's merge of scalar values made the compiler read a
    // register still being loaded, i.e. wait for the chunk's prefetch)
    int c = 0;
#pragma unroll 1
    for (; c + 1 < nch; c += 2) {
      out_chunk(c, P0());
      out_chunk(c + 1, P1());
    }
    if (c < nch) out_chunk(c, P0());
  }
}

template <int D, typename TY, typename TO>
hipError_t launch_prefill_t(const PrefillLaunch &p, hipStream_t stream) {
  const int64_t NC = max_chunks(p.n, p.T);
  char *ws = static_cast<char *>(p.workspace);
  Tables tb = carve_tables(ws, p.n, NC);
  tb.implicit = p.n == 1;
  tb.T = (int)p.T;
  char *units = ws + a256(tables_bytes(p.n, NC));
  char *kq = units + (size_t)NC * p.geo.Hv * unit_bytes(D);
  hipError_t e = hipSuccess;
  if (!tb.implicit) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, p.cu, p.n, NC, tb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((prep_kernel<D, TY>), dim3((unsigned)(NC * p.geo.Hk)), dim3(256), 0, stream, p, tb, units, kq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 16-column blocks while that is what it takes to give every CU a workgroup
  // (the chunk time of a block is bound by the operands it loads, nearly the same for
  // 16 or 32 columns); 32-column blocks, half the operand traffic, for larger batches,
  // and 64-column blocks (a quarter of it, one workgroup per CU for their 123-131 KiB
  // of LDS) once there are more than 256 of them.
  const int64_t wg16 = (int64_t)p.n * p.geo.Hv * (D / kCB);
  if (D >= 64 && wg16 > 4 * kSpineWideMinBlocks)
    hipLaunchKernelGGL((spine_kernel<D, 4, TY, TO>), dim3((unsigned)(wg16 / 4)), dim3(512), 0, stream, p, tb,
                       static_cast<const char *>(units), static_cast<const char *>(kq));
  else if (D >= 32 && wg16 > 2 * kSpineWideMinBlocks)
    hipLaunchKernelGGL((spine_kernel<D, 2, TY, TO>), dim3((unsigned)(wg16 / 2)), dim3(512), 0, stream, p, tb,
                       static_cast<const char *>(units), static_cast<const char *>(kq));
  else
    hipLaunchKernelGGL((spine_kernel<D, 1, TY, TO>), dim3((unsigned)wg16), dim3(512), 0, stream, p, tb,
                       static_cast<const char *>(units), static_cast<const char *>(kq));
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

// ---- scratch of the allocation-free prefill ---------------------------------
// The workspace of gdn_prefill_chunked_noalloc: one copy of this array on every
// GPU that loads the library, held until the process ends.  Calls on one GPU share
// it (overlapping calls race) and it keeps the last call's contents; no byte of it
// needs to start at zero, since each call writes everything it reads first.  On
// the host the name is only a stand-in for the device symbol: host code passes the
// address hipGetSymbolAddress returns for the current device, cached per device.
static __device__ __align__(256) char scratch[kPrefillScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t prefill_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

size_t prefill_core_workspace(const Geometry &geo, int n, int64_t T, bool y_bf16) {
  const int64_t NC = max_chunks(n, T);
  return a256(tables_bytes(n, NC)) + (size_t)NC * geo.Hv * unit_bytes(geo.D) +
         (size_t)NC * geo.Hk * kq_bytes(geo.D, y_bf16 ? 1 : 2);
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
