// The token-recurrent kernel family: one-token batched decode, the decode of up
// to 17 consecutive tokens per sequence, the k-row verify that stores every
// intermediate state through the WY pointer tables, and the write-on-accept
// verify that stashes each row's rank-1 update instead.
//
// Decode (decode_multi_seq on the metrale_model_layers/layer/transformer_layer.rs
// page; the strided one-launch kernels conv1d_l2norm_f32_strided_k,
// gdn_f32_strided_norm_k and gated_rms_norm_f32_strided_k on the
// metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page), the k-token decode
// (decode_batched, transformer_layer.rs; gated_delta_rule_wy17, layer_struct.rs),
// verify (decode_verify_multi and the VERIFY_WY_* table constants,
// transformer_layer.rs; gdn_wyn_table_k, gdn_f32_strided_norm_snap_k,
// layer_struct.rs) and the write-on-accept verify (gdn_wy4_woa_k, layer_struct.rs)
// are one kernel template: the mode decides which states are stored and whether
// the conv state advances.
//
// Design (MI355X): the path is HBM-bound -- each value head's 128x128 fp32 state
// (64 KiB; 32 KiB as binary16) is read once and written once (decode, k-token
// decode), k times (verify) or not at all (write-on-accept).  One workgroup owns
// one (sequence, key head) pair: the conv + L2 prologue of the shared q/k channels
// runs once and feeds the H_v/H_k value heads of the group through LDS, and
// because one workgroup owns all channels of the group the in-place conv-state
// update has no cross-workgroup race.  256 threads own one value head: thread t
// holds column quad (t % 32) of 16 rows of the 32-row span of its wave
// (state_row below), so every wave-wide load or store covers two whole
// consecutive 512-byte state rows, a thread's share of k_hat and q_hat is four
// 16-byte LDS reads, and the state stays in registers across the rows of a
// sequence.  S k and S q are reduced over row groups with
// wave shuffles and one LDS exchange per row.  All arithmetic is fp32 (the
// recurrence per token is
//   kv = S k;  u = b (v - a kv);  S <- a S + u k^T;  o = scale (a S q + (k.q) u),
// the last being S_new q expanded); a binary16 state is rounded when stored and
// the state carried to the next row is the stored value.
#pragma once

#include "common.h"
#include "internal.h"

namespace gdn {

constexpr int kSlot = 256;          // threads per value head
constexpr int kTableSeqs = 128;     // entries per WY pointer table
// s_waitcnt immediate: vector-memory counter 0 (bits 3:0 and 15:14), expcnt and
// lgkmcnt at their maxima (no wait)
constexpr int kWaitVmem0 = (7 << 4) | (15 << 8);

typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

// 4 consecutive state elements of either storage type: raw load, widening, and
// the value a 4-vector takes once stored (binary16: rounded to nearest even).
// Loads and store() carry the non-temporal hint: a state is read once and written
// once per call, and streaming it past the caches' normal allocation moves it
// faster (cache-cold batched decode 109 -> 97.5 us, fold 64 -> 55 us on one
// MI355X).  store_kept() is the plain store, for the verify that records a state
// after every row: with the hint its stores ran 6 % slower.
template <typename TS>
struct StateIO;
template <>
struct StateIO<float> {
  typedef floatx4 raw;
  static __device__ __forceinline__ raw load(gptr<const float> p) {
    return __builtin_nontemporal_load(reinterpret_cast<gptr<const floatx4>>(p));
  }
  static __device__ __forceinline__ floatx4 widen(raw r) { return r; }
  static __device__ __forceinline__ floatx4 as_stored(floatx4 v) { return v; }
  static __device__ __forceinline__ void store(gptr<float> p, floatx4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<gptr<floatx4>>(p));
  }
  static __device__ __forceinline__ void store_kept(gptr<float> p, floatx4 v) { *reinterpret_cast<gptr<floatx4>>(p) = v; }
};
template <>
struct StateIO<_Float16> {
  typedef halfx4 raw;
  static __device__ __forceinline__ raw load(gptr<const _Float16> p) {
    return __builtin_nontemporal_load(reinterpret_cast<gptr<const halfx4>>(p));
  }
  static __device__ __forceinline__ floatx4 widen(raw r) { return __builtin_convertvector(r, floatx4); }
  static __device__ __forceinline__ floatx4 as_stored(floatx4 v) {
    return __builtin_convertvector(__builtin_convertvector(v, halfx4), floatx4);
  }
  static __device__ __forceinline__ void store(gptr<_Float16> p, floatx4 v) {
    __builtin_nontemporal_store(__builtin_convertvector(v, halfx4), reinterpret_cast<gptr<halfx4>>(p));
  }
  static __device__ __forceinline__ void store_kept(gptr<_Float16> p, floatx4 v) {
    *reinterpret_cast<gptr<halfx4>>(p) = __builtin_convertvector(v, halfx4);
  }
};

// S <- a S + u k^T on one row of 4 columns: the same operation order in every
// kernel that advances a state, so that a fold of rows stashed by this kernel
// reproduces the verify's recorded states bit for bit.
__device__ __forceinline__ floatx4 rank1_update(floatx4 s, float a, float k, floatx4 u) {
  floatx4 r;
  r.x = __builtin_fmaf(k, u.x, a * s.x);
  r.y = __builtin_fmaf(k, u.y, a * s.y);
  r.z = __builtin_fmaf(k, u.z, a * s.z);
  r.w = __builtin_fmaf(k, u.w, a * s.w);
  return r;
}

// The sequence that workgroup `rank` of a multi-row launch takes: sequences go
// longest first (rank r is the sequence with r sequences ahead of it, a longer one
// or an equally long one of lower index), so the long ones do not trail at the end
// of the grid.  n <= 128: lane l holds the lengths of sequences l and l + 64; each
// wave tests its share of the candidates, counting the sequences ahead of one with
// two ballots.  (length, index) is a strict total order whatever the lengths, so
// the ranks are a permutation of 0 .. n-1 and exactly one candidate matches.
// Block-uniform result (read back through LDS after a barrier).
__device__ __forceinline__ int seq_of_rank(const int32_t *cu, int n, int rank, int nthreads, int *s_seq) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const bool v0 = lane < n, v1 = lane + kWave < n;  // lanes past n are never ahead
  const int l0 = v0 ? cu[lane + 1] - cu[lane] : 0;
  const int l1 = v1 ? cu[lane + kWave + 1] - cu[lane + kWave] : 0;
  for (int t = wave; t < n; t += nthreads / kWave) {
    const int lt = t < kWave ? __shfl(l0, t) : __shfl(l1, t - kWave);
    const bool a0 = v0 && (l0 > lt || (l0 == lt && lane < t));
    const bool a1 = v1 && (l1 > lt || (l1 == lt && lane + kWave < t));
    const int ahead = __popcll(__ballot(a0)) + __popcll(__ballot(a1));
    if (ahead == rank && lane == 0) *s_seq = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_seq);
}

// Thread layout over a d x d head of the state: kSlot threads, each holding RPT
// rows of one column quad (4 consecutive columns).  Row group rg's rows are
// state_row(rg, 0 .. RPT-1).  The RGW row groups that share a wave (in the layout
// of one-token decode and verify) interleave over one contiguous span of RGW * RPT
// rows: each state load or store of the wave then covers RGW consecutive whole
// rows (1 KiB at d = 128, 64 and 32), and the wave's successive accesses the next
// ones, an order in which the HBM streams run about 4 % faster than with each row
// group's rows contiguous (measured on cache-cold 128 KiB blocks).
template <int D>
struct HeadLayout {
  static constexpr int CQ = D / 4;        // column quads
  static constexpr int RG = kSlot / CQ;   // row groups
  static constexpr int RPT = D / RG;      // rows per thread
  static constexpr int RGW = kWave / CQ;  // row groups per wave
};
template <int D>
__device__ __forceinline__ int state_row(int rg, int rr) {
  using Lh = HeadLayout<D>;
  return (rg / Lh::RGW) * (Lh::RGW * Lh::RPT) + Lh::RGW * rr + rg % Lh::RGW;
}
// Where q or k channel c (a state row) is staged in LDS: at rg * RPT + rr for
// c = state_row(rg, rr), so that a thread's RPT values are consecutive.
template <int D>
__device__ __forceinline__ int staged_slot(int c) {
  using Lh = HeadLayout<D>;
  const int span = Lh::RGW * Lh::RPT, w = c / span, rem = c - w * span;
  const int rr = rem / Lh::RGW, rg = w * Lh::RGW + (rem - rr * Lh::RGW);
  return rg * Lh::RPT + rr;
}

__device__ __forceinline__ void store4(float *p, const float v[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16 *p, const float v[4]) {
  union {
    bf16 b[4];
    uint2 u;
  } w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w.b[e] = (bf16)v[e];
  *reinterpret_cast<uint2 *>(p) = w.u;
}

// A pointer every lane holds the same value of (read from LDS, say), moved to
// scalar registers: stores through it then take a scalar base address.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// Gate of the fused norm: SiLU(z) or sigmoid(z).
__device__ __forceinline__ float norm_gate(float z, int sigmoid) {
  return sigmoid ? __builtin_amdgcn_rcpf(1.0f + __expf(-z)) : silu(z);
}

// Raw gate inputs: a = exp(-softplus(g)) = 1 / (1 + e^g), b = 1 / (1 + e^-beta).
__device__ __forceinline__ float decay_from_raw(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(g)); }
__device__ __forceinline__ float strength_from_raw(float beta) { return __builtin_amdgcn_rcpf(1.0f + __expf(-beta)); }

// Waves per SIMD the kernel is compiled for: in the multi-row modes two workgroups
// per CU (4 waves per SIMD at H_v/H_k = 2, <= 128 VGPRs) overlap one workgroup's
// loads and row arithmetic with another's stores.
template <int G, int MODE, int STATE_BYTES>
constexpr int rec_waves_per_eu() {
  // (the binary16 verify keeps its default: at 128 VGPRs it would spill inside the
  // row loop, and a reload there waits for every store still in flight)
  return (MODE == kModeDecode || (MODE == kModeVerify && STATE_BYTES == 2)) ? 1 : (G == 1 ? 2 : 4);
}

template <int D, int G, int MAXR, int MODE, typename TA, typename TS>
__global__ __launch_bounds__(kSlot *G) __attribute__((amdgpu_waves_per_eu(rec_waves_per_eu<G, MODE, sizeof(TS)>())))
void recurrent_kernel(RecurrentLaunch p) {
  constexpr int CQ = HeadLayout<D>::CQ;    // column quads of a head
  constexpr int RG = HeadLayout<D>::RG;    // row groups
  constexpr int RPT = HeadLayout<D>::RPT;  // state rows held by a thread
  constexpr int NCH = (2 + G) * D;     // q, k, and G v heads
  constexpr int NT = kSlot * G;
  constexpr bool kStoresEveryRow = MODE == kModeVerify;
  constexpr bool kAdvancesRing = MODE == kModeDecode || MODE == kModeTokens;
  // Write-on-accept verify and k-token decode: a wave holds every row group of its
  // CQW column quads, so the per-row reductions are shuffles within the wave and
  // the row loop has no barrier (the fused norm, which needs a whole head, runs
  // after the loop).  The one-token decode and the verify that stores every state
  // keep a wave over 2 row groups x all column quads: their stores then cover whole
  // consecutive 512-byte rows, which the HBM write stream takes faster than
  // 128-byte pieces.
  constexpr bool kInWave = MODE == kModeWoa || MODE == kModeTokens;
  constexpr int CQW = CQ / 4;  // column quads per wave (in-wave layout)
  // Multi-row modes apply the fused norm after the row loop (one wave per row and
  // value head), the same code for both layouts; together with reductions of the
  // same association (a butterfly over row groups in the in-wave layout, pairs of
  // wave partials in the other) every multi-row mode produces bit-identical
  // outputs and update vectors, so a fold of the stash equals the recorded states
  // (the write-on-accept verify runs here for binary16 states and d = 32; fp32
  // states at d >= 64 take the WY form of recurrent_wy.h).
  constexpr bool kPostNorm = MODE != kModeDecode;
  static_assert(RPT * RG == D, "head dim must split over the row groups");
  static_assert((MODE == kModeDecode) == (MAXR == 1), "one-token decode is the MAXR = 1 instance");

  __shared__ float s_qkv[MAXR][NCH];
  __shared__ float s_a[MAXR][G], s_b[MAXR][G];
  __shared__ float s_qk[MAXR];
  __shared__ float s_zw[kPostNorm ? 1 : MAXR][G * D];  // gate(z) * norm weight (decode)
  __shared__ TS *s_dst[kStoresEveryRow ? MAXR : 1];  // verify: where the state after each row goes
  __shared__ float4 s_red[kInWave ? 1 : 2][G][4][CQ][2];
  __shared__ float s_o[kPostNorm ? MAXR : 1][G * D];  // pre-norm outputs (multi-row modes, with z)

  const int Hk = p.geo.Hk, Hv = p.geo.Hv, K = p.geo.K, C = p.geo.conv_dim;
  const int rank = blockIdx.x / Hk;
  const int g = blockIdx.x - rank * Hk;
  const int tid = threadIdx.x;

  int i, r0, nrows;
  if (MODE == kModeDecode) {
    i = rank;
    r0 = i;
    nrows = 1;
  } else {
    // several rows per sequence: workgroups take sequences longest first
    __shared__ int s_seq;
    i = seq_of_rank(p.cu, p.n, rank, NT, &s_seq);
    // uniform over the block: read into scalar registers, so that every address
    // derived from them is scalar too
    r0 = __builtin_amdgcn_readfirstlane(p.cu[i]);
    nrows = __builtin_amdgcn_readfirstlane(p.cu[i + 1]) - r0;
    nrows = nrows < 0 ? 0 : (nrows > MAXR ? MAXR : nrows);
  }
  if (nrows == 0) return;  // uniform over the block

  // ---- prologue loads: conv taps, conv state, input rows, gates, z ------------
  // All issued first, unconditionally from valid addresses, and kept raw until the
  // state loads below have been issued: a conditional or converted load would make
  // the compiler wait for it (and, the counter being in order, for everything
  // issued before it) in the middle of the prologue.
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  TA *ring = static_cast<TA *>(p.conv_state[i]);
  constexpr int NIT = (NCH + NT - 1) / NT;  // channels per thread
  const bool has_z = p.z != nullptr;
  auto chan = [&](int cl) {  // conv channel of group channel cl (q, k, then the G v heads)
    if (cl < D) return g * D + cl;
    if (cl < 2 * D) return Hk * D + g * D + (cl - D);
    return 2 * Hk * D + g * G * D + (cl - 2 * D);
  };
  TA rw[NIT][4], rr3[NIT][3], rx[NIT][MAXR];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = chan(min(tid + it * NT, NCH - 1));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) rw[it][jj] = w[(size_t)c * K + max(jj - (4 - K), 0)];  // tap for row t-3+jj
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) rr3[it][jj] = ring[(size_t)max(K - 4 + jj, 0) * C + c];  // row jj-3
#pragma unroll
    for (int r = 0; r < MAXR; ++r) rx[it][r] = x[(size_t)(r0 + min(r, nrows - 1)) * C + c];
  }
  // gates of (row, value head) tid / G, tid % G; z and the norm weight of value
  // channel tid of the group, for every row
  const int gr = min(tid / G, MAXR - 1), gs = tid % G;
  const float ga = p.a[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];
  const float gb = p.b[(size_t)(r0 + min(gr, nrows - 1)) * Hv + g * G + gs];
  // destination of the state after row tid: table tid + 1, table 0 after the last
  TS *dst_mid = nullptr;
  if (kStoresEveryRow)
    dst_mid = static_cast<TS *>(p.states[(min(tid, max(nrows - 2, 0)) + (nrows > 1 ? 1 : 0)) * kTableSeqs + i]);
  TS *const dst_last = static_cast<TS *>(p.states[i]);
  const TA *zp = has_z ? static_cast<const TA *>(p.z) : x;
  const TA *nwp = has_z ? static_cast<const TA *>(p.norm_w) : x;
  const int zc = min(tid, G * D - 1);
  constexpr int NZ = kPostNorm ? 1 : MAXR;  // z rows staged by the prologue (decode)
  TA rz[NZ];
#pragma unroll
  for (int r = 0; r < NZ; ++r)
    rz[r] = zp[has_z ? (size_t)(r0 + min(r, nrows - 1)) * Hv * D + (size_t)g * G * D + zc : 0];
  const TA rnw = nwp[has_z ? zc % D : 0];

  // ---- the state loads -------------------------------------------------------
  // One-token decode issues them here, so the prologue's arithmetic hides their
  // latency.  The multi-row modes issue them after the prologue has consumed its
  // raw rows: the two sets of registers are then never live together, which keeps
  // the kernel within the register budget of two workgroups per CU, and the other
  // workgroup on the CU hides the latency instead.
  const int s = tid / kSlot, t = tid % kSlot;
  const int h = g * G + s;
  const int cq = kInWave ? (t / kWave) * CQW + (t % kWave) % CQW : t % CQ;
  const int rg = kInWave ? (t % kWave) / CQW : t / CQ;
  const gptr<const TS> S_in = to_global(static_cast<const TS *>(p.states[i])) + (size_t)h * D * D;
  typename StateIO<TS>::raw st_raw[RPT];
  auto load_state = [&]() {
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) st_raw[rr] = StateIO<TS>::load(S_in + (size_t)state_row<D>(rg, rr) * D + 4 * cq);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (MODE == kModeDecode) load_state();

  // ---- prologue: conv + SiLU of the group's channels for every row ----------
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int cl = tid + it * NT;
    if (cl >= NCH) break;
    const int c = chan(cl);
    // q and k in the staging order of the state rows; v in channel order
    const int slot = cl < D ? staged_slot<D>(cl) : (cl < 2 * D ? D + staged_slot<D>(cl - D) : cl);
    float wt[4], win[3];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wt[jj] = (jj >= 4 - K) ? (float)rw[it][jj] : 0.0f;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) win[jj] = (K - 4 + jj >= 0) ? (float)rr3[it][jj] : 0.0f;
    // (a guarded body per row rather than an exit from the unrolled loop: the exit
    // sends the row arrays of some instances to scratch memory)
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nrows) {
        const float xv = (float)rx[it][r];
        s_qkv[r][slot] = silu(wt[0] * win[0] + wt[1] * win[1] + wt[2] * win[2] + wt[3] * xv);
        win[0] = win[1];
        win[1] = win[2];
        win[2] = xv;
      }
    }
    if (kAdvancesRing) {  // the conv state becomes the last K-1 rows of [conv state ; rows]
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        // row j of the new state is win[j + 4 - K]; selected with constant indices (a
        // register array indexed by the run-time K would live in scratch memory)
        const int idx = j + 4 - K;
        const float v = idx == 0 ? win[0] : (idx == 1 ? win[1] : win[2]);
        if (j < K - 1) st(ring, (size_t)j * C + c, v);
      }
    }
  }
  if (tid < MAXR * G && gr < nrows) {
    s_a[gr][gs] = p.gates_raw ? decay_from_raw(ga) : ga;
    s_b[gr][gs] = p.gates_raw ? strength_from_raw(gb) : gb;
  }
  if (kStoresEveryRow && tid < MAXR) s_dst[tid] = tid < nrows - 1 ? dst_mid : dst_last;
  if (!kPostNorm && has_z && tid < G * D) {
    const float nwv = (float)rnw;
#pragma unroll
    for (int r = 0; r < NZ; ++r)
      if (r < nrows) {
        const float zv = (float)rz[r];
        s_zw[kPostNorm ? 0 : r][tid] = norm_gate(zv, p.norm_sigmoid) * nwv;
      }
  }
  __syncthreads();

  // ---- L2 norm of q and k, and q_hat . k_hat, one wave per row --------------
  {
    const int wave = tid / kWave, lane = tid % kWave;
    for (int r = wave; r < nrows; r += NT / kWave) {
      float sq = 0.0f, sk = 0.0f, dqk = 0.0f;
      for (int c = lane; c < D; c += kWave) {  // channel order (the slots are a permutation)
        const int sc = staged_slot<D>(c);
        const float qv = s_qkv[r][sc], kv = s_qkv[r][D + sc];
        sq += qv * qv;
        sk += kv * kv;
        dqk += qv * kv;
      }
      sq = wave_sum(sq);
      sk = wave_sum(sk);
      dqk = wave_sum(dqk);
      const float iq = rsqrt_hw(sq + p.l2_eps), ik = rsqrt_hw(sk + p.l2_eps);
      for (int c = lane; c < D; c += kWave) {
        s_qkv[r][c] *= iq;  // every slot once, whatever its channel
        s_qkv[r][D + c] *= ik;
      }
      if (lane == 0) s_qk[r] = dqk * iq * ik;
    }
  }
  if constexpr (MODE != kModeDecode) load_state();
  __syncthreads();

  // ---- the recurrence, row by row --------------------------------------------
  // Every load is done by now (the state arrived during the prologue): the loop
  // issues only stores, and no wait inside it makes a row wait for the previous
  // row's state stores to complete.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  floatx4 st_reg[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) st_reg[rr] = StateIO<TS>::widen(st_raw[rr]);
  const int wv = t / kWave, lane = t % kWave;
  const int stash_u = Hk * D + h * D, stash_a = Hk * D + Hv * D + g * G;
  for (int r = 0; r < nrows; ++r) {
    const float *qh = &s_qkv[r][0];
    const float *kh = &s_qkv[r][D];
    // this thread's rows of k_hat (kept for the update) and of q_hat (four at a time),
    // consecutive in the staging order
    float kr[RPT];
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (RPT % 4 == 0) {  // 16-byte aligned groups of 4 rows
#pragma unroll
      for (int j = 0; j < RPT; j += 4) {
        *reinterpret_cast<floatx4 *>(&kr[j]) = *reinterpret_cast<const floatx4 *>(&kh[rg * RPT + j]);
        const floatx4 q4 = *reinterpret_cast<const floatx4 *>(&qh[rg * RPT + j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const floatx4 sv = st_reg[j + e];
          const float kk = kr[j + e], qq = q4[e];
          pk.x += kk * sv.x; pk.y += kk * sv.y; pk.z += kk * sv.z; pk.w += kk * sv.w;
          pq.x += qq * sv.x; pq.y += qq * sv.y; pq.z += qq * sv.z; pq.w += qq * sv.w;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        kr[j] = kh[rg * RPT + j];
        const float kk = kr[j], qq = qh[rg * RPT + j];
        const floatx4 sv = st_reg[j];
        pk.x += kk * sv.x; pk.y += kk * sv.y; pk.z += kk * sv.z; pk.w += kk * sv.w;
        pq.x += qq * sv.x; pq.y += qq * sv.y; pq.z += qq * sv.z; pq.w += qq * sv.w;
      }
    }
    float4 kv, sq;
    if constexpr (kInWave) {  // the lanes sharing lane % CQW hold all rows of these columns
      kv = make_float4(sum_across_groups<CQW>(pk.x), sum_across_groups<CQW>(pk.y), sum_across_groups<CQW>(pk.z),
                       sum_across_groups<CQW>(pk.w));
      sq = make_float4(sum_across_groups<CQW>(pq.x), sum_across_groups<CQW>(pq.y), sum_across_groups<CQW>(pq.z),
                       sum_across_groups<CQW>(pq.w));
    } else {
      pk.x = sum_across_groups<CQ>(pk.x); pk.y = sum_across_groups<CQ>(pk.y);
      pk.z = sum_across_groups<CQ>(pk.z); pk.w = sum_across_groups<CQ>(pk.w);
      pq.x = sum_across_groups<CQ>(pq.x); pq.y = sum_across_groups<CQ>(pq.y);
      pq.z = sum_across_groups<CQ>(pq.z); pq.w = sum_across_groups<CQ>(pq.w);
      if (lane < CQ) {
        s_red[r & 1][s][wv][cq][0] = pk;
        s_red[r & 1][s][wv][cq][1] = pq;
      }
      __syncthreads();
      // the four wave partials in pairs, (w0 + w1) + (w2 + w3): the association of
      // the in-wave butterfly
      float4 k01 = s_red[r & 1][s][0][cq][0], q01 = s_red[r & 1][s][0][cq][1];
      float4 k23 = s_red[r & 1][s][2][cq][0], q23 = s_red[r & 1][s][2][cq][1];
      const float4 k1 = s_red[r & 1][s][1][cq][0], q1 = s_red[r & 1][s][1][cq][1];
      const float4 k3 = s_red[r & 1][s][3][cq][0], q3 = s_red[r & 1][s][3][cq][1];
      k01.x += k1.x; k01.y += k1.y; k01.z += k1.z; k01.w += k1.w;
      q01.x += q1.x; q01.y += q1.y; q01.z += q1.z; q01.w += q1.w;
      k23.x += k3.x; k23.y += k3.y; k23.z += k3.z; k23.w += k3.w;
      q23.x += q3.x; q23.y += q3.y; q23.z += q3.z; q23.w += q3.w;
      kv = make_float4(k01.x + k23.x, k01.y + k23.y, k01.z + k23.z, k01.w + k23.w);
      sq = make_float4(q01.x + q23.x, q01.y + q23.y, q01.z + q23.z, q01.w + q23.w);
    }
    const float av = s_a[r][s], bv = s_b[r][s];
    const float4 v = *reinterpret_cast<const float4 *>(&s_qkv[r][2 * D + s * D + 4 * cq]);
    floatx4 u;
    u.x = bv * (v.x - av * kv.x); u.y = bv * (v.y - av * kv.y);
    u.z = bv * (v.z - av * kv.z); u.w = bv * (v.w - av * kv.w);

    // the one-token decode stores its state here; the k-token decode once after
    // the loop, so that no store in the loop depends on the row
    const bool store_now = kStoresEveryRow || (MODE == kModeDecode && r == nrows - 1);
    gptr<TS> dst = to_global(kStoresEveryRow ? uniform_ptr(s_dst[r]) : dst_last) + (size_t)h * D * D;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const floatx4 nv = StateIO<TS>::as_stored(rank1_update(st_reg[rr], av, kr[rr], u));
      st_reg[rr] = nv;
      if (store_now) {
        if constexpr (kStoresEveryRow)
          StateIO<TS>::store_kept(dst + (size_t)state_row<D>(rg, rr) * D + 4 * cq, nv);
        else
          StateIO<TS>::store(dst + (size_t)state_row<D>(rg, rr) * D + 4 * cq, nv);
        // binary16: issue each narrowed row now rather than holding them all
        if constexpr (sizeof(TS) == 2 && kStoresEveryRow) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (MODE == kModeWoa) {  // stash row r0 + r: k_hat of the key head, u and a of the value heads
      gptr<float> srow = to_global(p.stash) + (size_t)(r0 + r) * p.stash_row;
      if (rg == 0) *reinterpret_cast<gptr<floatx4>>(srow + stash_u + 4 * cq) = u;
      if (tid < CQ)  // channel order
        *reinterpret_cast<gptr<floatx4>>(srow + g * D + 4 * tid) =
            floatx4{kh[staged_slot<D>(4 * tid)], kh[staged_slot<D>(4 * tid + 1)], kh[staged_slot<D>(4 * tid + 2)],
                    kh[staged_slot<D>(4 * tid + 3)]};
      if (tid < G) srow[stash_a + tid] = s_a[r][tid];
    }

    if (rg == 0) {  // row group 0 holds each column quad's outputs once
      const float qk = s_qk[r];
      float o[4];
      o[0] = p.scale * (av * sq.x + qk * u.x); o[1] = p.scale * (av * sq.y + qk * u.y);
      o[2] = p.scale * (av * sq.z + qk * u.z); o[3] = p.scale * (av * sq.w + qk * u.w);
      const size_t obase = (size_t)(r0 + r) * Hv * D + (size_t)h * D + 4 * cq;
      if (kPostNorm && has_z) {  // normalised after the loop
        *reinterpret_cast<float4 *>(&s_o[kPostNorm ? r : 0][s * D + 4 * cq]) = make_float4(o[0], o[1], o[2], o[3]);
      } else if (has_z) {
        float ss2 = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
        ss2 = sum_within_span<CQ>(ss2);
        const float inv = rsqrt_hw(ss2 / D + p.norm_eps);
        const float4 zw = *reinterpret_cast<const float4 *>(&s_zw[kPostNorm ? 0 : r][s * D + 4 * cq]);
        o[0] *= inv * zw.x; o[1] *= inv * zw.y; o[2] *= inv * zw.z; o[3] *= inv * zw.w;
      }
      if (!(kPostNorm && has_z)) {
        if (p.geo.out_bf16)
          store4(static_cast<bf16 *>(p.out) + obase, o);
        else
          store4(static_cast<float *>(p.out) + obase, o);
      }
    }
  }
  if constexpr (MODE == kModeTokens) {
    const gptr<TS> dst = to_global(dst_last) + (size_t)h * D * D;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) StateIO<TS>::store(dst + (size_t)state_row<D>(rg, rr) * D + 4 * cq, st_reg[rr]);
  }
  if constexpr (kPostNorm) {
    if (has_z) {  // the gated norm of every (row, value head), one wave each
      __syncthreads();
      constexpr int VPL = (D + kWave - 1) / kWave;  // values per lane
      const int wave = tid / kWave, ln = tid % kWave;
      const TA *zq = static_cast<const TA *>(p.z), *nw = static_cast<const TA *>(p.norm_w);
      for (int item = wave; item < nrows * G; item += NT / kWave) {
        const int r = item / G, s2 = item - r * G;
        const size_t obase = (size_t)(r0 + r) * Hv * D + (size_t)(g * G + s2) * D;
        float ov[VPL], zv[VPL], wv[VPL], ss = 0.0f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = min(ln + kWave * j, D - 1);
          zv[j] = (float)zq[obase + c];
          wv[j] = (float)nw[c];
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = ln + kWave * j;
          ov[j] = c < D ? s_o[r][s2 * D + c] : 0.0f;
          ss += ov[j] * ov[j];
        }
        ss = wave_sum(ss);
        const float inv = rsqrt_hw(ss / D + p.norm_eps);
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int c = ln + kWave * j;
          if (c < D) {
            const float v = ov[j] * inv * (norm_gate(zv[j], p.norm_sigmoid) * wv[j]);
            if (p.geo.out_bf16)
              st(static_cast<bf16 *>(p.out), obase + c, v);
            else
              st(static_cast<float *>(p.out), obase + c, v);
          }
        }
      }
    }
  }
}

// Launch of one mode over the supported shapes: D in {32, 64, 128}, H_v / H_k in
// {1, 2, 4}, activations fp32 or bf16, states fp32 or binary16.
template <int D, int G, int MAXR, int MODE, typename TA>
hipError_t launch_rec_ts(const RecurrentLaunch &p, hipStream_t stream) {
  const dim3 grid(p.n * p.geo.Hk), block(kSlot * G);
  // the write-on-accept verify over fp32 states at d >= 64 takes the WY form
  // (recurrent_wy.h); this kernel serves it with binary16 states and at d = 32.
  constexpr bool kF32ViaWy = MODE == kModeWoa && D >= 64;
  if (p.state_f16)
    hipLaunchKernelGGL((recurrent_kernel<D, G, MAXR, MODE, TA, _Float16>), grid, block, 0, stream, p);
  else if constexpr (kF32ViaWy)
    return hipErrorInvalidValue;
  else
    hipLaunchKernelGGL((recurrent_kernel<D, G, MAXR, MODE, TA, float>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, int MAXR, int MODE>
hipError_t launch_rec_ta(const RecurrentLaunch &p, hipStream_t stream) {
  return p.geo.act_bf16 ? launch_rec_ts<D, G, MAXR, MODE, bf16>(p, stream)
                        : launch_rec_ts<D, G, MAXR, MODE, float>(p, stream);
}

template <int D, int MAXR, int MODE>
hipError_t launch_rec_g(const RecurrentLaunch &p, hipStream_t stream) {
  switch (p.geo.Hv / p.geo.Hk) {
    case 1: return launch_rec_ta<D, 1, MAXR, MODE>(p, stream);
    case 2: return launch_rec_ta<D, 2, MAXR, MODE>(p, stream);
    case 4: return launch_rec_ta<D, 4, MAXR, MODE>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int MAXR, int MODE>
hipError_t launch_rec_mode(const RecurrentLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  switch (p.geo.D) {
    case 32: return launch_rec_g<32, MAXR, MODE>(p, stream);
    case 64: return launch_rec_g<64, MAXR, MODE>(p, stream);
    case 128: return launch_rec_g<128, MAXR, MODE>(p, stream);
  }
  return hipErrorInvalidValue;
}

// One translation unit per mode defines its launcher.
hipError_t launch_rec_decode(const RecurrentLaunch &p, hipStream_t stream);
hipError_t launch_rec_tokens(const RecurrentLaunch &p, hipStream_t stream);
hipError_t launch_rec_verify(const RecurrentLaunch &p, hipStream_t stream);
hipError_t launch_rec_woa(const RecurrentLaunch &p, hipStream_t stream);

}  // namespace gdn
