// One-token batched decode, k-row verify with every intermediate state written
// through the WY pointer tables, and the commit of the accepted prefix.
//
// Decode (decode_multi_seq on the metrale_model_layers/layer/transformer_layer.rs
// page; the strided one-launch kernels conv1d_l2norm_f32_strided_k,
// gdn_f32_strided_norm_k and gated_rms_norm_f32_strided_k on the
// metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page) and verify
// (decode_verify_multi and the VERIFY_WY_* table constants, transformer_layer.rs;
// gdn_wyn_table_k, gdn_f32_strided_norm_snap_k, layer_struct.rs) are one kernel:
// verify runs k rows from the state in table 0 and stores the state after each
// row, decode is one row that also advances the conv state.
//
// Design (MI355X): the path is HBM-bound -- each value head's 128x128 fp32 state
// (64 KiB) is read once and written once (decode) or k times (verify).  One
// workgroup owns one (sequence, key head) pair: the conv + L2 prologue of the
// shared q/k channels runs once and feeds the H_v/H_k value heads of the group
// through LDS, and because one workgroup owns all channels of the group the
// in-place conv-state update has no cross-workgroup race.  256 threads own one
// value head: thread t holds column quad (t % 32) of rows {rr * 8 + t / 32}, so
// every wave-wide 16-byte load or store covers whole contiguous 512-byte state
// rows, and the state stays in registers across the k verify rows.  S k and S q
// are reduced over row groups with wave shuffles and one LDS exchange per row.
// All arithmetic is fp32 (the recurrence per token is
//   kv = S k;  u = b (v - a kv);  S <- a S + u k^T;  o = scale (a S q + (k.q) u),
// the last being S_new q expanded).
#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kSlot = 256;          // threads per value head

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
constexpr int kTableSeqs = 128;     // entries per WY pointer table
// s_waitcnt immediate: vector-memory counter 0 (bits 3:0 and 15:14), expcnt and
// lgkmcnt at their maxima (no wait)
constexpr int kWaitVmem0 = (7 << 4) | (15 << 8);

template <int D, int G, int MAXR, typename TA, typename TO>
__global__ __launch_bounds__(kSlot *G) void recurrent_kernel(RecurrentLaunch p) {
  constexpr int CQ = D / 4;            // column quads of a head
  constexpr int RG = kSlot / CQ;       // row groups
  constexpr int RPT = D / RG;          // state rows held by a thread
  constexpr int NCH = (2 + G) * D;     // q, k, and G v heads
  constexpr int NT = kSlot * G;
  static_assert(RPT * RG == D, "head dim must split over the row groups");

  __shared__ float s_qkv[MAXR][NCH];
  __shared__ float s_a[MAXR][G], s_b[MAXR][G];
  __shared__ float s_qk[MAXR];
  __shared__ float s_zw[MAXR][G * D];  // silu(z) * norm weight of the group's value channels
  __shared__ float *s_dst[MAXR];       // where the state after each row is stored
  __shared__ float4 s_red[2][G][4][CQ][2];

  const int Hk = p.geo.Hk, Hv = p.geo.Hv, K = p.geo.K, C = p.geo.conv_dim;
  const int rank = blockIdx.x / Hk;
  const int g = blockIdx.x - rank * Hk;
  const int tid = threadIdx.x;

  int i, r0, nrows;
  if (MAXR == 1) {
    i = rank;
    r0 = i;
    nrows = 1;
  } else {
    // verify: workgroups take sequences longest draft first, so the long ones
    // do not trail at the end of the grid (ranks of the <= 128 lengths, ties by index)
    __shared__ int s_cu[kTableSeqs + 1];
    __shared__ int s_seq;
    for (int t = tid; t <= p.n; t += NT) s_cu[t] = p.cu[t];
    __syncthreads();
    for (int t = tid; t < p.n; t += NT) {
      const int kt = s_cu[t + 1] - s_cu[t];
      int rk = 0;
      for (int s2 = 0; s2 < p.n; ++s2) {
        const int k2 = s_cu[s2 + 1] - s_cu[s2];
        rk += (k2 > kt) || (k2 == kt && s2 < t);
      }
      if (rk == rank) s_seq = t;
    }
    __syncthreads();
    i = s_seq;
    r0 = s_cu[i];
    nrows = s_cu[i + 1] - r0;
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
  float *const dst_mid = p.states[(min(tid, max(nrows - 2, 0)) + (nrows > 1 ? 1 : 0)) * kTableSeqs + i];
  float *const dst_last = p.states[i];
  const TA *zp = has_z ? static_cast<const TA *>(p.z) : x;
  const TA *nwp = has_z ? static_cast<const TA *>(p.norm_w) : x;
  const int zc = min(tid, G * D - 1);
  TA rz[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
    rz[r] = zp[has_z ? (size_t)(r0 + min(r, nrows - 1)) * Hv * D + (size_t)g * G * D + zc : 0];
  const TA rnw = nwp[has_z ? zc % D : 0];

  // ---- the state loads; the prologue's arithmetic hides their latency ---------
  const int s = tid / kSlot, t = tid % kSlot;
  const int h = g * G + s;
  const int cq = t % CQ, rg = t / CQ;
  const gptr<float> S_in = to_global(p.states[i]) + (size_t)h * D * D;  // table 0 / decode pointer
  floatx4 st_reg[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr)
    st_reg[rr] = *reinterpret_cast<const gptr<floatx4>>(S_in + (size_t)(rr * RG + rg) * D + 4 * cq);
  __builtin_amdgcn_sched_barrier(0);

  // ---- prologue: conv + SiLU of the group's channels for every row ----------
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int cl = tid + it * NT;
    if (cl >= NCH) break;
    const int c = chan(cl);
    float wt[4], win[3];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wt[jj] = (jj >= 4 - K) ? (float)rw[it][jj] : 0.0f;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) win[jj] = (K - 4 + jj >= 0) ? (float)rr3[it][jj] : 0.0f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r >= nrows) break;
      const float xv = (float)rx[it][r];
      s_qkv[r][cl] = silu(wt[0] * win[0] + wt[1] * win[1] + wt[2] * win[2] + wt[3] * xv);
      win[0] = win[1];
      win[1] = win[2];
      win[2] = xv;
    }
    if (MAXR == 1) {  // decode advances the conv state by one row: new rows are t-2, t-1, t
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) st(ring, (size_t)j * C + c, win[3 - (K - 1) + j]);
    }
  }
  if (tid < MAXR * G && gr < nrows) {
    s_a[gr][gs] = ga;
    s_b[gr][gs] = gb;
  }
  if (tid < MAXR) s_dst[tid] = (MAXR > 1 && tid < nrows - 1) ? dst_mid : dst_last;
  if (has_z && tid < G * D) {
    const float nwv = (float)rnw;
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
      if (r < nrows) s_zw[r][tid] = silu((float)rz[r]) * nwv;
  }
  __syncthreads();

  // ---- L2 norm of q and k, and q_hat . k_hat, one wave per row --------------
  {
    const int wave = tid / kWave, lane = tid % kWave;
    for (int r = wave; r < nrows; r += NT / kWave) {
      float sq = 0.0f, sk = 0.0f, dqk = 0.0f;
      for (int c = lane; c < D; c += kWave) {
        const float qv = s_qkv[r][c], kv = s_qkv[r][D + c];
        sq += qv * qv;
        sk += kv * kv;
        dqk += qv * kv;
      }
      sq = wave_sum(sq);
      sk = wave_sum(sk);
      dqk = wave_sum(dqk);
      const float iq = rsqrt_hw(sq + p.l2_eps), ik = rsqrt_hw(sk + p.l2_eps);
      for (int c = lane; c < D; c += kWave) {
        s_qkv[r][c] *= iq;
        s_qkv[r][D + c] *= ik;
      }
      if (lane == 0) s_qk[r] = dqk * iq * ik;
    }
  }
  __syncthreads();

  // ---- the recurrence, row by row --------------------------------------------
  // Every load is done by now (the state arrived during the prologue): the loop
  // issues only stores, and no wait inside it makes a row wait for the previous
  // row's state stores to complete.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  const int wv = t / kWave, lane = t % kWave;
  for (int r = 0; r < nrows; ++r) {
    const float *qh = &s_qkv[r][0];
    const float *kh = &s_qkv[r][D];
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int row = rr * RG + rg;
      const float kk = kh[row], qq = qh[row];
      pk.x += kk * st_reg[rr].x; pk.y += kk * st_reg[rr].y; pk.z += kk * st_reg[rr].z; pk.w += kk * st_reg[rr].w;
      pq.x += qq * st_reg[rr].x; pq.y += qq * st_reg[rr].y; pq.z += qq * st_reg[rr].z; pq.w += qq * st_reg[rr].w;
    }
    pk.x = sum_across_groups<CQ>(pk.x); pk.y = sum_across_groups<CQ>(pk.y);
    pk.z = sum_across_groups<CQ>(pk.z); pk.w = sum_across_groups<CQ>(pk.w);
    pq.x = sum_across_groups<CQ>(pq.x); pq.y = sum_across_groups<CQ>(pq.y);
    pq.z = sum_across_groups<CQ>(pq.z); pq.w = sum_across_groups<CQ>(pq.w);
    if (lane < CQ) {
      s_red[r & 1][s][wv][cq][0] = pk;
      s_red[r & 1][s][wv][cq][1] = pq;
    }
    __syncthreads();
    float4 kv = s_red[r & 1][s][0][cq][0], sq = s_red[r & 1][s][0][cq][1];
#pragma unroll
    for (int wj = 1; wj < 4; ++wj) {
      const float4 a0 = s_red[r & 1][s][wj][cq][0], a1 = s_red[r & 1][s][wj][cq][1];
      kv.x += a0.x; kv.y += a0.y; kv.z += a0.z; kv.w += a0.w;
      sq.x += a1.x; sq.y += a1.y; sq.z += a1.z; sq.w += a1.w;
    }
    const float av = s_a[r][s], bv = s_b[r][s];
    const float4 v = *reinterpret_cast<const float4 *>(&s_qkv[r][2 * D + s * D + 4 * cq]);
    float4 u;
    u.x = bv * (v.x - av * kv.x); u.y = bv * (v.y - av * kv.y);
    u.z = bv * (v.z - av * kv.z); u.w = bv * (v.w - av * kv.w);

    gptr<float> dst = to_global(s_dst[r]) + (size_t)h * D * D;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int row = rr * RG + rg;
      const float kk = kh[row];
      floatx4 nv;
      nv.x = av * st_reg[rr].x + kk * u.x; nv.y = av * st_reg[rr].y + kk * u.y;
      nv.z = av * st_reg[rr].z + kk * u.z; nv.w = av * st_reg[rr].w + kk * u.w;
      st_reg[rr] = nv;
      *reinterpret_cast<gptr<floatx4>>(dst + (size_t)row * D + 4 * cq) = nv;
    }

    if (rg == 0) {  // lanes 0..CQ-1 of the slot's first wave hold the head's outputs
      const float qk = s_qk[r];
      float o[4];
      o[0] = p.scale * (av * sq.x + qk * u.x); o[1] = p.scale * (av * sq.y + qk * u.y);
      o[2] = p.scale * (av * sq.z + qk * u.z); o[3] = p.scale * (av * sq.w + qk * u.w);
      const size_t obase = (size_t)(r0 + r) * Hv * D + (size_t)h * D + 4 * cq;
      if (has_z) {
        float ss2 = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
        ss2 = sum_within_span<CQ>(ss2);
        const float inv = rsqrt_hw(ss2 / D + p.norm_eps);
        const float4 zw = *reinterpret_cast<const float4 *>(&s_zw[r][s * D + 4 * cq]);
        o[0] *= inv * zw.x; o[1] *= inv * zw.y; o[2] *= inv * zw.z; o[3] *= inv * zw.w;
      }
      store4(static_cast<TO *>(p.out) + obase, o);
    }
  }
}

// Commit: copy the state after the last accepted row into table 0 and advance the
// conv state over the accepted rows.  blockIdx.y < kCommitSplit: one eighth of the
// state copy, 8 loads in flight per thread; otherwise conv-state channels.
constexpr int kCommitSplit = 8;

template <typename TE>
__global__ __launch_bounds__(256) void commit_kernel(CommitLaunch p, int64_t n4) {
  const int i = blockIdx.x;
  const int k = p.cu[i + 1] - p.cu[i];
  const int na = p.n_accepted[i];
  if (na < 1 || na > k) return;  // outside the caller's contract: sequence untouched
  if ((int)blockIdx.y < kCommitSplit) {
    if (na == k) return;  // table 0 already holds the last state
    // (native 4-float vectors: the struct-based float4 array ends up in scratch)
    const gptr<const floatx4> src = to_global(reinterpret_cast<const floatx4 *>(p.tables[na * kTableSeqs + i]));
    const gptr<floatx4> dst = to_global(reinterpret_cast<floatx4 *>(p.tables[i]));
    const int64_t per = (n4 + kCommitSplit - 1) / kCommitSplit;
    const int64_t beg = (int64_t)blockIdx.y * per, end = min(n4, beg + per);
    // whole tiles of 256 x 8 float4 without conditions, then the tail
    int64_t i0 = beg;
    for (; i0 + 256 * 8 <= end; i0 += 256 * 8) {
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[i0 + threadIdx.x + u * 256];
#pragma unroll
      for (int u = 0; u < 8; ++u) dst[i0 + threadIdx.x + u * 256] = v[u];
    }
    for (int64_t idx = i0 + threadIdx.x; idx < end; idx += 256) dst[idx] = src[idx];
  } else {
    const int C = p.geo.conv_dim, R = p.geo.K - 1;
    const int c = ((int)blockIdx.y - kCommitSplit) * 256 + threadIdx.x;
    if (c >= C) return;
    TE *ring = static_cast<TE *>(p.conv_state[i]);
    const TE *x = static_cast<const TE *>(p.x) + (size_t)p.cu[i] * C;
    TE vals[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {  // position na + r of [old conv state ; accepted rows]
      const int idx = na + min(r, R - 1);
      const TE vr = ring[(size_t)min(idx, R - 1) * C + c], vx = x[(size_t)max(idx - R, 0) * C + c];
      vals[r] = (idx < R) ? vr : vx;
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
      if (r < R) ring[(size_t)r * C + c] = vals[r];
  }
}

template <int D, int G, int MAXR, typename TA>
hipError_t launch_rec_to(const RecurrentLaunch &p, hipStream_t stream) {
  const dim3 grid(p.n * p.geo.Hk), block(kSlot * G);
  if (p.geo.out_bf16)
    hipLaunchKernelGGL((recurrent_kernel<D, G, MAXR, TA, bf16>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_kernel<D, G, MAXR, TA, float>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, int MAXR>
hipError_t launch_rec_ta(const RecurrentLaunch &p, hipStream_t stream) {
  return p.geo.act_bf16 ? launch_rec_to<D, G, MAXR, bf16>(p, stream)
                        : launch_rec_to<D, G, MAXR, float>(p, stream);
}

template <int D, int G>
hipError_t launch_rec_mode(const RecurrentLaunch &p, hipStream_t stream) {
  return p.verify ? launch_rec_ta<D, G, 16>(p, stream) : launch_rec_ta<D, G, 1>(p, stream);
}

template <int D>
hipError_t launch_rec_g(const RecurrentLaunch &p, hipStream_t stream) {
  switch (p.geo.Hv / p.geo.Hk) {
    case 1: return launch_rec_mode<D, 1>(p, stream);
    case 2: return launch_rec_mode<D, 2>(p, stream);
    case 4: return launch_rec_mode<D, 4>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const RecurrentLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  switch (p.geo.D) {
    case 32: return launch_rec_g<32>(p, stream);
    case 64: return launch_rec_g<64>(p, stream);
    case 128: return launch_rec_g<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_commit(const CommitLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  const int64_t n4 = (int64_t)p.geo.Hv * p.geo.D * p.geo.D / 4;
  const int nblk_ring = (p.geo.conv_dim + 255) / 256;
  const dim3 grid(p.n, kCommitSplit + nblk_ring), block(256);
  if (p.geo.act_bf16)
    hipLaunchKernelGGL((commit_kernel<uint16_t>), grid, block, 0, stream, p, n4);
  else
    hipLaunchKernelGGL((commit_kernel<float>), grid, block, 0, stream, p, n4);
  return hipGetLastError();
}

}  // namespace gdn
