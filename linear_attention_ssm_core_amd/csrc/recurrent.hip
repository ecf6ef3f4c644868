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
constexpr int kTableSeqs = 128;     // entries per WY pointer table

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

  // ---- issue the state loads first; the prologue hides their latency --------
  const int s = tid / kSlot, t = tid % kSlot;
  const int h = g * G + s;
  const int cq = t % CQ, rg = t / CQ;
  const float *S_in = p.states[i] + (size_t)h * D * D;  // table 0 / decode pointer
  float4 st_reg[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr)
    st_reg[rr] = *reinterpret_cast<const float4 *>(S_in + (size_t)(rr * RG + rg) * D + 4 * cq);

  // ---- prologue: conv + SiLU of the group's channels for every row ----------
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  TA *ring = static_cast<TA *>(p.conv_state[i]);
  for (int cl = tid; cl < NCH; cl += NT) {
    int c;
    if (cl < D) c = g * D + cl;
    else if (cl < 2 * D) c = Hk * D + g * D + (cl - D);
    else c = 2 * Hk * D + g * G * D + (cl - 2 * D);
    float wt[3], hist[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) wt[j] = (j < K - 1) ? ld(w, (size_t)c * K + j) : 0.0f;
    const float wlast = ld(w, (size_t)c * K + K - 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) hist[j] = (j < K - 1) ? ld(ring, (size_t)j * C + c) : 0.0f;
    for (int r = 0; r < nrows; ++r) {
      const float xv = ld(x, (size_t)(r0 + r) * C + c);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) acc += wt[j] * hist[j];
      acc += wlast * xv;
      s_qkv[r][cl] = silu(acc);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j < K - 2) hist[j] = hist[j + 1];
      if (K >= 2) {
        if (K == 2) hist[0] = xv;
        else if (K == 3) hist[1] = xv;
        else hist[2] = xv;
      }
    }
    if (MAXR == 1) {  // decode advances the conv state by one row
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) st(ring, (size_t)j * C + c, hist[j]);
    }
  }
  for (int e = tid; e < nrows * G; e += NT) {
    const int r = e / G, ss = e - r * G;
    s_a[r][ss] = p.a[(size_t)(r0 + r) * Hv + g * G + ss];
    s_b[r][ss] = p.b[(size_t)(r0 + r) * Hv + g * G + ss];
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
      const float iq = 1.0f / sqrtf(sq + p.l2_eps), ik = 1.0f / sqrtf(sk + p.l2_eps);
      for (int c = lane; c < D; c += kWave) {
        s_qkv[r][c] *= iq;
        s_qkv[r][D + c] *= ik;
      }
      if (lane == 0) s_qk[r] = dqk * iq * ik;
    }
  }
  __syncthreads();

  // ---- the recurrence, row by row --------------------------------------------
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

    float *dst;
    if (MAXR == 1) dst = p.states[i];
    else dst = (r < nrows - 1) ? p.states[(r + 1) * kTableSeqs + i] : p.states[i];
    dst += (size_t)h * D * D;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int row = rr * RG + rg;
      const float kk = kh[row];
      float4 nv;
      nv.x = av * st_reg[rr].x + kk * u.x; nv.y = av * st_reg[rr].y + kk * u.y;
      nv.z = av * st_reg[rr].z + kk * u.z; nv.w = av * st_reg[rr].w + kk * u.w;
      st_reg[rr] = nv;
      *reinterpret_cast<float4 *>(dst + (size_t)row * D + 4 * cq) = nv;
    }

    if (rg == 0) {  // lanes 0..CQ-1 of the slot's first wave hold the head's outputs
      const float qk = s_qk[r];
      float o[4];
      o[0] = p.scale * (av * sq.x + qk * u.x); o[1] = p.scale * (av * sq.y + qk * u.y);
      o[2] = p.scale * (av * sq.z + qk * u.z); o[3] = p.scale * (av * sq.w + qk * u.w);
      const size_t obase = (size_t)(r0 + r) * Hv * D + (size_t)h * D + 4 * cq;
      if (p.z != nullptr) {
        float ss2 = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
        ss2 = sum_within_span<CQ>(ss2);
        const float inv = 1.0f / sqrtf(ss2 / D + p.norm_eps);
        const TA *zp = static_cast<const TA *>(p.z);
        const TA *nw = static_cast<const TA *>(p.norm_w);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = o[e] * inv * ld(nw, 4 * cq + e) * silu(ld(zp, obase + e));
      }
      TO *out = static_cast<TO *>(p.out);
#pragma unroll
      for (int e = 0; e < 4; ++e) st(out, obase + e, o[e]);
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
    const float4 *src = reinterpret_cast<const float4 *>(p.tables[na * kTableSeqs + i]);
    float4 *dst = reinterpret_cast<float4 *>(p.tables[i]);
    const int64_t per = (n4 + kCommitSplit - 1) / kCommitSplit;
    const int64_t beg = (int64_t)blockIdx.y * per, end = min(n4, beg + per);
    for (int64_t i0 = beg + threadIdx.x; i0 < end; i0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t idx = i0 + (int64_t)u * 256;
        if (idx < end) v[u] = src[idx];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t idx = i0 + (int64_t)u * 256;
        if (idx < end) dst[idx] = v[u];
      }
    }
  } else {
    const int C = p.geo.conv_dim, R = p.geo.K - 1;
    const int c = ((int)blockIdx.y - kCommitSplit) * 256 + threadIdx.x;
    if (c >= C) return;
    TE *ring = static_cast<TE *>(p.conv_state[i]);
    const TE *x = static_cast<const TE *>(p.x) + (size_t)p.cu[i] * C;
    TE vals[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      if (r < R) {
        const int idx = na + r;  // position in [old conv state ; accepted rows]
        vals[r] = (idx < R) ? ring[(size_t)idx * C + c] : x[(size_t)(idx - R) * C + c];
      }
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
