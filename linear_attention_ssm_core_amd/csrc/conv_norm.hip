// Prefill front and back of the mixer core:
//  * causal depthwise conv1d + SiLU over packed [Q|K|V] rows, then L2 norm of
//    every q and k head (conv1d_prefill_k, conv1d_l2norm_k, l2_norm_k on the
//    metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page), and the
//    advance of each sequence's conv state;
//  * Z-gated RMSNorm per (token, value head) (gated_rms_norm_k,
//    gated_rms_norm_prefill_k, same page).
//
// Both are streaming, HBM-bound kernels with 16-byte accesses.  The conv state is
// advanced by a second small kernel, ordered after the first on the stream,
// because the rows that read the old state may belong to a different workgroup
// than the one that would write the new state.
#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kConvRows = 32;   // packed rows per workgroup
constexpr int kConvGroup = 8;   // rows whose loads are issued together

// Eight consecutive channels of one row, widened to fp32.
__device__ __forceinline__ void load8(const bf16 *p, float v[8]) {
  const bf16x8 r = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)r[e];
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16 *p, const float v[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8 *>(p) = r;
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Each thread owns 8 consecutive channels and walks kConvRows packed rows in order
// with the K-1 previous rows of its channels in registers, so every input row is
// read once with 16-byte (bf16) loads; a q or k head (d channels) is d/8
// consecutive lanes, which reduce its squared norm with shuffles.
template <int D, typename TA, typename TY>
__global__ __launch_bounds__(256) void conv_l2norm_kernel(ConvLaunch p) {
  constexpr int TPH = D / 8;  // lanes per head
  const int C = p.geo.conv_dim, K = p.geo.K, Hk = p.geo.Hk;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  const bool active = c0 < C;  // uniform per head (C is a multiple of d)
  const int cc = active ? c0 : 0;
  const bool normalise = cc < 2 * Hk * D;
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  TY *y = static_cast<TY *>(p.y);

  float wt[4][8];  // tap j of channel cc + e
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[j][e] = (j < K) ? ld(w, (size_t)(cc + e) * K + j) : 0.0f;

  const int64_t t0 = (int64_t)blockIdx.x * kConvRows;
  const int64_t t1 = min((int64_t)p.T, t0 + kConvRows);
  // sequence of row t0 (invariant cu[lo] <= t0 < cu[hi]), then walk forward
  int seq;
  {
    int lo = 0, hi = p.n;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu[mid] <= t0) lo = mid;
      else hi = mid;
    }
    seq = lo;
  }
  int seq_start = p.cu[seq], seq_end = p.cu[seq + 1];
  // history window: hist[j] = row t-(K-1)+j of the current sequence
  float hist[3][8];
  auto load_hist = [&](int64_t t) {
    const TA *ring = static_cast<const TA *>(p.conv_state[seq]);
    const int64_t tau = t - seq_start;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j < K - 1) {
        const int64_t rel = tau - (K - 1) + j;
        if (rel >= 0) load8(x + (size_t)(seq_start + rel) * C + cc, hist[j]);
        else load8(ring + (size_t)(K - 1 + rel) * C + cc, hist[j]);
      }
    }
  };
  load_hist(t0);
  for (int64_t tg = t0; tg < t1; tg += kConvGroup) {
    float xr[kConvGroup][8];
#pragma unroll
    for (int u = 0; u < kConvGroup; ++u) {
      const int64_t t = min(tg + u, t1 - 1);
      load8(x + (size_t)t * C + cc, xr[u]);
    }
#pragma unroll
    for (int u = 0; u < kConvGroup; ++u) {
      const int64_t t = tg + u;
      if (t >= t1) break;
      while (t >= seq_end) {  // a new sequence starts at t (skip empty ones)
        ++seq;
        seq_start = p.cu[seq];
        seq_end = p.cu[seq + 1];
        if (t == seq_start && t < seq_end) load_hist(t);
      }
      float yv[8];
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < K - 1) acc += wt[j][e] * hist[j][e];
        acc += (K == 2 ? wt[1][e] : K == 3 ? wt[2][e] : wt[3][e]) * xr[u][e];
        yv[e] = silu(acc);
        ss += yv[e] * yv[e];
      }
      if (normalise) {
#pragma unroll
        for (int off = 1; off < TPH; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = 1.0f / sqrtf(ss + p.l2_eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) yv[e] *= inv;
      }
      if (active) store8(y + (size_t)t * C + cc, yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (K == 4) { hist[0][e] = hist[1][e]; hist[1][e] = hist[2][e]; hist[2][e] = xr[u][e]; }
        else if (K == 3) { hist[0][e] = hist[1][e]; hist[1][e] = xr[u][e]; }
        else { hist[0][e] = xr[u][e]; }
      }
    }
  }
}

// New conv state of sequence s: the last K-1 rows of [old state ; its rows].
template <typename TE>
__global__ __launch_bounds__(256) void conv_state_advance_kernel(ConvLaunch p) {
  const int s = blockIdx.y;
  const int C = p.geo.conv_dim, R = p.geo.K - 1;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int len = p.cu[s + 1] - p.cu[s];
  if (len <= 0) return;
  TE *ring = static_cast<TE *>(p.conv_state[s]);
  const TE *x = static_cast<const TE *>(p.x) + (size_t)p.cu[s] * C;
  TE vals[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    if (r < R) {
      const int idx = len + r;
      vals[r] = (idx < R) ? ring[(size_t)idx * C + c] : x[(size_t)(idx - R) * C + c];
    }
  }
#pragma unroll
  for (int r = 0; r < 3; ++r)
    if (r < R) ring[(size_t)r * C + c] = vals[r];
}

// One (token, value head) row of d values is d/8 consecutive lanes, 8 values each
// (16-byte bf16 accesses); the mean square is reduced with shuffles.
template <int D, typename TI, typename TA, typename TO>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormLaunch p) {
  constexpr int TPR = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int c0 = (threadIdx.x % TPR) * 8;
  const bool active = row < p.T * p.Hv;
  const int64_t r = active ? row : 0;
  const TI *o = static_cast<const TI *>(p.o);
  const TA *z = static_cast<const TA *>(p.z);
  const TA *nw = static_cast<const TA *>(p.norm_w);
  TO *out = static_cast<TO *>(p.out);
  float ov[8], zv[8], wv[8];
  load8(o + (size_t)r * D + c0, ov);
  load8(z + (size_t)r * D + c0, zv);
  load8(nw + c0, wv);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += ov[e] * ov[e];
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / D + p.eps);
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) res[e] = ov[e] * inv * wv[e] * silu(zv[e]);
  if (active) store8(out + (size_t)r * D + c0, res);
}

template <int D, typename TA>
hipError_t conv_launch_y(const ConvLaunch &p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.T + kConvRows - 1) / kConvRows), (p.geo.conv_dim / 8 + 255) / 256), block(256);
  const bool y_bf16 = !p.y_f32 && p.geo.out_bf16;
  if (y_bf16) hipLaunchKernelGGL((conv_l2norm_kernel<D, TA, bf16>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((conv_l2norm_kernel<D, TA, float>), grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((p.geo.conv_dim + 255) / 256, p.n);
  if (p.geo.act_bf16) hipLaunchKernelGGL((conv_state_advance_kernel<uint16_t>), grid2, block, 0, stream, p);
  else hipLaunchKernelGGL((conv_state_advance_kernel<float>), grid2, block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t conv_launch_a(const ConvLaunch &p, hipStream_t stream) {
  return p.geo.act_bf16 ? conv_launch_y<D, bf16>(p, stream) : conv_launch_y<D, float>(p, stream);
}

template <int D, typename TI, typename TA>
hipError_t norm_launch_o(const NormLaunch &p, hipStream_t stream) {
  const int64_t threads = p.T * p.Hv * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (p.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, TI, TA, bf16>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, TI, TA, float>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, typename TI>
hipError_t norm_launch_a(const NormLaunch &p, hipStream_t stream) {
  return p.act_bf16 ? norm_launch_o<D, TI, bf16>(p, stream) : norm_launch_o<D, TI, float>(p, stream);
}

template <int D>
hipError_t norm_launch_i(const NormLaunch &p, hipStream_t stream) {
  return p.in_bf16 ? norm_launch_a<D, bf16>(p, stream) : norm_launch_a<D, float>(p, stream);
}

}  // namespace

hipError_t launch_conv_l2norm(const ConvLaunch &p, hipStream_t stream) {
  if (p.T == 0 || p.n == 0) return hipSuccess;
  switch (p.geo.D) {
    case 32: return conv_launch_a<32>(p, stream);
    case 64: return conv_launch_a<64>(p, stream);
    case 128: return conv_launch_a<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gated_rmsnorm(const NormLaunch &p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  switch (p.D) {
    case 32: return norm_launch_i<32>(p, stream);
    case 64: return norm_launch_i<64>(p, stream);
    case 128: return norm_launch_i<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
