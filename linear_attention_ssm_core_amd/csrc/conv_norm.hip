// Prefill front and back of the mixer core:
//  * causal depthwise conv1d + SiLU over packed [Q|K|V] rows, then L2 norm of
//    every q and k head (conv1d_prefill_k, conv1d_l2norm_k, l2_norm_k on the
//    metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page), and the
//    advance of each sequence's conv state;
//  * Z-gated RMSNorm per (token, value head) (gated_rms_norm_k,
//    gated_rms_norm_prefill_k, same page).
//
// Both are streaming, HBM-bound kernels.  Conv: a workgroup owns 64 packed rows
// of one head block (d channels); a wave produces one row of the block at a time
// with consecutive lanes on consecutive channels (coalesced), so the L2 norm is a
// single wave reduction.  The K-1 history rows are re-read through L1/L2.  The
// conv state is advanced by a second small kernel, ordered after the first on the
// stream, because the rows that read the old state may belong to a different
// workgroup than the one that would write the new state.
#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kConvRows = 64;

template <int D, typename TA, typename TY>
__global__ __launch_bounds__(256) void conv_l2norm_kernel(ConvLaunch p) {
  constexpr int PER = (D + kWave - 1) / kWave;
  const int hb = blockIdx.y;
  const int Hk = p.geo.Hk, C = p.geo.conv_dim, K = p.geo.K;
  const bool normalise = hb < 2 * Hk;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  TY *y = static_cast<TY *>(p.y);

  float wt[PER][4];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int cc = lane + kWave * m;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wt[m][j] = (cc < D && j < K) ? ld(w, (size_t)(hb * D + cc) * K + j) : 0.0f;
  }

  const int64_t t0 = (int64_t)blockIdx.x * kConvRows;
  for (int tt = wave; tt < kConvRows; tt += 4) {
    const int64_t t = t0 + tt;
    if (t >= p.T) break;
    int lo = 0, hi = p.n;  // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int64_t tau = t - p.cu[lo];
    const TA *ring = static_cast<const TA *>(p.conv_state[lo]);
    float yv[PER];
    float ss = 0.0f;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int cc = lane + kWave * m;
      yv[m] = 0.0f;
      if (cc < D) {
        const int c = hb * D + cc;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < K) {
            const int64_t rel = tau - (K - 1) + j;  // row of the sequence; < 0: history
            const float xv = (rel >= 0) ? ld(x, (size_t)(t - tau + rel) * C + c)
                                        : ld(ring, (size_t)(K - 1 + rel) * C + c);
            acc += wt[m][j] * xv;
          }
        }
        yv[m] = silu(acc);
        ss += yv[m] * yv[m];
      }
    }
    if (normalise) {
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss + p.l2_eps);
#pragma unroll
      for (int m = 0; m < PER; ++m) yv[m] *= inv;
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int cc = lane + kWave * m;
      if (cc < D) st(y, (size_t)t * C + hb * D + cc, yv[m]);
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

template <int D, int PER_LANE, typename TI, typename TA, typename TO>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormLaunch p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;  // (token, head)
  if (row >= p.T * p.Hv) return;  // whole wave leaves together
  const int lane = threadIdx.x % kWave;
  const TI *o = static_cast<const TI *>(p.o);
  const TA *z = static_cast<const TA *>(p.z);
  const TA *nw = static_cast<const TA *>(p.norm_w);
  TO *out = static_cast<TO *>(p.out);
  float ov[PER_LANE];
  float ss = 0.0f;
#pragma unroll
  for (int m = 0; m < PER_LANE; ++m) {
    const int cc = lane + kWave * m;
    ov[m] = (cc < D) ? ld(o, (size_t)row * D + cc) : 0.0f;
    ss += ov[m] * ov[m];
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / D + p.eps);
#pragma unroll
  for (int m = 0; m < PER_LANE; ++m) {
    const int cc = lane + kWave * m;
    if (cc < D) st(out, (size_t)row * D + cc, ov[m] * inv * ld(nw, cc) * silu(ld(z, (size_t)row * D + cc)));
  }
}

template <int D, typename TA>
hipError_t conv_launch_y(const ConvLaunch &p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.T + kConvRows - 1) / kConvRows), p.geo.conv_dim / D), block(256);
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
  constexpr int PER = (D + kWave - 1) / kWave;
  const dim3 grid((unsigned)((p.T * p.Hv + 3) / 4)), block(256);
  if (p.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, PER, TI, TA, bf16>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, PER, TI, TA, float>), grid, block, 0, stream, p);
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
