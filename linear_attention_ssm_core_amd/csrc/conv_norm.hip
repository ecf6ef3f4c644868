// Prefill front and back of the mixer core:
//  * causal depthwise conv1d + SiLU over packed [Q|K|V] rows, then L2 norm of
//    every q and k head (conv1d_prefill_k, conv1d_l2norm_k, l2_norm_k on the
//    metrale_model_layers/layers/qwen3_ssm/layer_struct.rs page), and the
//    advance of each sequence's conv state;
//  * Z-gated RMSNorm per (token, value head) (gated_rms_norm_k,
//    gated_rms_norm_prefill_k, same page), gate SiLU(z) or, for a model of the
//    gdn_norm_sigmoid kind, sigmoid(z).
//
// Both are streaming, HBM-bound kernels with 16-byte accesses.  The conv state is
// advanced by a second small kernel, ordered after the first on the stream,
// because the rows that read the old state may belong to a different workgroup
// than the one that would write the new state.
#include "common.h"
#include "internal.h"

namespace gdn {
namespace {

// Packed rows per thread: every row load of a thread is issued at once (kept raw
// until used).  Short blocks (8 rows plus 3 history rows, re-read from L2 by the
// neighbouring block) and up to four waves per SIMD let the loads, the arithmetic
// and the stores of different workgroups overlap; measured faster than 16 or 32
// rows per thread at two waves per SIMD.
template <typename TA>
constexpr int conv_rows() { return 8; }

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
// Rows read exactly once (the gated norm's pre-norm input): fp32 rows -- the fused
// prefill's staged outputs -- with the non-temporal hint (the norm of 64,831 staged
// rows 356 -> 331 us on one MI355X); bf16 rows as load8.
__device__ __forceinline__ void load8_once(const bf16 *p, float v[8]) { load8(p, v); }
__device__ __forceinline__ void load8_once(const float *p, float v[8]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 a = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
  const f4 b = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p) + 1);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3]; v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
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
// raw 8-channel words, widened when used
template <typename TA>
struct Raw8;
template <>
struct Raw8<bf16> {
  uint4 w;
  __device__ __forceinline__ void load(const bf16 *p) { w = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void get(float v[8]) const {
    const bf16x8 r = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)r[e];
  }
};
template <>
struct Raw8<float> {
  uint4 w0, w1;
  __device__ __forceinline__ void load(const float *p) {
    w0 = reinterpret_cast<const uint4 *>(p)[0];
    w1 = reinterpret_cast<const uint4 *>(p)[1];
  }
  __device__ __forceinline__ void get(float v[8]) const {
    const float4 a = __builtin_bit_cast(float4, w0), b = __builtin_bit_cast(float4, w1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Each thread owns 8 consecutive channels of conv_rows<TA>() consecutive packed
// rows; every input row is read once with 16-byte loads (plus 3 history rows per
// workgroup); a q or k head (d channels) is d/8 consecutive lanes, which reduce
// its squared norm with shuffles.
template <int D, int K, typename TA, typename TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void conv_l2norm_kernel(ConvLaunch p) {
  constexpr int TPH = D / 8;  // lanes per head
  constexpr int R = conv_rows<TA>();
  const int C = p.geo.conv_dim, Hk = p.geo.Hk;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  const bool active = c0 < C;  // uniform per head (C is a multiple of d)
  const int cc = active ? c0 : 0;
  const bool normalise = cc < 2 * Hk * D;
  const TA *x = static_cast<const TA *>(p.x);
  const TA *w = static_cast<const TA *>(p.conv_w);
  TY *y = static_cast<TY *>(p.y);

  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int64_t t1 = min((int64_t)p.T, t0 + R);
  // sequence of row t0 (invariant cu[lo] <= t0 < cu[hi])
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

  // The thread's 8 K taps are 8 K contiguous values: K 16-byte words (bf16).  They
  // are loaded after the rows (the rows' latency is the one that matters) and
  // aligned to rows t-3 .. t: ws[jj] multiplies row t - 3 + jj, zero for the 4 - K
  // rows before the window.
  Raw8<TA> wr[K];
  auto load_w = [&]() {
#pragma unroll
    for (int q = 0; q < K; ++q) wr[q].load(w + (size_t)cc * K + 8 * q);
  };
  float ws[4][8];
  auto unpack_w = [&]() {
    float wv[K][8];
#pragma unroll
    for (int q = 0; q < K; ++q) wr[q].get(wv[q]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = jj - (4 - K), idx = e * K + (j < 0 ? 0 : j);
        ws[jj][e] = (j >= 0) ? wv[idx / 8][idx % 8] : 0.0f;
      }
  };

  // conv + SiLU + L2 norm of row t from rows t-3 .. t (r[3] is row t)
  auto emit = [&](int64_t t, const float (&r)[4][8]) {
    float yv[8];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc += ws[jj][e] * r[jj][e];
      yv[e] = silu(acc);
      ss += yv[e] * yv[e];
    }
    if (normalise) {
      ss = sum_lanes<TPH>(ss);
      const float inv = rsqrt_hw(ss + p.l2_eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] *= inv;
    }
    if (active) store8(y + (size_t)t * C + cc, yv);
  };

  if (t1 - t0 == R && t0 - 3 >= seq_start && t1 <= seq_end) {
    // Fast path: the block and its 3 predecessors lie in one sequence.  Every load
    // is issued first (raw), then the rows are walked with no branch.
    Raw8<TA> xr[R + 3];  // rows t0 - 3 .. t1 - 1
#pragma unroll
    for (int u = 0; u < R + 3; ++u) xr[u].load(x + (size_t)(t0 - 3 + u) * C + cc);
    load_w();
    unpack_w();
    // sliding window of widened rows: each raw row is widened once
    float r[4][8];
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) xr[jj].get(r[jj]);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      xr[u + 3].get(r[3]);
      emit(t0 + u, r);
#pragma unroll
      for (int jj = 0; jj < 3; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) r[jj][e] = r[jj + 1][e];
    }
    return;
  }

  // General path (blocks at sequence starts, the ragged tail): row by row, with
  // rows t-3 .. t-1 of the current sequence in registers (from the conv state
  // before the sequence's first row; zero where no tap reaches).
  load_w();
  unpack_w();
  float r[4][8];
  auto load_win = [&](int64_t t) {
    // (through the global address space, so that its loads are not FLAT)
    const TA *ring = (const TA *)to_global(static_cast<const TA *>(p.conv_state[seq]));
    const int64_t tau = t - seq_start;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int64_t rel = tau - 3 + jj;
      if (rel >= 0) load8(x + (size_t)(seq_start + rel) * C + cc, r[jj]);
      else if (K - 1 + rel >= 0) load8(ring + (size_t)(K - 1 + rel) * C + cc, r[jj]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) r[jj][e] = 0.0f;
    }
  };
  load_win(t0);
#pragma unroll 1
  for (int64_t t = t0; t < t1; ++t) {
    while (t >= seq_end) {  // a new sequence starts at t (skip empty ones)
      ++seq;
      seq_start = p.cu[seq];
      seq_end = p.cu[seq + 1];
      if (t == seq_start && t < seq_end) load_win(t);
    }
    load8(x + (size_t)t * C + cc, r[3]);
    emit(t, r);
#pragma unroll
    for (int jj = 0; jj < 3; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) r[jj][e] = r[jj + 1][e];
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
  load8_once(o + (size_t)r * D + c0, ov);
  load8(z + (size_t)r * D + c0, zv);
  load8(nw + c0, wv);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += ov[e] * ov[e];
  ss = sum_lanes<TPR>(ss);
  const float inv = rsqrt_hw(ss / D + p.eps);
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    res[e] = ov[e] * inv * wv[e] * (p.norm_sigmoid ? __builtin_amdgcn_rcpf(1.0f + __expf(-zv[e])) : silu(zv[e]));
  if (active) store8(out + (size_t)r * D + c0, res);
}

template <int D, typename TA>
hipError_t conv_launch_y(const ConvLaunch &p, hipStream_t stream) {
  constexpr int R = conv_rows<TA>();
  const dim3 grid((unsigned)((p.T + R - 1) / R), (p.geo.conv_dim / 8 + 255) / 256), block(256);
  const bool y_bf16 = !p.y_f32 && p.geo.out_bf16;
  // the conv width is a template parameter: the taps are then whole 16-byte words
  // with compile-time positions
  switch (p.geo.K) {
    case 2:
      if (y_bf16) hipLaunchKernelGGL((conv_l2norm_kernel<D, 2, TA, bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((conv_l2norm_kernel<D, 2, TA, float>), grid, block, 0, stream, p);
      break;
    case 3:
      if (y_bf16) hipLaunchKernelGGL((conv_l2norm_kernel<D, 3, TA, bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((conv_l2norm_kernel<D, 3, TA, float>), grid, block, 0, stream, p);
      break;
    default:
      if (y_bf16) hipLaunchKernelGGL((conv_l2norm_kernel<D, 4, TA, bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((conv_l2norm_kernel<D, 4, TA, float>), grid, block, 0, stream, p);
      break;
  }
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
