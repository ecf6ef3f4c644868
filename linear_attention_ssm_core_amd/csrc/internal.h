// Host-side launch interface between the ABI layer (api.cpp) and the kernel
// translation units.  Arguments arrive validated; every launcher enqueues on
// `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Shape and dtype selection shared by all launchers.
struct Geometry {
  int Hk, Hv, D, K;     // key heads, value heads, head dim (d_k == d_v), conv taps
  int conv_dim;         // 2*Hk*D + Hv*D
  int act_bf16;         // activation dtype is bf16 (else fp32)
  int out_bf16;         // output dtype is bf16 (else fp32)
};

// One-token decode (rows == sequences) and k-row verify share one kernel family.
struct RecurrentLaunch {
  Geometry geo;
  int n;                        // sequences
  int verify;                   // 0: decode, 1: verify
  const int32_t *cu;            // verify row offsets [n+1] (device), unused for decode
  const void *x, *conv_w;
  void *const *conv_state;
  const float *a, *b;
  float *const *states;         // decode: [n] state pointers; verify: [16][128] tables
  const void *z, *norm_w;
  void *out;
  float scale, l2_eps, norm_eps;
};
hipError_t launch_recurrent(const RecurrentLaunch &p, hipStream_t stream);

struct CommitLaunch {
  Geometry geo;
  int n;
  const int32_t *cu, *n_accepted;
  float *const *tables;
  const void *x;
  void *const *conv_state;
};
hipError_t launch_commit(const CommitLaunch &p, hipStream_t stream);

struct ConvLaunch {
  Geometry geo;
  int n;
  int64_t T;
  const int32_t *cu;
  const void *x, *conv_w;
  void *const *conv_state;
  void *y;
  int y_f32;                    // overrides geo.out_bf16 for y (front of the prefill)
  float l2_eps;
};
hipError_t launch_conv_l2norm(const ConvLaunch &p, hipStream_t stream);

struct NormLaunch {
  int Hv, D;
  int64_t T;
  int in_bf16, act_bf16, out_bf16;
  const void *o, *z, *norm_w;
  void *out;
  float eps;
};
hipError_t launch_gated_rmsnorm(const NormLaunch &p, hipStream_t stream);

struct PrefillLaunch {
  Geometry geo;
  int n;
  int64_t T;
  const int32_t *cu;
  const void *y;                // [T][conv_dim] q_hat|k_hat|v
  int y_bf16;                   // dtype of y
  const float *a, *b;
  float *const *h_state;
  void *o;                      // [T][Hv*D] written by the chunk kernels
  int o_f32;                    // o is fp32 (else geo.out_bf16 decides)
  float scale;
  void *workspace;              // prefill workspace (chunk tables and per-chunk operands)
};
// Bytes of workspace the chunk kernels need for n sequences and T tokens.
size_t prefill_core_workspace(const Geometry &geo, int n, int64_t T);
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);

}  // namespace gdn
