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

// The token-recurrent forms share one kernel family.
enum RecurrentMode {
  kModeDecode = 0,   // one token per sequence: state and conv state advance in place
  kModeTokens = 1,   // up to 17 tokens per sequence, state written once at the end
  kModeVerify = 2,   // k rows, the state after every row stored through the WY tables
  kModeWoa = 3       // k rows, no state stored; (k_hat, u, a) of every row stashed
};

struct RecurrentLaunch {
  Geometry geo;
  int n;                        // sequences
  int mode;                     // RecurrentMode
  int state_f16;                // states are binary16 (else fp32)
  int gates_raw;                // a, b hold g and beta
  int norm_sigmoid;             // the norm gate is sigmoid(z) (else SiLU(z))
  const int32_t *cu;            // row offsets [n+1] (device), unused for decode
  const void *x, *conv_w;
  void *const *conv_state;
  const float *a, *b;
  void *const *states;          // decode/tokens/woa: [n] state pointers; verify: [16][128] tables
  const void *z, *norm_w;
  void *out;
  float *stash;                 // woa: [rows][stash_row] floats
  int stash_row;                // floats per stash row
  float scale, l2_eps, norm_eps;
};
hipError_t launch_recurrent(const RecurrentLaunch &p, hipStream_t stream);

struct CommitLaunch {
  Geometry geo;
  int n;
  int state_f16;
  const int32_t *cu, *n_accepted;
  void *const *tables;
  const void *x;
  void *const *conv_state;
};
hipError_t launch_commit(const CommitLaunch &p, hipStream_t stream);

// Fold of the accepted rows of a write-on-accept verify.
struct FoldLaunch {
  Geometry geo;
  int n;
  int state_f16;
  const int32_t *cu, *n_accepted;
  void *const *states;          // [n] state pointers
  const float *stash;
  int stash_row;
  const void *x;
  void *const *conv_state;
};
hipError_t launch_fold(const FoldLaunch &p, hipStream_t stream);

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
  int norm_sigmoid;             // gate sigmoid(z) (else SiLU(z))
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
  int gates_raw;                // a, b hold g and beta
  void *const *h_state;
  int state_f16;                // states are binary16 (else fp32)
  void *o;                      // [T][Hv*D] written by the chunk kernels
  int o_f32;                    // o is fp32 (else geo.out_bf16 decides)
  float scale;
  void *workspace;              // prefill workspace (chunk tables and per-chunk operands)
};
// Bytes of workspace the chunk kernels need for n sequences and T tokens.
size_t prefill_core_workspace(const Geometry &geo, int n, int64_t T, bool y_bf16);
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);

// Scratch of the allocation-free prefill: a device array of this many bytes per
// GPU, defined in prefill.hip.  prefill_scratch() returns its device address on
// the current device (looked up once per device; no allocation).
constexpr size_t kPrefillScratchBytes = size_t(64) << 20;
hipError_t prefill_scratch(void **ptr);

}  // namespace gdn
