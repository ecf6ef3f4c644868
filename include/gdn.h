/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet mixer core.
 *
 * The library computes the GDN mixer core of a Qwen3-style SSM layer:
 *   1. causal depthwise conv1d + SiLU over the packed [Q | K | V] projection rows
 *      and L2 normalisation of every q and k head     -> gdn_conv_l2norm
 *   2. the gated delta rule
 *          S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = scale * S_t q_t
 *      (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025, section 3) in
 *      three forms:
 *        - chunked WY/UT-form prefill over packed variable-length sequences
 *                                                      -> gdn_prefill_chunked
 *        - one token for each of many sequences      -> gdn_decode_batched
 *        - k draft rows per sequence that records every intermediate state through
 *          the WY pointer tables, and the commit of the accepted prefix
 *                                                      -> gdn_verify_multi, gdn_verify_commit
 *   3. Z-gated RMSNorm  out = o / sqrt(mean(o^2) + eps) * w * SiLU(z)
 *                                                      -> gdn_gated_rmsnorm
 *
 * Where each operation is defined on the source pages (rustdoc source views of the
 * metrale_model_layers crate):
 *   - conv1d / L2 / gated-norm / recurrence kernel families and the [Q | K | V | Z]
 *     row order: struct Qwen3SsmLayer and its doc comments, page
 *     metrale_model_layers/layers/qwen3_ssm/layer_struct.rs (handles conv1d_k,
 *     conv1d_l2norm_f32_strided_k, l2_norm_k, gdn_f32_strided_norm_k,
 *     gated_rms_norm_f32_strided_k, gated_rms_norm_prefill_k, the
 *     gdn_prefill_fla_* chunked-prefill handles, gdn_wyn_table_k; the per-sequence
 *     state sizes h_state_bytes / conv_state_bytes).
 *   - per-sequence state pointer arrays and the varlen descriptor: the
 *     prefill_gdn_full_batched_fla_varlen entry of LayerSplitPrefill, page
 *     metrale_model_layers/layers/qwen3_ssm/trait_layer.rs.
 *   - the verify pointer tables and their limits: constants VERIFY_WY_TABLE_SEQS,
 *     VERIFY_WY_TABLES_PER_LAYER and the two stride constants, page
 *     metrale_model_layers/layer/transformer_layer.rs; the verify entry
 *     decode_verify_multi on that page; gdn_fold_accepted on the trait_layer.rs page.
 *
 * Conventions for every entry point
 *   - Every pointer in an argument struct is a DEVICE pointer unless its comment
 *     says "host".  The caller owns all memory; the library allocates nothing.
 *   - Work is enqueued on the caller's hipStream_t (NULL = default stream); no
 *     call synchronises the host with the device.
 *   - Shapes: H_k key heads, H_v value heads (a multiple of H_k), d_k = d_v = d,
 *     conv_dim = 2*H_k*d_k + H_v*d_v.  Value head h reads key head h / (H_v/H_k).
 *   - Activation rows are packed [q (H_k*d_k) | k (H_k*d_k) | v (H_v*d_v)],
 *     head-major inside each block, row stride conv_dim elements.
 *   - The recurrent state of a sequence is fp32 h[H_v][d_k][d_v] = S^T per value
 *     head (d_v fastest), reached through a device array of per-sequence pointers.
 *     The conv state of a sequence is its last (K-1) raw pre-conv rows, oldest
 *     first, [K-1][conv_dim] in the activation dtype, also through a pointer array.
 *   - a, b are fp32 [rows][H_v]; z is [rows][H_v*d_v]; norm_w is [d_v], shared by
 *     all heads; z and norm_w use the activation dtype.
 *   - Errors: any status other than GDN_OK except GDN_ERR_HIP means nothing was
 *     launched.  GDN_ERR_HIP reports a launch failure (hipGetLastError).
 *   - Calls on one stream are ordered; state buffers must not be shared by calls
 *     running concurrently on different streams.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

/* Batched-verify pointer-table layout: per layer, 16 tables of 128 u64 entries
 * back to back.  Table 0 holds each sequence's state, table t+1 its state after
 * draft row t.  (transformer_layer.rs page, the VERIFY_WY_* constants.) */
#define GDN_VERIFY_WY_TABLE_SEQS 128
#define GDN_VERIFY_WY_TABLES_PER_LAYER 16
#define GDN_VERIFY_WY_TABLE_STRIDE_BYTES 1024  /* GDN_VERIFY_WY_TABLE_SEQS * 8 */
#define GDN_VERIFY_WY_LAYER_STRIDE_BYTES 16384 /* 16 tables * 1024 bytes */
#define GDN_VERIFY_MIN_K 2
#define GDN_VERIFY_MAX_K 16

/* Chunk length of the chunked prefill (tokens). */
#define GDN_PREFILL_CHUNK 64

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* NULL required pointer, bad sizes, struct_size mismatch   */
  GDN_ERR_UNSUPPORTED = 2, /* valid shape with no kernel (d not in {32,64,128}, ...)   */
  GDN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required              */
  GDN_ERR_HIP = 4          /* the HIP runtime reported a launch error                 */
} gdn_status;

typedef enum gdn_dtype {
  GDN_DTYPE_F32 = 0,
  GDN_DTYPE_BF16 = 1
} gdn_dtype;

/* Head geometry.  Supported: d_k == d_v in {32, 64, 128}; H_v / H_k in {1, 2, 4};
 * conv_kernel (taps K) in {2, 3, 4}. */
typedef struct gdn_dims {
  int32_t num_k_heads; /* H_k */
  int32_t num_v_heads; /* H_v */
  int32_t head_dim_k;  /* d_k */
  int32_t head_dim_v;  /* d_v */
  int32_t conv_kernel; /* K   */
  int32_t reserved;    /* must be 0 */
} gdn_dims;

/* ---------------------------------------------------------------------------
 * gdn_conv_l2norm -- causal depthwise conv1d + SiLU, then L2 norm of q and k.
 *   y[t][c] = SiLU(sum_{j<K} conv_w[c][j] * x[t-K+1+j][c]); rows before a
 *   sequence's first row come from its conv state; no bias.  Every q and k head
 *   is then divided by sqrt(sum of squares + l2_eps); v is not normalised.
 *   Each sequence's conv state is replaced by the last K-1 rows of
 *   [old conv state ; its x rows] (unchanged for a zero-length sequence).
 *   Defined by: conv1d_prefill_k, conv1d_l2norm_k, l2_norm_k (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_conv_args {
  uint32_t struct_size;        /* sizeof(gdn_conv_args)                         */
  int32_t act_dtype;           /* dtype of x, conv_w, conv states               */
  int32_t out_dtype;           /* dtype of y                                    */
  gdn_dims dims;
  int32_t num_seqs;            /* n >= 0                                        */
  int64_t total_tokens;        /* T = cu_seqlens[n] (host value)                */
  const int32_t *cu_seqlens;   /* [n+1] non-decreasing, cu[0] = 0               */
  const void *x;               /* [T][conv_dim]                                 */
  const void *conv_w;          /* [conv_dim][K]; tap K-1 multiplies row t        */
  void *const *conv_state;     /* [n] pointers to [K-1][conv_dim], in/out        */
  void *y;                     /* [T][conv_dim] out = [q_hat | k_hat | v]; must
                                  not alias x                                   */
  float l2_eps;                /* >= 0, typically 1e-6                          */
} gdn_conv_args;

gdn_status gdn_conv_l2norm(const gdn_conv_args *args, void *stream /* hipStream_t */);

/* ---------------------------------------------------------------------------
 * gdn_prefill_chunked -- chunked WY/UT-form gated delta rule over packed
 *   variable-length sequences (chunks of 64 tokens restart at every sequence;
 *   the last chunk may be partial).  Result equals the token-by-token rule.
 *   Input is either y = [q_hat | k_hat | v] (x == NULL), or, with x, conv_w and
 *   conv_state given, pre-conv rows x: the conv + SiLU + L2 front then runs
 *   inside the call and advances the conv states as gdn_conv_l2norm does.
 *   Each sequence's state is read from *h_state[i] and overwritten with the state
 *   after its last token (zero-length sequences keep their state).
 *   out = scale * o, or, when z != NULL, the Z-gated RMSNorm of scale * o.
 *   Defined by: the gdn_prefill_fla_recompute_wu_k / _chunk_delta_h_k /
 *   _chunk_fwd_o_k handles (layer_struct.rs) and
 *   prefill_gdn_full_batched_fla_varlen (trait_layer.rs).
 *   Needs a caller-owned workspace of gdn_prefill_workspace_bytes() bytes.
 * ------------------------------------------------------------------------- */
typedef struct gdn_prefill_args {
  uint32_t struct_size;        /* sizeof(gdn_prefill_args)                      */
  int32_t act_dtype;           /* dtype of y or x/conv_w/conv states, z, norm_w  */
  int32_t out_dtype;           /* dtype of out                                  */
  gdn_dims dims;
  int32_t num_seqs;            /* n >= 0                                        */
  int64_t total_tokens;        /* T = cu_seqlens[n] (host value)                */
  int32_t chunk_size;          /* must be GDN_PREFILL_CHUNK                      */
  int32_t reserved;            /* must be 0                                     */
  const int32_t *cu_seqlens;   /* [n+1]                                         */
  const void *y;               /* [T][conv_dim] (used when x == NULL)           */
  const void *x;               /* [T][conv_dim] pre-conv rows, or NULL          */
  const void *conv_w;          /* [conv_dim][K] (with x)                        */
  void *const *conv_state;     /* [n] pointers (with x), in/out                  */
  const float *a;              /* [T][H_v] decay a_t in [0, 1]                   */
  const float *b;              /* [T][H_v] write strength b_t                    */
  float *const *h_state;       /* [n] pointers to fp32 [H_v][d_k][d_v], in/out    */
  const void *z;               /* [T][H_v*d_v] or NULL                          */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [T][H_v*d_v]                                  */
  float scale;                 /* output scale (1.0 = the plain rule)           */
  float l2_eps;                /* front L2 epsilon (with x)                     */
  float norm_eps;              /* RMSNorm epsilon (with z)                      */
  float reserved_f;            /* must be 0                                     */
  void *workspace;             /* device scratch, >= required bytes             */
  size_t workspace_bytes;
} gdn_prefill_args;

/* Workspace bytes gdn_prefill_chunked needs for these arguments (pointers are not
 * read).  Writes *bytes; returns the validation status. */
gdn_status gdn_prefill_workspace_bytes(const gdn_prefill_args *args, size_t *bytes /* host */);

gdn_status gdn_prefill_chunked(const gdn_prefill_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_decode_batched -- one token for each of n sequences, one launch.
 *   Per sequence: conv of one row with its conv state (which advances), L2 of q
 *   and k, then per value head  kv = S k;  u = b (v - a kv);  S <- a S + u k^T;
 *   o = scale * S q, the state updated in place.  out = o, or the Z-gated RMSNorm
 *   of o when z != NULL.  The per-sequence pointers must be distinct.
 *   Defined by: decode_multi_seq (transformer_layer.rs) and the strided kernels
 *   conv1d_l2norm_f32_strided_k, gdn_f32_strided_norm_k,
 *   gated_rms_norm_f32_strided_k (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_decode_args {
  uint32_t struct_size;        /* sizeof(gdn_decode_args)                       */
  int32_t act_dtype;           /* x, conv_w, conv states, z, norm_w             */
  int32_t out_dtype;
  gdn_dims dims;
  int32_t num_seqs;            /* n >= 0                                        */
  const void *x;               /* [n][conv_dim] pre-conv rows                   */
  const void *conv_w;          /* [conv_dim][K]                                 */
  void *const *conv_state;     /* [n] pointers, in/out                          */
  const float *a;              /* [n][H_v]                                      */
  const float *b;              /* [n][H_v]                                      */
  float *const *h_state;       /* [n] pointers to fp32 [H_v][d_k][d_v], in/out    */
  const void *z;               /* [n][H_v*d_v] or NULL                          */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [n][H_v*d_v]                                  */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
} gdn_decode_args;

gdn_status gdn_decode_batched(const gdn_decode_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_verify_multi -- k_i draft rows for each of n sequences in one launch,
 *   every intermediate state written through this layer's WY pointer tables:
 *   wy_tables[t * GDN_VERIFY_WY_TABLE_SEQS + i] is sequence i's pointer in table t.
 *   Table 0 = the sequence state: read as S_0, overwritten with S_{k_i - 1}.
 *   Table t+1 (t < k_i - 1) receives S_t, the state after row t.  Entries of
 *   tables >= k_i are never read.  Rows are packed sequence-major
 *   (cu_ks[i]..cu_ks[i+1]); the conv of row t uses the conv state and rows
 *   0..t-1 of the same sequence; the conv state itself is only read.
 *   Outputs for every row as in gdn_decode_batched.
 *   Limits: n <= GDN_VERIFY_WY_TABLE_SEQS, 1 <= k_i <= max_k, max_k in 2..16.
 *   Defined by: decode_verify_multi and the VERIFY_WY_* constants
 *   (transformer_layer.rs); gdn_wyn_table_k, gdn_f32_strided_norm_snap_k
 *   (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_verify_args {
  uint32_t struct_size;        /* sizeof(gdn_verify_args)                       */
  int32_t act_dtype;
  int32_t out_dtype;
  gdn_dims dims;
  int32_t num_seqs;            /* n in 0..128                                   */
  int32_t max_k;               /* host: upper bound of every k_i, 2..16         */
  int32_t total_rows;          /* host: sum of k_i = cu_ks[n]                   */
  int32_t reserved;            /* must be 0                                     */
  const int32_t *cu_ks;        /* [n+1] row offsets                             */
  const void *x;               /* [total_rows][conv_dim]                        */
  const void *conv_w;          /* [conv_dim][K]                                 */
  void *const *conv_state;     /* [n] pointers, read only                       */
  const float *a;              /* [total_rows][H_v]                             */
  const float *b;              /* [total_rows][H_v]                             */
  float *const *wy_tables;     /* [16][128] state pointers (this layer's slice)  */
  const void *z;               /* [total_rows][H_v*d_v] or NULL                 */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [total_rows][H_v*d_v]                         */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
} gdn_verify_args;

gdn_status gdn_verify_multi(const gdn_verify_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_verify_commit -- fold the accepted prefix of a verify.
 *   For sequence i with n_i accepted rows (1 <= n_i <= k_i, the caller's
 *   contract; it is not checked on the host because it lives on the device):
 *   if n_i < k_i the state in table n_i (S_{n_i - 1}) is copied into table 0;
 *   the conv state becomes the last K-1 rows of [old conv state ; rows 0..n_i-1].
 *   Defined by: gdn_fold_accepted (trait_layer.rs), gdn_wy4_fold_k (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_commit_args {
  uint32_t struct_size;        /* sizeof(gdn_commit_args)                       */
  int32_t act_dtype;           /* dtype of x and the conv states                */
  gdn_dims dims;
  int32_t num_seqs;            /* n in 0..128                                   */
  int32_t reserved;            /* must be 0                                     */
  const int32_t *cu_ks;        /* [n+1]                                         */
  const int32_t *n_accepted;   /* [n]                                           */
  float *const *wy_tables;     /* [16][128]                                     */
  const void *x;               /* [sum k][conv_dim] rows given to the verify    */
  void *const *conv_state;     /* [n] pointers, in/out                          */
} gdn_commit_args;

gdn_status gdn_verify_commit(const gdn_commit_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_gated_rmsnorm -- out = o / sqrt(mean_j o_j^2 + eps) * w * SiLU(z), per
 *   (token, value head) over d_v.
 *   Defined by: gated_rms_norm_k, gated_rms_norm_prefill_k (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_norm_args {
  uint32_t struct_size;        /* sizeof(gdn_norm_args)                         */
  int32_t in_dtype;            /* dtype of o                                    */
  int32_t act_dtype;           /* dtype of z and norm_w                         */
  int32_t out_dtype;
  gdn_dims dims;               /* uses num_v_heads and head_dim_v               */
  int64_t total_tokens;        /* rows T >= 0                                   */
  const void *o;               /* [T][H_v*d_v]                                  */
  const void *z;               /* [T][H_v*d_v]                                  */
  const void *norm_w;          /* [d_v]                                         */
  void *out;                   /* [T][H_v*d_v]; may alias o                     */
  float eps;
  float reserved_f;            /* must be 0                                     */
} gdn_norm_args;

gdn_status gdn_gated_rmsnorm(const gdn_norm_args *args, void *stream);

/* Static description of a status code. */
const char *gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
