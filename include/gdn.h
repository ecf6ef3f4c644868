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
 *        - the write-on-accept verify, which stores per-row update vectors instead
 *          of states, and the fold of the accepted rows into the state
 *                                                      -> gdn_verify_woa, gdn_fold_accepted
 *        - k consecutive tokens for each of many sequences, state written once
 *                                                      -> gdn_decode_tokens
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
 *   - The recurrent state of a sequence is h[H_v][d_k][d_v] = S^T per value head
 *     (d_v fastest), fp32 by default or IEEE binary16 (gdn_options.state_dtype),
 *     reached through a device array of per-sequence pointers.  All recurrence
 *     arithmetic is fp32; a binary16 state is widened when read and rounded to
 *     nearest-even when stored (FP16 h-state variants and the ssm_h_f16_to_f32_k /
 *     ssm_h_f32_to_f16_k converters, layer_struct.rs page).
 *     The conv state of a sequence is its last (K-1) raw pre-conv rows, oldest
 *     first, [K-1][conv_dim] in the activation dtype, also through a pointer array.
 *   - a, b are fp32 [rows][H_v]: the decay and write strength, or, with
 *     gdn_options.gate_mode = GDN_GATES_RAW, the raw gate inputs g and beta from
 *     which the kernels form a = exp(-softplus(g)) and b = sigmoid(beta) (the
 *     ba_gates / compute_gdn_gates handles of the layer_struct.rs page name this
 *     step; the pages give no formula, this is the plainest one).
 *   - z is [rows][H_v*d_v]; norm_w is [d_v], shared by all heads; z and norm_w use
 *     the activation dtype.  The norm gate is SiLU(z), or sigmoid(z) with
 *     gdn_options.norm_gate = GDN_NORM_GATE_SIGMOID (a gdn_norm_sigmoid model,
 *     doc comment of gated_rms_norm_f32_strided_k on the layer_struct.rs page).
 *   - Alignment: every buffer passed directly in an argument struct starts on a
 *     16-byte boundary (hipMalloc and framework allocations do; a view into the
 *     middle of one may not): the kernels move rows, outputs and the stash in 8- and
 *     16-byte vectors.  A misaligned one makes the call return GDN_ERR_INVALID_ARG.
 *     The per-sequence state and conv-state buffers reached through the pointer
 *     arrays must be 16-byte aligned too; the library cannot check those.
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

#define GDN_ABI_VERSION 2

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

/* Most tokens per sequence in one gdn_decode_tokens call (16 drafts plus one; the
 * K = 17 gated_delta_rule_wy17 handle, layer_struct.rs page). */
#define GDN_DECODE_MAX_TOKENS 17

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* NULL required pointer, bad sizes, struct_size mismatch   */
  GDN_ERR_UNSUPPORTED = 2, /* valid shape with no kernel (d not in {32,64,128}, ...)   */
  GDN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required              */
  GDN_ERR_HIP = 4          /* the HIP runtime reported a launch error                 */
} gdn_status;

typedef enum gdn_dtype {
  GDN_DTYPE_F32 = 0,
  GDN_DTYPE_BF16 = 1,
  GDN_DTYPE_F16 = 2  /* IEEE binary16: recurrent states only (gdn_options.state_dtype) */
} gdn_dtype;

typedef enum gdn_gate_mode {
  GDN_GATES_DIRECT = 0, /* a = decay a_t in [0, 1], b = write strength b_t           */
  GDN_GATES_RAW = 1     /* a = g, b = beta; a_t = exp(-softplus(g)), b_t = sigmoid(beta) */
} gdn_gate_mode;

typedef enum gdn_norm_gate {
  GDN_NORM_GATE_SILU = 0,   /* out = rmsnorm(o) * w * SiLU(z)    */
  GDN_NORM_GATE_SIGMOID = 1 /* out = rmsnorm(o) * w * sigmoid(z) */
} gdn_norm_gate;

/* Options of the recurrence and norm entry points, the last member of their
 * argument structs.  All zero = fp32 states, direct gates, SiLU norm gate.  An
 * entry point refuses (GDN_ERR_INVALID_ARG) a non-zero option it does not take:
 * gdn_verify_commit and gdn_fold_accepted take only state_dtype,
 * gdn_gated_rmsnorm only norm_gate. */
typedef struct gdn_options {
  int32_t state_dtype; /* GDN_DTYPE_F32 or GDN_DTYPE_F16: element type of every
                          recurrent state the call reads or writes              */
  int32_t gate_mode;   /* gdn_gate_mode                                         */
  int32_t norm_gate;   /* gdn_norm_gate (fused or standalone gated norm)        */
  int32_t reserved;    /* must be 0                                             */
} gdn_options;

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
 *   With T = 0 (every sequence empty) the per-token arrays (a, b, x or y, z,
 *   out) may be NULL and nothing changes; cu_seqlens and h_state are still
 *   required for n > 0.
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
  void *const *h_state;        /* [n] pointers to [H_v][d_k][d_v] states, in/out  */
  const void *z;               /* [T][H_v*d_v] or NULL                          */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [T][H_v*d_v]                                  */
  float scale;                 /* output scale (1.0 = the plain rule)           */
  float l2_eps;                /* front L2 epsilon (with x)                     */
  float norm_eps;              /* RMSNorm epsilon (with z)                      */
  float reserved_f;            /* must be 0                                     */
  void *workspace;             /* device scratch, >= required bytes             */
  size_t workspace_bytes;
  gdn_options opt;             /* state dtype (the stored state is widened at a
                                  sequence's start and narrowed at its end), gate
                                  mode, norm gate of the epilogue                 */
} gdn_prefill_args;

/* Workspace bytes gdn_prefill_chunked needs for these arguments (pointers are not
 * read).  Writes *bytes; returns the validation status. */
gdn_status gdn_prefill_workspace_bytes(const gdn_prefill_args *args, size_t *bytes /* host */);

gdn_status gdn_prefill_chunked(const gdn_prefill_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_prefill_chunked_noalloc -- gdn_prefill_chunked without a caller workspace
 *   and without any allocation, for callers that cannot allocate device memory:
 *   code under HIP graph capture, tight serving loops, harnesses that forbid
 *   allocation.  Same arguments, results and validation as gdn_prefill_chunked,
 *   except: workspace must be NULL and workspace_bytes 0 (else
 *   GDN_ERR_INVALID_ARG), and the workspace the call needs
 *   (gdn_prefill_workspace_bytes) must not exceed GDN_PREFILL_SCRATCH_BYTES (else
 *   GDN_ERR_WORKSPACE; nothing launched).  The call runs in a library-owned device
 *   array of GDN_PREFILL_SCRATCH_BYTES bytes, one per GPU, present from the
 *   library's load on that GPU until the process ends; its address is looked up
 *   on the first call on each device.  Every call on one GPU uses the same array:
 *   calls that overlap on one GPU (other streams, other threads) race and must be
 *   serialised by the caller.  Returns GDN_ERR_HIP if the array's address cannot
 *   be obtained.
 * ------------------------------------------------------------------------- */
#define GDN_PREFILL_SCRATCH_BYTES ((size_t)64 << 20)

gdn_status gdn_prefill_chunked_noalloc(const gdn_prefill_args *args, void *stream);

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
  void *const *h_state;        /* [n] pointers to [H_v][d_k][d_v] states, in/out  */
  const void *z;               /* [n][H_v*d_v] or NULL                          */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [n][H_v*d_v]                                  */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
  gdn_options opt;
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
  void *const *wy_tables;      /* [16][128] state pointers (this layer's slice)  */
  const void *z;               /* [total_rows][H_v*d_v] or NULL                 */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [total_rows][H_v*d_v]                         */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
  gdn_options opt;             /* with binary16 states every stored state, and the
                                  state carried to the next row, is rounded     */
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
  void *const *wy_tables;      /* [16][128]                                     */
  const void *x;               /* [sum k][conv_dim] rows given to the verify    */
  void *const *conv_state;     /* [n] pointers, in/out                          */
  gdn_options opt;             /* state_dtype only                              */
} gdn_commit_args;

gdn_status gdn_verify_commit(const gdn_commit_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_verify_woa -- write-on-accept verify: the rows, outputs and limits of
 *   gdn_verify_multi, but no state is written.  Each sequence's state is read from
 *   *h_state[i]; for every packed row r the call stores in stash row r what the
 *   rank-1 update S_r = a_r S_{r-1} + u_r k_r^T needs:
 *       stash[r * row_floats + g * d_k + j]                k_hat of key head g
 *       stash[r * row_floats + H_k*d_k + h * d_v + j]      u of value head h
 *       stash[r * row_floats + H_k*d_k + H_v*d_v + h]      a_r of value head h
 *   with row_floats = H_k*d_k + H_v*d_v + H_v rounded up to a multiple of 4, and
 *   u = b (v - a S k) computed from the state the row starts from.
 *   gdn_fold_accepted then applies the accepted rows to the state.  The verify
 *   moves one state read per sequence instead of k_i state writes.
 *   Defined by: the write-on-accept handles gdn_wy4_woa_k, gdn_wy4_fold_k and the
 *   woa_stash binding (layer_struct.rs), gdn_woa_stash_seq_floats, gdn_woa_bind
 *   and gdn_fold_accepted (trait_layer.rs).  The pages name the stash, not its
 *   contents; the (k_hat, u, a) rows are the plainest contents that let the fold
 *   reproduce the recorded states.  fp32 states at d_k = d_v = 64 or 128 are
 *   verified in the WY form over the k_i rows (outputs and u within fp32 rounding
 *   of the row-by-row values); binary16 states and d = 32 row by row, whose fold
 *   reproduces gdn_verify_multi's states bit for bit.
 * ------------------------------------------------------------------------- */
typedef struct gdn_woa_args {
  uint32_t struct_size;        /* sizeof(gdn_woa_args)                          */
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
  void *const *h_state;        /* [n] pointers to [H_v][d_k][d_v], read only     */
  const void *z;               /* [total_rows][H_v*d_v] or NULL                 */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [total_rows][H_v*d_v]                         */
  float *stash;                /* [total_rows][row_floats] fp32, out             */
  size_t stash_bytes;          /* bytes available at stash                      */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
  gdn_options opt;
} gdn_woa_args;

/* Bytes of stash gdn_verify_woa needs for these arguments (pointers are not
 * read): total_rows * row_floats * 4.  Writes *bytes; returns the validation
 * status. */
gdn_status gdn_woa_stash_bytes(const gdn_woa_args *args, size_t *bytes /* host */);

gdn_status gdn_verify_woa(const gdn_woa_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_fold_accepted -- apply the accepted rows of a write-on-accept verify.
 *   For sequence i with n_i accepted rows (1 <= n_i <= k_i, the caller's
 *   contract, as for gdn_verify_commit): for r = cu_ks[i] .. cu_ks[i] + n_i - 1 in
 *   order, every value head's state becomes a_r S + u_r k_r^T (rounded after every
 *   row when the state is binary16), reading stash row r; the state is read and
 *   written once.  The conv state becomes the last K-1 rows of
 *   [old conv state ; rows 0..n_i-1].  The result is the state
 *   gdn_verify_multi records after row n_i - 1 (bit for bit when the stash comes
 *   from a row-by-row verify, within fp32 rounding when it comes from the WY form;
 *   see gdn_verify_woa).
 *   Defined by: gdn_fold_accepted (trait_layer.rs), gdn_wy4_fold_k (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_fold_args {
  uint32_t struct_size;        /* sizeof(gdn_fold_args)                         */
  int32_t act_dtype;           /* dtype of x and the conv states                */
  gdn_dims dims;
  int32_t num_seqs;            /* n in 0..128                                   */
  int32_t total_rows;          /* host: cu_ks[n]                                */
  const int32_t *cu_ks;        /* [n+1], as given to gdn_verify_woa             */
  const int32_t *n_accepted;   /* [n]                                           */
  void *const *h_state;        /* [n] pointers, in/out                          */
  const float *stash;          /* written by gdn_verify_woa                     */
  size_t stash_bytes;
  const void *x;               /* [total_rows][conv_dim] rows given to the verify */
  void *const *conv_state;     /* [n] pointers, in/out                          */
  gdn_options opt;             /* state_dtype only                              */
} gdn_fold_args;

gdn_status gdn_fold_accepted(const gdn_fold_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_decode_tokens -- k_i consecutive tokens for each of n sequences in one
 *   launch, equal to k_i gdn_decode_batched steps in a row: conv rows use the conv
 *   state and the earlier rows, outputs for every token, and each sequence's
 *   state (*h_state[i]) and conv state advance over all k_i tokens, the state
 *   being read and written once.  Rows are packed sequence-major.
 *   Limits: n <= 128, 1 <= k_i <= max_tokens <= GDN_DECODE_MAX_TOKENS.
 *   Defined by: decode_batched, the k-consecutive-token decode of one sequence
 *   (transformer_layer.rs page), batched over sequences as decode_multi_seq is;
 *   gated_delta_rule_wy17 for K = 17 (layer_struct.rs).
 * ------------------------------------------------------------------------- */
typedef struct gdn_tokens_args {
  uint32_t struct_size;        /* sizeof(gdn_tokens_args)                       */
  int32_t act_dtype;
  int32_t out_dtype;
  gdn_dims dims;
  int32_t num_seqs;            /* n in 0..128                                   */
  int32_t max_tokens;          /* host: upper bound of every k_i, 1..17         */
  int32_t total_rows;          /* host: cu_tokens[n]                            */
  int32_t reserved;            /* must be 0                                     */
  const int32_t *cu_tokens;    /* [n+1] row offsets                             */
  const void *x;               /* [total_rows][conv_dim]                        */
  const void *conv_w;          /* [conv_dim][K]                                 */
  void *const *conv_state;     /* [n] pointers, in/out                          */
  const float *a;              /* [total_rows][H_v]                             */
  const float *b;              /* [total_rows][H_v]                             */
  void *const *h_state;        /* [n] pointers, in/out                          */
  const void *z;               /* [total_rows][H_v*d_v] or NULL                 */
  const void *norm_w;          /* [d_v] (with z)                                */
  void *out;                   /* [total_rows][H_v*d_v]                         */
  float scale;
  float l2_eps;
  float norm_eps;
  float reserved_f;            /* must be 0                                     */
  gdn_options opt;
} gdn_tokens_args;

gdn_status gdn_decode_tokens(const gdn_tokens_args *args, void *stream);

/* ---------------------------------------------------------------------------
 * gdn_gated_rmsnorm -- out = o / sqrt(mean_j o_j^2 + eps) * w * SiLU(z), per
 *   (token, value head) over d_v.
 *   Defined by: gated_rms_norm_k, gated_rms_norm_prefill_k (layer_struct.rs);
 *   sigmoid(z) in place of SiLU(z) with opt.norm_gate = GDN_NORM_GATE_SIGMOID.
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
  gdn_options opt;             /* norm_gate only                                */
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
