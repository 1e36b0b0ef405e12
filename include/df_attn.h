/*
 * df_attn.h — exact disentangled (C2P/P2C) self-attention for AMD gfx950.
 *
 * The operation is the DeBERTa-v2/v3 attention that the DisentangledFlash
 * 1.1.1 page describes ("Status": bidirectional DeBERTa-v2/v3-style C2P/P2C
 * attention without the [B,H,L,L] matrix; FP16, BF16 and strict FP32; head
 * dims 32, 64, 128; factorized 2-D padding masks; packed cu_seqlens layouts.
 * "Hugging Face usage": an LSE-producing forward, and Q/K/V and
 * relative-projection gradients). Per sequence and head, with local positions
 * i (query) and j (key):
 *
 *   S[i,j] = s * ( Q_i.K_j + Q_i.K_r[delta(i,j)] + K_j.Q_r[delta(j,i)] ),
 *   (with p2c_convention = DF_P2C_SHARED the last index is delta(i,j)),
 *   s = 1/sqrt(3*head_dim),
 *   delta(a,b) = clamp(bucket(a-b) + att, 0, R-1),  R = 2*att,
 *   att = buckets > 0 ? buckets : span,
 *   bucket(d) = d                       if buckets == 0 or |d| <= buckets/2,
 *             = sign(d)*(mid + ceil((mid-1)*ln(|d|/mid)/ln((span-1)/mid)))
 *                                        otherwise (mid = buckets/2),
 *   O_i = sum_j softmax_j(S[i,:]) V_j,   LSE_i = ln sum_j exp(S[i,j]).
 *
 * Pair (i,j) is scored only if both tokens are valid (factorized mask) and
 * belong to the same sequence. A masked query row gets O = 0, LSE = -inf, and
 * zero gradients.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronises; work is enqueued on `stream`
 *    (a hipStream_t; NULL = the null stream) and results are valid once that
 *    stream has reached this point.
 *  - Every argument is validated on the host before anything is enqueued. On
 *    an error nothing is launched and the outputs are untouched; the code is
 *    returned and df_last_error() describes the failed check. There is no
 *    fallback path of any kind.
 *  - q,k,v,out,dout,dq,dk,dv are [T, H, D] with element strides tok_stride
 *    and head_stride (D contiguous; both strides multiples of 8 elements for
 *    16-bit types and of 4 for fp32; base pointers 16-byte aligned).
 *    q_r,k_r,dq_r,dk_r are contiguous [H, R, D]. lse is fp32 [H, T].
 *  - key_mask: uint8 [T] (nonzero = valid token) or NULL (all valid).
 *  - cu_seqlens: int32 [batch+1] on the device, or NULL for the padded layout
 *    (batch sequences of max_seqlen tokens, T = batch*max_seqlen). With
 *    cu_seqlens the caller guarantees cu_seqlens[0] = 0, non-decreasing,
 *    cu_seqlens[batch] = T and every length <= max_seqlen (not checked: the
 *    array lives on the device).
 *  - The workspace is a caller-owned device buffer of at least
 *    df_attn_workspace_size() bytes, 256-byte aligned. Its contents are
 *    scratch and need no initialisation.
 *  - Results are deterministic: the same inputs, shapes and device give
 *    bitwise-identical outputs. No kernel uses atomics.
 */
#ifndef DF_ATTN_H
#define DF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DF_BF16 = 0, DF_FP16 = 1, DF_FP32 = 2 } df_dtype;

enum {
  DF_OK = 0,
  DF_ERR_INVALID = 1,      /* null pointer, bad shape/stride/alignment/index parameters */
  DF_ERR_UNSUPPORTED = 2,  /* head_dim not in {32,64,128}, unknown dtype */
  DF_ERR_WORKSPACE = 3,    /* workspace smaller than df_attn_workspace_size() */
  DF_ERR_HIP = 4           /* a HIP launch reported an error */
};

/* Which row of Q_r the P2C term of pair (query i, key j) uses:
 * DF_P2C_LITERAL: delta(j, i), the score formula as written above;
 * DF_P2C_SHARED:  delta(i, j), the row C2P uses, which is how deployed
 *                 DeBERTa-v2/v3 code indexes P2C in self-attention (for
 *                 parity with its checkpoints). Only this index changes. */
enum { DF_P2C_LITERAL = 0, DF_P2C_SHARED = 1 };

typedef struct {
  int32_t batch;          /* number of sequences (padded: B) */
  int32_t max_seqlen;     /* L (padded) or the longest sequence (packed) */
  int64_t total_tokens;   /* T: batch*max_seqlen (padded) or cu_seqlens[batch] */
  int32_t num_heads;      /* H */
  int32_t head_dim;       /* D in {32, 64, 128} */
  int32_t dtype;          /* df_dtype of q,k,v,q_r,k_r,out,dout and all gradients */
  int64_t tok_stride;     /* element stride between tokens of [T,H,D] tensors */
  int64_t head_stride;    /* element stride between heads of [T,H,D] tensors */
  int32_t p2c_convention; /* DF_P2C_LITERAL (0) or DF_P2C_SHARED (1) */
  int32_t flags;          /* 0 or DF_FLAG_BWD_REUSE_FWD */
} df_attn_shape;

/* df_attn_shape.flags. DF_FLAG_BWD_REUSE_FWD (df_attn_bwd only): the
 * workspace still holds what the df_attn_fwd call with the same inputs,
 * shape and index configuration left in it (the caller gave both calls the
 * same buffer, of df_attn_workspace_size(1, ...) bytes, and nothing wrote to
 * it in between); the backward then reuses that call's index tables and
 * relative-position strips instead of recomputing them. The results are the
 * same bit for bit; if the contents are not the forward's, they are wrong. */
enum { DF_FLAG_BWD_REUSE_FWD = 1 };

/* Non-raising eligibility check (the strict-contract idea of the
 * FastFlashAttention page, "Strict policy + fallback"). Returns DF_OK when
 * df_attn_fwd/df_attn_bwd accept this shape and index configuration, else the
 * error code they would return. `span` is DeBERTa's max_relative_positions
 * (>= 1), `buckets` its position_buckets (0 = no log bucketing; otherwise
 * >= 2, with span-1 > buckets/2). The shape is checked against the packed
 * contract (cu_seqlens given): the padded layout (cu_seqlens NULL) further
 * needs total_tokens == batch*max_seqlen, which df_attn_fwd/df_attn_bwd
 * check and this function does not. Host only; touches no device. */
int df_attn_supported(const df_attn_shape* shape, int32_t span, int32_t buckets);

/* Bytes of workspace needed by df_attn_fwd (pass 0) or df_attn_bwd (pass 1);
 * 0 if the arguments are invalid. Host only. */
size_t df_attn_workspace_size(int pass, const df_attn_shape* shape,
                              int32_t span, int32_t buckets);

/* The relative-position index tables over d = i - j in
 * [-(max_seqlen-1), max_seqlen-1], entry d + max_seqlen - 1:
 *   c2p_lut[.] = delta(i, j)  (row of K_r used by query i against key j)
 *   p2c_lut[.] = delta(j, i)  (row of Q_r used by key j against query i)
 * Both are int32 device arrays of 2*max_seqlen-1 entries, written on `stream`.
 * (These are the DF_P2C_LITERAL tables; under DF_P2C_SHARED the P2C row of a
 * pair is its c2p_lut entry.)
 * The ceiling of the log bucket is evaluated in fp64 with exact detection of
 * integer arguments, so the tables are exact for every configuration whose
 * ceiling arguments are not within ~1e-12 of an integer without being one. */
int df_build_rel_index(int32_t max_seqlen, int32_t span, int32_t buckets,
                       int32_t* c2p_lut, int32_t* p2c_lut, void* stream);

/* Forward pass: writes out [T,H,D] (dtype) and lse [H,T] (fp32, natural log;
 * -inf on masked rows). q_r and k_r must have R = 2*att rows: the library
 * sees only their pointers and cannot check this, so the caller (or the
 * Python binding, which does) must ensure it; fewer rows make the kernels
 * read past the allocation. */
int df_attn_fwd(const df_attn_shape* shape,
                const void* q, const void* k, const void* v,
                const void* q_r, const void* k_r,
                int32_t span, int32_t buckets,
                const uint8_t* key_mask, const int32_t* cu_seqlens,
                void* out, float* lse,
                void* workspace, size_t workspace_bytes, void* stream);

/* Inference forward (DisentangledFlash 1.1.1 page, "Bundled H200 tuning
 * profile": inference is a phase of its own, next to the training forward):
 * the same computation as df_attn_fwd, writing out [T,H,D] only; no LSE and
 * nothing for a backward pass is kept. Arguments, layouts, workspace
 * (df_attn_workspace_size pass 0) and error codes as df_attn_fwd; the
 * caller owns every buffer. */
int df_attn_fwd_inference(const df_attn_shape* shape,
                          const void* q, const void* k, const void* v,
                          const void* q_r, const void* k_r,
                          int32_t span, int32_t buckets,
                          const uint8_t* key_mask, const int32_t* cu_seqlens,
                          void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments as df_attn_fwd (lse may be NULL, then
 * as df_attn_fwd_inference), without a workspace argument. The workspace is
 * a static device array of DF_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, which every device it runs on holds until the process ends; the
 * call allocates and frees nothing. A shape whose df_attn_workspace_size(0,
 * ...) exceeds that size is rejected with DF_ERR_WORKSPACE before anything
 * is enqueued (bf16/fp16 with R = 512 fit about 32,000 token-heads, e.g.
 * 2,600 tokens at 12 heads). The stream must belong to the current device.
 * The first call on a device looks up the array's device address there (it
 * may load the library's device code), so make it before capturing a graph.
 * All calls on one device share the array and it keeps the last call's
 * contents: calls that overlap on one device (concurrent streams or threads)
 * race and must be ordered by the caller. Nothing in the array needs
 * clearing between calls. */
#define DF_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int df_attn_fwd_noalloc(const df_attn_shape* shape,
                        const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r,
                        int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens,
                        void* out, float* lse, void* stream);

/* Backward pass: given the forward's out and lse and the output gradient
 * dout, writes dq, dk, dv [T,H,D] and dq_r, dk_r [H,R,D] (all dtype). The
 * gradients overwrite the outputs (never accumulate). Scores are recomputed
 * from the inputs and lse; the index tables and relative-position strips are
 * recomputed too, unless shape->flags has DF_FLAG_BWD_REUSE_FWD (then they
 * are taken from the forward's workspace, see there). For a packed batch
 * (cu_seqlens) whose grid, the longest sequence's 128-row blocks for every
 * sequence, is at least 1.5 times total_tokens, the dK/dV and dQ kernels run
 * side by side: dQ on a second stream of the current device (default
 * priority; the first such call on a device creates it and two events, kept
 * until the process ends, so make that call before capturing a graph),
 * forked from `stream` after the preceding work and joined back before the
 * relative-gradient kernels, so every result is ordered on `stream` as
 * usual and is bitwise the same either way. The stream must belong to the
 * current device. */
int df_attn_bwd(const df_attn_shape* shape,
                const void* q, const void* k, const void* v,
                const void* q_r, const void* k_r,
                int32_t span, int32_t buckets,
                const uint8_t* key_mask, const int32_t* cu_seqlens,
                const void* out, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, void* dq_r, void* dk_r,
                void* workspace, size_t workspace_bytes, void* stream);

/* Training forward and backward with attention-probability dropout
 * (DisentangledFlash 1.1.1 page, "Status": dropout is applied inside the
 * fused kernels; the backward recomputes the mask from the Philox counter
 * rather than reading a saved one). After the softmax each probability is kept with probability
 * 1 - dropout_p and scaled by 1 / (1 - dropout_p), or set to 0; the LSE is
 * that of the undropped scores. The mask is a function of (seed, offset) and
 * the pair: for sequence n, head h, local query i and local key j, the call
 * of Philox4x32-10 with counter (j / 8, i, n * num_heads + h, offset) and key
 * (seed mod 2^32, seed >> 32) covers keys 8 (j / 8) .. 8 (j / 8) + 7; key j
 * takes the low (j even) or high (j odd) 16 bits of its word (j % 8) / 2 and
 * keeps the pair iff they are >= floor(p * 2^16).
 * The backward must be called with the forward's (dropout_p, seed, offset).
 * Arguments otherwise as df_attn_fwd / df_attn_bwd; dropout_p must be in
 * [0, 1) (DF_ERR_INVALID otherwise; for DF_FP16 at most 0.999, else
 * DF_ERR_UNSUPPORTED, since the backward carries dP / (1 - dropout_p) in fp16
 * operands); dropout_p = 0 is the plain path. */
int df_attn_fwd_dropout(const df_attn_shape* shape,
                        const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r,
                        int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens,
                        float dropout_p, uint64_t seed, uint32_t offset,
                        void* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);
int df_attn_bwd_dropout(const df_attn_shape* shape,
                        const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r,
                        int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens,
                        float dropout_p, uint64_t seed, uint32_t offset,
                        const void* out, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv, void* dq_r, void* dk_r,
                        void* workspace, size_t workspace_bytes, void* stream);


/* Fused Q/K/V and relative-position projections (DisentangledFlash 1.1.1
 * page, "Status": the fused QKV projection is always enabled; "Hugging Face
 * usage": the Q/K/V and relative-position projections stay in the model's
 * graph). One GEMM with the three maps' weights stacked as w [3*H*D, hidden]
 * (row-major, rows W_q, W_k, W_v) and bias [3*H*D] (or NULL):
 *   q[t,h,d]   = sum_e x[t,e]   w[h*D+d, e]       + bias[h*D+d]
 *   k[t,h,d]   = sum_e x[t,e]   w[H*D+h*D+d, e]   + bias[H*D+h*D+d]
 *   v[t,h,d]   = sum_e x[t,e]   w[2*H*D+h*D+d, e] + bias[2*H*D+h*D+d]
 *   q_r[h,r,d] = sum_e rel[r,e] w[h*D+d, e]       + bias[h*D+d]
 *   k_r[h,r,d] = sum_e rel[r,e] w[H*D+h*D+d, e]   + bias[H*D+h*D+d]
 * (the relative-position embedding rows go through the query and key maps:
 * DeBERTa-v2/v3's shared attention key). x is [tokens, hidden] and rel
 * [rel_rows, hidden], both row-major with rows of `hidden` elements; q, k, v
 * are written contiguous [tokens, H, D] (tok_stride H*D, head_stride D, the
 * layout df_attn_fwd takes) and q_r, k_r contiguous [H, rel_rows, D]. With
 * rel == NULL (and rel_rows == 0) only q, k, v are written. dtype is DF_BF16
 * or DF_FP16 for every operand and output (fp32 accumulation; DF_FP32 gives
 * DF_ERR_UNSUPPORTED); head_dim in {32, 64, 128}; hidden a positive multiple
 * of 8; x, w and rel 16-byte aligned. All pointers are caller-owned device
 * pointers; nothing is allocated; work is enqueued on `stream`; errors as
 * for df_attn_fwd (checked on the host before anything is enqueued).
 * DF_ERR_UNSUPPORTED also for tokens >= 2^30, hidden >= 2^23 or
 * tokens * H * D >= 2^40. */
int df_qkv_proj(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim, int32_t rel_rows,
                int32_t dtype, const void* x, const void* w, const void* bias, const void* rel,
                void* q, void* k, void* v, void* q_r, void* k_r, void* stream);


/* Backward of df_qkv_proj (the same maps, 16-bit operands, fp32
 * accumulation): given the output gradients dqkv [tokens, 3*H*D] (row-major:
 * dq, dk, dv side by side per token, the layout df_attn_bwd writes with
 * tok_stride 3*H*D and head_stride D) and, when rel is given, dq_r and dk_r
 * [H, rel_rows, D] (as df_attn_bwd writes them), writes
 *   dx [tokens, hidden]      = dY W
 *   drel [rel_rows, hidden]  = dY_r W[:2HD]        (when rel is given)
 *   dw [3*H*D, hidden]       = dY^T x + [dY_r^T rel; 0]
 *   db [3*H*D] (or NULL)     = column sums of dY and dY_r
 * with dY the [tokens, 3HD] gradient and dY_r the [rel_rows, 2HD] one
 * (column h*D + d of its first half is dq_r[h][r][d], of its second half
 * dk_r[h][r][d]). The dw sum over tokens runs in fixed chunks added in a
 * fixed order (deterministic). The workspace is caller-owned, of at least
 * df_qkv_proj_bwd_workspace_size() bytes, 256-byte aligned; other
 * conventions as df_qkv_proj. DF_ERR_UNSUPPORTED for tokens >= 2^23,
 * hidden >= 2^20, 3*H*D >= 2^20 or rel_rows >= 2^20 (the workspace size is
 * then 0). */
size_t df_qkv_proj_bwd_workspace_size(int64_t tokens, int32_t hidden, int32_t num_heads,
                                      int32_t head_dim, int32_t rel_rows, int32_t dtype);
int df_qkv_proj_bwd(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim,
                    int32_t rel_rows, int32_t dtype, const void* x, const void* w, const void* rel,
                    const void* dqkv, const void* dq_r, const void* dk_r,
                    void* dx, void* dw, void* db, void* drel,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Packing helpers for the packed layout (DisentangledFlash 1.1.1 page,
 * "Packed unpadded inference and training": right-padded [B, L, ...] input
 * becomes FlashAttention-style [total_tokens, ...] rows with cu_seqlens, and
 * the packed output goes back). Rows are opaque: row_bytes bytes each (a
 * positive multiple of 16), padded is [batch, max_len] rows, mask uint8
 * [batch, max_len] (nonzero = valid token). Sequence b's length is the
 * number of valid tokens in mask row b, and its valid tokens, in order,
 * become packed rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (for a right-padded
 * mask: its first tokens, the layout df_attn_fwd takes with cu_seqlens).
 *
 * df_pack_padded writes packed (capacity batch*max_len rows; only the first
 * cu_seqlens[batch] are written), cu_seqlens int32 [batch+1] and, unless
 * NULL, the largest length into *max_seqlen (an int32 in device memory).
 * df_unpack_packed writes every row of padded: the packed row of each valid
 * position, zeros elsewhere (cu_seqlens as written by df_pack_padded for
 * the same mask). All pointers are caller-owned device pointers (padded and
 * packed 16-byte aligned); work is enqueued on `stream`; host-side checks
 * and error codes as for df_attn_fwd. */
int df_pack_padded(int32_t batch, int32_t max_len, int64_t row_bytes, const void* padded,
                   const uint8_t* mask, void* packed, int32_t* cu_seqlens, int32_t* max_seqlen,
                   void* stream);
int df_unpack_packed(int32_t batch, int32_t max_len, int64_t row_bytes, const void* packed,
                     const uint8_t* mask, const int32_t* cu_seqlens, void* padded, void* stream);

/* Static description of an error code. */
const char* df_strerror(int code);

/* Description of the last error returned on the calling thread ("" if none). */
const char* df_last_error(void);

/* Per-kernel timing for measurement. df_attn_profile_enable(1) creates a pool
 * of HIP events (no device memory); while enabled, every kernel launch of
 * df_attn_fwd / df_attn_bwd is bracketed by two events recorded on the
 * caller's stream. df_attn_profile_read() waits for the recorded events, adds
 * the elapsed milliseconds of each launch to ms[stage] and the launch count to
 * launches[stage] for stage < n_stages (arrays of at least n_stages entries,
 * zeroed by the caller), and forgets the records. Launches beyond the pool
 * (4096 per read) are not timed. df_attn_profile_enable(0) releases the pool.
 * Not thread-safe; meant for a single benchmarking thread. */
enum {
  DF_STAGE_INDEX = 0, DF_STAGE_STRIPS = 1, DF_STAGE_FWD = 2, DF_STAGE_DELTA = 3,
  DF_STAGE_DKV = 4, DF_STAGE_DQ = 5,
  DF_STAGE_RELGRAD_DX = 6, /* not launched: the dQ and dK/dV kernels add the per-token
                              relative terms themselves */
  DF_STAGE_RELGRAD_DW = 7, DF_STAGE_RELGRAD_SUM = 8, DF_NUM_STAGES = 9
};
int df_attn_profile_enable(int on);
int df_attn_profile_read(float* ms, int* launches, int n_stages);
const char* df_attn_stage_name(int stage);

/* Library version, as major*10000 + minor*100 + patch. */
int df_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DF_ATTN_H */
