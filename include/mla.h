/*
 * libmla — Multi-Latent Attention (MLA) forward pass for AMD Instinct MI355X
 * (gfx950 / CDNA4).  C ABI: plain pointers and sizes only.
 *
 * The layer (as stated by "CSDN walkthrough of HF DeepseekV3Attention",
 * __init__/forward, and "kimi_vl.py - KimiVL attention adapter", sections
 * "Q projection and KV compression" and "concatenating the final Q and K"):
 *
 *   q        = q_lora_rank ? W_qb * RMSNorm_q(W_qa x) : W_q x     [N, H, d_nope + d_rope]
 *   [c|k_pe] = W_kva x                                            [N, r_kv + d_rope]
 *   c_n      = RMSNorm_kv(c)
 *   kv       = W_kvb c_n                                          [N, H, d_nope + d_v]
 *   q_pe, k_pe rotated by RoPE (plain or YaRN) at each token's position, k_pe
 *   being ONE head shared by all H heads; not rotated for MLA_ROPE_NONE (the
 *   unrotated shared part of "Kimi-K3 atlas: Gated MLA")
 *   A_h      = softmax(scale * [q_nope|q_pe]_h [k_nope_h|k_pe]^T + causal) v_h
 *   A        = A * sigmoid(W_g x)          (output_gate, "Kimi-K3 atlas" mla-init)
 *   out      = W_o A                                              [N, hidden]
 *
 * Conventions for every call
 *   - Ownership: the caller owns every buffer.  The library allocates no device
 *     or host memory, keeps no device state between calls and never
 *     synchronises: device work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and runs asynchronously.
 *   - Errors: all argument checks run on the host before anything is enqueued,
 *     so a call enqueues all of its work or none of it.  A failed check returns
 *     a status other than MLA_OK; mla_last_error() returns a message for the
 *     last failure on the calling thread.  A failed kernel launch returns
 *     MLA_ERR_HIP (work enqueued before it in the same call may have run).
 *   - Layout: row-major, token-major ("THD": packed tokens, no padding).
 *     Linear weights use the nn.Linear layout [out_features, in_features] and
 *     compute y = x W^T ("MiniMind: attention forward pass" section 2).  Device
 *     pointers must be 16-byte aligned and row strides multiples of 8 elements
 *     (MLA_ERR_MISALIGNED otherwise).
 *   - Dtypes: cfg.dtype MLA_BF16 (bf16 storage, fp32 accumulation and fp32
 *     softmax/norm arithmetic) or MLA_F32 (fp32 everywhere).  Norm gains use the
 *     weight dtype; RoPE tables are fp32; index arrays are int32.  Inside the
 *     bf16 prefill layer the attention operands (q, kv, the shared k_pe) are
 *     held in the workspace in the type cfg.attn_operand selects:
 *     MLA_ATTN_F16 (the default, 0): fp16, three more mantissa bits than bf16,
 *       which the DeepSeek-V3-shaped layer needs to stay within the parity
 *       bound; its range is |x| <= 65504, and a q, kv or k_pe value beyond it
 *       SATURATES to +-65504 (NaN stays NaN), so this mode is for layers whose
 *       activations stay in that range (the attention output is a convex
 *       combination of v, so it then does too);
 *     MLA_ATTN_BF16: bf16 operands, the full bf16 range, less precise.
 *     Everything the caller passes or receives stays bf16.
 *   - Shapes supported by the bf16 kernels: d_nope = 128, d_rope = 64,
 *     d_v = 128, r_kv = 512 (the DeepSeek-V3 / Kimi head shape); other shapes
 *     return MLA_ERR_UNSUPPORTED for bf16.  The fp32 kernels take any
 *     d_nope, d_v <= 256, even d_rope <= 128 and r_kv <= 1024.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 6

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,   /* null pointer, bad dimension, inconsistent sizes      */
  MLA_ERR_UNSUPPORTED = 2,   /* valid MLA configuration with no compiled kernel       */
  MLA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace_size */
  MLA_ERR_MISALIGNED = 4,    /* pointer not 16-byte aligned / stride not a multiple of 8 */
  MLA_ERR_HIP = 5            /* a HIP launch or copy failed                            */
} mla_status;

/* MLA_F16 is accepted only as the operand type of mla_attention_prefill and
 * mla_attention_prefix. */
typedef enum mla_dtype { MLA_BF16 = 0, MLA_F32 = 1, MLA_F16 = 2 } mla_dtype;

/* Element type of the attention operands inside the bf16 prefill layer. */
typedef enum mla_attn_operand { MLA_ATTN_F16 = 0, MLA_ATTN_BF16 = 1 } mla_attn_operand;

/* RoPE variant ("Megatron-LM MLA guide", normalization and position-encoding
 * parameters: rope or yarn; "Kimi-K3 atlas": no rotary embedding). */
typedef enum mla_rope_kind { MLA_ROPE_NONE = 0, MLA_ROPE_PLAIN = 1, MLA_ROPE_YARN = 2 } mla_rope_kind;

/* Layer configuration.  Every field is explicit; nothing is defaulted.
 * Dimension names follow "CSDN walkthrough of HF DeepseekV3Attention" (__init__):
 * q_head_dim = qk_nope_dim + qk_rope_dim. */
typedef struct mla_config {
  int32_t hidden;            /* model width                                           */
  int32_t num_heads;         /* H                                                     */
  int32_t q_lora_rank;       /* r_q; 0 => direct q projection (no query latent)       */
  int32_t kv_lora_rank;      /* r_kv                                                  */
  int32_t qk_nope_dim;       /* d_nope                                                */
  int32_t qk_rope_dim;       /* d_rope (even)                                         */
  int32_t v_head_dim;        /* d_v (may differ from d_nope + d_rope; never padded)   */
  int32_t dtype;             /* mla_dtype                                             */
  int32_t rope_kind;         /* mla_rope_kind                                         */
  int32_t yarn_original_max_pos; /* YaRN original_max_position_embeddings              */
  int32_t output_gate;       /* 1 => out = W_o (A * sigmoid(W_g x))                    */
  float norm_eps;            /* RMSNorm epsilon (inside the mean)                     */
  float softmax_scale;       /* > 0: used as is; <= 0: derived (mla_softmax_scale)     */
  double rope_theta;         /* rotary base                                           */
  double yarn_factor;        /* YaRN scale s                                          */
  double yarn_beta_fast;
  double yarn_beta_slow;
  double yarn_mscale;
  double yarn_mscale_all_dim;
  /* Layout / config variants (0 = the DeepSeek-V3 defaults above). */
  int32_t rope_interleave;   /* 1 => RoPE rotates interleaved pairs (2i, 2i+1) in place
                              * instead of (i, i + d_rope/2): the rope_interleave branch
                              * of the forward in the "CSDN walkthrough of HF
                              * DeepseekV3Attention", for weights with interleaved pairs                                    */
  int32_t o_groups;          /* > 0 => grouped low-rank output projection ("Megatron-LM
                              * MLA guide", output_projection_groups): the H*d_v
                              * attention features split into o_groups consecutive
                              * groups, group g projected to o_lora_rank by its block of
                              * w_o_a, the groups' results concatenated and projected to
                              * hidden by w_o_b; w_o unused                            */
  int32_t o_lora_rank;       /* output_projection_lora_rank (o_groups > 0)            */
  int32_t attn_operand;      /* bf16 layers: mla_attn_operand, the element type of the
                              * attention operands q, kv and k_pe inside mla_prefill_fwd
                              * and mla_prefill_chunk_fwd (see Dtypes above); must be 0
                              * for MLA_F32                                            */
} mla_config;

/* Device pointers to the layer weights, nn.Linear layout, dtype = cfg.dtype. */
typedef struct mla_weights {
  const void* w_q_a;       /* [r_q, hidden]            (q_lora_rank > 0, else NULL)   */
  const void* q_a_gamma;   /* [r_q]                    (q_lora_rank > 0, else NULL)   */
  const void* w_q_b;       /* [H*(d_nope+d_rope), r_q] (q_lora_rank > 0, else NULL)   */
  const void* w_q;         /* [H*(d_nope+d_rope), hidden] (q_lora_rank == 0, else NULL) */
  const void* w_kv_a;      /* [r_kv + d_rope, hidden]                                 */
  const void* kv_a_gamma;  /* [r_kv]                                                  */
  const void* w_kv_b;      /* [H*(d_nope+d_v), r_kv]; rows of head h: [k_nope | v]    */
  const void* w_o;         /* [hidden, H*d_v]                                         */
  const void* w_g;         /* [H*d_v, hidden] (output_gate, else NULL)                */
  const void* w_o_a;       /* [o_groups*o_lora_rank, H*d_v/o_groups] (o_groups > 0): rows
                            * g*o_lora_rank .. of group g                               */
  const void* w_o_b;       /* [hidden, o_groups*o_lora_rank] (o_groups > 0)           */
} mla_weights;

/* ---------------------------------------------------------------- host-only */

/* ABI version of the loaded library (MLA_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Checks a configuration (dims positive, rope dim even, YaRN parameters
 * sensible).  Host-only, no device work. */
mla_status mla_validate_config(const mla_config* cfg);

/* Softmax scale: (d_nope + d_rope)^-0.5, times mscale^2 for YaRN with a
 * non-zero mscale_all_dim, where mscale = 0.1 * mscale_all_dim * ln(s) + 1 for
 * s > 1 ("CSDN walkthrough of HF DeepseekV3Attention", __init__, citing the
 * YaRN paper's equations 21-22; "Megatron-LM MLA guide", softmax_scale =
 * mscale * mscale / sqrt(q_head_dim)).  Returns cfg->softmax_scale when it is
 * positive.  Host-only.  Returns 0 for an invalid configuration. */
float mla_softmax_scale(const mla_config* cfg);

/* RoPE table, host-only: cos_out/sin_out are caller-owned HOST arrays of
 * max_pos * (d_rope/2) floats, row p = position p, column i = frequency i.
 * Angles are p * theta_i evaluated in double and rounded once to float.
 * Plain: theta_i = base^(-2i/d_rope).  YaRN ("Megatron-LM MLA guide",
 * rotary_base, scaling factor, original_max_position_embeddings, beta_fast,
 * beta_slow, mscale, mscale_all_dim): pairs turning more than beta_fast times
 * over the original context keep theta_i, pairs turning fewer than beta_slow
 * times use theta_i / s, linear ramp in the pair index between them; amplitude
 * mscale(s, mscale) / mscale(s, mscale_all_dim).  Upload the arrays to device
 * memory for the device calls.  MLA_ERR_INVALID_ARG for rope_kind NONE. */
mla_status mla_rope_table(const mla_config* cfg, int32_t max_pos, float* cos_out, float* sin_out);

/* Workspace (device bytes) needed by mla_prefill_fwd for num_tokens packed
 * tokens in num_seqs documents. */
size_t mla_prefill_workspace_size(const mla_config* cfg, int32_t num_tokens, int32_t num_seqs);

/* Workspace (device bytes) needed by mla_prefill_chunk_fwd; both arrays are
 * HOST arrays (cu_seqlens [num_seqs + 1], prefix_lens [num_seqs]). */
size_t mla_prefill_chunk_workspace_size(const mla_config* cfg, const int32_t* cu_seqlens_host,
                                        const int32_t* prefix_lens_host, int32_t num_seqs);

/* Workspace (device bytes) needed by mla_decode_absorbed_fwd; seq_lens_host
 * is a HOST array of batch lengths. */
size_t mla_decode_workspace_size(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch);

/* Workspace (device bytes) needed by mla_decode_absorbed_fp8_fwd (its split
 * works on tiles of 64 keys; the plan differs from the bf16 decode's). */
size_t mla_decode_fp8_workspace_size(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch);

const char* mla_status_string(mla_status s);
/* Message for the last failed call on this thread ("" if none). */
const char* mla_last_error(void);

/* -------------------------------------------------------------- device calls */

/* Fused latent RMSNorm + RoPE (+ optional paged scatter) over token rows.
 * Follows the latent path of "CSDN walkthrough of HF DeepseekV3Attention"
 * (kv_a_layernorm on the compressed part, RoPE on the single k_pe head) and the
 * fused rope-for-kv of "Megatron-LM MLA guide"; the same call applies RoPE in
 * place to the H rope slices of q (rope_slices = H).
 *   src  [n_rows, src_row_stride] (dtype), row r read from src + r*stride.
 *   For each row, columns [0, row_width) are written to the destination row:
 *     c <  norm_dim              : gamma[c] * x[c] / sqrt(mean(x[0:norm_dim]^2) + eps)
 *     c in a rope slice          : rotate_half RoPE at positions[r] ("MiniMind"
 *                                  section 3); slice s covers [rope_offset +
 *                                  s*rope_slice_stride, + d_rope)
 *     otherwise                  : copied.
 *   norm_dim = 0 disables the norm; rope_slices = 0 (or rope_kind NONE)
 *   disables RoPE.  rope_cos/rope_sin: DEVICE tables from mla_rope_table with
 *   rope_table_len rows; positions: DEVICE [n_rows] (may be NULL without RoPE);
 *   a position outside [0, rope_table_len) writes NaN into that row's slices.
 *   Destination: slot_mapping NULL -> dst + r*dst_row_stride; else DEVICE
 *   slot_mapping[r] gives the destination row (a paged-cache slot); rows with a
 *   slot < 0 or >= num_slots are skipped.  src == dst (in place) is allowed
 *   without a slot mapping. */
mla_status mla_latent_norm_rope(const mla_config* cfg,
                                const void* src, int64_t src_row_stride, int32_t n_rows,
                                int32_t row_width, int32_t norm_dim, const void* gamma,
                                int32_t rope_offset, int32_t rope_slices, int32_t rope_slice_stride,
                                const float* rope_cos, const float* rope_sin, int32_t rope_table_len,
                                const int32_t* positions,
                                void* dst, int64_t dst_row_stride,
                                const int32_t* slot_mapping, int64_t num_slots,
                                void* stream);

/* Linear layer y = x W^T (the nn.Linear projections of the layer).
 *   x [m, k] with row stride ldx, w [n, k] (row stride k), y [m, n] with row
 *   stride ldy; all DEVICE, dtype = cfg.dtype.  fp32 accumulation. */
mla_status mla_linear(const mla_config* cfg, const void* x, int64_t ldx, const void* w,
                      void* y, int64_t ldy, int32_t m, int32_t n, int32_t k, void* stream);

/* Causal varlen attention core of the layer (MLA step "A" above) on
 * already-projected tensors, all DEVICE:
 *   operand_dtype: type of q, kv and kpe: MLA_BF16 or MLA_F16 for a bf16
 *          config (the prefill layer itself keeps these operands in fp16),
 *          MLA_F32 for an fp32 config
 *   q      [N, H, d_nope + d_rope]  per head [q_nope | q_pe] (q_pe rotated)
 *   kv     [N, H, d_nope + d_v]     per head [k_nope | v]
 *   kpe    the shared rope key (rotated), ONE head broadcast to every head:
 *          row r at kpe + r * kpe_stride elements (for a latent-cache row
 *          buffer [N, r_kv + d_rope]: kpe = latent + r_kv, stride r_kv + d_rope)
 *   cu_seqlens_dev / cu_seqlens_host: [num_seqs + 1] offsets (DEVICE / HOST,
 *          same values), documents attend only within themselves, causally
 *          ("Megatron-LM MLA guide", THD packing)
 *   attn   [N, H, d_v] output, cfg.dtype (bf16 for both bf16 operand types).
 *          d_v != d_nope + d_rope is handled natively (no padding of v, unlike
 *          the FlashAttention adapters on the pages).
 *   lse    NULL, or DEVICE fp32 [H, N] receiving per (head, query) the
 *          base-2 log-sum-exp of the query's scores in base-2 units,
 *          log2 sum_j 2^(scale * log2(e) * q.k_j) over the keys it sees (the
 *          softmax denominator as the kernel formed it), for
 *          mla_attention_prefill_bwd; bf16 configs only (MLA_ERR_UNSUPPORTED
 *          for fp32)
 *   workspace may be NULL (no scratch is needed). */
mla_status mla_attention_prefill(const mla_config* cfg, int32_t operand_dtype, const void* q, const void* kv,
                                 const void* kpe, int64_t kpe_stride,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                 int32_t num_seqs, void* attn, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* The attention core for new queries over longer key sequences (a chunk of
 * new tokens over a cached prefix): document d has queries [cu_q[d],
 * cu_q[d+1]) and keys [cu_k[d], cu_k[d+1]), at least as many keys as
 * queries, aligned at the end, so query t of d sees the keys of d up to row
 * cu_k[d+1] - (cu_q[d+1] - t): every key before the document's queries and
 * the queries' own keys up to itself ("MiniMind: attention forward pass",
 * section 5, the mask with a cache).  cu_q == cu_k gives
 * mla_attention_prefill.  Operands and output as for mla_attention_prefill,
 * with kv and kpe indexed by key rows (cu_k_host[num_seqs] of them).
 * MLA_ERR_INVALID_ARG when a document has fewer keys than queries. */
mla_status mla_attention_prefix(const mla_config* cfg, int32_t operand_dtype, const void* q, const void* kv,
                                const void* kpe, int64_t kpe_stride,
                                const int32_t* cu_q_dev, const int32_t* cu_q_host,
                                const int32_t* cu_k_dev, const int32_t* cu_k_host,
                                int32_t num_seqs, void* attn, void* stream);

/* The full MLA prefill layer on packed documents.
 *   x [N, hidden] DEVICE; N = cu_seqlens_host[num_seqs].
 *   positions_dev: DEVICE [N] RoPE positions, or NULL for 0..len-1 within each
 *     document.
 *   rope_cos/rope_sin: DEVICE tables (mla_rope_table) with rope_table_len rows,
 *     NULL for rope_kind NONE.
 *   out [N, hidden] DEVICE (the attention output before any residual).
 *   latent_out: NULL, or DEVICE [N, r_kv + d_rope] receiving [c_n | k_pe'] per
 *     token, the latent-cache row ("Megatron-LM MLA guide", inference section).
 *   workspace: DEVICE, >= mla_prefill_workspace_size(cfg, N, num_seqs). */
mla_status mla_prefill_fwd(const mla_config* cfg, const mla_weights* w, const void* x,
                           const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                           int32_t num_seqs, const int32_t* positions_dev,
                           const float* rope_cos, const float* rope_sin, int32_t rope_table_len,
                           void* out, void* latent_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The MLA prefill layer for new tokens of sequences whose first tokens are
 * already in the paged latent cache (chunked prefill, mixed prefill/decode).
 * The cached latent rows are decompressed with the kv up-projection, as the
 * new tokens' are ("Megatron-LM MLA guide", inference section: prefill and
 * mixed steps decompress the cached latents; only decode-only steps absorb),
 * and new token i of sequence s, at position prefix_lens[s] + i, attends to
 * every cached token of s and to the new tokens of s up to itself (the mask of
 * a forward with a cache, "MiniMind: attention forward pass", section 5).
 *   x [N, hidden] DEVICE: the new tokens, packed by cu_seqlens (DEVICE / HOST,
 *     [num_seqs + 1], same values); N = cu_seqlens_host[num_seqs].
 *   prefix_lens_dev / prefix_lens_host: [num_seqs] cached tokens per sequence
 *     (DEVICE / HOST, same values, each >= 0; 0 = a plain causal prefill).
 *   kv_cache [num_blocks, block_size, r_kv + d_rope] in cfg.dtype, rows
 *     [c_n | k_pe'] as mla_latent_norm_rope / latent_out store them; cached
 *     token j of sequence s lives in slot block_table[s, j / block_size] *
 *     block_size + j % block_size.  block_table [num_seqs, max_blocks].
 *     May be NULL when every prefix is 0.  block_size: a power of two.
 *     A block id outside [0, num_blocks) makes that sequence's outputs NaN;
 *     slots past a prefix are never read.  The new tokens are NOT written to
 *     the cache: latent_out receives their rows for the caller to store.
 *   rope_cos/rope_sin: as for mla_prefill_fwd (positions up to the longest
 *     prefix + chunk must be in the table).
 *   out [N, hidden], latent_out NULL or [N, r_kv + d_rope], as for
 *     mla_prefill_fwd.
 *   workspace: DEVICE, >= mla_prefill_chunk_workspace_size(cfg, cu_seqlens_host,
 *     prefix_lens_host, num_seqs).
 * Errors: MLA_ERR_INVALID_ARG for a negative prefix, a prefix beyond
 * max_blocks * block_size, or missing cache arguments with a non-zero
 * prefix; MLA_ERR_UNSUPPORTED past 2^31 - 1 context rows. */
mla_status mla_prefill_chunk_fwd(const mla_config* cfg, const mla_weights* w, const void* x,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 const int32_t* prefix_lens_dev, const int32_t* prefix_lens_host,
                                 const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const float* rope_cos, const float* rope_sin, int32_t rope_table_len,
                                 void* out, void* latent_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Weight-absorbed MLA decode over a paged latent cache ("Megatron-LM MLA
 * guide", inference section: kv up-projection split per head into up_k and
 * up_v; up_k folded into the no-position query, attention over the cached
 * latents, up_v restoring d_v), bf16 only.
 *   w_kv_b   [H*(d_nope+d_v), r_kv]  rows of head h = [W_UK (d_nope rows) | W_UV (d_v rows)]
 *   q_nope   [B, H, d_nope], q_pe [B, H, d_rope] (already rotated)
 *   kv_cache [num_blocks, block_size, r_kv + d_rope]: per token [c_n | k_pe']
 *   block_table [B, max_blocks]: block ids; token j of sequence b lives in slot
 *            block_table[b, j / block_size] * block_size + j % block_size
 *   seq_lens_dev / seq_lens_host: [B] keys to attend, INCLUDING the current
 *            token (already written to the cache by the caller)
 *   out      [B, H, d_v]: attention output before the output projection.
 *   A block id outside [0, num_blocks) makes that sequence's output NaN; cache
 *   slots past seq_lens are never read.  block_size must be a power of two
 *   >= 16.
 *   workspace: DEVICE, >= mla_decode_workspace_size(cfg, seq_lens_host, B). */
mla_status mla_decode_absorbed_fwd(const mla_config* cfg, const void* w_kv_b,
                                   const void* q_nope, const void* q_pe,
                                   const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                                   int32_t batch, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode_absorbed_fwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, kernels and
 * results as mla_decode_absorbed_fwd; its scratch (absorbed query, partial
 * results) lives in a static device array of 64 MiB that every GPU the
 * library runs on holds for the life of the process.  The call allocates
 * nothing: its first call on a device only looks the array's address up.
 * A batch whose plan needs more scratch than that (mla_decode_workspace_size
 * > 64 MiB) returns MLA_ERR_WORKSPACE before anything is enqueued.  All calls
 * on one GPU share the array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give undefined results; calls ordered on one stream do not.  Nothing in the
 * array needs clearing between calls: each call writes every part it
 * reads. */
mla_status mla_decode_absorbed_fwd_noalloc(const mla_config* cfg, const void* w_kv_b,
                                           const void* q_nope, const void* q_pe,
                                           const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                           const int32_t* block_table, int32_t max_blocks,
                                           const int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                                           int32_t batch, void* out, void* stream);

/* ------------------------------------------------------------------- backward
 * Backward of the attention core of mla_attention_prefill ("Megatron-LM MLA
 * guide", training section: the layer is trained end to end; gradients reach
 * the query, the per-head k_nope and v of the latent and the one shared k_pe).
 * With S = scale [q_nope|q_pe] [k_nope|k_pe]^T per head, causal within each
 * document, P = softmax(S), O = P v and the output gradient dO:
 *   dv = P^T dO, dP = dO v^T, dS = P * (dP - rowsum(dO * O)),
 *   dq = scale dS k, dk = scale dS^T q, dk_pe = sum over heads of dk's rope part.
 * bf16 config and head shape only (d_nope 128, d_rope 64, d_v 128).
 *   q, kv, kpe, kpe_stride, cu_seqlens: the forward's bf16 operands, as for
 *          mla_attention_prefill (MLA_BF16 operands)
 *   out    [N, H, d_v] bf16, the forward's output for these operands; D =
 *          rowsum(dO * out) is formed from it as given
 *   lse    NULL, or DEVICE fp32 [H, N]: the log-sum-exp that
 *          mla_attention_prefill wrote for these operands (MLA_BF16); then
 *          the softmax statistics are taken from it instead of recomputed
 *   dout   [N, H, d_v] bf16, the gradient of the output
 *   dq     [N, H, d_nope + d_rope] fp32, dkv [N, H, d_nope + d_v] fp32
 *          (per head [dk_nope | dv]), dkpe [N, d_rope] fp32 — all DEVICE,
 *          16-byte aligned, written completely
 *   workspace: DEVICE, >= mla_attention_bwd_workspace_size(cfg, N) bytes.
 * Without lse the forward's softmax statistics are recomputed (one extra
 * QK^T pass); P and dS are rounded to bf16 as MFMA operands, accumulation is
 * fp32.
 * Errors: MLA_ERR_UNSUPPORTED for another dtype or head shape, more than
 * 65535 documents or a document longer than 65535 * 128 tokens;
 * MLA_ERR_INVALID_ARG for a missing pointer or bad offsets; MLA_ERR_MISALIGNED;
 * MLA_ERR_WORKSPACE for a missing or short workspace.  N = 0 is a no-op. */
size_t mla_attention_bwd_workspace_size(const mla_config* cfg, int32_t num_tokens);
mla_status mla_attention_prefill_bwd(const mla_config* cfg, const void* q, const void* kv, const void* kpe,
                                     int64_t kpe_stride, const int32_t* cu_seqlens_dev,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs, const void* out,
                                     const float* lse, const void* dout, void* dq, void* dkv, void* dkpe,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Gradients of the layer's weights (mla_prefill_bwd): fp32 DEVICE arrays of
 * the shapes of the mla_weights fields of the same name, 16-byte aligned;
 * those the configuration does not use are NULL. */
typedef struct mla_weight_grads {
  float* w_q_a;
  float* q_a_gamma;
  float* w_q_b;
  float* w_q;
  float* w_kv_a;
  float* kv_a_gamma;
  float* w_kv_b;
  float* w_o;
  float* w_g;
  float* w_o_a;
  float* w_o_b;
} mla_weight_grads;

/* Backward of the whole prefill layer ("Megatron-LM MLA guide", training
 * section: the layer is trained end to end, its weight gradients including
 * the ones backward_dw produces; the pages print no backward formulas, so it
 * is the chain rule through the forward of mla_prefill_fwd):
 *   output projection (plain or grouped low-rank): dW = dout^T A2, dA2;
 *   gate: dA = dA2 sigmoid(g), dg = dA2 A sigmoid(g) (1 - sigmoid(g)), dW_g;
 *   attention core: mla_attention_prefill_bwd;
 *   RoPE: the rotation by -theta of the q and k_pe gradients;
 *   kv up-projection: dW_kv_b = dkv^T c_n, dc_n = dkv W_kv_b (through the
 *     latent: every head's k_nope / v gradient reaches the one latent row);
 *   RMSNorm: dx = g dy / r - x mean(g dy x) / r^3, dgamma = sum_rows dy x / r;
 *   down-projections: dW = dY^T x, and dx = sum of dY W over the projections
 *     that read x.
 * The forward is recomputed inside the call (activation recomputation), with
 * bf16 attention operands whatever cfg->attn_operand says.  bf16 config only.
 *   w, x, cu_seqlens, positions, rope tables: as for mla_prefill_fwd
 *   dout   [N, hidden] bf16 DEVICE, the gradient of the layer output
 *   dx     [N, hidden] fp32 DEVICE, written (not accumulated)
 *   dw     the weight gradients (fp32, written, not accumulated)
 *   workspace: DEVICE, >= mla_prefill_bwd_workspace_size(cfg, N) bytes.
 * Gradients are fp32 sums of products of bf16 operands: every GEMM operand,
 * the attention's P and dS, and the gradients between the steps are rounded
 * to bf16 once.
 * Errors: MLA_ERR_UNSUPPORTED for an fp32 config or an unsupported head
 * shape; MLA_ERR_INVALID_ARG for a missing tensor (any weight gradient the
 * configuration uses included); MLA_ERR_MISALIGNED; MLA_ERR_WORKSPACE.  N = 0
 * is a no-op. */
size_t mla_prefill_bwd_workspace_size(const mla_config* cfg, int32_t num_tokens);
mla_status mla_prefill_bwd(const mla_config* cfg, const mla_weights* w, const void* x, const int32_t* cu_seqlens_dev,
                           const int32_t* cu_seqlens_host, int32_t num_seqs, const int32_t* positions_dev,
                           const float* rope_cos, const float* rope_sin, int32_t rope_table_len, const void* dout,
                           float* dx, const mla_weight_grads* dw, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---------------------------------------------------- FP8 (E4M3) latent cache
 * The pages name FP8 only as the MXFP8 recipe of "Megatron-LM MLA guide"
 * (parameter section: use_fused_mla_q_uproj, fp8_dot_product_attention) and
 * give no cache format.  The format here: each latent-cache row [c_n | k_pe']
 * stored as r_kv + d_rope codes of the OCP 8-bit floating point E4M3 type
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest
 * finite 448, S.1111.111 = NaN), with ONE float32 scale for the whole cache:
 * value = code * scale.  Half the bytes of the bf16 cache. */

/* Converts bf16 latent-cache rows to E4M3 codes:
 *   dst[r, c] = E4M3(fl32(src[r, c] * fl32(1 / scale)))
 * rounding to nearest, ties to even, magnitudes above 448 saturated to 448
 * (the OCP Microscaling conversion rule); a NaN gives a NaN code.
 *   src  DEVICE bf16 [n_rows, src_row_stride] (elements), 16-byte aligned
 *   dst  DEVICE uint8 [n_rows, dst_row_stride] (bytes), 8-byte aligned
 *   row_width, src_row_stride, dst_row_stride: multiples of 8
 *   (MLA_ERR_MISALIGNED otherwise), strides >= row_width.
 *   scale: positive and finite (MLA_ERR_INVALID_ARG otherwise).
 * Quantising a paged cache [num_blocks, block_size, 576] is one call with
 * n_rows = num_blocks * block_size and row_width = 576.  The layout is the
 * caller's: rows are converted where they are, slot for slot. */
mla_status mla_cache_quantize_fp8(const void* src, int64_t src_row_stride, int64_t n_rows, int32_t row_width,
                                  float scale, void* dst, int64_t dst_row_stride, void* stream);

/* The fused query up-projection of "Megatron-LM MLA guide" (parameter
 * section, use_fused_mla_q_uproj: query up-projection, per-head RoPE and MXFP8
 * quantisation in one kernel):
 *   q = q_latent W_qb^T viewed [N, H, d_nope + d_rope], the rope part of each
 *       head rotated at positions[t] (plain or YaRN tables, rotate_half or
 *       interleaved pairs as cfg says; no rotation for MLA_ROPE_NONE)
 *   quantised to MXFP8 along each row, blocks of 32 consecutive columns (a
 *   head of d_qk = 192 is 6 blocks), by the OCP Microscaling rule for E4M3:
 *   shared scale X = 2^(floor(log2 max|q_i|) - 8), elements E4M3(q_i / X),
 *   round to nearest even, saturating at 448; a zero block takes X = 2^-127.
 *   q_latent  DEVICE bf16 [N, ldq] (the normalised query latent, RMSNorm_q
 *             applied), 16-byte aligned, ldq a multiple of 8
 *   w_q_b     DEVICE bf16 [H * d_qk, q_lora_rank]
 *   positions DEVICE int32 [N]; rope_cos/rope_sin DEVICE tables of
 *             mla_rope_table with rope_table_len rows (unused for
 *             MLA_ROPE_NONE); a position outside the table gives NaN values
 *   q_codes   DEVICE uint8 [N, H * d_qk] E4M3 codes, 16-byte aligned
 *   q_scales  DEVICE uint8 [N, H * d_qk / 32] E8M0 bytes (exponent + 127),
 *             8-byte aligned
 * The product is accumulated in fp32 and rounded once, to MXFP8.  bf16
 * configs with a query latent (q_lora_rank > 0, a multiple of 32) and the
 * supported head shape only (MLA_ERR_INVALID_ARG / MLA_ERR_UNSUPPORTED). */
mla_status mla_q_uproj_rope_mxfp8(const mla_config* cfg, const void* q_latent, int64_t ldq, int32_t n_tokens,
                                  const void* w_q_b, const int32_t* positions, const float* rope_cos,
                                  const float* rope_sin, int32_t rope_table_len, void* q_codes, void* q_scales,
                                  void* stream);

/* mla_decode_absorbed_fwd over an E4M3 latent cache (same arguments, bf16
 * queries, weights and output; "Megatron-LM MLA guide", inference section, as
 * for the bf16 decode).  The result approximates the absorbed decode over the
 * dequantised cache (code * cache_scale): inside, the absorbed query and the
 * probabilities are rounded to MXFP8 (blocks of 32 values sharing a
 * power-of-two scale, E4M3 elements) and both contractions run on fp8 MFMAs
 * with fp32 accumulation.
 *   kv_cache_fp8 [num_blocks, block_size, r_kv + d_rope] uint8 codes (as
 *            mla_cache_quantize_fp8 writes them), 16-byte aligned
 *   cache_scale: the cache's scale, positive and finite
 *   workspace: DEVICE, >= mla_decode_fp8_workspace_size(cfg, seq_lens_host, B).
 * Other arguments, errors and guarantees as for mla_decode_absorbed_fwd. */
mla_status mla_decode_absorbed_fp8_fwd(const mla_config* cfg, const void* w_kv_b,
                                       const void* q_nope, const void* q_pe,
                                       const void* kv_cache_fp8, float cache_scale,
                                       int32_t num_blocks, int32_t block_size,
                                       const int32_t* block_table, int32_t max_blocks,
                                       const int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                                       int32_t batch, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMLA_MLA_H */
