// Internal declarations shared by the libmla HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <type_traits>

#include "mla.h"

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// MFMA wrappers (lane layouts checked on gfx950):
//  16x16x32: A lane l -> row l%16, k (l/16)*8+[0,8); B lane l -> col l%16, same k;
//            C lane l -> col l%16, rows (l/16)*4+[0,4).
//  32x32x16: A lane l -> row l%32, k (l/32)*8+[0,8); B lane l -> col l%32, same k;
//            C lane l -> col l%32, rows (i/4)*8 + (l/32)*4 + i%4, i in [0,16).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp16 operands, same lane layouts.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA with the accumulator held in VGPRs whatever form the
// compiler picks for the other MFMAs of the kernel (inline asm; the first of a
// chain starts from 0).  Back-to-back MFMAs accumulating into the same
// registers need no wait states; before the VALU reads the result, call
// mfma_result_wait().  The compiler does not see an MFMA in the asm, so it
// inserts no wait states between a VALU write of an operand (for instance a
// copy out of an AGPR it parked the operand in) and the MFMA's read of it:
// the asm carries them itself (they pass while the chain's previous MFMA is
// still running).
__device__ __forceinline__ void mfma32_vacc(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vacc0(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
// Wait states between an MFMA writing VGPRs and a VALU instruction reading them.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 15"); }

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// L supplies the address of 4 consecutive 16-bit elements ("row" L); the result
// of lane i is element i%4 of rows i/4, i/4+4, i/4+8, i/4+12.
// Used so that lane i of a group receives X[k0 + j][n0 + i], j = 0..3, from a
// row-major X[k][n] tile: lane L then addresses &X[k0 + L/4][n0 + 4*(L%4)].
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// A pointer the caller knows to be the same in every lane, moved to SGPRs.
template <typename T> __device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(MLA_LDS const void*)(p);
}

// Asynchronous global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4).
// The destination of lane l is lds_base + 16 * l; lds_base must be uniform
// across the wave.  Completion is awaited with vm_wait_all() before a barrier.
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (MLA_LDS void*)(lds_base), 16, 0, 0);
}
// The same copy issued from inline asm.  The compiler does not see it as an LDS
// write, so it inserts no wait for it before later LDS reads (it would wait for
// every outstanding copy, including ones into other buffers); the caller must
// order the copy against the reads of its destination itself, with
// vm_wait_all() / vm_wait_keep<N>() and a barrier.  The instruction has no
// register result.
__device__ __forceinline__ void lds_dma16_raw(const void* gsrc, const void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS const void*)(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(m) : "memory", "m0");
}
// As lds_dma16_raw, with the address split into a wave-uniform base (SGPR
// pair) and a per-lane 32-bit byte offset (the SADDR form), so moving a tile
// costs no per-lane address arithmetic.
__device__ __forceinline__ void lds_dma16_sv(const void* base, uint32_t off_bytes, const void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS const void*)(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off_bytes), "s"(base), "s"(m) : "memory", "m0");
}
// As lds_dma16_sv with the LDS destination given as a wave-uniform 32-bit LDS
// address (the M0 value).
__device__ __forceinline__ void lds_dma16_sv_m0(const void* base, uint32_t off_bytes, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off_bytes), "s"(base), "s"(lds_addr) : "memory", "m0");
}
// As lds_dma16_raw with the LDS destination given as a wave-uniform 32-bit
// LDS address.
__device__ __forceinline__ void lds_dma16_m0(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Wait until at most N vector-memory instructions are outstanding (gfx9
// s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at
// their maxima).  Loads complete in issue order, so this waits for all but the
// N most recent.
template <int N> __device__ __forceinline__ void vm_wait_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the release fence of __syncthreads() (which makes
// the compiler wait for every outstanding memory operation, in-flight LDS DMA
// included).  Callers wait for their own DMA explicitly and consume every LDS
// read before the barrier; the asm memory clobber keeps memory operations from
// moving across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Wait until this wave's LDS operations (stores included) have completed.
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp32 -> fp16 with values beyond the fp16 range saturated to +-65504 (a
// plain conversion would give +-inf); NaN stays NaN.
__device__ __forceinline__ f16 to_f16_sat(float v) {
  return (f16)(__builtin_fabsf(v) > 65504.f ? __builtin_copysignf(65504.f, v) : v);
}

// acc + sum of the 8 values of v, accumulated in fp32 (two-element dot
// products with (1, 1)): the sum of exactly the rounded values an MFMA takes
// as its operand.
__device__ __forceinline__ float sum8(f16x8 v, float acc) {
  const f16x2 one = {(f16)1.f, (f16)1.f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}
__device__ __forceinline__ float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// Calls f(std::integral_constant<int, i>) for i = B .. E - 1, so that the index
// is a constant expression in the body whatever the loop unroller decides.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- launchers
struct GemmArgs {
  const void* a; int64_t lda; int64_t a_bstride;   // A [m, k]
  const void* b; int64_t ldb; int64_t b_bstride;   // B [n, k] (NT) or [k, n] (NN)
  void* c; int64_t ldc; int64_t c_bstride;         // C [m, n]
  const void* gate_src; int64_t ldg;               // epilogue "gate": c = gate_src * sigmoid(acc)
  // epilogue "rope": columns [h*rope_head_stride + rope_off, + 64) of each head
  // are rotated at positions[m]: rotate_half pairs (i, i+32), or interleaved
  // pairs (2i, 2i+1) with rope_interleave
  const float* cos_t; const float* sin_t; int table_len; const int32_t* positions;
  int rope_head_stride; int rope_off; int rope_interleave;
  int m, n, k, batch;
  bool b_kn;                                       // true: B stored [k, n] (NN)
  bool c_f32;                                      // true: C stored as fp32
  bool c_f16;                                      // true: C stored as fp16
  int epilogue;                                    // EPI_*
  // MXFP8 output (after the epilogue): C holds E4M3 codes (ldc in bytes) and
  // c_scale one E8M0 byte per 32 consecutive columns of a row (row stride
  // ld_scale bytes); n a multiple of 32
  bool c_mx; void* c_scale; int64_t ld_scale;
  bool c_acc;                                      // fp32 C (128x128 kernel): C += result instead of C = result
  // both operands stored K-major, A [k, m] and B [k, n] (C = A^T B, the form
  // of a weight gradient dY^T X over tokens): the 256x256 kernel only, fp32
  // output, K a multiple of 32, m and n multiples of 8
  bool kmajor;
};
enum { EPI_STORE = 0, EPI_GATE = 1, EPI_ROPE = 2 };

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);

struct NormRopeArgs {
  const void* src; int64_t src_stride; int n_rows; int row_width;
  int norm_dim; const void* gamma; float eps;
  int rope_offset; int rope_slices; int rope_stride; int rope_dim;
  const float* cos_t; const float* sin_t; int table_len; const int32_t* positions;
  void* dst; int64_t dst_stride; const int32_t* slots; int64_t num_slots;
  f16* rope_aux; int64_t rope_aux_stride;          // optional fp16 copy of the rotated slice (one slice)
  int interleave;                                  // pairs (2i, 2i+1) instead of (i, i + d/2)
  int64_t src2_off;                                // non-zero: each source value is the sum of the
                                                   // elements at p and p + src2_off (two split-K partials)
};
// src/dst element types: bf16 -> bf16, fp32 -> fp32, or fp32 -> bf16 (src_f32 with bf16_io).
hipError_t launch_norm_rope(const NormRopeArgs& a, bool bf16_io, hipStream_t s, bool src_f32 = false);

// pos[t] = t - cu[d] (+ prefix[d] when prefix_dev is given) for t in document d.
hipError_t launch_positions(const int32_t* cu_dev, int num_seqs, int n_tokens, int32_t* pos, hipStream_t s,
                            const int32_t* prefix_dev = nullptr);

// A chunk over a cached prefix: context rows of sequence s are rows
// [cuk[s], cuk[s+1]) of ctx, its prefix[s] cached rows then its new rows.
struct ChunkGatherArgs {
  const int32_t* cu; const int32_t* prefix; const int32_t* cuk;
  const void* cache; const int32_t* block_table; int max_blocks; int num_blocks; int log2_block;
  const void* lat;                       // new rows [N, row_width]
  void* ctx;                             // [n_ctx, row_width]
  const f16* kpe16_new; f16* kpe16_ctx;  // fp16 rope keys (bf16 rows only; NULL otherwise)
  int row_width; int rope_dim; int n_ctx; int n_new;
};
hipError_t launch_chunk_offsets(const int32_t* cu_dev, const int32_t* prefix_dev, int num_seqs, int32_t* cuk,
                                hipStream_t s);
hipError_t launch_gather_context(const ChunkGatherArgs& g, bool bf16_rows, int max_ctx_len, int num_seqs,
                                 hipStream_t s);

struct FlashArgs {
  const void* q; const void* kv;
  const void* kpe; int64_t kpe_stride;             // shared rope key: row r at kpe + r * kpe_stride
  const int32_t* cu_dev; void* out;
  // Key rows of each document when they are not its query rows (a chunk over
  // a cached prefix): document d's keys are rows [cuk[d], cuk[d+1]) of kv and
  // kpe, aligned at the end, so query row t of d sees keys up to
  // t + cuk[d+1] - cu[d+1].  NULL: the keys are the query rows (causal).
  const int32_t* cuk_dev; int n_keys;
  int n_tokens; int heads; int nope; int rope; int dv; int kv_lora;
  float scale; int num_seqs;
  // optional [heads, n_tokens]: per (head, query) the base-2 log-sum-exp of
  // scale * q.k (m + log2 l of the softmax as formed), for a backward;
  // MFMA kernel, queries without a cached prefix
  float* lse_out;
};
// MFMA kernel (nope 128, rope 64, dv 128) with bf16 or fp16 operands (q, kv,
// kpe of that type); the output is bf16.  The tile plan is built from the host
// offsets inside.
// cuk_host: the key offsets when a.cuk_dev is set (for the plan), else NULL.
hipError_t launch_flash_mfma(const FlashArgs& a, bool f16_operands, const int32_t* cu_host, const int32_t* cuk_host,
                             int num_seqs, hipStream_t s);
hipError_t launch_flash_f32(const FlashArgs& a, hipStream_t s);

// Backward of the bf16 attention core (nope 128, rope 64, dv 128): bf16
// operands, fp32 gradients; lse / dsum / dkr are scratch.
struct AttnBwdArgs {
  const void* q; const void* kv; const void* kpe; int64_t kpe_stride;
  const void* o; const void* dout;
  const int32_t* cu_dev; int n_tokens; int heads; float scale;
  float* lse; float* dsum; float* dkr;                 // [H, N], [H, N], [N, H, 64]
  float* dq; float* dkv; float* dkpe;                  // [N, H, 192], [N, H, 256], [N, 64]
  bool lse_ready;   // lse holds the forward's values: no statistics pass, D formed in the dq pass
  // optional bf16 outputs replacing dq and dkv's [dk_nope | dv] (dkr and dkpe
  // stay fp32); dq16 has the rotary map undone on its rope dims when rope is set
  bf16* dq16 = nullptr; bf16* dkv16 = nullptr;
  const float* cos_t = nullptr; const float* sin_t = nullptr; const int32_t* positions = nullptr;
  int table_len = 0; bool rope = false; bool rope_interleave = false;
};
hipError_t launch_attention_bwd(const AttnBwdArgs& a, const int32_t* cu_host, int num_seqs, hipStream_t s);

// ---------------------------------------------------------------- layer backward helpers
// dst[c, r] = src[r, c] (bf16 or fp32 source, rounded to bf16), zero for
// rows <= r < rows_pad.
hipError_t launch_transpose_bf16(const void* src, bool src_f32, int64_t ld_src, int rows, int cols, bf16* dst,
                                 int64_t ld_dst, int rows_pad, hipStream_t s);
// a2 = a * sigmoid(g), and the gate's backward (dA, dg) from dA2; n elements, dense.
hipError_t launch_gate_fwd(const bf16* a, const float* g, bf16* a2, int64_t n, hipStream_t s);
hipError_t launch_gate_bwd(const float* da2, const bf16* a, const float* g, bf16* da, bf16* dg, int64_t n,
                           hipStream_t s);
struct RopeBackArgs {
  const float* src; int64_t ld_src; int n_rows; int width;
  bf16* dst; int64_t ld_dst;
  int rope_off; int rope_slices; int rope_stride; int rope_dim; int interleave;
  const float* cos_t; const float* sin_t; int table_len; const int32_t* positions;
};
// dst = bf16(src) with the rope columns rotated by -theta (no rotation with rope_slices = 0).
hipError_t launch_rope_back(const RopeBackArgs& a, hipStream_t s);
struct RmsNormBwdArgs {
  const float* x; int64_t ld_x;                    // the norm's fp32 input
  const float* dy; int64_t ld_dy;                  // gradient of its output
  const void* gamma; int n_rows; int width; float eps;
  bf16* dx; int64_t ld_dx;                         // gradient of its input
  float* rinv;                                     // [n_rows] 1 / r (scratch)
};
// out[i] = sum over s < splits of part[s * count + i] (count a multiple of 4,
// 16-byte aligned): the split-K partial products of a GEMM.
hipError_t launch_sum_partials(const float* part, int splits, int64_t count, float* out, hipStream_t s);
// dx and dgamma [width]; partials: (n_rows + 255) / 256 * width floats of scratch.
hipError_t launch_rms_norm_bwd(const RmsNormBwdArgs& a, float* partials, float* dgamma, hipStream_t s);

// Most paged-cache blocks one decode segment may span (its block ids are staged in LDS).
constexpr int kDecodeMaxChunkBlocks = 512;
// Placeholder keys ahead of each sequence in the decode work order: the work
// of one more segment for the workgroup that starts it, in keys.
constexpr int kDecodeSegmentCost = 256;

struct DecodeArgs {
  const bf16* qt;         // [B, H, 512] absorbed query
  const bf16* q_nope;     // [B, H, 128]
  const bf16* w_uk;       // W_UK of head h: rows [128] of 512 at w_uk + h * w_uv_hstride
  const bf16* q_pe;       // [B, H, 64]
  const bf16* cache;      // [num_blocks, block_size, 576]
  const int32_t* block_table; int max_blocks; int num_blocks; int log2_block;
  const int32_t* seq_lens;
  // Partial results, one entry per (workgroup g, sequence b) segment at index
  // g + b (injective: the workgroups that touch sequence b + 1 start at or
  // after the last one that touches b), so [num_items + B] entries:
  f16* part_o;            // [num_items + B, H, 512] partial outputs, normalised (O / l)
  float* part_ml;         // [num_items + B, H, 2] exponent origin and sum (sum 0: empty slot)
  const bf16* w_uv;       // W_UV of head h: rows [dv] of 512 at w_uv + h * w_uv_hstride
  int64_t w_uv_hstride;
  bf16* out;              // [B, H, dv]
  int dv;
  int batch; int heads;
  int quota;              // keys per workgroup of the concatenated key sequence (multiple of 32)
  int max_slots;          // most segments of one sequence (host plan)
  int num_items;          // workgroups of the split kernel
  float scale;
  // E4M3 latent cache (the fp8 decode): codes [num_blocks, block_size, 576],
  // value = code * cache_scale
  const uint8_t* cache8;
  float cache_scale;
};

hipError_t launch_decode_absorb_q(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_combine_unabsorb(const DecodeArgs& a, hipStream_t s);
// Split kernel of the decode over an E4M3 cache (64-key tiles, fp8 MFMAs);
// same partial-buffer contract as launch_decode_split.
hipError_t launch_decode_split_fp8(const DecodeArgs& a, hipStream_t s);

// bf16 rows -> E4M3 codes: dst = E4M3(fl32(x * inv)), saturating at +-448.
struct CacheQuantArgs {
  const bf16* src; int64_t src_stride;   // elements
  uint8_t* dst; int64_t dst_stride;      // bytes
  int64_t rows; int width;               // width: a multiple of 8
  float inv;
};
hipError_t launch_cache_quant_fp8(const CacheQuantArgs& a, hipStream_t s);

}  // namespace mla
