// Prefill of new tokens over a cached latent prefix: the per-sequence key
// offsets and the gather that lays out each sequence's context latent rows
// (its cached prefix from the paged pool, then its new rows) contiguously,
// so that the kv up-projection and the attention run over them as over a
// packed prefill batch.
//
// "Megatron-LM MLA guide", inference section: prefill and mixed steps
// decompress k/v from the cached latents with the kv up-projection (only
// decode-only steps take the absorbed form).  "MiniMind: attention forward
// pass", section 5: with a cache, the new queries see every cached key and the
// causal mask applies only inside the block of new tokens.
#include "mla_internal.hpp"

namespace mla {
namespace {

// cuk[s] = sum over i < s of (prefix[i] + cu[i+1] - cu[i]), s = 0 .. S: one
// wave, 64 sequences per step (inclusive scan by shuffles).
__global__ __launch_bounds__(64) void chunk_offsets_kernel(const int32_t* cu, const int32_t* prefix, int num_seqs,
                                                           int32_t* cuk) {
  const int lane = threadIdx.x;
  int base = 0;
  if (lane == 0) cuk[0] = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += 64) {
    const int s = s0 + lane;
    const int n = s < num_seqs ? max(0, prefix[s]) + max(0, cu[s + 1] - cu[s]) : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (s < num_seqs) cuk[s + 1] = base + incl;
    base += __shfl(incl, 63, 64);
  }
}

// Context rows of sequence blockIdx.y, rows [blockIdx.x * GR, + GR): row j < P
// is cached row j (pool slot table[j / bs] * bs + j % bs), row j >= P is new
// row cu[s] + j - P.  16-byte pieces, one per thread and step.  A block id
// outside the pool makes the row NaN (the sequence's outputs become NaN).
// With kpe16_ctx, the shared rope key of every row is also written in fp16:
// converted from the cached bf16 row, copied from kpe16_new for new rows.
// Every index is bounded by the buffer sizes the host planned with, whatever
// the device offsets hold.
constexpr int GR = 16;
template <typename T>
__global__ __launch_bounds__(256) void gather_context_kernel(ChunkGatherArgs g) {
  const int s = blockIdx.y, r0 = blockIdx.x * GR;
  const int cs = g.cuk[s], ce = g.cuk[s + 1];
  const int P = max(0, g.prefix[s]), a = g.cu[s];
  // new row of context row j (j >= P): a + j - P, valid inside [0, n_new)
  auto new_ok = [&](int j) { return a + j - P >= 0 && a + j - P < g.n_new; };
  const int len = min(ce, g.n_ctx) - cs;
  if (cs < 0 || r0 >= len) return;
  const int rows = min(GR, len - r0);
  const int lw = g.row_width, pieces = lw * (int)sizeof(T) / 16;
  const int bmask = (1 << g.log2_block) - 1;
  // block id of cached row j, -1 when outside the table or the pool
  auto block_of = [&](int j) -> int {
    const int e = j >> g.log2_block;
    if (e >= g.max_blocks) return -1;
    const int blk = g.block_table[(int64_t)s * g.max_blocks + e];
    return (blk < 0 || blk >= g.num_blocks) ? -1 : blk;
  };
  for (int i = threadIdx.x; i < rows * pieces; i += 256) {
    const int r = i / pieces, pc = i - r * pieces, j = r0 + r;
    const T* src = nullptr;
    if (j < P) {
      const int blk = block_of(j);
      if (blk >= 0) src = (const T*)g.cache + (((int64_t)blk << g.log2_block) + (j & bmask)) * lw;
    } else if (new_ok(j)) {
      src = (const T*)g.lat + (int64_t)(a + j - P) * lw;
    }
    const bool bad = src == nullptr;
    uint4 v;
    if (bad) {
      const uint32_t nan = sizeof(T) == 2 ? 0x7fc07fc0u : 0x7fc00000u;
      v = make_uint4(nan, nan, nan, nan);
    } else {
      v = ((const uint4*)src)[pc];
    }
    ((uint4*)((T*)g.ctx + (int64_t)(cs + j) * lw))[pc] = v;
  }
  if (g.kpe16_ctx) {
    const int dr = g.rope_dim;
    for (int i = threadIdx.x; i < rows * dr; i += 256) {
      const int r = i / dr, c = i - r * dr, j = r0 + r;
      f16 v = (f16)__builtin_nanf("");
      if (j < P) {
        const int blk = block_of(j);
        if (blk >= 0) {
          const bf16* row = (const bf16*)g.cache + (((int64_t)blk << g.log2_block) + (j & bmask)) * lw;
          v = to_f16_sat((float)row[lw - dr + c]);   // bf16 -> fp16, exact in fp16's normal range
        }
      } else if (new_ok(j)) {
        v = g.kpe16_new[(int64_t)(a + j - P) * dr + c];
      }
      g.kpe16_ctx[(int64_t)(cs + j) * dr + c] = v;
    }
  }
}

}  // namespace

hipError_t launch_chunk_offsets(const int32_t* cu_dev, const int32_t* prefix_dev, int num_seqs, int32_t* cuk,
                                hipStream_t s) {
  chunk_offsets_kernel<<<1, 64, 0, s>>>(cu_dev, prefix_dev, num_seqs, cuk);
  return hipGetLastError();
}

hipError_t launch_gather_context(const ChunkGatherArgs& g, bool bf16_rows, int max_ctx_len, int num_seqs,
                                 hipStream_t s) {
  if (max_ctx_len <= 0 || num_seqs <= 0) return hipSuccess;
  dim3 grid((max_ctx_len + GR - 1) / GR, num_seqs);
  if (bf16_rows) gather_context_kernel<bf16><<<grid, 256, 0, s>>>(g);
  else gather_context_kernel<float><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mla
