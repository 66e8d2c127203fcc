// Fused latent RMSNorm + RoPE (+ paged scatter) over token rows, and the
// per-document position helper.
//
// One wavefront per row.  The sum of squares is accumulated in fp32 and reduced
// across the wavefront with butterfly shuffles; each element is then scaled once
// and rounded once.  RoPE pairs (i, i + d/2) of every slice are handled by one
// lane each, so an in-place update never races.  HBM-bound: every element is
// read once and written once.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int ROWS_PER_BLOCK = 4;

template <typename TS, typename T>
__global__ __launch_bounds__(64 * ROWS_PER_BLOCK) void norm_rope_kernel(NormRopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  int64_t drow = row;
  if (a.slots) {
    const int64_t s = a.slots[row];
    if (s < 0 || s >= a.num_slots) return;
    drow = s;
  }
  const TS* src = (const TS*)a.src + (int64_t)row * a.src_stride;
  T* dst = (T*)a.dst + drow * a.dst_stride;

  float rinv = 1.f;
  if (a.norm_dim > 0) {
    float ss = 0.f;
    if (sizeof(TS) == 2 && (a.norm_dim & 7) == 0 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
      for (int c = lane * 8; c < a.norm_dim; c += 64 * 8) {
        const bf16x8 v = *(const bf16x8*)(src + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float f = (float)v[e]; ss = fmaf(f, f, ss); }
      }
    } else {
      for (int c = lane; c < a.norm_dim; c += 64) { const float f = to_f32(src[c]); ss = fmaf(f, f, ss); }
    }
    ss = wave_sum(ss);
    rinv = rsqrtf(ss / (float)a.norm_dim + a.eps);
  }
  const int half = a.rope_dim >> 1;
  const bool do_rope = a.rope_slices > 0 && half > 0;
  auto in_rope = [&](int c) {
    if (!do_rope || c < a.rope_offset) return false;
    const int rel = c - a.rope_offset;
    const int s = rel / a.rope_stride;
    return s < a.rope_slices && (rel - s * a.rope_stride) < a.rope_dim;
  };
  // normalised / copied columns
  for (int c = lane; c < a.row_width; c += 64) {
    if (in_rope(c)) continue;
    float v = to_f32(src[c]);
    if (c < a.norm_dim) v = v * rinv * to_f32(((const T*)a.gamma)[c]);   // gain has the output dtype
    dst[c] = from_f32<T>(v);
    if (a.rope_aux && c >= a.rope_offset && c < a.rope_offset + a.rope_dim)   // unrotated shared part
      a.rope_aux[(int64_t)row * a.rope_aux_stride + (c - a.rope_offset)] = (f16)v;
  }
  if (!do_rope) return;
  const int pos = a.positions ? a.positions[row] : 0;
  const bool pos_ok = pos >= 0 && pos < a.table_len;
  const int pairs = a.rope_slices * half;
  for (int p = lane; p < pairs; p += 64) {
    const int s = p / half, i = p - s * half;
    // pair (i, i + half), or (2i, 2i + 1) for interleaved pairs
    const int l0 = a.interleave ? 2 * i : i, l1 = a.interleave ? 2 * i + 1 : i + half;
    const int c0 = a.rope_offset + s * a.rope_stride + l0, c1 = a.rope_offset + s * a.rope_stride + l1;
    const float x0 = to_f32(src[c0]), x1 = to_f32(src[c1]);
    float y0, y1;
    if (pos_ok) {
      const float cs = a.cos_t[(int64_t)pos * half + i], sn = a.sin_t[(int64_t)pos * half + i];
      y0 = x0 * cs - x1 * sn;
      y1 = x1 * cs + x0 * sn;
    } else {
      y0 = y1 = __builtin_nanf("");
    }
    dst[c0] = from_f32<T>(y0);
    dst[c1] = from_f32<T>(y1);
    if (a.rope_aux) {   // fp16 copy of the rotated slice, rounded once from fp32
      f16* aux = a.rope_aux + (int64_t)row * a.rope_aux_stride + (int64_t)s * a.rope_dim;
      aux[l0] = (f16)y0;
      aux[l1] = (f16)y1;
    }
  }
}

// positions[t] = t - start of t's document, one thread per token.
__global__ void positions_kernel(const int32_t* cu, int num_seqs, int n, int32_t* pos, const int32_t* prefix) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  int lo = 0, hi = num_seqs;       // find d with cu[d] <= t < cu[d+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  pos[t] = t - cu[lo] + (prefix ? prefix[lo] : 0);
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a, bool bf16_io, hipStream_t s, bool src_f32) {
  if (a.n_rows <= 0) return hipSuccess;
  const int blocks = (a.n_rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (bf16_io && src_f32)
    norm_rope_kernel<float, bf16><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
  else if (bf16_io)
    norm_rope_kernel<bf16, bf16><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
  else
    norm_rope_kernel<float, float><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_positions(const int32_t* cu_dev, int num_seqs, int n_tokens, int32_t* pos, hipStream_t s,
                            const int32_t* prefix_dev) {
  if (n_tokens <= 0) return hipSuccess;
  positions_kernel<<<(n_tokens + 255) / 256, 256, 0, s>>>(cu_dev, num_seqs, n_tokens, pos, prefix_dev);
  return hipGetLastError();
}

}  // namespace mla
