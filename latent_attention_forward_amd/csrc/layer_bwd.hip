// Element-wise and reduction kernels of the MLA layer's backward (bf16 layer).
// The projections' gradients are GEMMs (gemm.hip) and the attention's is
// attn_bwd.hip; what remains between them is here:
//   * transpose (+ fp32 -> bf16): the K-major operand of a weight gradient
//     dW = dY^T X, whose reduction runs over the tokens;
//   * the output gate: A2 = A sigmoid(g) and its backward
//     dA = dA2 sigmoid(g), dg = dA2 A sigmoid(g) (1 - sigmoid(g));
//   * RoPE's backward, the rotation by -theta (the forward's rotation with the
//     sine negated), fused with the fp32 -> bf16 rounding of the gradient;
//   * RMSNorm's backward y = g x / r, r = sqrt(mean(x^2) + eps):
//     dx = g dy / r - x mean(g dy x) / r^3, dg = sum over rows of dy x / r.
#include "mla_internal.hpp"

namespace mla {
namespace {

// ----------------------------------------------------------------------------- transpose
// dst[c, r] = src[r, c] for r < rows; dst[c, r] = 0 for rows <= r < rows_pad.
// 64 x 64 tiles through LDS (row pitch 65 words, so the column reads of the
// second half do not collide on a bank).
template <bool SRC_F32>
__global__ __launch_bounds__(256) void transpose_kernel(const void* src, int64_t ld_src, int rows, int cols,
                                                        bf16* dst, int64_t ld_dst, int rows_pad) {
  __shared__ float t[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    float v = 0.f;
    if (r < rows && c < cols)
      v = SRC_F32 ? ((const float*)src)[(int64_t)r * ld_src + c] : (float)((const bf16*)src)[(int64_t)r * ld_src + c];
    t[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) dst[(int64_t)c * ld_dst + r] = (bf16)t[tx][i];
  }
}

// bf16 source, 16-byte accesses: a 64 x 64 tile is read as rows of 8
// chunks of 16 bytes, kept in LDS with rows padded to 72 elements, and
// written as 8 chunks per output row (8 elements gathered down a column);
// cols, ld_src and ld_dst multiples of 8, rows_pad a multiple of 64,
// 16-byte aligned base addresses.
__global__ __launch_bounds__(256) void transpose_vec_kernel(const bf16* src, int64_t ld_src, int rows, int cols,
                                                            bf16* dst, int64_t ld_dst, int rows_pad) {
  __shared__ __attribute__((aligned(16))) bf16 t[64][72];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int seg = (threadIdx.x & 7) * 8, sub = threadIdx.x >> 3;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = sub + 32 * it;
    bf16x8 v = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    if (r0 + r < rows && c0 + seg < cols) v = *(const bf16x8*)(src + (int64_t)(r0 + r) * ld_src + c0 + seg);
    *(bf16x8*)&t[r][seg] = v;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int c = sub + 32 * it;
    if (c0 + c >= cols) continue;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = t[seg + e][c];
    *(bf16x8*)(dst + (int64_t)(c0 + c) * ld_dst + r0 + seg) = o;
  }
}

// ----------------------------------------------------------------------------- gate
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// a2 = bf16(a * sigmoid(g)) (the forward's gate epilogue, same arithmetic)
__global__ __launch_bounds__(256) void gate_fwd_kernel(const bf16* a, const float* g, bf16* a2, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  a2[i] = (bf16)((float)a[i] * sigmoid(g[i]));
}

__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* da2, const bf16* a, const float* g, bf16* da,
                                                       bf16* dg, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float s = sigmoid(g[i]), d = da2[i];
  da[i] = (bf16)(d * s);
  dg[i] = (bf16)(d * (float)a[i] * s * (1.f - s));
}

// ----------------------------------------------------------------------------- RoPE backward
// One thread per element of an [n_rows, width] fp32 source; the columns
// [rope_off + j * rope_stride, + rope_dim) of a row (j < rope_slices) are
// rotated by -theta at positions[row]: with the forward's tables c, s
// (amplitude included), pair (a, b) = (i, i + d/2) or (2i, 2i + 1):
//   dx_a = dy_a c_i + dy_b s_i,  dx_b = dy_b c_i - dy_a s_i.
// A position outside the table gives NaN in the rotated columns.
__global__ __launch_bounds__(256) void rope_back_kernel(RopeBackArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_rows * a.width) return;
  const int64_t row = i / a.width;
  const int col = (int)(i - row * a.width);
  const float* src = a.src + row * a.ld_src;
  float v = src[col];
  const int rel = col - a.rope_off;
  if (a.rope_slices > 0 && rel >= 0) {
    const int slice = rel / a.rope_stride, j = rel - slice * a.rope_stride;
    if (slice < a.rope_slices && j < a.rope_dim) {
      const int half = a.rope_dim / 2;
      const int base = col - j;
      int pi, partner;
      bool first;
      if (a.interleave) { pi = j >> 1; first = (j & 1) == 0; partner = base + (j ^ 1); }
      else { pi = j < half ? j : j - half; first = j < half; partner = base + (first ? j + half : j - half); }
      const int pos = a.positions[row];
      float c = __builtin_nanf(""), s = __builtin_nanf("");
      if (pos >= 0 && pos < a.table_len) { c = a.cos_t[(int64_t)pos * half + pi]; s = a.sin_t[(int64_t)pos * half + pi]; }
      const float p = src[partner];
      v = first ? v * c + p * s : v * c - p * s;
    }
  }
  a.dst[row * a.ld_dst + col] = (bf16)v;
}

// The same on 8-element chunks (one thread per chunk: two 16-byte loads, one
// 16-byte store; a rope chunk also loads its partner chunk), for widths, row
// strides, rope offsets, strides and halves that are multiples of 8 and
// 16-byte aligned rows.
__global__ __launch_bounds__(256) void rope_back_vec_kernel(RopeBackArgs a) {
  const int nch = a.width >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_rows * nch) return;
  const int64_t row = i / nch;
  const int ch = (int)(i - row * nch), col = ch * 8;
  const float* src = a.src + row * a.ld_src;
  const float4 v0 = *(const float4*)(src + col), v1 = *(const float4*)(src + col + 4);
  float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const int rel = col - a.rope_off;
  if (a.rope_slices > 0 && rel >= 0) {
    const int slice = rel / a.rope_stride, j0 = rel - slice * a.rope_stride;
    if (slice < a.rope_slices && j0 < a.rope_dim) {
      const int half = a.rope_dim / 2;
      const int pos = a.positions[row];
      const bool ok = pos >= 0 && pos < a.table_len;
      const float* ct = a.cos_t + (int64_t)(ok ? pos : 0) * half;
      const float* st = a.sin_t + (int64_t)(ok ? pos : 0) * half;
      const float nan = __builtin_nanf("");
      float y[8];
      if (a.interleave) {
        // pairs (2i, 2i + 1) inside the chunk, i = j0/2 .. j0/2 + 3
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int pi = (j0 + e) >> 1;
          const float c = ok ? ct[pi] : nan, sn = ok ? st[pi] : nan;
          y[e] = v[e] * c + v[e + 1] * sn;
          y[e + 1] = v[e + 1] * c - v[e] * sn;
        }
      } else {
        // pairs (i, i + half): the partner chunk is half away
        const bool first = j0 < half;
        const int pi0 = first ? j0 : j0 - half;
        const float* pp = src + col + (first ? half : -half);
        const float4 p0 = *(const float4*)pp, p1 = *(const float4*)(pp + 4);
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = ok ? ct[pi0 + e] : nan, sn = ok ? st[pi0 + e] : nan;
          y[e] = first ? v[e] * c + pv[e] * sn : v[e] * c - pv[e] * sn;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = y[e];
    }
  }
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
  *(bf16x8*)(a.dst + row * a.ld_dst + col) = o;
}

// ----------------------------------------------------------------------------- RMSNorm backward
// One wave per row of width <= 64 * 32: x, dy fp32, gamma bf16 -> dx bf16 and
// 1 / r for the gain's gradient.
__global__ __launch_bounds__(256) void rms_norm_bwd_kernel(RmsNormBwdArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.n_rows) return;
  const float* x = a.x + (int64_t)row * a.ld_x;
  const float* dy = a.dy + (int64_t)row * a.ld_dy;
  float ss = 0.f, sgx = 0.f;
  for (int c = lane; c < a.width; c += 64) {
    const float xv = x[c], gd = (float)((const bf16*)a.gamma)[c] * dy[c];
    ss += xv * xv;
    sgx += gd * xv;
  }
  ss = wave_sum(ss);
  sgx = wave_sum(sgx);
  const float rinv = 1.f / __builtin_sqrtf(ss / (float)a.width + a.eps);
  const float k = sgx / (float)a.width * rinv * rinv * rinv;
  bf16* dx = a.dx + (int64_t)row * a.ld_dx;
  for (int c = lane; c < a.width; c += 64) dx[c] = (bf16)((float)((const bf16*)a.gamma)[c] * dy[c] * rinv - x[c] * k);
  if (lane == 0) a.rinv[row] = rinv;
}

// Partial sums over row chunks of 256: part[chunk, c] = sum_r dy[r, c] x[r, c] rinv[r].
__global__ __launch_bounds__(256) void dgamma_partial_kernel(RmsNormBwdArgs a, float* part) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), w = threadIdx.x >> 6;
  const int r0 = blockIdx.y * 256, r1 = min(r0 + 256, a.n_rows);
  float s = 0.f;
  if (c < a.width)
    for (int r = r0 + w; r < r1; r += 4) s += a.dy[(int64_t)r * a.ld_dy + c] * a.x[(int64_t)r * a.ld_x + c] * a.rinv[r];
  red[w][threadIdx.x & 63] = s;
  __syncthreads();
  if (w == 0 && c < a.width) part[(int64_t)blockIdx.y * a.width + c] = red[0][threadIdx.x] + red[1][threadIdx.x] +
                                                                        red[2][threadIdx.x] + red[3][threadIdx.x];
}

__global__ __launch_bounds__(256) void dgamma_sum_kernel(const float* part, int chunks, int width, float* dgamma) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= width) return;
  float s = 0.f;
  for (int k = 0; k < chunks; ++k) s += part[(int64_t)k * width + c];
  dgamma[c] = s;
}

// out[i] = sum over s of part[s * count + i], four floats per thread
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* part, int splits, int64_t count, float* out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  float4 acc = *(const float4*)(part + i);
  for (int sp = 1; sp < splits; ++sp) {
    const float4 v = *(const float4*)(part + (int64_t)sp * count + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *(float4*)(out + i) = acc;
}

}  // namespace

hipError_t launch_sum_partials(const float* part, int splits, int64_t count, float* out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (count % 4) return hipErrorInvalidValue;
  sum_partials_kernel<<<(unsigned)((count / 4 + 255) / 256), 256, 0, s>>>(part, splits, count, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* src, bool src_f32, int64_t ld_src, int rows, int cols, bf16* dst,
                                 int64_t ld_dst, int rows_pad, hipStream_t s) {
  if (cols <= 0 || rows_pad <= 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows_pad + 63) / 64));
  if (!src_f32 && cols % 8 == 0 && ld_src % 8 == 0 && ld_dst % 8 == 0 && rows_pad % 64 == 0 &&
      (reinterpret_cast<uintptr_t>(src) % 16) == 0 && (reinterpret_cast<uintptr_t>(dst) % 16) == 0) {
    transpose_vec_kernel<<<grid, 256, 0, s>>>((const bf16*)src, ld_src, rows, cols, dst, ld_dst, rows_pad);
    return hipGetLastError();
  }
  if (src_f32) transpose_kernel<true><<<grid, 256, 0, s>>>(src, ld_src, rows, cols, dst, ld_dst, rows_pad);
  else transpose_kernel<false><<<grid, 256, 0, s>>>(src, ld_src, rows, cols, dst, ld_dst, rows_pad);
  return hipGetLastError();
}

hipError_t launch_gate_fwd(const bf16* a, const float* g, bf16* a2, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  gate_fwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, g, a2, n);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float* da2, const bf16* a, const float* g, bf16* da, bf16* dg, int64_t n,
                           hipStream_t s) {
  if (n <= 0) return hipSuccess;
  gate_bwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(da2, a, g, da, dg, n);
  return hipGetLastError();
}

hipError_t launch_rope_back(const RopeBackArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_rows * a.width;
  if (n <= 0) return hipSuccess;
  const bool rope = a.rope_slices > 0;
  const bool vec = a.width % 8 == 0 && a.ld_src % 8 == 0 && a.ld_dst % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.src) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.dst) % 16) == 0 &&
                   (!rope || (a.rope_off % 8 == 0 && a.rope_stride % 8 == 0 && a.rope_dim % 16 == 0));
  if (vec) {
    const int64_t nc = n / 8;
    rope_back_vec_kernel<<<(unsigned)((nc + 255) / 256), 256, 0, s>>>(a);
  } else {
    rope_back_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_rms_norm_bwd(const RmsNormBwdArgs& a, float* partials, float* dgamma, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  rms_norm_bwd_kernel<<<(unsigned)((a.n_rows + 3) / 4), 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunks = (a.n_rows + 255) / 256;
  dgamma_partial_kernel<<<dim3((unsigned)((a.width + 63) / 64), (unsigned)chunks), 256, 0, s>>>(a, partials);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dgamma_sum_kernel<<<(unsigned)((a.width + 255) / 256), 256, 0, s>>>(partials, chunks, a.width, dgamma);
  return hipGetLastError();
}

}  // namespace mla
