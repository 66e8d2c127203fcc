// Fused latent RMSNorm + RoPE (+ paged scatter) over token rows, and the
// per-document position helper.
//
// One wavefront per row.  The sum of squares is accumulated in fp32 and reduced
// across the wavefront with butterfly shuffles; each element is then scaled once
// and rounded once.  RoPE pairs (i, i + d/2) of every slice are handled by one
// lane each, so an in-place update never races.  HBM-bound: every element is
// read once from HBM and written once.  Rows whose layout allows it take the
// 8-element-chunk kernel; the element-wise kernel covers the rest.
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
  // source value c (the sum of two split-K partials when src2_off is set)
  auto ld = [&](int c) { return a.src2_off ? to_f32(src[c]) + to_f32(src[c + a.src2_off]) : to_f32(src[c]); };

  float rinv = 1.f;
  if (a.norm_dim > 0) {
    float ss = 0.f;
    if (sizeof(TS) == 2 && !a.src2_off && (a.norm_dim & 7) == 0 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
      for (int c = lane * 8; c < a.norm_dim; c += 64 * 8) {
        const bf16x8 v = *(const bf16x8*)(src + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float f = (float)v[e]; ss = fmaf(f, f, ss); }
      }
    } else {
      for (int c = lane; c < a.norm_dim; c += 64) { const float f = ld(c); ss = fmaf(f, f, ss); }
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
    float v = ld(c);
    if (c < a.norm_dim) v = v * rinv * to_f32(((const T*)a.gamma)[c]);   // gain has the output dtype
    dst[c] = from_f32<T>(v);
    if (a.rope_aux && c >= a.rope_offset && c < a.rope_offset + a.rope_dim)   // unrotated shared part
      a.rope_aux[(int64_t)row * a.rope_aux_stride + (c - a.rope_offset)] = to_f16_sat(v);
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
    const float x0 = ld(c0), x1 = ld(c1);
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
      aux[l0] = to_f16_sat(y0);
      aux[l1] = to_f16_sat(y1);
    }
  }
}

// The same operation with 8-element chunks (16 or 32 bytes) per lane access,
// for rows whose column splits (norm_dim, rope offset / stride / width) and
// addresses are multiples of 8 elements, which is every call the layer makes.
// Pass 1 sums the squares of the normalised chunks; pass 2 writes every
// chunk outside the rope slices (scaled or copied; the row is then in the
// cache); pass 3 rotates the rope slices, one lane per pair of chunks: for
// rotate_half the chunk at i and the one at i + d/2, for interleaved pairs
// one chunk holding four pairs.  A lane reads everything it writes before
// writing, and no two lanes write one chunk, so in-place updates are safe.
template <typename TS>
__device__ __forceinline__ void load8f(const TS* p, float (&v)[8]) {
  if constexpr (sizeof(TS) == 4) {
    const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
  }
}
// A source chunk: 8 values at p, plus the 8 at p + src2_off when the source
// is two split-K partials.
template <typename TS>
__device__ __forceinline__ void load8src(const NormRopeArgs& a, const TS* p, float (&v)[8]) {
  load8f(p, v);
  if (a.src2_off) {
    float t[8];
    load8f(p + a.src2_off, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += t[e];
  }
}
template <typename T>
__device__ __forceinline__ void store8f(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    ((float4*)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    ((float4*)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)v[e];
    *(bf16x8*)p = a;
  }
}
__device__ __forceinline__ void store8_f16(f16* p, const float (&v)[8]) {
  f16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = to_f16_sat(v[e]);
  *(f16x8*)p = a;
}

template <typename TS, typename T>
__global__ __launch_bounds__(64 * ROWS_PER_BLOCK) void norm_rope_vec_kernel(NormRopeArgs a) {
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
  const int nch = a.row_width >> 3, nnorm = a.norm_dim >> 3;
  const bool do_rope = a.rope_slices > 0 && a.rope_dim > 0;
  const int rch0 = a.rope_offset >> 3, rstride = a.rope_stride >> 3, rwidth = a.rope_dim >> 3;
  // chunk ch lies in a rope slice
  auto in_rope = [&](int ch) {
    if (!do_rope || ch < rch0) return false;
    const int rel = ch - rch0, s = rel / rstride;
    return s < a.rope_slices && rel - s * rstride < rwidth;
  };
  float rinv = 1.f;
  if (nnorm > 0) {
    float ss = 0.f;
    for (int ch = lane; ch < nnorm; ch += 64) {
      float v[8];
      load8src(a, src + ch * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    }
    ss = wave_sum(ss);
    rinv = rsqrtf(ss / (float)a.norm_dim + a.eps);
  }
  f16* aux = a.rope_aux ? a.rope_aux + (int64_t)row * a.rope_aux_stride : nullptr;
  for (int ch = lane; ch < nch; ch += 64) {
    if (in_rope(ch)) continue;
    float v[8];
    load8src(a, src + ch * 8, v);
    if (ch < nnorm) {
      float g[8];
      load8f((const T*)a.gamma + ch * 8, g);    // the gain has the output dtype
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * rinv * g[e];
    }
    store8f(dst + ch * 8, v);
    if (aux && ch >= rch0 && ch < rch0 + rwidth) store8_f16(aux + (ch - rch0) * 8, v);   // unrotated shared part
  }
  if (!do_rope) return;
  const int pos = a.positions ? a.positions[row] : 0;
  const bool pos_ok = pos >= 0 && pos < a.table_len;
  const int half = a.rope_dim >> 1;
  const float* cs_row = a.cos_t + (int64_t)(pos_ok ? pos : 0) * half;
  const float* sn_row = a.sin_t + (int64_t)(pos_ok ? pos : 0) * half;
  const float nan = __builtin_nanf("");
  if (!a.interleave) {
    // pair chunk j of a slice: elements 8j .. 8j + 7 with their partners d/2 later
    const int per = half >> 3;
    for (int p = lane; p < a.rope_slices * per; p += 64) {
      const int s = p / per, j = p - s * per;
      const int c0 = a.rope_offset + s * a.rope_stride + 8 * j, c1 = c0 + half;
      float x0[8], x1[8], cs[8], sn[8];
      load8src(a, src + c0, x0);
      load8src(a, src + c1, x1);
      load8f(cs_row + 8 * j, cs);
      load8f(sn_row + 8 * j, sn);
      float y0[8], y1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y0[e] = pos_ok ? x0[e] * cs[e] - x1[e] * sn[e] : nan;
        y1[e] = pos_ok ? x1[e] * cs[e] + x0[e] * sn[e] : nan;
      }
      store8f(dst + c0, y0);
      store8f(dst + c1, y1);
      if (aux) {          // fp16 copy of the rotated slice, rounded once from fp32
        store8_f16(aux + s * a.rope_dim + 8 * j, y0);
        store8_f16(aux + s * a.rope_dim + 8 * j + half, y1);
      }
    }
  } else {
    // chunk j of a slice holds pairs (2i, 2i + 1), i = 4j .. 4j + 3
    const int per = a.rope_dim >> 3;
    for (int p = lane; p < a.rope_slices * per; p += 64) {
      const int s = p / per, j = p - s * per;
      const int c0 = a.rope_offset + s * a.rope_stride + 8 * j;
      float x[8], y[8];
      load8src(a, src + c0, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = pos_ok ? cs_row[4 * j + e] : nan, sv = pos_ok ? sn_row[4 * j + e] : nan;
        y[2 * e] = x[2 * e] * c - x[2 * e + 1] * sv;
        y[2 * e + 1] = x[2 * e + 1] * c + x[2 * e] * sv;
      }
      store8f(dst + c0, y);
      if (aux) store8_f16(aux + s * a.rope_dim + 8 * j, y);
    }
  }
}

// The 8-element-chunk operation with the whole row in registers: lane l
// holds chunks l, l + 64, ... (up to NPL of them) and, for rotate_half RoPE,
// the rope pair chunks l, l + 64, ... (up to RPL of them); every load (row
// chunks, gains, rope chunk pairs, cos/sin) is issued before the sum of
// squares is reduced, so a row costs one memory round trip.  Rows up to
// 512 * NPL elements with at most 64 * RPL rope pair chunks.
template <typename TS, typename T, int NPL, int RPL>
__global__ __launch_bounds__(64 * ROWS_PER_BLOCK) void norm_rope_reg_kernel(NormRopeArgs a) {
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
  const int nch = a.row_width >> 3, nnorm = a.norm_dim >> 3;
  const bool do_rope = a.rope_slices > 0 && a.rope_dim > 0;
  const int rch0 = a.rope_offset >> 3, rstride = a.rope_stride >> 3, rwidth = a.rope_dim >> 3;
  auto in_rope = [&](int ch) {
    if (!do_rope || ch < rch0) return false;
    const int rel = ch - rch0, s = rel / rstride;
    return s < a.rope_slices && rel - s * rstride < rwidth;
  };
  // row chunks outside the rope slices, and their gains
  float v[NPL][8], g[NPL][8];
  bool own[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int ch = lane + 64 * i;
    own[i] = ch < nch && !in_rope(ch);
    if (own[i]) {
      load8src(a, src + ch * 8, v[i]);
      if (ch < nnorm) load8f((const T*)a.gamma + ch * 8, g[i]);   // the gain has the output dtype
    }
  }
  // rope pair chunks (rotate_half: chunk j of a slice with its partner d/2 later)
  const int half = a.rope_dim >> 1, per = half >> 3;
  const int pos = do_rope && a.positions ? a.positions[row] : 0;
  const bool pos_ok = pos >= 0 && pos < a.table_len;
  float x0[RPL][8], x1[RPL][8], cs[RPL][8], sn[RPL][8];
  bool rp[RPL];
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int p = lane + 64 * j;
    rp[j] = do_rope && p < a.rope_slices * per;
    if (rp[j]) {
      const int s = p / per, jj = p - s * per;
      const int c0 = a.rope_offset + s * a.rope_stride + 8 * jj;
      load8src(a, src + c0, x0[j]);
      load8src(a, src + c0 + half, x1[j]);
      const int64_t trow = (int64_t)(pos_ok ? pos : 0) * half + 8 * jj;
      load8f(a.cos_t + trow, cs[j]);
      load8f(a.sin_t + trow, sn[j]);
    }
  }
  float rinv = 1.f;
  if (nnorm > 0) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (own[i] && lane + 64 * i < nnorm)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[i][e], v[i][e], ss);
    ss = wave_sum(ss);
    rinv = rsqrtf(ss / (float)a.norm_dim + a.eps);
  }
  f16* aux = a.rope_aux ? a.rope_aux + (int64_t)row * a.rope_aux_stride : nullptr;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int ch = lane + 64 * i;
    if (!own[i]) continue;
    if (ch < nnorm)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = v[i][e] * rinv * g[i][e];
    store8f(dst + ch * 8, v[i]);
    if (aux && ch >= rch0 && ch < rch0 + rwidth) store8_f16(aux + (ch - rch0) * 8, v[i]);   // unrotated shared part
  }
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    if (!rp[j]) continue;
    const int p = lane + 64 * j, s = p / per, jj = p - s * per;
    const int c0 = a.rope_offset + s * a.rope_stride + 8 * jj;
    float y0[8], y1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y0[e] = pos_ok ? x0[j][e] * cs[j][e] - x1[j][e] * sn[j][e] : nan;
      y1[e] = pos_ok ? x1[j][e] * cs[j][e] + x0[j][e] * sn[j][e] : nan;
    }
    store8f(dst + c0, y0);
    store8f(dst + c0 + half, y1);
    if (aux) {            // fp16 copy of the rotated slice, rounded once from fp32
      store8_f16(aux + s * a.rope_dim + 8 * jj, y0);
      store8_f16(aux + s * a.rope_dim + 8 * jj + half, y1);
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
  // 8-element chunks: every column split, row stride and base address a
  // multiple of 8 elements (16-byte aligned), a rope width split into halves
  // of whole chunks, and a table row of whole chunks
  const bool rope = a.rope_slices > 0 && a.rope_dim > 0;
  const bool vec = (a.row_width % 8) == 0 && (a.norm_dim % 8) == 0 && (a.src_stride % 8) == 0 &&
                   (a.dst_stride % 8) == 0 && (reinterpret_cast<uintptr_t>(a.src) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.dst) % 16) == 0 &&
                   (!a.gamma || (reinterpret_cast<uintptr_t>(a.gamma) % 16) == 0) &&
                   (!rope || ((a.rope_offset % 8) == 0 && (a.rope_stride % 8) == 0 && (a.rope_dim % 16) == 0 &&
                              (reinterpret_cast<uintptr_t>(a.cos_t) % 16) == 0 &&
                              (reinterpret_cast<uintptr_t>(a.sin_t) % 16) == 0)) &&
                   (!a.rope_aux || ((reinterpret_cast<uintptr_t>(a.rope_aux) % 16) == 0 && (a.rope_aux_stride % 8) == 0));
  // rows of up to 1024 elements in registers (rotate_half, at most 64 rope
  // pair chunks): one memory round trip per row (bf16 [4096, 576] rows with
  // norm and RoPE: 7.2 -> 5.8 us); wider rows keep the chunk loops, which
  // measured faster for [4096, 1536] fp32 rows (8.4 against 9.2 us)
  const int nch = a.row_width / 8, pairs = rope ? a.rope_slices * (a.rope_dim / 16) : 0;
  if (vec && !a.interleave && nch <= 128 && pairs <= 64) {
    auto go = [&](auto npl) {
      constexpr int NPL = decltype(npl)::value;
      if (bf16_io && src_f32)
        norm_rope_reg_kernel<float, bf16, NPL, 1><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
      else if (bf16_io)
        norm_rope_reg_kernel<bf16, bf16, NPL, 1><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
      else
        norm_rope_reg_kernel<float, float, NPL, 1><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
    };
    if (nch <= 64) go(std::integral_constant<int, 1>{});
    else go(std::integral_constant<int, 2>{});
    return hipGetLastError();
  }
  if (vec) {
    if (bf16_io && src_f32)
      norm_rope_vec_kernel<float, bf16><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
    else if (bf16_io)
      norm_rope_vec_kernel<bf16, bf16><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
    else
      norm_rope_vec_kernel<float, float><<<blocks, 64 * ROWS_PER_BLOCK, 0, s>>>(a);
    return hipGetLastError();
  }
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
