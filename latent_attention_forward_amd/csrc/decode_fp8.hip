// Weight-absorbed MLA decode over an FP8 (E4M3) latent cache, and the
// conversion of bf16 cache rows into that format.
//
// Cache format: each [c_n (512) | k_pe' (64)] row is 576 E4M3 codes (OCP 8-bit
// floating point: bias 7, subnormals, largest finite 448), one float32 scale
// for the whole cache (value = code * scale).  The pages name FP8 only as the
// MXFP8 recipe of "Megatron-LM MLA guide" (parameter section,
// use_fused_mla_q_uproj, fp8_dot_product_attention) and give no cache format;
// this is the plainest one that halves the cached bytes.
//
// The split kernel has the work order, partial-buffer contract and softmax
// origin rule of the bf16 split kernel (decode.hip), so the absorption and the
// combine + un-absorb kernels are shared; what changes is the tile loop:
//   * tiles of 64 cached rows (36 KB in LDS, the bytes of a 32-row bf16 tile),
//     segment cuts on multiples of 64 keys;
//   * both contractions on the block-scaled 32x32x64 fp8 MFMA
//     (v_mfma_scale_f32_32x32x64_f8f6f4), twice the rate of bf16 per element:
//       S^T[key, head]  = C[key, :] . Qc[head, :]    A = cache rows, B = Qc
//       O^T[dim, head] += C^T[dim, key] . P^T[key, head]
//                                                    A = C^T (ds_read_b64_tr_b8)
//   * the MFMA's K = 64 operand bytes of a column (row) sit in two lanes, l
//     and l + 32, 32 bytes each; its two E8M0 block scales come from those two
//     lanes, the scale of lane half h applying to bytes 16 h .. 16 h + 15 of
//     BOTH lanes (checked on gfx950).  So an MX block of 32 elements is 16
//     bytes of each lane of the pair, and a pair exchanges its partial maxima
//     (permlane32 swap) to form the block scale;
//   * the absorbed query Qc is quantised per segment, in registers, to MXFP8:
//     each block of 32 consecutive dims gets the OCP Microscaling shared scale
//     2^(floor(log2 max|x|) - 8) (an E8M0 exponent, the MFMA's B scale) and
//     E4M3 elements, saturating at 448;
//   * the probabilities are quantised the same way, per block of 32 keys of
//     the tile: P = 2^x with x = s c2 - origin is stored as E4M3(2^(x - e))
//     with e = floor(max x over the block) - 7, so every block sits at the
//     top of the E4M3 range whatever its distance from the origin; the MFMA
//     applies 2^e;
//   * the softmax denominator sums the same E4M3 values (converted back), so
//     numerator and denominator carry the same rounding.
// The cache scale is folded into the score scale and into the stored partial
// outputs, so the partials are in the units of the bf16 kernel.
#include "mla_internal.hpp"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int DK8 = 64;                    // keys per tile
constexpr int NB8 = 4;                     // LDS tile buffers (ring)
constexpr int RB = 576;                    // bytes (codes) per cached row
constexpr int RKL = 512, DRL = 64;         // latent / rope widths
constexpr int CH8 = RB / 16;               // 16 B chunks per row (36)
constexpr int TB8 = DK8 * RB;              // tile bytes (36864)
constexpr float kMaxExcursion8 = 64.f;     // log2 units above the origin

// Tile [64 rows][576 B]: 16 B chunk c of row r at c ^ fsw(r).  Rows are
// 2.25 x 256 B, so rows r and r + 4 start on the same banks; the swizzle (row
// bits 2..3 into chunk bits 0..1) puts the 16 rows one 16-lane phase of a
// score-operand read touches on 16 distinct 16 B bank groups.  It changes only
// the two low chunk bits, so a chunk stays in its aligned group of four.
__device__ __forceinline__ int fsw(int r) { return (r >> 2) & 3; }

template <int BYTE> __device__ __forceinline__ float fp8_value(int word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, BYTE);
}

// Scaled fp8 MFMA, accumulator in VGPRs (inline asm, as mfma32_vacc): the
// score chain stays in VGPRs while the AGPRs hold the 32 x 512 output.  The
// asm carries the wait states for VALU-written operands and scales.
__device__ __forceinline__ void mfma_f8_vacc(f32x16& c, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 2\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void mfma_f8_vacc0(f32x16& c, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 2\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// The same MFMA accumulating in AGPRs (the 32 x 512 output).  As asm it stays
// where it is written: the compiler would sink the builtin past the step's
// wait and barrier and issue every operand read of the tile first.
__device__ __forceinline__ void mfma_f8_aacc(f32x16& c, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 2\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(c) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// Wait states between the 16-pass MFMA writing VGPRs and a VALU read of them.
__device__ __forceinline__ void mfma16p_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// E4M3 codes of 4 floats (already within +-448), packed little-endian.
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
__device__ __forceinline__ float sat448(float v) {
  return __builtin_fabsf(v) > 448.f ? __builtin_copysignf(448.f, v) : v;
}
// The same clamp for finite values (one v_med3).
__device__ __forceinline__ float clamp448(float v) { return __builtin_amdgcn_fmed3f(v, -448.f, 448.f); }

// max of v over this lane and its partner lane l ^ 32
__device__ __forceinline__ float pair_max(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// MXFP8 quantisation of the lane's 32 operand bytes: v[0..15] are 16 elements
// of block 0 and v[16..31] 16 elements of block 1, the other 16 of each block
// being in the partner lane.  Codes, and the E8M0 byte of block `half` (the
// scale this lane supplies to the MFMA).
__device__ __forceinline__ void mx_pair(const float (&v)[32], int half, i32x8& codes, int& scale_byte) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a0 = fmaxf(a0, __builtin_fabsf(v[i]));
    a1 = fmaxf(a1, __builtin_fabsf(v[16 + i]));
  }
  a0 = pair_max(a0);
  a1 = pair_max(a1);
  // floor(log2 amax) - 8 as a biased exponent (a zero or subnormal block takes
  // the smallest scale; its codes are then exact or flushed)
  const int s0 = max(0, min(254, (int)((__float_as_uint(a0) >> 23) & 255) - 8));
  const int s1 = max(0, min(254, (int)((__float_as_uint(a1) >> 23) & 255) - 8));
  const float i0 = __uint_as_float((uint32_t)(254 - s0) << 23);   // 2^(127 - s0)
  const float i1 = __uint_as_float((uint32_t)(254 - s1) << 23);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    codes[w] = pack4_fp8(clamp448(v[4 * w] * i0), clamp448(v[4 * w + 1] * i0), clamp448(v[4 * w + 2] * i0),
                         clamp448(v[4 * w + 3] * i0));
    codes[4 + w] = pack4_fp8(clamp448(v[16 + 4 * w] * i1), clamp448(v[17 + 4 * w] * i1),
                             clamp448(v[18 + 4 * w] * i1), clamp448(v[19 + 4 * w] * i1));
  }
  scale_byte = half ? s1 : s0;
}

// fp32 online softmax over keys [k0, k1) of sequence b for heads [h0, h0 + 32),
// one wave, reading the E4M3 cache from global memory; writes the partials in
// the bf16 kernel's units.  Used only by a wave whose scores left the range of
// its fixed exponent origin.
__device__ __forceinline__ void decode_chunk_exact_fp8(const DecodeArgs& a, int b, int64_t part, int h0, int k0,
                                                       int k1) {
  const int lane = threadIdx.x & 63;
  const int H = a.heads, lbs = a.log2_block, bmask = (1 << lbs) - 1;
  const float cs = a.cache_scale;
  const float c2 = a.scale * kLog2e;
  for (int h = h0; h < h0 + 32; ++h) {
    const bf16* qt = a.qt + ((int64_t)b * H + h) * RKL;
    const bf16* qp = a.q_pe + ((int64_t)b * H + h) * DRL;
    float q[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int d = lane + 64 * i;
      q[i] = d < RKL ? (float)qt[d] : (float)qp[d - RKL];
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int j = k0; j < k1; ++j) {
      const int64_t row = ((int64_t)a.block_table[(int64_t)b * a.max_blocks + (j >> lbs)] << lbs) + (j & bmask);
      const uint8_t* cr = a.cache8 + row * RB;
      float part_s = 0.f;
#pragma unroll
      for (int i = 0; i < 9; ++i) part_s = fmaf(q[i], fp8_value<0>(cr[lane + 64 * i]), part_s);
      const float sj = wave_sum(part_s) * cs;            // score in latent units
      const float mn = fmaxf(m, sj);
      const float al = __builtin_amdgcn_exp2f((m - mn) * c2), p = __builtin_amdgcn_exp2f((sj - mn) * c2);
      l = l * al + p;
      const i32x2 w8 = *(const i32x2*)(cr + lane * 8);
      const float cv[8] = {fp8_value<0>(w8[0]), fp8_value<1>(w8[0]), fp8_value<2>(w8[0]), fp8_value<3>(w8[0]),
                           fp8_value<0>(w8[1]), fp8_value<1>(w8[1]), fp8_value<2>(w8[1]), fp8_value<3>(w8[1])};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * al + p * cv[e];
      m = mn;
    }
    f16* po = a.part_o + (part + h) * RKL + lane * 8;
    const float inv = cs / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) po[e] = (f16)(acc[e] * inv);
    if (lane == 0) {
      a.part_ml[(part + h) * 2 + 0] = m;
      a.part_ml[(part + h) * 2 + 1] = l;
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_fp8_kernel(DecodeArgs a) {
  constexpr int NTH = NW * 64;
  constexpr int BLOCKS = TB8 / 1024;                // 1 KB LDS blocks per tile (36)
  static_assert(BLOCKS % NW == 0, "tile must split evenly over the waves");
  constexpr int BPW = BLOCKS / NW;
  __shared__ __attribute__((aligned(16))) uint8_t sC[NB8][TB8];
  __shared__ int sBlk[kDecodeMaxChunkBlocks];
  __shared__ int s_badw[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads;
  const int lbs = a.log2_block, bmask = (1 << lbs) - 1;
  const int cap = a.max_blocks << lbs;
  const int64_t R = a.quota;
  // work item of this workgroup (the bf16 kernel's order: consecutive items on one XCD)
  const int G = gridDim.x, g8 = G >> 3, r8 = G & 7, xc = blockIdx.x & 7;
  const int item = xc * g8 + min(xc, r8) + (int)(blockIdx.x >> 3);
  const int64_t S0 = (int64_t)item * R, S1 = S0 + R;
  __shared__ long long s_first[2];
  auto seg_len = [&](int bq) -> long long {
    const int Lq = max(0, min(a.seq_lens[bq], cap));
    return Lq > 0 ? (long long)Lq + kDecodeSegmentCost : 0;
  };
  if (wave == 0) {
    if (lane == 0) { s_first[0] = a.batch; s_first[1] = 0; }
    long long seen = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      const int bb = b0 + lane;
      const int Lb = (bb < a.batch) ? max(0, min(a.seq_lens[bb], cap)) : 0;
      const long long n = Lb > 0 ? (long long)Lb + kDecodeSegmentCost : 0;
      long long incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const long long v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (n > 0 && seen + incl - n <= S0 && S0 < seen + incl) { s_first[0] = bb; s_first[1] = seen + incl - n; }
      seen += __shfl(incl, 63, 64);
      if (seen > S0) break;
    }
  }
  __syncthreads();
  int b = (int)s_first[0];
  int64_t st = s_first[1];
  for (; b < a.batch && st < S1; st += seg_len(b), ++b) {
  __syncthreads();                         // the previous segment is done with sBlk and the tiles
  int tid_s = tid;
  asm volatile("" : "+v"(tid_s));
  const int tid = tid_s, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = max(0, min(a.seq_lens[b], cap));
  const int64_t r0 = st + kDecodeSegmentCost;
  if (L == 0 || S1 <= r0) continue;
  // cut points inside the sequence move to the nearest multiple of 64 keys (one tile)
  auto cut = [&](int64_t x) -> int {
    return x <= 0 ? 0 : (x >= L ? L : (int)min<int64_t>(L, ((x + 32) >> 6) << 6));
  };
  const int k0 = cut(S0 - r0), k1 = cut(S1 - r0);
  const int64_t part = ((int64_t)item + b) * H;
  if (k0 >= k1) {
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = -INFINITY; a.part_ml[(part + i) * 2 + 1] = 0.f; }
    continue;
  }
  const int nt = (k1 - k0 + DK8 - 1) / DK8;

  const int blk0 = k0 >> lbs;
  const int nblk = ((k1 - 1) >> lbs) - blk0 + 1;
  constexpr int TBL = (kDecodeMaxChunkBlocks + NTH - 1) / NTH;
  int tv[TBL];
#pragma unroll
  for (int u = 0; u < TBL; ++u) {
    const int i = tid + u * NTH;
    tv[u] = i < nblk ? a.block_table[(int64_t)b * a.max_blocks + blk0 + i] : 0;
  }
  __builtin_amdgcn_sched_barrier(0);
  const int hsel = lane >> 5;
  const int my_h = wave * 32 + (lane & 31);
  // absorbed query of this lane's head, MXFP8: in k-step ks, operand byte
  // 16 g + i (g = 0, 1; i < 16) of lane half hsel is dim 64 ks + 32 g +
  // 16 hsel + i; the MX blocks are dims 64 ks + [0, 32) and 64 ks + [32, 64)
  i32x8 q8[RB / 64];
  int qsc[RB / 64];
  {
    const bf16* qt = a.qt + ((int64_t)b * H + my_h) * RKL;
    const bf16* qp = a.q_pe + ((int64_t)b * H + my_h) * DRL;
#pragma unroll
    for (int ks = 0; ks < RB / 64; ++ks) {
      float v[32];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int d = ks * 64 + g * 32 + hsel * 16;
        const bf16* src = d < RKL ? qt + d : qp + (d - RKL);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 x = *(const bf16x8*)(src + c * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[g * 16 + c * 8 + e] = (float)x[e];
        }
      }
      mx_pair(v, hsel, q8[ks], qsc[ks]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  int bad = 0;
#pragma unroll
  for (int u = 0; u < TBL; ++u) {
    const int i = tid + u * NTH;
    if (i < nblk) {
      bad |= (tv[u] < 0 || tv[u] >= a.num_blocks);
      sBlk[i] = tv[u];
    }
  }
  const bool wbad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (lane == 0) s_badw[wave] = wbad;
  lds_wait_all();
  wg_barrier();
  int anybad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) anybad |= s_badw[w];
  if (anybad) {
    for (int i = tid; i < H * RKL; i += NTH) a.part_o[part * RKL + i] = (f16)__builtin_nanf("");
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = 0.f; a.part_ml[(part + i) * 2 + 1] = __builtin_nanf(""); }
    continue;
  }

  // Lane-constant parts of the swizzled LDS byte addresses.
  //  score read (mt, ks, g): row mt*32 + lane%32, chunk 4 ks + 2 g + hsel
  //  (operand bytes 16 g .. 16 g + 15, the query's dim order)
  const int rs = lane & 31, fs = fsw(rs);
  int base_s[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) base_s[g] = rs * RB + (((2 * g + hsel) ^ fs) << 4);
  //  transpose read (d, q): within a 16-lane group, source lane s = 2 j + t
  //  addresses row key_j and dims 32 d + 16 (group & 1) + 8 t; result lane i
  //  receives byte i % 8 of source lanes 2 j + i / 8, j = 0..7.  Byte 8 q + j of
  //  the operand of lane (dim, hsel) is key (q/2) 32 + 8 (2 (q%2) + j/4) +
  //  4 hsel + j%4, the key order of the score output (P^T byte 16 mt + e is
  //  score element e of key block mt).
  const int grp = lane >> 4, sl = lane & 15, tj = sl >> 1, tt = sl & 1;
  const int trow = 8 * (tj >> 2) + 4 * hsel + (tj & 3);
  const int ft = fsw(trow);
  int base_t[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) base_t[u] = trow * RB + (((2 * u + (grp & 1)) ^ ft) << 4) + 8 * tt;

  uint32_t doff[BPW];                      // byte offsets inside a tile of 64 contiguous rows
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int P = (wave + NW * i) * 64 + lane;
    const int r = P / CH8, pc = P - r * CH8;
    doff[i] = (uint32_t)(r * RB + ((pc ^ fsw(r)) << 4));
  }
  const uint32_t dst0 = lds_addr_of(&sC[0][0]) + (uint32_t)wave * 1024u;
  auto issue_tile = [&](int t, int buf) {
    const int kb = k0 + t * DK8;
    const uint32_t dst = dst0 + (uint32_t)buf * TB8;
    if (lbs >= 6 && kb + DK8 <= k1) {
      const uint8_t* tb = uniform_ptr(a.cache8 + (((int64_t)sBlk[(kb >> lbs) - blk0] << lbs) + (kb & bmask)) * RB);
#pragma unroll
      for (int i = 0; i < BPW; ++i) lds_dma16_sv_m0(tb, doff[i], dst + i * NW * 1024);
    } else {
#pragma unroll 1
      for (int i = 0; i < BPW; ++i) {
        const int P = (wave + NW * i) * 64 + lane;
        const int r = P / CH8, pc = P - r * CH8;
        const int key = (kb + r < k1) ? kb + r : k0;
        const int64_t row = ((int64_t)sBlk[(key >> lbs) - blk0] << lbs) + (key & bmask);
        lds_dma16_m0(a.cache8 + row * RB + ((pc ^ fsw(r)) << 4), dst + i * NW * 1024);
      }
    }
  };

  const float c2 = a.scale * kLog2e * a.cache_scale;   // raw score (codes) -> base-2 exponent
  float m_ref = -INFINITY, l_run = 0.f;
  bool exact_path = false;
  f32x16 o[RKL / 32];
#pragma unroll
  for (int d = 0; d < RKL / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  const int one_scale = 127;                 // E8M0 1.0 for the cache operand

  // S^T for the 64 keys of buffer buf: two key blocks x 9 k-steps, operands
  // read two MFMAs ahead; group(I) places work between the MFMAs
  auto s_tile = [&](f32x16 (&s)[2], int buf, auto&& group) __attribute__((always_inline)) {
    const uint8_t* sb = sC[buf];
    constexpr int NS = 2 * (RB / 64), D = 2;
    auto rd = [&](int i) -> i32x8 {
      const int mt = i & 1, ks = i >> 1;
      const uint8_t* p0 = sb + base_s[0] + ks * 64 + mt * 32 * RB;
      const uint8_t* p1 = sb + base_s[1] + ks * 64 + mt * 32 * RB;
      const int4 lo = *(const int4*)p0, hi = *(const int4*)p1;
      i32x8 r;
      r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w; r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
      return r;
    };
    i32x8 cf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) cf[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NS>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      const i32x8 cur = cf[i % D];
      if constexpr (i + D < NS) cf[i % D] = rd(i + D);
      if constexpr (i < 2) mfma_f8_vacc0(s[i & 1], cur, q8[i >> 1], one_scale, qsc[i >> 1]);
      else mfma_f8_vacc(s[i & 1], cur, q8[i >> 1], one_scale, qsc[i >> 1]);
      group(I);
      __builtin_amdgcn_sched_barrier(0);
    });
    mfma16p_result_wait();
  };
  // softmax of one tile: mask + lane max, head max / origin / excursion check,
  // then the 32 probabilities of the lane (one MX block) in groups of 4
  float mb = 0.f, mx_b[2] = {0.f, 0.f}, eb[2] = {0.f, 0.f};
  int psc = 0;
  i32x8 pb;
  auto prep_a = [&](f32x16 (&s)[2], int t) __attribute__((always_inline)) {
    const int kb = k0 + t * DK8;
    if (kb + DK8 > k1) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3) >= k1) s[mt][e] = -INFINITY;
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
      mx_b[mt] = mx;
    }
  };
  auto prep_b = [&](int t) __attribute__((always_inline)) {
    // maxima of the two 32-key blocks over both lane halves; the head's max
    const float b0 = pair_max(mx_b[0]), b1 = pair_max(mx_b[1]);
    const float mx = fmaxf(b0, b1);
    if (t == 0) m_ref = mx;
    exact_path |= __builtin_amdgcn_ballot_w64((mx - m_ref) * c2 > kMaxExcursion8) != 0;
    mb = m_ref * c2;
    // block exponents: 2^(x - e) <= 2^8 for every x of the block (x <=
    // kMaxExcursion8 on this path; a fully masked block gives zeros)
    const float x0 = b0 * c2 - mb, x1 = b1 * c2 - mb;
    eb[0] = x0 > -120.f ? __builtin_floorf(x0) - 7.f : -127.f;
    eb[1] = x1 > -120.f ? __builtin_floorf(x1) - 7.f : -127.f;
    psc = (int)(hsel ? eb[1] : eb[0]) + 127;     // this lane supplies block hsel's scale
  };
  auto prob4 = [&](f32x16 (&s)[2], int w) __attribute__((always_inline)) {   // bytes 4w .. 4w+3 of P^T
    const int mt = w >> 2, e0 = (w & 3) * 4;
    const float sh = mb + eb[mt];
    float p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = __builtin_amdgcn_exp2f(fmaf(s[mt][e0 + k], c2, -sh));
    asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
    pb[w] = pack4_fp8(p[0], p[1], p[2], p[3]);
  };
  // the denominator: the E4M3 probabilities converted back, times 2^e
  auto psum = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float acc = 0.f;
#pragma unroll
      for (int w = 4 * mt; w < 4 * mt + 4; ++w) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pb[w], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pb[w], true);
        acc += (lo[0] + lo[1]) + (hi[0] + hi[1]);
      }
      l_run = fmaf(acc, __builtin_amdgcn_ldexpf(1.f, (int)eb[mt]), l_run);
    }
    asm volatile("" : "+v"(l_run));       // computed here, between the PV MFMAs
  };
  auto no_group = [](auto) {};
  // O^T += C^T P^T over the 64 keys: 16 dim blocks, each one MFMA with the
  // operand from four transpose reads, two blocks ahead
  auto pv_tile = [&](int buf, auto&& group) __attribute__((always_inline)) {
    const uint8_t* sb = sC[buf];
    constexpr int NP = RKL / 32, D = 2;
    auto rd = [&](int d) -> i32x8 {
      i32x8 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint8_t* p = sb + base_t[d & 1] + (q >> 1) * 32 * RB + (q & 1) * 16 * RB + (d >> 1) * 64;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(MLA_LDS void*)(p));
        r[2 * q] = v[0];
        r[2 * q + 1] = v[1];
      }
      return r;
    };
    i32x8 vf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) vf[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NP>([&](auto I) __attribute__((always_inline)) {
      constexpr int d = decltype(I)::value;
      const i32x8 cur = vf[d % D];
      if constexpr (d + D < NP) vf[d % D] = rd(d + D);
      mfma_f8_aacc(o[d], cur, pb, one_scale, psc);
      group(I);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Iteration t: the MFMAs of S(t + 1) carry the softmax of tile t (mask and
  // lane max at MFMA 0, origin at 1, four probabilities at each odd MFMA from
  // 3 to 17) and the copies of tile t + 3 (MFMAs 2 to 16); then PV(t) carries
  // the denominator.
  auto step = [&](int t, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) __attribute__((always_inline)) {
    const int kn = k0 + (t + 3) * DK8;
    const bool issue = t + 3 < nt, fast = lbs >= 6 && kn + DK8 <= k1;
    const uint32_t dstn = dst0 + (uint32_t)((t + 3) % NB8) * TB8;
    if (issue && !fast) issue_tile(t + 3, (t + 3) % NB8);
    if (t + 1 < nt) {
      const uint8_t* tb = nullptr;
      s_tile(s_nxt, (t + 1) % NB8, [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) {
          prep_a(s_cur, t);
          if (issue && fast) tb = uniform_ptr(a.cache8 + (((int64_t)sBlk[(kn >> lbs) - blk0] << lbs) + (kn & bmask)) * RB);
        }
        if constexpr (i == 1) prep_b(t);
        if constexpr (i >= 3 && (i & 1) && (i - 3) / 2 < 8) prob4(s_cur, (i - 3) >> 1);
        if constexpr (i >= 2 && i < 2 + BPW)
          if (issue && fast) lds_dma16_sv_m0(tb, doff[i - 2], dstn + (i - 2) * NW * 1024);
      });
    } else {
      if (issue && fast) issue_tile(t + 3, (t + 3) % NB8);
      prep_a(s_cur, t);
      prep_b(t);
#pragma unroll
      for (int w = 0; w < 8; ++w) prob4(s_cur, w);
    }
    pv_tile(t % NB8, [&](auto I) __attribute__((always_inline)) {
      constexpr int d = decltype(I)::value;
      if constexpr (d == 2) psum();
    });
    if (t + 3 < nt) vm_wait_keep<BPW>();
    else vm_wait_all();
    wg_barrier();
  };

  issue_tile(0, 0);
  if (1 < nt) issue_tile(1, 1);
  vm_wait_all();
#pragma unroll
  for (int ks = 0; ks < RB / 64; ++ks) asm volatile("" : : "v"(q8[ks]), "v"(qsc[ks]));
  wg_barrier();
  if (2 < nt) issue_tile(2, 2);
  f32x16 sa[2], sbv[2];
  s_tile(sa, 0, no_group);
  for (int t = 0; t < nt; ++t) {
    step(t, sa, sbv);
    sa[0] = sbv[0];
    sa[1] = sbv[1];
  }
  mfma16p_result_wait();                  // the output accumulators are read next

  if (exact_path) {
    decode_chunk_exact_fp8(a, b, part, wave * 32, k0, k1);
  } else {
    // O / l times the cache scale (latent units), fp16 through this wave's
    // 32 KB of the idle tile buffers, one 1 KB row per store; the origin in
    // latent units
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = a.cache_scale / l_tot;
    char* wb = (char*)&sC[0][0] + wave * (32 * RKL * 2);
    const int hl = lane & 31;
#pragma unroll
    for (int d = 0; d < RKL / 32; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)(o[d][q * 4 + e] * inv);
        *(f16x4*)(wb + hl * (RKL * 2) + (((d * 4 + q) ^ (hl & 15)) << 4) + hsel * 8) = v;
      }
    f16* po = a.part_o + (part + wave * 32) * RKL + lane * 8;
#pragma unroll
    for (int r = 0; r < 32; ++r)
      *(f16x8*)(po + r * RKL) = *(const f16x8*)(wb + r * (RKL * 2) + ((lane ^ (r & 15)) << 4));
    if (hsel == 0) {
      a.part_ml[(part + my_h) * 2 + 0] = m_ref * a.cache_scale;
      a.part_ml[(part + my_h) * 2 + 1] = l_tot;
    }
  }
  }
}

// bf16 rows -> E4M3 codes, 8 elements per thread per step (16 B in, 8 B out).
__global__ __launch_bounds__(256) void cache_quant_fp8_kernel(CacheQuantArgs a) {
  const int cpr = a.width >> 3;
  const int64_t n = a.rows * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cpr;
    const int c = (int)(i - r * cpr);
    const bf16x8 x = *(const bf16x8*)(a.src + r * a.src_stride + c * 8);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = sat448((float)x[e] * a.inv);
    i32x2 w;
    w[0] = pack4_fp8(y[0], y[1], y[2], y[3]);
    w[1] = pack4_fp8(y[4], y[5], y[6], y[7]);
    *(i32x2*)(a.dst + r * a.dst_stride + c * 8) = w;
  }
}

}  // namespace

hipError_t launch_decode_split_fp8(const DecodeArgs& a, hipStream_t s) {
  if (a.num_items <= 0) return hipSuccess;
  dim3 grid(a.num_items);
  switch (a.heads) {
    case 32: decode_split_fp8_kernel<1><<<grid, 64, 0, s>>>(a); break;
    case 64: decode_split_fp8_kernel<2><<<grid, 128, 0, s>>>(a); break;
    case 96: decode_split_fp8_kernel<3><<<grid, 192, 0, s>>>(a); break;
    case 128: decode_split_fp8_kernel<4><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cache_quant_fp8(const CacheQuantArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t n = a.rows * (a.width >> 3);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
  cache_quant_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
