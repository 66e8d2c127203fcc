// Projection GEMMs of the MLA layer: y = x W^T (nn.Linear layout), and the
// batched per-head products of the absorbed decode.
//
// bf16 kernel: 128x128 output tile per 256-thread workgroup, K step 64, fp32
// accumulation on v_mfma_f32_32x32x16_bf16.  Operand tiles are staged through
// LDS with double buffering; global->register prefetch of tile k+1 overlaps
// the MFMAs of tile k.  Each wave owns a 64x64 quadrant (2x2 MFMA tiles).
//
// The MFMA "A" operand is taken from the weight tile and the "B" operand from
// the activation tile, so each lane ends up holding 4 consecutive output
// columns of one row and stores them with one 8-byte write.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;

// K-contiguous tile [rows][64]: 8 chunks of 16 B per row (128 B), so rows of
// one parity start at the same bank.  Chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7): the 16 consecutive rows that one 16-lane phase of an
// operand read (ds_read_b128, same logical chunk) touches cover all 64 banks.
__device__ __forceinline__ int kmaj(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }
// N-contiguous tile [64 k][128 n] for the transposed (NN) operand: 16 chunks per
// row, chunk c of row k stored at c ^ ((k & 3) << 1).  A transpose read touches
// 4 consecutive k rows x 32 B; the swizzle spreads them over 128 B.
__device__ __forceinline__ int nmaj(int k, int n) { return k * BN + ((((n >> 3) ^ ((k & 3) << 1))) << 3) + (n & 7); }

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ int2 tile_coords(int pid, int num_m, int num_n) {
  // Spread consecutive tiles of one band across the workgroups that share an
  // XCD (workgroup ids are dealt to the 8 XCDs round-robin), then walk bands of
  // 8 m-tiles so that a band's activation rows and weight columns stay in L2.
  const int total = num_m * num_n;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int group = 8 * num_n;
  const int first_m = (pid / group) * 8;
  const int gsize = min(num_m - first_m, 8);
  const int in_group = pid % group;
  return make_int2(first_m + in_group % gsize, in_group / gsize);
}

template <bool B_KN, int EPI, int CT>   // CT: 0 bf16, 1 fp32, 2 fp16 output
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * BK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int num_m = (g.m + BM - 1) / BM, num_n = (g.n + BN - 1) / BN;
  const int2 tc = tile_coords(blockIdx.x, num_m, num_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  const bf16* A = (const bf16*)g.a + (int64_t)blockIdx.z * g.a_bstride;
  const bf16* B = (const bf16*)g.b + (int64_t)blockIdx.z * g.b_bstride;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = (g.k + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      const int gm = m0 + r, gk = k0 + c * 8;
      ra[i] = (gm < g.m && gk < g.k) ? *(const bf16x8*)(A + (int64_t)gm * g.lda + gk) : zero8();
      if (!B_KN) {
        const int gn = n0 + r;
        rb[i] = (gn < g.n && gk < g.k) ? *(const bf16x8*)(B + (int64_t)gn * g.ldb + gk) : zero8();
      } else {
        const int rk = id >> 4, cn = id & 15;
        const int gk2 = k0 + rk, gn = n0 + cn * 8;
        rb[i] = (gk2 < g.k && gn < g.n) ? *(const bf16x8*)(B + (int64_t)gk2 * g.ldb + gn) : zero8();
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      *(bf16x8*)&sA[buf][kmaj(r, c)] = ra[i];
      if (!B_KN) {
        *(bf16x8*)&sB[buf][kmaj(r, c)] = rb[i];
      } else {
        const int rk = id >> 4, cn = id & 15;
        *(bf16x8*)&sB[buf][nmaj(rk, cn * 8)] = rb[i];
      }
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 xa[2], wb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        xa[mi] = *(const bf16x8*)&sA[buf][kmaj(r, ks * 2 + (lane >> 5))];
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int rn = wn * 64 + ni * 32;
        if (!B_KN) {
          wb[ni] = *(const bf16x8*)&sB[buf][kmaj(rn + (lane & 31), ks * 2 + (lane >> 5))];
        } else {
          const int L = lane & 15, grp = lane >> 4;
          const int nb = rn + (grp & 1) * 16 + 4 * (L & 3);
          const int kr = ks * 16 + (grp >> 1) * 8 + (L >> 2);
          const bf16x4 lo = lds_read_tr(&sB[buf][nmaj(kr, nb)]);
          const bf16x4 hi = lds_read_tr(&sB[buf][nmaj(kr + 4, nb)]);
          wb[ni] = cat8(lo, hi);
        }
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) acc[ni][mi] = mfma32(wb[ni], xa[mi], acc[ni][mi]);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(buf);
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // RoPE epilogue.  Rope slices start at multiples of 64 columns and are 64
  // wide, so a slice is exactly one wave's 64-column window: pair (i, i + 32)
  // is register e of N-tile 0 and register e of N-tile 1 in the same lane.
  if (EPI == EPI_ROPE) {
    const int c0 = n0 + wn * 64;
    if (c0 + 64 <= g.n && (c0 % g.rope_head_stride) == g.rope_off) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int m = m0 + wm * 64 + mi * 32 + (lane & 31);
        if (m >= g.m) continue;
        const int pos = g.positions[m];
        const bool ok = pos >= 0 && pos < g.table_len;
        const float* cs = g.cos_t + (int64_t)(ok ? pos : 0) * 32;
        const float* sn = g.sin_t + (int64_t)(ok ? pos : 0) * 32;
        if (!g.rope_interleave) {
          // rotate_half pairs (i, i + 32): column i in acc[0], i + 32 in acc[1]
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = q * 8 + (lane >> 5) * 4 + e;
              const float x0 = acc[0][mi][q * 4 + e], x1 = acc[1][mi][q * 4 + e];
              const float c = ok ? cs[i] : __builtin_nanf(""), sv = ok ? sn[i] : __builtin_nanf("");
              acc[0][mi][q * 4 + e] = x0 * c - x1 * sv;
              acc[1][mi][q * 4 + e] = x1 * c + x0 * sv;
            }
        } else {
          // interleaved pairs (2i, 2i + 1): both columns in one lane's run of 4
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; e += 2) {
                const int i = (ni * 32 + q * 8 + (lane >> 5) * 4 + e) >> 1;
                const float x0 = acc[ni][mi][q * 4 + e], x1 = acc[ni][mi][q * 4 + e + 1];
                const float c = ok ? cs[i] : __builtin_nanf(""), sv = ok ? sn[i] : __builtin_nanf("");
                acc[ni][mi][q * 4 + e] = x0 * c - x1 * sv;
                acc[ni][mi][q * 4 + e + 1] = x1 * c + x0 * sv;
              }
        }
      }
    }
  }

  // store: lane holds row m = col index of the MFMA output, 4 runs of 4
  // consecutive n.
  const bf16* G = (const bf16*)g.gate_src + (EPI == EPI_GATE ? (int64_t)blockIdx.z * g.c_bstride : 0);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int m = m0 + wm * 64 + mi * 32 + (lane & 31);
      if (m >= g.m) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + ni * 32 + q * 8 + (lane >> 5) * 4;
        if (n >= g.n) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[ni][mi][q * 4 + e];
        if (EPI == EPI_GATE) {
          const bf16x4 gs = *(const bf16x4*)(G + (int64_t)m * g.ldg + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (float)gs[e] * (1.f / (1.f + __expf(-v[e])));
        }
        if (CT == 1) {
          float* C = (float*)g.c + (int64_t)blockIdx.z * g.c_bstride;
          float4* cp = (float4*)(C + (int64_t)m * g.ldc + n);
          if (g.c_acc) {
            const float4 o = *cp;
            v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
          }
          *cp = make_float4(v[0], v[1], v[2], v[3]);
        } else if (CT == 2) {
          f16* C = (f16*)g.c + (int64_t)blockIdx.z * g.c_bstride;
          f16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = to_f16_sat(v[e]);
          *(f16x4*)(C + (int64_t)m * g.ldc + n) = o;
        } else {
          bf16* C = (bf16*)g.c + (int64_t)blockIdx.z * g.c_bstride;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *(bf16x4*)(C + (int64_t)m * g.ldc + n) = o;
        }
      }
    }
}

// Large bf16 GEMMs (the projections whose grid fills the GPU many times):
// 256x256 output tile per 256-thread workgroup, one wave per SIMD, each wave a
// 128x128 quadrant (4x4 MFMA tiles, the fp32 accumulators in AGPRs).  K steps
// of 32; the operand tiles go global->LDS with global_load_lds_dwordx4 (no
// register staging), 4 LDS stages with 3 in flight, one barrier per step.
// Per step and CU: 1024 MFMA cycles per SIMD against 64 KB of operand reads
// and 32 KB of copies in LDS (~768 cycles at 128 B/clk).
// LDS tile [256 rows][32 k]: 4 chunks of 16 B per row, chunk c of row r at
// c ^ ((r >> 2) & 3), so the 16 rows one 16-lane phase of an operand read
// touches (4 rows per 256 B of banks) land on distinct banks.
// K-major operands (KM bit 0: A [k, m], bit 1: B [k, n]): a stage is
// [32 k][256 columns], 32 chunks of 16 B
// per k row, chunk c of row k at c ^ 2 (k & 3); an MFMA operand is read with
// two transposing reads (ds_read_b64_tr_b16) per 8 k, each 16-lane phase
// touching 4 k rows x 32 B, which the swizzle puts on distinct banks.
constexpr int GBM = 256, GBN = 256, GBK = 32, GSTAGES = 4;
__device__ __forceinline__ int gsw(int r, int c) { return r * GBK + ((c ^ ((r >> 2) & 3)) << 3); }

template <int EPI, int CT, int KM = 0>   // CT: 0 bf16, 1 fp32, 2 fp16, 3 MXFP8 (E4M3 codes + E8M0 block scales) output
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(GemmArgs g) {
  // operand stages, then (after the K loop) the 256x256 output tile in 16-bit
  // values: row r of 512 B with 16-byte chunk c at c ^ (r & 31)
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * GSTAGES * GBM * GBK];
  bf16 (*sX)[GBM * GBK] = (bf16 (*)[GBM * GBK])smem;                          // activation rows (m)
  bf16 (*sW)[GBN * GBK] = (bf16 (*)[GBN * GBK])(smem + GSTAGES * GBM * GBK);  // weight rows (n)
  static_assert(2 * GSTAGES * GBM * GBK >= GBM * GBN, "the output tile reuses the operand stages");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int num_m = (g.m + GBM - 1) / GBM, num_n = (g.n + GBN - 1) / GBN;
  const int2 tc = tile_coords(blockIdx.x, num_m, num_n);
  const int m0 = tc.x * GBM, n0 = tc.y * GBN;
  constexpr bool KA = (KM & 1) != 0, KB = (KM & 2) != 0;
  const bf16* A = (const bf16*)g.a + (int64_t)blockIdx.z * g.a_bstride + (KA ? (int64_t)m0 : (int64_t)m0 * g.lda);
  const bf16* B = (const bf16*)g.b + (int64_t)blockIdx.z * g.b_bstride + (KB ? (int64_t)n0 : (int64_t)n0 * g.ldb);
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = g.k / GBK;
  // RoPE: the position of tile row tid, requested now for the table staging
  const int spos = EPI == EPI_ROPE ? g.positions[min(m0 + tid, g.m - 1)] : 0;

  // Copies: instruction i of wave w fills the 1 KB block w + 4 i (16 rows) of a
  // tile; lane l takes row P / 4 and logical chunk (P % 4) ^ swizzle, P = 64
  // (w + 4 i) + l.  Rows past the matrix read its last row (never stored).
  uint32_t offx[4], offw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = (wave + 4 * i) * 64 + lane;
    // K-major: row k = P / 32, physical chunk P % 32 holds logical chunk
    // (P % 32) ^ 2 (k & 3); columns past the matrix read its last chunk
    const int k = P >> 5, kc = (P & 31) ^ ((k & 3) << 1);
    const int r = P >> 2, c = (P & 3) ^ ((r >> 2) & 3);
    if constexpr (KA) offx[i] = (uint32_t)(((int64_t)k * g.lda + min(m0 + kc * 8, g.m - 8) - m0) * 2);
    else offx[i] = (uint32_t)(((int64_t)(min(m0 + r, g.m - 1) - m0) * g.lda + c * 8) * 2);
    if constexpr (KB) offw[i] = (uint32_t)(((int64_t)k * g.ldb + min(n0 + kc * 8, g.n - 8) - n0) * 2);
    else offw[i] = (uint32_t)(((int64_t)(min(n0 + r, g.n - 1) - n0) * g.ldb + c * 8) * 2);
  }
  // LDS byte address of this wave's first block in stage 0 of each operand
  const uint32_t lx = lds_addr_of(&sX[0][0]) + (uint32_t)wave * 1024u;
  const uint32_t lw = lds_addr_of(&sW[0][0]) + (uint32_t)wave * 1024u;
  // copy j (0..7) of step kt: x blocks for j < 4, w blocks for j >= 4
  auto issue_part = [&](int kt, int j) __attribute__((always_inline)) {
    const uint32_t st = (uint32_t)(kt % GSTAGES) * (GBM * GBK * 2);
    const int64_t ka = KA ? (int64_t)kt * GBK * g.lda : (int64_t)kt * GBK;
    const int64_t kb = KB ? (int64_t)kt * GBK * g.ldb : (int64_t)kt * GBK;
    if (j < 4) lds_dma16_sv_m0(uniform_ptr(A + ka), offx[j], lx + st + j * 4096u);
    else lds_dma16_sv_m0(uniform_ptr(B + kb), offw[j - 4], lw + st + (j - 4) * 4096u);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_part(kt, j);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // operand reads: tile row wm*128 + mi*32 + lane%32 (x) / wn*128 + ni*32 + lane%32 (w),
  // chunk 2 ks + lane/32; the swizzle depends on the row only through bits 2-3,
  // the same for every mi / ni
  const int r32 = lane & 31, hs = lane >> 5;
  // K-major operand, transposing reads: lane L of 16-lane group q addresses
  // k row ks*16 + (q/2)*8 + u*4 + L/4 at column 32 i + (q%2)*16 + 4 (L%4) of
  // the wave's 128; the swizzle term 2 (k & 3) = 2 (L/4 & 3) flips bit 2 of
  // the chunk index (bit 0 of i), so element offsets are base[i % 2] +
  // 64 (i/2) + 256 (16 ks + 4 u).  Row-major operand: base[ks].
  int xoff[2], woff[2];
  {
    const int q = lane >> 4, L = lane & 15, sw = ((L >> 2) & 3) << 1;
    const int rowk = ((q >> 1) * 8 + (L >> 2)) * GBM;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cx = wm * 16 + 4 * j + 2 * (q & 1) + ((L & 3) >> 1);
      const int cw = wn * 16 + 4 * j + 2 * (q & 1) + ((L & 3) >> 1);
      xoff[j] = KA ? rowk + ((cx ^ sw) << 3) + 4 * (L & 1) : gsw(wm * 128 + r32, 2 * j + hs);
      woff[j] = KB ? rowk + ((cw ^ sw) << 3) + 4 * (L & 1) : gsw(wn * 128 + r32, 2 * j + hs);
    }
  }
  // The copies of step kiss (when >= 0) go out one per 4 MFMAs: issued all at
  // once, right after the barrier, the four waves' copies queue at the address
  // unit they share for ~400 cycles.
  // Both k halves' operands are requested up front, so the MFMAs of the
  // second half find theirs in registers instead of waiting on LDS.
  auto compute = [&](int st, int kiss) {
    bf16x8 x[2][4], w[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (i >> 1) * 64 + ks * 16 * GBM;
        if constexpr (KA)
          x[ks][i] = cat8(lds_read_tr(&sX[st][xoff[i & 1] + o]), lds_read_tr(&sX[st][xoff[i & 1] + o + 4 * GBM]));
        else
          x[ks][i] = *(const bf16x8*)&sX[st][xoff[ks] + i * 32 * GBK];
        if constexpr (KB)
          w[ks][i] = cat8(lds_read_tr(&sW[st][woff[i & 1] + o]), lds_read_tr(&sW[st][woff[i & 1] + o + 4 * GBM]));
        else
          w[ks][i] = *(const bf16x8*)&sW[st][woff[ks] + i * 32 * GBK];
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[ni][mi] = mfma32(w[ks][ni], x[ks][mi], acc[ni][mi]);
        __builtin_amdgcn_sched_barrier(0);
        if (kiss >= 0) issue_part(kiss, ks * 4 + ni);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < GSTAGES - 1; ++t)
    if (t < nk) issue(t);
  for (int kt = 0; kt < nk; ++kt) {
    // step kt's copies have landed (later steps' may still fly), for every wave
    const int ahead = min(nk - 1 - kt, GSTAGES - 2);
    if (ahead >= 2) vm_wait_keep<16>();
    else if (ahead == 1) vm_wait_keep<8>();
    else vm_wait_all();
    wg_barrier();
    // the stage step kt + 3 reuses was last read in step kt - 1, which every
    // wave has finished (barrier above)
    compute(kt % GSTAGES, kt + GSTAGES - 1 < nk ? kt + GSTAGES - 1 : -1);
  }

  // RoPE epilogue: rope slices are 64 columns starting at multiples of 64, so
  // a slice is N-tiles (2p, 2p+1) of a wave: rotate_half pair (i, i + 32) is
  // register e of tile 2p and of tile 2p+1 in the same lane; interleaved pairs
  // (2i, 2i+1) are neighbours in a lane's run of 4.  The cos / sin rows of the
  // tile's 256 output rows are staged in the freed operand LDS first (thread t
  // reads row t's, all in one memory round trip; NaN rows for positions
  // outside the table).  Every pair of the wave's two 64-column slices is
  // then rotated, the slices that are not rope slices by the angle 0
  // (cos 1, sin 0: the same finite values), so the epilogue has no branch.
  if (EPI == EPI_ROPE) {
    float rc[2], rs[2];                    // cos / sin override: (1, 0) outside rope slices
    bool on[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c0 = n0 + wn * 128 + p * 64;
      on[p] = c0 + 64 <= g.n && (c0 % g.rope_head_stride) == g.rope_off;
      rc[p] = 1.f;
      rs[p] = 0.f;
    }
    lds_wait_all();
    wg_barrier();                          // every wave is done with the operand stages
    float* tcs = (float*)smem;             // [256 rows][32], 16-byte chunk c of row r at c ^ (r & 7)
    float* tsn = tcs + GBM * 32;
    {
      const int pos = spos;
      const bool ok = pos >= 0 && pos < g.table_len;
      const float* cs = g.cos_t + (int64_t)(ok ? pos : 0) * 32;
      const float* sn = g.sin_t + (int64_t)(ok ? pos : 0) * 32;
      const float nan = __builtin_nanf("");
      const bool vec = ((reinterpret_cast<uintptr_t>(g.cos_t) | reinterpret_cast<uintptr_t>(g.sin_t)) & 15) == 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float4 cv = make_float4(nan, nan, nan, nan), sv = cv;
        if (ok && vec) {
          cv = *(const float4*)(cs + 4 * c);
          sv = *(const float4*)(sn + 4 * c);
        } else if (ok) {
          cv = make_float4(cs[4 * c], cs[4 * c + 1], cs[4 * c + 2], cs[4 * c + 3]);
          sv = make_float4(sn[4 * c], sn[4 * c + 1], sn[4 * c + 2], sn[4 * c + 3]);
        }
        *(float4*)&tcs[tid * 32 + ((c ^ (tid & 7)) << 2)] = cv;
        *(float4*)&tsn[tid * 32 + ((c ^ (tid & 7)) << 2)] = sv;
      }
    }
    lds_wait_all();
    wg_barrier();
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int ml = wm * 128 + mi * 32 + r32;
        const float* crow = tcs + ml * 32;
        const float* srow = tsn + ml * 32;
        if (!g.rope_interleave) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 c4 = *(const float4*)&crow[((2 * q + hs) ^ (ml & 7)) << 2];
            const float4 s4 = *(const float4*)&srow[((2 * q + hs) ^ (ml & 7)) << 2];
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float c = on[p] ? cv[e] : rc[p], ss = on[p] ? sv[e] : rs[p];
              const float x0 = acc[2 * p][mi][q * 4 + e], x1 = acc[2 * p + 1][mi][q * 4 + e];
              acc[2 * p][mi][q * 4 + e] = x0 * c - x1 * ss;
              acc[2 * p + 1][mi][q * 4 + e] = x1 * c + x0 * ss;
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; e += 2) {
                const int i = (t * 32 + q * 8 + hs * 4 + e) >> 1;
                const int at = (((i >> 2) ^ (ml & 7)) << 2) + (i & 3);
                const float c = on[p] ? crow[at] : rc[p], ss = on[p] ? srow[at] : rs[p];
                const float x0 = acc[2 * p + t][mi][q * 4 + e], x1 = acc[2 * p + t][mi][q * 4 + e + 1];
                acc[2 * p + t][mi][q * 4 + e] = x0 * c - x1 * ss;
                acc[2 * p + t][mi][q * 4 + e + 1] = x1 * c + x0 * ss;
              }
        }
      }
  }

  if constexpr (CT == 1) {
    // fp32 output (plain store): the lane's 4 consecutive columns of a row
    // leave as one 16-byte store, added to what C holds with c_acc
    float* C = (float*)g.c + (int64_t)blockIdx.z * g.c_bstride;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int m = m0 + wm * 128 + mi * 32 + r32;
        if (m >= g.m) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * 128 + ni * 32 + q * 8 + hs * 4;
          if (n >= g.n) continue;
          float4 v = make_float4(acc[ni][mi][q * 4 + 0], acc[ni][mi][q * 4 + 1], acc[ni][mi][q * 4 + 2],
                                 acc[ni][mi][q * 4 + 3]);
          float4* cp = (float4*)(C + (int64_t)m * g.ldc + n);
          if (g.c_acc) {
            const float4 o = *cp;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *cp = v;
        }
      }
    return;
  }

  if constexpr (CT == 3) {
    // MXFP8 output: an MX block is the 32 columns of one N-tile in one row,
    // 16 of them in this lane and 16 in lane l ^ 32 (same row): shared scale
    // 2^(floor(log2 amax) - 8) as an E8M0 byte, E4M3 codes saturating at
    // 448.  Codes go to an LDS tile [256 rows][256 B] (16 B chunk c of row r at
    // c ^ (r & 15)), scale bytes to [256 rows][8], then out as whole rows.
    lds_wait_all();
    wg_barrier();                          // every wave is done with the operand stages
    uint8_t* tile8 = (uint8_t*)smem;
    uint8_t* tsc = tile8 + GBM * GBN;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int ml = wm * 128 + mi * 32 + r32;
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, __builtin_fabsf(acc[ni][mi][e]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const int sb = max(0, min(254, (int)((__float_as_uint(amax) >> 23) & 255) - 8));
        const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);   // 2^(127 - sb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * 128 + ni * 32 + q * 8 + hs * 4;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = acc[ni][mi][q * 4 + e] * inv;
            y[e] = __builtin_fabsf(y[e]) > 448.f ? __builtin_copysignf(448.f, y[e]) : y[e];
          }
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          *(int*)(tile8 + ml * 256 + ((((nl >> 4) ^ (ml & 15))) << 4) + (nl & 15)) = w;
        }
        if (hs == 0) tsc[ml * 8 + wn * 4 + ni] = (uint8_t)sb;
      }
    lds_wait_all();
    wg_barrier();
    uint8_t* C8 = (uint8_t*)g.c + (int64_t)blockIdx.z * g.c_bstride;
#pragma unroll 4
    for (int i = 0; i < GBM * GBN / 16 / 256; ++i) {
      const int id = i * 256 + tid, r = id >> 4, c = id & 15;
      const int m = m0 + r, n = n0 + c * 16;
      if (m < g.m && n < g.n)
        *(uint4*)(C8 + (int64_t)m * g.ldc + n) = *(const uint4*)(tile8 + r * 256 + ((c ^ (r & 15)) << 4));
    }
    {
      const int r = tid, m = m0 + r;
      uint8_t* S = (uint8_t*)g.c_scale + (int64_t)m * g.ld_scale + n0 / 32;
      if (m < g.m)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n0 + 32 * j < g.n) S[j] = tsc[r * 8 + j];
    }
    return;
  }

  // Store through LDS: the lane holds output row wm*128 + mi*32 + lane%32 and,
  // per N-tile, 4 runs of 4 consecutive columns; those go to the LDS tile, and
  // the tile leaves as whole rows, 16 bytes per lane, consecutive lanes on
  // consecutive addresses.
  const bf16* G = (const bf16*)g.gate_src + (EPI == EPI_GATE ? (int64_t)blockIdx.z * g.c_bstride : 0);
  lds_wait_all();
  wg_barrier();                            // every wave is done with the operand stages
  char* tile = (char*)smem;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ml = wm * 128 + mi * 32 + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * 128 + ni * 32 + q * 8 + hs * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[ni][mi][q * 4 + e];
        if (EPI == EPI_GATE) {
          const int m = min(m0 + ml, g.m - 1), n = min(n0 + nl, g.n - 4);
          const bf16x4 gs = *(const bf16x4*)(G + (int64_t)m * g.ldg + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (float)gs[e] * (1.f / (1.f + __expf(-v[e])));
        }
        char* dst = tile + ml * 512 + ((((nl >> 3) ^ (ml & 31))) << 4) + ((nl >> 2) & 1) * 8;
        if (CT == 2) {
          f16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = to_f16_sat(v[e]);
          *(f16x4*)dst = o;
        } else {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *(bf16x4*)dst = o;
        }
      }
    }
  lds_wait_all();
  wg_barrier();
  char* C = (char*)g.c + ((int64_t)blockIdx.z * g.c_bstride) * 2;
#pragma unroll 4
  for (int i = 0; i < GBM * GBN * 2 / 16 / 256; ++i) {
    const int id = i * 256 + tid, r = id >> 5, c = id & 31;
    const int m = m0 + r, n = n0 + c * 8;
    if (m < g.m && n < g.n)
      *(uint4*)(C + ((int64_t)m * g.ldc + n) * 2) = *(const uint4*)(tile + r * 512 + ((c ^ (r & 31)) << 4));
  }
}

// fp32 kernel for the fp32 dtype: 16x16 outputs per 256-thread block, K tiles of
// 16 through LDS, one output per thread.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float sa[16][17], sb[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  const float* A = (const float*)g.a + (int64_t)blockIdx.z * g.a_bstride;
  const float* B = (const float*)g.b + (int64_t)blockIdx.z * g.b_bstride;
  float* C = (float*)g.c + (int64_t)blockIdx.z * g.c_bstride;
  float acc = 0.f;
  for (int k0 = 0; k0 < g.k; k0 += 16) {
    const int am = blockIdx.y * 16 + ty, ak = k0 + tx;
    sa[ty][tx] = (am < g.m && ak < g.k) ? A[(int64_t)am * g.lda + ak] : 0.f;
    const int bn = blockIdx.x * 16 + ty, bk = k0 + tx;   // sb[n][k]
    if (!g.b_kn)
      sb[ty][tx] = (bn < g.n && bk < g.k) ? B[(int64_t)bn * g.ldb + bk] : 0.f;
    else {
      const int kk = k0 + ty, nn = blockIdx.x * 16 + tx;    // B[k][n] -> sb[n][k]
      sb[tx][ty] = (kk < g.k && nn < g.n) ? B[(int64_t)kk * g.ldb + nn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sa[ty][kk], sb[tx][kk], acc);
    __syncthreads();
  }
  if (m < g.m && n < g.n) {
    if (EPI == EPI_GATE) {
      const float* G = (const float*)g.gate_src + (int64_t)blockIdx.z * g.c_bstride;
      acc = G[(int64_t)m * g.ldg + n] * (1.f / (1.f + expf(-acc)));
    }
    C[(int64_t)m * g.ldc + n] = acc;
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.m <= 0 || g.n <= 0 || g.batch <= 0) return hipSuccess;
  const int num_m = (g.m + BM - 1) / BM, num_n = (g.n + BN - 1) / BN;
  dim3 grid(num_m * num_n, 1, g.batch);
  const int ct = g.c_f32 ? 1 : (g.c_f16 ? 2 : 0);
  if (g.c_acc && (ct != 1 || g.c_mx)) return hipErrorInvalidValue;   // accumulation is for fp32 outputs
  // MXFP8 output: the 256x256 kernel whatever the grid size
  if (g.c_mx) {
    const bool ok = !g.b_kn && g.k >= GBK && g.k % GBK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.n % 32 == 0 &&
                    g.ldc % 16 == 0 && g.a_bstride % 8 == 0 && g.b_bstride % 8 == 0 &&
                    (int64_t)GBM * g.lda * 2 < ((int64_t)1 << 31) && (int64_t)GBN * g.ldb * 2 < ((int64_t)1 << 31) &&
                    (g.epilogue == EPI_STORE ||
                     (g.epilogue == EPI_ROPE && g.rope_head_stride % 64 == 0 && g.rope_off % 64 == 0));
    if (!ok) return hipErrorInvalidValue;
    dim3 gb((unsigned)(((g.m + GBM - 1) / GBM) * ((g.n + GBN - 1) / GBN)), 1, g.batch);
    if (g.epilogue == EPI_ROPE) gemm_bf16_big_kernel<EPI_ROPE, 3><<<gb, 256, 0, s>>>(g);
    else gemm_bf16_big_kernel<EPI_STORE, 3><<<gb, 256, 0, s>>>(g);
    return hipGetLastError();
  }
  // K-major operands: the 256x256 kernel, fp32 output, nothing else
  if (g.kmajor) {
    const bool ok = !g.b_kn && ct == 1 && g.epilogue == EPI_STORE && g.k >= GBK && g.k % GBK == 0 && g.m % 8 == 0 &&
                    g.n % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.lda >= g.m && g.ldb >= g.n &&
                    g.ldc % 4 == 0 && g.a_bstride % 8 == 0 && g.b_bstride % 8 == 0 &&
                    (int64_t)GBK * g.lda * 2 < ((int64_t)1 << 31) && (int64_t)GBK * g.ldb * 2 < ((int64_t)1 << 31);
    if (!ok) return hipErrorInvalidValue;
    dim3 gb((unsigned)(((g.m + GBM - 1) / GBM) * ((g.n + GBN - 1) / GBN)), 1, g.batch);
    gemm_bf16_big_kernel<EPI_STORE, 1, 3><<<gb, 256, 0, s>>>(g);
    return hipGetLastError();
  }
  // NN with fp32 output (B [k, n] K-major): the 256x256 kernel when its grid
  // covers every CU at least once, else the 128x128 kernel below
  if (g.b_kn) {
    const int64_t bm = (g.m + GBM - 1) / GBM, bn = (g.n + GBN - 1) / GBN;
    const bool ok = ct == 1 && g.epilogue == EPI_STORE && g.k >= GBK && g.k % GBK == 0 && g.n % 8 == 0 &&
                    g.lda % 8 == 0 && g.ldb % 8 == 0 && g.ldb >= g.n && g.ldc % 4 == 0 && g.a_bstride % 8 == 0 &&
                    g.b_bstride % 8 == 0 && (int64_t)GBM * g.lda * 2 < ((int64_t)1 << 31) &&
                    (int64_t)GBK * g.ldb * 2 < ((int64_t)1 << 31);
    if (ok && bm * bn * g.batch >= 256) {
      dim3 gb((unsigned)(bm * bn), 1, g.batch);
      gemm_bf16_big_kernel<EPI_STORE, 1, 2><<<gb, 256, 0, s>>>(g);
      return hipGetLastError();
    }
  }
  // the 256x256 kernel when its grid covers every CU at least once and the
  // operands suit its copies (K a multiple of 32, 16-byte rows and batch
  // strides, 256 rows of an operand within 32-bit byte offsets)
  {
    const int64_t bm = (g.m + GBM - 1) / GBM, bn = (g.n + GBN - 1) / GBN;
    const bool fits = !g.b_kn && (ct != 1 || (g.epilogue == EPI_STORE && g.ldc % 4 == 0 && g.n % 4 == 0)) &&
                      g.k >= GBK && g.k % GBK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
                      g.a_bstride % 8 == 0 && g.b_bstride % 8 == 0 && (int64_t)GBM * g.lda * 2 < ((int64_t)1 << 31) &&
                      (int64_t)GBN * g.ldb * 2 < ((int64_t)1 << 31) &&
                      (g.epilogue != EPI_ROPE || (g.rope_head_stride % 64 == 0 && g.rope_off % 64 == 0));
    if (fits && bm * bn * g.batch >= 256) {
      dim3 gb((unsigned)(bm * bn), 1, g.batch);
      if (g.epilogue == EPI_GATE) {
        if (ct != 0) return hipErrorInvalidValue;
        gemm_bf16_big_kernel<EPI_GATE, 0><<<gb, 256, 0, s>>>(g);
      } else if (g.epilogue == EPI_ROPE) {
        if (ct == 2) gemm_bf16_big_kernel<EPI_ROPE, 2><<<gb, 256, 0, s>>>(g);
        else gemm_bf16_big_kernel<EPI_ROPE, 0><<<gb, 256, 0, s>>>(g);
      } else if (ct == 2) {
        gemm_bf16_big_kernel<EPI_STORE, 2><<<gb, 256, 0, s>>>(g);
      } else if (ct == 1) {
        gemm_bf16_big_kernel<EPI_STORE, 1><<<gb, 256, 0, s>>>(g);
      } else {
        gemm_bf16_big_kernel<EPI_STORE, 0><<<gb, 256, 0, s>>>(g);
      }
      return hipGetLastError();
    }
  }
  if (g.b_kn) {
    if (g.epilogue != EPI_STORE || ct == 2) return hipErrorInvalidValue;
    if (ct == 1) gemm_bf16_kernel<true, EPI_STORE, 1><<<grid, NT, 0, s>>>(g);
    else gemm_bf16_kernel<true, EPI_STORE, 0><<<grid, NT, 0, s>>>(g);
  } else if (g.epilogue == EPI_GATE) {
    if (ct != 0) return hipErrorInvalidValue;
    gemm_bf16_kernel<false, EPI_GATE, 0><<<grid, NT, 0, s>>>(g);
  } else if (g.epilogue == EPI_ROPE) {
    if (ct == 1 || g.rope_head_stride % 64 || g.rope_off % 64) return hipErrorInvalidValue;
    if (ct == 2)
      gemm_bf16_kernel<false, EPI_ROPE, 2><<<grid, NT, 0, s>>>(g);
    else
      gemm_bf16_kernel<false, EPI_ROPE, 0><<<grid, NT, 0, s>>>(g);
  } else if (ct == 1) {
    gemm_bf16_kernel<false, EPI_STORE, 1><<<grid, NT, 0, s>>>(g);
  } else if (ct == 2) {
    gemm_bf16_kernel<false, EPI_STORE, 2><<<grid, NT, 0, s>>>(g);
  } else {
    gemm_bf16_kernel<false, EPI_STORE, 0><<<grid, NT, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.m <= 0 || g.n <= 0 || g.batch <= 0) return hipSuccess;
  if (g.epilogue == EPI_ROPE) return hipErrorInvalidValue;
  dim3 grid((g.n + 15) / 16, (g.m + 15) / 16, g.batch);
  if (g.epilogue == EPI_GATE)
    gemm_f32_kernel<EPI_GATE><<<grid, 256, 0, s>>>(g);
  else
    gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mla
