// Weight-absorbed MLA decode over the paged latent cache: split-KV attention in
// the 576-wide latent space and the log-sum-exp combine of the splits.
//
// Split kernel: one workgroup per (sequence, chunk of keys) computes, for every
// head at once, the partial softmax state of its keys.  Each of its waves owns
// 32 heads (v_mfma_f32_32x32x16_bf16, one wave per SIMD so that the 32 x 512
// fp32 accumulator and the query operand both stay in registers).  A tile of
// 64 cached rows [c_n (512) | k_pe' (64)] is copied into LDS once per
// workgroup (asynchronous global->LDS loads, double buffered) and used twice:
//   S^T[key, head]  = C[key, :] . Qc[head, :]        (A = C rows, B = absorbed query)
//   O^T[dim, head] += C^T[dim, key] . P^T[key, head] (A = C^T by LDS transpose read)
// so each cached row is read from HBM exactly once per query group.  The
// absorbed query Qc = [W_UK^T q_nope | q_pe] stays in registers as the MFMA B
// operand for the whole chunk.  The chunk's block ids are staged in LDS first,
// so issuing a tile's loads never waits on a dependent global load.
//
// Softmax origin: the exponent origin of each head is the max of the chunk's
// first tile and is never moved, so the accumulators are never rescaled.
// Later scores may exceed it by up to 64 in log2 units (probabilities up to
// 2^64, exact in fp32 and in the bf16 exponent range).  A wave that meets a
// larger excursion recomputes its heads for the chunk with an fp32 online
// softmax (decode_chunk_exact) instead.  Partial outputs are unnormalised fp32
// with the origin and the sum per head.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int DKT = 32;                    // keys per tile
constexpr int NBUF = 4;                    // LDS tile buffers (NBUF - 1 tiles in flight)
constexpr int RC = 576, RK = 512, DRP = 64;
constexpr int CCH = RC / 8;                // 16 B chunks per cached row (72)
constexpr float kMaxExcursion = 64.f;      // log2 units above the origin

// Cache tile [64 keys][576]: chunk c of row r at c ^ sw(r).  sw maps any 8
// consecutive rows to distinct values (row reads of the score MFMA) and any 4
// rows 4a..4a+3 to distinct 32 B pairs (transpose reads of the PV MFMA).
__device__ __forceinline__ int csw(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// fp32 online softmax over keys [k0, k1) of sequence b for heads [h0, h0 + 32),
// one wave, reading the cache from global memory; writes the partials.  Used
// only by a wave whose scores left the range of its fixed exponent origin.
__device__ __forceinline__ void decode_chunk_exact(const DecodeArgs& a, int b, int c, int h0, int k0,
                                                             int k1) {
  const int lane = threadIdx.x & 63;
  const int H = a.heads, lbs = a.log2_block, bmask = (1 << lbs) - 1;
  const float c2 = a.scale * kLog2e;
  const int64_t part = ((int64_t)b * a.max_chunks + c) * H;
  for (int h = h0; h < h0 + 32; ++h) {
    const bf16* qt = a.qt + ((int64_t)b * H + h) * RK;
    const bf16* qp = a.q_pe + ((int64_t)b * H + h) * DRP;
    float q[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int d = lane + 64 * i;
      q[i] = d < RK ? (float)qt[d] : (float)qp[d - RK];
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int j = k0; j < k1; ++j) {
      const int64_t row = ((int64_t)a.block_table[(int64_t)b * a.max_blocks + (j >> lbs)] << lbs) + (j & bmask);
      const bf16* cr = a.cache + row * RC;
      float part_s = 0.f;
#pragma unroll
      for (int i = 0; i < 9; ++i) part_s = fmaf(q[i], (float)cr[lane + 64 * i], part_s);
      const float sj = wave_sum(part_s);
      const float mn = fmaxf(m, sj);
      const float al = __builtin_amdgcn_exp2f((m - mn) * c2), p = __builtin_amdgcn_exp2f((sj - mn) * c2);
      l = l * al + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * al + p * (float)cr[lane * 8 + e];
      m = mn;
    }
    float* po = a.part_o + (part + h) * RK + lane * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) po[e] = acc[e];
    if (lane == 0) {
      a.part_ml[(part + h) * 2 + 0] = m;
      a.part_ml[(part + h) * 2 + 1] = l;
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_kernel(DecodeArgs a) {
  constexpr int NTH = NW * 64;
  constexpr int BLOCKS = DKT * CCH / 64;            // 1 KB LDS blocks per tile (36)
  static_assert(BLOCKS % NW == 0, "tile must split evenly over the waves");
  constexpr int BPW = BLOCKS / NW;
  __shared__ __attribute__((aligned(16))) bf16 sC[NBUF][DKT * RC];
  __shared__ int sBlk[kDecodeMaxChunkBlocks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads;
  const int lbs = a.log2_block, bmask = (1 << lbs) - 1;
  // Work item blockIdx.x -> (sequence b, chunk c): items are numbered sequence
  // by sequence, so consecutive workgroups (dealt round-robin to the XCDs)
  // spread every sequence's chunks over all XCDs.
  __shared__ int s_item[2];
  if (wave == 0) {
    if (lane == 0) { s_item[0] = -1; s_item[1] = 0; }
    int seen = 0;
    const int id = blockIdx.x;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      const int bb = b0 + lane;
      int n = 0;
      if (bb < a.batch) n = (min(a.seq_lens[bb], a.max_blocks << lbs) + a.chunk - 1) / a.chunk;
      int incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (id >= seen + incl - n && id < seen + incl) { s_item[0] = bb; s_item[1] = id - (seen + incl - n); }
      seen += __shfl(incl, 63, 64);
      if (seen > id) break;
    }
  }
  __syncthreads();
  const int b = s_item[0], c = s_item[1];
  if (b < 0) return;
  const int L = min(a.seq_lens[b], a.max_blocks << lbs);
  const int k0 = c * a.chunk;
  if (k0 >= L) return;
  const int k1 = min(k0 + a.chunk, L);
  const int nt = (k1 - k0 + DKT - 1) / DKT;
  const int64_t part = ((int64_t)b * a.max_chunks + c) * H;

  // the chunk's block ids; an id outside the pool poisons this sequence's output
  const int blk0 = k0 >> lbs;
  const int nblk = ((k1 - 1) >> lbs) - blk0 + 1;
  int bad = 0;
  for (int i = tid; i < nblk; i += NTH) {
    const int v = a.block_table[(int64_t)b * a.max_blocks + blk0 + i];
    bad |= (v < 0 || v >= a.num_blocks);
    sBlk[i] = v;
  }
  if (__syncthreads_or(bad)) {
    for (int i = tid; i < H * RK; i += NTH) a.part_o[part * RK + i] = __builtin_nanf("");
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = 0.f; a.part_ml[(part + i) * 2 + 1] = __builtin_nanf(""); }
    return;
  }

  const int hsel = lane >> 5;
  const int my_h = wave * 32 + (lane & 31);
  bf16x8 qreg[RC / 16];
  {
    const bf16* qt = a.qt + ((int64_t)b * H + my_h) * RK;
    const bf16* qp = a.q_pe + ((int64_t)b * H + my_h) * DRP;
#pragma unroll
    for (int ks = 0; ks < RC / 16; ++ks) {
      const int d = ks * 16 + hsel * 8;
      qreg[ks] = (d < RK) ? *(const bf16x8*)(qt + d) : *(const bf16x8*)(qp + d - RK);
    }
  }

  // Lane-constant parts of the swizzled LDS addresses (elements); the rest of
  // every address is a compile-time offset.
  //  score read (mt, ks): row mt*32 + lane%32, chunk ks*2 + hsel
  const int rs = lane & 31, sws = csw(rs & 7);
  int base_s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) base_s[q] = rs * RC + ((((q * 2 + hsel) ^ sws)) << 3);
  //  transpose read (j, half, d): row (j/2)*32 + (j%2)*16 + half*8 + rt, column d*32 + (g&1)*16 + 4*(L%4)
  const int grp = lane >> 4, L4 = lane & 15;
  const int rt = (grp >> 1) * 4 + (L4 >> 2), swt = csw(rt & 7);
  const int xb = (L4 >> 1) & 1;
  int base_t[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) base_t[q] = rt * RC + ((((q * 4 + (grp & 1) * 2 + xb) ^ swt)) << 3) + 4 * (L4 & 1);

  // Tile loads.  A full tile in one block (blocks of >= 32 tokens) is 32
  // contiguous cache rows, so each lane's BPW source offsets are fixed for the
  // whole chunk.  The chunk's last, partial tile and blocks of 16 tokens take
  // the per-row path (rows past the chunk are clamped to its first key, whose
  // probability is masked to 0).
  int doff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int P = (wave + NW * i) * 64 + lane;
    const int r = P / CCH, pc = P - r * CCH;
    doff[i] = r * RC + ((pc ^ csw(r)) << 3);
  }
  auto issue_tile = [&](int t, int buf) {
    const int kb = k0 + t * DKT;
    if (lbs >= 5 && kb + DKT <= k1) {
      const bf16* tb = a.cache + (((int64_t)sBlk[(kb >> lbs) - blk0] << lbs) + (kb & bmask)) * RC;
#pragma unroll
      for (int i = 0; i < BPW; ++i) lds_dma16(tb + doff[i], &sC[buf][(wave + NW * i) * 512]);
    } else {
#pragma unroll 1
      for (int i = 0; i < BPW; ++i) {
        const int blk = wave + NW * i;
        const int P = blk * 64 + lane;
        const int r = P / CCH, pc = P - r * CCH;
        const int key = (kb + r < k1) ? kb + r : k0;
        const int64_t row = ((int64_t)sBlk[(key >> lbs) - blk0] << lbs) + (key & bmask);
        lds_dma16(a.cache + row * RC + ((pc ^ csw(r)) << 3), &sC[buf][blk * 512]);
      }
    }
  };

  const float c2 = a.scale * kLog2e;
  float m_ref = -INFINITY, l_run = 0.f;
  bool exact_path = false;   // wave-uniform; once set, this wave's tile results are discarded
  f32x16 o[RK / 32];
#pragma unroll
  for (int d = 0; d < RK / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;

  // NBUF - 1 tiles in flight: tile t + NBUF - 1 is requested while tile t is
  // multiplied.  Each wave issues BPW loads per tile; before a barrier it waits
  // until the next tile's loads are done and keeps the newer tiles' pending.
  static_assert(NBUF == 4, "wait_tile is written for 3 tiles in flight");
  constexpr int KEEP2 = (2 * BPW < 64) ? 2 * BPW : BPW;   // vmcnt holds at most 63
  auto wait_tile = [&](int newer) {          // newer: tiles issued after the awaited one
    if (newer >= 2) vm_wait_keep<KEEP2>();
    else if (newer == 1) vm_wait_keep<BPW>();
    else vm_wait_all();
  };
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < nt) issue_tile(t, t);
  wait_tile(min(NBUF - 2, nt - 1));
  wg_barrier();
  for (int t = 0; t < nt; ++t) {
    const int buf = t % NBUF;
    const int kb = k0 + t * DKT;
    if (t + NBUF - 1 < nt) issue_tile(t + NBUF - 1, (t + NBUF - 1) % NBUF);
    {
      const bf16* sb = sC[buf];
      constexpr int MT = DKT / 32;
      f32x16 s[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
      {
        // software-pipelined operand reads: step i = (mt, ks) reads 4 steps ahead
        constexpr int NS = MT * (RC / 16), D = 4;
        auto addr = [&](int i) { const int mt = i / (RC / 16), ks = i % (RC / 16);
                                 return sb + base_s[ks & 3] + mt * 32 * RC + (ks >> 2) * 64; };
        bf16x8 cf[D];
#pragma unroll
        for (int i = 0; i < D; ++i) cf[i] = *(const bf16x8*)addr(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const bf16x8 cur = cf[i % D];
          if (i + D < NS) cf[i % D] = *(const bf16x8*)addr(i + D);
          const int mt = i / (RC / 16), ks = i % (RC / 16);
          s[mt] = mfma32(cur, qreg[ks], s[mt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // lane holds head my_h, keys mt*32 + (e/4)*8 + hsel*4 + e%4
      if (kb + DKT > k1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3) >= k1) s[mt][e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (t == 0) m_ref = mx;                       // the first tile holds at least one key
      exact_path |= __builtin_amdgcn_ballot_w64((mx - m_ref) * c2 > kMaxExcursion) != 0;
      {
        const float mb = m_ref * c2;
        bf16x8 pb[2 * MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][e], c2, -mb));
            l_run += p;
            pb[mt * 2 + (e >> 3)][e & 7] = (bf16)p;
          }
        // O^T += C^T P^T; step j covers keys (j/2)*32 + (j%2)*16 + {h*4 + [0,4), 8 + h*4 + [0,4)}
        {
          // software-pipelined transpose reads: step i = (j, d) reads 4 steps ahead
          constexpr int NP = 2 * MT * (RK / 32), D = 4;
          auto taddr = [&](int i) { const int j = i / (RK / 32), d = i % (RK / 32);
                                    return sb + base_t[d & 1] + ((j >> 1) * 32 + (j & 1) * 16) * RC + (d >> 1) * 64; };
          bf16x4 lo[D], hi[D];
#pragma unroll
          for (int i = 0; i < D; ++i) { lo[i] = lds_read_tr(taddr(i)); hi[i] = lds_read_tr(taddr(i) + 8 * RC); }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const bf16x8 cur = cat8(lo[i % D], hi[i % D]);
            if (i + D < NP) { lo[i % D] = lds_read_tr(taddr(i + D)); hi[i % D] = lds_read_tr(taddr(i + D) + 8 * RC); }
            const int j = i / (RK / 32), d = i % (RK / 32);
            o[d] = mfma32(cur, pb[j], o[d]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    // tile t + 1 must have landed; newer tiles may still be in flight
    wait_tile(min(NBUF - 2, nt - 2 - t));
    wg_barrier();
  }

  if (exact_path) {
    decode_chunk_exact(a, b, c, wave * 32, k0, k1);
    return;
  }
  // lane holds head my_h, dims d*32 + q*8 + hsel*4 + [0,4)
  float* po = a.part_o + (part + my_h) * RK;
#pragma unroll
  for (int d = 0; d < RK / 32; ++d)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(po + d * 32 + q * 8 + hsel * 4) = make_float4(o[d][q * 4], o[d][q * 4 + 1], o[d][q * 4 + 2], o[d][q * 4 + 3]);
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (hsel == 0) {
    a.part_ml[(part + my_h) * 2 + 0] = m_ref;
    a.part_ml[(part + my_h) * 2 + 1] = l_tot;
  }
}

// Combine: o_lat[b, h, :] = sum_c w_c o_c / sum_c w_c l_c with w_c = 2^((m_c - M) * c2).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.heads;
  const int L = min(a.seq_lens[b], a.max_blocks << a.log2_block);
  const int nch = min((L + a.chunk - 1) / a.chunk, a.max_chunks);
  const float c2 = a.scale * kLog2e;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, a.part_ml[(((int64_t)b * a.max_chunks + c) * H + h) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int64_t part = ((int64_t)b * a.max_chunks + c) * H + h;
    const float w = __builtin_amdgcn_exp2f((a.part_ml[part * 2] - M) * c2);
    lsum += w * a.part_ml[part * 2 + 1];
    const float4 v = *(const float4*)(a.part_o + part * RK + tid * 4);
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  const float inv = 1.f / lsum;
  bf16x4 r;
  r[0] = (bf16)(acc.x * inv); r[1] = (bf16)(acc.y * inv); r[2] = (bf16)(acc.z * inv); r[3] = (bf16)(acc.w * inv);
  *(bf16x4*)(a.o_lat + ((int64_t)b * H + h) * RK + tid * 4) = r;
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s) {
  if (a.num_items <= 0) return hipSuccess;
  dim3 grid(a.num_items);
  switch (a.heads) {
    case 32: decode_split_kernel<1><<<grid, 64, 0, s>>>(a); break;
    case 64: decode_split_kernel<2><<<grid, 128, 0, s>>>(a); break;
    case 96: decode_split_kernel<3><<<grid, 192, 0, s>>>(a); break;
    case 128: decode_split_kernel<4><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.heads, a.batch);
  decode_combine_kernel<<<grid, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
