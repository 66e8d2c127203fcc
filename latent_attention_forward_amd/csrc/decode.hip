// Weight-absorbed MLA decode over the paged latent cache: split-KV attention in
// the 576-wide latent space and the log-sum-exp combine of the splits.
//
// Work split: the keys of all sequences, taken one sequence after another,
// form one long sequence; workgroup g takes the keys [g R, (g+1) R) of it (R,
// the quota, a multiple of 64 chosen so that about one workgroup per CU
// results), cut at each sequence boundary into segments.  A cut that falls
// inside a sequence is moved to the nearest multiple of 64 keys of that
// sequence (both workgroups sharing it round it the same way), so every
// workgroup gets R +- 64 keys whatever the length mix.  Segment (g, b) writes
// its partial result to slot g - floor(start_b / R) of sequence b.
//
// Split kernel: for every head at once, the partial softmax state of a
// segment's keys.  Each wave owns 32 heads (v_mfma_f32_32x32x16_bf16, one wave
// per SIMD so that the 32 x 512 fp32 accumulator and the query operand both
// stay in registers).  A tile of 32 cached rows [c_n (512) | k_pe' (64)] is
// copied into LDS once per workgroup (asynchronous global->LDS loads, three
// tiles in flight) and used twice:
//   S^T[key, head]  = C[key, :] . Qc[head, :]        (A = C rows, B = absorbed query)
//   O^T[dim, head] += C^T[dim, key] . P^T[key, head] (A = C^T by LDS transpose read)
// so each cached row is read from HBM exactly once per query group.  The
// absorbed query Qc = [W_UK^T q_nope | q_pe] stays in registers as the MFMA B
// operand for the whole segment.  The segment's block ids are staged in LDS
// first, so issuing a tile's loads never waits on a dependent global load.
//
// Softmax origin: the exponent origin of each head is the max of the
// segment's first tile and is never moved, so the accumulators are never
// rescaled.  Later scores may exceed it by up to 64 in log2 units
// (probabilities up to 2^64, exact in fp32 and in the bf16 exponent range).  A
// wave that meets a larger excursion recomputes its heads for the segment with
// an fp32 online softmax (decode_chunk_exact) instead.  Partial outputs are
// stored normalised (O / l, |O / l| <= max |c|) in fp16, with the origin and
// the sum per head in fp32.
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
__device__ __forceinline__ void decode_chunk_exact(const DecodeArgs& a, int b, int slot, int h0, int k0, int k1) {
  const int lane = threadIdx.x & 63;
  const int H = a.heads, lbs = a.log2_block, bmask = (1 << lbs) - 1;
  const float c2 = a.scale * kLog2e;
  const int64_t part = ((int64_t)b * a.max_slots + slot) * H;
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
    f16* po = a.part_o + (part + h) * RK + lane * 8;
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) po[e] = (f16)(acc[e] * inv);
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
  // This workgroup's keys [S0, S1) of the concatenated sequence: find the
  // first sequence that reaches past S0 (wave 0, a prefix sum of the lengths).
  const int cap = a.max_blocks << lbs;
  const int64_t R = a.quota;
  const int64_t S0 = (int64_t)blockIdx.x * R, S1 = S0 + R;
  __shared__ long long s_first[2];
  if (wave == 0) {
    if (lane == 0) { s_first[0] = a.batch; s_first[1] = 0; }
    long long seen = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      const int bb = b0 + lane;
      const long long n = (bb < a.batch) ? (long long)max(0, min(a.seq_lens[bb], cap)) : 0;
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
  for (; b < a.batch && st < S1; st += max(0, min(a.seq_lens[b], cap)), ++b) {
  __syncthreads();                         // the previous segment is done with sBlk and the tiles
  // Lane-dependent values are rebuilt per segment from an opaque copy of the
  // thread id, so none of them is kept live across the segment loop.
  int tid_s = tid;
  asm volatile("" : "+v"(tid_s));
  const int tid = tid_s, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = max(0, min(a.seq_lens[b], cap));
  // cut points inside the sequence move to the nearest multiple of 64 keys
  auto cut = [&](int64_t x) -> int {
    return x <= 0 ? 0 : (x >= L ? L : (int)min<int64_t>(L, ((x + 32) >> 6) << 6));
  };
  const int k0 = cut(S0 - st), k1 = cut(S1 - st);
  const int slot = (int)(blockIdx.x - st / R);
  const int64_t part = ((int64_t)b * a.max_slots + slot) * H;
  if (k0 >= k1) {                          // empty after the cut: weight 0 in the combine
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = -INFINITY; a.part_ml[(part + i) * 2 + 1] = 0.f; }
    continue;
  }
  const int nt = (k1 - k0 + DKT - 1) / DKT;

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
    for (int i = tid; i < H * RK; i += NTH) a.part_o[part * RK + i] = (f16)__builtin_nanf("");
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = 0.f; a.part_ml[(part + i) * 2 + 1] = __builtin_nanf(""); }
    continue;
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
  // the query must have landed before the tile copies go out: the copies are
  // issued from inline asm and the waits inside the tile loop only track them
  vm_wait_all();

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
  uint32_t doff[BPW];                      // byte offsets inside a tile of 32 contiguous rows
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int P = (wave + NW * i) * 64 + lane;
    const int r = P / CCH, pc = P - r * CCH;
    doff[i] = (uint32_t)((r * RC + ((pc ^ csw(r)) << 3)) * 2);
  }
  const uint32_t dst0 = lds_addr_of(&sC[0][0]) + (uint32_t)wave * 1024u;   // this wave's first block
  auto issue_tile = [&](int t, int buf) {
    const int kb = k0 + t * DKT;
    const uint32_t dst = dst0 + (uint32_t)buf * (DKT * RC * 2);
    if (lbs >= 5 && kb + DKT <= k1) {
      const bf16* tb = uniform_ptr(a.cache + (((int64_t)sBlk[(kb >> lbs) - blk0] << lbs) + (kb & bmask)) * RC);
#pragma unroll
      for (int i = 0; i < BPW; ++i) lds_dma16_sv_m0(tb, doff[i], dst + i * NW * 1024);
    } else {
#pragma unroll 1
      for (int i = 0; i < BPW; ++i) {
        const int blk = wave + NW * i;
        const int P = blk * 64 + lane;
        const int r = P / CCH, pc = P - r * CCH;
        const int key = (kb + r < k1) ? kb + r : k0;
        const int64_t row = ((int64_t)sBlk[(key >> lbs) - blk0] << lbs) + (key & bmask);
        lds_dma16_m0(a.cache + row * RC + ((pc ^ csw(r)) << 3), dst + i * NW * 1024);
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
    decode_chunk_exact(a, b, slot, wave * 32, k0, k1);
  } else {
    // lane holds head my_h, dims d*32 + q*8 + hsel*4 + [0,4); stored as O / l in fp16
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    f16* po = a.part_o + (part + my_h) * RK;
#pragma unroll
    for (int d = 0; d < RK / 32; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)(o[d][q * 4 + e] * inv);
        *(f16x4*)(po + d * 32 + q * 8 + hsel * 4) = v;
      }
    if (hsel == 0) {
      a.part_ml[(part + my_h) * 2 + 0] = m_ref;
      a.part_ml[(part + my_h) * 2 + 1] = l_tot;
    }
  }
  }
}

// Combine: o_lat[b, h, :] = sum_s w_s l_s (O_s / l_s) / sum_s w_s l_s over the
// sequence's slots s, with w_s = 2^((m_s - M) * c2); slots emptied by a cut
// (l_s = 0) are skipped.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.heads;
  const int cap = a.max_blocks << a.log2_block;
  // start of sequence b in the concatenated key sequence
  __shared__ long long s_part[2];
  long long st = 0;
  for (int i = tid; i < b; i += 128) st += max(0, min(a.seq_lens[i], cap));
  st = wave_sum_ll(st);
  if ((tid & 63) == 0) s_part[tid >> 6] = st;
  __syncthreads();
  st = s_part[0] + s_part[1];
  const int L = max(0, min(a.seq_lens[b], cap));
  const int64_t R = a.quota;
  const int nslot = L > 0 ? (int)((st + L - 1) / R - st / R + 1) : 0;
  const float c2 = a.scale * kLog2e;
  float M = -INFINITY;
  for (int sl = 0; sl < nslot; ++sl) {
    const int64_t part = ((int64_t)b * a.max_slots + sl) * H + h;
    if (a.part_ml[part * 2 + 1] != 0.f) M = fmaxf(M, a.part_ml[part * 2]);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int sl = 0; sl < nslot; ++sl) {
    const int64_t part = ((int64_t)b * a.max_slots + sl) * H + h;
    const float l = a.part_ml[part * 2 + 1];
    if (l == 0.f) continue;
    const float w = __builtin_amdgcn_exp2f((a.part_ml[part * 2] - M) * c2) * l;
    lsum += w;
    const f16x4 v = *(const f16x4*)(a.part_o + part * RK + tid * 4);
    acc.x += w * (float)v[0]; acc.y += w * (float)v[1]; acc.z += w * (float)v[2]; acc.w += w * (float)v[3];
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
