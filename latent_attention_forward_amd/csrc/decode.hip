// Weight-absorbed MLA decode over the paged latent cache: split-KV attention in
// the 576-wide latent space, then the log-sum-exp combine of the splits fused
// with the W_UV un-absorb.
//
// Work split: the keys of all sequences, taken one sequence after another,
// each preceded by kDecodeSegmentCost placeholder keys (the fixed cost of a
// segment, charged to the workgroup that starts the sequence), form one long
// sequence; workgroup g takes the keys [g R, (g+1) R) of it (R, the quota, a
// multiple of 32 chosen so that about one workgroup per CU results), cut at
// each sequence boundary into segments.  A cut that falls
// inside a sequence is moved to the nearest multiple of 32 keys of that
// sequence (both workgroups sharing it round it the same way), so every
// workgroup gets R +- 32 keys of work whatever the length mix.  Segment (g, b)
// is slot g - floor(r_b / R) of sequence b (r_b the position of b's first
// key) and writes its partial result to entry g + b of the partial buffers.
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

// Cache tile [32 keys][576]: chunk c of row r at c ^ sw(r), sw(r) a
// permutation of row bits 1..3.  A row is 4.5 x 256 B, so rows of one parity
// start at the same bank; sw spreads the 16 rows that one 16-lane phase of a
// score-operand read (ds_read_b128) touches over all 64 banks, and keeps the
// transpose reads of the PV operand (rows 4a .. 4a + 3 and 4a + 4 .. 4a + 7
// in one 32-lane phase) on distinct banks too.  sw(r + 8) = sw(r) ^ 2 and
// sw(r + 16) = sw(r).
__device__ __forceinline__ int csw(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1); }

// fp32 online softmax over keys [k0, k1) of sequence b for heads [h0, h0 + 32),
// one wave, reading the cache from global memory; writes the partials.  Used
// only by a wave whose scores left the range of its fixed exponent origin.
__device__ __forceinline__ void decode_chunk_exact(const DecodeArgs& a, int b, int64_t part, int h0, int k0, int k1) {
  const int lane = threadIdx.x & 63;
  const int H = a.heads, lbs = a.log2_block, bmask = (1 << lbs) - 1;
  const float c2 = a.scale * kLog2e;
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
  __shared__ int s_badw[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads;
  const int lbs = a.log2_block, bmask = (1 << lbs) - 1;
  // This workgroup's keys [S0, S1) of the concatenated sequence: find the
  // first sequence that reaches past S0 (wave 0, a prefix sum of the lengths).
  const int cap = a.max_blocks << lbs;
  const int64_t R = a.quota;
  // Work item of this workgroup.  Workgroup x runs on XCD x % 8; consecutive
  // items, which mostly share a sequence and so its query, go to one XCD so
  // that the query is read from that XCD's L2 after the first of them.
  const int G = gridDim.x, g8 = G >> 3, r8 = G & 7, xc = blockIdx.x & 7;
  const int item = xc * g8 + min(xc, r8) + (int)(blockIdx.x >> 3);
  const int64_t S0 = (int64_t)item * R, S1 = S0 + R;
  __shared__ long long s_first[2];
  // length of sequence b in the work order (its keys plus the placeholders)
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
  // Lane-dependent values are rebuilt per segment from an opaque copy of the
  // thread id, so none of them is kept live across the segment loop.
  int tid_s = tid;
  asm volatile("" : "+v"(tid_s));
  const int tid = tid_s, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = max(0, min(a.seq_lens[b], cap));
  const int64_t r0 = st + kDecodeSegmentCost;   // work-order position of key 0 of b
  if (L == 0 || S1 <= r0) continue;             // none of b's keys fall to this workgroup
  // cut points inside the sequence move to the nearest multiple of 32 keys (one tile)
  auto cut = [&](int64_t x) -> int {
    return x <= 0 ? 0 : (x >= L ? L : (int)min<int64_t>(L, ((x + 16) >> 5) << 5));
  };
  const int k0 = cut(S0 - r0), k1 = cut(S1 - r0);
  // entry item + b of the partial buffers (num_items + batch entries, item <
  // num_items and b < batch by the loops): in bounds whatever the lengths
  const int64_t part = ((int64_t)item + b) * H;
  if (k0 >= k1) {                          // empty after the cut: weight 0 in the combine
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = -INFINITY; a.part_ml[(part + i) * 2 + 1] = 0.f; }
    continue;
  }
  const int nt = (k1 - k0 + DKT - 1) / DKT;

  // The chunk's block ids are requested first, then the absorbed query; the
  // ids are waited for (loads complete in order) while the query is still in
  // flight.  An id outside the pool poisons this sequence's output.
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
  bf16x8 qreg[RC / 16];                  // absorbed query, in registers for the whole segment
  {
    const bf16* qt = a.qt + ((int64_t)b * H + my_h) * RK;
    const bf16* qp = a.q_pe + ((int64_t)b * H + my_h) * DRP;
#pragma unroll
    for (int ks = 0; ks < RC / 16; ++ks) {
      const int d = ks * 16 + hsel * 8;
      qreg[ks] = (d < RK) ? *(const bf16x8*)(qt + d) : *(const bf16x8*)(qp + d - RK);
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
  // workgroup OR of the flags, one word per wave (no zeroing needed), behind
  // an LDS-only wait so that the query stays in flight
  const bool wbad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (lane == 0) s_badw[wave] = wbad;
  lds_wait_all();
  wg_barrier();
  int anybad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) anybad |= s_badw[w];
  if (anybad) {
    for (int i = tid; i < H * RK; i += NTH) a.part_o[part * RK + i] = (f16)__builtin_nanf("");
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = 0.f; a.part_ml[(part + i) * 2 + 1] = __builtin_nanf(""); }
    continue;
  }

  // Lane-constant parts of the swizzled LDS addresses (elements); the rest of
  // every address is a compile-time offset.
  //  score read (mt, ks): row mt*32 + lane%32, chunk ks*2 + hsel
  const int rs = lane & 31, sws = csw(rs);
  int base_s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) base_s[q] = rs * RC + ((((q * 2 + hsel) ^ sws)) << 3);
  //  transpose read (j, half, d): row j*16 + half*8 + rt, column d*32 + (g&1)*16 + 4*(L%4);
  //  the rows of half 1 carry the swizzle of rt ^ 8
  const int grp = lane >> 4, L4 = lane & 15;
  const int rt = (grp >> 1) * 4 + (L4 >> 2), swt = csw(rt);
  const int xb = (L4 >> 1) & 1;
  int base_t[2], base_th[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    base_t[q] = rt * RC + ((((q * 4 + (grp & 1) * 2 + xb) ^ swt)) << 3) + 4 * (L4 & 1);
    base_th[q] = (rt + 8) * RC + ((((q * 4 + (grp & 1) * 2 + xb) ^ csw(rt + 8))) << 3) + 4 * (L4 & 1);
  }

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

  // Pipelined tile loop.  In iteration t the scores of tile t + 1 are formed
  // on the MFMA unit (accumulated in VGPRs, inline asm) while the softmax of
  // tile t runs on the VALU between those MFMAs; then PV(t) accumulates into
  // the AGPR-resident output.  Tile t + 3 is requested at the start of
  // iteration t (ring of NBUF = 4 LDS buffers); at its end tile t + 2 must
  // have landed (the copies of tile t + 3, BPW per wave, may still fly).
  static_assert(NBUF == 4, "the pipeline is written for a ring of 4 tiles");
  auto s_tile = [&](f32x16& s, int buf, auto&& group) __attribute__((always_inline)) {
    const bf16* sb = sC[buf];
    constexpr int NS = RC / 16, D = 4;
    auto addr = [&](int i) { return sb + base_s[i & 3] + (i >> 2) * 64; };
    bf16x8 cf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) cf[i] = *(const bf16x8*)addr(i);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NS>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      const bf16x8 cur = cf[i % D];
      if constexpr (i + D < NS) cf[i % D] = *(const bf16x8*)addr(i + D);
      if constexpr (i == 0) mfma32_vacc0(s, cur, qreg[0]);
      else mfma32_vacc(s, cur, qreg[i]);
      group(I);
      __builtin_amdgcn_sched_barrier(0);
    });
    mfma_result_wait();                  // the VALU reads s next
  };
  // softmax of one tile: prep (mask, max, excursion check), then 16 probabilities
  // in groups interleaved with the next tile's MFMAs
  float mb = 0.f;
  bf16x8 pb[2];
  float mx_part = 0.f;
  auto prep_a = [&](f32x16& s, int t) __attribute__((always_inline)) {   // mask, lane max
    const int kb = k0 + t * DKT;
    if (kb + DKT > k1) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kb + (e >> 2) * 8 + hsel * 4 + (e & 3) >= k1) s[e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
    mx_part = mx;
  };
  auto prep_b = [&](int t) __attribute__((always_inline)) {   // head max, origin, excursion check
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx_part), __float_as_uint(mx_part), false, false);
    const float mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    if (t == 0) m_ref = mx;                       // the first tile holds at least one key
    exact_path |= __builtin_amdgcn_ballot_w64((mx - m_ref) * c2 > kMaxExcursion) != 0;
    mb = m_ref * c2;
  };
  // The opaque statement keeps each probability between the MFMAs it was
  // placed among: without it the compiler sinks all of them past the branches
  // of the copy issue, into one block of VALU work that stalls the MFMA chain.
  auto prob = [&](f32x16& s, int e) __attribute__((always_inline)) {
    float p = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -mb));
    asm volatile("" : "+v"(p));
    pb[e >> 3][e & 7] = (bf16)p;
  };
  // The softmax denominator sums the same bf16-rounded probabilities the PV
  // MFMA multiplies, so that rounding P scales numerator and denominator alike.
  auto psum = [&]() __attribute__((always_inline)) { l_run = sum8(pb[1], sum8(pb[0], l_run)); };
  auto no_group = [](auto) {};
  // O^T += C^T P^T; step j covers keys j*16 + {h*4 + [0,4), 8 + h*4 + [0,4)}
  auto pv_tile = [&](int buf) __attribute__((always_inline)) {
    const bf16* sb = sC[buf];
    constexpr int NP = 2 * (RK / 32), D = 4;
    auto taddr = [&](int i) { const int j = i / (RK / 32), d = i % (RK / 32);
                              return sb + base_t[d & 1] + (j * 16) * RC + (d >> 1) * 64; };
    auto thaddr = [&](int i) { const int j = i / (RK / 32), d = i % (RK / 32);
                               return sb + base_th[d & 1] + (j * 16) * RC + (d >> 1) * 64; };
    bf16x4 lo[D], hi[D];
#pragma unroll
    for (int i = 0; i < D; ++i) { lo[i] = lds_read_tr(taddr(i)); hi[i] = lds_read_tr(thaddr(i)); }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const bf16x8 cur = cat8(lo[i % D], hi[i % D]);
      if (i + D < NP) { lo[i % D] = lds_read_tr(taddr(i + D)); hi[i % D] = lds_read_tr(thaddr(i + D)); }
      const int j = i / (RK / 32), d = i % (RK / 32);
      o[d] = mfma32(cur, pb[j], o[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Iteration t: the MFMAs of S(t + 1) carry, between them, the softmax
  // preparation of tile t (MFMAs 0 and 1), its 16 probabilities (odd MFMAs 3
  // to 33) and the copies of tile t + 3 (spread evenly over MFMAs 4 to 33, so
  // that the address unit the four waves share keeps up with them; the source
  // block is read from LDS at MFMA 0), so the MFMA unit waits for none of them.
  auto step = [&](int t, f32x16& s_cur, f32x16& s_nxt) __attribute__((always_inline)) {
    const int kn = k0 + (t + 3) * DKT;
    const bool issue = t + 3 < nt, fast = lbs >= 5 && kn + DKT <= k1;
    const uint32_t dstn = dst0 + (uint32_t)((t + 3) % NBUF) * (DKT * RC * 2);
    if (issue && !fast) issue_tile(t + 3, (t + 3) % NBUF);
    if (t + 1 < nt) {
      const bf16* tb = nullptr;
      s_tile(s_nxt, (t + 1) % NBUF, [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) {
          prep_a(s_cur, t);
          if (issue && fast) tb = uniform_ptr(a.cache + (((int64_t)sBlk[(kn >> lbs) - blk0] << lbs) + (kn & bmask)) * RC);
        }
        if constexpr (i == 1) prep_b(t);
        if constexpr (i >= 3 && i <= 33 && (i & 1)) prob(s_cur, (i - 3) >> 1);
        if constexpr (i == 35) psum();
        if constexpr (i >= 4 && i < 34) {            // copy k at MFMA 4 + floor(30 k / BPW)
          constexpr int ka = ((i - 4) * BPW + 29) / 30;
          if constexpr (ka < BPW && 4 + ka * 30 / BPW == i)
            if (issue && fast) lds_dma16_sv_m0(tb, doff[ka], dstn + ka * NW * 1024);
          if constexpr (ka + 1 < BPW && 4 + (ka + 1) * 30 / BPW == i)
            if (issue && fast) lds_dma16_sv_m0(tb, doff[ka + 1], dstn + (ka + 1) * NW * 1024);
        }
      });
    } else {
      if (issue && fast) issue_tile(t + 3, (t + 3) % NBUF);
      prep_a(s_cur, t);
      prep_b(t);
#pragma unroll
      for (int e = 0; e < 16; ++e) prob(s_cur, e);
      psum();
    }
    pv_tile(t % NBUF);
    if (t + 3 < nt) vm_wait_keep<BPW>();   // tile t + 2 landed, t + 3 may fly
    else vm_wait_all();
    wg_barrier();
  };

  // Tiles 0 and 1 and the query land before the loop starts; tile 2 is
  // requested after that, so the waits inside the loop count only tile
  // copies (the compiler's own waits for the query are all met here: the
  // empty statements use every query register).
  issue_tile(0, 0);
  if (1 < nt) issue_tile(1, 1);
  vm_wait_all();
#pragma unroll
  for (int ks = 0; ks < RC / 16; ++ks) asm volatile("" : : "v"(qreg[ks]));
  wg_barrier();
  if (2 < nt) issue_tile(2, 2);
  f32x16 sa, sbv;
  s_tile(sa, 0, no_group);
  for (int t = 0; t < nt; ++t) {
    step(t, sa, sbv);
    sa = sbv;                             // the next tile's scores become the current ones
  }

  if (exact_path) {
    decode_chunk_exact(a, b, part, wave * 32, k0, k1);
  } else {
    // Lane holds head my_h, dims d*32 + q*8 + hsel*4 + [0,4).  O / l goes in
    // fp16 through this wave's 32 KB of the (now idle) tile buffers, as 32 rows
    // of 1 KB with 16 B chunk c of row r at c ^ (r & 15), and leaves as one 1 KB
    // row per store.
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    char* wb = (char*)&sC[0][0] + wave * (32 * RK * 2);
    const int hl = lane & 31;
#pragma unroll
    for (int d = 0; d < RK / 32; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)(o[d][q * 4 + e] * inv);
        *(f16x4*)(wb + hl * (RK * 2) + (((d * 4 + q) ^ (hl & 15)) << 4) + hsel * 8) = v;
      }
    f16* po = a.part_o + (part + wave * 32) * RK + lane * 8;
#pragma unroll
    for (int r = 0; r < 32; ++r)
      *(f16x8*)(po + r * RK) = *(const f16x8*)(wb + r * (RK * 2) + ((lane ^ (r & 15)) << 4));
    if (hsel == 0) {
      a.part_ml[(part + my_h) * 2 + 0] = m_ref;
      a.part_ml[(part + my_h) * 2 + 1] = l_tot;
    }
  }
  }
}

// Query absorption: qt[b, h, :] = W_UK[h]^T q_nope[b, h, :] for every
// sequence, with W_UK[h] the [128, 512] block of W_kv_b rows of head h.
// Workgroup (256 latent columns c0.., head h), one per CU: the [128 x 256]
// slab of W_UK[h] (64 KB) is copied to LDS (16 B chunk c of row k at
// c ^ 2 (k & 3)) and read back transposed as the A operand of 32x32x16
// MFMAs, D^T[col, b] = W^T[col, :] . q^T[:, b]; wave w takes columns c0 + 64 w
// .. + 63 (two blocks of 32) for every sequence, 64 at a time (two blocks of
// 32), with the q_nope rows read straight from memory as the B operand.  The
// slab copy and the first 64 sequences' query loads are issued before
// anything waits.  Each block of 64 sequences leaves through LDS as whole
// 512 B row pieces.  The two column halves of a head run on one XCD
// (workgroup i on XCD i % 8), so the head's q_nope rows come from HBM once.
constexpr int ADN = 128, ANC = 256;        // contraction (d_nope), columns per workgroup
constexpr int ASB = 64;                    // sequences per block
__global__ __launch_bounds__(256, 1) void absorb_q_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sW[ADN * ANC];
  // output block [64 sequences][256 columns]: 16 B chunk c of row r at c ^ (r & 31)
  __shared__ __attribute__((aligned(16))) bf16 sOut[ASB * ANC];
  constexpr int NCB = RK / ANC;            // column blocks per head
  constexpr int CPR = ANC / 8;             // 16 B chunks per slab row
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int c0 = (slot % NCB) * ANC, h = xcd + 8 * (slot / NCB);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.heads, B = a.batch;
  {
    const bf16* src = a.w_uk + (int64_t)h * a.w_uv_hstride + c0;   // row k at + k * RK
    const uint32_t sb = lds_addr_of(&sW[0]);
#pragma unroll
    for (int i = 0; i < ADN * CPR / 256; ++i) {
      const int P = i * 256 + tid, k = P / CPR, pc = P % CPR;
      lds_dma16_m0(src + (int64_t)k * RK + ((pc ^ ((k & 3) << 1)) << 3), sb + (uint32_t)(i * 256 + wave * 64) * 16);
    }
  }
  // B operand of sequence block j: lane holds sequence m0 + 32 j + lane % 32,
  // d_nope (lane / 32) * 8 + 16 ks + [0, 8)
  const int col = lane & 31, hsel = lane >> 5;
  auto load_q = [&](bf16x8 (&qb)[2][ADN / 16], int m0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int b = m0 + 32 * j + col;
      const bf16* q = a.q_nope + ((int64_t)b * H + h) * ADN + hsel * 8;
#pragma unroll
      for (int ks = 0; ks < ADN / 16; ++ks) {
        if (b < B) qb[j][ks] = *(const bf16x8*)(q + ks * 16);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) qb[j][ks][e] = (bf16)0.f;
      }
    }
  };
  bf16x8 qb[2][ADN / 16];
  load_q(qb, 0);
  vm_wait_all();                           // the slab copies (inline asm) and the queries
  __syncthreads();
  // A operand of column block i by transpose reads: lane group g = lane / 16
  // reads rows 16 ks + (g / 2) * 8 + [0, 8) of columns 64 w + 32 i + (g % 2) * 16 + [0, 16)
  const int g = lane >> 4, L = lane & 15;
  bf16x8 wa[2][ADN / 16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = wave * 64 + i * 32 + (g & 1) * 16 + 4 * (L & 3);
#pragma unroll
    for (int ks = 0; ks < ADN / 16; ++ks) {
      bf16x4 v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = ks * 16 + (g >> 1) * 8 + u * 4 + (L >> 2);
        v[u] = lds_read_tr(&sW[k * ANC + ((((n >> 3) ^ ((k & 3) << 1))) << 3) + (n & 7)]);
      }
      wa[i][ks] = cat8(v[0], v[1]);
    }
  }
  for (int mb = 0; mb < B; mb += ASB) {
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < ADN / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(wa[i][ks], qb[j][ks], acc[i][j]);
    if (mb + ASB < B) load_q(qb, mb + ASB);
    // lane holds sequence mb + 32 j + lane % 32, columns 64 w + 32 i + (e / 4) * 8 + hsel * 4 + e % 4
    if (mb > 0) __syncthreads();           // the previous block has left sOut
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * j + col;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][q * 4 + e];
          const int chunk = wave * 8 + i * 4 + q;
          *(bf16x4*)&sOut[r * ANC + ((chunk ^ (r & 31)) << 3) + hsel * 4] = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < ASB * CPR / 256; ++u) {
      const int id = u * 256 + tid, rr = id / CPR, c = id % CPR, b = mb + rr;
      if (b < B)
        *(bf16x8*)((bf16*)a.qt + ((int64_t)b * H + h) * RK + c0 + c * 8) =
            *(const bf16x8*)&sOut[rr * ANC + ((c ^ (rr & 31)) << 3)];
    }
  }
}

// Combine and un-absorb, fused.  Workgroup (h, block of 32 sequences), 8
// waves:
//  1. o_lat[b, h, :] = sum_s w_s l_s (O_s / l_s) / sum_s w_s l_s over the
//     sequence's slots s, with w_s = 2^((m_s - M) * c2); slots emptied by a
//     cut (l_s = 0) are skipped.  Stored into LDS as two bf16 parts, hi =
//     bf16(o_lat) and lo = bf16(o_lat - hi), which carry o_lat to about 16
//     significant bits; each wave takes 4 sequences, with all their slots
//     (up to CMAXS each) loaded before any is used, 8 latent dims per lane.
//  2. out[b, h, :] = W_UV[h] . o_lat[b, h, :] for the 32 sequences at once:
//     O^T[dv, b] = W_UV[h][dv, :] . (hi + lo)[b, :]^T on 16x16x32 MFMAs (two
//     per step, one per part), each wave 16 output dims for both blocks of 16
//     sequences.  Its W_UV rows are requested while step 1 runs.
// W_UV[h] (128 KB) is read once per 32 sequences; the workgroups of one head
// run on one XCD (x = h), so it comes from HBM about once.
constexpr int CB = 32;                     // sequences per combine workgroup
constexpr int CMAXS = 8;                   // slots per sequence loaded at once
constexpr int CNW = 8;                     // waves per combine workgroup
__global__ __launch_bounds__(CNW * 64, 1) void decode_combine_unabsorb_kernel(DecodeArgs a) {
  // latent rows of the block: 16 B chunk c of row j at c ^ (j & 15), so the
  // 16 rows one MFMA operand read touches spread over the banks
  __shared__ __attribute__((aligned(16))) bf16 sO[2][CB * RK];
  __shared__ int s_ns[CB];
  __shared__ int s_base[CB];
  __shared__ long long s_red[CNW];
  const int h = blockIdx.x, b0 = blockIdx.y * CB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads, B = a.batch;
  const int cap = a.max_blocks << a.log2_block;
  const int64_t R = a.quota;
  // work-order position of sequence b0, then the slot counts of b0 .. b0 + 31
  long long part_sum = 0;
  for (int i = tid; i < b0; i += CNW * 64) {
    const int Li = max(0, min(a.seq_lens[i], cap));
    part_sum += Li > 0 ? (long long)Li + kDecodeSegmentCost : 0;
  }
  part_sum = wave_sum_ll(part_sum);
  if (lane == 0) s_red[wave] = part_sum;
  __syncthreads();
  if (wave == 0) {
    long long base = 0;
#pragma unroll
    for (int w = 0; w < CNW; ++w) base += s_red[w];
    const int b = b0 + lane;
    const int Lb = (lane < CB && b < B) ? max(0, min(a.seq_lens[b], cap)) : 0;
    const long long n = Lb > 0 ? (long long)Lb + kDecodeSegmentCost : 0;
    long long incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const long long r0 = base + incl - n + kDecodeSegmentCost;   // work-order position of key 0
    // slot count and first partial entry (r0 / R + b, see the split kernel),
    // the count bounded so that every entry read lies in the buffers
    if (lane < CB) {
      const long long base = r0 / R + b;
      const long long ns = Lb > 0 ? (r0 + Lb - 1) / R - r0 / R + 1 : 0;
      s_base[lane] = (int)min<long long>(base, (long long)a.num_items + B);
      s_ns[lane] = (int)max<long long>(0, min<long long>(ns, (long long)a.num_items + B - base));
    }
  }
  __syncthreads();

  const float c2 = a.scale * kLog2e;
  // A operand of the un-absorb: lane holds row 16 w + lane % 16 of W_UV[h],
  // k = 32 ks + (lane / 16) * 8 + [0, 8)
  const int r16 = lane & 15, kq = lane >> 4;
  bf16x8 wf[RK / 32];
  // all partials of the wave's 4 sequences, then its W_UV rows, are requested
  // before any of them is used: one memory round trip.  The (origin, sum)
  // pairs are loaded one per lane (lane 8 u + s: slot s of the wave's u-th
  // sequence) and read back as wave-uniform values.
  constexpr int SPW = CB / CNW;            // sequences per wave
  static_assert(SPW * CMAXS <= 64, "one (origin, sum) pair per lane");
  f16x8 pv[SPW][CMAXS];
  int nslot[SPW];
  int64_t part0[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int j = wave * SPW + u;
    nslot[u] = s_ns[j];                                  // 0 past the batch
    part0[u] = (int64_t)s_base[j] * H + h;               // slot s at part0 + s * H
#pragma unroll
    for (int sl = 0; sl < CMAXS; ++sl)
      if (sl < nslot[u]) pv[u][sl] = *(const f16x8*)(a.part_o + (part0[u] + (int64_t)sl * H) * RK + lane * 8);
  }
  float2 ml_lane = make_float2(-INFINITY, 0.f);
  {
    const int u = lane / CMAXS, sl = lane % CMAXS;
    if (u < SPW && sl < s_ns[wave * SPW + u])
      ml_lane = *(const float2*)(a.part_ml + ((int64_t)s_base[wave * SPW + u] * H + h + (int64_t)sl * H) * 2);
  }
  {
    const bf16* wr = a.w_uv + (int64_t)h * a.w_uv_hstride + (int64_t)(16 * wave + r16) * RK + kq * 8;
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) wf[ks] = *(const bf16x8*)(wr + ks * 32);
  }
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int j = wave * SPW + u;
    float mv[CMAXS], lv[CMAXS];
#pragma unroll
    for (int sl = 0; sl < CMAXS; ++sl) {
      mv[sl] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml_lane.x), u * CMAXS + sl));
      lv[sl] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml_lane.y), u * CMAXS + sl));
    }
    float M = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < CMAXS; ++sl)
      if (lv[sl] != 0.f) M = fmaxf(M, mv[sl]);
    for (int sl = CMAXS; sl < nslot[u]; ++sl) {
      const int64_t part = part0[u] + (int64_t)sl * H;
      if (a.part_ml[part * 2 + 1] != 0.f) M = fmaxf(M, a.part_ml[part * 2]);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int sl = 0; sl < CMAXS; ++sl) {
      if (lv[sl] != 0.f) {
        const float w = __builtin_amdgcn_exp2f((mv[sl] - M) * c2) * lv[sl];
        lsum += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * (float)pv[u][sl][e];
      }
    }
    for (int sl = CMAXS; sl < nslot[u]; ++sl) {
      const int64_t part = part0[u] + (int64_t)sl * H;
      const float l = a.part_ml[part * 2 + 1];
      if (l == 0.f) continue;
      const float w = __builtin_amdgcn_exp2f((a.part_ml[part * 2] - M) * c2) * l;
      lsum += w;
      const f16x8 v = *(const f16x8*)(a.part_o + part * RK + lane * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * (float)v[e];
    }
    // sequences past the batch and empty ones leave a zero row
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    bf16x8 rh, rl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = acc[e] * inv;
      rh[e] = (bf16)v;
      rl[e] = (bf16)(v - (float)rh[e]);
    }
    *(bf16x8*)&sO[0][j * RK + ((lane ^ (j & 15)) << 3)] = rh;
    *(bf16x8*)&sO[1][j * RK + ((lane ^ (j & 15)) << 3)] = rl;
  }
  __syncthreads();

  // O^T[dv, b]: wave w takes output dims 16 w .. 16 w + 15 (dv = 128) for
  // sequence blocks n = 0, 1; the B operand lane holds sequence b0 + 16 n +
  // lane % 16, k = 32 ks + (lane / 16) * 8
  f32x4 o[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[n][e] = 0.f;
#pragma unroll
  for (int ks = 0; ks < RK / 32; ++ks)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int j = n * 16 + r16;
      const int off = j * RK + (((ks * 4 + kq) ^ (j & 15)) << 3);
      o[n] = mfma16(wf[ks], *(const bf16x8*)&sO[0][off], o[n]);
      o[n] = mfma16(wf[ks], *(const bf16x8*)&sO[1][off], o[n]);
    }
  // lane holds sequence b0 + 16 n + lane % 16, dims 16 w + (lane / 16) * 4 + [0, 4)
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int b = b0 + n * 16 + r16;
    if (b < B) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)o[n][e];
      *(bf16x4*)(a.out + ((int64_t)b * H + h) * a.dv + 16 * wave + kq * 4) = v;
    }
  }
}

}  // namespace

hipError_t launch_decode_absorb_q(const DecodeArgs& a, hipStream_t s) {
  // one workgroup per (column block, head); XCD x takes heads x, x + 8, ...
  if (a.heads % 8) return hipErrorInvalidValue;
  absorb_q_kernel<<<(RK / ANC) * a.heads, 256, 0, s>>>(a);
  return hipGetLastError();
}

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

hipError_t launch_decode_combine_unabsorb(const DecodeArgs& a, hipStream_t s) {
  if (a.dv != 128) return hipErrorInvalidValue;
  dim3 grid(a.heads, (a.batch + CB - 1) / CB);
  decode_combine_unabsorb_kernel<<<grid, CNW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
