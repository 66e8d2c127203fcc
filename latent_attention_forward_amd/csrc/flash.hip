// Causal varlen attention of the MLA prefill (d_qk = 192 = 128 + 64, d_v = 128).
//
// One 256-thread workgroup computes 128 query rows of one head of one packed
// document; each of its 4 waves owns 32 query rows.  Keys are walked in tiles
// of 64 from the document start to the last query of the tile (causal).  The
// key tile [k_nope_h (from kv) | k_pe (the one shared rope head)] and the value
// tile v_h are copied into LDS by asynchronous global->LDS loads, double
// buffered, so tile t+1 streams in while tile t is multiplied.  Each lane's
// source offsets inside a tile are computed once; a tile only moves two
// uniform base pointers.
//
// Contractions are 32x32x16 MFMAs in the transposed orientation:
//   S^T[key, query]  = K[key, :] . Q[query, :]      (A = K from LDS, B = Q^T from registers)
//   O^T[dv, query]  += V^T[dv, key] . P^T[key, query] (A = V^T by LDS transpose read, B = P^T)
// so every lane holds one query row: the softmax max / sum need only an
// in-lane reduction plus one swap with the lane 32 away, and P^T feeds the
// second MFMA straight from the first MFMA's registers (the key order of the
// S^T output layout is matched by the transpose reads of V).  LDS operand
// reads are issued several MFMAs ahead of their use.
//
// Softmax: fp32, exp2 with the scale folded in.  The exponent origin m is
// kept as long as every lane's sum of P = 2^(s - m) over a tile stays at or
// below 2^15 (so no P exceeds it): most tiles need neither the tile's max nor
// a rescale of the accumulators.  Otherwise (and on a wave's first tile) the
// max is taken and m moves when a score exceeds it by more than 8 in base-2
// units.  P is rounded to the operand type (bf16, or fp16 inside the prefill
// layer) for the PV MFMA; O / l is formed in fp32 and rounded once to bf16.
// d_v = 128 is used as is: v is never padded to d_qk.
//
// Work order: the workgroups of one head are kept on one XCD (workgroup i runs
// on XCD i mod 8), so the tiles that stream the same k/v rows share that XCD's
// L2; each XCD takes its tiles longest first across all its heads, so that
// the last workgroups to start are short ones.  Documents go one after
// another (longest first).  When the queries follow a cached prefix (keys
// offset per document, see FlashArgs), every tile of a document streams the
// whole prefix, and the tiles of one head are issued in groups that run
// together instead.
#include "mla_internal.hpp"

#include <vector>
#include <algorithm>

namespace mla {
namespace {

constexpr int FQ = 128, FK = 64;
constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int MAX_TILES = 880;
constexpr float kRescaleSlack = 8.f;  // base-2 headroom before the exponent origin moves
constexpr float kPSumMax = 32768.f;   // a lane's sum of P (32 keys) accepted against the current origin

struct TilePlan {
  int n;                              // query tiles per head in this launch
  int heads_per_xcd;                  // ceil(H / 8)
  int group;                          // tiles of one head issued back to back (see the work order)
  uint32_t t[MAX_TILES];              // (document << 16) | query-tile index in the document
};
// Tiles per group when the queries follow a cached prefix: all of a group's
// tiles stream the prefix keys, so they run together on one XCD.
constexpr int kPrefixTileGroup = 8;

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<f16> { typedef f16x8 v8; typedef f16x4 v4; };
template <int B> struct BufC { static constexpr int value = B; };

template <typename V8> __device__ __forceinline__ V8 zero8() { return __builtin_bit_cast(V8, make_uint4(0, 0, 0, 0)); }
template <typename V4, typename T> __device__ __forceinline__ V4 read_tr(const T* p) {
  return __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(p)));
}
// LDS tiles, 16-byte chunks XOR-swizzled by key row so that the rows one
// operand read touches spread over the banks:
//   k_nope [64][128]: chunk c (0..15) of row r at c ^ (r & 15)
//   k_pe   [64][64]:  chunk c (0..7)  of row r at c ^ ((r >> 1) & 7)
//   v      [64][128]: chunk c (0..15) of row r at c ^ ((r & 3) << 2), so the
//                     four rows a transpose read takes land in four different
//                     64-byte bank groups
__device__ __forceinline__ int ksw_n(int r) { return r & 15; }
__device__ __forceinline__ int ksw_r(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int kn_off(int r, int c) { return r * DN + ((c ^ ksw_n(r)) << 3); }
__device__ __forceinline__ int kr_off(int r, int c) { return r * DR + ((c ^ ksw_r(r)) << 3); }
__device__ __forceinline__ int vsw(int r, int c) { return c ^ ((r & 3) << 2); }
__device__ __forceinline__ int voff(int r, int n) { return r * DV + (vsw(r, n >> 3) << 3) + (n & 7); }

template <typename T>
__global__ __launch_bounds__(256, 2) void flash_mfma_kernel(FlashArgs a, TilePlan plan) {
  typedef typename Vec<T>::v8 V8;
  typedef typename Vec<T>::v4 V4;
  __shared__ __attribute__((aligned(16))) T sKn[2][FK * DN];
  __shared__ __attribute__((aligned(16))) T sKr[2][FK * DR];
  __shared__ __attribute__((aligned(16))) T sV[2][FK * DV];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.heads;
  // workgroup -> (head, tile): XCD x = blockIdx % 8 takes heads x, x+8, ...;
  // within an XCD the plan's tiles go out in groups of plan.group, each group
  // head by head and the group's tiles of one head back to back (a group of 1:
  // tile index major across all the XCD's heads)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hpx = plan.heads_per_xcd, tg = plan.group;
  const int gbase = slot / (tg * hpx) * tg, gs = min(tg, plan.n - gbase);
  const int rem = slot - gbase * hpx;
  const int hj = rem / gs, ti = gbase + rem - hj * gs;
  const int head = xcd + 8 * hj;
  if (head >= H) return;
  const uint32_t td = plan.t[ti];
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = max(0, min(a.cu_dev[doc], a.n_tokens));
  const int de = max(ds, min(a.cu_dev[doc + 1], a.n_tokens));
  // keys of the document: rows [kst, ...); query row t sees keys up to t + koff
  int kst = ds, koff = 0;
  if (a.cuk_dev) {
    const int k_s = max(0, min(a.cuk_dev[doc], a.n_keys));
    const int k_e = max(k_s, min(a.cuk_dev[doc + 1], a.n_keys));
    if (k_e - k_s < de - ds) return;       // fewer keys than queries: rejected by the host
    kst = k_s;
    koff = k_e - de;
  }
  const int q0 = ds + tix * FQ;
  if (q0 >= de) return;
  const int q1 = min(q0 + FQ, de);
  const int kend = q1 + koff;              // keys [kst, kend) are seen by some query of the tile
  const int ntiles = (kend - kst + FK - 1) / FK;

  const T* Q = (const T*)a.q;
  const T* KV = (const T*)a.kv;
  const T* KPE = (const T*)a.kpe;
  bf16* O = (bf16*)a.out;
  const int64_t q_row = (int64_t)H * DQK, kv_row = (int64_t)H * (DN + DV);

  // ---- this wave's queries, held as the B operand (Q^T) for 12 k-steps of 16
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + (lane & 31);
  const int hsel = lane >> 5;
  V8 qreg[DQK / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    qreg[ks] = (my_q < q1) ? *(const V8*)(Q + my_q * q_row + head * DQK + ks * 16 + hsel * 8) : zero8<V8>();

  // ---- global->LDS copies.  Lane l of a wave fills the l-th 16 bytes of a
  // 1 KB block; each LDS position is mapped back to the (key row, logical
  // chunk) that the swizzled layout keeps there.  Per-lane byte offsets
  // relative to the tile's first key are fixed for the whole walk (the host
  // bounds them to 32 bits).
  uint32_t o_kn[4], o_kr[2], o_v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = (wave + 4 * i) * 64 + lane;
    const int r = P >> 4;
    o_kn[i] = (uint32_t)((r * kv_row + (((P & 15) ^ ksw_n(r)) << 3)) * sizeof(T));
    o_v[i] = (uint32_t)((r * kv_row + DN + (vsw(r, P & 15) << 3)) * sizeof(T));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = (wave + 4 * i) * 64 + lane;
    const int r = P >> 3;
    o_kr[i] = (uint32_t)((r * a.kpe_stride + (((P & 7) ^ ksw_r(r)) << 3)) * sizeof(T));
  }
  const T* kv_head = KV + head * (DN + DV);
  // copy k (0..9) of a full tile: k_nope blocks 0-3, k_pe blocks 4-5, v blocks 6-9
  auto issue_part = [&](const T* kvb, const T* kpb, int k, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if (k < 4) lds_dma16_sv(kvb, o_kn[k], &sKn[buf][(wave + 4 * k) * 512]);
    else if (k < 6) lds_dma16_sv(kpb, o_kr[k - 4], &sKr[buf][(wave + 4 * (k - 4)) * 512]);
    else lds_dma16_sv(kvb, o_v[k - 6], &sV[buf][(wave + 4 * (k - 6)) * 512]);
  };
  auto issue_tile = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = kst + t * FK;
    if (kb + FK <= kend) {
      const T* kvb = kv_head + (int64_t)kb * kv_row;
      const T* kpb = KPE + (int64_t)kb * a.kpe_stride;
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16_sv(kvb, o_kn[i], &sKn[buf][(wave + 4 * i) * 512]);
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_sv(kpb, o_kr[i], &sKr[buf][(wave + 4 * i) * 512]);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16_sv(kvb, o_v[i], &sV[buf][(wave + 4 * i) * 512]);
    } else {
      // last, partial tile: keys at or past kend read the tile's first key
      // instead (they are masked out of the softmax, probability exactly 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int P = (wave + 4 * i) * 64 + lane;
        const int r = P >> 4;
        const int key = (kb + r < kend) ? kb + r : kb;
        lds_dma16_raw(kv_head + (int64_t)key * kv_row + (((P & 15) ^ ksw_n(r)) << 3), &sKn[buf][(wave + 4 * i) * 512]);
        lds_dma16_raw(kv_head + (int64_t)key * kv_row + DN + (vsw(r, P & 15) << 3), &sV[buf][(wave + 4 * i) * 512]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int P = (wave + 4 * i) * 64 + lane;
        const int r = P >> 3;
        const int key = (kb + r < kend) ? kb + r : kb;
        lds_dma16_raw(KPE + (int64_t)key * a.kpe_stride + (((P & 7) ^ ksw_r(r)) << 3), &sKr[buf][(wave + 4 * i) * 512]);
      }
    }
  };

  const float c2 = a.scale * kLog2e;     // scores to base-2 exponent units
  float m_ref = -INFINITY, l_run = 0.f;  // exponent origin (base-2 units), running sum
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;

  // LDS operand addresses: a lane-constant part per operand column, computed
  // once (the swizzles depend only on the lane's row within 16 or 4 rows), plus
  // compile-time row offsets, so an operand read costs no address arithmetic.
  // S operand i (0..23): key block mt = i & 1 (rows + 32, same swizzle), k-step ks = i >> 1
  const int krow = lane & 31;
  int kbase[DN / 16], rbase[DR / 16];
#pragma unroll
  for (int ks = 0; ks < DN / 16; ++ks) kbase[ks] = kn_off(krow, (ks << 1) | hsel);
#pragma unroll
  for (int ks = 0; ks < DR / 16; ++ks) rbase[ks] = kr_off(krow, (ks << 1) | hsel);
  auto kread = [&](int i, auto bufc) -> V8 {
    constexpr int buf = decltype(bufc)::value;
    const int mt = i & 1, ks = i >> 1;
    if (ks < DN / 16) return *(const V8*)&sKn[buf][kbase[ks] + mt * 32 * DN];
    return *(const V8*)&sKr[buf][rbase[ks - DN / 16] + mt * 32 * DR];
  };
  // PV operand i (0..15): key group j = i >> 2 (16 keys: rows (j/2)*32 + (j%2)*16
  // + 4 (g/2) + L/4, and + 8), dv block d = i & 3; the V swizzle depends on the
  // row only through row & 3, the same for every j and both halves
  const int grp = lane >> 4, L16 = lane & 15;
  int vbase[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
    vbase[d] = voff((grp >> 1) * 4 + (L16 >> 2), d * 32 + (grp & 1) * 16 + 4 * (L16 & 3));
  auto vread = [&](int i, auto bufc) -> V8 {
    constexpr int buf = decltype(bufc)::value;
    const int j = i >> 2, d = i & 3;
    const int r0 = ((j >> 1) * 32 + (j & 1) * 16) * DV;
    const V4 lo = read_tr<V4>(&sV[buf][vbase[d] + r0]);
    const V4 hi = read_tr<V4>(&sV[buf][vbase[d] + r0 + 8 * DV]);
    return cat8(lo, hi);
  };
  constexpr int SD = 4;   // S operand reads in flight
  constexpr int PD = 3;   // PV operands in flight

  // The copies of tile t + 1 go out between the score MFMAs of tile t (one
  // per other MFMA) rather than all at once after the barrier, where the
  // copies of all eight waves of the CU queue at the address unit together.
  auto step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = kst + t * FK;
    const int kn = kb + FK;
    const bool active = (qw0 < q1) && (kb <= qw0 + 31 + koff);
    const bool spread = active && t + 1 < ntiles && kn + FK <= kend;
    if (t + 1 < ntiles && !spread) issue_tile(t + 1, BufC<buf ^ 1>{});
    const T* kvn = kv_head + (int64_t)kn * kv_row;
    const T* kpn = KPE + (int64_t)kn * a.kpe_stride;
    if (active) {
      // MFMA phases run at a raised wave priority, so that when the other wave
      // on this SIMD is in its softmax the MFMAs issue first
      __builtin_amdgcn_s_setprio(2);
      // ---- S^T for 64 keys (2 blocks of 32) x 32 queries, operands read SD ahead
      f32x16 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
      V8 kf[SD];
#pragma unroll
      for (int i = 0; i < SD; ++i) kf[i] = kread(i, bufc);
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const V8 cur = kf[i % SD];
        if (i + SD < 24) kf[i % SD] = kread(i + SD, bufc);
        s[i & 1] = mfma32(cur, qreg[i >> 1], s[i & 1]);
        if ((i & 1) && i < 20 && spread) issue_part(uniform_ptr(kvn), uniform_ptr(kpn), i >> 1, BufC<buf ^ 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
      // first PV operands, independent of the softmax
      V8 vf[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) vf[i] = vread(i, bufc);
      // ---- causal mask (only tiles that reach past this wave's first query)
      if (kb + FK - 1 > qw0 + koff) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
            if (key > my_q + koff) s[mt][e] = -INFINITY;
          }
      }
      __builtin_amdgcn_s_setprio(0);
      // ---- online softmax (one query per lane, keys split across lane and lane^32).
      // Once every lane has an exponent origin, P is formed against it
      // directly and accepted if no lane's sum of P exceeds 2^15 (then every P
      // is at most 2^15, exact in range for the operand type); otherwise, and
      // on a wave's first tile, the tile's max is taken and the origin moved
      // (by the slack rule, which then always applies) before P is formed.
      V8 pb[4];
      auto probs = [&](float mb) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            pb[mt * 2 + (e >> 3)][e & 7] = (T)__builtin_amdgcn_exp2f(fmaf(s[mt][e], c2, -mb));
        float ps0 = sum8(pb[0], 0.f), ps1 = sum8(pb[1], 0.f);
        ps0 = sum8(pb[2], ps0);
        ps1 = sum8(pb[3], ps1);
        return ps0 + ps1;
      };
      float ps = 0.f;
      bool redo = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
      if (!redo) {
        ps = probs(m_ref);
        redo = __builtin_amdgcn_ballot_w64(!(ps <= kPSumMax)) != 0;
      }
      if (redo) {
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack) != 0) {
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
          m_ref = m_new;
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < DV / 32; ++d)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
        }
        ps = probs((m_ref == -INFINITY) ? 0.f : m_ref);
      }
      l_run += ps;
      __builtin_amdgcn_s_setprio(2);
      // ---- O^T += V^T P^T ; step j covers keys (j/2)*32 + (j%2)*16 + {h*4+0..3, 8+h*4+0..3}
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const V8 vv = vf[i % PD];
        if (i + PD < 16) vf[i % PD] = vread(i + PD, bufc);
        o[i & 3] = mfma32(vv, pb[i >> 2], o[i & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < ntiles) vm_wait_all();
    wg_barrier();
  };

  issue_tile(0, BufC<0>{});
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(t, BufC<0>{});
    if (t + 1 < ntiles) step(t + 1, BufC<1>{});
  }

  // ---- normalise and store: lane holds query my_q, dv rows d*32 + qd*8 + h*4 + [0,4)
  if (my_q >= q1) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  if (a.lse_out && hsel == 0) a.lse_out[(int64_t)head * a.n_tokens + my_q] = m_ref + __builtin_log2f(l_tot);
  bf16* orow = O + (int64_t)my_q * H * DV + head * DV;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[d][qd * 4 + e] * inv);
      *(bf16x4*)(orow + d * 32 + qd * 8 + hsel * 4) = v;
    }
}

// fp32 attention for the fp32 dtype (small shapes): one wavefront per (query,
// head), keys walked one at a time with an online softmax.
__global__ __launch_bounds__(64) void flash_f32_kernel(FlashArgs a) {
  __shared__ float sq[512];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int dqk = a.nope + a.rope, dv = a.dv, H = a.heads;
  const int* cu = a.cu_dev;
  if (t >= a.n_tokens) return;
  // document of t
  int d = 0;
  while (d + 1 < a.num_seqs && cu[d + 1] <= t) ++d;
  // keys lo .. hi: the document's own tokens up to t, or with separate key
  // rows, everything up to t's place counted from the end of both
  int lo = max(0, cu[d]), hi = t;
  if (a.cuk_dev) {
    lo = max(0, a.cuk_dev[d]);
    hi = min(t + a.cuk_dev[d + 1] - cu[d + 1], a.n_keys - 1);
  }
  const float* Q = (const float*)a.q + ((int64_t)t * H + h) * dqk;
  for (int d = lane; d < dqk; d += 64) sq[d] = Q[d];
  __syncthreads();
  const float* KV = (const float*)a.kv;
  const float* KPE = (const float*)a.kpe;
  const int kvw = a.nope + a.dv;
  float m = -INFINITY, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = lo; j <= hi; ++j) {
    const float* kr = KV + ((int64_t)j * H + h) * kvw;
    const float* pr = KPE + (int64_t)j * a.kpe_stride;
    float part = 0.f;
    for (int d = lane; d < dqk; d += 64) part = fmaf(sq[d], d < a.nope ? kr[d] : pr[d - a.nope], part);
    const float s = wave_sum(part) * a.scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = lane + 64 * i;
      acc[i] = acc[i] * al + (d < dv ? p * kr[a.nope + d] : 0.f);
    }
    m = mn;
  }
  float* orow = (float*)a.out + ((int64_t)t * H + h) * dv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d < dv) orow[d] = acc[i] / l;
  }
}

}  // namespace

hipError_t launch_flash_mfma(const FlashArgs& a, bool f16_operands, const int32_t* cu_host, const int32_t* cuk_host,
                             int num_seqs, hipStream_t s) {
  // Tile plan: every (document, 128-query tile), longest key range first; each
  // head walks the whole list on its XCD.
  struct T { int keys; uint32_t id; };
  std::vector<T> tiles;
  int64_t prefix_total = 0;
  for (int d = 0; d < num_seqs; ++d) {
    const int len = cu_host[d + 1] - cu_host[d];
    const int prefix = cuk_host ? (cuk_host[d + 1] - cuk_host[d]) - len : 0;
    prefix_total += prefix;
    const int nt = (len + FQ - 1) / FQ;
    for (int i = 0; i < nt; ++i)
      tiles.push_back({prefix + std::min((i + 1) * FQ, len), ((uint32_t)d << 16) | (uint32_t)i});
  }
  // Documents in decreasing order of their longest tile, each document's
  // tiles longest first.  Tile-major across the XCD's heads (a group of 1):
  // the few tiles of one head in flight together share their keys in the L2,
  // and the longest tiles start first.  Queries after a cached prefix all
  // stream the same long key prefix: groups of kPrefixTileGroup consecutive
  // tiles go out head by head, so those tiles run together.
  std::vector<int> doc_max(num_seqs, 0);
  for (const T& t : tiles) doc_max[t.id >> 16] = std::max(doc_max[t.id >> 16], t.keys);
  std::stable_sort(tiles.begin(), tiles.end(), [&](const T& x, const T& y) {
    const int dx = (int)(x.id >> 16), dy = (int)(y.id >> 16);
    if (doc_max[dx] != doc_max[dy]) return doc_max[dx] > doc_max[dy];
    if (dx != dy) return dx < dy;
    return x.keys > y.keys;
  });
  TilePlan plan;
  plan.heads_per_xcd = (a.heads + 7) / 8;
  plan.group = prefix_total > 0 ? kPrefixTileGroup : 1;
  // When every workgroup of an XCD is resident at once (at most two per CU,
  // 32 CUs per XCD), a CU keeps the two it is first given for the whole
  // launch, slot s beside slot s + 32: then the tiles go longest first across
  // documents with the second half reversed, so the k-th longest shares a CU
  // with the k-th shortest (two documents of 2048 tokens, 16 heads: the
  // busiest CU had 64 key tiles against an average of 34).
  if (prefix_total == 0 && tiles.size() >= 2 && (int64_t)plan.heads_per_xcd * (int64_t)tiles.size() <= 64) {
    std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.keys > y.keys; });
    std::reverse(tiles.begin() + tiles.size() / 2, tiles.end());
  }
  for (size_t base = 0; base < tiles.size(); base += MAX_TILES) {
    const int n = (int)std::min<size_t>(MAX_TILES, tiles.size() - base);
    plan.n = n;
    for (int i = 0; i < n; ++i) plan.t[i] = tiles[base + i].id;
    const int64_t blocks = (int64_t)8 * plan.heads_per_xcd * n;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    if (f16_operands)
      flash_mfma_kernel<f16><<<grid, 256, 0, s>>>(a, plan);
    else
      flash_mfma_kernel<bf16><<<grid, 256, 0, s>>>(a, plan);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_flash_f32(const FlashArgs& a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  dim3 grid(a.n_tokens, a.heads);
  flash_f32_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
