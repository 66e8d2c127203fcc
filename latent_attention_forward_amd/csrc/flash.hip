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
// together instead.  A launch small enough that all its workgroups would be
// resident at once, two to a CU, runs paired instead (8-wave workgroups, one
// per CU, a long and a short tile shared out evenly between two halves; see
// the kernel).
#include "mla_internal.hpp"

#include <vector>
#include <algorithm>
#include <type_traits>

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

// Geometry of one 128-query tile of a document (keys as described in FlashArgs).
struct TileGeom {
  int q0, q1;     // query rows [q0, q1); empty when q0 >= q1
  int kst, kend;  // keys [kst, kend) are seen by some query of the tile
  int koff;       // query row t sees keys up to t + koff
  int ntiles;     // key tiles of FK from kst
};
__device__ __forceinline__ TileGeom tile_geom(const FlashArgs& a, uint32_t td) {
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = max(0, min(a.cu_dev[doc], a.n_tokens));
  const int de = max(ds, min(a.cu_dev[doc + 1], a.n_tokens));
  TileGeom g;
  g.kst = ds;
  g.koff = 0;
  g.q0 = ds + tix * FQ;
  if (a.cuk_dev) {
    const int k_s = max(0, min(a.cuk_dev[doc], a.n_keys));
    const int k_e = max(k_s, min(a.cuk_dev[doc + 1], a.n_keys));
    if (k_e - k_s < de - ds) {
      g.q0 = de;                           // fewer keys than queries: rejected by the host
    } else {
      g.kst = k_s;
      g.koff = k_e - de;
    }
  }
  g.q1 = min(g.q0 + FQ, de);
  g.kend = g.q1 + g.koff;
  g.ntiles = g.q0 < g.q1 ? (g.kend - g.kst + FK - 1) / FK : 0;
  return g;
}
constexpr uint32_t kNoTile = 0xffffffffu;

// PAIRED: an 8-wave workgroup of two halves of 4 waves, for launches whose
// workgroups all run at once (one per CU).  The plan gives each workgroup a
// long tile and a short one of the same head (the k-th longest with the k-th
// shortest); half 0 walks the long tile's first key tiles, half 1 the short
// tile and then the rest of the long one, the split chosen so that both walk
// about the same number of key tiles; at the end half 1 merges half 0's
// partial result for the long tile (log-sum-exp weights) and stores it.
// Both halves pass the same barriers (one per step; the shorter walk idles).
template <typename T, bool PAIRED>
__global__ __launch_bounds__(PAIRED ? 512 : 256, PAIRED ? 1 : 2) void flash_mfma_kernel(FlashArgs a, TilePlan plan) {
  typedef typename Vec<T>::v8 V8;
  typedef typename Vec<T>::v4 V4;
  constexpr int NHALF = PAIRED ? 2 : 1;
  __shared__ __attribute__((aligned(16))) T sKn_[NHALF][2][FK * DN];
  __shared__ __attribute__((aligned(16))) T sKr_[NHALF][2][FK * DR];
  __shared__ __attribute__((aligned(16))) T sV_[NHALF][2][FK * DV];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = PAIRED ? (wid & 3) : wid;     // wave within its half
  const int half = PAIRED ? (wid >> 2) : 0;
  T (*sKn)[FK * DN] = sKn_[half];
  T (*sKr)[FK * DR] = sKr_[half];
  T (*sV)[FK * DV] = sV_[half];
  const int H = a.heads;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hpx = plan.heads_per_xcd;
  // this half's walk: item 0 = key tiles [t00, t00 + n0) of tile g0, then
  // item 1 = key tiles [t10, t10 + n1) of tile g1; nsteps = loop steps of the
  // workgroup (the longer walk of its halves)
  int head;
  TileGeom g0, g1;
  int t00 = 0, n0 = 0, t10 = 0, n1 = 0, nsteps = 0;
  bool merge = false;
  if constexpr (!PAIRED) {
    // workgroup -> (head, tile): XCD x = blockIdx % 8 takes heads x, x+8, ...;
    // within an XCD the plan's tiles go out in groups of plan.group, each
    // group head by head and the group's tiles of one head back to back (a
    // group of 1: tile index major across all the XCD's heads)
    const int tg = plan.group;
    const int gbase = slot / (tg * hpx) * tg, gs = min(tg, plan.n - gbase);
    const int rem = slot - gbase * hpx;
    const int hj = rem / gs, ti = gbase + rem - hj * gs;
    head = xcd + 8 * hj;
    if (head >= H) return;
    g0 = tile_geom(a, plan.t[ti]);
    if (g0.q0 >= g0.q1) return;
    n0 = g0.ntiles;
    nsteps = n0;
    g1 = g0;
  } else {
    // workgroup -> (head, pair): XCD x takes heads x, x+8, ..., each head's
    // plan.n pairs back to back
    const int hj = slot / plan.n, p = slot - hj * plan.n;
    head = xcd + 8 * hj;
    if (head >= H) return;
    const TileGeom gb = tile_geom(a, plan.t[2 * p]);
    const uint32_t tsm = plan.t[2 * p + 1];
    const TileGeom gsm = tile_geom(a, tsm == kNoTile ? plan.t[2 * p] : tsm);
    const int nb = gb.ntiles, ns = tsm == kNoTile ? 0 : gsm.ntiles;
    const int split = min(nb, (nb + ns + 1) >> 1);   // long-tile key tiles walked by half 0
    merge = split < nb;
    nsteps = max(split, ns + nb - split);
    g0 = gb;
    g1 = gb;
    if (half == 0) {
      n0 = split;
    } else if (ns > 0) {
      g0 = gsm;
      n0 = ns;
      t10 = split;
      n1 = nb - split;
    } else {
      t00 = split;
      n0 = nb - split;
    }
  }
  const int nmine = n0 + n1;

  const T* Q = (const T*)a.q;
  const T* KV = (const T*)a.kv;
  const T* KPE = (const T*)a.kpe;
  bf16* O = (bf16*)a.out;
  const int64_t q_row = (int64_t)H * DQK, kv_row = (int64_t)H * (DN + DV);

  // the item being walked: its keys, and this wave's queries
  int c_kst = g0.kst, c_kend = g0.kend, c_koff = g0.koff, c_q1 = g0.q1, c_t0 = t00;
  int qw0 = g0.q0 + wave * 32;
  int my_q = qw0 + (lane & 31);
  const int hsel = lane >> 5;
  // ---- this wave's queries, held as the B operand (Q^T) for 12 k-steps of 16
  V8 qreg[DQK / 16];
  auto load_q = [&](int row, int q_end) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      qreg[ks] = (row < q_end) ? *(const V8*)(Q + row * q_row + head * DQK + ks * 16 + hsel * 8) : zero8<V8>();
  };
  load_q(my_q, c_q1);
  // (paired) item 1's queries, requested during item 0's last step once its
  // score MFMAs no longer read them
  auto load_next_q = [&]() __attribute__((always_inline)) { load_q(g1.q0 + wave * 32 + (lane & 31), g1.q1); };

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
  // the key tile starting at kb of a query tile whose keys end at kend
  auto issue_tile = [&](int kb, int kend, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
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

  // ---- normalise and store the walked item: lane holds query my_q, dv rows
  // d*32 + qd*8 + h*4 + [0,4)
  auto finish = [&]() __attribute__((always_inline)) {
    if (my_q < c_q1) {
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
  };
  // (paired) item 0 done: store it, start item 1 from a fresh state
  auto next_item = [&]() __attribute__((always_inline)) {
    finish();
    c_kst = g1.kst;
    c_kend = g1.kend;
    c_koff = g1.koff;
    c_q1 = g1.q1;
    c_t0 = t10 - n0;
    qw0 = g1.q0 + wave * 32;
    my_q = qw0 + (lane & 31);
    m_ref = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  };

  // Step v of this half's walk.  The copies of the next key tile go out
  // between the score MFMAs of this one (one per other MFMA) rather than all
  // at once after the barrier, where the copies of all eight waves of the CU
  // queue at the address unit together.
  auto step = [&](int v, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    if constexpr (PAIRED) {
      if (v >= nmine) {                      // the shorter walk idles at the barrier
        wg_barrier();
        return;
      }
      if (n1 > 0 && v == n0) next_item();
    }
    const int kb = c_kst + (c_t0 + v) * FK;
    const bool has_next = v + 1 < nmine;
    // the next key tile: this item's next one, or item 1's first
    int kn = kb + FK, kend_n = c_kend;
    if constexpr (PAIRED) {
      if (n1 > 0 && v + 1 == n0) {
        kn = g1.kst + t10 * FK;
        kend_n = g1.kend;
      }
    }
    const bool active = (qw0 < c_q1) && (kb <= qw0 + 31 + c_koff);
    const bool spread = active && has_next && kn + FK <= kend_n;
    if (has_next && !spread) issue_tile(kn, kend_n, BufC<buf ^ 1>{});
    const bool pre_q = PAIRED && n1 > 0 && v + 1 == n0;
    if (pre_q && !active) load_next_q();
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
      if (pre_q) load_next_q();
      // first PV operands, independent of the softmax
      V8 vf[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) vf[i] = vread(i, bufc);
      // ---- causal mask (only tiles that reach past this wave's first query)
      if (kb + FK - 1 > qw0 + c_koff) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
            if (key > my_q + c_koff) s[mt][e] = -INFINITY;
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
    if (has_next) vm_wait_all();
    wg_barrier();
  };

  if (!PAIRED || nmine > 0) issue_tile(c_kst + c_t0 * FK, c_kend, BufC<0>{});
  vm_wait_all();
  __syncthreads();
  for (int v = 0; v < nsteps; v += 2) {
    step(v, BufC<0>{});
    if (v + 1 < nsteps) step(v + 1, BufC<1>{});
  }

  if constexpr (PAIRED) {
    if (merge) {
      // half 0's partial result for the long tile through LDS (the tiles are
      // no longer read): wave w of either half holds the same queries
      float* xo = reinterpret_cast<float*>(&sKn_[0][0][0]);   // 4 waves x 64 accumulators x 64 lanes
      float* xm = reinterpret_cast<float*>(&sKr_[0][0][0]);   // 4 waves x (m, l) x 64 lanes
      if (half == 0) {
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) xo[(wave * 64 + d * 16 + e) * 64 + lane] = o[d][e];
        xm[(wave * 2) * 64 + lane] = m_ref;
        xm[(wave * 2 + 1) * 64 + lane] = l_run;
      }
      __syncthreads();
      if (half == 1) {
        const float ma = xm[(wave * 2) * 64 + lane], la = xm[(wave * 2 + 1) * 64 + lane];
        const float m = fmaxf(ma, m_ref);
        const float wa = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - m);
        const float wb = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m);
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[d][e] = xo[(wave * 64 + d * 16 + e) * 64 + lane] * wa + o[d][e] * wb;
        l_run = la * wa + l_run * wb;
        m_ref = m;
        finish();
      }
      return;
    }
    if (nmine > 0) finish();
  } else {
    finish();
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
  const int64_t nt = (int64_t)tiles.size();
  auto launch = [&](auto paired, int64_t blocks) -> hipError_t {
    constexpr bool P = decltype(paired)::value;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    if (f16_operands)
      flash_mfma_kernel<f16, P><<<grid, P ? 512 : 256, 0, s>>>(a, plan);
    else
      flash_mfma_kernel<bf16, P><<<grid, P ? 512 : 256, 0, s>>>(a, plan);
    return hipGetLastError();
  };
  // A launch whose 4-wave workgroups would all be resident at once, two to a
  // CU (32 CUs per XCD), keeps each CU's two for the whole launch, and the
  // CU with the longest pair sets the time (two documents of 2048 tokens, 16
  // heads: 64 key tiles against an average of 34, the longest tile of a pair
  // running alone at one wave per SIMD once its partner is done).  Such a
  // launch runs paired instead: one 8-wave workgroup per CU, the k-th longest
  // tile of a head with its k-th shortest, the pair's key tiles split evenly
  // between the two halves.
  const int64_t pairs = (nt + 1) / 2;
  if (prefix_total == 0 && nt >= 2 && plan.heads_per_xcd * nt > 32 && plan.heads_per_xcd * pairs <= 32) {
    std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.keys > y.keys; });
    plan.n = (int)pairs;
    for (int64_t k = 0; k < pairs; ++k) {
      plan.t[2 * k] = tiles[k].id;
      plan.t[2 * k + 1] = (nt - 1 - k > k) ? tiles[nt - 1 - k].id : kNoTile;
    }
    return launch(std::true_type{}, (int64_t)8 * plan.heads_per_xcd * pairs);
  }
  // Otherwise, when the 4-wave workgroups are all resident at once, the
  // tiles go longest first across documents with the second half reversed,
  // so that slot s and slot s + 32 of an XCD (one CU) hold the k-th longest
  // and the k-th shortest tile.
  if (prefix_total == 0 && nt >= 2 && plan.heads_per_xcd * nt <= 64) {
    std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.keys > y.keys; });
    std::reverse(tiles.begin() + tiles.size() / 2, tiles.end());
  }
  for (size_t base = 0; base < tiles.size(); base += MAX_TILES) {
    const int n = (int)std::min<size_t>(MAX_TILES, tiles.size() - base);
    plan.n = n;
    for (int i = 0; i < n; ++i) plan.t[i] = tiles[base + i].id;
    const hipError_t e = launch(std::false_type{}, (int64_t)8 * plan.heads_per_xcd * n);
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
