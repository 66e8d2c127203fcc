// Backward of the causal varlen MLA attention core (d_qk = 192 = 128 + 64 with
// the 64-wide key part shared by all heads, d_v = 128), bf16 operands, fp32
// accumulation and fp32 gradients.
//
// With S = scale q k^T (causal within each document), P = softmax(S),
// O = P v and the output gradient dO:
//   dv = P^T dO,  dP = dO v^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dq = scale dS k,  dk = scale dS^T q,  dk_pe = sum over heads of dk's
//   64-wide shared part.
// Three passes, each on 32x32x16 bf16 MFMAs:
//   1. stats: per (head, query) the log-sum-exp of the scaled scores in
//      base-2 units (the forward's softmax statistics, recomputed: one QK^T
//      pass) and D; skipped when the forward left its log-sum-exp (the dq
//      pass then forms D);
//   2. dq, query-major (workgroup = 128 queries of one head, keys in tiles of
//      64): S^T = K Q^T and dP^T = V dO^T from the recomputed P^T, then
//      dQ^T += K^T dS^T, K^T by transposing LDS reads;
//   3. dk and dv, key-major (workgroup = 128 keys of one head, queries in
//      tiles of 64): S = Q K^T, P, dV^T += dO^T P, dP = dO V^T, dS,
//      dK^T += Q^T dS, dO^T and Q^T by transposing LDS reads.
// P and dS are rounded to bf16 as MFMA operands.  Every lane owns one query
// (pass 2) or one key (pass 3) column, so the per-row statistics are per lane.
//
// The streamed tiles go global -> LDS by asynchronous copies
// (global_load_lds), double buffered: tile t + 1 is requested right after the
// barrier that opens tile t, so it lands while tile t is multiplied; one
// barrier per tile.  Rows past the document end are copied from its last row
// (finite values; their scores are masked).  In LDS a 128-wide part is stored
// as rows of 16 chunks of 16 bytes, chunk c of row r at c ^ swn(r), the
// 64-wide part as rows of 8 chunks at c ^ swr(r): with a 64-bank model both
// are free of bank conflicts for the row reads of an MFMA operand (16 rows,
// one chunk, per 16-lane phase) and for the transposing reads (4 rows x 32
// bytes per 16 lanes, 4 rows x 64 bytes per 32 lanes).
//
// Work order: workgroup b runs on XCD b mod 8; the heads are dealt to the
// XCDs (head h on XCD h mod 8), and an XCD takes its heads one after another,
// the tiles of a head longest first, so the workgroups that run together on
// an XCD stream the same head's rows from its L2.  With fewer than 8 heads
// the workgroups take (head, tile) pairs head fastest instead.
#include "mla_internal.hpp"

#include <vector>
#include <algorithm>

namespace mla {
namespace {

constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int BT = 128;              // rows (queries or keys) per workgroup
constexpr int ST = 64;               // rows of the streamed tile
constexpr int MAX_ITEMS = 880;
constexpr int SD = 4;                // row-read operands in flight
constexpr int PD = 3;                // transposing-read operands in flight

struct BwdPlan {
  int n;                             // tiles per head in this launch
  int by_xcd;                        // heads dealt to XCDs (else workgroup b: head b % H, tile b / H)
  uint32_t t[MAX_ITEMS];             // (document << 16) | 128-row tile index in the document
};

struct BwdArgs {
  const bf16* q; const bf16* kv; const bf16* kpe; int64_t kpe_stride;
  const bf16* o; const bf16* dout;
  const int32_t* cu; int n_tokens; int heads;
  float scale;                       // softmax scale
  float* lse;                        // [H, N] base-2 log-sum-exp of scale * q.k
  float* dsum;                       // [H, N] D = rowsum(dO * O)
  float* dq;                         // [N, H, 192]
  float* dkv;                        // [N, H, 256] = [dk_nope | dv]
  float* dkr;                        // [N, H, 64] per-head gradient of the shared key part
  float* dkpe;                       // [N, 64]
  int d_in_dq;                       // the dq pass forms D (lse given by the forward)
  // bf16 outputs in place of dq and of the [dk_nope | dv] part of dkv: dq16
  // with the rotary map undone on dims 128..191 (rope set), the gradient with
  // respect to the query before its rotation
  bf16* dq16; bf16* dkv16;
  const float* cos_t; const float* sin_t; const int32_t* positions;
  int table_len; int rope; int rope_interleave;
};

// chunk swizzles (bits of the row permuted; see the header)
__device__ __forceinline__ int swn(int r) { return ((r & 1) << 3) | ((r & 2) << 1) | ((r >> 1) & 2) | ((r >> 3) & 1); }
__device__ __forceinline__ int swr(int r) { return ((r & 2) << 1) | ((r >> 1) & 2) | ((r >> 3) & 1); }
// element offsets of (row, column) in a 128-wide and a 64-wide tile
__device__ __forceinline__ int offn(int r, int col) { return r * 128 + (((col >> 3) ^ swn(r)) << 3) + (col & 7); }
__device__ __forceinline__ int offr(int r, int col) { return r * 64 + (((col >> 3) ^ swr(r)) << 3) + (col & 7); }

__device__ __forceinline__ bf16x8 zero8b() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// 4-byte asynchronous global -> LDS copy (lane l lands at lds_addr + 4 l, a
// wave-uniform LDS address); awaited like the 16-byte copies.
__device__ __forceinline__ void lds_dma4_m0(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(gsrc), "s"(lds_addr) : "memory", "m0");
}

// Transposing read of a swizzled tile: the A operand of 32 columns
// c0 .. c0 + 31 (rows of the MFMA) and 16 K rows r0 .. r0 + 15 taken in the
// order {4h + j, 8 + 4h + j}, h = lane / 32: the row order of a score tile's
// C layout.  Within a 16-lane group, lane L addresses row r0 + 4 (group / 2)
// + L / 4, columns c0 + 16 (group % 2) + 4 (L % 4) .. + 3 (see lds_read_tr).
template <bool WIDE>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int r0, int c0, int lane) {
  const int grp = lane >> 4, L16 = lane & 15;
  const int row = r0 + (grp >> 1) * 4 + (L16 >> 2);
  const int col = c0 + (grp & 1) * 16 + 4 * (L16 & 3);
  const bf16x4 lo = lds_read_tr(tile + (WIDE ? offn(row, col) : offr(row, col)));
  const bf16x4 hi = lds_read_tr(tile + (WIDE ? offn(row + 8, col) : offr(row + 8, col)));
  return cat8(lo, hi);
}

// Which (head, tile) a workgroup takes; false when it has none.
__device__ __forceinline__ bool work_item(const BwdPlan& plan, int H, int& h, uint32_t& td) {
  if (!plan.by_xcd) {
    h = (int)(blockIdx.x % (unsigned)H);
    td = plan.t[blockIdx.x / (unsigned)H];
    return true;
  }
  const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
  const int hl = s / plan.n, ti = s - hl * plan.n;
  h = x + 8 * hl;
  if (h >= H) return false;
  td = plan.t[ti];
  return true;
}

// Per-lane copy sources of a 64-row tile [64][W] (W = 128: 16 copies of 1 KB,
// 4 per wave; W = 64: 8 copies, 2 per wave): copy i of wave w fills LDS chunk
// positions P = (w + 4 i) 64 + lane, i.e. row P / (W / 8), physical chunk
// P % (W / 8), which holds logical chunk physical ^ swizzle(row).  The row
// bits the swizzle reads do not depend on i, so a lane's chunk is the same in
// all of its copies and its rows step by 2048 / W.
template <int W>
struct TileCopy {
  static constexpr int NC = W == 128 ? 4 : 2;
  static constexpr int STEP = 2048 / W;
  int row0;                          // tile row of the first copy
  int col_bytes;                     // byte offset of the logical chunk in the row
  __device__ __forceinline__ void init(int wave, int lane) {
    const int P = wave * 64 + lane;
    row0 = P / (W / 8);
    const int pc = P % (W / 8);
    col_bytes = (pc ^ (W == 128 ? swn(row0) : swr(row0))) << 4;
  }
  // rows at or past `valid` repeat row valid - 1; lds_tile: LDS byte address
  // of the tile, wave: the wave index held in a scalar register
  __device__ __forceinline__ void issue(const bf16* base, int row_bytes, int valid, uint32_t lds_tile,
                                        int wave) const {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int r = min(row0 + i * STEP, valid - 1);
      lds_dma16_sv_m0(base, (uint32_t)(r * row_bytes + col_bytes), lds_tile + (uint32_t)(wave + 4 * i) * 1024u);
    }
  }
};

template <int B> struct BufC { static constexpr int value = B; };

// ----------------------------------------------------------------------------- pass 1
__global__ __launch_bounds__(256, 2) void bwd_stats_kernel(BwdArgs a, BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) bf16 sKn[2][ST * DN];
  __shared__ __attribute__((aligned(16))) bf16 sKr[2][ST * DR];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  int h;
  uint32_t td;
  if (!work_item(plan, H, h, td)) return;
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = a.cu[doc], de = a.cu[doc + 1];
  const int q0 = ds + tix * BT;
  if (q0 >= de) return;
  const int q1 = min(q0 + BT, de);
  const int qw0 = q0 + wave * 32, my_q = qw0 + (lane & 31), hsel = lane >> 5;
  const int64_t qrow = (int64_t)H * DQK, kvrow = (int64_t)H * (DN + DV);
  bf16x8 qreg[DQK / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    qreg[ks] = my_q < q1 ? *(const bf16x8*)(a.q + my_q * qrow + h * DQK + ks * 16 + hsel * 8) : zero8b();
  TileCopy<DN> cn;
  TileCopy<DR> cr;
  cn.init(wave, lane);
  cr.init(wave, lane);
  const bf16* kvh = uniform_ptr(a.kv + h * (DN + DV));
  const int nt = (q1 - ds + ST - 1) / ST;
  auto issue = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = ds + it * ST;
    cn.issue(kvh + (int64_t)kb * kvrow, (int)(kvrow * 2), de - kb, lds_addr_of(sKn[buf]), wave);
    cr.issue(uniform_ptr(a.kpe + (int64_t)kb * a.kpe_stride), (int)(a.kpe_stride * 2), de - kb, lds_addr_of(sKr[buf]),
             wave);
  };
  const float c2 = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = ds + it * ST;
    vm_wait_all();
    wg_barrier();
    if (it + 1 < nt) issue(it + 1, BufC<buf ^ 1>{});
    if (qw0 >= q1 || kb > qw0 + 31) return;
    // S^T for two key blocks of 32 (alternating chains), operands read SD ahead
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
    auto kread = [&](int i) {
      const int kr = (i & 1) * 32 + (lane & 31), ks = i >> 1;
      return ks < 8 ? *(const bf16x8*)&sKn[buf][offn(kr, ks * 16 + hsel * 8)]
                    : *(const bf16x8*)&sKr[buf][offr(kr, (ks - 8) * 16 + hsel * 8)];
    };
    bf16x8 kf[SD];
#pragma unroll
    for (int i = 0; i < SD; ++i) kf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = kf[i % SD];
      if (i + SD < 24) kf[i % SD] = kread(i + SD);
      s[i & 1] = mfma32(cur, qreg[i >> 1], s[i & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
        if (key > my_q) s[mt][e] = -INFINITY;
        mx = fmaxf(mx, s[mt][e] * c2);
      }
    const float mn = fmaxf(m, mx);
    if (mn > -INFINITY) {
      float acc = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += __builtin_amdgcn_exp2f(s[mt][e] * c2 - mn);
      l = l * __builtin_amdgcn_exp2f(m - mn) + acc;
      m = mn;
    }
  };
  issue(0, BufC<0>{});
  for (int it = 0; it < nt; it += 2) {
    step(it, BufC<0>{});
    if (it + 1 < nt) step(it + 1, BufC<1>{});
  }
  // combine the two lanes of a query (each saw half of every key block)
  const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
  const float mm = fmaxf(m, mo);
  const float lt = (m > -INFINITY ? l * __builtin_amdgcn_exp2f(m - mm) : 0.f) +
                   (mo > -INFINITY ? lo * __builtin_amdgcn_exp2f(mo - mm) : 0.f);
  // D = rowsum(dO * O): lane half hsel takes 64 of the 128 dims
  float d = 0.f;
  if (my_q < q1) {
    const bf16* orow = a.o + ((int64_t)my_q * H + h) * DV + hsel * 64;
    const bf16* grow = a.dout + ((int64_t)my_q * H + h) * DV + hsel * 64;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 ov = *(const bf16x8*)(orow + c * 8), gv = *(const bf16x8*)(grow + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf((float)ov[e], (float)gv[e], d);
    }
  }
  d += __shfl_xor(d, 32, 64);
  if (my_q < q1 && hsel == 0) {
    a.lse[(int64_t)h * a.n_tokens + my_q] = mm + __builtin_log2f(lt);
    a.dsum[(int64_t)h * a.n_tokens + my_q] = d;
  }
}

// ----------------------------------------------------------------------------- pass 2: dq
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) bf16 sKn[2][ST * DN];
  __shared__ __attribute__((aligned(16))) bf16 sKr[2][ST * DR];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][ST * DV];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  int h;
  uint32_t td;
  if (!work_item(plan, H, h, td)) return;
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = a.cu[doc], de = a.cu[doc + 1];
  const int q0 = ds + tix * BT;
  if (q0 >= de) return;
  const int q1 = min(q0 + BT, de);
  const int qw0 = q0 + wave * 32, my_q = qw0 + (lane & 31), hsel = lane >> 5;
  const bool live = my_q < q1;
  const int64_t qrow = (int64_t)H * DQK, kvrow = (int64_t)H * (DN + DV);
  // B operands held for the whole walk: Q^T (k = dims) and dO^T (k = dv)
  bf16x8 qreg[DQK / 16], greg[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    qreg[ks] = live ? *(const bf16x8*)(a.q + my_q * qrow + h * DQK + ks * 16 + hsel * 8) : zero8b();
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    greg[ks] = live ? *(const bf16x8*)(a.dout + ((int64_t)my_q * H + h) * DV + ks * 16 + hsel * 8) : zero8b();
  const float c2 = a.scale * kLog2e;
  const float lse = live ? a.lse[(int64_t)h * a.n_tokens + my_q] : 0.f;
  float dsum;
  if (a.d_in_dq) {
    // D = rowsum(dO * O) over the dims this lane holds of dO, then the other half
    float d = 0.f;
    if (live) {
      const bf16* orow = a.o + ((int64_t)my_q * H + h) * DV + hsel * 8;
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) {
        const bf16x8 ov = *(const bf16x8*)(orow + ks * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf((float)ov[e], (float)greg[ks][e], d);
      }
    }
    d += __shfl_xor(d, 32, 64);
    dsum = d;
    if (live && hsel == 0) a.dsum[(int64_t)h * a.n_tokens + my_q] = d;
  } else {
    dsum = live ? a.dsum[(int64_t)h * a.n_tokens + my_q] : 0.f;
  }
  f32x16 acc[DQK / 32];
#pragma unroll
  for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  TileCopy<DN> cn;
  TileCopy<DR> cr;
  cn.init(wave, lane);
  cr.init(wave, lane);
  const bf16* kvh = uniform_ptr(a.kv + h * (DN + DV));
  const int nt = (q1 - ds + ST - 1) / ST;
  auto issue = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = ds + it * ST;
    cn.issue(kvh + (int64_t)kb * kvrow, (int)(kvrow * 2), de - kb, lds_addr_of(sKn[buf]), wave);
    cr.issue(uniform_ptr(a.kpe + (int64_t)kb * a.kpe_stride), (int)(a.kpe_stride * 2), de - kb, lds_addr_of(sKr[buf]),
             wave);
    cn.issue(kvh + (int64_t)kb * kvrow + DN, (int)(kvrow * 2), de - kb, lds_addr_of(sV[buf]), wave);
  };

  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = ds + it * ST;
    vm_wait_all();
    wg_barrier();
    if (it + 1 < nt) issue(it + 1, BufC<buf ^ 1>{});
    if (qw0 >= q1 || kb > qw0 + 31) return;
    // one key block of 32 at a time: S^T [key, query] and dP^T = V dO^T on
    // alternating chains (operands read SD ahead), dS^T = P^T (dP^T - D) with
    // P^T = 2^(s c2 - lse) masked past the query, then dQ^T [d, query] +=
    // K^T [d, key] dS^T [key, query], the block's two k-steps covering keys
    // mt*32 + jj*16 + {4h + [0,4), 8 + 4h + [0,4)} (operands read PD ahead)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int kr = mt * 32 + (lane & 31);
      auto aread = [&](int i) {
        if (i < 16) {
          const int ks = i >> 1;
          return (i & 1) ? *(const bf16x8*)&sV[buf][offn(kr, ks * 16 + hsel * 8)]
                         : *(const bf16x8*)&sKn[buf][offn(kr, ks * 16 + hsel * 8)];
        }
        return *(const bf16x8*)&sKr[buf][offr(kr, (i - 16) * 16 + hsel * 8)];
      };
      auto bread = [&](int i) {
        const int jj = i / 6, b = i % 6, r0 = mt * 32 + jj * 16;
        return b < 4 ? tr_operand<true>(sKn[buf], r0, b * 32, lane) : tr_operand<false>(sKr[buf], r0, (b - 4) * 32, lane);
      };
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
      bf16x8 af[SD];
#pragma unroll
      for (int i = 0; i < SD; ++i) af[i] = aread(i);
#pragma unroll
      for (int i = 0; i < 20; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = af[i % SD];
        if (i + SD < 20) af[i % SD] = aread(i + SD);
        if (i < 16 && (i & 1)) dp = mfma32(cur, greg[i >> 1], dp);
        else s = mfma32(cur, qreg[i < 16 ? i >> 1 : 8 + (i - 16)], s);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 bf[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) bf[i] = bread(i);
      bf16x8 dsb[2];
      if (kb + mt * 32 + 31 <= qw0) {
        // every key of the block is at or before the wave's first query
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[e] * c2 - lse);
          dsb[e >> 3][e & 7] = (bf16)(p * (dp[e] - dsum));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
          const float p = key <= my_q ? __builtin_amdgcn_exp2f(s[e] * c2 - lse) : 0.f;
          dsb[e >> 3][e & 7] = (bf16)(p * (dp[e] - dsum));
        }
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = bf[i % PD];
        if (i + PD < 12) bf[i % PD] = bread(i + PD);
        acc[i % 6] = mfma32(cur, dsb[i / 6], acc[i % 6]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  issue(0, BufC<0>{});
  for (int it = 0; it < nt; it += 2) {
    step(it, BufC<0>{});
    if (it + 1 < nt) step(it + 1, BufC<1>{});
  }
  if (!live) return;
  // lane holds query my_q, dims b*32 + (e/4)*8 + hsel*4 + e%4
  if (a.dq16) {
    f32x16 y[DQK / 32];
#pragma unroll
    for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) y[b][e] = acc[b][e] * a.scale;
    if (a.rope) {
      // the transpose of the rotation on the pairs of the 64 rotary dims
      // (blocks 4 and 5): (i, i + 32) or, interleaved, (2i, 2i + 1)
      const int pos = a.positions[my_q];
      const bool ok = pos >= 0 && pos < a.table_len;
      const float* ct = a.cos_t + (int64_t)(ok ? pos : 0) * (DR / 2);
      const float* sn = a.sin_t + (int64_t)(ok ? pos : 0) * (DR / 2);
      const float nan = __builtin_nanf("");
      if (a.rope_interleave) {
#pragma unroll
        for (int b = 4; b < 6; ++b)
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const int pi = ((b - 4) * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3)) >> 1;
            const float c = ok ? ct[pi] : nan, s = ok ? sn[pi] : nan;
            const float v0 = y[b][e], v1 = y[b][e + 1];
            y[b][e] = v0 * c + v1 * s;
            y[b][e + 1] = v1 * c - v0 * s;
          }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int pi = (e >> 2) * 8 + hsel * 4 + (e & 3);
          const float c = ok ? ct[pi] : nan, s = ok ? sn[pi] : nan;
          const float v0 = y[4][e], v1 = y[5][e];
          y[4][e] = v0 * c + v1 * s;
          y[5][e] = v1 * c - v0 * s;
        }
      }
    }
    bf16* out16 = a.dq16 + ((int64_t)my_q * H + h) * DQK;
#pragma unroll
    for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 v = {(bf16)y[b][g * 4 + 0], (bf16)y[b][g * 4 + 1], (bf16)y[b][g * 4 + 2], (bf16)y[b][g * 4 + 3]};
        *(bf16x4*)(out16 + b * 32 + g * 8 + hsel * 4) = v;
      }
    return;
  }
  float* out = a.dq + ((int64_t)my_q * H + h) * DQK;
#pragma unroll
  for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = acc[b][g * 4 + 0] * a.scale; v.y = acc[b][g * 4 + 1] * a.scale;
      v.z = acc[b][g * 4 + 2] * a.scale; v.w = acc[b][g * 4 + 3] * a.scale;
      *(float4*)(out + b * 32 + g * 8 + hsel * 4) = v;
    }
}

// ----------------------------------------------------------------------------- pass 3: dk, dv
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a, BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) bf16 sQn[2][ST * DN];
  __shared__ __attribute__((aligned(16))) bf16 sQr[2][ST * DR];
  __shared__ __attribute__((aligned(16))) bf16 sG[2][ST * DV];
  __shared__ __attribute__((aligned(16))) float sL[2][ST];
  __shared__ __attribute__((aligned(16))) float sD[2][ST];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  int h;
  uint32_t td;
  if (!work_item(plan, H, h, td)) return;
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = a.cu[doc], de = a.cu[doc + 1];
  const int k0 = ds + tix * BT;
  if (k0 >= de) return;
  const int k1 = min(k0 + BT, de);
  const int kw0 = k0 + wave * 32, my_k = kw0 + (lane & 31), hsel = lane >> 5;
  const bool live = my_k < k1;
  const int64_t qrow = (int64_t)H * DQK, kvrow = (int64_t)H * (DN + DV);
  // B operands held for the whole walk: K^T (k = dims) and V^T (k = dv) of this lane's key
  bf16x8 kreg[DQK / 16], vreg[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks) {
    const int d = ks * 16 + hsel * 8;
    kreg[ks] = !live ? zero8b()
                     : d < DN ? *(const bf16x8*)(a.kv + my_k * kvrow + h * (DN + DV) + d)
                              : *(const bf16x8*)(a.kpe + my_k * a.kpe_stride + (d - DN));
  }
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    vreg[ks] = live ? *(const bf16x8*)(a.kv + my_k * kvrow + h * (DN + DV) + DN + ks * 16 + hsel * 8) : zero8b();
  const float c2 = a.scale * kLog2e;
  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[b][e] = 0.f;
#pragma unroll
  for (int b = 0; b < DV / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) dv[b][e] = 0.f;
  TileCopy<DN> cn;
  TileCopy<DR> cr;
  cn.init(wave, lane);
  cr.init(wave, lane);
  const bf16* qh = uniform_ptr(a.q + h * DQK);
  const bf16* gh = uniform_ptr(a.dout + h * DV);
  const float* lh = a.lse + (int64_t)h * a.n_tokens;
  const float* dh = a.dsum + (int64_t)h * a.n_tokens;
  const int64_t grow = (int64_t)H * DV;
  // queries that see these keys: from the tile holding key k0 to the document end
  const int qb0 = ds + ((k0 - ds) / ST) * ST;
  const int nt = (de - qb0 + ST - 1) / ST;
  auto issue = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int qb = qb0 + it * ST;
    cn.issue(qh + (int64_t)qb * qrow, (int)(qrow * 2), de - qb, lds_addr_of(sQn[buf]), wave);
    cr.issue(qh + (int64_t)qb * qrow + DN, (int)(qrow * 2), de - qb, lds_addr_of(sQr[buf]), wave);
    cn.issue(gh + (int64_t)qb * grow, (int)(grow * 2), de - qb, lds_addr_of(sG[buf]), wave);
    if (wave == 0) {
      const int t = min(qb + lane, de - 1);
      lds_dma4_m0(lh + t, lds_addr_of(sL[buf]));
      lds_dma4_m0(dh + t, lds_addr_of(sD[buf]));
    }
  };

  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int qb = qb0 + it * ST;
    vm_wait_all();
    wg_barrier();
    if (it + 1 < nt) issue(it + 1, BufC<buf ^ 1>{});
    if (kw0 >= k1 || qb + ST - 1 < kw0) return;
    // one query block of 32 at a time: S [query, key] = Q K^T and
    // dP = dO V^T on alternating chains (operands read SD ahead),
    // P = 2^(s c2 - lse[q]) for q >= key (same document), dS = P (dP - D[q]),
    // then dV^T [dv, key] += dO^T [dv, query] P and dK^T [d, key] += Q^T dS
    // (operands read PD ahead)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int qr = mt * 32 + (lane & 31);
      auto aread = [&](int i) {
        if (i < 16) {
          const int ks = i >> 1;
          return (i & 1) ? *(const bf16x8*)&sG[buf][offn(qr, ks * 16 + hsel * 8)]
                         : *(const bf16x8*)&sQn[buf][offn(qr, ks * 16 + hsel * 8)];
        }
        return *(const bf16x8*)&sQr[buf][offr(qr, (i - 16) * 16 + hsel * 8)];
      };
      auto bread = [&](int i) {
        const int jj = i / 10, b = i % 10, r0 = mt * 32 + jj * 16;
        return b < 4 ? tr_operand<true>(sG[buf], r0, b * 32, lane)
                     : b < 8 ? tr_operand<true>(sQn[buf], r0, (b - 4) * 32, lane)
                             : tr_operand<false>(sQr[buf], r0, (b - 8) * 32, lane);
      };
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
      bf16x8 af[SD];
#pragma unroll
      for (int i = 0; i < SD; ++i) af[i] = aread(i);
#pragma unroll
      for (int i = 0; i < 20; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = af[i % SD];
        if (i + SD < 20) af[i % SD] = aread(i + SD);
        if (i < 16 && (i & 1)) dp = mfma32(cur, vreg[i >> 1], dp);
        else s = mfma32(cur, kreg[i < 16 ? i >> 1 : 8 + (i - 16)], s);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 bf[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) bf[i] = bread(i);
      // lse and D of this lane's query rows mt*32 + g*8 + hsel*4 + [0, 4),
      // read one group of 4 at a time
      bf16x8 pb[2], dsb[2];
      // every query row of the block after every key of the wave, inside the
      // document, every key live: no mask
      const bool nomask = qb + mt * 32 >= kw0 + 31 && qb + mt * 32 + 31 < de && kw0 + 31 < k1;
      if (nomask) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 lq = *(const float4*)&sL[buf][mt * 32 + g * 8 + hsel * 4];
          const float4 dq4 = *(const float4*)&sD[buf][mt * 32 + g * 8 + hsel * 4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = g * 4 + j;
            const float p = __builtin_amdgcn_exp2f(s[e] * c2 - lq[j]);
            pb[e >> 3][e & 7] = (bf16)p;
            dsb[e >> 3][e & 7] = (bf16)(p * (dp[e] - dq4[j]));
          }
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 lq = *(const float4*)&sL[buf][mt * 32 + g * 8 + hsel * 4];
          const float4 dq4 = *(const float4*)&sD[buf][mt * 32 + g * 8 + hsel * 4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = g * 4 + j;
            const int t = qb + mt * 32 + g * 8 + hsel * 4 + j;
            const float p = (t >= my_k && t < de && live) ? __builtin_amdgcn_exp2f(s[e] * c2 - lq[j]) : 0.f;
            pb[e >> 3][e & 7] = (bf16)p;
            dsb[e >> 3][e & 7] = (bf16)(p * (dp[e] - dq4[j]));
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 20; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = bf[i % PD];
        if (i + PD < 20) bf[i % PD] = bread(i + PD);
        const int jj = i / 10, b = i % 10;
        if (b < 4) dv[b] = mfma32(cur, pb[jj], dv[b]);
        else dk[b - 4] = mfma32(cur, dsb[jj], dk[b - 4]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  issue(0, BufC<0>{});
  for (int it = 0; it < nt; it += 2) {
    step(it, BufC<0>{});
    if (it + 1 < nt) step(it + 1, BufC<1>{});
  }
  if (!live) return;
  // lane holds key my_k, dims b*32 + (e/4)*8 + hsel*4 + e%4
  float* okr = a.dkr + ((int64_t)my_k * H + h) * DR;
  if (a.dkv16) {
    bf16* o16 = a.dkv16 + ((int64_t)my_k * H + h) * (DN + DV);
#pragma unroll
    for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float x0 = dk[b][g * 4 + 0] * a.scale, x1 = dk[b][g * 4 + 1] * a.scale;
        const float x2 = dk[b][g * 4 + 2] * a.scale, x3 = dk[b][g * 4 + 3] * a.scale;
        const int d = b * 32 + g * 8 + hsel * 4;
        if (d < DN) {
          const bf16x4 v = {(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
          *(bf16x4*)(o16 + d) = v;
        } else {
          *(float4*)(okr + d - DN) = make_float4(x0, x1, x2, x3);
        }
      }
#pragma unroll
    for (int b = 0; b < DV / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 v = {(bf16)dv[b][g * 4 + 0], (bf16)dv[b][g * 4 + 1], (bf16)dv[b][g * 4 + 2],
                          (bf16)dv[b][g * 4 + 3]};
        *(bf16x4*)(o16 + DN + b * 32 + g * 8 + hsel * 4) = v;
      }
    return;
  }
  float* okv = a.dkv + ((int64_t)my_k * H + h) * (DN + DV);
#pragma unroll
  for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = dk[b][g * 4 + 0] * a.scale; v.y = dk[b][g * 4 + 1] * a.scale;
      v.z = dk[b][g * 4 + 2] * a.scale; v.w = dk[b][g * 4 + 3] * a.scale;
      const int d = b * 32 + g * 8 + hsel * 4;
      if (d < DN) *(float4*)(okv + d) = v;
      else *(float4*)(okr + d - DN) = v;
    }
#pragma unroll
  for (int b = 0; b < DV / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = dv[b][g * 4 + 0]; v.y = dv[b][g * 4 + 1]; v.z = dv[b][g * 4 + 2]; v.w = dv[b][g * 4 + 3];
      *(float4*)(okv + DN + b * 32 + g * 8 + hsel * 4) = v;
    }
}

// dk_pe[t, :] = sum over heads of the per-head shared-part gradients, in
// head order; a thread takes 4 columns (16-byte loads), 8 heads' loads in
// flight
__global__ __launch_bounds__(256) void bwd_kpe_sum_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_tokens * (DR / 4)) return;
  const int64_t t = i / (DR / 4);
  const int c = (int)(i - t * (DR / 4)) * 4;
  const float* src = a.dkr + t * a.heads * DR + c;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int h = 0;
  for (; h + 8 <= a.heads; h += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const float4*)(src + (h + u) * DR);
#pragma unroll
    for (int u = 0; u < 8; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
  }
  for (; h < a.heads; ++h) {
    const float4 v = *(const float4*)(src + h * DR);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *(float4*)(a.dkpe + t * DR + c) = s;
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdArgs& g, const int32_t* cu_host, int num_seqs, hipStream_t s) {
  BwdArgs a{};
  a.q = (const bf16*)g.q; a.kv = (const bf16*)g.kv; a.kpe = (const bf16*)g.kpe; a.kpe_stride = g.kpe_stride;
  a.o = (const bf16*)g.o; a.dout = (const bf16*)g.dout; a.cu = g.cu_dev; a.n_tokens = g.n_tokens; a.heads = g.heads;
  a.scale = g.scale; a.lse = g.lse; a.dsum = g.dsum; a.dq = g.dq; a.dkv = g.dkv; a.dkr = g.dkr; a.dkpe = g.dkpe;
  a.d_in_dq = g.lse_ready ? 1 : 0;
  a.dq16 = g.dq16; a.dkv16 = g.dkv16; a.cos_t = g.cos_t; a.sin_t = g.sin_t; a.positions = g.positions;
  a.table_len = g.table_len; a.rope = g.rope ? 1 : 0; a.rope_interleave = g.rope_interleave ? 1 : 0;
  if (g.n_tokens <= 0) return hipSuccess;
  // every (document, 128-row tile); the query-major passes take the tiles
  // with the longest key range first, the key-major pass those with the
  // longest query range
  struct T { int q_work, k_work; uint32_t id; };
  std::vector<T> tiles;
  for (int d = 0; d < num_seqs; ++d) {
    const int len = cu_host[d + 1] - cu_host[d];
    for (int i = 0; i * BT < len; ++i)
      tiles.push_back({std::min((i + 1) * BT, len), len - i * BT, ((uint32_t)d << 16) | (uint32_t)i});
  }
  BwdPlan plan;
  plan.by_xcd = g.heads >= 8;
  const unsigned heads_per_xcd = (unsigned)((g.heads + 7) / 8);
  for (int pass = g.lse_ready ? 1 : 0; pass < 3; ++pass) {
    if (pass != 2)
      std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.q_work > y.q_work; });
    else
      std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.k_work > y.k_work; });
    for (size_t base = 0; base < tiles.size(); base += MAX_ITEMS) {
      plan.n = (int)std::min<size_t>(MAX_ITEMS, tiles.size() - base);
      for (int i = 0; i < plan.n; ++i) plan.t[i] = tiles[base + i].id;
      const unsigned grid = (plan.by_xcd ? 8u * heads_per_xcd : (unsigned)g.heads) * (unsigned)plan.n;
      if (pass == 0) bwd_stats_kernel<<<grid, 256, 0, s>>>(a, plan);
      else if (pass == 1) bwd_dq_kernel<<<grid, 256, 0, s>>>(a, plan);
      else bwd_dkdv_kernel<<<grid, 256, 0, s>>>(a, plan);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t n = (int64_t)g.n_tokens * (DR / 4);
  bwd_kpe_sum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
