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
//   1. stats: per (query, head) the log-sum-exp of the scaled scores in
//      base-2 units (the forward's softmax statistics, recomputed: one QK^T
//      pass) and D;
//   2. dq, query-major (workgroup = 128 queries of one head, keys in tiles of
//      64): S^T = K Q^T and dP^T = V dO^T from the recomputed P^T, then
//      dQ^T += K^T dS^T, K^T by transposing LDS reads;
//   3. dk and dv, key-major (workgroup = 128 keys of one head, queries in
//      tiles of 64): S = Q K^T, P, dV^T += dO^T P, dP = dO V^T, dS,
//      dK^T += Q^T dS, dO^T and Q^T by transposing LDS reads.
// P and dS are rounded to bf16 as MFMA operands.  Every lane owns one query
// (pass 2) or one key (pass 3) column, so the per-row statistics are per lane.
// Tiles are staged through LDS with rows padded by 16 bytes (row stride 400
// or 272 B), which keeps the 16 rows of a row read and the 4 rows of a
// transposing read on different banks.
#include "mla_internal.hpp"

#include <vector>
#include <algorithm>

namespace mla {
namespace {

constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int QP = DQK + 8;          // padded row of a q / k tile (elements)
constexpr int VP = DV + 8;           // padded row of a v / dO tile
constexpr int BT = 128;              // rows (queries or keys) per workgroup
constexpr int ST = 64;               // rows of the streamed tile
constexpr int MAX_ITEMS = 880;

struct BwdPlan {
  int n;                             // work items in this launch
  uint32_t t[MAX_ITEMS];             // (document << 16) | 128-row tile index in the document
};

struct BwdArgs {
  const bf16* q; const bf16* kv; const bf16* kpe; int64_t kpe_stride;
  const bf16* o; const bf16* dout;
  const int32_t* cu; int n_tokens; int heads;
  float scale;                       // softmax scale
  float* lse;                        // [N, H] base-2 log-sum-exp of scale * q.k
  float* dsum;                       // [N, H] D = rowsum(dO * O)
  float* dq;                         // [N, H, 192]
  float* dkv;                        // [N, H, 256] = [dk_nope | dv]
  float* dkr;                        // [N, H, 64] per-head gradient of the shared key part
  float* dkpe;                       // [N, 64]
};

__device__ __forceinline__ bf16x8 zero8b() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// transposing read of a padded row-major tile X[row][col] (stride P elements):
// lane i of a 16-lane group receives X[r0 + j][c0 + i] for j = 0..3 (see
// lds_read_tr); a lane L addresses &X[r0 + L/4][c0 + 4 (L%4)]
template <int P>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int r0, int c0, int lane) {
  // A operand of 32 columns (rows of the MFMA) c0 .. c0 + 31 and 16 K rows
  // r0 .. r0 + 15 in the order {4h + j, 8 + 4h + j}, h = lane / 32: the key
  // (or query) order of a score tile's C layout
  const int grp = lane >> 4, L16 = lane & 15;
  const int row = r0 + (grp >> 1) * 4 + (L16 >> 2);
  const int col = c0 + (grp & 1) * 16 + 4 * (L16 & 3);
  const bf16x4 lo = lds_read_tr(tile + row * P + col);
  const bf16x4 hi = lds_read_tr(tile + (row + 8) * P + col);
  return cat8(lo, hi);
}

// Copies rows [r0, r0 + nrows) of a [*, width] bf16 source (row stride
// src_stride elements, rows past `valid` replaced by zeros) into a padded LDS
// tile (stride P), 8 elements per thread and step.
template <int P>
__device__ __forceinline__ void load_tile(bf16* tile, const bf16* src, int64_t src_stride, int r0, int nrows,
                                          int valid, int width, int col0 = 0) {
  const int cpr = width / 8;
  for (int i = threadIdx.x; i < nrows * cpr; i += 256) {
    const int r = i / cpr, c = i - r * cpr;
    bf16x8 v = zero8b();
    if (r0 + r < valid) v = *(const bf16x8*)(src + (int64_t)(r0 + r) * src_stride + c * 8);
    *(bf16x8*)(tile + r * P + col0 + c * 8) = v;
  }
}

// ----------------------------------------------------------------------------- pass 1
__global__ __launch_bounds__(256, 2) void bwd_stats_kernel(BwdArgs a, BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) bf16 sK[ST * QP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, H = a.heads;
  const uint32_t td = plan.t[blockIdx.x];
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
  const float c2 = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  for (int kb = ds; kb < q1; kb += ST) {
    __syncthreads();
    load_tile<QP>(sK, a.kv + h * (DN + DV), kvrow, kb, ST, de, DN);
    load_tile<QP>(sK, a.kpe, a.kpe_stride, kb, ST, de, DR, DN);
    __syncthreads();
    if (qw0 >= q1 || kb > qw0 + 31) continue;
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks)
        s[mt] = mfma32(*(const bf16x8*)&sK[(mt * 32 + (lane & 31)) * QP + ks * 16 + hsel * 8], qreg[ks], s[mt]);
    }
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
    a.lse[(int64_t)my_q * H + h] = mm + __builtin_log2f(lt);
    a.dsum[(int64_t)my_q * H + h] = d;
  }
}

// ----------------------------------------------------------------------------- pass 2: dq
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, BwdPlan plan) {
  __shared__ __attribute__((aligned(16))) bf16 sK[ST * QP];
  __shared__ __attribute__((aligned(16))) bf16 sV[ST * VP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, H = a.heads;
  const uint32_t td = plan.t[blockIdx.x];
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
  const float lse = live ? a.lse[(int64_t)my_q * H + h] : 0.f;
  const float dsum = live ? a.dsum[(int64_t)my_q * H + h] : 0.f;
  f32x16 acc[DQK / 32];
#pragma unroll
  for (int b = 0; b < DQK / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

  for (int kb = ds; kb < q1; kb += ST) {
    __syncthreads();
    load_tile<QP>(sK, a.kv + h * (DN + DV), kvrow, kb, ST, de, DN);
    load_tile<QP>(sK, a.kpe, a.kpe_stride, kb, ST, de, DR, DN);
    load_tile<VP>(sV, a.kv + h * (DN + DV) + DN, kvrow, kb, ST, de, DV);
    __syncthreads();
    if (qw0 >= q1 || kb > qw0 + 31) continue;
    // S^T [key, query] and dP^T = V dO^T, two key blocks of 32
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[mt][e] = 0.f; dp[mt][e] = 0.f; }
      const int kr = mt * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks)
        s[mt] = mfma32(*(const bf16x8*)&sK[kr * QP + ks * 16 + hsel * 8], qreg[ks], s[mt]);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        dp[mt] = mfma32(*(const bf16x8*)&sV[kr * VP + ks * 16 + hsel * 8], greg[ks], dp[mt]);
    }
    // dS^T = P^T (dP^T - D), P^T = 2^(s c2 - lse), masked past the query
    bf16x8 dsb[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
        const float p = (key <= my_q && key < de) ? __builtin_amdgcn_exp2f(s[mt][e] * c2 - lse) : 0.f;
        dsb[mt * 2 + (e >> 3)][e & 7] = (bf16)(p * (dp[mt][e] - dsum));
      }
    // dQ^T [d, query] += K^T [d, key] dS^T [key, query]; k-step j covers keys
    // (j/2)*32 + (j%2)*16 + {4h + [0,4), 8 + 4h + [0,4)}
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = (j >> 1) * 32 + (j & 1) * 16;
#pragma unroll
      for (int b = 0; b < DQK / 32; ++b) acc[b] = mfma32(tr_operand<QP>(sK, r0, b * 32, lane), dsb[j], acc[b]);
    }
  }
  if (!live) return;
  // lane holds query my_q, dims b*32 + (e/4)*8 + hsel*4 + e%4
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
  __shared__ __attribute__((aligned(16))) bf16 sQ[ST * QP];
  __shared__ __attribute__((aligned(16))) bf16 sG[ST * VP];
  __shared__ float sL[ST], sD[ST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, H = a.heads;
  const uint32_t td = plan.t[blockIdx.x];
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

  // queries that see these keys: from the tile holding key k0 to the document end
  for (int qb = ds + ((k0 - ds) / ST) * ST; qb < de; qb += ST) {
    __syncthreads();
    load_tile<QP>(sQ, a.q + h * DQK, qrow, qb, ST, de, DQK);
    load_tile<VP>(sG, a.dout + h * DV, (int64_t)H * DV, qb, ST, de, DV);
    if (threadIdx.x < ST) {
      const int t = qb + threadIdx.x;
      sL[threadIdx.x] = t < de ? a.lse[(int64_t)t * H + h] : 0.f;
      sD[threadIdx.x] = t < de ? a.dsum[(int64_t)t * H + h] : 0.f;
    }
    __syncthreads();
    if (kw0 >= k1 || qb + ST - 1 < kw0) continue;
    // S [query, key] = Q K^T and dP = dO V^T, two query blocks of 32
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[mt][e] = 0.f; dp[mt][e] = 0.f; }
      const int qr = mt * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks)
        s[mt] = mfma32(*(const bf16x8*)&sQ[qr * QP + ks * 16 + hsel * 8], kreg[ks], s[mt]);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        dp[mt] = mfma32(*(const bf16x8*)&sG[qr * VP + ks * 16 + hsel * 8], vreg[ks], dp[mt]);
    }
    // P = 2^(s c2 - lse[q]) for q >= key (same document), dS = P (dP - D[q])
    bf16x8 pb[4], dsb[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ql = mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
        const int t = qb + ql;
        const float p = (t >= my_k && t < de && live) ? __builtin_amdgcn_exp2f(s[mt][e] * c2 - sL[ql]) : 0.f;
        pb[mt * 2 + (e >> 3)][e & 7] = (bf16)p;
        dsb[mt * 2 + (e >> 3)][e & 7] = (bf16)(p * (dp[mt][e] - sD[ql]));
      }
    // dV^T [dv, key] += dO^T [dv, query] P [query, key]; dK^T [d, key] += Q^T dS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = (j >> 1) * 32 + (j & 1) * 16;
#pragma unroll
      for (int b = 0; b < DV / 32; ++b) dv[b] = mfma32(tr_operand<VP>(sG, r0, b * 32, lane), pb[j], dv[b]);
#pragma unroll
      for (int b = 0; b < DQK / 32; ++b) dk[b] = mfma32(tr_operand<QP>(sQ, r0, b * 32, lane), dsb[j], dk[b]);
    }
  }
  if (!live) return;
  // lane holds key my_k, dims b*32 + (e/4)*8 + hsel*4 + e%4
  float* okv = a.dkv + ((int64_t)my_k * H + h) * (DN + DV);
  float* okr = a.dkr + ((int64_t)my_k * H + h) * DR;
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

// dk_pe[t, :] = sum over heads of the per-head shared-part gradients
__global__ __launch_bounds__(256) void bwd_kpe_sum_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_tokens * DR) return;
  const int64_t t = i / DR;
  const int c = (int)(i - t * DR);
  float s = 0.f;
  for (int h = 0; h < a.heads; ++h) s += a.dkr[(t * a.heads + h) * DR + c];
  a.dkpe[i] = s;
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdArgs& g, const int32_t* cu_host, int num_seqs, hipStream_t s) {
  BwdArgs a{};
  a.q = (const bf16*)g.q; a.kv = (const bf16*)g.kv; a.kpe = (const bf16*)g.kpe; a.kpe_stride = g.kpe_stride;
  a.o = (const bf16*)g.o; a.dout = (const bf16*)g.dout; a.cu = g.cu_dev; a.n_tokens = g.n_tokens; a.heads = g.heads;
  a.scale = g.scale; a.lse = g.lse; a.dsum = g.dsum; a.dq = g.dq; a.dkv = g.dkv; a.dkr = g.dkr; a.dkpe = g.dkpe;
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
  for (int pass = 0; pass < 3; ++pass) {
    if (pass != 2)
      std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.q_work > y.q_work; });
    else
      std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.k_work > y.k_work; });
    for (size_t base = 0; base < tiles.size(); base += MAX_ITEMS) {
      plan.n = (int)std::min<size_t>(MAX_ITEMS, tiles.size() - base);
      for (int i = 0; i < plan.n; ++i) plan.t[i] = tiles[base + i].id;
      dim3 grid((unsigned)plan.n, (unsigned)g.heads);
      if (pass == 0) bwd_stats_kernel<<<grid, 256, 0, s>>>(a, plan);
      else if (pass == 1) bwd_dq_kernel<<<grid, 256, 0, s>>>(a, plan);
      else bwd_dkdv_kernel<<<grid, 256, 0, s>>>(a, plan);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t n = (int64_t)g.n_tokens * DR;
  bwd_kpe_sum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
