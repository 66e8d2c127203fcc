// Causal varlen attention of the MLA prefill (d_qk = 192 = 128 + 64, d_v = 128).
//
// One 256-thread workgroup computes 128 query rows of one head of one packed
// document; each of its 4 waves owns 32 query rows.  Keys are walked in tiles
// of 64 from the document start to the last query of the tile (causal).  The
// key tile [k_nope_h (from kv) | k_pe (the one shared rope head, from the
// latent rows)] and the value tile v_h are copied into LDS by asynchronous
// global->LDS loads, double buffered, so tile t+1 streams in while tile t is
// multiplied.
//
// Contractions are v_mfma_f32_32x32x16_bf16 in the transposed orientation:
//   S^T[key, query]  = K[key, :] . Q[query, :]      (A = K from LDS, B = Q^T from registers)
//   O^T[dv, query]  += V^T[dv, key] . P^T[key, query] (A = V^T by LDS transpose read, B = P^T)
// so every lane holds one query row: the softmax max / sum need only an
// in-lane reduction plus one swap with the lane 32 away, and P^T feeds the
// second MFMA straight from the first MFMA's registers (the key order of the
// S^T output layout is matched by the transpose reads of V).  The online
// softmax is fp32 with exp2 and the scale folded in; P is rounded to the
// operand type (bf16, or fp16 inside the prefill layer) for the PV MFMA; the
// output is normalised in fp32 and rounded once to bf16.  d_v = 128 is used
// as is: v is never padded to d_qk.
#include "mla_internal.hpp"

#include <vector>
#include <algorithm>

namespace mla {
namespace {

constexpr int FQ = 128, FK = 64;
constexpr int DN = 128, DQK = 192, DV = 128;
constexpr int KCH = DQK / 8;          // 16-byte chunks per key row (24)
constexpr int MAX_TILES = 896;

struct TilePlan {
  int n;
  uint32_t t[MAX_TILES];              // (document << 16) | query-tile index in the document
};

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<f16> { typedef f16x8 v8; typedef f16x4 v4; };

template <typename V8> __device__ __forceinline__ V8 zero8() { return __builtin_bit_cast(V8, make_uint4(0, 0, 0, 0)); }
template <typename V4, typename T> __device__ __forceinline__ V4 read_tr(const T* p) {
  return __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(p)));
}
// K tile [64][192]: chunk c (0..23) of key row r at c ^ (r & 7) (stays within its group of 8).
__device__ __forceinline__ int koff(int r, int c) { return r * DQK + ((c ^ (r & 7)) << 3); }
// V tile [64][128]: 16 B chunk of column n in key row r at (n/8) ^ ((r & 3) << 1).
__device__ __forceinline__ int voff(int r, int n) { return r * DV + ((((n >> 3) ^ ((r & 3) << 1))) << 3) + (n & 7); }

template <typename T>
__global__ __launch_bounds__(256, 2) void flash_mfma_kernel(FlashArgs a, TilePlan plan) {
  typedef typename Vec<T>::v8 V8;
  typedef typename Vec<T>::v4 V4;
  __shared__ __attribute__((aligned(16))) T sK[2][FK * DQK];
  __shared__ __attribute__((aligned(16))) T sV[2][FK * DV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x;
  const int H = a.heads;
  const uint32_t td = plan.t[blockIdx.y];
  const int doc = (int)(td >> 16), tix = (int)(td & 0xffff);
  const int ds = max(0, min(a.cu_dev[doc], a.n_tokens));
  const int de = max(ds, min(a.cu_dev[doc + 1], a.n_tokens));
  const int q0 = ds + tix * FQ;
  if (q0 >= de) return;
  const int q1 = min(q0 + FQ, de);
  const int ntiles = (q1 - ds + FK - 1) / FK;

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

  // Tile loads go straight to LDS (16 B per lane, lane l of a wave fills the
  // l-th 16 B of a 1 KB block).  Each LDS position is mapped back to the
  // (key row, logical chunk) that the swizzled layout keeps there.  Keys past
  // the last query of the tile are clamped to the tile's first key: they are
  // masked out of the softmax (their probability is exactly 0) and are never
  // read out of bounds.
  auto issue_tile = [&](int t, int buf) {
    const int kb = ds + t * FK;
#pragma unroll
    for (int i = 0; i < 6; ++i) {                       // K: 24 blocks of 64 chunks
      const int blk = wave + 4 * i;
      const int P = blk * 64 + lane;
      const int r = P / KCH, pc = P - r * KCH;
      const int c = pc ^ (r & 7);
      const int key = (kb + r < q1) ? kb + r : kb;
      const T* src = (c < DN / 8) ? KV + key * kv_row + head * (DN + DV) + c * 8
                                  : KPE + key * a.kpe_stride + (c - DN / 8) * 8;
      lds_dma16(src, &sK[buf][blk * 512]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {                       // V: 16 blocks of 64 chunks
      const int blk = wave + 4 * i;
      const int P = blk * 64 + lane;
      const int r = P >> 4, pc = P & 15;
      const int c = pc ^ ((r & 3) << 1);
      const int key = (kb + r < q1) ? kb + r : kb;
      lds_dma16(KV + key * kv_row + head * (DN + DV) + DN + c * 8, &sV[buf][blk * 512]);
    }
  };

  const float c2 = a.scale * kLog2e;     // scores to base-2 exponent units
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;

  issue_tile(0, 0);
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kb = ds + t * FK;
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const bool active = (qw0 < q1) && (kb <= qw0 + 31);
    if (active) {
      // ---- S^T for 64 keys (2 tiles of 32) x 32 queries
      f32x16 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks) {
          const V8 kf = *(const V8*)&sK[buf][koff(mt * 32 + (lane & 31), ks * 2 + hsel)];
          s[mt] = mfma32(kf, qreg[ks], s[mt]);
        }
      }
      // ---- causal mask (only tiles that reach past this wave's first query)
      if (kb + FK - 1 > qw0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + mt * 32 + (e >> 2) * 8 + hsel * 4 + (e & 3);
            if (key > my_q) s[mt][e] = -INFINITY;
          }
      }
      // ---- online softmax (one query per lane, keys split across lane and lane^32)
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      m_run = m_new;
      const float mb = m_use * c2;
      float psum = 0.f;
      V8 pb[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][e], c2, -mb));
          psum += p;
          pb[mt * 2 + (e >> 3)][e & 7] = (T)p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
      // ---- O^T += V^T P^T ; step j covers keys mt*32 + hf*16 + {h*4+0..3, 8+h*4+0..3}
      const int grp = lane >> 4, L = lane & 15;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = (j >> 1) * 32 + (j & 1) * 16 + (grp >> 1) * 4 + (L >> 2);
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const int nb = d * 32 + (grp & 1) * 16 + 4 * (L & 3);
          const V4 lo = read_tr<V4>(&sV[buf][voff(kr, nb)]);
          const V4 hi = read_tr<V4>(&sV[buf][voff(kr + 8, nb)]);
          o[d] = mfma32(cat8(lo, hi), pb[j], o[d]);
        }
      }
    }
    vm_wait_all();
    __syncthreads();
  }

  // ---- normalise and store: lane holds query my_q, dv rows d*32 + qd*8 + h*4 + [0,4)
  if (my_q >= q1) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
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
  const int lo = max(0, cu[d]);
  const float* Q = (const float*)a.q + ((int64_t)t * H + h) * dqk;
  for (int d = lane; d < dqk; d += 64) sq[d] = Q[d];
  __syncthreads();
  const float* KV = (const float*)a.kv;
  const float* KPE = (const float*)a.kpe;
  const int kvw = a.nope + a.dv;
  float m = -INFINITY, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = lo; j <= t; ++j) {
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

hipError_t launch_flash_mfma(const FlashArgs& a, bool f16_operands, const int32_t* cu_host, int num_seqs, hipStream_t s) {
  // Tile plan: every (document, 128-query tile), longest key range first.
  struct T { int keys; uint32_t id; };
  std::vector<T> tiles;
  for (int d = 0; d < num_seqs; ++d) {
    const int len = cu_host[d + 1] - cu_host[d];
    const int nt = (len + FQ - 1) / FQ;
    for (int i = 0; i < nt; ++i) tiles.push_back({std::min((i + 1) * FQ, len), ((uint32_t)d << 16) | (uint32_t)i});
  }
  std::stable_sort(tiles.begin(), tiles.end(), [](const T& x, const T& y) { return x.keys > y.keys; });
  TilePlan plan;
  for (size_t base = 0; base < tiles.size(); base += MAX_TILES) {
    const int n = (int)std::min<size_t>(MAX_TILES, tiles.size() - base);
    plan.n = n;
    for (int i = 0; i < n; ++i) plan.t[i] = tiles[base + i].id;
    dim3 grid(a.heads, n);
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
