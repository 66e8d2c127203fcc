// Weight-absorbed MLA decode over the paged latent cache: split-KV attention in
// the 576-wide latent space and the log-sum-exp combine of the splits.
//
// Split kernel: one workgroup per (sequence, chunk of keys) computes, for every
// head at once, the partial softmax state of its keys.  Each wave owns 16
// heads (v_mfma_f32_16x16x32_bf16).  A tile of DK cached rows [c_n (512) |
// k_pe' (64)] is copied into LDS once per workgroup (asynchronous global->LDS
// loads, double buffered) and used twice:
//   S^T[key, head]  = C[key, :] . Qc[head, :]        (A = C rows, B = absorbed query)
//   O^T[dim, head] += C^T[dim, key] . P^T[key, head] (A = C^T by LDS transpose read)
// so each cached row is read from HBM exactly once per query group.  The
// absorbed query Qc = [W_UK^T q_nope | q_pe] stays in registers as the MFMA B
// operand for the whole chunk.  Partial outputs are unnormalised fp32 with the
// running max and sum per head.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int DK_TILE = 32;                // keys per tile
constexpr int RC = 576, RK = 512, DRP = 64;
constexpr int CCH = RC / 8;                // 16 B chunks per cached row (72)

// Cache tile [DK keys][576]: chunk c of row r at c ^ sw(r).  sw maps any 8
// consecutive rows to distinct values (row reads of the score MFMA) and any 4
// rows 4a..4a+3 to distinct 32 B pairs (transpose reads of the PV MFMA).
__device__ __forceinline__ int csw(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int cchunk(int r, int c) { return r * RC + ((c ^ csw(r)) << 3); }
__device__ __forceinline__ int celem(int r, int n) { return r * RC + ((((n >> 3) ^ csw(r))) << 3) + (n & 7); }



template <int NW, int DK>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_kernel(DecodeArgs a) {
  constexpr int NTH = NW * 64;
  constexpr int BLOCKS = DK * CCH / 64;            // 1 KB LDS blocks per tile
  constexpr int BPW = (BLOCKS + NW - 1) / NW;
  constexpr int MT = DK / 16;                       // 16-key score tiles
  static_assert(MT % 2 == 0 && BLOCKS * 64 == DK * CCH, "tile shape");
  static_assert(DK * RC * 2 <= 65536, "one tile must be addressable with immediate LDS offsets");
  __shared__ __attribute__((aligned(16))) bf16 sC[2][DK * RC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, b = blockIdx.y;
  const int H = a.heads;
  const int L = min(a.seq_lens[b], a.max_blocks * a.block_size);
  const int k0 = c * a.chunk;
  if (k0 >= L) return;
  const int k1 = min(k0 + a.chunk, L);
  const int nt = (k1 - k0 + DK - 1) / DK;
  const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;
  const int64_t part = ((int64_t)b * a.max_chunks + c) * H;

  // a block id outside the pool poisons this sequence's output
  int bad = 0;
  for (int i = k0 / a.block_size + tid; i <= (k1 - 1) / a.block_size; i += NTH) {
    const int blk = table[i];
    bad |= (blk < 0 || blk >= a.num_blocks);
  }
  if (__syncthreads_or(bad)) {
    for (int i = tid; i < H * RK; i += NTH) a.part_o[part * RK + i] = __builtin_nanf("");
    for (int i = tid; i < H; i += NTH) { a.part_ml[(part + i) * 2] = 0.f; a.part_ml[(part + i) * 2 + 1] = __builtin_nanf(""); }
    return;
  }

  const int g4 = lane >> 4, l16 = lane & 15;
  const int my_h = wave * 16 + l16;
  bf16x8 qreg[RC / 32];
  {
    const bf16* qt = a.qt + ((int64_t)b * H + my_h) * RK;
    const bf16* qp = a.q_pe + ((int64_t)b * H + my_h) * DRP;
#pragma unroll
    for (int ks = 0; ks < RC / 32; ++ks) {
      const int d = ks * 32 + g4 * 8;
      qreg[ks] = (d < RK) ? *(const bf16x8*)(qt + d) : *(const bf16x8*)(qp + d - RK);
    }
  }

  // Lane-constant parts of the swizzled LDS addresses (elements); the rest of
  // every address is a compile-time offset.
  //  score read (mt, ks): row mt*16 + l16, chunk ks*4 + g4
  const int swa = csw(l16 & 7);
  const int base_s0 = l16 * RC + (((0 * 4 + g4) ^ swa) << 3);
  const int base_s1 = l16 * RC + (((1 * 4 + g4) ^ swa) << 3);
  //  transpose read (half, d): row half*16 + g4*4 + l16/4, column d*16 + 4*(l16%4)
  const int rt = g4 * 4 + (l16 >> 2);
  const int swt = csw(rt & 7);
  const int xb = (l16 >> 1) & 1;
  int base_t[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) base_t[q] = rt * RC + ((((q * 2 + xb) ^ swt)) << 3) + 4 * (l16 & 1);

  auto issue_tile = [&](int t, int buf) {
    const int kb = k0 + t * DK;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + NW * i;
      if (blk < BLOCKS) {
        const int P = blk * 64 + lane;
        const int r = P / CCH, pc = P - r * CCH;
        const int cc = pc ^ csw(r);
        const int key = (kb + r < k1) ? kb + r : k0;       // clamped rows are masked out
        const int64_t row = (int64_t)table[key / a.block_size] * a.block_size + key % a.block_size;
        lds_dma16(a.cache + row * RC + cc * 8, &sC[buf][blk * 512]);
      }
    }
  };

  const float c2 = a.scale * kLog2e;
  // m_ref: the max used as the exponent origin.  It is raised (and the
  // accumulators rescaled) only when a tile's max exceeds it by more than 8 in
  // log2 units, so probabilities stay <= 2^8 and the rescale is rare.
  float m_ref = -INFINITY, l_run = 0.f;
  f32x4 o[RK / 16];
#pragma unroll
  for (int d = 0; d < RK / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_tile(0, 0);
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    const int kb = k0 + t * DK;
    if (t + 1 < nt) issue_tile(t + 1, buf ^ 1);
    const bf16* sb = sC[buf];
    f32x4 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < RC / 32; ++ks) {
        const int off = mt * 16 * RC + (ks >> 1) * 64;
        const bf16x8 cf = *(const bf16x8*)(sb + ((ks & 1) ? base_s1 : base_s0) + off);
        s[mt] = mfma16(cf, qreg[ks], s[mt]);
      }
    }
    // lane holds head my_h, keys mt*16 + g4*4 + e
    if (kb + DK > k1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kb + mt * 16 + g4 * 4 + e >= k1) s[mt][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[mt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool raise = (mx - m_ref) * c2 > 8.f;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < RK / 16; ++d) o[d] *= alpha;
      m_ref = m_new;
    }
    const float mb = m_ref * c2;
    bf16x8 pb[MT / 2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][e], c2, -mb));
        l_run += p;
        pb[mt >> 1][(mt & 1) * 4 + e] = (bf16)p;
      }
    // O^T += C^T P^T; step j covers keys {2j*16 + g*4 + [0,4), (2j+1)*16 + g*4 + [0,4)}
#pragma unroll
    for (int j = 0; j < MT / 2; ++j) {
#pragma unroll
      for (int d = 0; d < RK / 16; ++d) {
        const bf16* pt = sb + base_t[d & 3] + (2 * j) * 16 * RC + (d >> 2) * 64;
        const bf16x4 lo = lds_read_tr(pt);
        const bf16x4 hi = lds_read_tr(pt + 16 * RC);
        o[d] = mfma16(cat8(lo, hi), pb[j], o[d]);
      }
    }
    vm_wait_all();
    __syncthreads();
  }

  // lane holds head my_h, dims d*16 + g4*4 + [0,4)
  float* po = a.part_o + (part + my_h) * RK;
#pragma unroll
  for (int d = 0; d < RK / 16; ++d)
    *(float4*)(po + d * 16 + g4 * 4) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (g4 == 0) {
    a.part_ml[(part + my_h) * 2 + 0] = m_ref;
    a.part_ml[(part + my_h) * 2 + 1] = l_tot;
  }
}

// Combine: o_lat[b, h, :] = sum_c w_c o_c / sum_c w_c l_c with w_c = 2^((m_c - M) * c2).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.heads;
  const int L = min(a.seq_lens[b], a.max_blocks * a.block_size);
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
  dim3 grid(a.max_chunks, a.batch);
  switch (a.heads) {
    case 32: decode_split_kernel<2, DK_TILE><<<grid, 128, 0, s>>>(a); break;
    case 64: decode_split_kernel<4, DK_TILE><<<grid, 256, 0, s>>>(a); break;
    case 96: decode_split_kernel<6, DK_TILE><<<grid, 384, 0, s>>>(a); break;
    case 128: decode_split_kernel<8, DK_TILE><<<grid, 512, 0, s>>>(a); break;
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
