// libmla C ABI: argument checks, workspace carving, the RoPE / YaRN table
// builder, and the launch sequences of the prefill layer and the absorbed
// decode.  Host code; every device step runs in the kernels of this library.
#include "mla_internal.hpp"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>
#include <algorithm>
#include <mutex>

using namespace mla;

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(const mla_config* c) { return c->dtype == MLA_BF16 ? 2 : 4; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

mla_status check_config(const mla_config* c) {
  if (!c) return fail(MLA_ERR_INVALID_ARG, "config is NULL");
  if (c->hidden <= 0 || c->num_heads <= 0 || c->kv_lora_rank <= 0 || c->qk_nope_dim <= 0 ||
      c->v_head_dim <= 0 || c->qk_rope_dim < 0 || c->q_lora_rank < 0)
    return fail(MLA_ERR_INVALID_ARG, "dimensions must be positive (q_lora_rank, qk_rope_dim may be 0)");
  if (c->qk_rope_dim % 2) return fail(MLA_ERR_INVALID_ARG, "qk_rope_dim must be even");
  if (c->dtype != MLA_BF16 && c->dtype != MLA_F32) return fail(MLA_ERR_INVALID_ARG, "config dtype must be bf16 or fp32, got %d", c->dtype);
  if (c->rope_kind < MLA_ROPE_NONE || c->rope_kind > MLA_ROPE_YARN)
    return fail(MLA_ERR_INVALID_ARG, "unknown rope_kind %d", c->rope_kind);
  if (c->rope_kind != MLA_ROPE_NONE) {
    if (c->qk_rope_dim <= 0) return fail(MLA_ERR_INVALID_ARG, "rope needs qk_rope_dim > 0");
    if (!(c->rope_theta > 0.0)) return fail(MLA_ERR_INVALID_ARG, "rope_theta must be > 0");
  }
  if (c->rope_kind == MLA_ROPE_YARN) {
    if (!(c->yarn_factor > 0.0) || c->yarn_original_max_pos <= 0 || !(c->yarn_beta_fast > 0.0) ||
        !(c->yarn_beta_slow > 0.0) || !(c->yarn_beta_fast >= c->yarn_beta_slow))
      return fail(MLA_ERR_INVALID_ARG, "YaRN needs factor > 0, original_max_pos > 0, beta_fast >= beta_slow > 0");
  }
  if (!(c->norm_eps >= 0.f) || !std::isfinite(c->norm_eps)) return fail(MLA_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if (!std::isfinite(c->softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (c->output_gate != 0 && c->output_gate != 1) return fail(MLA_ERR_INVALID_ARG, "output_gate must be 0 or 1");
  if (c->rope_interleave != 0 && c->rope_interleave != 1) return fail(MLA_ERR_INVALID_ARG, "rope_interleave must be 0 or 1");
  if (c->o_groups < 0) return fail(MLA_ERR_INVALID_ARG, "o_groups must be >= 0");
  if (c->attn_operand != MLA_ATTN_F16 && c->attn_operand != MLA_ATTN_BF16)
    return fail(MLA_ERR_INVALID_ARG, "attn_operand must be MLA_ATTN_F16 or MLA_ATTN_BF16");
  if (c->dtype == MLA_F32 && c->attn_operand != 0)
    return fail(MLA_ERR_INVALID_ARG, "attn_operand must be 0 for an fp32 config");
  if (c->o_groups > 0) {
    if (c->o_lora_rank <= 0) return fail(MLA_ERR_INVALID_ARG, "o_groups > 0 needs o_lora_rank > 0");
    if (((int64_t)c->num_heads * c->v_head_dim) % c->o_groups)
      return fail(MLA_ERR_INVALID_ARG, "o_groups must divide num_heads * v_head_dim");
  }
  return MLA_OK;
}

// Shapes the compiled kernels cover.
mla_status check_supported(const mla_config* c) {
  if (c->dtype == MLA_BF16) {
    if (c->qk_nope_dim != 128 || c->qk_rope_dim != 64 || c->v_head_dim != 128 || c->kv_lora_rank != 512)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 kernels need d_nope=128, d_rope=64, d_v=128, r_kv=512");
    if (c->hidden % 8 || c->q_lora_rank % 8)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 kernels need hidden and q_lora_rank multiples of 8");
    if (c->o_groups > 0 && ((c->num_heads * c->v_head_dim / c->o_groups) % 8 || c->o_lora_rank % 8))
      return fail(MLA_ERR_UNSUPPORTED, "bf16 kernels need the output group width and o_lora_rank multiples of 8");
  } else {
    if (c->qk_nope_dim + c->qk_rope_dim > 512 || c->v_head_dim > 256 || c->qk_rope_dim > 128 || c->kv_lora_rank > 1024)
      return fail(MLA_ERR_UNSUPPORTED, "fp32 kernels need d_nope+d_rope <= 512, d_v <= 256, d_rope <= 128, r_kv <= 1024");
  }
  return MLA_OK;
}

double yarn_mscale(double s, double m) { return s <= 1.0 ? 1.0 : 0.1 * m * std::log(s) + 1.0; }

double derived_scale(const mla_config* c) {
  double s = std::pow((double)(c->qk_nope_dim + c->qk_rope_dim), -0.5);
  if (c->rope_kind == MLA_ROPE_YARN && c->yarn_mscale_all_dim != 0.0) {
    const double m = yarn_mscale(c->yarn_factor, c->yarn_mscale_all_dim);
    s = s * m * m;
  }
  return s;
}

float scale_of(const mla_config* c) { return c->softmax_scale > 0.f ? c->softmax_scale : (float)derived_scale(c); }

// Rotation frequency of each pair; YaRN blends theta_i and theta_i / s over the
// pair index between the pairs that turn beta_fast and beta_slow times over the
// original context.
std::vector<double> rope_frequencies(const mla_config* c) {
  const int d = c->qk_rope_dim, half = d / 2;
  std::vector<double> f(half);
  for (int i = 0; i < half; ++i) f[i] = std::pow(c->rope_theta, -2.0 * (double)i / (double)d);
  if (c->rope_kind != MLA_ROPE_YARN) return f;
  const double L = (double)c->yarn_original_max_pos, base = c->rope_theta, s = c->yarn_factor;
  auto turns_to_index = [&](double turns) {
    return (double)d * std::log(L / (turns * 2.0 * M_PI)) / (2.0 * std::log(base));
  };
  double lo = std::max(std::floor(turns_to_index(c->yarn_beta_fast)), 0.0);
  double hi = std::min(std::ceil(turns_to_index(c->yarn_beta_slow)), (double)(d - 1));
  if (lo == hi) hi += 0.001;
  for (int i = 0; i < half; ++i) {
    double r = ((double)i - lo) / (hi - lo);
    r = std::min(std::max(r, 0.0), 1.0);
    f[i] = f[i] * (1.0 - r) + (f[i] / s) * r;
  }
  return f;
}

// ---------------------------------------------------------------- prefill workspace
struct PrefillWs {
  size_t pos, q_lat32, q_lat, q, ckv32, latent, kpe16, kv, attn, ot, ctx, kpe16ctx, cuk, total;
};

// n new tokens; n_ctx >= 0 for a chunk over a cached prefix (context rows of
// all sequences, num_seqs sequences), else -1.
PrefillWs prefill_layout(const mla_config* c, int64_t n, int64_t n_ctx = -1, int64_t num_seqs = 0) {
  const size_t es = elem_size(c);
  const int64_t H = c->num_heads, dqk = c->qk_nope_dim + c->qk_rope_dim;
  const int64_t lw = c->kv_lora_rank + c->qk_rope_dim;
  PrefillWs w;
  size_t off = 0;
  w.pos = off; off += align256(n * 4);
  w.q_lat32 = off; off += align256(n * c->q_lora_rank * 4);   // fp32 down-projection before the norm
  w.q_lat = off; off += align256(n * c->q_lora_rank * es);
  w.q = off; off += align256(n * H * dqk * es);
  w.ckv32 = off; off += align256(2 * n * lw * 4);              // fp32 [c | k_pe] before norm / RoPE, two split-K partials
  w.latent = off; off += align256(n * lw * es);
  w.kpe16 = off; off += align256(n * c->qk_rope_dim * 2);      // fp16 shared rope key for attention
  const int64_t kv_rows = n_ctx >= 0 ? n_ctx : n;
  w.kv = off; off += align256(kv_rows * H * (c->qk_nope_dim + c->v_head_dim) * es);
  w.attn = off; off += align256(n * H * c->v_head_dim * es);
  w.ot = off;
  if (c->o_groups > 0) off += align256(n * (int64_t)c->o_groups * c->o_lora_rank * es);   // grouped low-rank o-proj
  w.ctx = w.kpe16ctx = w.cuk = off;
  if (n_ctx >= 0) {
    w.ctx = off; off += align256(n_ctx * lw * es);                     // context latent rows
    w.kpe16ctx = off; off += align256(n_ctx * c->qk_rope_dim * 2);     // their fp16 rope keys
    w.cuk = off; off += align256((num_seqs + 1) * 4);                  // context row offsets
  }
  w.total = off;
  return w;
}

mla_status check_cu(const int32_t* cu_host, int num_seqs, int* n_out) {
  if (!cu_host) return fail(MLA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if (num_seqs <= 0) return fail(MLA_ERR_INVALID_ARG, "num_seqs must be > 0");
  if (cu_host[0] != 0) return fail(MLA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int i = 0; i < num_seqs; ++i)
    if (cu_host[i + 1] < cu_host[i]) return fail(MLA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
  if (num_seqs >= 65536) return fail(MLA_ERR_UNSUPPORTED, "at most 65535 documents per call");
  for (int i = 0; i < num_seqs; ++i)
    if (cu_host[i + 1] - cu_host[i] >= 65536 * 128) return fail(MLA_ERR_UNSUPPORTED, "documents are limited to 8388607 tokens");
  *n_out = cu_host[num_seqs];
  return MLA_OK;
}

// ---------------------------------------------------------------- decode plan
constexpr int kDecodeTargetGroups = 256;   // one workgroup per CU

struct DecodePlan {
  int quota, groups, max_slots;
  size_t qt, part_o, part_ml, total;
};

// The keys of all sequences, one after another, each sequence preceded by
// kDecodeSegmentCost placeholder keys, are dealt to workgroups in runs of
// `quota` keys (a multiple of the split kernel's tile, 32 keys for the bf16
// cache and 64 for the E4M3 cache; the cuts inside a sequence move to the
// nearest tile boundary, so a workgroup's keys, quota + one tile at most, span
// no more blocks of the smallest allowed size, 16, than it can stage).  The
// placeholders charge the workgroup that starts a sequence for the fixed cost
// of one more segment
// (staging, query load, pipeline fill, partial stores), so workgroups that
// span a sequence end take fewer keys.  Sequence b, whose first key sits at
// r_b in that order, collects partials in slots 0 .. (r_b + L_b - 1) / quota -
// r_b / quota.
DecodePlan decode_plan(const mla_config* c, const int32_t* lens, int batch, int64_t key_cap, int tile = 32) {
  DecodePlan p{};
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t L = std::min<int64_t>(std::max(lens[b], 0), key_cap);
    if (L > 0) total += L + kDecodeSegmentCost;
  }
  const int kTile = tile, kMaxQuota = ((kDecodeMaxChunkBlocks - 2) * 16 - kTile) / kTile * kTile;
  int64_t quota = kTile * std::max<int64_t>(1, (total + (int64_t)kTile * kDecodeTargetGroups - 1) /
                                                   ((int64_t)kTile * kDecodeTargetGroups));
  quota = std::min<int64_t>(quota, kMaxQuota);
  p.quota = (int)quota;
  p.groups = (int)((total + quota - 1) / quota);
  int64_t st = 0, max_slots = 1;
  for (int b = 0; b < batch; ++b) {
    const int64_t L = std::min<int64_t>(std::max(lens[b], 0), key_cap);
    if (L == 0) continue;
    const int64_t r0 = st + kDecodeSegmentCost;
    max_slots = std::max<int64_t>(max_slots, (r0 + L - 1) / quota - r0 / quota + 1);
    st = r0 + L;
  }
  p.max_slots = (int)max_slots;
  const int64_t H = c->num_heads, R = c->kv_lora_rank;
  size_t off = 0;
  p.qt = off; off += align256((size_t)batch * H * R * 2);
  // one partial entry per (workgroup, sequence) segment, at index g + b
  const size_t parts = (size_t)p.groups + (size_t)batch;
  p.part_o = off; off += align256(parts * H * R * 2);
  p.part_ml = off; off += align256(parts * H * 2 * 4);
  p.total = off;
  return p;
}

}  // namespace

// ---------------------------------------------------------------- static scratch
// Device memory of mla_decode_absorbed_fwd_noalloc, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of the array for
// the life of the process.  In host code the array's name stands for the
// host-side shadow, not a device address: the device address is obtained once
// per device with hipGetSymbolAddress (with that device current) and only that
// address is passed to kernels.
static constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device `stream` belongs to (the
// current device for the null stream).
mla_status static_scratch(hipStream_t stream, char** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "current device");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "select the stream's device");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
    if (!p) return fail(MLA_ERR_HIP, "address of the static scratch is NULL");
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

// ============================================================================ C ABI
extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_validate_config(const mla_config* cfg) {
  const mla_status s = check_config(cfg);
  return s == MLA_OK ? ok() : s;
}

float mla_softmax_scale(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0.f;
  return scale_of(cfg);
}

mla_status mla_rope_table(const mla_config* cfg, int32_t max_pos, float* cos_out, float* sin_out) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->rope_kind == MLA_ROPE_NONE) return fail(MLA_ERR_INVALID_ARG, "rope_kind NONE has no table");
  if (max_pos <= 0 || !cos_out || !sin_out) return fail(MLA_ERR_INVALID_ARG, "max_pos > 0 and host outputs required");
  const std::vector<double> f = rope_frequencies(cfg);
  double amp = 1.0;
  if (cfg->rope_kind == MLA_ROPE_YARN)
    amp = yarn_mscale(cfg->yarn_factor, cfg->yarn_mscale) / yarn_mscale(cfg->yarn_factor, cfg->yarn_mscale_all_dim);
  const int half = cfg->qk_rope_dim / 2;
  for (int64_t p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * f[i];
      cos_out[p * half + i] = (float)(std::cos(ang) * amp);
      sin_out[p * half + i] = (float)(std::sin(ang) * amp);
    }
  return ok();
}

size_t mla_prefill_workspace_size(const mla_config* cfg, int32_t num_tokens, int32_t num_seqs) {
  (void)num_seqs;
  if (check_config(cfg) != MLA_OK || num_tokens < 0) return 0;
  return prefill_layout(cfg, num_tokens).total;
}

size_t mla_prefill_chunk_workspace_size(const mla_config* cfg, const int32_t* cu_seqlens_host,
                                        const int32_t* prefix_lens_host, int32_t num_seqs) {
  if (check_config(cfg) != MLA_OK || !cu_seqlens_host || !prefix_lens_host || num_seqs <= 0) return 0;
  int64_t n_ctx = 0;
  for (int i = 0; i < num_seqs; ++i)
    n_ctx += std::max(0, prefix_lens_host[i]) + std::max(0, cu_seqlens_host[i + 1] - cu_seqlens_host[i]);
  return prefill_layout(cfg, cu_seqlens_host[num_seqs], n_ctx, num_seqs).total;
}

size_t mla_decode_workspace_size(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch) {
  if (check_config(cfg) != MLA_OK || !seq_lens_host || batch <= 0) return 0;
  return decode_plan(cfg, seq_lens_host, batch, INT32_MAX).total;
}

size_t mla_decode_fp8_workspace_size(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch) {
  if (check_config(cfg) != MLA_OK || !seq_lens_host || batch <= 0) return 0;
  return decode_plan(cfg, seq_lens_host, batch, INT32_MAX, 64).total;
}

mla_status mla_latent_norm_rope(const mla_config* cfg, const void* src, int64_t src_row_stride, int32_t n_rows,
                                int32_t row_width, int32_t norm_dim, const void* gamma, int32_t rope_offset,
                                int32_t rope_slices, int32_t rope_slice_stride, const float* rope_cos,
                                const float* rope_sin, int32_t rope_table_len, const int32_t* positions, void* dst,
                                int64_t dst_row_stride, const int32_t* slot_mapping, int64_t num_slots,
                                void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (n_rows < 0 || row_width < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows and row_width must be >= 0");
  if (n_rows == 0) return ok();
  if (!src || !dst) return fail(MLA_ERR_INVALID_ARG, "src and dst are required");
  if (src_row_stride < row_width || (!slot_mapping && dst_row_stride < row_width) || dst_row_stride < row_width)
    return fail(MLA_ERR_INVALID_ARG, "row strides must be >= row_width");
  if (norm_dim < 0 || norm_dim > row_width) return fail(MLA_ERR_INVALID_ARG, "norm_dim must be in [0, row_width]");
  if (norm_dim > 0 && !gamma) return fail(MLA_ERR_INVALID_ARG, "gamma is required when norm_dim > 0");
  const bool rope = rope_slices > 0 && cfg->rope_kind != MLA_ROPE_NONE;
  if (rope_slices < 0) return fail(MLA_ERR_INVALID_ARG, "rope_slices must be >= 0");
  if (rope) {
    const int d = cfg->qk_rope_dim;
    if (!rope_cos || !rope_sin || !positions || rope_table_len <= 0)
      return fail(MLA_ERR_INVALID_ARG, "RoPE needs device cos/sin tables, their length and positions");
    if (rope_offset < norm_dim) return fail(MLA_ERR_INVALID_ARG, "rope slices must not overlap the normalised columns");
    if (rope_slices > 1 && rope_slice_stride < d) return fail(MLA_ERR_INVALID_ARG, "rope_slice_stride must be >= d_rope");
    const int64_t last = (int64_t)rope_offset + (int64_t)(rope_slices - 1) * std::max(rope_slice_stride, d) + d;
    if (last > row_width) return fail(MLA_ERR_INVALID_ARG, "rope slices exceed row_width");
  }
  if (slot_mapping && num_slots <= 0) return fail(MLA_ERR_INVALID_ARG, "num_slots must be > 0 with a slot mapping");
  if (slot_mapping && src == dst) return fail(MLA_ERR_INVALID_ARG, "in-place update cannot use a slot mapping");
  NormRopeArgs a{};
  a.src = src; a.src_stride = src_row_stride; a.n_rows = n_rows; a.row_width = row_width;
  a.norm_dim = norm_dim; a.gamma = gamma; a.eps = cfg->norm_eps; a.interleave = cfg->rope_interleave;
  a.rope_offset = rope_offset; a.rope_slices = rope ? rope_slices : 0;
  a.rope_stride = std::max(rope_slice_stride, cfg->qk_rope_dim); a.rope_dim = cfg->qk_rope_dim;
  a.cos_t = rope_cos; a.sin_t = rope_sin; a.table_len = rope_table_len; a.positions = positions;
  a.dst = dst; a.dst_stride = dst_row_stride; a.slots = slot_mapping; a.num_slots = num_slots;
  const hipError_t e = launch_norm_rope(a, cfg->dtype == MLA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "latent_norm_rope launch");
  return ok();
}

static mla_status linear_impl(const mla_config* cfg, const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                              int m, int n, int k, const void* gate_src, int64_t ldg, hipStream_t st) {
  GemmArgs g{};
  g.a = x; g.lda = ldx; g.b = w; g.ldb = k; g.c = y; g.ldc = ldy;
  g.gate_src = gate_src; g.ldg = ldg; g.m = m; g.n = n; g.k = k; g.batch = 1;
  g.b_kn = false; g.epilogue = gate_src ? EPI_GATE : EPI_STORE;
  const hipError_t e = cfg->dtype == MLA_BF16 ? launch_gemm_bf16(g, st) : launch_gemm_f32(g, st);
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return MLA_OK;
}

mla_status mla_linear(const mla_config* cfg, const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                      int32_t m, int32_t n, int32_t k, void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (m < 0 || n <= 0 || k <= 0) return fail(MLA_ERR_INVALID_ARG, "linear needs m >= 0, n > 0, k > 0");
  if (m == 0) return ok();
  if (!x || !w || !y) return fail(MLA_ERR_INVALID_ARG, "x, w and y are required");
  if (ldx < k || ldy < n) return fail(MLA_ERR_INVALID_ARG, "ldx >= k and ldy >= n required");
  if (cfg->dtype == MLA_BF16) {
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || ldx % 8 || ldy % 8 || k % 8 || n % 8)
      return fail(MLA_ERR_MISALIGNED, "bf16 linear needs 16-byte aligned pointers and k, n, ldx, ldy multiples of 8");
  }
  s = linear_impl(cfg, x, ldx, w, y, ldy, m, n, k, nullptr, 0, (hipStream_t)stream);
  return s == MLA_OK ? ok() : s;
}

// Attention core.  cuk_dev / cuk_host (both or neither): key rows per document
// when they differ from the query rows (a chunk over a cached prefix), n_keys
// the rows of kv and kpe.
static mla_status attention_impl(const mla_config* cfg, const void* q, const void* kv, const void* kpe,
                                 int64_t kpe_stride, bool f16_operands, const int32_t* cu_dev,
                                 const int32_t* cu_host, int num_seqs, int n, void* attn, hipStream_t st,
                                 const int32_t* cuk_dev = nullptr, const int32_t* cuk_host = nullptr,
                                 int n_keys = -1, float* lse_out = nullptr) {
  // the MFMA kernel addresses the 64 key rows of a tile with 32-bit byte offsets
  if (cfg->dtype == MLA_BF16 &&
      (64 * kpe_stride * 2 >= ((int64_t)1 << 31) ||
       64 * (int64_t)cfg->num_heads * (cfg->qk_nope_dim + cfg->v_head_dim) * 2 >= ((int64_t)1 << 31)))
    return fail(MLA_ERR_UNSUPPORTED, "64 rows of kv or kpe must span less than 2 GiB");
  FlashArgs f{};
  f.q = q; f.kv = kv; f.kpe = kpe; f.kpe_stride = kpe_stride; f.cu_dev = cu_dev; f.out = attn;
  f.n_tokens = n; f.heads = cfg->num_heads; f.nope = cfg->qk_nope_dim; f.rope = cfg->qk_rope_dim;
  f.dv = cfg->v_head_dim; f.kv_lora = cfg->kv_lora_rank; f.scale = scale_of(cfg); f.num_seqs = num_seqs;
  f.cuk_dev = cuk_dev; f.n_keys = cuk_dev ? n_keys : n; f.lse_out = lse_out;
  const hipError_t e = cfg->dtype == MLA_BF16 ? launch_flash_mfma(f, f16_operands, cu_host, cuk_host, num_seqs, st)
                                              : launch_flash_f32(f, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MLA_OK;
}

mla_status mla_attention_prefill(const mla_config* cfg, int32_t operand_dtype, const void* q, const void* kv,
                                 const void* kpe, int64_t kpe_stride, const int32_t* cu_seqlens_dev,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs, void* attn, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  const bool ok_type = cfg->dtype == MLA_BF16 ? (operand_dtype == MLA_BF16 || operand_dtype == MLA_F16)
                                              : operand_dtype == MLA_F32;
  if (!ok_type) return fail(MLA_ERR_INVALID_ARG, "operand_dtype %d does not match the config dtype", operand_dtype);
  int n = 0;
  if ((s = check_cu(cu_seqlens_host, num_seqs, &n)) != MLA_OK) return s;
  if (n == 0) return ok();
  if (!q || !kv || !kpe || !cu_seqlens_dev || !attn) return fail(MLA_ERR_INVALID_ARG, "q, kv, kpe, cu_seqlens_dev and attn are required");
  if (kpe_stride < cfg->qk_rope_dim) return fail(MLA_ERR_INVALID_ARG, "kpe_stride < d_rope");
  if (cfg->dtype == MLA_BF16 && (!aligned16(q) || !aligned16(kv) || !aligned16(kpe) || !aligned16(attn) || kpe_stride % 8))
    return fail(MLA_ERR_MISALIGNED, "bf16 attention needs 16-byte aligned tensors and kpe_stride % 8 == 0");
  if (lse && cfg->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the log-sum-exp output needs a bf16 config");
  if (lse && ((uintptr_t)lse & 3)) return fail(MLA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  s = attention_impl(cfg, q, kv, kpe, kpe_stride, operand_dtype == MLA_F16, cu_seqlens_dev, cu_seqlens_host,
                     num_seqs, n, attn, (hipStream_t)stream, nullptr, nullptr, -1, lse);
  return s == MLA_OK ? ok() : s;
}

// A chunk of new tokens over a cached prefix (see mla_prefill_chunk_fwd).
struct ChunkIn {
  const int32_t* prefix_dev;
  const void* cache; int num_blocks; int log2_block; const int32_t* block_table; int max_blocks;
  int n_ctx; int max_ctx_len;
  std::vector<int32_t> cuk_host;                     // context row offsets, for the attention plan
};

static mla_status check_weights(const mla_config* cfg, const mla_weights* w) {
  if (!w) return fail(MLA_ERR_INVALID_ARG, "weights are NULL");
  if (cfg->q_lora_rank > 0 && (!w->w_q_a || !w->q_a_gamma || !w->w_q_b))
    return fail(MLA_ERR_INVALID_ARG, "q_lora_rank > 0 needs w_q_a, q_a_gamma, w_q_b");
  if (cfg->q_lora_rank == 0 && !w->w_q) return fail(MLA_ERR_INVALID_ARG, "q_lora_rank == 0 needs w_q");
  if (!w->w_kv_a || !w->kv_a_gamma || !w->w_kv_b) return fail(MLA_ERR_INVALID_ARG, "w_kv_a, kv_a_gamma, w_kv_b are required");
  if (cfg->o_groups == 0 && !w->w_o) return fail(MLA_ERR_INVALID_ARG, "w_o is required");
  if (cfg->o_groups > 0 && (!w->w_o_a || !w->w_o_b)) return fail(MLA_ERR_INVALID_ARG, "o_groups > 0 needs w_o_a and w_o_b");
  if (cfg->output_gate && !w->w_g) return fail(MLA_ERR_INVALID_ARG, "output_gate needs w_g");
  if (cfg->dtype == MLA_BF16 && ((w->w_o_a && !aligned16(w->w_o_a)) || (w->w_o_b && !aligned16(w->w_o_b))))
    return fail(MLA_ERR_MISALIGNED, "bf16 weights must be 16-byte aligned");
  return MLA_OK;
}

static mla_status prefill_core(const mla_config* cfg, const mla_weights* w, const void* x, const int32_t* cu_seqlens_dev,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int n, const int32_t* positions_dev,
                               const float* rope_cos, const float* rope_sin, int32_t rope_table_len, void* out,
                               void* latent_out, void* workspace, size_t workspace_bytes, void* stream,
                               const ChunkIn* chunk);

mla_status mla_attention_prefix(const mla_config* cfg, int32_t operand_dtype, const void* q, const void* kv,
                                const void* kpe, int64_t kpe_stride, const int32_t* cu_q_dev, const int32_t* cu_q_host,
                                const int32_t* cu_k_dev, const int32_t* cu_k_host, int32_t num_seqs, void* attn,
                                void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  const bool ok_type = cfg->dtype == MLA_BF16 ? (operand_dtype == MLA_BF16 || operand_dtype == MLA_F16)
                                              : operand_dtype == MLA_F32;
  if (!ok_type) return fail(MLA_ERR_INVALID_ARG, "operand_dtype %d does not match the config dtype", operand_dtype);
  int n = 0, nk = 0;
  if ((s = check_cu(cu_q_host, num_seqs, &n)) != MLA_OK) return s;
  if (!cu_k_host) return fail(MLA_ERR_INVALID_ARG, "cu_k_host is NULL");
  if (cu_k_host[0] != 0) return fail(MLA_ERR_INVALID_ARG, "cu_k[0] must be 0");
  for (int i = 0; i < num_seqs; ++i)
    if (cu_k_host[i + 1] - cu_k_host[i] < cu_q_host[i + 1] - cu_q_host[i])
      return fail(MLA_ERR_INVALID_ARG, "document %d has fewer keys than queries", i);
  nk = cu_k_host[num_seqs];
  if (n == 0) return ok();
  if (!q || !kv || !kpe || !cu_q_dev || !cu_k_dev || !attn)
    return fail(MLA_ERR_INVALID_ARG, "q, kv, kpe, both device offset arrays and attn are required");
  if (kpe_stride < cfg->qk_rope_dim) return fail(MLA_ERR_INVALID_ARG, "kpe_stride < d_rope");
  if (cfg->dtype == MLA_BF16 && (!aligned16(q) || !aligned16(kv) || !aligned16(kpe) || !aligned16(attn) || kpe_stride % 8))
    return fail(MLA_ERR_MISALIGNED, "bf16 attention needs 16-byte aligned tensors and kpe_stride % 8 == 0");
  s = attention_impl(cfg, q, kv, kpe, kpe_stride, operand_dtype == MLA_F16, cu_q_dev, cu_q_host, num_seqs, n, attn,
                     (hipStream_t)stream, cu_k_dev, cu_k_host, nk);
  return s == MLA_OK ? ok() : s;
}

mla_status mla_prefill_fwd(const mla_config* cfg, const mla_weights* w, const void* x, const int32_t* cu_seqlens_dev,
                           const int32_t* cu_seqlens_host, int32_t num_seqs, const int32_t* positions_dev,
                           const float* rope_cos, const float* rope_sin, int32_t rope_table_len, void* out,
                           void* latent_out, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  if ((s = check_weights(cfg, w)) != MLA_OK) return s;
  int n = 0;
  if ((s = check_cu(cu_seqlens_host, num_seqs, &n)) != MLA_OK) return s;
  if (n == 0) return ok();
  if (!x || !out || !cu_seqlens_dev) return fail(MLA_ERR_INVALID_ARG, "x, out and cu_seqlens_dev are required");
  s = prefill_core(cfg, w, x, cu_seqlens_dev, cu_seqlens_host, num_seqs, n, positions_dev, rope_cos, rope_sin,
                   rope_table_len, out, latent_out, workspace, workspace_bytes, stream, nullptr);
  return s == MLA_OK ? ok() : s;
}

mla_status mla_prefill_chunk_fwd(const mla_config* cfg, const mla_weights* w, const void* x,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 const int32_t* prefix_lens_dev, const int32_t* prefix_lens_host,
                                 const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                 const int32_t* block_table, int32_t max_blocks, const float* rope_cos,
                                 const float* rope_sin, int32_t rope_table_len, void* out, void* latent_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  if ((s = check_weights(cfg, w)) != MLA_OK) return s;
  int n = 0;
  if ((s = check_cu(cu_seqlens_host, num_seqs, &n)) != MLA_OK) return s;
  if (n == 0) return ok();
  if (!x || !out || !cu_seqlens_dev || !prefix_lens_dev || !prefix_lens_host)
    return fail(MLA_ERR_INVALID_ARG, "x, out, cu_seqlens_dev and both prefix_lens arrays are required");
  ChunkIn c{};
  c.prefix_dev = prefix_lens_dev;
  c.cuk_host.assign(num_seqs + 1, 0);
  int64_t n_ctx = 0, max_prefix = 0;
  int max_len = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int64_t P = prefix_lens_host[i];
    if (P < 0) return fail(MLA_ERR_INVALID_ARG, "prefix_lens[%d] = %lld < 0", i, (long long)P);
    const int64_t len = P + cu_seqlens_host[i + 1] - cu_seqlens_host[i];
    n_ctx += len;
    if (n_ctx >= INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 context rows");
    c.cuk_host[i + 1] = (int32_t)n_ctx;
    max_prefix = std::max(max_prefix, P);
    max_len = std::max<int>(max_len, (int)len);
  }
  c.n_ctx = (int)n_ctx;
  c.max_ctx_len = max_len;
  if (max_prefix > 0) {
    if (!kv_cache || !block_table) return fail(MLA_ERR_INVALID_ARG, "a cached prefix needs kv_cache and block_table");
    if (num_blocks <= 0 || max_blocks <= 0) return fail(MLA_ERR_INVALID_ARG, "num_blocks and max_blocks must be > 0");
    if (block_size <= 0 || (block_size & (block_size - 1))) return fail(MLA_ERR_INVALID_ARG, "block_size must be a power of two");
    if (max_prefix > (int64_t)max_blocks * block_size)
      return fail(MLA_ERR_INVALID_ARG, "a prefix is longer than max_blocks * block_size");
    if (cfg->dtype == MLA_BF16 && !aligned16(kv_cache)) return fail(MLA_ERR_MISALIGNED, "kv_cache must be 16-byte aligned");
    if (cfg->dtype == MLA_F32 && ((uintptr_t)kv_cache & 15)) return fail(MLA_ERR_MISALIGNED, "kv_cache must be 16-byte aligned");
  }
  const int lw = cfg->kv_lora_rank + cfg->qk_rope_dim;
  if ((lw * (int)elem_size(cfg)) % 16) return fail(MLA_ERR_UNSUPPORTED, "latent rows must be a multiple of 16 bytes");
  c.cache = kv_cache; c.num_blocks = num_blocks; c.block_table = block_table; c.max_blocks = max_blocks;
  c.log2_block = 0;
  while (max_prefix > 0 && (1 << c.log2_block) < block_size) ++c.log2_block;
  s = prefill_core(cfg, w, x, cu_seqlens_dev, cu_seqlens_host, num_seqs, n, nullptr, rope_cos, rope_sin,
                   rope_table_len, out, latent_out, workspace, workspace_bytes, stream, &c);
  return s == MLA_OK ? ok() : s;
}

static mla_status prefill_core(const mla_config* cfg, const mla_weights* w, const void* x, const int32_t* cu_seqlens_dev,
                               const int32_t* cu_seqlens_host, int32_t num_seqs, int n, const int32_t* positions_dev,
                               const float* rope_cos, const float* rope_sin, int32_t rope_table_len, void* out,
                               void* latent_out, void* workspace, size_t workspace_bytes, void* stream,
                               const ChunkIn* chunk) {
  mla_status s = MLA_OK;
  const bool rope = cfg->rope_kind != MLA_ROPE_NONE;
  if (rope && (!rope_cos || !rope_sin || rope_table_len <= 0))
    return fail(MLA_ERR_INVALID_ARG, "RoPE needs device cos/sin tables and their length");
  const PrefillWs L = chunk ? prefill_layout(cfg, n, chunk->n_ctx, num_seqs) : prefill_layout(cfg, n);
  if (!workspace || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  if (cfg->dtype == MLA_BF16) {
    const void* ptrs[] = {x, out, w->w_kv_a, w->kv_a_gamma, w->w_kv_b, w->w_o, workspace};
    for (const void* p : ptrs)
      if (!aligned16(p)) return fail(MLA_ERR_MISALIGNED, "bf16 prefill needs 16-byte aligned tensors");
    if ((latent_out && !aligned16(latent_out)) || (w->w_q && !aligned16(w->w_q)) || (w->w_q_a && !aligned16(w->w_q_a)) ||
        (w->w_q_b && !aligned16(w->w_q_b)) || (w->w_g && !aligned16(w->w_g)))
      return fail(MLA_ERR_MISALIGNED, "bf16 prefill needs 16-byte aligned tensors");
  }
  const hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int H = cfg->num_heads, hid = cfg->hidden, rq = cfg->q_lora_rank, rkv = cfg->kv_lora_rank;
  const int dn = cfg->qk_nope_dim, dr = cfg->qk_rope_dim, dv = cfg->v_head_dim, dqk = dn + dr, lw = rkv + dr;
  int32_t* pos = (int32_t*)(ws + L.pos);
  float* q_lat32 = (float*)(ws + L.q_lat32);
  void* q_lat = ws + L.q_lat;
  void* q = ws + L.q;
  float* ckv32 = (float*)(ws + L.ckv32);
  void* lat = latent_out ? latent_out : (void*)(ws + L.latent);
  void* kv = ws + L.kv;
  void* attn = ws + L.attn;
  const bool bf = cfg->dtype == MLA_BF16;
  hipError_t e;

  // positions (0..len-1 per document, after the cached prefix of a chunk)
  // unless the caller gives them
  const int32_t* positions = positions_dev;
  if (rope && !positions) {
    if ((e = launch_positions(cu_seqlens_dev, num_seqs, n, pos, st, chunk ? chunk->prefix_dev : nullptr)) != hipSuccess)
      return hip_fail(e, "positions");
    positions = pos;
  }
  // Down-projections are kept in fp32 until their norm, so every stored bf16
  // tensor is rounded once.
  // Output storage of each GEMM: OUT_ACT (the layer dtype), OUT_F32 (kept for a
  // following norm), OUT_F16 (attention operands of the bf16 layer).
  enum { OUT_ACT, OUT_F32, OUT_F16 };
  // split > 1: the K range in `split` equal slices, one batch entry each,
  // partial products at c + s * m * ldc (summed by the following norm)
  auto gemm = [&](const void* a, int64_t lda, const void* b, void* c, int64_t ldc, int m, int nn, int k,
                  int out_kind, int epi, const void* gate, int split = 1) -> mla_status {
    GemmArgs g{};
    g.a = a; g.lda = lda; g.b = b; g.ldb = k; g.c = c; g.ldc = ldc; g.m = m; g.n = nn; g.k = k / split;
    g.batch = split;
    if (split > 1) {
      g.a_bstride = k / split; g.b_bstride = k / split; g.c_bstride = (int64_t)m * ldc;
    }
    g.c_f32 = out_kind == OUT_F32 && bf; g.c_f16 = out_kind == OUT_F16 && bf;
    g.epilogue = epi; g.gate_src = gate; g.ldg = ldc;
    g.cos_t = rope_cos; g.sin_t = rope_sin; g.table_len = rope_table_len; g.positions = positions;
    g.rope_head_stride = dqk; g.rope_off = dn; g.rope_interleave = cfg->rope_interleave;
    const hipError_t err = bf ? launch_gemm_bf16(g, st) : launch_gemm_f32(g, st);
    if (err != hipSuccess) return hip_fail(err, "linear launch");
    return MLA_OK;
  };
  auto norm = [&](const void* src, int64_t stride, int width, int norm_dim, const void* gamma, int rope_off,
                  int rope_slices, int rope_stride, void* dst, int64_t dst_stride, bool src_f32,
                  f16* aux = nullptr, int64_t src2_off = 0) -> mla_status {
    NormRopeArgs a{};
    a.src2_off = src2_off;
    a.rope_aux = aux; a.rope_aux_stride = dr; a.interleave = cfg->rope_interleave;
    a.src = src; a.src_stride = stride; a.n_rows = n; a.row_width = width; a.norm_dim = norm_dim; a.gamma = gamma;
    a.eps = cfg->norm_eps; a.rope_offset = rope_off; a.rope_slices = rope_slices; a.rope_stride = rope_stride;
    a.rope_dim = dr; a.cos_t = rope_cos; a.sin_t = rope_sin; a.table_len = rope_table_len; a.positions = positions;
    a.dst = dst; a.dst_stride = dst_stride;
    const hipError_t err = launch_norm_rope(a, bf, st, src_f32 && bf);
    if (err != hipSuccess) return hip_fail(err, "latent norm / rope launch");
    return MLA_OK;
  };
  // bf16: RoPE on q is fused into the q GEMM epilogue; fp32: applied in place after it.
  // In the bf16 layer the attention operands q, kv and the shared k_pe are
  // rounded once from fp32 to the type cfg->attn_operand selects: fp16 (k_pe
  // gets an fp16 copy of its own; values beyond the fp16 range saturate) or
  // bf16 (k_pe is read from the latent rows).
  const bool f16op = bf && cfg->attn_operand == MLA_ATTN_F16;
  const int q_epi = (rope && bf) ? EPI_ROPE : EPI_STORE;
  const int att_kind = f16op ? OUT_F16 : OUT_ACT;
  f16* kpe16 = (f16*)(ws + L.kpe16);
  // The joint down-projection (N = r_kv + d_rope = 576: 160 output tiles of
  // 128 x 128 over K = hidden, a third of the CUs idle) runs as two K halves
  // whose fp32 partials the latent norm adds (kv_a of the DeepSeek-V3 layer
  // 127 -> 77 us; the q down-projection, 384 tiles, gained nothing so)
  const int dsplit = (bf && hid % 64 == 0) ? 2 : 1;
  if (rq > 0) {
    void* ql_raw = bf ? (void*)q_lat32 : q_lat;
    if ((s = gemm(x, hid, w->w_q_a, ql_raw, rq, n, rq, hid, OUT_F32, EPI_STORE, nullptr)) != MLA_OK) return s;
    if ((s = norm(ql_raw, rq, rq, rq, w->q_a_gamma, 0, 0, 1, q_lat, rq, true)) != MLA_OK) return s;
    if ((s = gemm(q_lat, rq, w->w_q_b, q, (int64_t)H * dqk, n, H * dqk, rq, att_kind, q_epi, nullptr)) != MLA_OK) return s;
  } else {
    if ((s = gemm(x, hid, w->w_q, q, (int64_t)H * dqk, n, H * dqk, hid, att_kind, q_epi, nullptr)) != MLA_OK) return s;
  }
  if (rope && !bf) {
    if ((s = norm(q, (int64_t)H * dqk, H * dqk, 0, nullptr, dn, H, dqk, q, (int64_t)H * dqk, false)) != MLA_OK) return s;
  }
  // joint latent: down-projection, latent norm + k_pe RoPE -> [c_n | k_pe']
  {
    void* ckv_raw = bf ? (void*)ckv32 : (void*)(ws + L.ckv32);
    if ((s = gemm(x, hid, w->w_kv_a, ckv_raw, lw, n, lw, hid, OUT_F32, EPI_STORE, nullptr, dsplit)) != MLA_OK) return s;
    if ((s = norm(ckv_raw, lw, lw, rkv, w->kv_a_gamma, rkv, rope ? 1 : 0, dr, lat, lw, true, f16op ? kpe16 : nullptr,
                  dsplit > 1 ? (int64_t)n * lw : 0)) != MLA_OK)
      return s;
  }
  // The rows keys and values are formed from: the new tokens' latent rows, or
  // for a chunk each sequence's cached prefix rows followed by its new rows.
  const void* kv_src = lat;
  const f16* kpe_src16 = kpe16;
  int kv_rows = n;
  const int32_t* cuk_dev = nullptr;
  if (chunk) {
    int32_t* cuk = (int32_t*)(ws + L.cuk);
    if ((e = launch_chunk_offsets(cu_seqlens_dev, chunk->prefix_dev, num_seqs, cuk, st)) != hipSuccess)
      return hip_fail(e, "chunk offsets");
    ChunkGatherArgs g{};
    g.cu = cu_seqlens_dev; g.prefix = chunk->prefix_dev; g.cuk = cuk;
    g.cache = chunk->cache; g.block_table = chunk->block_table; g.max_blocks = chunk->max_blocks;
    g.num_blocks = chunk->num_blocks; g.log2_block = chunk->log2_block;
    g.lat = lat; g.ctx = ws + L.ctx;
    g.kpe16_new = f16op ? kpe16 : nullptr; g.kpe16_ctx = f16op ? (f16*)(ws + L.kpe16ctx) : nullptr;
    g.row_width = lw; g.rope_dim = dr; g.n_ctx = chunk->n_ctx; g.n_new = n;
    if ((e = launch_gather_context(g, bf, chunk->max_ctx_len, num_seqs, st)) != hipSuccess)
      return hip_fail(e, "context gather");
    kv_src = ws + L.ctx;
    kpe_src16 = (const f16*)(ws + L.kpe16ctx);
    kv_rows = chunk->n_ctx;
    cuk_dev = cuk;
  }
  // per-head keys/values from the normalised latent
  if ((s = gemm(kv_src, lw, w->w_kv_b, kv, (int64_t)H * (dn + dv), kv_rows, H * (dn + dv), rkv, att_kind, EPI_STORE,
                nullptr)) != MLA_OK)
    return s;
  // attention
  {
    const void* kpe = f16op ? (const void*)kpe_src16 : (const void*)((const char*)kv_src + (size_t)rkv * elem_size(cfg));
    const int64_t kpe_stride = f16op ? dr : lw;
    if ((s = attention_impl(cfg, q, kv, kpe, kpe_stride, f16op, cu_seqlens_dev, cu_seqlens_host, num_seqs, n, attn, st,
                            cuk_dev, chunk ? chunk->cuk_host.data() : nullptr, kv_rows)) != MLA_OK)
      return s;
  }
  // optional gate, output projection
  if (cfg->output_gate) {
    if ((s = gemm(x, hid, w->w_g, attn, (int64_t)H * dv, n, H * dv, hid, OUT_ACT, EPI_GATE, attn)) != MLA_OK) return s;
  }
  if (cfg->o_groups > 0) {
    // grouped low-rank output projection: group g of the attention features
    // [n, H d_v / G] times its block of W_o_a -> columns g r_o .. of ot, then
    // ot W_o_b^T
    const int G = cfg->o_groups, ro = cfg->o_lora_rank, fg = H * dv / G;
    void* ot = ws + L.ot;
    GemmArgs g{};
    g.a = attn; g.lda = (int64_t)H * dv; g.a_bstride = fg;
    g.b = w->w_o_a; g.ldb = fg; g.b_bstride = (int64_t)ro * fg;
    g.c = ot; g.ldc = (int64_t)G * ro; g.c_bstride = ro;
    g.m = n; g.n = ro; g.k = fg; g.batch = G; g.epilogue = EPI_STORE;
    e = bf ? launch_gemm_bf16(g, st) : launch_gemm_f32(g, st);
    if (e != hipSuccess) return hip_fail(e, "grouped output projection launch");
    if ((s = gemm(ot, (int64_t)G * ro, w->w_o_b, out, hid, n, hid, G * ro, OUT_ACT, EPI_STORE, nullptr)) != MLA_OK) return s;
  } else {
    if ((s = gemm(attn, (int64_t)H * dv, w->w_o, out, hid, n, hid, H * dv, OUT_ACT, EPI_STORE, nullptr)) != MLA_OK) return s;
  }
  return MLA_OK;
}

// Argument checks and split plan of the absorbed decode (host only).
static mla_status decode_check(const mla_config* cfg, const void* w_kv_b, const void* q_nope, const void* q_pe,
                               const void* kv_cache, int32_t num_blocks, int32_t block_size,
                               const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens_dev,
                               const int32_t* seq_lens_host, int32_t batch, void* out, DecodePlan* plan,
                               int tile = 32) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "absorbed decode is compiled for bf16 only");
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  const int H = cfg->num_heads;
  if (H != 32 && H != 64 && H != 96 && H != 128) return fail(MLA_ERR_UNSUPPORTED, "decode supports 32, 64, 96 or 128 heads");
  if (batch <= 0) return fail(MLA_ERR_INVALID_ARG, "batch must be > 0");
  if (!w_kv_b || !q_nope || !q_pe || !kv_cache || !block_table || !seq_lens_dev || !seq_lens_host || !out)
    return fail(MLA_ERR_INVALID_ARG, "all tensors are required");
  if (num_blocks <= 0 || max_blocks <= 0) return fail(MLA_ERR_INVALID_ARG, "num_blocks and max_blocks must be > 0");
  if (block_size < 16 || (block_size & (block_size - 1)))
    return fail(MLA_ERR_INVALID_ARG, "block_size must be a power of two >= 16");
  // the kernels hold a sequence's key count (up to max_blocks * block_size) in 32 bits
  if ((int64_t)max_blocks * block_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "max_blocks * block_size must be below 2^31");
  for (int b = 0; b < batch; ++b)
    if (seq_lens_host[b] <= 0 || (int64_t)seq_lens_host[b] > (int64_t)max_blocks * block_size)
      return fail(MLA_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [1, max_blocks * block_size]", b, seq_lens_host[b]);
  const void* ptrs[] = {w_kv_b, q_nope, q_pe, kv_cache, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MLA_ERR_MISALIGNED, "decode needs 16-byte aligned tensors");
  *plan = decode_plan(cfg, seq_lens_host, batch, (int64_t)max_blocks * block_size, tile);
  return MLA_OK;
}

// Launch sequence of the absorbed decode over a checked plan; ws holds at
// least P.total bytes (a caller workspace or the static scratch).
static mla_status decode_launch(const mla_config* cfg, const DecodePlan& P, const void* w_kv_b, const void* q_nope,
                                const void* q_pe, const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens_dev,
                                int32_t batch, void* out, char* ws, hipStream_t st, bool fp8_cache = false,
                                float cache_scale = 1.f) {
  const int H = cfg->num_heads, dn = cfg->qk_nope_dim, dv = cfg->v_head_dim, R = cfg->kv_lora_rank;
  bf16* qt = (bf16*)(ws + P.qt);
  hipError_t e;
  DecodeArgs d{};
  d.qt = qt; d.q_pe = (const bf16*)q_pe; d.cache = (const bf16*)kv_cache; d.block_table = block_table;
  int lbs = 0;
  while ((1 << lbs) < block_size) ++lbs;
  d.max_blocks = max_blocks; d.num_blocks = num_blocks; d.log2_block = lbs; d.seq_lens = seq_lens_dev;
  d.part_o = (f16*)(ws + P.part_o); d.part_ml = (float*)(ws + P.part_ml);
  d.batch = batch; d.heads = H; d.quota = P.quota; d.max_slots = P.max_slots; d.num_items = P.groups;
  d.scale = scale_of(cfg);
  // absorb W_UK into the query: qt[b, h, :] = q_nope[b, h, :] . W_kv_b[h*(dn+dv) + 0:dn, :]
  d.q_nope = (const bf16*)q_nope; d.w_uk = (const bf16*)w_kv_b; d.w_uv_hstride = (int64_t)(dn + dv) * R;
  if ((e = launch_decode_absorb_q(d, st)) != hipSuccess) return hip_fail(e, "absorb q");
  if (fp8_cache) {
    d.cache = nullptr; d.cache8 = (const uint8_t*)kv_cache; d.cache_scale = cache_scale;
    if ((e = launch_decode_split_fp8(d, st)) != hipSuccess) return hip_fail(e, "decode split (fp8 cache)");
  } else if ((e = launch_decode_split(d, st)) != hipSuccess) {
    return hip_fail(e, "decode split");
  }
  // combine the splits and un-absorb W_UV: out[b, h, :] = W_kv_b[h*(dn+dv) + dn : +dv, :] . o_lat[b, h, :]
  d.w_uv = (const bf16*)w_kv_b + (int64_t)dn * R; d.w_uv_hstride = (int64_t)(dn + dv) * R;
  d.out = (bf16*)out; d.dv = dv;
  if ((e = launch_decode_combine_unabsorb(d, st)) != hipSuccess) return hip_fail(e, "decode combine");
  return MLA_OK;
}

mla_status mla_decode_absorbed_fwd(const mla_config* cfg, const void* w_kv_b, const void* q_nope, const void* q_pe,
                                   const void* kv_cache, int32_t num_blocks, int32_t block_size,
                                   const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens_dev,
                                   const int32_t* seq_lens_host, int32_t batch, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  DecodePlan P;
  mla_status s = decode_check(cfg, w_kv_b, q_nope, q_pe, kv_cache, num_blocks, block_size, block_table, max_blocks,
                              seq_lens_dev, seq_lens_host, batch, out, &P);
  if (s != MLA_OK) return s;
  if (workspace && !aligned16(workspace)) return fail(MLA_ERR_MISALIGNED, "decode needs a 16-byte aligned workspace");
  if (!workspace || workspace_bytes < P.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", P.total, workspace_bytes);
  s = decode_launch(cfg, P, w_kv_b, q_nope, q_pe, kv_cache, num_blocks, block_size, block_table, max_blocks,
                    seq_lens_dev, batch, out, (char*)workspace, (hipStream_t)stream);
  return s == MLA_OK ? ok() : s;
}

mla_status mla_decode_absorbed_fwd_noalloc(const mla_config* cfg, const void* w_kv_b, const void* q_nope,
                                           const void* q_pe, const void* kv_cache, int32_t num_blocks,
                                           int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                                           const int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                                           int32_t batch, void* out, void* stream) {
  DecodePlan P;
  mla_status s = decode_check(cfg, w_kv_b, q_nope, q_pe, kv_cache, num_blocks, block_size, block_table, max_blocks,
                              seq_lens_dev, seq_lens_host, batch, out, &P);
  if (s != MLA_OK) return s;
  if (P.total > kStaticScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "this batch needs %zu bytes of scratch; the static scratch holds %zu "
                "(use mla_decode_absorbed_fwd with a workspace)", P.total, kStaticScratchBytes);
  char* ws = nullptr;
  if ((s = static_scratch((hipStream_t)stream, &ws)) != MLA_OK) return s;
  s = decode_launch(cfg, P, w_kv_b, q_nope, q_pe, kv_cache, num_blocks, block_size, block_table, max_blocks,
                    seq_lens_dev, batch, out, ws, (hipStream_t)stream);
  return s == MLA_OK ? ok() : s;
}

mla_status mla_decode_absorbed_fp8_fwd(const mla_config* cfg, const void* w_kv_b, const void* q_nope,
                                       const void* q_pe, const void* kv_cache_fp8, float cache_scale,
                                       int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                                       int32_t max_blocks, const int32_t* seq_lens_dev,
                                       const int32_t* seq_lens_host, int32_t batch, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  DecodePlan P;
  mla_status s = decode_check(cfg, w_kv_b, q_nope, q_pe, kv_cache_fp8, num_blocks, block_size, block_table,
                              max_blocks, seq_lens_dev, seq_lens_host, batch, out, &P, 64);
  if (s != MLA_OK) return s;
  if (!(cache_scale > 0.f) || !std::isfinite(cache_scale))
    return fail(MLA_ERR_INVALID_ARG, "cache_scale must be a positive finite number");
  if (workspace && !aligned16(workspace)) return fail(MLA_ERR_MISALIGNED, "decode needs a 16-byte aligned workspace");
  if (!workspace || workspace_bytes < P.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", P.total, workspace_bytes);
  s = decode_launch(cfg, P, w_kv_b, q_nope, q_pe, kv_cache_fp8, num_blocks, block_size, block_table, max_blocks,
                    seq_lens_dev, batch, out, (char*)workspace, (hipStream_t)stream, true, cache_scale);
  return s == MLA_OK ? ok() : s;
}

size_t mla_attention_bwd_workspace_size(const mla_config* cfg, int32_t num_tokens) {
  if (check_config(cfg) != MLA_OK || num_tokens < 0) return 0;
  const size_t n = (size_t)num_tokens, H = (size_t)cfg->num_heads;
  return align256(n * H * 4) * 2 + align256(n * H * (size_t)cfg->qk_rope_dim * 4);
}

mla_status mla_attention_prefill_bwd(const mla_config* cfg, const void* q, const void* kv, const void* kpe,
                                     int64_t kpe_stride, const int32_t* cu_seqlens_dev,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs, const void* out,
                                     const float* lse, const void* dout, void* dq, void* dkv, void* dkpe,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the attention backward is compiled for bf16 only");
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  int n = 0;
  if ((s = check_cu(cu_seqlens_host, num_seqs, &n)) != MLA_OK) return s;
  if (n == 0) return ok();
  if (num_seqs > 65535) return fail(MLA_ERR_UNSUPPORTED, "the attention backward takes at most 65535 documents");
  for (int d = 0; d < num_seqs; ++d)
    if (cu_seqlens_host[d + 1] - cu_seqlens_host[d] > 65535 * 128)
      return fail(MLA_ERR_UNSUPPORTED, "the attention backward takes documents of at most 65535 * 128 tokens");
  if (!q || !kv || !kpe || !cu_seqlens_dev || !out || !dout || !dq || !dkv || !dkpe)
    return fail(MLA_ERR_INVALID_ARG, "q, kv, kpe, cu_seqlens_dev, out, dout, dq, dkv and dkpe are required");
  if (kpe_stride < cfg->qk_rope_dim) return fail(MLA_ERR_INVALID_ARG, "kpe_stride < d_rope");
  const void* ptrs[] = {q, kv, kpe, out, dout, dq, dkv, dkpe};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MLA_ERR_MISALIGNED, "the attention backward needs 16-byte aligned tensors");
  if (kpe_stride % 8) return fail(MLA_ERR_MISALIGNED, "kpe_stride must be a multiple of 8");
  if (lse && ((uintptr_t)lse & 3)) return fail(MLA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const size_t need = mla_attention_bwd_workspace_size(cfg, n);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(MLA_ERR_WORKSPACE, "an aligned workspace of %zu bytes is needed", need);
  const size_t H = (size_t)cfg->num_heads;
  char* ws = (char*)workspace;
  AttnBwdArgs a{};
  a.q = q; a.kv = kv; a.kpe = kpe; a.kpe_stride = kpe_stride; a.o = out; a.dout = dout;
  a.cu_dev = cu_seqlens_dev; a.n_tokens = n; a.heads = cfg->num_heads; a.scale = scale_of(cfg);
  a.lse = lse ? const_cast<float*>(lse) : (float*)ws;   // given: read only
  a.lse_ready = lse != nullptr;
  a.dsum = (float*)(ws + align256((size_t)n * H * 4));
  a.dkr = (float*)(ws + 2 * align256((size_t)n * H * 4));
  a.dq = (float*)dq; a.dkv = (float*)dkv; a.dkpe = (float*)dkpe;
  const hipError_t e = launch_attention_bwd(a, cu_seqlens_host, num_seqs, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return ok();
}

// ---------------------------------------------------------------- layer backward
namespace {
struct LayerBwdWs {
  size_t pos, q_lat32, q_lat, q, ckv32, lat, kv, attn, gpre, a2, ot, dt, da2, da, dg, dkpe32, abw,
      dq16, dkv16, dckv, dcn32, dqln32, dql16, rinv, part, tr, trb, xt, wot, split, total;
  int64_t npad;
};

// the latent-side NN products of the layer backward (K = H * 256 or H * 192,
// few output tiles) run as kSplitK products over K slices, summed after
constexpr int kSplitK = 4;

LayerBwdWs layer_bwd_layout(const mla_config* c, int64_t n) {
  const int64_t H = c->num_heads, rq = c->q_lora_rank, rkv = c->kv_lora_rank, dr = c->qk_rope_dim;
  const int64_t dqk = c->qk_nope_dim + dr, dkv = c->qk_nope_dim + c->v_head_dim, F = H * c->v_head_dim;
  const int64_t lw = rkv + dr, gro = c->o_groups > 0 ? (int64_t)c->o_groups * c->o_lora_rank : 0;
  LayerBwdWs w{};
  w.npad = (n + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  w.pos = take(n * 4);
  w.q_lat32 = take(n * rq * 4);
  w.q_lat = take(n * rq * 2);
  w.q = take(n * H * dqk * 2);
  w.ckv32 = take(n * lw * 4);
  w.lat = take(n * lw * 2);
  w.kv = take(n * H * dkv * 2);
  w.attn = take(n * F * 2);
  w.gpre = take(c->output_gate ? n * F * 4 : 0);
  w.a2 = take(c->output_gate ? n * F * 2 : 0);
  w.ot = take(n * gro * 2);
  w.dt = take(n * gro * 2);
  w.da2 = take(c->output_gate ? n * F * 4 : 0);        // fp32 dA2 for the gate's backward
  w.da = take(n * F * 2);
  w.dg = take(c->output_gate ? n * F * 2 : 0);
  w.dkpe32 = take(n * dr * 4);
  w.abw = take(mla_attention_bwd_workspace_size(c, (int32_t)n));
  w.dq16 = take(n * H * dqk * 2);
  w.dkv16 = take(n * H * dkv * 2);
  w.dckv = take(n * lw * 2);
  w.dcn32 = take(n * rkv * 4);
  w.dqln32 = take(n * rq * 4);
  w.dql16 = take(n * rq * 2);
  w.rinv = take(n * 4);
  w.part = take((n + 255) / 256 * std::max(rkv, rq) * 4);
  const int64_t tcols = std::max({(int64_t)c->hidden, F, H * dkv, H * dqk, lw, rq, gro});
  w.tr = take(tcols * w.npad * 2);                       // dY^T of a weight gradient
  w.trb = take(std::max({F, rq, rkv, gro}) * w.npad * 2);  // X^T of a weight gradient
  w.xt = take((int64_t)c->hidden * w.npad * 2);           // x^T (three weight gradients read it)
  w.wot = take(c->o_groups > 0 ? 0 : F * c->hidden * 2);  // W_o^T (NT form of dA2 = dout W_o)
  w.split = take(n * std::max(kSplitK * std::max(rkv, rq), 2 * kSplitK * rkv) * 4);   // split-K partials of dc_n, dq_lat_n
  w.total = off;
  return w;
}
}  // namespace

size_t mla_prefill_bwd_workspace_size(const mla_config* cfg, int32_t num_tokens) {
  if (check_config(cfg) != MLA_OK || num_tokens < 0) return 0;
  return layer_bwd_layout(cfg, num_tokens).total;
}

mla_status mla_prefill_bwd(const mla_config* cfg, const mla_weights* w, const void* x, const int32_t* cu_seqlens_dev,
                           const int32_t* cu_seqlens_host, int32_t num_seqs, const int32_t* positions_dev,
                           const float* rope_cos, const float* rope_sin, int32_t rope_table_len, const void* dout,
                           float* dx, const mla_weight_grads* dw, void* workspace, size_t workspace_bytes,
                           void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the layer backward is compiled for bf16 only");
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  if ((s = check_weights(cfg, w)) != MLA_OK) return s;
  int n = 0;
  if ((s = check_cu(cu_seqlens_host, num_seqs, &n)) != MLA_OK) return s;
  if (n == 0) return ok();
  if (!x || !dout || !dx || !cu_seqlens_dev || !dw)
    return fail(MLA_ERR_INVALID_ARG, "x, dout, dx, dw and cu_seqlens_dev are required");
  const bool rope = cfg->rope_kind != MLA_ROPE_NONE;
  if (rope && (!rope_cos || !rope_sin || rope_table_len <= 0))
    return fail(MLA_ERR_INVALID_ARG, "RoPE needs device cos/sin tables and their length");
  const int H = cfg->num_heads, hid = cfg->hidden, rq = cfg->q_lora_rank, rkv = cfg->kv_lora_rank;
  const int dn = cfg->qk_nope_dim, dr = cfg->qk_rope_dim, dv = cfg->v_head_dim, dqk = dn + dr, lw = rkv + dr;
  const int dkvw = dn + dv, F = H * dv, G = cfg->o_groups, ro = cfg->o_lora_rank, gro = G > 0 ? G * ro : 0;
  const int fg = G > 0 ? F / G : 0;
  // the weight gradients this configuration needs
  struct Need { const void* have; const char* name; };
  const Need need[] = {
      {rq > 0 ? dw->w_q_a : (void*)1, "w_q_a"}, {rq > 0 ? dw->q_a_gamma : (void*)1, "q_a_gamma"},
      {rq > 0 ? dw->w_q_b : (void*)1, "w_q_b"}, {rq == 0 ? dw->w_q : (void*)1, "w_q"},
      {dw->w_kv_a, "w_kv_a"}, {dw->kv_a_gamma, "kv_a_gamma"}, {dw->w_kv_b, "w_kv_b"},
      {G == 0 ? dw->w_o : (void*)1, "w_o"}, {cfg->output_gate ? dw->w_g : (void*)1, "w_g"},
      {G > 0 ? dw->w_o_a : (void*)1, "w_o_a"}, {G > 0 ? dw->w_o_b : (void*)1, "w_o_b"}};
  for (const Need& q : need)
    if (!q.have) return fail(MLA_ERR_INVALID_ARG, "the gradient of %s is required by this configuration", q.name);
  {
    const void* ptrs[] = {x, dout, dx, w->w_kv_a, w->kv_a_gamma, w->w_kv_b, workspace};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return fail(MLA_ERR_MISALIGNED, "the layer backward needs 16-byte aligned tensors");
    const void* opt[] = {w->w_q_a, w->w_q_b, w->w_q, w->w_o, w->w_g, w->w_o_a, w->w_o_b, dw->w_q_a, dw->w_q_b,
                         dw->w_q, dw->w_kv_a, dw->w_kv_b, dw->w_o, dw->w_g, dw->w_o_a, dw->w_o_b};
    for (const void* p : opt)
      if (p && !aligned16(p)) return fail(MLA_ERR_MISALIGNED, "the layer backward needs 16-byte aligned tensors");
  }
  const LayerBwdWs L = layer_bwd_layout(cfg, n);
  if (!workspace || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  const hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto at = [&](size_t off) { return (void*)(ws + off); };
  bf16* tr = (bf16*)at(L.tr);
  const int64_t npad = L.npad;
  hipError_t e;

  const int32_t* positions = positions_dev;
  if (rope && !positions) {
    if ((e = launch_positions(cu_seqlens_dev, num_seqs, n, (int32_t*)at(L.pos), st)) != hipSuccess)
      return hip_fail(e, "positions");
    positions = (const int32_t*)at(L.pos);
  }
  // y = a b^T (b [n, k]) or, nn, y = a b (b [k, n]); fp32 or bf16 output
  auto gemm = [&](const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc, int m, int nn, int k,
                  bool nn_layout, bool f32_out, bool acc, int epi = EPI_STORE, int batch = 1, int64_t abs = 0,
                  int64_t bbs = 0, int64_t cbs = 0) -> mla_status {
    GemmArgs g{};
    g.a = a; g.lda = lda; g.a_bstride = abs; g.b = b; g.ldb = ldb; g.b_bstride = bbs; g.c = c; g.ldc = ldc;
    g.c_bstride = cbs; g.m = m; g.n = nn; g.k = k; g.batch = batch; g.b_kn = nn_layout; g.c_f32 = f32_out;
    g.c_acc = acc; g.epilogue = epi;
    g.cos_t = rope_cos; g.sin_t = rope_sin; g.table_len = rope_table_len; g.positions = positions;
    g.rope_head_stride = dqk; g.rope_off = dn; g.rope_interleave = cfg->rope_interleave;
    const hipError_t err = launch_gemm_bf16(g, st);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "layer backward GEMM");
  };
  // dW [cols(dy), cols(xin)] = dy^T xin over the n tokens.  With at least
  // 256 output tiles of 256 x 256 the first n - n % 32 tokens run on the
  // 256x256 kernel reading dy and xin as stored (K-major operands) and the
  // last n % 32 are added from their transposes (zero-padded to 64 tokens);
  // otherwise dy and xin are transposed (rounded to bf16, zero past the last
  // token) into K-major buffers for an NT product over the padded token count
  // (x^T, which three gradients read, is transposed once).
  bf16* trb = (bf16*)at(L.trb);
  bf16* xt = (bf16*)at(L.xt);
  bool xt_ready = false;
  auto weight_grad = [&](const void* dy, bool dy_f32, int64_t ld_dy, int dy_cols, const void* xin, int64_t ld_x,
                         int x_cols, float* out) -> mla_status {
    const int n32 = n / 32 * 32;
    const int64_t out_tiles = (int64_t)((dy_cols + 255) / 256) * ((x_cols + 255) / 256);
    if (!dy_f32 && n32 > 0 && out_tiles >= 256 && dy_cols % 8 == 0 && x_cols % 8 == 0 && ld_dy % 8 == 0 &&
        ld_x % 8 == 0 && aligned16(dy) && aligned16(xin)) {
      GemmArgs g{};
      g.a = dy; g.lda = ld_dy; g.b = xin; g.ldb = ld_x; g.c = out; g.ldc = x_cols;
      g.m = dy_cols; g.n = x_cols; g.k = n32; g.batch = 1; g.c_f32 = true; g.epilogue = EPI_STORE; g.kmajor = true;
      hipError_t err = launch_gemm_bf16(g, st);
      if (err != hipSuccess) return hip_fail(err, "weight-gradient GEMM");
      if (n32 == n) return MLA_OK;
      const int rows = n - n32;
      bf16* xb = xin == x ? xt : trb;
      if (xin == x) xt_ready = false;     // xt now holds the tail only
      if ((err = launch_transpose_bf16((const bf16*)dy + (int64_t)n32 * ld_dy, false, ld_dy, rows, dy_cols, tr, 64,
                                       64, st)) != hipSuccess ||
          (err = launch_transpose_bf16((const bf16*)xin + (int64_t)n32 * ld_x, false, ld_x, rows, x_cols, xb, 64, 64,
                                       st)) != hipSuccess)
        return hip_fail(err, "transpose");
      return gemm(tr, 64, xb, 64, out, x_cols, dy_cols, x_cols, 64, false, true, true);
    }
    hipError_t err = launch_transpose_bf16(dy, dy_f32, ld_dy, n, dy_cols, tr, npad, (int)npad, st);
    if (err != hipSuccess) return hip_fail(err, "transpose");
    const bf16* bt = trb;
    if (xin == x) {
      if (!xt_ready && (err = launch_transpose_bf16(x, false, hid, n, hid, xt, npad, (int)npad, st)) != hipSuccess)
        return hip_fail(err, "transpose");
      xt_ready = true;
      bt = xt;
    } else if ((err = launch_transpose_bf16(xin, false, ld_x, n, x_cols, trb, npad, (int)npad, st)) != hipSuccess) {
      return hip_fail(err, "transpose");
    }
    return gemm(tr, npad, bt, npad, out, x_cols, dy_cols, x_cols, (int)npad, false, true, false);
  };
  // c [m, nn] fp32 = a [m, k] b [k, nn] (NN) as kSplitK products over slices
  // of k (batched, into partial buffers) and their sum; 2 kSplitK slices when
  // that (and only that) gives the 256x256 kernel its 256 tiles (nn <= r_kv)
  auto gemm_nn_splitk = [&](const void* a, int64_t lda, const void* b, int64_t ldb, float* c, int m, int nn,
                            int k) -> mla_status {
    float* part = (float*)at(L.split);
    if (k % (kSplitK * 8) != 0 || (int64_t)m * nn % 4 != 0)
      return gemm(a, lda, b, ldb, c, nn, m, nn, k, true, true, false);
    const int64_t tiles = (int64_t)((m + 255) / 256) * ((nn + 255) / 256);
    const int split = tiles * kSplitK < 256 && tiles * 2 * kSplitK >= 256 && k % (2 * kSplitK * 32) == 0 &&
                              nn <= rkv ? 2 * kSplitK : kSplitK;
    const int ks = k / split;
    mla_status r = gemm(a, lda, b, ldb, part, nn, m, nn, ks, true, true, false, EPI_STORE, split, ks,
                        (int64_t)ks * ldb, (int64_t)m * nn);
    if (r != MLA_OK) return r;
    const hipError_t err = launch_sum_partials(part, split, (int64_t)m * nn, c, st);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "split-K sum");
  };
  auto norm = [&](const void* src, int64_t stride, int width, int norm_dim, const void* gamma, int rope_off,
                  int rope_slices, void* dst, int64_t dst_stride) -> mla_status {
    NormRopeArgs a{};
    a.interleave = cfg->rope_interleave;
    a.src = src; a.src_stride = stride; a.n_rows = n; a.row_width = width; a.norm_dim = norm_dim; a.gamma = gamma;
    a.eps = cfg->norm_eps; a.rope_offset = rope_off; a.rope_slices = rope_slices; a.rope_stride = dr;
    a.rope_dim = dr; a.cos_t = rope_cos; a.sin_t = rope_sin; a.table_len = rope_table_len; a.positions = positions;
    a.dst = dst; a.dst_stride = dst_stride;
    const hipError_t err = launch_norm_rope(a, true, st, true);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "latent norm / rope launch");
  };
  auto rope_back = [&](const float* src, int64_t ld_src, int width, bf16* dst, int64_t ld_dst, int rope_off,
                       int slices, int stride) -> mla_status {
    RopeBackArgs a{};
    a.src = src; a.ld_src = ld_src; a.n_rows = n; a.width = width; a.dst = dst; a.ld_dst = ld_dst;
    a.rope_off = rope_off; a.rope_slices = rope ? slices : 0; a.rope_stride = stride; a.rope_dim = dr;
    a.interleave = cfg->rope_interleave; a.cos_t = rope_cos; a.sin_t = rope_sin; a.table_len = rope_table_len;
    a.positions = positions;
    const hipError_t err = launch_rope_back(a, st);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "rope backward");
  };
  auto norm_back = [&](const float* xin, int64_t ld_x, const float* dy, int64_t ld_dy, const void* gamma, int width,
                       bf16* dxo, int64_t ld_dx, float* dgamma) -> mla_status {
    RmsNormBwdArgs a{};
    a.x = xin; a.ld_x = ld_x; a.dy = dy; a.ld_dy = ld_dy; a.gamma = gamma; a.n_rows = n; a.width = width;
    a.eps = cfg->norm_eps; a.dx = dxo; a.ld_dx = ld_dx; a.rinv = (float*)at(L.rinv);
    const hipError_t err = launch_rms_norm_bwd(a, (float*)at(L.part), dgamma, st);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "rmsnorm backward");
  };

  // ---- forward, recomputed (bf16 attention operands)
  bf16* q = (bf16*)at(L.q);
  bf16* lat = (bf16*)at(L.lat);
  bf16* kv = (bf16*)at(L.kv);
  bf16* attn = (bf16*)at(L.attn);
  float* q_lat32 = (float*)at(L.q_lat32);
  bf16* q_lat = (bf16*)at(L.q_lat);
  float* ckv32 = (float*)at(L.ckv32);
  const int q_epi = rope ? EPI_ROPE : EPI_STORE;
  if (rq > 0) {
    if ((s = gemm(x, hid, w->w_q_a, hid, q_lat32, rq, n, rq, hid, false, true, false)) != MLA_OK) return s;
    if ((s = norm(q_lat32, rq, rq, rq, w->q_a_gamma, 0, 0, q_lat, rq)) != MLA_OK) return s;
    if ((s = gemm(q_lat, rq, w->w_q_b, rq, q, (int64_t)H * dqk, n, H * dqk, rq, false, false, false, q_epi)) != MLA_OK)
      return s;
  } else {
    if ((s = gemm(x, hid, w->w_q, hid, q, (int64_t)H * dqk, n, H * dqk, hid, false, false, false, q_epi)) != MLA_OK)
      return s;
  }
  if ((s = gemm(x, hid, w->w_kv_a, hid, ckv32, lw, n, lw, hid, false, true, false)) != MLA_OK) return s;
  if ((s = norm(ckv32, lw, lw, rkv, w->kv_a_gamma, rkv, rope ? 1 : 0, lat, lw)) != MLA_OK) return s;
  if ((s = gemm(lat, lw, w->w_kv_b, rkv, kv, (int64_t)H * dkvw, n, H * dkvw, rkv, false, false, false)) != MLA_OK)
    return s;
  // the forward leaves its softmax statistics for the attention backward
  float* lse_fwd = (float*)at(L.abw);
  if ((s = attention_impl(cfg, q, kv, lat + rkv, lw, false, cu_seqlens_dev, cu_seqlens_host, num_seqs, n, attn, st,
                          nullptr, nullptr, -1, lse_fwd)) != MLA_OK)
    return s;
  const bf16* a2 = attn;                         // the output projection's input
  float* gpre = (float*)at(L.gpre);
  if (cfg->output_gate) {
    if ((s = gemm(x, hid, w->w_g, hid, gpre, F, n, F, hid, false, true, false)) != MLA_OK) return s;
    if ((e = launch_gate_fwd(attn, gpre, (bf16*)at(L.a2), (int64_t)n * F, st)) != hipSuccess) return hip_fail(e, "gate");
    a2 = (const bf16*)at(L.a2);
  }
  bf16* ot = (bf16*)at(L.ot);
  if (G > 0) {
    if ((s = gemm(a2, F, w->w_o_a, fg, ot, gro, n, ro, fg, false, false, false, EPI_STORE, G, fg, (int64_t)ro * fg,
                  ro)) != MLA_OK)
      return s;
  }

  // ---- output projection
  float* da2 = (float*)at(L.da2);
  if (G > 0) {
    bf16* dt = (bf16*)at(L.dt);
    if ((s = weight_grad(dout, false, hid, hid, ot, gro, gro, dw->w_o_b)) != MLA_OK) return s;
    if ((s = gemm(dout, hid, w->w_o_b, gro, dt, gro, n, gro, hid, true, false, false)) != MLA_OK) return s;
    // dW_o_a[g] = dt_g^T a2_g (groups batched over the transposed dt)
    if ((e = launch_transpose_bf16(dt, false, gro, n, gro, tr, npad, (int)npad, st)) != hipSuccess)
      return hip_fail(e, "transpose");
    if ((s = gemm(tr, npad, a2, F, dw->w_o_a, fg, ro, fg, n, true, true, false, EPI_STORE, G, (int64_t)ro * npad, fg,
                  (int64_t)ro * fg)) != MLA_OK)
      return s;
    // dA2 in fp32 for the gate's backward, else straight to bf16 dA
    if ((s = gemm(dt, gro, w->w_o_a, fg, cfg->output_gate ? (void*)da2 : at(L.da), F, n, fg, ro, true,
                  cfg->output_gate, false, EPI_STORE, G, ro, (int64_t)ro * fg, fg)) != MLA_OK)
      return s;
  } else {
    if ((s = weight_grad(dout, false, hid, hid, a2, F, F, dw->w_o)) != MLA_OK) return s;
    // dA2 = dout W_o as an NT product against W_o^T
    bf16* wot = (bf16*)at(L.wot);
    if ((e = launch_transpose_bf16(w->w_o, false, F, hid, F, wot, hid, hid, st)) != hipSuccess)
      return hip_fail(e, "transpose");
    if ((s = gemm(dout, hid, wot, hid, cfg->output_gate ? (void*)da2 : at(L.da), F, n, F, hid, false,
                  cfg->output_gate, false)) != MLA_OK)
      return s;
  }
  // ---- gate
  bf16* da = (bf16*)at(L.da);
  bf16* dgp = (bf16*)at(L.dg);
  if (cfg->output_gate) {
    if ((e = launch_gate_bwd(da2, attn, gpre, da, dgp, (int64_t)n * F, st)) != hipSuccess) return hip_fail(e, "gate backward");
  }
  // ---- attention core: bf16 dq (rotary map undone) and [dk_nope | dv],
  // fp32 shared-key gradient
  float* dkpe32 = (float*)at(L.dkpe32);
  bf16* dq16 = (bf16*)at(L.dq16);
  bf16* dkv16 = (bf16*)at(L.dkv16);
  {
    AttnBwdArgs a{};
    char* aw = (char*)at(L.abw);
    a.q = q; a.kv = kv; a.kpe = lat + rkv; a.kpe_stride = lw; a.o = attn; a.dout = da;
    a.cu_dev = cu_seqlens_dev; a.n_tokens = n; a.heads = H; a.scale = scale_of(cfg);
    a.lse = (float*)aw;
    a.dsum = (float*)(aw + align256((size_t)n * H * 4));
    a.dkr = (float*)(aw + 2 * align256((size_t)n * H * 4));
    a.dkpe = dkpe32;
    a.lse_ready = true;
    a.dq16 = dq16; a.dkv16 = dkv16;
    a.rope = rope; a.rope_interleave = cfg->rope_interleave != 0; a.cos_t = rope_cos; a.sin_t = rope_sin;
    a.table_len = rope_table_len; a.positions = positions;
    if ((e = launch_attention_bwd(a, cu_seqlens_host, num_seqs, st)) != hipSuccess) return hip_fail(e, "attention backward");
  }
  // ---- RoPE backward of the shared key part, bf16
  bf16* dckv = (bf16*)at(L.dckv);
  if ((s = rope_back(dkpe32, dr, dr, dckv + rkv, lw, 0, 1, dr)) != MLA_OK) return s;
  // ---- kv up-projection, latent norm, joint down-projection
  float* dcn32 = (float*)at(L.dcn32);
  if ((s = weight_grad(dkv16, false, (int64_t)H * dkvw, H * dkvw, lat, lw, rkv, dw->w_kv_b)) != MLA_OK) return s;
  if ((s = gemm_nn_splitk(dkv16, (int64_t)H * dkvw, w->w_kv_b, rkv, dcn32, n, rkv, H * dkvw)) != MLA_OK) return s;
  if ((s = norm_back(ckv32, lw, dcn32, rkv, w->kv_a_gamma, rkv, dckv, lw, dw->kv_a_gamma)) != MLA_OK) return s;
  if ((s = weight_grad(dckv, false, lw, lw, x, hid, hid, dw->w_kv_a)) != MLA_OK) return s;
  if ((s = gemm(dckv, lw, w->w_kv_a, hid, dx, hid, n, hid, lw, true, true, false)) != MLA_OK) return s;
  // ---- query path
  if (rq > 0) {
    float* dqln32 = (float*)at(L.dqln32);
    bf16* dql16 = (bf16*)at(L.dql16);
    if ((s = weight_grad(dq16, false, (int64_t)H * dqk, H * dqk, q_lat, rq, rq, dw->w_q_b)) != MLA_OK) return s;
    if ((s = gemm_nn_splitk(dq16, (int64_t)H * dqk, w->w_q_b, rq, dqln32, n, rq, H * dqk)) != MLA_OK) return s;
    if ((s = norm_back(q_lat32, rq, dqln32, rq, w->q_a_gamma, rq, dql16, rq, dw->q_a_gamma)) != MLA_OK) return s;
    if ((s = weight_grad(dql16, false, rq, rq, x, hid, hid, dw->w_q_a)) != MLA_OK) return s;
    if ((s = gemm(dql16, rq, w->w_q_a, hid, dx, hid, n, hid, rq, true, true, true)) != MLA_OK) return s;
  } else {
    if ((s = weight_grad(dq16, false, (int64_t)H * dqk, H * dqk, x, hid, hid, dw->w_q)) != MLA_OK) return s;
    if ((s = gemm(dq16, (int64_t)H * dqk, w->w_q, hid, dx, hid, n, hid, H * dqk, true, true, true)) != MLA_OK) return s;
  }
  // ---- gate projection
  if (cfg->output_gate) {
    if ((s = weight_grad(dgp, false, F, F, x, hid, hid, dw->w_g)) != MLA_OK) return s;
    if ((s = gemm(dgp, F, w->w_g, hid, dx, hid, n, hid, F, true, true, true)) != MLA_OK) return s;
  }
  return ok();
}

mla_status mla_q_uproj_rope_mxfp8(const mla_config* cfg, const void* q_latent, int64_t ldq, int32_t n_tokens,
                                  const void* w_q_b, const int32_t* positions, const float* rope_cos,
                                  const float* rope_sin, int32_t rope_table_len, void* q_codes, void* q_scales,
                                  void* stream) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the MXFP8 query projection is compiled for bf16 only");
  if ((s = check_supported(cfg)) != MLA_OK) return s;
  if (cfg->q_lora_rank <= 0) return fail(MLA_ERR_INVALID_ARG, "the fused query up-projection needs a query latent (q_lora_rank > 0)");
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens == 0) return ok();
  const bool rope = cfg->rope_kind != MLA_ROPE_NONE;
  if (!q_latent || !w_q_b || !q_codes || !q_scales) return fail(MLA_ERR_INVALID_ARG, "q_latent, w_q_b, q_codes and q_scales are required");
  if (rope && (!positions || !rope_cos || !rope_sin || rope_table_len <= 0))
    return fail(MLA_ERR_INVALID_ARG, "positions and the RoPE tables are required with RoPE");
  const int R = cfg->q_lora_rank, H = cfg->num_heads, dqk = cfg->qk_nope_dim + cfg->qk_rope_dim;
  if (ldq < R) return fail(MLA_ERR_INVALID_ARG, "ldq >= q_lora_rank required");
  if (!aligned16(q_latent) || !aligned16(w_q_b) || !aligned16(q_codes) || ((uintptr_t)q_scales & 7) || ldq % 8)
    return fail(MLA_ERR_MISALIGNED, "q_latent, w_q_b, q_codes need 16-byte alignment, q_scales 8, ldq a multiple of 8");
  if (R % 32) return fail(MLA_ERR_UNSUPPORTED, "q_lora_rank must be a multiple of 32");
  GemmArgs g{};
  g.a = q_latent; g.lda = ldq; g.b = w_q_b; g.ldb = R; g.c = q_codes; g.ldc = (int64_t)H * dqk;
  g.m = n_tokens; g.n = H * dqk; g.k = R; g.batch = 1;
  g.c_mx = true; g.c_scale = q_scales; g.ld_scale = (int64_t)H * dqk / 32;
  g.epilogue = rope ? EPI_ROPE : EPI_STORE;
  g.cos_t = rope_cos; g.sin_t = rope_sin; g.table_len = rope_table_len; g.positions = positions;
  g.rope_head_stride = dqk; g.rope_off = cfg->qk_nope_dim; g.rope_interleave = cfg->rope_interleave;
  const hipError_t e = launch_gemm_bf16(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "MXFP8 query projection");
  return ok();
}

mla_status mla_cache_quantize_fp8(const void* src, int64_t src_row_stride, int64_t n_rows, int32_t row_width,
                                  float scale, void* dst, int64_t dst_row_stride, void* stream) {
  if (n_rows < 0 || row_width <= 0) return fail(MLA_ERR_INVALID_ARG, "n_rows >= 0 and row_width > 0 required");
  if (n_rows == 0) return ok();
  if (!src || !dst) return fail(MLA_ERR_INVALID_ARG, "src and dst are required");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARG, "scale must be a positive finite number");
  if (row_width % 8 || src_row_stride < row_width || dst_row_stride < row_width || src_row_stride % 8 ||
      dst_row_stride % 8)
    return fail(MLA_ERR_MISALIGNED, "row_width and both strides must be multiples of 8 (strides >= row_width)");
  if (!aligned16(src) || ((uintptr_t)dst & 7))
    return fail(MLA_ERR_MISALIGNED, "src must be 16-byte aligned and dst 8-byte aligned");
  CacheQuantArgs q{};
  q.src = (const bf16*)src; q.src_stride = src_row_stride;
  q.dst = (uint8_t*)dst; q.dst_stride = dst_row_stride;
  q.rows = n_rows; q.width = row_width;
  q.inv = 1.0f / scale;
  const hipError_t e = launch_cache_quant_fp8(q, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache quantisation");
  return ok();
}

}  // extern "C"
