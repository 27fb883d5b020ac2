// The C ABI of libtv.so (declared in include/tv.h): argument checks, launch
// planning and kernel dispatch.  Nothing here allocates or synchronises.
#include <math.h>

#include <atomic>
#include <mutex>

#include "tv.h"
#include "tv_kernels.h"

// Split-kv scratch of tv_verify_attn_noalloc: one copy per device, held until
// the process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Flags tv_verify_attn_ex knows.
constexpr uint32_t kAttnFlags = TV_ATTN_BF16_QUERIES | TV_ATTN_F32_WIDE;

// Most rotated pairs one RoPE launch takes (its grid strides over them).
constexpr int64_t kMaxRopePairs = int64_t{1} << 40;

bool supported_attn(int32_t d_c, int32_t d_r, tv_dtype_t dt) {
  const bool dc_ok = d_c == 64 || d_c == 128 || d_c == 256 || d_c == 512;
  const bool dr_ok = d_r == 32 || d_r == 64;
  const bool dt_ok = dt == TV_F32 || dt == TV_BF16;
  return dc_ok && dr_ok && dt_ok;
}

tv::RopeFreq make_freq(int32_t d_r, double theta) {
  tv::RopeFreq f{};
  const int half = d_r / 2;
  for (int k = 0; k < half; ++k) f.inv_freq[k] = 1.0 / pow(theta, (2.0 * k) / static_cast<double>(d_r));
  return f;
}

// Shape checks shared by tv_verify_attn and tv_verify_step.
tv_status_t check_attn_shape(int32_t prefix_len, int32_t B, int32_t H, int32_t q_len, int32_t d_c, int32_t d_r,
                             tv_dtype_t kv_dtype) {
  if (B < 1 || H < 1 || q_len < 1 || prefix_len < 0) return TV_ERR_INVALID;
  if (d_c < 1 || d_r < 1 || (d_r & 1)) return TV_ERR_INVALID;
  if (kv_dtype != TV_F32 && kv_dtype != TV_BF16) return TV_ERR_INVALID;
  if (q_len > TV_MAX_Q_LEN) return TV_ERR_UNSUPPORTED;
  if (prefix_len > INT32_MAX - TV_MAX_Q_LEN) return TV_ERR_INVALID;
  if (static_cast<int64_t>(q_len) * H > (1 << 24)) return TV_ERR_UNSUPPORTED;
  if (!supported_attn(d_c, d_r, kv_dtype)) return TV_ERR_UNSUPPORTED;
  // The kernels address one tree's latent rows with 32-bit byte offsets.
  const int64_t elem = kv_dtype == TV_BF16 ? 2 : 4;
  if ((static_cast<int64_t>(prefix_len) + q_len) * d_c * elem >= (int64_t{1} << 31)) return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

tv::AttnShape make_shape(int32_t prefix_len, int32_t B, int32_t H, int32_t q_len, int32_t d_c, int32_t d_r,
                         tv_dtype_t kv_dtype, uint32_t flags = 0) {
  return tv::AttnShape{B,   H,   q_len, prefix_len, prefix_len + q_len,
                       d_c, d_r, kv_dtype == TV_BF16, (flags & TV_ATTN_BF16_QUERIES) != 0,
                       (flags & TV_ATTN_F32_WIDE) != 0};
}

tv_status_t run_attention(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                          const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                          int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream, uint32_t flags = 0) {
  const tv::AttnShape s = make_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype, flags);
  const tv::AttnPlan plan = tv::plan_attention(s);
  if (workspace_bytes < plan.ws_bytes || (plan.ws_bytes > 0 && (workspace == nullptr || !aligned16(workspace))))
    return TV_ERR_INVALID;
  tv::AttnArgs a{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.parent = parent;
  a.out = out;
  a.lse = lse;
  if (plan.ws_bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws + plan.ws_o_off);
    a.ws_m = reinterpret_cast<float*>(ws + plan.ws_m_off);
    a.ws_l = reinterpret_cast<float*>(ws + plan.ws_l_off);
  }
  a.B = B;
  a.H = H;
  a.q_len = q_len;
  a.prefix_len = prefix_len;
  a.kv_len = s.kv_len;
  a.R = q_len * H;
  a.rows_per_block = plan.rows_per_block;
  a.n_rb = plan.n_rb;
  a.full_rb = plan.full_rb;
  a.split_full = plan.split_full;
  a.chunk_full = plan.chunk_full;
  a.split_tail = plan.split_tail;
  a.chunk_tail = plan.chunk_tail;
  a.sm_scale = sm_scale;
  return tv::launch_attention(s, plan, a, stream) == hipSuccess ? TV_OK : TV_ERR_LAUNCH;
}

// Shape checks and plan of a ragged batch (bounds max_q_len, kv_stride).
tv_status_t plan_ragged(int32_t B, int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r,
                        tv_dtype_t kv_dtype, tv::AttnShape& s, tv::AttnPlan& plan) {
  if (kv_stride < max_q_len) return TV_ERR_INVALID;
  const tv_status_t st = check_attn_shape(kv_stride - max_q_len, B, H, max_q_len, d_c, d_r, kv_dtype);
  if (st != TV_OK) return st;
  s = make_shape(kv_stride - max_q_len, B, H, max_q_len, d_c, d_r, kv_dtype);
  plan = tv::plan_attention_ragged(s);
  // Unit, slot and row counts are int32 on the device.
  if (plan.units > INT32_MAX || static_cast<int64_t>(B) * max_q_len * H > INT32_MAX) return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

// Checks and kernel arguments of a ragged call (tv_verify_attn_ragged,
// tv_verify_step_ragged).
tv_status_t ragged_args(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                        const int32_t* parent, const int32_t* prefix_len, const int32_t* q_len, int32_t n_nodes,
                        int32_t B, int32_t H,
                        int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype,
                        float sm_scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                        tv::AttnShape& s, tv::AttnPlan& plan, tv::AttnArgs& a) {
  const tv_status_t st = plan_ragged(B, H, max_q_len, kv_stride, d_c, d_r, kv_dtype, s, plan);
  if (st != TV_OK) return st;
  if (n_nodes < 0) return TV_ERR_INVALID;
  if (static_cast<int64_t>(n_nodes) * H > INT32_MAX) return TV_ERR_UNSUPPORTED;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !parent || !prefix_len || !q_len || !out) return TV_ERR_INVALID;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(parent) & 3u) || (reinterpret_cast<uintptr_t>(prefix_len) & 3u) ||
      (reinterpret_cast<uintptr_t>(q_len) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return TV_ERR_INVALID;
  if (!isfinite(sm_scale)) return TV_ERR_INVALID;
  if (workspace_bytes < plan.ws_bytes || workspace == nullptr || !aligned16(workspace)) return TV_ERR_INVALID;
  char* ws = static_cast<char*>(workspace);
  a = tv::AttnArgs{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.parent = parent;
  a.out = out;
  a.lse = lse;
  a.req = reinterpret_cast<const int32_t*>(ws);
  a.merge_tab = reinterpret_cast<const int4*>(ws + tv::merge_table_word0(B) * sizeof(int32_t));
  a.queue = reinterpret_cast<int*>(ws + tv::queue_word0(B, plan.merge_blocks) * sizeof(int32_t));
  a.ws_o = reinterpret_cast<float*>(ws + plan.ws_o_off);
  a.ws_m = reinterpret_cast<float*>(ws + plan.ws_m_off);
  a.ws_l = reinterpret_cast<float*>(ws + plan.ws_l_off);
  a.B = B;
  a.H = H;
  a.q_len = max_q_len;
  a.prefix_len = kv_stride - max_q_len;
  a.kv_len = kv_stride;
  a.R = max_q_len * H;
  a.rows_per_block = plan.rows_per_block;
  a.n_rb = plan.n_rb;
  a.full_rb = plan.full_rb;
  a.split_full = plan.split_full;
  a.chunk_full = plan.chunk_full;
  a.split_tail = plan.split_tail;
  a.chunk_tail = plan.chunk_tail;
  a.sm_scale = sm_scale;
  a.kv_stride = kv_stride;
  a.n_nodes = n_nodes;
  return TV_OK;
}

}  // namespace

extern "C" {

size_t tv_verify_attn_ragged_workspace_size(int32_t B, int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c,
                                            int32_t d_r, tv_dtype_t kv_dtype) {
  tv::AttnShape s;
  tv::AttnPlan plan;
  if (plan_ragged(B, H, max_q_len, kv_stride, d_c, d_r, kv_dtype, s, plan) != TV_OK) return 0;
  return plan.ws_bytes;
}

tv_status_t tv_verify_attn_ragged(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                                  const int32_t* parent, const int32_t* prefix_len, const int32_t* q_len,
                                  int32_t n_nodes, int32_t B,
                                  int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r,
                                  tv_dtype_t kv_dtype, float sm_scale, float* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  tv::AttnShape s;
  tv::AttnPlan plan;
  tv::AttnArgs a;
  const tv_status_t st = ragged_args(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, n_nodes, B, H, max_q_len,
                                     kv_stride, d_c, d_r, kv_dtype, sm_scale, out, lse, workspace, workspace_bytes, s,
                                     plan, a);
  if (st != TV_OK) return st;
  if (tv::launch_ragged_prep(s, plan, a, prefix_len, q_len, stream) != hipSuccess) return TV_ERR_LAUNCH;
  return tv::launch_attention(s, plan, a, stream) == hipSuccess ? TV_OK : TV_ERR_LAUNCH;
}

tv_status_t tv_verify_step_ragged(const float* q_lat, float* q_rope, const void* c_kv, void* k_rope,
                                  const int32_t* parent, const int32_t* prefix_len, const int32_t* q_len,
                                  int32_t n_nodes, int32_t B,
                                  int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r,
                                  tv_dtype_t kv_dtype, double theta, float sm_scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!(theta > 0.0) || !isfinite(theta)) return TV_ERR_INVALID;
  if (d_r > 2 * tv::kMaxHalf) return TV_ERR_UNSUPPORTED;
  tv::AttnShape s;
  tv::AttnPlan plan;
  tv::AttnArgs a;
  const tv_status_t st = ragged_args(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, q_len, n_nodes, B, H, max_q_len,
                                     kv_stride, d_c, d_r, kv_dtype, sm_scale, out, lse, workspace, workspace_bytes, s,
                                     plan, a);
  if (st != TV_OK) return st;
  if (tv::launch_ragged_prep(s, plan, a, prefix_len, q_len, stream) != hipSuccess) return TV_ERR_LAUNCH;
  const tv::RopeFreq f = make_freq(d_r, theta);
  if (tv::launch_tree_rope_ragged(q_rope, k_rope, kv_dtype == TV_BF16, parent, a.req, B, max_q_len, H, d_r,
                                  kv_stride, f, stream) != hipSuccess)
    return TV_ERR_LAUNCH;
  return tv::launch_attention(s, plan, a, stream) == hipSuccess ? TV_OK : TV_ERR_LAUNCH;
}

const char* tv_status_str(tv_status_t s) {
  switch (s) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID: return "TV_ERR_INVALID: invalid argument";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: shape or dtype not supported";
    case TV_ERR_LAUNCH: return "TV_ERR_LAUNCH: kernel launch failed";
  }
  return "TV_ERR_UNKNOWN";
}

tv_status_t tv_tree_positions(const int32_t* parent, int32_t B, int32_t q_len, int32_t prefix_len, int32_t* pos,
                              hipStream_t stream) {
  if (!parent || !pos || B < 1 || q_len < 1 || prefix_len < 0) return TV_ERR_INVALID;
  if (q_len > TV_MAX_Q_LEN) return TV_ERR_UNSUPPORTED;
  if (prefix_len > INT32_MAX - TV_MAX_Q_LEN) return TV_ERR_INVALID;
  return tv::launch_tree_positions(parent, B, q_len, prefix_len, pos, stream) == hipSuccess ? TV_OK
                                                                                            : TV_ERR_LAUNCH;
}

tv_status_t tv_rope_neox_strided(void* x, tv_dtype_t dtype, const int32_t* pos, int32_t n_seq, int32_t n_tok,
                                 int32_t n_head, int32_t d_r, int64_t seq_stride, int64_t tok_stride,
                                 int64_t pos_seq_stride, double theta, hipStream_t stream) {
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID;
  if (n_seq < 0 || n_tok < 0 || n_head < 1 || d_r < 2 || (d_r & 1)) return TV_ERR_INVALID;
  if (d_r > 2 * tv::kMaxHalf) return TV_ERR_UNSUPPORTED;
  if (!(theta > 0.0) || !isfinite(theta)) return TV_ERR_INVALID;
  if (n_seq == 0 || n_tok == 0) return TV_OK;
  if (!x || seq_stride < 0 || tok_stride < 0 || pos_seq_stride < 0) return TV_ERR_INVALID;
  if (!aligned16(x) || (pos && (reinterpret_cast<uintptr_t>(pos) & 3u))) return TV_ERR_INVALID;
  if (static_cast<int64_t>(n_seq) * n_tok * n_head * (d_r / 2) > kMaxRopePairs) return TV_ERR_UNSUPPORTED;
  const tv::RopeFreq f = make_freq(d_r, theta);
  return tv::launch_rope_neox(x, dtype == TV_BF16, pos, n_seq, n_tok, n_head, d_r, seq_stride, tok_stride,
                              pos_seq_stride, f, stream) == hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

tv_status_t tv_rope_neox(void* x, tv_dtype_t dtype, const int32_t* pos, int64_t n_tok, int32_t n_head,
                         int32_t d_r, int64_t tok_stride, double theta, hipStream_t stream) {
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID;
  if (n_tok < 0 || n_head < 1 || d_r < 2 || (d_r & 1)) return TV_ERR_INVALID;
  if (d_r > 2 * tv::kMaxHalf) return TV_ERR_UNSUPPORTED;
  if (!(theta > 0.0) || !isfinite(theta)) return TV_ERR_INVALID;
  if (n_tok == 0) return TV_OK;
  if (!x || tok_stride < 0) return TV_ERR_INVALID;
  if (!aligned16(x) || (pos && (reinterpret_cast<uintptr_t>(pos) & 3u))) return TV_ERR_INVALID;
  if (n_tok > kMaxRopePairs / (static_cast<int64_t>(n_head) * (d_r / 2))) return TV_ERR_UNSUPPORTED;
  const tv::RopeFreq f = make_freq(d_r, theta);
  // One sequence of n_tok tokens.
  return tv::launch_rope_neox(x, dtype == TV_BF16, pos, 1, n_tok, n_head, d_r, 0, tok_stride, 0, f, stream) ==
                 hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

size_t tv_verify_attn_ex_workspace_size(int32_t B, int32_t H, int32_t q_len, int32_t prefix_len, int32_t d_c,
                                        int32_t d_r, tv_dtype_t kv_dtype, uint32_t flags) {
  if (flags & ~kAttnFlags) return 0;
  if (check_attn_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype) != TV_OK) return 0;
  return tv::plan_attention(make_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype, flags)).ws_bytes;
}

size_t tv_verify_attn_workspace_size(int32_t B, int32_t H, int32_t q_len, int32_t prefix_len, int32_t d_c,
                                     int32_t d_r, tv_dtype_t kv_dtype) {
  return tv_verify_attn_ex_workspace_size(B, H, q_len, prefix_len, d_c, d_r, kv_dtype, 0);
}

tv_status_t tv_verify_attn_ex(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                              const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                              int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, uint32_t flags,
                              float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (flags & ~kAttnFlags) return TV_ERR_INVALID;
  const tv_status_t st = check_attn_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype);
  if (st != TV_OK) return st;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !parent || !out) return TV_ERR_INVALID;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(parent) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return TV_ERR_INVALID;
  if (!isfinite(sm_scale)) return TV_ERR_INVALID;
  return run_attention(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, B, H, q_len, d_c, d_r, kv_dtype, sm_scale,
                       out, lse, workspace, workspace_bytes, stream, flags);
}

tv_status_t tv_verify_attn(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                           const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                           int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return tv_verify_attn_ex(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, B, H, q_len, d_c, d_r, kv_dtype,
                           sm_scale, 0, out, lse, workspace, workspace_bytes, stream);
}

tv_status_t tv_verify_attn_noalloc(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                                   const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                                   int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, float* out,
                                   float* lse, hipStream_t stream) {
  const tv_status_t st = check_attn_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype);
  if (st != TV_OK) return st;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !parent || !out) return TV_ERR_INVALID;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(parent) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return TV_ERR_INVALID;
  if (!isfinite(sm_scale)) return TV_ERR_INVALID;
  const size_t need = tv::plan_attention(make_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype)).ws_bytes;
  if (need > TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return TV_ERR_LAUNCH;
  }
  return run_attention(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, B, H, q_len, d_c, d_r, kv_dtype, sm_scale,
                       out, lse, ws, TV_NOALLOC_SCRATCH_BYTES, stream);
}

tv_status_t tv_tree_rope(float* q_rope, void* k_rope, tv_dtype_t kv_dtype, const int32_t* parent,
                         int32_t prefix_len, int32_t B, int32_t H, int32_t q_len, int32_t d_r, double theta,
                         hipStream_t stream) {
  if (kv_dtype != TV_F32 && kv_dtype != TV_BF16) return TV_ERR_INVALID;
  if (B < 1 || H < 1 || q_len < 1 || prefix_len < 0 || d_r < 2 || (d_r & 1)) return TV_ERR_INVALID;
  if (q_len > TV_MAX_Q_LEN || d_r > 2 * tv::kMaxHalf) return TV_ERR_UNSUPPORTED;
  if (prefix_len > INT32_MAX - TV_MAX_Q_LEN) return TV_ERR_INVALID;
  if (static_cast<int64_t>(q_len) * (H + 1) * (d_r / 2) > INT32_MAX) return TV_ERR_UNSUPPORTED;
  if (!(theta > 0.0) || !isfinite(theta)) return TV_ERR_INVALID;
  if (!q_rope || !k_rope || !parent) return TV_ERR_INVALID;
  if (!aligned16(q_rope) || !aligned16(k_rope) || (reinterpret_cast<uintptr_t>(parent) & 3u)) return TV_ERR_INVALID;
  const tv::RopeFreq f = make_freq(d_r, theta);
  return tv::launch_tree_rope(q_rope, k_rope, kv_dtype == TV_BF16, parent, B, q_len, H, d_r, prefix_len, f, stream) ==
                 hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

tv_status_t tv_verify_step(const float* q_lat, float* q_rope, const void* c_kv, void* k_rope,
                           const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                           int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, double theta, float sm_scale,
                           float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const tv_status_t st = check_attn_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype);
  if (st != TV_OK) return st;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !parent || !out) return TV_ERR_INVALID;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(parent) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return TV_ERR_INVALID;
  if (!isfinite(sm_scale) || !(theta > 0.0) || !isfinite(theta)) return TV_ERR_INVALID;
  const tv::AttnPlan plan = tv::plan_attention(make_shape(prefix_len, B, H, q_len, d_c, d_r, kv_dtype));
  if (workspace_bytes < plan.ws_bytes || (plan.ws_bytes > 0 && (workspace == nullptr || !aligned16(workspace))))
    return TV_ERR_INVALID;
  const tv_status_t rs = tv_tree_rope(q_rope, k_rope, kv_dtype, parent, prefix_len, B, H, q_len, d_r, theta, stream);
  if (rs != TV_OK) return rs;
  return run_attention(q_lat, q_rope, c_kv, k_rope, parent, prefix_len, B, H, q_len, d_c, d_r, kv_dtype, sm_scale,
                       out, lse, workspace, workspace_bytes, stream);
}

tv_status_t tv_argmax_rows(const void* logits, tv_dtype_t dtype, int64_t n_rows, int32_t vocab, int32_t* out,
                           hipStream_t stream) {
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_INVALID;
  if (n_rows < 0 || vocab < 1) return TV_ERR_INVALID;
  if (n_rows > INT32_MAX) return TV_ERR_UNSUPPORTED;
  if (n_rows == 0) return TV_OK;
  if (!logits || !out || (reinterpret_cast<uintptr_t>(out) & 3u)) return TV_ERR_INVALID;
  const int elem = dtype == TV_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) & static_cast<uintptr_t>(elem - 1)) return TV_ERR_INVALID;
  // 16-byte loads when every row starts 16-byte aligned and is whole 16-byte chunks.
  const bool vec = aligned16(logits) && (static_cast<int64_t>(vocab) * elem) % 16 == 0;
  return tv::launch_argmax_rows(logits, dtype == TV_BF16, vec, n_rows, vocab, out, stream) == hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

tv_status_t tv_tree_accept(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok, int32_t B,
                           int32_t q_len, int32_t* path, int32_t* accept_len, int32_t* bonus_tok, hipStream_t stream) {
  if (B < 1 || q_len < 1) return TV_ERR_INVALID;
  if (q_len > TV_MAX_Q_LEN) return TV_ERR_UNSUPPORTED;
  const void* ptrs[] = {parent, draft_tok, target_tok, path, accept_len, bonus_tok};
  for (const void* p : ptrs)
    if (!p || (reinterpret_cast<uintptr_t>(p) & 3u)) return TV_ERR_INVALID;
  return tv::launch_tree_accept(parent, draft_tok, target_tok, B, q_len, path, accept_len, bonus_tok, stream) ==
                 hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

tv_status_t tv_kv_compact(void* c_kv, void* k_rope, tv_dtype_t kv_dtype, const int32_t* path,
                          const int32_t* accept_len, int32_t prefix_len, int32_t B, int32_t kv_len, int32_t q_len,
                          int32_t d_c, int32_t d_r, hipStream_t stream) {
  if (kv_dtype != TV_F32 && kv_dtype != TV_BF16) return TV_ERR_INVALID;
  if (B < 1 || q_len < 1 || prefix_len < 0 || d_c < 1 || d_r < 1) return TV_ERR_INVALID;
  if (q_len > TV_MAX_Q_LEN) return TV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(prefix_len) + q_len > kv_len) return TV_ERR_INVALID;
  const int elem = kv_dtype == TV_BF16 ? 2 : 4;
  if ((d_c * elem) % 16 != 0 || (d_r * elem) % 16 != 0) return TV_ERR_UNSUPPORTED;
  if (!c_kv || !k_rope || !path || !accept_len) return TV_ERR_INVALID;
  if (!aligned16(c_kv) || !aligned16(k_rope) || (reinterpret_cast<uintptr_t>(path) & 3u) ||
      (reinterpret_cast<uintptr_t>(accept_len) & 3u))
    return TV_ERR_INVALID;
  return tv::launch_kv_compact(c_kv, k_rope, elem, path, accept_len, prefix_len, B, kv_len, q_len, d_c, d_r,
                               stream) == hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

tv_status_t tv_tree_build(const float* logp, const int32_t* cand_tok, const int32_t* root_tok, int32_t B, int32_t D,
                          int32_t K, int32_t budget, int32_t* parent, int32_t* token, int32_t* depth, float* score,
                          int32_t* n_nodes, hipStream_t stream) {
  if (B < 1 || D < 1 || K < 1 || budget < 0) return TV_ERR_INVALID;
  if (K > 64 || budget > TV_MAX_BUILD_BUDGET) return TV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(D < budget ? D : budget) * K > TV_MAX_BUILD_CANDIDATES) return TV_ERR_UNSUPPORTED;
  const void* ptrs[] = {logp, cand_tok, root_tok, parent, token, depth, score, n_nodes};
  for (const void* p : ptrs)
    if (!p || (reinterpret_cast<uintptr_t>(p) & 3u)) return TV_ERR_INVALID;
  return tv::launch_tree_build(logp, cand_tok, root_tok, B, D, K, budget, parent, token, depth, score, n_nodes,
                               stream) == hipSuccess
             ? TV_OK
             : TV_ERR_LAUNCH;
}

}  // extern "C"
