// Internal launch interface between the C ABI (tv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tv_device.h"

namespace tv {

constexpr int kMaxQ = 64;     // one 64-bit ancestor word per tree node
constexpr int kMaxHalf = 64;  // d_r <= 128

// inv_freq[k] = 1 / theta^(2k/d_r), computed on the host in float64 and passed
// by value so every thread of a launch uses the same table.
struct RopeFreq {
  double inv_freq[kMaxHalf];
};

hipError_t launch_rope_neox(void* x, bool bf16, const int32_t* pos, int n_seq, int n_tok, int n_head, int d_r,
                            int64_t seq_stride, int64_t tok_stride, int64_t pos_seq_stride, const RopeFreq& f,
                            hipStream_t stream);
hipError_t launch_tree_positions(const int32_t* parent, int B, int q_len, int prefix_len, int32_t* pos,
                                 hipStream_t stream);
hipError_t launch_tree_rope(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, int B, int q_len, int H,
                            int d_r, int prefix_len, const RopeFreq& f, hipStream_t stream);

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------
enum class AttnKernel : int { kValu = 0, kMfmaBf16 = 1, kMfmaF32 = 2 };

// How one tv_verify_attn call is cut into workgroups.  A pure function of the
// shapes (never of the device), so the workspace size can be asked for ahead.
struct AttnPlan {
  AttnKernel kernel;
  int rows_per_block;  // query rows (node, head) per workgroup
  int keys_per_tile;   // kv rows staged per LDS tile
  int n_rb;            // row blocks per batch entry
  int n_split;         // kv splits (1 = no merge pass)
  int chunk;           // kv rows per split (multiple of keys_per_tile)
  size_t ws_bytes;     // workspace for split partials
  size_t ws_o_off, ws_m_off, ws_l_off;
};

struct AttnShape {
  int B, H, q_len, prefix_len, kv_len, d_c, d_r;
  bool kv_bf16;
};

AttnPlan plan_attention(const AttnShape& s);

struct AttnArgs {
  const float* q_lat;
  const float* q_rope;
  const void* c_kv;
  const void* k_rope;
  const int32_t* parent;
  float* out;
  float* lse;
  float* ws_o;  // [n_split][B][R][d_c]
  float* ws_m;  // [n_split][B][R]
  float* ws_l;  // [n_split][B][R]
  int B, H, q_len, prefix_len, kv_len, R, n_rb, n_split, chunk;
  float sm_scale;
};

hipError_t launch_attention(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);

}  // namespace tv
