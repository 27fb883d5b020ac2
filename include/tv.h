/*
 * tv.h — C ABI of libtv.so: tree-verify MLA-absorb attention on MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [RoPE page]   "Precision as Correctness: The Float64 RoPE Decision in a
 *                 Custom CUDA Inference Engine"
 *   [Verify page] "The Precision Imperative: Validating Numerical Accuracy in a
 *                 Custom CUDA Attention Kernel"
 *   [Golden page] "The Golden Reference: A Pivotal Moment in Building a Native
 *                 DDTree Inference Engine"
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or keeps caller memory, and holds no global mutable
 *     state: concurrent calls on different streams are safe.
 *   - Calls are asynchronous: work is enqueued on `stream` (NULL = the null
 *     stream) and nothing is synchronised.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns TV_ERR_INVALID (malformed) or TV_ERR_UNSUPPORTED (well
 *     formed but outside what the kernels implement) and launches nothing.
 *     TV_ERR_LAUNCH reports a failed kernel launch.  No C++ exception crosses
 *     the ABI.
 *   - Tensors are dense and row-major with the shapes given below, and every
 *     pointer is 16-byte aligned.
 *   - The tree of each batch entry is a parent array parent[b][0..q_len):
 *     node 0 is the root (parent -1) and every other node's parent is an
 *     earlier node (0 <= parent[i] < i).  Node m's key/latent row sits at kv
 *     index prefix_len + m, so kv_len = prefix_len + q_len (the kv_len of each
 *     test shape on the Verify page, "The Message in Full").  A parent outside
 *     [0, i) is not detected on the device; the kernels treat such a node as a
 *     child of nobody (it sees the prefix and itself), so no access leaves the
 *     buffers.
 */
#ifndef TV_H
#define TV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_INVALID = 1,     /* null pointer, bad size, misaligned pointer, too small workspace */
  TV_ERR_UNSUPPORTED = 2, /* shape or dtype outside what the kernels implement */
  TV_ERR_LAUNCH = 3       /* a kernel launch failed (hipGetLastError) */
} tv_status_t;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype_t;

/* Largest tree (nodes per request, root included): four 64-bit ancestor
 * words per node. */
#define TV_MAX_Q_LEN 256

/* Largest draft budget of tv_tree_build (a tree of TV_MAX_Q_LEN nodes with
 * its root), and the most ranked candidates it holds: min(D, budget) * K. */
#define TV_MAX_BUILD_BUDGET (TV_MAX_Q_LEN - 1)
#define TV_MAX_BUILD_CANDIDATES 8192

/* Human-readable name of a status code (static string, never NULL). */
const char* tv_status_str(tv_status_t s);

/*
 * tv_tree_positions — rotary position of every tree node.
 *   pos[b][i] = prefix_len + depth(i), depth(root) = 0: siblings share a
 *   position and a chain gives prefix_len + i.  (The pages leave node
 *   positions implicit; the Golden page, "Recursive Refinement of the Decode
 *   Loop Design", has the engine track positions of the root and draft tokens.
 *   Depth-based positions are the reading under which a chain tree is exactly
 *   causal decoding.)
 *   parent [B][q_len] int32 (device), pos [B][q_len] int32 (device, written).
 *   1 <= q_len <= TV_MAX_Q_LEN, B >= 1, prefix_len >= 0.
 */
tv_status_t tv_tree_positions(const int32_t* parent, int32_t B, int32_t q_len, int32_t prefix_len,
                              int32_t* pos, hipStream_t stream);

/*
 * tv_rope_neox — in-place NeoX rotary embedding with float64 angles.
 *   [RoPE page, "The Message", "The Float64 Decision", "What Input Knowledge
 *   Is Required" item 1]
 *   x is viewed as [n_tok][n_head][d_r] elements of `dtype`: token t's heads
 *   start at element t * tok_stride and are contiguous rows of d_r elements.
 *   Token t turns at position p = pos[t] (pos: int32 [n_tok], device), or at
 *   p = t when pos is NULL.  For k < d_r/2 the pair (x[k], x[k + d_r/2]) turns
 *   by the angle p * inv_freq[k], inv_freq[k] = 1 / theta^(2k/d_r); angle,
 *   cos, sin and the rotation are float64 and the result is rounded once
 *   (nearest-even) to dtype.
 *   d_r even, 2 <= d_r <= 128; n_tok >= 0 (0 = nothing to do); n_head >= 1;
 *   tok_stride >= 0; theta > 0.  x 16-byte aligned, pos 4-byte aligned.
 *   n_tok * n_head * d_r / 2 above 2^40 returns TV_ERR_UNSUPPORTED.
 */
tv_status_t tv_rope_neox(void* x, tv_dtype_t dtype, const int32_t* pos, int64_t n_tok, int32_t n_head,
                         int32_t d_r, int64_t tok_stride, double theta, hipStream_t stream);

/*
 * tv_rope_neox_strided — tv_rope_neox over a batch of sequences, for strided
 *   views such as a slice of a cache.  [RoPE page, as for tv_rope_neox]
 *   x is viewed as [n_seq][n_tok][n_head][d_r] elements of `dtype` with element
 *   strides seq_stride (between sequences) and tok_stride (between tokens);
 *   heads are contiguous rows of d_r elements.  Token t of sequence s turns at
 *   position p = pos[s * pos_seq_stride + t], or p = t when pos is NULL; the
 *   rotation is that of tv_rope_neox.
 *   d_r even, 2 <= d_r <= 128; n_seq, n_tok >= 0 (0 = nothing to do); n_head >= 1;
 *   strides >= 0; theta > 0.
 */
tv_status_t tv_rope_neox_strided(void* x, tv_dtype_t dtype, const int32_t* pos, int32_t n_seq, int32_t n_tok,
                                 int32_t n_head, int32_t d_r, int64_t seq_stride, int64_t tok_stride,
                                 int64_t pos_seq_stride, double theta, hipStream_t stream);

/*
 * tv_verify_attn — tree-verify attention in MLA absorb form.
 *   [Verify page, "The Context: What Led to This Moment" (visibility-masked
 *   absorb attention: scores, normalisation, weighted accumulation);
 *   Golden page, "The Absorb Form of MLA" and "Principled Abstraction"]
 *   For batch b, node i, head h (row r = i*H + h of the batch):
 *     s_j   = sm_scale * (q_lat[b,i,h,:] . c_kv[b,j,:] + q_rope[b,i,h,:] . k_rope[b,j,:])
 *     vis_j = j < prefix_len, or j - prefix_len is node i or an ancestor of i
 *     out[b,i,h,:] = sum_j softmax_j(s over visible j) * c_kv[b,j,:]
 *     lse[b,i,h]   = log sum_{visible j} exp(s_j)
 *   The rope slices must already be rotated (tv_rope_neox).  The output stays
 *   in latent space (the value up-projection is not applied).
 *   Shapes (kv_len = prefix_len + q_len):
 *     q_lat  [B][q_len][H][d_c] f32      q_rope [B][q_len][H][d_r] f32
 *     c_kv   [B][kv_len][d_c] kv_dtype   k_rope [B][kv_len][d_r] kv_dtype
 *     parent [B][q_len] int32
 *     out    [B][q_len][H][d_c] f32      lse    [B][q_len][H] f32, or NULL
 *   Supported (d_c, d_r, kv_dtype): d_c in {64, 128, 256, 512}, d_r in {32, 64},
 *   kv_dtype TV_F32 or TV_BF16.  1 <= q_len <= TV_MAX_Q_LEN.  One tree's
 *   latent rows (kv_len * d_c elements of kv_dtype) must stay below 2^31
 *   bytes (TV_ERR_UNSUPPORTED otherwise).
 *   Arithmetic: with a bf16 cache at (512, 64) both contractions run on
 *   16-bit matrix cores.  Scores: each scaled query x = sm_scale * log2(e) * q
 *   (rounded to fp32) enters as two bf16 terms, hi = bf16(x) and
 *   lo = bf16(x - hi), so the scores are those of the fp32 queries to fp32
 *   accumulation.  Values: the softmax weights are rounded to fp16, and the
 *   latent rows are converted from bf16 to fp16: exactly for magnitudes from
 *   2^-17 to 65504, smaller ones rounded to fp16's 2^-24 spacing (fp32
 *   accumulation, row sums of the rounded weights).  Latent cache values of
 *   magnitude 65520 or more are outside this path's range and give
 *   non-finite outputs (use an fp32 cache for such data).
 *   With an fp32 cache at (512, 64) on fp32 matrix cores; other shapes on the
 *   fp32 vector ALU.  The sums run in a different order than the plain
 *   definition.
 *   workspace: caller-owned device scratch of at least
 *   tv_verify_attn_workspace_size(...) bytes (NULL allowed when that is 0).
 *   out must not overlap any input.
 */
tv_status_t tv_verify_attn(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                           const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                           int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tv_verify_attn_noalloc — tv_verify_attn with no workspace argument, for
 *   callers that cannot allocate device memory (code under HIP graph capture,
 *   tight serving loops, harnesses that forbid allocation).  It allocates
 *   nothing: the split-kv partial results go to a static device array of
 *   TV_NOALLOC_SCRATCH_BYTES in the library (one per device, held until the
 *   process ends; its address is looked up on a device's first call).
 *   Arguments, results and kernels are those of tv_verify_attn.
 *   Shapes whose tv_verify_attn_workspace_size exceeds TV_NOALLOC_SCRATCH_BYTES
 *   return TV_ERR_UNSUPPORTED before anything else happens.  Every call on a
 *   device shares that device's array (nothing in it needs to start at zero):
 *   calls that overlap on one device -- on different streams or threads --
 *   race and give wrong results; serialise them.
 */
#define TV_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
tv_status_t tv_verify_attn_noalloc(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                                   const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                                   int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, float* out,
                                   float* lse, hipStream_t stream);

/*
 * tv_verify_attn_ex — tv_verify_attn with option flags (0 gives tv_verify_attn
 *   exactly).  [Verify page, as for tv_verify_attn]
 *   TV_ATTN_BF16_QUERIES: with a bf16 cache at (512, 64), round each scaled
 *   query to ONE bf16 term and the softmax weights to bf16, with the values
 *   in bf16 (a single score pass over twice the rows per workgroup: faster,
 *   and no range limit on the latent cache, but every score moves by up to
 *   2^-9 of its terms and every weight by 2^-9; right when the queries are
 *   bf16 values already, or when that error is acceptable).  No effect on
 *   other shapes.
 *   TV_ATTN_F32_WIDE: with an fp32 cache at (512, 64), run every batch on
 *   the 64-row workgroups.  By default a batch of at most 128 such row
 *   blocks runs on 32-row workgroups that split each unit's keys in two
 *   halves (combined by log-sum-exp weights); both forms compute the same
 *   products in fp32 and agree to fp32 rounding.  For comparisons; no effect
 *   on other shapes.
 *   Unknown flag bits return TV_ERR_INVALID.  The workspace must hold
 *   tv_verify_attn_ex_workspace_size(..., flags) bytes.
 */
#define TV_ATTN_BF16_QUERIES 1u
#define TV_ATTN_F32_WIDE 2u
tv_status_t tv_verify_attn_ex(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                              const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                              int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, float sm_scale, uint32_t flags,
                              float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes of tv_verify_attn_ex with these flags (0 for bad flags). */
size_t tv_verify_attn_ex_workspace_size(int32_t B, int32_t H, int32_t q_len, int32_t prefix_len, int32_t d_c,
                                        int32_t d_r, tv_dtype_t kv_dtype, uint32_t flags);

/* Bytes of workspace tv_verify_attn / tv_verify_step need for these shapes
 * (split-kv partial results); 0 when the launch needs none.  Depends on the
 * shapes only, never on the device. */
size_t tv_verify_attn_workspace_size(int32_t B, int32_t H, int32_t q_len, int32_t prefix_len, int32_t d_c,
                                     int32_t d_r, tv_dtype_t kv_dtype);

/*
 * tv_verify_attn_ragged — tv_verify_attn for a batch whose requests have their
 *   own prefix length and tree size.  Each request's result is exactly that
 *   of tv_verify_attn on it alone [Verify page, "The Context: What Led to This
 *   Moment" (the tree-verify attention)]; batching requests of different
 *   lengths in one launch is this library's addition, not a step the pages
 *   describe.
 *   Per-request lengths are in DEVICE memory: prefix_len[B], q_len[B] int32,
 *   with 0 <= q_len[b] <= max_q_len and prefix_len[b] + q_len[b] <= kv_stride
 *   (lengths outside are clamped into these bounds; q_len 0 means nothing to
 *   do).  Nodes are packed request after request: request b's nodes start at
 *   node s_b = q_len[0] + ... + q_len[b-1] in
 *     q_lat [n_nodes][H][d_c], q_rope [n_nodes][H][d_r] f32, parent [n_nodes]
 *     int32 (node indices local to the request, as for tv_verify_attn), out
 *     [n_nodes][H][d_c] f32, lse [n_nodes][H] f32 (optional).
 *   n_nodes (host value, >= 0) is the caller's row count of those buffers:
 *   the kernels never touch a node at or past it.  If the device lengths sum
 *   to more, the request that crosses n_nodes keeps only its nodes below it
 *   and the requests after it get q_len 0 (their rows are not computed);
 *   rows from the sum of the lengths up to n_nodes are not touched;
 *   the cache holds kv_stride rows per request, the first prefix_len[b] +
 *   q_len[b] of which are used: c_kv [B][kv_stride][d_c], k_rope
 *   [B][kv_stride][d_r] (kv_dtype), rope slices already rotated.
 *   Workspace (device, 16-byte aligned, caller-owned, reused across calls on
 *   one stream): at least tv_verify_attn_ragged_workspace_size(...) bytes; it
 *   always holds the per-request records and the merge table (the slots and
 *   rows of each row block cut into kv pieces) that a small prep kernel
 *   writes from the device lengths, then the split partials.  Launch sizes come from the
 *   bounds, so nothing is read back to the host and the call can be captured
 *   in a graph.  1 <= max_q_len <= TV_MAX_Q_LEN; kv_stride >= max_q_len;
 *   other limits as for tv_verify_attn with prefix_len = kv_stride -
 *   max_q_len.
 */
tv_status_t tv_verify_attn_ragged(const float* q_lat, const float* q_rope, const void* c_kv, const void* k_rope,
                                  const int32_t* parent, const int32_t* prefix_len, const int32_t* q_len,
                                  int32_t n_nodes, int32_t B,
                                  int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r,
                                  tv_dtype_t kv_dtype, float sm_scale, float* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * tv_verify_step_ragged — the whole step for a ragged batch: each request's
 *   query rows and tree key rows rotated in place at prefix_len[b] + depth
 *   (as tv_tree_rope does for one request), then tv_verify_attn_ragged.
 *   Arguments as for tv_verify_attn_ragged plus theta; q_rope and k_rope are
 *   modified (only the rows of nodes below n_nodes after the clamp above).
 *   The request records are computed once and serve both steps.
 */
tv_status_t tv_verify_step_ragged(const float* q_lat, float* q_rope, const void* c_kv, void* k_rope,
                                  const int32_t* parent, const int32_t* prefix_len, const int32_t* q_len,
                                  int32_t n_nodes, int32_t B,
                                  int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c, int32_t d_r,
                                  tv_dtype_t kv_dtype, double theta, float sm_scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes tv_verify_attn_ragged and tv_verify_step_ragged need for
 * these bounds (0 if the shape is invalid or unsupported). */
size_t tv_verify_attn_ragged_workspace_size(int32_t B, int32_t H, int32_t max_q_len, int32_t kv_stride, int32_t d_c,
                                            int32_t d_r, tv_dtype_t kv_dtype);

/*
 * tv_tree_rope — the step's rotation: for every tree b and node i, turn the
 *   query rows q_rope[b,i,h,:] (all heads) and the tree's own key row
 *   k_rope[b, prefix_len+i, :] in place at position prefix_len + depth(i), as
 *   tv_tree_positions and tv_rope_neox define them (one fused launch; the
 *   positions never reach memory).
 *   q_rope [B][q_len][H][d_r] f32, k_rope [B][prefix_len+q_len][d_r] kv_dtype,
 *   parent [B][q_len] int32.  d_r even, 2 <= d_r <= 128; 1 <= q_len <= TV_MAX_Q_LEN.
 */
tv_status_t tv_tree_rope(float* q_rope, void* k_rope, tv_dtype_t kv_dtype, const int32_t* parent,
                         int32_t prefix_len, int32_t B, int32_t H, int32_t q_len, int32_t d_r, double theta,
                         hipStream_t stream);

/*
 * tv_verify_step — the whole verify step for one batch of trees:
 *   1. tv_tree_rope (queries and the tree's own key rows, in place), then
 *   2. tv_verify_attn on the result.
 *   The prefix key rows k_rope[b, 0:prefix_len) are taken as already rotated
 *   (the cache holds keys rotated when they were written).  Arguments as in
 *   tv_verify_attn, plus theta; q_rope and k_rope are modified.
 */
tv_status_t tv_verify_step(const float* q_lat, float* q_rope, const void* c_kv, void* k_rope,
                           const int32_t* parent, int32_t prefix_len, int32_t B, int32_t H, int32_t q_len,
                           int32_t d_c, int32_t d_r, tv_dtype_t kv_dtype, double theta, float sm_scale,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * tv_argmax_rows — the target's greedy token per tree node: for each of n_rows
 *   rows of logits [n_rows][vocab] (dtype TV_F32 or TV_BF16, row-major, dense),
 *   out[r] = the index of the row's largest value, the lowest index on ties; a
 *   NaN counts as larger than every number (the first NaN wins) and -0.0 equals
 *   +0.0.  [RoPE page, "The Broader Context: A Full Native Engine from Scratch"
 *   (greedy tree accept; the loop's greedy output must match autoregressive
 *   greedy output)]
 *   logits must be aligned to its element size; 16-byte aligned rows whose byte
 *   length is a multiple of 16 take a vectorised path.  out: int32 [n_rows],
 *   4-byte aligned.  n_rows = 0 is a no-op; n_rows > INT32_MAX returns
 *   TV_ERR_UNSUPPORTED.
 */
tv_status_t tv_argmax_rows(const void* logits, tv_dtype_t dtype, int64_t n_rows, int32_t vocab, int32_t* out,
                           hipStream_t stream);

/*
 * tv_tree_accept — greedy acceptance of each batch entry's draft tree.
 *   [RoPE page, "The Broader Context: A Full Native Engine from Scratch";
 *   Golden page, "Context: The Quest for a Hyper-Optimized Inference Stack"
 *   (greedy tree-accept kernel) and "Recursive Refinement of the Decode Loop
 *   Design" (root, draft and bonus tokens)]
 *   Node 0 (the root) is already committed.  From the current node cur the
 *   target's next token is target_tok[b][cur]; the walk moves to the child of
 *   cur (parent[b][c] == cur) whose draft_tok[b][c] equals it -- the lowest
 *   index c if several do -- and stops when none does.
 *   Inputs (int32, [B][q_len], 4-byte aligned): parent (as for tv_verify_attn;
 *   a node whose parent is outside [0, i) is never accepted), draft_tok (entry
 *   0 is the root's token and is not compared), target_tok (the target's
 *   greedy token after each node, e.g. from tv_argmax_rows).
 *   Outputs: path [B][q_len] int32: path[b][0] = 0, then the accepted nodes in
 *   order, then -1; accept_len [B] int32: accepted draft nodes; bonus_tok [B]
 *   int32: target_tok at the last accepted node.  The step commits the draft
 *   tokens of path[b][1..accept_len] and then bonus_tok.
 *   1 <= q_len <= TV_MAX_Q_LEN.
 */
tv_status_t tv_tree_accept(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok, int32_t B,
                           int32_t q_len, int32_t* path, int32_t* accept_len, int32_t* bonus_tok, hipStream_t stream);

/*
 * tv_kv_compact — post-verify compaction of the latent cache, in place.
 *   [RoPE page, "The Broader Context: A Full Native Engine from Scratch" (KV
 *   cache with post-verify compaction)]
 *   For each b and k = 1 .. accept_len[b]: row prefix_len + k of c_kv[b] and of
 *   k_rope[b] takes row prefix_len + path[b][k] (the tv_tree_accept outputs);
 *   every other row is unchanged.  The accepted path's node k has depth k, so
 *   its rope row (rotated at prefix_len + depth) is already right for its new
 *   row.  The next step's prefix is prefix_len + accept_len + 1 rows.
 *   c_kv [B][kv_len][d_c], k_rope [B][kv_len][d_r] (kv_dtype), 16-byte aligned,
 *   with d_c and d_r rows a multiple of 16 bytes (else TV_ERR_UNSUPPORTED);
 *   prefix_len + q_len <= kv_len.  path [B][q_len] and accept_len [B] int32 are
 *   device data: accept_len is clamped to [0, q_len - 1] and path entries to
 *   [0, q_len - 1], so malformed values move rows of the tree only.
 */
tv_status_t tv_kv_compact(void* c_kv, void* k_rope, tv_dtype_t kv_dtype, const int32_t* path,
                          const int32_t* accept_len, int32_t prefix_len, int32_t B, int32_t kv_len, int32_t q_len,
                          int32_t d_c, int32_t d_r, hipStream_t stream);

/*
 * tv_tree_build — best-first draft tree per request, the step before verify.
 *   [Verify page, "The Context: What Led to This Moment" (a GPU best-first
 *   tree builder in place of a per-request CPU heap); RoPE page, "The Broader
 *   Context: A Full Native Engine from Scratch" (a drafter proposes candidate
 *   tokens; the kernels are bit-exact against their reference)]
 *   The drafter proposes, at each depth d = 1..D, K candidates: token
 *   cand_tok[b][d-1][c] with log-prob logp[b][d-1][c] (a NaN counts as -inf;
 *   +inf is outside the contract).  A node is a path of candidates; its score
 *   is the float32 sum of their log-probs, added from the root down.  Starting
 *   from the root, budget times the best node whose parent is in the tree
 *   joins it as the next node: the higher score, then the smaller depth, the
 *   smaller parent index, the smaller candidate rank (candidates of a depth
 *   ranked by log-prob, higher first, equal ones by index).  Nodes come out in
 *   topological order, ready for tv_verify_attn.
 *   Inputs (device, 4-byte aligned): logp f32 [B][D][K], cand_tok int32
 *   [B][D][K], root_tok int32 [B].  Only depths 1..min(D, budget) are read.
 *   Outputs (device, 4-byte aligned), [B][budget + 1] each: parent int32 (-1
 *   for the root), token int32 (root_tok for the root), depth int32 (0 for the
 *   root), score f32 (0 for the root); slots past the drafted nodes hold -1, -1,
 *   -1, -inf.  n_nodes int32 [B]: drafted nodes (budget unless the candidates
 *   run out: K + K^2 + ... + K^D < budget).
 *   1 <= K <= 64, D >= 1, 0 <= budget <= TV_MAX_BUILD_BUDGET, B >= 1,
 *   min(D, budget) * K <= TV_MAX_BUILD_CANDIDATES (else TV_ERR_UNSUPPORTED).
 */
tv_status_t tv_tree_build(const float* logp, const int32_t* cand_tok, const int32_t* root_tok, int32_t B, int32_t D,
                          int32_t K, int32_t budget, int32_t* parent, int32_t* token, int32_t* depth, float* score,
                          int32_t* n_nodes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H */
