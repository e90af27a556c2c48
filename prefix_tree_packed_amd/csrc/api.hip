// C-ABI entry points that touch the device: plan upload, the two attention
// forwards and the decision epilogue. Every argument is checked before
// anything is enqueued (include/tree_attn.h states the contract).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace ta {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static ta_status hip_fail(hipError_t e, const char* what) {
  return fail(TA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static ta_status check_tensors(ta_plan_t p, const void* const* ptrs, const char* const* names, int n,
                               float* lse) {
  if (!p) return fail(TA_ERR_INVALID_ARGUMENT, "NULL plan");
  if (!p->d_ws) return fail(TA_ERR_WORKSPACE, "plan has not been uploaded");
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(TA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(TA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (lse && !p->cfg.write_lse)
    return fail(TA_ERR_INVALID_ARGUMENT, "lse given but the plan was built with write_lse = 0");
  if (lse && ((uintptr_t)lse & 3u)) return fail(TA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  return TA_OK;
}

static AttnArgs attn_args(ta_plan_t p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const unsigned char* ws = (const unsigned char*)p->d_ws;
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.qtiles = ws + p->off_qtiles;
  a.ktiles = ws + p->off_ktiles;
  a.mbits = ws + p->off_mbits;
  a.segs = ws + p->off_segs;
  a.wg_ptr = ws + p->off_wg_ptr;
  a.wg_items = ws + p->off_wg_items;
  a.hq = p->cfg.num_q_heads;
  a.hkv = p->cfg.num_kv_heads;
  a.head_dim = p->cfg.head_dim;
  a.group = p->group;
  a.n_q = (int)p->n_q;
  a.n_wg = p->n_wg;
  a.scale_log2e = p->cfg.scale * 1.4426950408889634f;
  a.out_f32 = p->cfg.out_dtype == TA_F32;
  return a;
}

}  // namespace ta

extern "C" {

ta_status tree_attn_plan_upload(ta_plan_t p, void* d_workspace, size_t bytes, void* hip_stream) {
  ta::clear_error();
  if (!p || !d_workspace) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (bytes < p->ws_bytes)
    return ta::fail(TA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", bytes, p->ws_bytes);
  if ((uintptr_t)d_workspace & 255u) return ta::fail(TA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  // persistent grid: every workgroup that fits on the current device at once,
  // no more than there are work items (and no more than the caller's cap)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return ta::hip_fail(e, "querying the device");
  const int per_cu = ta::attention_blocks_per_cu(p->cfg.head_dim, p->group, p->cfg.out_dtype == TA_F32,
                                                 p->cfg.write_lse != 0);
  if (per_cu < 1) return ta::fail(TA_ERR_HIP, "attention kernel does not fit on a compute unit");
  long long n_wg = std::min<long long>((long long)cus * per_cu, ta::kMaxWorkgroups);
  if (p->max_workgroups > 0) n_wg = std::min<long long>(n_wg, p->max_workgroups);
  n_wg = std::min<long long>(n_wg, (long long)p->work.size());
  p->n_wg = (int)n_wg;
  if (n_wg > 0)
    ta::assign_workgroups(p, p->n_wg, (int32_t*)(p->image.data() + p->off_wg_ptr),
                          (int32_t*)(p->image.data() + p->off_wg_items));
  e = hipMemcpyAsync(d_workspace, p->image.data(), p->ws_bytes, hipMemcpyHostToDevice,
                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "plan upload");
  p->d_ws = d_workspace;
  return TA_OK;
}

ta_status tree_attn_forward(ta_plan_t p, const void* q, const void* k, const void* v, void* o,
                            float* lse, void* hip_stream) {
  ta::clear_error();
  if (p && p->n_q == 0) return TA_OK;
  const void* ptrs[] = {q, k, v, o};
  const char* names[] = {"q", "k", "v", "o"};
  ta_status st = ta::check_tensors(p, ptrs, names, 4, lse);
  if (st != TA_OK) return st;
  if (!p->one_shot)
    return ta::fail(TA_ERR_INVALID_ARGUMENT,
                    "plan has rows with cached tokens or later chunks; use tree_attn_forward_chunked");
  hipError_t e = ta::launch_tree_attention(ta::attn_args(p, q, k, v, o, lse), (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "tree attention launch");
  return TA_OK;
}

ta_status tree_attn_cache_write(ta_plan_t p, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, int64_t cache_tokens, void* hip_stream) {
  ta::clear_error();
  if (p && p->n_q == 0) return TA_OK;
  const void* ptrs[] = {k_new, v_new, k_cache, v_cache};
  const char* names[] = {"k_new", "v_new", "k_cache", "v_cache"};
  ta_status st = ta::check_tensors(p, ptrs, names, 4, nullptr);
  if (st != TA_OK) return st;
  if (cache_tokens < p->n_kv)
    return ta::fail(TA_ERR_WORKSPACE, "cache holds %lld tokens < %lld of the plan's row space",
                    (long long)cache_tokens, (long long)p->n_kv);
  const unsigned char* ws = (const unsigned char*)p->d_ws;
  hipError_t e = ta::launch_cache_write(k_new, v_new, k_cache, v_cache, ws + p->off_rowpos, (int)p->n_q,
                                        p->cfg.num_kv_heads, p->cfg.head_dim, (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "cache write launch");
  return TA_OK;
}

ta_status tree_attn_rope_cache_write(ta_plan_t p, const void* q_in, void* q_out, const void* k_new,
                                     const void* v_new, const float* cos_sin, int32_t max_pos,
                                     ta_rope_style style, void* k_cache, void* v_cache,
                                     int64_t cache_tokens, void* hip_stream) {
  ta::clear_error();
  if (p && p->n_q == 0) return TA_OK;
  const void* ptrs[] = {q_in, q_out, k_new, v_new, cos_sin, k_cache, v_cache};
  const char* names[] = {"q_in", "q_out", "k_new", "v_new", "cos_sin", "k_cache", "v_cache"};
  ta_status st = ta::check_tensors(p, ptrs, names, 7, nullptr);
  if (st != TA_OK) return st;
  if (style != TA_ROPE_HALF && style != TA_ROPE_INTERLEAVED)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "unknown rope style %d", (int)style);
  if (max_pos <= p->max_pos_id)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "cos_sin has %d positions; this forward needs position %d",
                    max_pos, p->max_pos_id);
  if (cache_tokens < p->n_kv)
    return ta::fail(TA_ERR_WORKSPACE, "cache holds %lld tokens < %lld of the plan's row space",
                    (long long)cache_tokens, (long long)p->n_kv);
  const unsigned char* ws = (const unsigned char*)p->d_ws;
  ta::RopeArgs a;
  a.q_in = q_in;
  a.q_out = q_out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cos_sin = cos_sin;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tok_rowpos = ws + p->off_rowpos;
  a.pos_id = ws + p->off_posid;
  a.n_q = (int)p->n_q;
  a.hq = p->cfg.num_q_heads;
  a.hkv = p->cfg.num_kv_heads;
  a.head_dim = p->cfg.head_dim;
  a.interleaved = style == TA_ROPE_INTERLEAVED;
  hipError_t e = ta::launch_rope_cache_write(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "rope cache write launch");
  return TA_OK;
}

ta_status tree_attn_forward_cached(ta_plan_t p, const void* q, const void* k_cache, const void* v_cache,
                                   int64_t cache_tokens, void* o, float* lse, void* hip_stream) {
  ta::clear_error();
  if (p && p->n_q == 0) return TA_OK;
  const void* ptrs[] = {q, k_cache, v_cache, o};
  const char* names[] = {"q", "k_cache", "v_cache", "o"};
  ta_status st = ta::check_tensors(p, ptrs, names, 4, lse);
  if (st != TA_OK) return st;
  if (cache_tokens < p->n_kv)
    return ta::fail(TA_ERR_WORKSPACE, "cache holds %lld tokens < %lld of the plan's row space",
                    (long long)cache_tokens, (long long)p->n_kv);
  hipError_t e = ta::launch_tree_attention(ta::attn_args(p, q, k_cache, v_cache, o, lse),
                                           (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "tree attention launch");
  return TA_OK;
}

ta_status tree_attn_forward_chunked(ta_plan_t p, const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, int64_t cache_tokens, void* o,
                                    float* lse, void* hip_stream) {
  ta::clear_error();
  if (p && p->n_q == 0) return TA_OK;
  // check everything both launches need before enqueuing the first
  const void* ptrs[] = {q, k_new, v_new, k_cache, v_cache, o};
  const char* names[] = {"q", "k_new", "v_new", "k_cache", "v_cache", "o"};
  ta_status st = ta::check_tensors(p, ptrs, names, 6, lse);
  if (st != TA_OK) return st;
  if (cache_tokens < p->n_kv)
    return ta::fail(TA_ERR_WORKSPACE, "cache holds %lld tokens < %lld of the plan's row space",
                    (long long)cache_tokens, (long long)p->n_kv);
  st = tree_attn_cache_write(p, k_new, v_new, k_cache, v_cache, cache_tokens, hip_stream);
  if (st != TA_OK) return st;
  return tree_attn_forward_cached(p, q, k_cache, v_cache, cache_tokens, o, lse, hip_stream);
}

ta_status decision_readout(const float* logits, int32_t n_rows, int32_t ld, const int32_t* row1,
                           const int32_t* row2, const int32_t* n_letters, const float* T,
                           int32_t n_dec, float* p_avg, float* p_cal, void* hip_stream) {
  ta::clear_error();
  if (n_dec < 0) return ta::fail(TA_ERR_INVALID_ARGUMENT, "n_dec %d < 0", n_dec);
  if (n_dec == 0) return TA_OK;
  if (!logits || !row1 || !row2 || !n_letters || !T || !p_avg || !p_cal)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (ld < 2) return ta::fail(TA_ERR_INVALID_ARGUMENT, "ld %d < 2", ld);
  if (n_rows < 1) return ta::fail(TA_ERR_INVALID_ARGUMENT, "n_rows %d < 1", n_rows);
  hipError_t e = ta::launch_decision(logits, n_rows, ld, row1, row2, n_letters, T, n_dec, p_avg, p_cal,
                                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "decision launch");
  return TA_OK;
}

}  // extern "C"

namespace ta {

constexpr int kReadoutMaxModel = 16384;

// K splits of the down projection: a function of the weight shape only (so a
// row's sums never depend on the batch): about 512 (64-row column block, split)
// pairs, i.e. about 256 eight-wave workgroups.
static int readout_splits(int d_model, int d_ff) {
  const int col_blocks = d_model / 64;
  int ks = 8;
  while (ks > 1 && (ks * col_blocks > 512 || d_ff % (ks * 256) != 0)) ks /= 2;
  return ks;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

struct ReadoutLayout {
  size_t xn, act, partial, total;
  int splits;
};

static ReadoutLayout readout_layout(int n, int d_model, int d_ff) {
  ReadoutLayout l;
  l.splits = readout_splits(d_model, d_ff);
  l.xn = 0;
  l.act = round256((size_t)n * d_model * 2);
  l.partial = l.act + round256((size_t)n * d_ff * 2);
  l.total = l.partial + (size_t)l.splits * n * d_model * 4;
  return l;
}

// Device scratch of readout_mlp_noalloc: the readout_mlp workspace layout
// (normalized rows, activations, the down product's partial sums) in a
// file-scope array instead of a caller's buffer. Each device holds its own
// copy from the moment the library's code is loaded on it until the process
// ends. Its address is looked up once per device (hipGetSymbolAddress) and
// only that address is handed to kernels: in host code the array's name is a
// host-side stand-in, not a device address.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static unsigned char* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up on the device's first call.
static ta_status device_scratch(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TA_ERR_LIMIT, "device index %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = (unsigned char*)p;
  }
  *out = g_scratch_ptr[dev];
  return TA_OK;
}

static ta_status check_mlp_shape(int32_t n, int32_t d_model, int32_t d_ff) {
  if (n < 0) return fail(TA_ERR_INVALID_ARGUMENT, "n_readout %d < 0", n);
  if (d_model < 256 || d_model > kReadoutMaxModel || d_model % 256)
    return fail(TA_ERR_LIMIT, "d_model %d is not a multiple of 256 in [256, %d]", d_model,
                kReadoutMaxModel);
  if (d_ff < 256 || d_ff % 256) return fail(TA_ERR_LIMIT, "d_ff %d is not a multiple of 256", d_ff);
  return TA_OK;
}

}  // namespace ta

extern "C" {

ta_status readout_mlp_workspace_size(int32_t n_readout, int32_t d_model, int32_t d_ff, size_t* bytes) {
  ta::clear_error();
  if (!bytes) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  ta_status st = ta::check_mlp_shape(n_readout, d_model, d_ff);
  if (st != TA_OK) return st;
  *bytes = ta::readout_layout(n_readout, d_model, d_ff).total;
  return TA_OK;
}

}  // extern "C"

namespace ta {

// readout_mlp's argument checks and launches; `workspace` is the caller's
// buffer or this device's scratch (noalloc: sizes beyond it are refused).
static ta_status readout_mlp_impl(const void* hidden, int64_t n_tokens, const int32_t* readout_tok,
                                  int32_t n_readout, const ta_mlp_weights* w, void* workspace,
                                  size_t workspace_bytes, void* h_out, void* hip_stream, bool noalloc) {
  if (!w) return fail(TA_ERR_INVALID_ARGUMENT, "NULL weights");
  ta_status st = check_mlp_shape(n_readout, w->d_model, w->d_ff);
  if (st != TA_OK) return st;
  if (n_readout == 0) return TA_OK;
  if (n_tokens < 1) return fail(TA_ERR_INVALID_ARGUMENT, "n_tokens %lld < 1", (long long)n_tokens);
  if (!(w->eps >= 0.f)) return fail(TA_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  const ReadoutLayout l = readout_layout(n_readout, w->d_model, w->d_ff);
  if (noalloc) {
    if (l.total > kNoAllocScratchBytes)
      return fail(TA_ERR_LIMIT,
                  "readout_mlp_noalloc: %d rows at d_model %d, d_ff %d need %zu bytes of scratch, "
                  "more than its fixed %zu; pass a workspace to readout_mlp instead",
                  n_readout, w->d_model, w->d_ff, l.total, kNoAllocScratchBytes);
    unsigned char* sp = nullptr;
    st = device_scratch(&sp);
    if (st != TA_OK) return st;
    workspace = sp;
    workspace_bytes = kNoAllocScratchBytes;
  }
  const void* ptrs[] = {hidden, readout_tok, w->norm_w, w->w_gate_up, w->w_down, workspace, h_out};
  const char* names[] = {"hidden", "readout_tok", "norm_w", "w_gate_up", "w_down", "workspace", "h_out"};
  for (int i = 0; i < 7; ++i) {
    if (!ptrs[i]) return fail(TA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(TA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (workspace_bytes < l.total)
    return fail(TA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, l.total);
  unsigned char* ws = (unsigned char*)workspace;
  ReadoutArgs a;
  a.hidden = hidden;
  a.n_tokens = n_tokens;
  a.readout_tok = readout_tok;
  a.norm_w = w->norm_w;
  a.w_gate_up = w->w_gate_up;
  a.w_down = w->w_down;
  a.xn = ws + l.xn;
  a.act = ws + l.act;
  a.partial = (float*)(ws + l.partial);
  a.h_out = h_out;
  a.n_rows = n_readout;
  a.d_model = w->d_model;
  a.d_ff = w->d_ff;
  a.splits = l.splits;
  a.eps = w->eps;
  hipError_t e = launch_readout_mlp(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "readout MLP launch");
  return TA_OK;
}

}  // namespace ta

extern "C" {

ta_status readout_mlp(const void* hidden, int64_t n_tokens, const int32_t* readout_tok,
                      int32_t n_readout, const ta_mlp_weights* w, void* workspace,
                      size_t workspace_bytes, void* h_out, void* hip_stream) {
  ta::clear_error();
  return ta::readout_mlp_impl(hidden, n_tokens, readout_tok, n_readout, w, workspace, workspace_bytes,
                              h_out, hip_stream, false);
}

ta_status readout_mlp_noalloc(const void* hidden, int64_t n_tokens, const int32_t* readout_tok,
                              int32_t n_readout, const ta_mlp_weights* w, void* h_out,
                              void* hip_stream) {
  ta::clear_error();
  return ta::readout_mlp_impl(hidden, n_tokens, readout_tok, n_readout, w, nullptr, 0, h_out,
                              hip_stream, true);
}

ta_status readout_pack_gate_up(const void* w_gate, const void* w_up, int32_t d_ff, int32_t d_model,
                               void* w_gate_up, void* hip_stream) {
  ta::clear_error();
  ta_status st = ta::check_mlp_shape(0, d_model, d_ff);
  if (st != TA_OK) return st;
  const void* ptrs[] = {w_gate, w_up, w_gate_up};
  const char* names[] = {"w_gate", "w_up", "w_gate_up"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return ta::fail(TA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!ta::aligned16(ptrs[i]))
      return ta::fail(TA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  hipError_t e = ta::launch_gate_up_pack(w_gate, w_up, d_ff, d_model, w_gate_up, (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "gate/up pack launch");
  return TA_OK;
}

ta_status letter_logits(const void* h, int32_t n_readout, int32_t d_model, const void* final_norm_w,
                        float eps, const void* lm_head, int32_t vocab, const int32_t* letter_ids,
                        const int32_t* n_letters, int32_t ld, float* logits, void* hip_stream) {
  ta::clear_error();
  if (n_readout < 0) return ta::fail(TA_ERR_INVALID_ARGUMENT, "n_readout %d < 0", n_readout);
  if (d_model < 8 || d_model > ta::kReadoutMaxModel || d_model % 8)
    return ta::fail(TA_ERR_LIMIT, "d_model %d is not a multiple of 8 in [8, %d]", d_model,
                    ta::kReadoutMaxModel);
  if (ld < 1 || ld > 255) return ta::fail(TA_ERR_INVALID_ARGUMENT, "ld %d not in [1, 255]", ld);
  if (vocab < 1) return ta::fail(TA_ERR_INVALID_ARGUMENT, "vocab %d < 1", vocab);
  if (!(eps >= 0.f)) return ta::fail(TA_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (n_readout == 0) return TA_OK;
  const void* ptrs[] = {h, final_norm_w, lm_head};
  const char* names[] = {"h", "final_norm_w", "lm_head"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return ta::fail(TA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!ta::aligned16(ptrs[i]))
      return ta::fail(TA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (!letter_ids || !n_letters || !logits) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  ta::LetterArgs a;
  a.h = h;
  a.norm_w = final_norm_w;
  a.lm_head = lm_head;
  a.letter_ids = letter_ids;
  a.n_letters = n_letters;
  a.logits = logits;
  a.n_rows = n_readout;
  a.d_model = d_model;
  a.vocab = vocab;
  a.ld = ld;
  a.eps = eps;
  hipError_t e = ta::launch_letter_logits(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "letter logits launch");
  return TA_OK;
}

ta_status tree_attn_mfma_peak_probe(int32_t n_wg, int32_t iters, float* out, int64_t* flops,
                                    void* hip_stream) {
  ta::clear_error();
  if (n_wg < 1 || n_wg > 65536 || iters < 1)
    return ta::fail(TA_ERR_INVALID_ARGUMENT, "n_wg %d or iters %d out of range", n_wg, iters);
  if (!out || !flops) return ta::fail(TA_ERR_INVALID_ARGUMENT, "NULL argument");
  *flops = ta::mfma_peak_flops(n_wg, iters);
  hipError_t e = ta::launch_mfma_peak(n_wg, iters, out, (hipStream_t)hip_stream);
  if (e != hipSuccess) return ta::hip_fail(e, "MFMA probe launch");
  return TA_OK;
}

}  // extern "C"
