// Host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

namespace ta {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* qtiles;
  const void* ktiles;
  const void* mbits;     // visibility bits of the flagged key tiles (layout.h)
  const void* segs;      // headers and segments of multi-segment key tiles
  const void* wg_ptr;    // [n_wg + 1] item ranges of the persistent workgroups
  const void* wg_items;  // work items (query tile * hkv + kv head), per workgroup
  int hq, hkv, head_dim, group, n_q, n_wg;
  float scale_log2e;
  bool out_f32;
};

hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st);
// Workgroups of the attention kernel variant for (head_dim, group, out_f32, lse)
// that fit on one compute unit at once (0 if the variant does not exist).
int attention_blocks_per_cu(int head_dim, int group, bool out_f32, bool lse);
hipError_t launch_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const void* tok_rowpos, int n_q, int hkv, int head_dim,
                              hipStream_t st);
struct RopeArgs {
  const void* q_in;
  void* q_out;
  const void* k_new;
  const void* v_new;
  const float* cos_sin;
  void* k_cache;
  void* v_cache;
  const void* tok_rowpos;
  const void* pos_id;
  int n_q, hq, hkv, head_dim;
  bool interleaved;
};
hipError_t launch_rope_cache_write(const RopeArgs& a, hipStream_t st);
struct ReadoutArgs {
  const void* hidden;       // f16 [n_tokens, d_model]
  long long n_tokens;
  const void* readout_tok;  // int32 [n_rows]
  const void* norm_w;       // f16 [d_model]
  const void* w_gate_up;    // f16 [2 d_ff, d_model], gate/up interleaved in 8-row blocks
  const void* w_down;       // f16 [d_model, d_ff]
  void* xn;                 // f16 [n_rows, d_model] workspace
  void* act;                // f16 [n_rows, d_ff] workspace
  float* partial;           // f32 [splits, n_rows, d_model] workspace
  void* h_out;              // f16 [n_rows, d_model]
  int n_rows, d_model, d_ff, splits;
  float eps;
};
hipError_t launch_readout_mlp(const ReadoutArgs& a, hipStream_t st);
hipError_t launch_gate_up_pack(const void* w_gate, const void* w_up, int d_ff, int d_model, void* out,
                               hipStream_t st);
struct LetterArgs {
  const void* h;          // f16 [n_rows, d_model]
  const void* norm_w;     // f16 [d_model]
  const void* lm_head;    // f16 [vocab, d_model]
  const void* letter_ids; // int32 [n_rows, ld]
  const void* n_letters;  // int32 [n_rows]
  float* logits;          // f32 [n_rows, ld]
  int n_rows, d_model, vocab, ld;
  float eps;
};
hipError_t launch_letter_logits(const LetterArgs& a, hipStream_t st);
hipError_t launch_mfma_peak(int n_wg, int iters, float* out, hipStream_t st);
long long mfma_peak_flops(int n_wg, int iters);
hipError_t launch_decision(const float* logits, int n_rows, int ld, const int* row1, const int* row2,
                           const int* n_letters, const float* T, int n_dec, float* p_avg,
                           float* p_cal, hipStream_t st);

}  // namespace ta
