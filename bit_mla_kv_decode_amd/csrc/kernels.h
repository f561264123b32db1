// Internal launch interface between the C ABI and the kernels.
#pragma once
#include "common.h"

namespace mla {

struct DecodeArgs {
  const __bf16* q;
  const uint8_t* cache;
  int64_t num_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int batch;
  int heads;             // rows per sequence: s_q * qheads
  int s_q;               // query tokens per sequence (causal among themselves)
  int qheads;            // heads per query token
  int chunk_heads;       // heads per workgroup row block (s_q * chunk_heads <= 128)
  int max_pages;
  int num_splits;
  int pages_per_split;
  float scale_log2;      // softmax scale * log2(e)
  float* o_part;         // [B][S][H][512]
  float* lse_part;       // [B][S][H]
  __bf16* out;           // [B][H][512] (direct mode)
  float* lse_out;        // [B][H] or null (direct mode)
  int* meta;             // balanced partition: [B][first slot, slot count]
  // fused append (null when not fused): row b is quantized into position
  // seq_lens[b] - 1 of sequence b before that position is read
  const __bf16* new_latent;  // [B][512]
  const __bf16* new_rope;    // [B][64]
  uint8_t* append_cache;     // the cache (writable alias of `cache`)
};

hipError_t launch_quant_append(int fmt, const void* latent, const void* rope, const int32_t* slots, int n_new,
                               void* cache, int64_t num_pages, hipStream_t stream);
hipError_t launch_decode(int fmt, bool direct, const DecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_flat(int fmt, const DecodeArgs& a, int groups, hipStream_t stream);
// Decode workgroups one compute unit holds at once for `rows` rows per
// sequence: 2 where the kernel splits channels (quantized formats, <= 32
// rows), else 1.  The balanced partition launches this many per unit.
int workgroups_per_cu(int fmt, int rows);
hipError_t launch_combine_flat(const float* o_part, const float* lse_part, const int* meta, int batch, int heads,
                               __bf16* out, float* lse_out, hipStream_t stream);
// q [B, H, 576] = [q_nope W_UK^T | q_pe] per head; o [B, H, 128] = out W_UV^T per head
hipError_t launch_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, int B, int H, void* q_out,
                           hipStream_t stream);
hipError_t launch_project_out(const void* latent, const void* w_uv, int B, int H, void* out, hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, int batch, int heads, int splits,
                          __bf16* out, float* lse_out, hipStream_t stream);

}  // namespace mla
