// Internal launch interface between the C ABI (oscar_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oscar {

struct KvWriteLaunch {
  const uint16_t *k, *v, *u_k, *u_v;
  float clip_k, clip_v;
  uint16_t *k_sink, *v_sink, *k_ring, *v_ring;
  uint8_t* pages;
  const int32_t *seq_idx, *pos, *page_table, *seq_lens_after;
  int32_t num_tokens, num_kv_heads, max_pages, sink, recent;
  int32_t group;   // 64 or 128 channels per quantization group
};

// Split-K plan of one decode call: the INT2 history of each (sequence, KV
// head) is cut into `n_split` ranges of `pages_per_split` logical pages; the
// BF16 sink+recent tokens into `n_bsplit` chunks of `bf16_chunk` tokens.  Every
// (sequence, query head) owns n_bsplit + n_split partial records.
struct DecodePlan {
  int32_t pages_per_split, n_split, n_bsplit, n_total, bf16_chunk;
  int32_t n_sh;     // cascade decode: shared-prefix ranges per (sequence, query head), else 0
  size_t qrot_off, part_off, ml_off, eff_off, bytes;
};

constexpr int kQrotBytes = 576;      // rotated-query record per (sequence, query head)
constexpr int kBf16Chunk = 320;      // BF16 tokens per split item (multiple of 64) ...
constexpr int kBf16ChunkFew = 64;    // ... or this many when few (sequence, KV head) pairs share the GPU
constexpr int kFewPairs = 32;        // "few": fewer (sequence, KV head) pairs than this in one call
constexpr int kMaxItems = 1024;      // partial records per (sequence, query head) the reduce can merge

DecodePlan make_decode_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t recent,
                            int32_t batch, int32_t max_pages);
// decode_attn's plan with records for the shared ranges of cascade groups whose shared
// prefix is at most max_shared_pages INT2 pages; bytes == 0 when that exceeds the reduce's limit
DecodePlan make_cascade_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t recent,
                             int32_t batch, int32_t max_pages, int32_t max_shared_pages);

struct DecodeLaunch {
  const uint8_t* pages;
  const uint16_t *k_sink, *v_sink, *k_ring, *v_ring, *u_k, *u_v;
  const uint16_t* q;
  const int32_t *page_table, *seq_lens;
  uint16_t* out;
  uint8_t* workspace;
  float sm_scale, clip_v;
  int32_t num_kv_heads, num_q_heads, max_pages, batch, sink, recent;
  int32_t group;   // 64 or 128 channels per quantization group
  DecodePlan plan;
  // cascade decode only (n_groups == 0 otherwise)
  const int32_t *cu_groups, *group_pages;
  int32_t n_groups, max_group;
};

// BF16 paged decode (the comparison kernel): `n_split` ranges of
// `pages_per_split` pages per (sequence, KV head), one partial record each.
struct B16Plan {
  int32_t pages_per_split, n_split;
  size_t part_off, ml_off, bytes;
};

B16Plan make_bf16_decode_plan(int32_t num_kv_heads, int32_t batch, int32_t max_pages, int32_t num_q_heads);

struct B16Launch {
  const uint8_t* pages;
  const uint16_t* q;
  const int32_t *page_table, *seq_lens;
  uint16_t* out;
  uint8_t* workspace;
  float sm_scale;
  int32_t num_kv_heads, num_q_heads, max_pages, batch;
  B16Plan plan;
};

// Extend (chunked prefill) plan: the INT2 pages of a prefix in n_split ranges of
// pages_per_split pages; n_qt tiles of 64 query vectors per (sequence, KV head); every
// (chunk token, query head) owns n_total = 1 + n_split partial records.
struct ExtendPlan {
  int32_t pages_per_split, n_split, n_total, n_qt;
  size_t qrot_off, part_off, ml_off, len_off, bytes;
};

ExtendPlan make_extend_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t num_tokens,
                            int32_t max_pages, int32_t max_chunk);

struct ExtendLaunch {
  const uint8_t* pages;
  const uint16_t *k_sink, *v_sink, *k_ring, *v_ring, *u_k, *u_v;
  const uint16_t *q, *k, *v;
  const int32_t *cu_seqlens, *prefix_lens, *page_table;
  uint16_t* out;
  uint8_t* workspace;
  float sm_scale, clip_v;
  int32_t num_kv_heads, num_q_heads, max_pages, batch, num_tokens, max_chunk, sink, recent;
  int32_t group;   // 64 or 128 channels per quantization group
  ExtendPlan plan;
};

int device_cus();   // compute units of the current device
int launch_kv_write(const KvWriteLaunch& L, hipStream_t stream);
int launch_decode_step(const KvWriteLaunch& W, const DecodeLaunch& D, hipStream_t stream);
int launch_decode(const DecodeLaunch& L, hipStream_t stream);
int launch_extend(const ExtendLaunch& L, hipStream_t stream);
int launch_bf16_decode(const B16Launch& L, hipStream_t stream);
// Device address of the current device's static decode scratch (decode_noalloc.hip).
hipError_t noalloc_scratch(void** out);
int launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);
constexpr int kProbeBlocks = 4096;

}  // namespace oscar
