// C ABI entry points (include/oscar.h): host-side argument checks, the
// split-K plan and kernel launches.  No allocation, no synchronisation.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/oscar.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int code, const char* fmt, const char* detail = "") {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
  return code;
}

int check_shape(const oscar_shape_t* s) {
  if (!s) return fail(OSCAR_EINVAL, "shape is NULL%s");
  if (s->head_dim != 128) return fail(OSCAR_EINVAL, "head_dim must be 128%s");
  if (s->page_size != 16) return fail(OSCAR_EINVAL, "page_size must be 16%s");
  if (s->group != 64 && s->group != 128) return fail(OSCAR_EINVAL, "group must be 64 or 128%s");
  if (s->num_kv_heads < 1) return fail(OSCAR_EINVAL, "num_kv_heads must be >= 1%s");
  if (s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(OSCAR_EINVAL, "num_q_heads must be a positive multiple of num_kv_heads%s");
  if (s->num_q_heads / s->num_kv_heads > 8) return fail(OSCAR_EINVAL, "num_q_heads / num_kv_heads must be <= 8%s");
  if (s->sink < 0 || s->sink > 1024 || s->sink % 16 != 0)
    return fail(OSCAR_EINVAL, "sink must be a multiple of 16 in [0, 1024]%s");
  if (s->recent < 1 || s->recent > 4096) return fail(OSCAR_EINVAL, "recent must be in [1, 4096]%s");
  return OSCAR_OK;
}

bool clip_ok(float c) { return std::isfinite(c) && c > 0.f && c <= 16384.f; }

// The kernels move bf16 rows and page blocks in 16-byte vectors (and page blocks by
// 16-byte direct-to-LDS loads); int32 index arrays are read as 32-bit words.
bool al16(const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; }
bool al4(const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 4 == 0; }

int check_layer_alignment(const oscar_layer_t* l) {
  if (!al16(l->pages) || !al16(l->k_sink) || !al16(l->v_sink) || !al16(l->k_ring) || !al16(l->v_ring) ||
      !al16(l->u_k) || !al16(l->u_v))
    return fail(OSCAR_EINVAL, "layer buffers must be 16-byte aligned%s");
  return OSCAR_OK;
}

int hip_fail(const char* what) {
  const hipError_t e = hipGetLastError();
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return OSCAR_EHIP;
}

}  // namespace

namespace {
// Checks of a kv_write call; fills L.  *nothing is set when there is nothing to write.
int prepare_kv_write(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* k, const uint16_t* v,
                     const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens, const int32_t* page_table,
                     int32_t max_pages, const int32_t* seq_lens_after, oscar::KvWriteLaunch& L, bool* nothing) {
  *nothing = false;
  if (int rc = check_shape(shape)) return rc;
  if (!layer) return fail(OSCAR_EINVAL, "layer is NULL%s");
  if (num_tokens < 0) return fail(OSCAR_EINVAL, "num_tokens < 0%s");
  if (max_pages < 1) return fail(OSCAR_EINVAL, "max_pages must be >= 1%s");
  if (num_tokens == 0 || (!k && !v)) {
    *nothing = true;
    return OSCAR_OK;
  }
  if (!seq_idx || !pos || !page_table || !seq_lens_after || !layer->pages)
    return fail(OSCAR_EINVAL, "NULL index array or pages%s");
  if (k && (!layer->u_k || !layer->k_ring || (shape->sink > 0 && !layer->k_sink) || !clip_ok(layer->clip_k)))
    return fail(OSCAR_EINVAL, "K half: NULL u_k/k_ring/k_sink or clip_k outside (0, 16384]%s");
  if (v && (!layer->u_v || !layer->v_ring || (shape->sink > 0 && !layer->v_sink) || !clip_ok(layer->clip_v)))
    return fail(OSCAR_EINVAL, "V half: NULL u_v/v_ring/v_sink or clip_v outside (0, 16384]%s");
  if (int rc = check_layer_alignment(layer)) return rc;
  if (!al16(k) || !al16(v)) return fail(OSCAR_EINVAL, "k and v must be 16-byte aligned%s");
  if (!al4(seq_idx) || !al4(pos) || !al4(page_table) || !al4(seq_lens_after))
    return fail(OSCAR_EINVAL, "int32 index arrays must be 4-byte aligned%s");
  L = oscar::KvWriteLaunch{};
  L.k = k;
  L.v = v;
  L.u_k = layer->u_k;
  L.u_v = layer->u_v;
  L.clip_k = layer->clip_k;
  L.clip_v = layer->clip_v;
  L.k_sink = layer->k_sink;
  L.v_sink = layer->v_sink;
  L.k_ring = layer->k_ring;
  L.v_ring = layer->v_ring;
  L.pages = layer->pages;
  L.seq_idx = seq_idx;
  L.pos = pos;
  L.page_table = page_table;
  L.seq_lens_after = seq_lens_after;
  L.num_tokens = num_tokens;
  L.num_kv_heads = shape->num_kv_heads;
  L.max_pages = max_pages;
  L.group = shape->group;
  L.sink = shape->sink;
  L.recent = shape->recent;
  return OSCAR_OK;
}

// Checks of a decode_attn call; fills L.  *nothing is set for batch == 0.
int prepare_decode(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q, const int32_t* page_table,
                   int32_t max_pages, const int32_t* seq_lens, int32_t batch, float sm_scale, uint16_t* out,
                   void* workspace, size_t workspace_bytes, oscar::DecodeLaunch& L, bool* nothing,
                   int32_t max_shared_pages = -1) {
  *nothing = false;
  if (int rc = check_shape(shape)) return rc;
  if (!layer) return fail(OSCAR_EINVAL, "layer is NULL%s");
  if (batch < 0) return fail(OSCAR_EINVAL, "batch < 0%s");
  if (max_pages < 1) return fail(OSCAR_EINVAL, "max_pages must be >= 1%s");
  if (!std::isfinite(sm_scale)) return fail(OSCAR_EINVAL, "sm_scale is not finite%s");
  if (batch == 0) {
    *nothing = true;
    return OSCAR_OK;
  }
  if (!q || !page_table || !seq_lens || !out || !layer->pages || !layer->k_ring || !layer->v_ring || !layer->u_k ||
      !layer->u_v || (shape->sink > 0 && (!layer->k_sink || !layer->v_sink)))
    return fail(OSCAR_EINVAL, "NULL tensor pointer%s");
  if (!clip_ok(layer->clip_v)) return fail(OSCAR_EINVAL, "clip_v outside (0, 16384]%s");
  if (int rc = check_layer_alignment(layer)) return rc;
  if (!al16(q) || !al16(out)) return fail(OSCAR_EINVAL, "q and out must be 16-byte aligned%s");
  if (!al4(page_table) || !al4(seq_lens)) return fail(OSCAR_EINVAL, "int32 index arrays must be 4-byte aligned%s");
  const oscar::DecodePlan plan =
      max_shared_pages < 0
          ? oscar::make_decode_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink, shape->recent, batch,
                                    max_pages)
          : oscar::make_cascade_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink, shape->recent, batch,
                                     max_pages, max_shared_pages);
  if (plan.n_total > oscar::kMaxItems) return fail(OSCAR_EINVAL, "max_pages too large (sequences over ~8M tokens)%s");
  if (!workspace || workspace_bytes < plan.bytes) return fail(OSCAR_ENOWS, "workspace smaller than required%s");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(OSCAR_EINVAL, "workspace not 256-byte aligned%s");
  L = oscar::DecodeLaunch{};
  L.pages = layer->pages;
  L.k_sink = layer->k_sink;
  L.v_sink = layer->v_sink;
  L.k_ring = layer->k_ring;
  L.v_ring = layer->v_ring;
  L.u_k = layer->u_k;
  L.u_v = layer->u_v;
  L.q = q;
  L.page_table = page_table;
  L.seq_lens = seq_lens;
  L.out = out;
  L.workspace = static_cast<uint8_t*>(workspace);
  L.sm_scale = sm_scale;
  L.clip_v = layer->clip_v;
  L.num_kv_heads = shape->num_kv_heads;
  L.num_q_heads = shape->num_q_heads;
  L.max_pages = max_pages;
  L.batch = batch;
  L.sink = shape->sink;
  L.recent = shape->recent;
  L.group = shape->group;
  L.plan = plan;
  return OSCAR_OK;
}

}  // namespace

extern "C" {

const char* oscar_status_string(int status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_EINVAL: return "invalid argument";
    case OSCAR_ENOWS: return "workspace too small";
    case OSCAR_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* oscar_last_error(void) { return g_last_error; }

int oscar_kv_write(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* k, const uint16_t* v,
                   const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens, const int32_t* page_table,
                   int32_t max_pages, const int32_t* seq_lens_after, hipStream_t stream) {
  oscar::KvWriteLaunch L;
  bool nothing = false;
  if (int rc = prepare_kv_write(shape, layer, k, v, seq_idx, pos, num_tokens, page_table, max_pages, seq_lens_after,
                                L, &nothing))
    return rc;
  if (nothing) return OSCAR_OK;
  if (oscar::launch_kv_write(L, stream)) return hip_fail("kv_write launch");
  return OSCAR_OK;
}

size_t oscar_decode_workspace_bytes(const oscar_shape_t* shape, int32_t batch, int32_t max_pages) {
  if (check_shape(shape) || batch < 0 || max_pages < 1) return 0;
  const oscar::DecodePlan plan = oscar::make_decode_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink,
                                                         shape->recent, batch, max_pages);
  return plan.n_total > oscar::kMaxItems ? 0 : plan.bytes;
}

int oscar_decode_attn(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q,
                      const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                      float sm_scale, uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  oscar::DecodeLaunch L;
  bool nothing = false;
  if (int rc = prepare_decode(shape, layer, q, page_table, max_pages, seq_lens, batch, sm_scale, out, workspace,
                              workspace_bytes, L, &nothing))
    return rc;
  if (nothing) return OSCAR_OK;
  if (oscar::launch_decode(L, stream)) return hip_fail("decode launch");
  return OSCAR_OK;
}

size_t oscar_cascade_workspace_bytes(const oscar_shape_t* shape, int32_t batch, int32_t max_pages,
                                     int32_t max_shared_pages) {
  if (check_shape(shape) || batch < 0 || max_pages < 1 || max_shared_pages < 0) return 0;
  return oscar::make_cascade_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink, shape->recent, batch,
                                  max_pages, max_shared_pages)
      .bytes;
}

int oscar_decode_attn_cascade(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                              const int32_t* cu_groups, const int32_t* group_pages, int32_t num_groups,
                              int32_t max_group, int32_t max_shared_pages, float sm_scale, uint16_t* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_groups < 0) return fail(OSCAR_EINVAL, "num_groups < 0%s");
  if (max_shared_pages < 0) return fail(OSCAR_EINVAL, "max_shared_pages < 0%s");
  if (num_groups > 0 && max_group < 1) return fail(OSCAR_EINVAL, "max_group must be >= 1%s");
  if (num_groups > 0 && (!cu_groups || !group_pages)) return fail(OSCAR_EINVAL, "NULL group array%s");
  if (num_groups > 0 && (!al4(cu_groups) || !al4(group_pages)))
    return fail(OSCAR_EINVAL, "int32 index arrays must be 4-byte aligned%s");
  oscar::DecodeLaunch L;
  bool nothing = false;
  if (int rc = prepare_decode(shape, layer, q, page_table, max_pages, seq_lens, batch, sm_scale, out, workspace,
                              workspace_bytes, L, &nothing, max_shared_pages))
    return rc;
  if (nothing) return OSCAR_OK;
  const long long G = shape->num_q_heads / shape->num_kv_heads, nq = (G + 3) / 4;
  const long long tiles = ((long long)std::min(max_group, batch) * G + 16 * nq - 1) / (16 * nq);
  const long long blocks = (long long)num_groups * shape->num_kv_heads * L.plan.n_sh * tiles +
                           (long long)batch * shape->num_kv_heads * (L.plan.n_split + L.plan.n_bsplit);
  if (blocks > 0x7FFFFFFFLL) return fail(OSCAR_EINVAL, "groups x KV heads x shared ranges exceed the grid limit%s");
  L.cu_groups = cu_groups;
  L.group_pages = group_pages;
  L.n_groups = num_groups;
  L.max_group = (int32_t)std::min(max_group, batch);
  if (oscar::launch_decode(L, stream)) return hip_fail("cascade decode launch");
  return OSCAR_OK;
}

int oscar_decode_step(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* k, const uint16_t* v,
                      const int32_t* seq_idx, const int32_t* pos, int32_t num_tokens, const int32_t* seq_lens_after,
                      const uint16_t* q, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, uint16_t* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  oscar::KvWriteLaunch W;
  oscar::DecodeLaunch D{};
  bool no_write = false, no_decode = false;
  if (int rc = prepare_kv_write(shape, layer, k, v, seq_idx, pos, num_tokens, page_table, max_pages, seq_lens_after,
                                W, &no_write))
    return rc;
  if (int rc = prepare_decode(shape, layer, q, page_table, max_pages, seq_lens, batch, sm_scale, out, workspace,
                              workspace_bytes, D, &no_decode))
    return rc;
  int err = 0;
  if (no_write && no_decode) return OSCAR_OK;
  if (no_write) err = oscar::launch_decode(D, stream);
  else if (no_decode) err = oscar::launch_kv_write(W, stream);
  else err = oscar::launch_decode_step(W, D, stream);
  if (err) return hip_fail("decode step launch");
  return OSCAR_OK;
}

namespace {
int check_bf16_heads(int32_t num_kv_heads, int32_t num_q_heads) {
  if (num_kv_heads < 1) return fail(OSCAR_EINVAL, "num_kv_heads must be >= 1%s");
  if (num_q_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(OSCAR_EINVAL, "num_q_heads must be a positive multiple of num_kv_heads%s");
  if (num_q_heads / num_kv_heads > 8) return fail(OSCAR_EINVAL, "num_q_heads / num_kv_heads must be <= 8%s");
  return OSCAR_OK;
}
}  // namespace

size_t oscar_bf16_decode_workspace_bytes(int32_t num_kv_heads, int32_t num_q_heads, int32_t batch,
                                         int32_t max_pages) {
  if (check_bf16_heads(num_kv_heads, num_q_heads) || batch < 0 || max_pages < 1) return 0;
  return oscar::make_bf16_decode_plan(num_kv_heads, batch, max_pages, num_q_heads).bytes;
}

int oscar_bf16_decode_attn(int32_t num_kv_heads, int32_t num_q_heads, const uint16_t* pages, const uint16_t* q,
                           const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                           float sm_scale, uint16_t* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (int rc = check_bf16_heads(num_kv_heads, num_q_heads)) return rc;
  if (batch < 0) return fail(OSCAR_EINVAL, "batch < 0%s");
  if (max_pages < 1) return fail(OSCAR_EINVAL, "max_pages must be >= 1%s");
  if (!std::isfinite(sm_scale)) return fail(OSCAR_EINVAL, "sm_scale is not finite%s");
  if (batch == 0) return OSCAR_OK;
  if (!pages || !q || !page_table || !seq_lens || !out) return fail(OSCAR_EINVAL, "NULL tensor pointer%s");
  if (!al16(pages) || !al16(q) || !al16(out)) return fail(OSCAR_EINVAL, "pages, q and out must be 16-byte aligned%s");
  if (!al4(page_table) || !al4(seq_lens)) return fail(OSCAR_EINVAL, "int32 index arrays must be 4-byte aligned%s");
  const oscar::B16Plan plan = oscar::make_bf16_decode_plan(num_kv_heads, batch, max_pages, num_q_heads);
  if ((long long)batch * num_kv_heads * plan.n_split > 0x7FFFFFFFLL)
    return fail(OSCAR_EINVAL, "batch x num_kv_heads x ranges exceeds the grid limit%s");
  if (!workspace || workspace_bytes < plan.bytes) return fail(OSCAR_ENOWS, "workspace smaller than required%s");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(OSCAR_EINVAL, "workspace not 256-byte aligned%s");
  oscar::B16Launch L{};
  L.pages = reinterpret_cast<const uint8_t*>(pages);
  L.q = q;
  L.page_table = page_table;
  L.seq_lens = seq_lens;
  L.out = out;
  L.workspace = static_cast<uint8_t*>(workspace);
  L.sm_scale = sm_scale;
  L.num_kv_heads = num_kv_heads;
  L.num_q_heads = num_q_heads;
  L.max_pages = max_pages;
  L.batch = batch;
  L.plan = plan;
  if (oscar::launch_bf16_decode(L, stream)) return hip_fail("bf16 decode launch");
  return OSCAR_OK;
}

size_t oscar_extend_workspace_bytes(const oscar_shape_t* shape, int32_t num_tokens, int32_t max_pages,
                                    int32_t max_chunk) {
  if (check_shape(shape) || num_tokens < 0 || max_pages < 1 || max_chunk < 1) return 0;
  return oscar::make_extend_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink, num_tokens, max_pages,
                                 max_chunk)
      .bytes;
}

int oscar_extend_attn(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const int32_t* cu_seqlens, const int32_t* prefix_lens, int32_t batch,
                      int32_t num_tokens, int32_t max_chunk, const int32_t* page_table, int32_t max_pages,
                      float sm_scale, uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int rc = check_shape(shape)) return rc;
  if (!layer) return fail(OSCAR_EINVAL, "layer is NULL%s");
  if (batch < 0 || num_tokens < 0) return fail(OSCAR_EINVAL, "batch and num_tokens must be >= 0%s");
  if (max_pages < 1 || max_chunk < 1) return fail(OSCAR_EINVAL, "max_pages and max_chunk must be >= 1%s");
  if (!std::isfinite(sm_scale)) return fail(OSCAR_EINVAL, "sm_scale is not finite%s");
  if (num_tokens == 0) return OSCAR_OK;
  if (batch == 0) return fail(OSCAR_EINVAL, "num_tokens > 0 with batch == 0%s");
  if ((long long)max_chunk * batch < num_tokens) return fail(OSCAR_EINVAL, "num_tokens exceeds batch x max_chunk%s");
  if (!q || !k || !v || !cu_seqlens || !prefix_lens || !page_table || !out || !layer->pages || !layer->k_ring ||
      !layer->v_ring || !layer->u_k || !layer->u_v || (shape->sink > 0 && (!layer->k_sink || !layer->v_sink)))
    return fail(OSCAR_EINVAL, "NULL tensor pointer%s");
  if (!clip_ok(layer->clip_v)) return fail(OSCAR_EINVAL, "clip_v outside (0, 16384]%s");
  if (int rc = check_layer_alignment(layer)) return rc;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(out)) return fail(OSCAR_EINVAL, "q, k, v and out must be 16-byte aligned%s");
  if (!al4(cu_seqlens) || !al4(prefix_lens) || !al4(page_table))
    return fail(OSCAR_EINVAL, "int32 index arrays must be 4-byte aligned%s");
  const oscar::ExtendPlan plan = oscar::make_extend_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink,
                                                         num_tokens, max_pages, max_chunk);
  const long long blocks = (long long)batch * shape->num_kv_heads * std::max(1, plan.n_split) * plan.n_qt;
  if (blocks > 0x7FFFFFFFLL) return fail(OSCAR_EINVAL, "batch x KV heads x ranges x query tiles exceeds the grid limit%s");
  if (!workspace || workspace_bytes < plan.bytes) return fail(OSCAR_ENOWS, "workspace smaller than required%s");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(OSCAR_EINVAL, "workspace not 256-byte aligned%s");
  oscar::ExtendLaunch L{};
  L.pages = layer->pages;
  L.k_sink = layer->k_sink;
  L.v_sink = layer->v_sink;
  L.k_ring = layer->k_ring;
  L.v_ring = layer->v_ring;
  L.u_k = layer->u_k;
  L.u_v = layer->u_v;
  L.q = q;
  L.k = k;
  L.v = v;
  L.cu_seqlens = cu_seqlens;
  L.prefix_lens = prefix_lens;
  L.page_table = page_table;
  L.out = out;
  L.workspace = static_cast<uint8_t*>(workspace);
  L.sm_scale = sm_scale;
  L.clip_v = layer->clip_v;
  L.num_kv_heads = shape->num_kv_heads;
  L.num_q_heads = shape->num_q_heads;
  L.max_pages = max_pages;
  L.batch = batch;
  L.num_tokens = num_tokens;
  L.max_chunk = max_chunk;
  L.sink = shape->sink;
  L.recent = shape->recent;
  L.group = shape->group;
  L.plan = plan;
  if (oscar::launch_extend(L, stream)) return hip_fail("extend launch");
  return OSCAR_OK;
}

int oscar_decode_attn_noalloc(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                              float sm_scale, uint16_t* out, hipStream_t stream) {
  oscar::DecodeLaunch L;
  bool nothing = false;
  if (int rc = check_shape(shape)) return rc;
  if (batch <= 0 || max_pages < 1)   // argument errors or an empty batch: no scratch needed
    return prepare_decode(shape, layer, q, page_table, max_pages, seq_lens, batch, sm_scale, out, nullptr, 0, L,
                          &nothing);
  const oscar::DecodePlan plan = oscar::make_decode_plan(shape->num_kv_heads, shape->num_q_heads, shape->sink,
                                                         shape->recent, batch, max_pages);
  if (plan.n_total <= oscar::kMaxItems && plan.bytes > (size_t)OSCAR_NOALLOC_SCRATCH_BYTES) {
    char need[64];
    std::snprintf(need, sizeof(need), "%zu", plan.bytes);
    return fail(OSCAR_EINVAL,
                "decode of this batch x max_pages needs %s bytes of scratch, more than the library's static "
                "OSCAR_NOALLOC_SCRATCH_BYTES; use oscar_decode_attn with a workspace",
                need);
  }
  void* scratch = nullptr;
  if (plan.n_total <= oscar::kMaxItems && oscar::noalloc_scratch(&scratch) != hipSuccess)
    return hip_fail("static decode scratch lookup");
  if (int rc = prepare_decode(shape, layer, q, page_table, max_pages, seq_lens, batch, sm_scale, out, scratch,
                              OSCAR_NOALLOC_SCRATCH_BYTES, L, &nothing))
    return rc;
  if (nothing) return OSCAR_OK;
  if (oscar::launch_decode(L, stream)) return hip_fail("decode launch");
  return OSCAR_OK;
}

size_t oscar_read_probe_sink_bytes(void) { return (size_t)oscar::kProbeBlocks * 256 * sizeof(uint32_t); }

int oscar_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_bytes, hipStream_t stream) {
  if (!buf || !sink) return fail(OSCAR_EINVAL, "NULL buffer%s");
  if (bytes == 0 || bytes % 16 != 0) return fail(OSCAR_EINVAL, "bytes must be a positive multiple of 16%s");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(OSCAR_EINVAL, "buffer not 16-byte aligned%s");
  if (sink_bytes < oscar_read_probe_sink_bytes()) return fail(OSCAR_ENOWS, "sink smaller than required%s");
  if (oscar::launch_read_probe(buf, bytes, sink, oscar::kProbeBlocks, stream)) return hip_fail("read probe launch");
  return OSCAR_OK;
}

}  // extern "C"
