/*
 * oscar.h -- C ABI of the MI355X (gfx950) OSCAR INT2 KV-cache library.
 *
 * OSCAR stores each new key/value token rotated by R_K = U_Q . H_Had . P_br
 * (keys) or R_V = U_S . H_Had . P_br (values), clipped and quantized to INT2,
 * in a paged cache whose first `sink` tokens and last `recent` tokens stay in
 * BF16; decode attention reads the mixed cache in one pass.
 *
 * Pages (title -> tag used below):
 *   [it] "OSCAR: Come Together AI Comprime la KV Cache a 2-bit per LLM"
 *   [ru] "Together AI vypustila ishodniki OSCAR - INT2-kvantovanie KV-kesha
 *         dlya dolgih kontekstov LLM" (cited by paragraph)
 *   [es] "Resumen Tecnico: OSCAR - Rotacion Consciente de la Covarianza
 *         Espectral Offline para Cuantizacion de Cache KV de 2 bits"
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers unless the comment says host.
 *     They are owned by the caller; the library never allocates, frees or
 *     synchronises, keeps no state between calls and is re-entrant.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Return codes report argument errors found on the host
 *     and launch errors; nothing checks device memory contents.
 *   - bf16 values travel as uint16_t bit patterns; fp16 as uint16_t.
 *   - Alignment: every bf16 / byte tensor (k, v, q, out, pages, sink, ring,
 *     u_k, u_v) must start on a 16-byte boundary (the kernels move them in
 *     16-byte vectors); int32 arrays on a 4-byte boundary; decode workspaces
 *     on a 256-byte boundary.  A misaligned pointer is OSCAR_EINVAL.
 *   - Row-vector convention: a stored token is k' = k R.
 *
 * Page block format (one block per physical page id and KV head; `pages` is
 * [num_pages][num_kv_heads][B] with B = 1280 bytes for group == 64 and 1152
 * for group == 128):
 *   [   0,  512) K codes, token-major: slot t at byte 32*t; post-rotation
 *                channel j at byte j/4, bits 2*(j%4).
 *   [ 512, 1024) V codes, channel-major: channel j is the little-endian uint32
 *                at 512 + 4*j; slot t at bits 2*t.
 *   group == 64 (2.5 bits per element):
 *   [1024, 1152) K group parameters, slot t at 1024 + 8*t: fp16 s0, z0, s1, z1
 *   [1152, 1280) V group parameters, slot t at 1152 + 8*t: fp16 s0, z0, s1, z1
 *   group == 128 (2.25 bits per element, the format of the Russian page's
 *   paragraph 4 "2.28 bits per KV element"):
 *   [1024, 1088) K parameters, slot t at 1024 + 4*t: fp16 s, z
 *   [1088, 1152) V parameters, slot t at 1088 + 4*t: fp16 s, z
 * Group g covers post-rotation channels [group*g, group*(g+1)); a code c
 * decodes to z_g + s_g * c.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define OSCAR_OK 0
#define OSCAR_EINVAL 1   /* bad argument (null pointer, unsupported shape, bad size) */
#define OSCAR_ENOWS 2    /* workspace smaller than oscar_decode_workspace_bytes() */
#define OSCAR_EHIP 3     /* a HIP call failed; oscar_last_error() has the detail */

/* Cache geometry.  The Italian page's section "Architettura del Sistema di
 * Serving e Layout di Memoria" gives 64 BF16 sink tokens and 256 BF16 recent
 * tokens (also configurable server flags on that page); group = 64 (or 128)
 * channels with an fp16 scale and zero per token-group is this library's INT2
 * format.
 * Supported: head_dim == 128, page_size == 16, group == 64 or 128,
 * 1 <= num_kv_heads, num_q_heads % num_kv_heads == 0,
 * 1 <= num_q_heads / num_kv_heads <= 8, 0 <= sink <= 1024 with
 * sink % 16 == 0, 1 <= recent <= 4096. */
typedef struct oscar_shape {
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t sink;
  int32_t recent;
  int32_t group;
} oscar_shape_t;

/* One layer's cache and rotation.  Sequence "slot" b indexes the sink and ring
 * buffers; for decode, batch entry b uses slot b.
 *   pages          [num_pages][H_kv][1280 or 1152] bytes (format above)
 *   k_sink, v_sink bf16 [num_slots][H_kv][sink][128]; row p holds position p
 *   k_ring, v_ring bf16 [num_slots][H_kv][recent][128]; row p % recent holds
 *                  position p while p is inside the recent window
 *   u_k, u_v       bf16 [H_kv][128][128] row-major U (eigenvectors in columns:
 *                  U[i][j], i = input channel), i.e. U_Q and U_S of the
 *                  Spanish summary, section 2.2 A.2
 *   clip_k, clip_v per-layer clip thresholds c: rotated values are clamped to
 *                  [-c, c] before quantization ([es] 2.2 A.4); finite,
 *                  0 < c <= 16384. */
typedef struct oscar_layer {
  uint8_t* pages;
  uint16_t* k_sink;
  uint16_t* v_sink;
  uint16_t* k_ring;
  uint16_t* v_ring;
  const uint16_t* u_k;
  const uint16_t* u_v;
  float clip_k;
  float clip_v;
} oscar_layer_t;

/* kv_write -- rotate, clip, quantize and pack new tokens into the cache.
 * [it] "Architettura del Sistema di Serving e Layout di Memoria" (each token
 * is rotated, clipped and quantized at write time; history is INT2, sink and
 * recent tokens BF16); [es] 2.2 B; rotation composition [it] "I tre fattori
 * della rotazione", [ru] paragraph 3.
 *
 *   k, v            bf16 [num_tokens][H_kv][128]; either may be NULL (that
 *                   half of the cache is not written)
 *   seq_idx, pos    int32 [num_tokens]: sequence slot and position of token t
 *   page_table      int32 [num_slots][max_pages]: physical page of logical page
 *   seq_lens_after  int32 [num_slots]: sequence length once this call's tokens
 *                   are in (decides which tokens enter the recent ring)
 * For every token with pos >= sink: INT2 codes and group parameters go to
 * page_table[seq][pos/16], slot pos%16 (also while the token is still recent,
 * so nothing is re-encoded when it leaves the window).  pos < sink: bf16 copy
 * to the sink row.  pos >= max(sink, seq_lens_after[seq] - recent): bf16 copy
 * to ring row pos % recent.
 * The caller guarantees: no two tokens of one call share a (physical page,
 * slot) or a (seq, pos); indices are in range.  Quantization: per 64-channel
 * group s = fp16_rne((max-min)/3), z = fp16_rne(min), code =
 * clamp(rne((w - z)/s), 0, 3), codes 0 when s == 0.
 * Returns OSCAR_OK, OSCAR_EINVAL or OSCAR_EHIP.  num_tokens == 0 is a no-op. */
int oscar_kv_write(const oscar_shape_t* shape, const oscar_layer_t* layer,
                   const uint16_t* k, const uint16_t* v, const int32_t* seq_idx,
                   const int32_t* pos, int32_t num_tokens, const int32_t* page_table,
                   int32_t max_pages, const int32_t* seq_lens_after, hipStream_t stream);

/* Bytes of device workspace oscar_decode_attn needs for `batch` sequences
 * whose page_table rows hold `max_pages` entries.  0 on invalid arguments,
 * including max_pages beyond what one call can split: the INT2 pages after the
 * sink pages go to at most 1,024 - ceil((sink + recent) / 320) ranges of at most
 * 512 pages (sink 64, recent 256: max_pages <= 4 + 523,776, about 8.4M tokens).
 * Calls that share a workspace must not overlap in time. */
size_t oscar_decode_workspace_bytes(const oscar_shape_t* shape, int32_t batch, int32_t max_pages);

/* decode_attn -- one decode step of attention over the mixed-precision paged
 * cache: the read path of [it] "Architettura del Sistema di Serving e Layout
 * di Memoria" and [es] 2.2 B (unpack, dequantize, inverse rotation and
 * attention in one pass).  The inverse rotation is folded: q is rotated once
 * by R_K and the accumulated INT2 output once by R_V^T.
 *
 *   q          bf16 [batch][num_q_heads][128]
 *   page_table int32 [batch][max_pages]
 *   seq_lens   int32 [batch], 0 <= L <= 16 * max_pages (a device value
 *              outside is clamped to that range)
 *   sm_scale   softmax scale (1/sqrt(128) for standard attention)
 *   out        bf16 [batch][num_q_heads][128] (written, round to nearest even)
 *   workspace  device scratch of at least oscar_decode_workspace_bytes(shape,
 *              batch, max_pages) bytes, 256-byte aligned; clobbered
 * For batch entry b, query head h, KV head h / (num_q_heads/num_kv_heads),
 * L = seq_lens[b]: out = softmax(sm_scale * q . K^T) V over positions [0, L)
 * where positions < min(sink, L) come from the sink rows, positions >=
 * max(sink, L - recent) from the ring, and the rest from the INT2 pages
 * (dequantized and inverse-rotated).  L == 0 writes zeros.
 * layer->clip_v must be the threshold the value pages were written with
 * (checked to be in (0, 16384]): it bounds the value scales, which sets how
 * far the kernel may defer rescaling its fp16 softmax weights.
 * Returns OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOWS or OSCAR_EHIP. */
int oscar_decode_attn(const oscar_shape_t* shape, const oscar_layer_t* layer,
                      const uint16_t* q, const int32_t* page_table, int32_t max_pages,
                      const int32_t* seq_lens, int32_t batch, float sm_scale, uint16_t* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* BF16 paged decode -- the baseline the pages measure OSCAR against: their
 * 100K-context decode speedups are relative to a BF16 KV cache ([it]
 * "Velocita di decodifica"; [es] section 4, which also gives the ~8x memory
 * reduction).  Plain attention over an all-BF16 paged cache at the same
 * shapes, so the INT2 path's gain can be measured per layer on one GPU.
 *
 * BF16 page block (one 8192-byte block per physical page id and KV head;
 * `pages` is [num_pages][num_kv_heads][4096] bf16):
 *   elements [   0, 2048) K, token-major: slot t, channel c at 128*t + c
 *   elements [2048, 4096) V, channel-major: channel c, slot t at 2048 + 16*c + t
 *
 * Workspace bytes for `batch` sequences whose page_table rows hold
 * `max_pages` entries; 0 on invalid arguments (1 <= num_kv_heads,
 * num_q_heads a multiple of it with ratio <= 8, batch >= 0, max_pages >= 1).
 * Calls that share a workspace must not overlap in time. */
size_t oscar_bf16_decode_workspace_bytes(int32_t num_kv_heads, int32_t num_q_heads, int32_t batch,
                                         int32_t max_pages);

/* bf16_decode_attn -- out = softmax(sm_scale * q . K^T) V over positions
 * [0, L) of each sequence, position p at slot p % 16 of page
 * page_table[b][p / 16], KV head h = query head / (num_q_heads/num_kv_heads).
 *   pages      bf16 [num_pages][num_kv_heads][4096] (format above)
 *   q          bf16 [batch][num_q_heads][128]
 *   page_table int32 [batch][max_pages]
 *   seq_lens   int32 [batch], 0 <= L <= 16 * max_pages (a device value
 *              outside is clamped to that range)
 *   out        bf16 [batch][num_q_heads][128] (round to nearest even); L == 0
 *              writes zeros
 *   workspace  >= oscar_bf16_decode_workspace_bytes(...) bytes, 256-byte
 *              aligned; clobbered
 * Slots past L in a sequence's last page may hold anything (they are
 * masked).  Returns OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOWS or OSCAR_EHIP. */
int oscar_bf16_decode_attn(int32_t num_kv_heads, int32_t num_q_heads, const uint16_t* pages,
                           const uint16_t* q, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t batch, float sm_scale, uint16_t* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Measurement aid, not part of the method: streams `bytes` (a positive
 * multiple of 16, 16-byte aligned device buffer) once with plain 16-byte
 * loads and writes one word per thread to `sink` (device, at least
 * oscar_read_probe_sink_bytes() bytes).  Timing it gives the HBM read rate
 * a plain stream reaches on the device: the practical ceiling reported next
 * to the 8 TB/s specification for the bandwidth-bound decode.  Returns
 * OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOWS or OSCAR_EHIP. */
size_t oscar_read_probe_sink_bytes(void);
int oscar_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_bytes, hipStream_t stream);

/* decode_step -- one decode step of a layer in one call: exactly
 * oscar_kv_write(shape, layer, k, v, seq_idx, pos, num_tokens, page_table,
 * max_pages, seq_lens_after) followed by oscar_decode_attn(shape, layer, q,
 * page_table, max_pages, seq_lens, batch, sm_scale, out, workspace,
 * workspace_bytes), with the same arguments, checks, results and return codes
 * ([it] "Architettura del Sistema di Serving e Layout di Memoria": the new
 * token is written rotated and quantized, then attention reads the mixed
 * cache).  Every argument of both calls is checked before anything is
 * launched, so a bad argument of either leaves the cache untouched; nothing
 * else differs.  num_tokens == 0 (or k and v both NULL) decodes only;
 * batch == 0 writes only. */
int oscar_decode_step(const oscar_shape_t* shape, const oscar_layer_t* layer,
                      const uint16_t* k, const uint16_t* v, const int32_t* seq_idx,
                      const int32_t* pos, int32_t num_tokens, const int32_t* seq_lens_after,
                      const uint16_t* q, const int32_t* page_table, int32_t max_pages,
                      const int32_t* seq_lens, int32_t batch, float sm_scale, uint16_t* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* calibrate_layer -- HOST, offline: the calibration of [es] 2.2 A (steps 1-4)
 * and [ru] paragraph 2 for one layer, in fp64 on host memory.
 *   q_cal  host double [H_kv][gqa][num_samples][128] calibration queries
 *   k_cal, v_cal host double [H_kv][num_samples][128]
 * Per KV head: C_Q = (1/N) sum q^T q pooled over the gqa query heads,
 * C_S = (1/N) sum (S V)^T (S V) with S the causal softmax(sm_scale q k^T) of
 * each query head; U_Q, U_S = eigenvectors as columns, eigenvalues
 * descending, each column signed so its largest-|.| entry is positive;
 * written as bf16 (nearest even) to u_k_out, u_v_out (host uint16
 * [H_kv][128][128]).  clip_k_out / clip_v_out (host float): the `quantile`
 * (linear interpolation) of |x U H P| over all calibration tokens, channels
 * and heads, with the bf16 U.  num_threads <= 0 uses the hardware count.
 * Returns OSCAR_OK or OSCAR_EINVAL. */
int oscar_calibrate_layer(int32_t num_kv_heads, int32_t gqa, int32_t num_samples,
                          const double* q_cal, const double* k_cal, const double* v_cal,
                          double sm_scale, double quantile, uint16_t* u_k_out,
                          uint16_t* u_v_out, float* clip_k_out, float* clip_v_out,
                          int32_t num_threads);

/* calibrate_clip -- HOST, offline: the clip threshold of [es] 2.2 A step 4
 * for a rotation basis the caller chooses (the clip oscar_calibrate_layer
 * returns, for any U: e.g. U = I, the Hadamard-only rotation of [es] section
 * 4).  x_cal host double [H_kv][num_samples][128] calibration keys or values,
 * u host uint16 bf16 [H_kv][128][128]; *clip_out = the `quantile` (linear
 * interpolation) of |x U H P| over all samples, channels and heads.  Returns
 * OSCAR_OK or OSCAR_EINVAL. */
int oscar_calibrate_clip(int32_t num_kv_heads, int32_t num_samples, const double* x_cal, const uint16_t* u,
                         double quantile, float* clip_out);

/* decode_attn_cascade -- decode_attn for a batch in which groups of sequences
 * share the physical pages of a common prefix (prefix caching: [es] 2.2 B and
 * section 3, item 3; [it] "Architettura del Sistema di Serving e Layout di
 * Memoria").  Computes exactly what oscar_decode_attn computes; only the reads
 * differ: the shared INT2 pages of a group are read once per block of 16
 * (G <= 4) or 32 (G >= 5) of the members' query heads instead of once per
 * member and KV head.
 *   cu_groups   int32 [num_groups + 1], nondecreasing: group g is batch entries
 *               cu_groups[g] .. cu_groups[g+1] - 1 (at most max_group of them
 *               take part; entries in no group decode alone)
 *   group_pages int32 [num_groups]: the group's members share INT2 pages
 *               sink/16 .. sink/16 + group_pages[g] - 1 of their page-table
 *               rows (the same physical pages, read through the first
 *               member's row); clamped on the device to [0, max_shared_pages]
 *               rounded up to whole ranges
 * A member whose own INT2 history does not hold every shared page whole
 * (seq_len < sink + 16 group_pages + recent) reads its pages itself, and so
 * does every member of a group whose first member is such a sequence; so any
 * device values give the decode_attn result as long as the members' rows do
 * name the same physical pages where they are shared.
 *   max_group        host bound on the members per group
 *   max_shared_pages host bound on group_pages
 *   workspace        >= oscar_cascade_workspace_bytes(shape, batch, max_pages,
 *                    max_shared_pages) bytes, 256-byte aligned; clobbered
 * Other arguments, errors and outputs as oscar_decode_attn. */
size_t oscar_cascade_workspace_bytes(const oscar_shape_t* shape, int32_t batch, int32_t max_pages,
                                     int32_t max_shared_pages);
int oscar_decode_attn_cascade(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                              const int32_t* cu_groups, const int32_t* group_pages, int32_t num_groups,
                              int32_t max_group, int32_t max_shared_pages, float sm_scale, uint16_t* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* extend_attn -- chunked prefill (extend) attention over the mixed cache: the
 * read path of [it] "Architettura del Sistema di Serving e Layout di Memoria"
 * and [es] 2.2 B (paged attention with prefix caching) for a chunk of new
 * tokens per sequence instead of one.  The chunk of sequence b is tokens
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, k, v; its i-th token sits at
 * position prefix_lens[b] + i and attends to
 *   - the cached prefix [0, L), L = prefix_lens[b], as the cache stores it for
 *     a sequence of length L (sink rows [0, min(sink, L)), ring rows
 *     [max(sink, L - recent), L), INT2 history in between, dequantized and
 *     inverse-rotated by folding as in decode_attn), and
 *   - the chunk's own keys 0..i, in BF16 as given (causal),
 * with softmax(sm_scale q . k) over all of them.  The chunk is not in the
 * cache yet: call oscar_kv_write for it afterwards (on the same stream; the
 * write replaces ring rows this call reads).
 *   q          bf16 [num_tokens][num_q_heads][128]
 *   k, v       bf16 [num_tokens][num_kv_heads][128]
 *   cu_seqlens int32 [batch + 1], nondecreasing, cu_seqlens[0] = 0,
 *              cu_seqlens[batch] = num_tokens, each chunk at most max_chunk
 *              tokens.  On the device a chunk is clamped to [0, num_tokens)
 *              and to max_chunk tokens; out rows no chunk covers are undefined
 *   prefix_lens int32 [batch], 0 <= L <= 16 * max_pages (clamped on the device)
 *   page_table int32 [batch][max_pages]; batch entry b uses sink/ring slot b
 *   out        bf16 [num_tokens][num_q_heads][128]
 *   workspace  >= oscar_extend_workspace_bytes(shape, num_tokens, max_pages,
 *              max_chunk) bytes, 256-byte aligned; clobbered
 * Returns OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOWS or OSCAR_EHIP; num_tokens == 0
 * is a no-op. */
size_t oscar_extend_workspace_bytes(const oscar_shape_t* shape, int32_t num_tokens, int32_t max_pages,
                                    int32_t max_chunk);
int oscar_extend_attn(const oscar_shape_t* shape, const oscar_layer_t* layer, const uint16_t* q,
                      const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
                      const int32_t* prefix_lens, int32_t batch, int32_t num_tokens, int32_t max_chunk,
                      const int32_t* page_table, int32_t max_pages, float sm_scale, uint16_t* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* decode_attn_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): exactly oscar_decode_attn(shape, layer, q, page_table,
 * max_pages, seq_lens, batch, sm_scale, out, <workspace>, <bytes>, stream),
 * same kernels, checks and results, except that the workspace is a static
 * device array inside the library of OSCAR_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * GPU, held from the library's first use of that GPU until the process ends.
 * Calls whose oscar_decode_workspace_bytes(shape, batch, max_pages) exceeds it
 * return OSCAR_EINVAL (at 32 query heads, 8 KV heads and 100K tokens per
 * sequence the need is about 0.3 MB per sequence).  Nothing is allocated or
 * freed and nothing in the scratch needs to start at zero.  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be serialised by the caller.  The first
 * call on each GPU looks the array's address up (hipGetSymbolAddress) with
 * that GPU current; a failure there is OSCAR_EHIP. */
#define OSCAR_NOALLOC_SCRATCH_BYTES (64u << 20)
int oscar_decode_attn_noalloc(const oscar_shape_t* shape, const oscar_layer_t* layer,
                              const uint16_t* q, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, int32_t batch, float sm_scale, uint16_t* out,
                              hipStream_t stream);

/* Static description of a return code. */
const char* oscar_status_string(int status);

/* Detail of the last OSCAR_EHIP / OSCAR_EINVAL on the calling thread. */
const char* oscar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
