// decode_attn: one decode step over the mixed-precision paged cache.
//
// Read path of the Italian page "OSCAR: Come Together AI Comprime la KV Cache
// a 2-bit per LLM", section "Architettura del Sistema di Serving e Layout di
// Memoria" (64 BF16 sink tokens, 256 BF16 recent tokens, INT2 history; the
// read kernel unpacks, dequantizes and inverts the rotation in one pass) and
// the Spanish summary "Resumen Tecnico: OSCAR ...", section 2.2 B.
//
// The inverse rotation is folded instead of applied per token: with
// k_hat = k_hat' R_K^T, q . k_hat = (q R_K) . k_hat', and
// sum_i p_i v_hat_i = (sum_i p_i v_hat'_i) R_V^T.  Two launches:
//   split     split-K over the pages: BF16 chunks with the plain q; INT2 page
//             ranges on v_mfma_f32_16x16x32_f16 -- each block first forms
//             q' = q U_K H P (times sm_scale*log2 e) of its G query heads as
//             fp16 hi/lo MFMA fragments while its first pages load, then
//             logits = codes x q' (the G query heads of a KV head share every
//             code) and acc = (p s) x codes; online softmax in base 2
//   reduce    log-sum-exp merge, acc_rot R_V^T = ((acc_rot P) H) U_V^T, bf16 out
// The extend and cascade kernels, whose blocks serve query heads of many rows,
// read q' from records a separate rotate_q launch stores.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace oscar {

namespace {

// Rotated query of one (sequence, query head) as B fragments of the logit
// MFMA.  q' = hi + lo with hi = fp16(q'), lo = fp16(q' - hi) (about 22
// significant bits).  frag[g][kh][limb][c] are the four registers that lane
// (column = head, k-group c) feeds to the MFMA over group g, k-half kh: pair v
// holds channels (64g + 16c + k_i, +8) with i = 4 kh + v and k_i = pair_k(i),
// the same pairs unpack16 makes of code word c of group g.
struct QrotRecord {
  uint32_t frag[2][2][2][4][4];
  float negc[2][2];   // [g][limb]: -sum over group g of limb_c * base(c): MFMA accumulator start
  float qsum[2];      // sum over the group of q'_c (fp32), for the zero-point term
  float pad[10];
};
static_assert(sizeof(QrotRecord) == kQrotBytes, "record size");

struct DecodeArgs {
  const uint8_t* pages;
  const uint16_t *k_sink, *v_sink, *k_ring, *v_ring, *u_k, *u_v, *q;
  const int32_t *page_table, *seq_lens;
  uint16_t* out;
  QrotRecord* qrot;
  float* part;     // partial accumulators acc[128] per (sequence, query head, item)
  float2* part_ml; // their (m, l)
  float sl2e;   // sm_scale * log2(e)
  float resc_thr;   // lazy rescale threshold tau: INT2 probabilities stay <= 2^tau
  int32_t H, Hq, G, B, max_pages, sink, recent, P, n_split, n_bsplit, n_total;
  int32_t bchunk;   // BF16 tokens per BF16 item (a multiple of 64)
  // extend (chunked prefill) reduce: every row (chunk token) has exactly one BF16 record,
  // index 0, and seq_lens holds the prefix length of the row's sequence
  int32_t ext;
  // 1: the split kernel's INT2 items rotate their own queries (no stored records)
  int32_t qrot_inline;
  // 1: one 128-channel quantization group per token (1152-byte page blocks)
  int32_t one_group;
  // cascade decode: groups of sequences (batch entries cu_groups[g] .. cu_groups[g+1] - 1, at
  // most max_group of them) share their first group_pages[g] INT2 pages.  The first n_cas
  // split blocks read each shared range once for all members' query heads (n_cqt tiles of
  // 16 NQ heads, or of 64 for more than 4 heads per KV head) into records n_bsplit + n_split + k; cas_eff[b] is the number of shared
  // pages sequence b takes from its group (0: none), written by the query rotation.
  const int32_t *cu_groups, *group_pages;
  int32_t* cas_eff;
  int32_t n_groups, max_group, n_sh, n_cqt, n_cas;
};

__device__ __forceinline__ int bf16_token_count(int L, int sink, int recent) {
  if (L <= sink) return L;
  return sink + (L - max(sink, L - recent));
}
__device__ __forceinline__ int int2_end(int L, int sink, int recent) {   // INT2 tokens [sink, end)
  return L <= sink ? sink : max(sink, L - recent);
}

__device__ __forceinline__ int whole_int2_pages(const DecodeArgs& a, int L) {   // pages sink/16 .. wholly INT2
  return int2_end(L, a.sink, a.recent) / kPage - a.sink / kPage;
}

// Members and shared pages of cascade group g, clamped so that no read leaves the batch, the
// records the plan provides or the part of the first member's page-table row its own length
// covers (the shared pages are read through that row): a group whose first member does not
// hold every shared page whole in its INT2 history shares nothing.
__device__ __forceinline__ void cascade_group(const DecodeArgs& a, int g, int& m0, int& members, int& shared) {
  m0 = min(max(scalar_load_i32(a.cu_groups, g), 0), a.B);
  const int m1 = min(max(scalar_load_i32(a.cu_groups, g + 1), m0), a.B);
  members = min(m1 - m0, a.max_group);
  shared = min(max(scalar_load_i32(a.group_pages, g), 0), a.n_sh * a.P);
  if (members == 0 || shared > whole_int2_pages(a, clamp_len(scalar_load_i32(a.seq_lens, m0), a.max_pages)))
    shared = 0;
}

// Shared pages sequence b (length L) takes from its group: the group's count when b is one
// of its members and every shared page lies whole inside b's INT2 history, else 0 (b then
// reads all of its pages itself).
__device__ int cascade_pages_of(const DecodeArgs& a, int b, int L) {
  int lo = 0, hi = a.n_groups - 1;   // the last group whose first member is <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_groups[mid] <= b) lo = mid; else hi = mid - 1;
  }
  int m0, members, shared;
  cascade_group(a, lo, m0, members, shared);
  if (b < m0 || b >= m0 + members) return 0;
  return shared <= whole_int2_pages(a, L) ? shared : 0;
}

// ---------------------------------------------------------------------------
// Query rotation of the G query heads of one (sequence, KV head), by one
// 256-thread block, in three steps shared by the split kernel's INT2 items
// (which rotate their own queries while their first page loads are in flight)
// and by rotate_q_kernel (which stores records for the extend and cascade
// kernels, whose blocks serve the query heads of many rows):
//   qrot_load     q rows and U_K columns into registers (A: head n, input
//                 channels 32 ks + 8 kg ..; B: each lane gathers eight 16-bit
//                 entries of a U_K column, U_K being row-major)
//   qrot_product  y = q U_K on v_mfma_f32_16x16x32_bf16 (exact bf16 products,
//                 fp32 sums); wave w makes output channels 32 w .. + 31
//   qrot_finish   per head, in one wave: Walsh-Hadamard transform (channel
//                 2 l + e in lane l: stage 1 in registers, the others across
//                 lanes), w_c = y_br(c) / sqrt(128) * sm_scale * log2(e), its
//                 fp16 hi / lo limbs, and per group the offset sums of the
//                 limbs and sum w (the accumulator starts of the logit MFMA)
// ---------------------------------------------------------------------------
constexpr int kSideThreads = 256;

struct QRotIn {
  bf16x8 bq[4];      // A: query head n, input channels 32 ks + 8 kg .. + 7 (zero beyond G)
  bf16x8 bu[2][4];   // B: U_K[32 ks + 8 kg + d][16 nt + n], nt = 2 wave + t
};

// LDS of the rotation (a view, so that the split kernel can place it in free ring slots)
struct QRotLds {
  float (*y)[kHeadDim];                 // [G][128]: q U_K, then w
  uint16_t (*qh)[kHeadDim], (*ql)[kHeadDim];   // [G][128]: fp16 limbs of w
  float (*negc)[2][2];                  // [G][group][limb]: -sum over the group of limb * base
  float (*qsum)[2];                     // [G][group]: sum over the group of w
};

__device__ __forceinline__ void qrot_load(const DecodeArgs& a, int b, int h, QRotIn& in) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4, G = a.G;
  const uint16_t* U = a.u_k + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* qg = a.q + ((size_t)b * a.Hq + h * G) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 v = *reinterpret_cast<const uint4*>(qg + min(n, G - 1) * kHeadDim + 32 * ks + 8 * kg);
    in.bq[ks] = __builtin_bit_cast(bf16x8, n < G ? v : make_uint4(0, 0, 0, 0));
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int d = 0; d < 8; ++d)
        in.bu[t][ks][d] = __builtin_bit_cast(__bf16, U[(32 * ks + 8 * kg + d) * kHeadDim + 16 * (2 * wave + t) + n]);
}

__device__ __forceinline__ void qrot_product(const DecodeArgs& a, const QRotIn& in, QRotLds v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(in.bq[ks], in.bu[t][ks], acc, 0, 0, 0);
    // lane (n, kg) holds heads 4 kg .. 4 kg + 3 of channel 16 nt + n
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kg + i < a.G) v.y[4 * kg + i][16 * (2 * wave + t) + n] = acc[i];
  }
}

// after a block barrier that makes every y visible; wave w finishes heads w, w + 4
__device__ __forceinline__ void qrot_finish(const DecodeArgs& a, QRotLds v) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int g = wave; g < a.G; g += 4) {
    const float2 yy = *reinterpret_cast<const float2*>(&v.y[g][2 * lane]);
    float y0 = yy.x + yy.y, y1 = yy.x - yy.y;   // stage 1: channels 2 l, 2 l + 1
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {           // stages 2 .. 64: lane bit m
      const float sgn = (lane & m) ? -1.f : 1.f;   // upper partner: partner - own
      y0 = fmaf(sgn, y0, lane_xor(y0, m));
      y1 = fmaf(sgn, y1, lane_xor(y1, m));
    }
    *reinterpret_cast<float2*>(&v.y[g][2 * lane]) = make_float2(y0, y1);
    wave_lds_sync();
    float w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * lane + e;
      w[e] = v.y[g][bitrev7(c)] * 0.08838834764831845f * a.sl2e;
      const uint32_t hb = f32_to_f16_bits(w[e]);
      v.qh[g][c] = (uint16_t)hb;
      v.ql[g][c] = (uint16_t)f32_to_f16_bits(w[e] - f16_bits_to_f32(hb));
    }
    *reinterpret_cast<float2*>(&v.y[g][2 * lane]) = make_float2(w[0], w[1]);   // after every lane's reads
    wave_lds_sync();
    const float base = (float)pair_base(pair_of_k(lane & 7));
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {   // lane l takes channel 64 gr + l
      const int c = 64 * gr + lane;
      const float nh = wave_sum_xor(-base * f16_bits_to_f32(v.qh[g][c]), 1, 32);
      const float nl = wave_sum_xor(-base * f16_bits_to_f32(v.ql[g][c]), 1, 32);
      const float qs = wave_sum_xor(v.y[g][c], 1, 32);
      if (lane == 0) {
        v.negc[g][gr][0] = nh;
        v.negc[g][gr][1] = nl;
        v.qsum[g][gr] = qs;
      }
    }
  }
}

// The two fp16 values of register v of fragment (group gr, k-half kh, k-group c) of head g.
__device__ __forceinline__ uint32_t qrot_frag_dword(const QRotLds& v, int g, int gr, int kh, int limb, int c, int vi) {
  const int ch = 64 * gr + 16 * c + pair_k(4 * kh + vi);
  const uint16_t* src = limb ? v.ql[g] : v.qh[g];
  return (uint32_t)src[ch] | ((uint32_t)src[ch + 8] << 16);
}

struct RotQSmem {
  float y[kMaxGqa][kHeadDim];
  uint16_t qh[kMaxGqa][kHeadDim], ql[kMaxGqa][kHeadDim];
  float negc[kMaxGqa][2][2], qsum[kMaxGqa][2];
};

// block for (sequence, KV head) bh = b H + h: the records of its G query heads
__device__ __forceinline__ void rotate_q_block(const DecodeArgs& a, RotQSmem& sm, int bh) {
  const int b = bh / a.H, h = bh % a.H, G = a.G;
  const int tid = threadIdx.x;
  if (a.cas_eff && h == 0 && tid == 0)
    a.cas_eff[b] = a.n_groups > 0 ? cascade_pages_of(a, b, clamp_len(a.seq_lens[b], a.max_pages)) : 0;
  const QRotLds v{sm.y, sm.qh, sm.ql, sm.negc, sm.qsum};
  QRotIn in;
  qrot_load(a, b, h, in);
  qrot_product(a, in, v);
  block_lds_barrier();
  qrot_finish(a, v);
  block_lds_barrier();
  for (int e = tid; e < G * kHeadDim; e += kSideThreads) {
    // dword e of head g: frag index (((gr*2 + kh)*2 + limb)*4 + c)*4 + v
    const int g = e >> 7, jj = e & 127;
    QrotRecord* rec = a.qrot + (size_t)b * a.Hq + h * G + g;
    (&rec->frag[0][0][0][0][0])[jj] =
        qrot_frag_dword(v, g, (jj >> 6) & 1, (jj >> 5) & 1, (jj >> 4) & 1, (jj >> 2) & 3, jj & 3);
  }
  if (tid < G * 6) {
    const int g = tid / 6, k = tid % 6;
    QrotRecord* rec = a.qrot + (size_t)b * a.Hq + h * G + g;
    if (k < 4) rec->negc[k >> 1][k & 1] = sm.negc[g][k >> 1][k & 1];
    else rec->qsum[k - 4] = sm.qsum[g][k - 4];
  }
}

__global__ __launch_bounds__(kSideThreads) void rotate_q_kernel(DecodeArgs a) {
  __shared__ RotQSmem sm;
  rotate_q_block(a, sm, blockIdx.x);
}

// ---------------------------------------------------------------------------
// split: block (item, KV head, sequence), 4 waves.
// ---------------------------------------------------------------------------
constexpr int kMaxPagesPerSplit = 512;
constexpr int kRing = 8;   // pages in flight per wave (LDS ring, even: pages go in pairs)
// while pages j, j+1 are read, the DMAs of pages j+2 .. j+kRing-1 (two instructions each) may be in flight
static_assert(2 * (kRing - 2) == 12, "s_waitcnt vmcnt immediate below assumes kRing == 8");

struct __attribute__((aligned(16))) SplitSmem {
  union {
    uint8_t ring[4][kRing][kBlockBytes];   // INT2 items: per-wave ring of page blocks
    struct {                               // BF16 items (inside wave 0's ring):
      float p[4][kMaxGqa][16];             //   probabilities per token
      uint4 q[kMaxGqa][kHeadDim / 8];      //   the G query rows (bf16)
    } b16;
  };
};

// A wave's (m, l, acc) for the block merge, in the upper half of its own page ring (slots
// 4..7): written as soon as the wave is done, without waiting for the other waves; clear of
// the BF16 probability scratch, which lies in wave 0's lower slots.
struct WaveResult {
  float acc[kMaxGqa][kHeadDim];
  float m[kMaxGqa], l[kMaxGqa];
};
static_assert(sizeof(WaveResult) <= (kRing - kRing / 2) * kBlockBytes, "wave result fits its ring's upper half");
static_assert(sizeof(float) * 4 * kMaxGqa * 16 + 2 * kMaxGqa * kHeadDim <= (kRing / 2) * kBlockBytes,
              "BF16 scratch below wave 0's results");
__device__ __forceinline__ WaveResult& wave_result(SplitSmem& sm, int w) {
  return *reinterpret_cast<WaveResult*>(&sm.ring[w][kRing / 2][0]);
}

template <int G>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs& a, int b, int h, int item,
                                                      SplitSmem& sm) {
  __syncthreads();
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o >> 7, c = o & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wave_result(sm, w).m[hh]);
    float val = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const WaveResult& r = wave_result(sm, w);
      const float e = r.m[hh] == -INFINITY ? 0.f : exp2f(r.m[hh] - M);
      val += e * r.acc[hh][c];
      lsum += e * r.l[hh];
    }
    const size_t rec = (size_t)(b * a.Hq + h * G + hh) * a.n_total + item;
    a.part[rec * kHeadDim + c] = val;   // whole 512-byte record, line-aligned
    if (c == 0) a.part_ml[rec] = make_float2(M, lsum);
  }
}

// BF16 sink + recent tokens, a.bchunk per item; the block's waves take 16-token
// groups round-robin and keep an online softmax across their groups; plain
// (unrotated) q.
template <int G>
__device__ void bf16_item(const DecodeArgs& a, int b, int h, int chunk, int L, SplitSmem& sm) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane >> 2, q = lane & 3;
  const int nsink = min(a.sink, L);
  const int r_lo = L > a.sink ? max(a.sink, L - a.recent) : L;
  const int nb = bf16_token_count(L, a.sink, a.recent);
  const size_t head_row = (size_t)b * a.H + h;

  const int ring0 = r_lo % a.recent;   // ring row of the oldest recent token; rows wrap at most once
  auto row_offset = [&](int jj) -> size_t {   // element offset of BF16 token jj's row
    if (jj < nsink) return (head_row * a.sink + jj) * kHeadDim;
    int row = ring0 + (jj - nsink);
    row = row >= a.recent ? row - a.recent : row;
    return (head_row * a.recent + row) * kHeadDim;
  };
  auto kbuf = [&](int jj) { return jj < nsink ? a.k_sink : a.k_ring; };
  auto vbuf = [&](int jj) { return jj < nsink ? a.v_sink : a.v_ring; };

  float m[G], lsum[G], acc[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    lsum[hh] = 0.f;
    acc[hh][0] = acc[hh][1] = 0.f;
  }
  // one 16-token group per wave and round; the next round's rows are requested before this
  // round's math, so the loads of consecutive rounds overlap
  struct RoundIn {
    uint4 kd[4];       // K row of token t: channels 32q .. 32q + 31
    uint32_t vv[16];   // V rows of the group's 16 tokens: channels 2 lane, + 1
  };
  auto load_round = [&](int round, RoundIn& in) {
    const int jbase = chunk * a.bchunk + 16 * (4 * round + wave);
    const int j = jbase + t;
#pragma unroll
    for (int x = 0; x < 4; ++x) in.kd[x] = make_uint4(0, 0, 0, 0);
    if (j < nb) {
      const uint16_t* krow = kbuf(j) + row_offset(j) + 32 * q;
#pragma unroll
      for (int x = 0; x < 4; ++x) in.kd[x] = load_nt(reinterpret_cast<const uint4*>(krow) + x);
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const int jj = jbase + tt;
      in.vv[tt] = jj < nb ? load_nt(reinterpret_cast<const uint32_t*>(vbuf(jj) + row_offset(jj) + 2 * lane)) : 0u;
    }
  };
  RoundIn nxt;
  load_round(0, nxt);
  // the G query rows, staged in LDS once (read per round without a memory latency)
  {
    const uint4* qg = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.Hq + h * G) * kHeadDim);
    if (threadIdx.x < G * kHeadDim / 8) (&sm.b16.q[0][0])[threadIdx.x] = qg[threadIdx.x];
    __syncthreads();
  }
  const int n_rounds = a.bchunk / 64;
  for (int round = 0; round < n_rounds; ++round) {
    const int jbase = chunk * a.bchunk + 16 * (4 * round + wave);
    if (jbase >= nb) break;   // wave-uniform
    const int j = jbase + t;
    const bool valid = j < nb;
    const RoundIn cur = nxt;
    if (round + 1 < n_rounds && jbase + 64 < nb) load_round(round + 1, nxt);
    const uint4* kd = cur.kd;
    const uint32_t* vv = cur.vv;
    float lg[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float d = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint4 qd = sm.b16.q[hh][4 * q + x];
        d = dot2_bf16(qd.x, kd[x].x, d);
        d = dot2_bf16(qd.y, kd[x].y, d);
        d = dot2_bf16(qd.z, kd[x].z, d);
        d = dot2_bf16(qd.w, kd[x].w, d);
      }
      d += lane_xor(d, 1);
      d += lane_xor(d, 2);
      lg[hh] = valid ? d * a.sl2e : -INFINITY;
    }
    wave_lds_sync();   // the previous group's weights have been read
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float m_new = fmaxf(m[hh], wave_max_xor(lg[hh], 4, 32));   // finite: the group has a token
      const float al = exp2f(m[hh] - m_new);
      const float p = valid ? exp2f(lg[hh] - m_new) : 0.f;
      lsum[hh] = lsum[hh] * al + wave_sum_xor(p, 4, 32);
      acc[hh][0] *= al;
      acc[hh][1] *= al;
      m[hh] = m_new;
      if (q == 0) sm.b16.p[wave][hh][t] = p;
    }
    wave_lds_sync();
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const float v0 = bf16_bits_to_f32(vv[tt] & 0xFFFFu), v1 = bf16_bits_to_f32(vv[tt] >> 16);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = sm.b16.p[wave][hh][tt];   // 0 beyond the last token
        acc[hh][0] = fmaf(p, v0, acc[hh][0]);
        acc[hh][1] = fmaf(p, v1, acc[hh][1]);
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      wave_result(sm, wave).m[hh] = m[hh];
      wave_result(sm, wave).l[hh] = lsum[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    wave_result(sm, wave).acc[hh][2 * lane] = acc[hh][0];
    wave_result(sm, wave).acc[hh][2 * lane + 1] = acc[hh][1];
  }
  merge_waves_and_store<G>(a, b, h, chunk, sm);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ half8 half8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, make_uint4(a, b, c, d));
}
__device__ __forceinline__ half8 half8_of(uint4 u) { return __builtin_bit_cast(half8, u); }

// One 1280-byte page block from global memory (wave-uniform base + per-lane offsets)
// straight into LDS at lds_base: 64 lanes x 16 bytes (global_load_lds_dwordx4), then
// the last 256 bytes as 64 lanes x 4 bytes (global_load_lds_dword), the LDS base of each
// in M0.  Issued as inline assembly so the compiler does not see an LDS write it cannot
// disambiguate from the ring slots being read (it would wait for every outstanding
// load before each LDS read, defeating the prefetch); the loop's own s_waitcnt vmcnt
// orders it (two vector-memory instructions per page).  M0 is saved and restored inside
// the statement, so whatever value the compiler keeps in it survives; one wait state
// between each M0 write and the load that reads it (the compiler puts the same s_nop in
// front of its own LDS-DMA loads; inline assembly is not checked for it).  A load reads
// M0 when it issues, so M0 may be rewritten right after it.  The page stream is loaded
// non-temporal (nt): read once, it would otherwise displace from the caches what is
// reused -- the split-K records, the q' records, U -- and measured 347 -> 328 us per
// call at 28 x 100K.
__device__ __forceinline__ void dma_page_to_lds(const void* sbase, uint32_t voff16, uint32_t voff4,
                                                uint32_t lds_base, uint32_t lds_tail) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5 nt\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %5 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff16), "v"(voff4), "s"(lds_base), "s"(lds_tail), "s"(sbase)
      : "memory");
}
__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return f32_to_f16_bits(a) | (f32_to_f16_bits(b) << 16);
}
// all-reduce max over the four 16-lane rows (lanes with the same lane%16)
__device__ __forceinline__ float rows_max(float x) { return swap32(swap16(x, true), true); }
__device__ __forceinline__ float rows_sum(float x) { return swap32(swap16(x, false), false); }

// Per-lane constants of the INT2 page math (lane l: n = l % 16, r = l / 16; logit MFMA
// column n = 4 hh + a4 with a4 = group gp + 2 limb) and the q' operands of its NQ quads.
template <int NQ>
struct Int2Lane {
  int r, a4, gp, limb;
  int off_kc, off_kp, off_vp, off_vw;   // this lane's byte offsets inside a page block
  uint32_t perm_sel;
  uint32_t wsel[4];
  PairConsts pk;
  ValueMasks<(NQ > 1)> vm;   // one quad: 128 VGPRs for 4 waves per SIMD, no room for them
  float tau;
  half8 qb[NQ][2][2];
  float cinit[NQ], qs[NQ];
};

// The value B operand's dword d holds the codes of token 4r + d as fp16 subnormals,
// code 2^(2d - 24); that token's weights carry c_d = 2^(3 - 2d), so every product is
// 2^-21 p s code.  c enters through the logit: each of the two group terms of token
// 4r + d carries half of log2 c_d, so the lane of token 4r + 2 limb (+ 1) adds
// hoff(limb, 0) (hoff(limb, 1)).  Both offsets and 1 / c are formed from the lane index
// where they are used (the rescale branch, the start and the end of an item), not held in
// registers through the page loop.
__device__ __forceinline__ float hoff(int i) {
  float limb = (float)((__lane_id() >> 1) & 1);
  asm volatile("" : "+v"(limb));   // formed here, not hoisted into a register
  return fmaf(-2.f, limb, i ? 0.5f : 1.5f);
}
__device__ __forceinline__ float inv_c() {   // 1 / c of the lane's token 4r + a4
  return __builtin_amdgcn_ldexpf(1.f, 2 * (int)(__lane_id() & 3) - 3);
}

// Running softmax state of the lane's NQ quads: m (reference maximum), hm[i] = -m / 2 +
// hoff(i), the lane's share of l, the zero-point sums and the value accumulators.  The
// lane's l and zero-point shares are scaled by its c, the accumulators by 2^-21.
template <int NQ>
struct Int2State {
  float m[NQ], hm[NQ][2], lsum[NQ], zs[NQ][2];
  f32x4 acc[NQ][8];
};

// Lane constants (everything but the q' operands) and a zero state.
template <int NQ, bool kOne>
__device__ __forceinline__ void int2_lane_init(Int2Lane<NQ>& L, int lane, float tau) {
  const int n = lane & 15;
  L.r = lane >> 4;
  L.a4 = n & 3;
  L.gp = L.a4 & 1;
  L.limb = L.a4 >> 1;
  const int t0 = 4 * L.r + 2 * L.limb;
  L.off_kc = kKCodes + 32 * n + 4 * L.r;        // token n: code word r of group 0 (+16: group 1)
  // (s, z) of group gp, tokens t0 and t0 + 1; (s0, z0, s1, z1) of token 4r + a4 -- with one
  // 128-channel group per token, its single (s, z) serves both groups
  L.off_kp = kOne ? kKParams + 4 * t0 : kKParams + 8 * t0 + 4 * L.gp;
  L.off_vp = kOne ? kVParams128 + 4 * (4 * L.r + L.a4) : kVParams + 8 * (4 * L.r + L.a4);
  L.off_vw = kVCodes + 4 * n;                   // value code word of channel 16t + n at + 64t
  L.perm_sel = (uint32_t)L.r | (0x0Cu << 8) | ((4u + L.r) << 16) | (0x0Cu << 24);
  L.tau = tau;
  // byte selectors placing the weight limbs in the A operand (v_perm: bytes 4-7 = hi, 0-3 =
  // lo, 0x0C = zero): dword a4 takes the hi limb, dword (a4 + 1) % 4 the lo limb from lane a4 + 1
#pragma unroll
  for (int d = 0; d < 4; ++d) L.wsel[d] = L.a4 == d ? 0x07060504u : ((L.a4 + 1) & 3) == d ? 0x03020100u : 0x0C0C0C0Cu;
}

template <int NQ>
__device__ __forceinline__ void int2_state_init(Int2State<NQ>& st) {
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    st.m[qd] = 0.f;   // set by the first pair, which always takes the rescale branch
    st.hm[qd][0] = hoff(0);
    st.hm[qd][1] = hoff(1);
    st.lsum[qd] = 0.f;
    st.zs[qd][0] = st.zs[qd][1] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[qd][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One pair of INT2 pages (blocks blk0 = logical page pp, blk1 = pp + 1, both in LDS): logits,
// online softmax and value accumulation for the lane's quads.  has1: page pp + 1 exists
// (otherwise its block holds stale bytes and is weighted 0); i_hi: first position past the
// INT2 tokens; first: the pair starts the item (forces the first rescale).
template <int NQ, bool kOne>
__device__ __forceinline__ void int2_pair(Int2State<NQ>& st, const Int2Lane<NQ>& L, const uint8_t* blk0,
                                          const uint8_t* blk1, bool has1, int pp, int i_hi, bool first) {
  struct PageRegs {
    uint32_t kc[2];   // token n: code words r of group 0 and of group 1
    uint32_t kp[2];   // (s, z) of group gp for tokens 4r + 2 limb and + 1
    uint32_t vp[2];   // (s0, z0), (s1, z1) of token 4r + a4
    uint32_t vw[8];   // value code words of channels 16t + n
  } cur[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint8_t* blk = k ? blk1 : blk0;   // without page pp + 1 its block holds stale bytes
    cur[k].kc[0] = *reinterpret_cast<const uint32_t*>(blk + L.off_kc);
    cur[k].kc[1] = *reinterpret_cast<const uint32_t*>(blk + L.off_kc + 16);
    cur[k].kp[0] = *reinterpret_cast<const uint32_t*>(blk + L.off_kp);
    cur[k].kp[1] = *reinterpret_cast<const uint32_t*>(blk + L.off_kp + (kOne ? 4 : 8));
    if constexpr (kOne) {
      cur[k].vp[0] = cur[k].vp[1] = *reinterpret_cast<const uint32_t*>(blk + L.off_vp);
    } else {
      const uint2 v2 = *reinterpret_cast<const uint2*>(blk + L.off_vp);
      cur[k].vp[0] = v2.x;
      cur[k].vp[1] = v2.y;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) cur[k].vw[t] = *reinterpret_cast<const uint32_t*>(blk + L.off_vw + 64 * t);
  }

  // ---- logits: lane (r, hh, a4) ends with token 4r + a4 of head 4 qd + hh ----
  // all MFMA chains of both pages first, so they overlap each other's latency
  f32x4 dq[2][NQ];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t e0[8], e1[8];
    unpack16(cur[k].kc[0], e0, L.pk);
    unpack16(cur[k].kc[1], e1, L.pk);
    const half8 a00 = half8_of(e0[0], e0[1], e0[2], e0[3]), a01 = half8_of(e0[4], e0[5], e0[6], e0[7]);
    const half8 a10 = half8_of(e1[0], e1[1], e1[2], e1[3]), a11 = half8_of(e1[4], e1[5], e1[6], e1[7]);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      f32x4 d = f32x4{L.cinit[qd], L.cinit[qd], L.cinit[qd], L.cinit[qd]};
      d = mfma16(a00, L.qb[qd][0][0], d);
      d = mfma16(a01, L.qb[qd][0][1], d);
      d = mfma16(a10, L.qb[qd][1][0], d);
      d = mfma16(a11, L.qb[qd][1][1], d);
      dq[k][qd] = d;
    }
  }
  float lg[NQ][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const PageRegs& P = cur[k];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const f32x4 d = dq[k][qd];
      // limbs: partner lane ^ 2 holds the other limb of the same group
      const float u0 = d[0] + dpp<kQuadXor2>(d[0]), u1 = d[1] + dpp<kQuadXor2>(d[1]);
      const float u2 = d[2] + dpp<kQuadXor2>(d[2]), u3 = d[3] + dpp<kQuadXor2>(d[3]);
      const float y0 = L.limb ? u2 : u0, y1 = L.limb ? u3 : u1;
      // scale and zero-point term of group gp (tokens 4r + 2 limb, + 1)
      const float x0 = fmaf(f16_bits_to_f32(P.kp[0]), y0, fmaf(f16_bits_to_f32(P.kp[0] >> 16), L.qs[qd], st.hm[qd][0]));
      const float x1 = fmaf(f16_bits_to_f32(P.kp[1]), y1, fmaf(f16_bits_to_f32(P.kp[1] >> 16), L.qs[qd], st.hm[qd][1]));
      // groups: partner lane ^ 1 holds the other group of the same tokens
      const float v0 = x0 + dpp<kQuadXor1>(x0), v1 = x1 + dpp<kQuadXor1>(x1);
      lg[qd][k] = L.gp ? v1 : v0;
    }
  }
  if (!has1 || (pp + 2) * kPage > i_hi) {   // wave-uniform: only the last pair can hold missing tokens
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool ok = (k == 0 || has1) && (pp + k) * kPage + 4 * L.r + L.a4 < i_hi;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) lg[qd][k] = ok ? lg[qd][k] : -INFINITY;
      // the value parameters of a masked slot (this lane's token in the value MFMA and
      // the zero-point sum) may be anything, NaN included: slots at or past the
      // sequence length were never written.  With s = z = 0 they contribute 0 * finite.
      cur[k].vp[0] = ok ? cur[k].vp[0] : 0u;
      cur[k].vp[1] = ok ? cur[k].vp[1] : 0u;
    }
  }

  // ---- online softmax per head (logits are relative to m); rescale only when the max
  // grows by more than tau.  A lane test first: the head maxima are reduced only on the
  // rare pairs that rescale.
  bool need_any = first;
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) need_any |= fmaxf(lg[qd][0], lg[qd][1]) > L.tau;
  if (__any(need_any)) {
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      float pm = fmaxf(lg[qd][0], lg[qd][1]);
      pm = fmaxf(pm, dpp<kQuadXor1>(pm));
      pm = fmaxf(pm, dpp<kQuadXor2>(pm));
      pm = rows_max(pm);   // finite: every pair has a valid token
      const float dm = first || pm > L.tau ? pm : 0.f;
      const float al = first ? 0.f : fast_exp2(-dm);   // the state is still zero: 0, not 2^-dm (may overflow)
      st.m[qd] += dm;
      st.hm[qd][0] = fmaf(-0.5f, st.m[qd], hoff(0));
      st.hm[qd][1] = fmaf(-0.5f, st.m[qd], hoff(1));
      lg[qd][0] -= dm;
      lg[qd][1] -= dm;
      st.lsum[qd] *= al;
      st.zs[qd][0] *= al;
      st.zs[qd][1] *= al;
      const float ai = __shfl(al, 4 * L.r);   // accumulator rows of this lane belong to head hh' = r
#pragma unroll
      for (int t = 0; t < 8; ++t) st.acc[qd][t] *= ai;
    }
  }

  // ---- weights W_g = p s_g of this lane's token in both pages as fp16 hi + lo ----
  // A single fp16 rounding of p s_g would leave a relative error on the code part of the
  // token's value but not on its zero-point part p z_g; the codes' common level (about 1.5)
  // turns that into an error shared by all 64 channels of the group, which the inverse
  // rotation concentrates in one or two output channels.  With hi + lo the products are
  // exact to about 2^-22.  Row (hh, a4) of the value MFMA carries the hi limb of token a4
  // at k-slot a4 and the lo limb of token (a4 + 1) % 4 (from the next lane of the quad)
  // at that token's k-slot; the four rows of a head are summed at the end.
  half8 A[NQ][2];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    const float p0 = fast_exp2(lg[qd][0]), p1 = fast_exp2(lg[qd][1]);
    st.lsum[qd] += p0 + p1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // (s_g, z_g) of the token in each page
      const half2v sz0 = __builtin_bit_cast(half2v, cur[0].vp[g]), sz1 = __builtin_bit_cast(half2v, cur[1].vp[g]);
      st.zs[qd][g] = fmaf(p0, (float)sz0[1], fmaf(p1, (float)sz1[1], st.zs[qd][g]));
      const float ps0 = fmaf(p0, (float)sz0[0], 0.f), ps1 = fmaf(p1, (float)sz1[0], 0.f);
      // hi = fp16(p s) rounded toward zero (one packed conversion for both pages), lo = the
      // rest: hi + lo carries p s to about 2^-21 relative whatever hi's rounding
      const half2v hi2 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(ps0, ps1));
      // (the rest in fp32, then one packed conversion: cheaper than two fp16-result FMAs)
      const half2v lo2 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(fmaf(p0, (float)sz0[0], -(float)hi2[0]),
                                                                              fmaf(p1, (float)sz1[0], -(float)hi2[1])));
      const uint32_t wh = __builtin_bit_cast(uint32_t, hi2);
      // lo of the next lane of the quad (every quad lane has a source)
      const uint32_t wl = (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, lo2), kQuadRot1, 0xF, 0xF, true);
      A[qd][g] = half8_of(__builtin_amdgcn_perm(wh, wl, L.wsel[0]), __builtin_amdgcn_perm(wh, wl, L.wsel[1]),
                          __builtin_amdgcn_perm(wh, wl, L.wsel[2]), __builtin_amdgcn_perm(wh, wl, L.wsel[3]));
    }
  }

  // ---- values ----
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    // slot 4r + d of both pages: the code at bits 2d, 2d + 1 of each half is the fp16
    // subnormal code 2^(2d - 24)
    const uint32_t x = __builtin_amdgcn_perm(cur[1].vw[t], cur[0].vw[t], L.perm_sel);
    const half8 bv = half8_of(x & L.vm.m[0], x & L.vm.m[1], x & L.vm.m[2], x & L.vm.m[3]);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) st.acc[qd][t] = mfma16(A[qd][t >> 2], bv, st.acc[qd][t]);
  }
}

// ---------------------------------------------------------------------------
// Column layout of the INT2 page math for 5..8 query heads per KV head.  The 16 MFMA
// columns are (head, limb): column n is head n % 8 with limb n / 8 of q' in the logit
// MFMAs and limb n / 8 of the value weights in the value MFMAs, so no column holds zeros:
// a page takes 4 logit MFMAs and a pair 8 value MFMAs for all the heads, half of what two
// quads of the decode layout take.  Lane (n, r) holds rows 4r .. 4r + 3 (tokens) of its
// column; of those, the lane "owns" tokens 4r + 2 limb + j (j = 0, 1): it adds the other
// limb's partial logit of those tokens from lane n ^ 8 (a rotation of the 16-lane row by 8),
// forms their logits, probabilities and zero-point sums, and takes the other two tokens'
// probabilities from lane n ^ 8, which owns them.  Lane n's value weights are limb n / 8 of
// c_i p s_g for all four tokens (hi = fp16 rounded toward zero, lo = the rest), so the
// head's output is the sum of its two limb lanes' accumulators, taken once at the end.
// ---------------------------------------------------------------------------
struct ColLane {
  int r, hc, limb;
  uint32_t lmask;     // all ones on the lo-limb lanes (n >= 8)
  uint32_t lmask13;   // the sign, exponent and top 10 mantissa bits of an fp32 on the lo-limb lanes
  int off_kc, off_vw, off_po;   // off_po: byte offset of the own tokens' parameters
  uint32_t perm_sel;
  PairConsts pk;
  ValueMasks<true> vm;
  float tau;
  half8 qb[2][2];   // [group][half]: limb `limb` of q' of head hc, channels 32 (2g + half) + 8r ..
  float cinit[2], qs[2];
};
struct ColState {
  // own token slots j (token 4r + 2 limb + j): hm[j] = log2 c - m, the lane's shares of l and
  // of the zero-point sums (carrying c)
  float m, hm[2], lsum[2], zs[2][2];
  f32x4 acc[8];   // tile t: channels 16t + 4r + i of column n
};

template <bool kOne>
__device__ __forceinline__ void col_lane_init(ColLane& L, int lane, float tau) {
  const int n = lane & 15;
  L.r = lane >> 4;
  L.hc = n & 7;
  L.limb = n >> 3;
  L.lmask = L.limb ? 0xFFFFFFFFu : 0u;
  L.lmask13 = L.limb ? 0xFFFFE000u : 0u;
  asm volatile("" : "+v"(L.lmask), "+v"(L.lmask13));
  L.off_kc = kKCodes + 32 * n + 4 * L.r;   // token n: code word r of group 0 (+16: group 1)
  L.off_vw = kVCodes + 4 * n;              // value code word of channel 16t + n at + 64t
  // (s, z) words of tokens 4r + 2 limb and + 1: 8 bytes per token (one 4-byte word with one
  // 128-channel group per token), K at kKParams + off_po, V at the V parameters + off_po
  L.off_po = (kOne ? 4 : 8) * (4 * L.r + 2 * L.limb);
  L.perm_sel = (uint32_t)L.r | (0x0Cu << 8) | ((4u + L.r) << 16) | (0x0Cu << 24);
  L.tau = tau;
}

__device__ __forceinline__ void col_state_init(ColState& st, int limb) {
  st.m = 0.f;   // set by the first pair, which always takes the rescale branch
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    st.hm[j] = (float)(3 - 4 * limb - 2 * j);   // log2 c of token slot 2 limb + j
    st.lsum[j] = st.zs[0][j] = st.zs[1][j] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <bool kOne>
__device__ __forceinline__ void col_pair(ColState& st, const ColLane& L, const uint8_t* blk0, const uint8_t* blk1,
                                         bool has1, int pp, int i_hi, bool first) {
  const uint8_t* blk[2] = {blk0, blk1};   // without page pp + 1 its block holds stale bytes
  constexpr int kVp = kOne ? kVParams128 : kVParams;
  uint32_t kc[2][2];
  uint32_t kpo[2][2][2];   // [page][j][group]: key (s, z) of own token j
  uint32_t vpo[2][2][2];   // [page][j][group]: value (s, z) of own token j
  uint32_t vp[2][4][2];    // [page][i][group]: value (s, z) of token 4r + i
  uint32_t vw[2][8];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint8_t* bk = blk[k];
    kc[k][0] = *reinterpret_cast<const uint32_t*>(bk + L.off_kc);
    kc[k][1] = *reinterpret_cast<const uint32_t*>(bk + L.off_kc + 16);
    if constexpr (kOne) {   // one (s, z) per token serves both groups
      const uint2 ko = *reinterpret_cast<const uint2*>(bk + kKParams + L.off_po);
      const uint2 vo = *reinterpret_cast<const uint2*>(bk + kVp + L.off_po);
      const uint4 vq = *reinterpret_cast<const uint4*>(bk + kVp + 16 * L.r);
      const uint32_t vv[4] = {vq.x, vq.y, vq.z, vq.w};
      kpo[k][0][0] = kpo[k][0][1] = ko.x;
      kpo[k][1][0] = kpo[k][1][1] = ko.y;
      vpo[k][0][0] = vpo[k][0][1] = vo.x;
      vpo[k][1][0] = vpo[k][1][1] = vo.y;
#pragma unroll
      for (int i = 0; i < 4; ++i) vp[k][i][0] = vp[k][i][1] = vv[i];
    } else {
      const uint4 ko = *reinterpret_cast<const uint4*>(bk + kKParams + L.off_po);
      const uint4 vo = *reinterpret_cast<const uint4*>(bk + kVp + L.off_po);
      const uint4 va = *reinterpret_cast<const uint4*>(bk + kVp + 32 * L.r);
      const uint4 vb = *reinterpret_cast<const uint4*>(bk + kVp + 32 * L.r + 16);
      kpo[k][0][0] = ko.x;
      kpo[k][0][1] = ko.y;
      kpo[k][1][0] = ko.z;
      kpo[k][1][1] = ko.w;
      vpo[k][0][0] = vo.x;
      vpo[k][0][1] = vo.y;
      vpo[k][1][0] = vo.z;
      vpo[k][1][1] = vo.w;
      const uint32_t vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 2; ++g) vp[k][i][g] = vv[2 * i + g];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) vw[k][t] = *reinterpret_cast<const uint32_t*>(bk + L.off_vw + 64 * t);
  }
  // ---- logits of the own tokens of both pages ----
  f32x4 dq[2][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t e0[8], e1[8];
    unpack16(kc[k][0], e0, L.pk);
    unpack16(kc[k][1], e1, L.pk);
    const half8 a00 = half8_of(e0[0], e0[1], e0[2], e0[3]), a01 = half8_of(e0[4], e0[5], e0[6], e0[7]);
    const half8 a10 = half8_of(e1[0], e1[1], e1[2], e1[3]), a11 = half8_of(e1[4], e1[5], e1[6], e1[7]);
    f32x4 d0 = f32x4{L.cinit[0], L.cinit[0], L.cinit[0], L.cinit[0]};
    f32x4 d1 = f32x4{L.cinit[1], L.cinit[1], L.cinit[1], L.cinit[1]};
    d0 = mfma16(a00, L.qb[0][0], d0);
    d1 = mfma16(a10, L.qb[1][0], d1);
    d0 = mfma16(a01, L.qb[0][1], d0);
    d1 = mfma16(a11, L.qb[1][1], d1);
    dq[k][0] = d0;
    dq[k][1] = d1;
  }
  // (the lane's limb as an opaque mask: two-way selects, not an element index)
  const bool lo_lane = L.lmask != 0u;
  float lg[2][2];   // [page][j]
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float y[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        // lane n ^ 8 holds the other limb; it owns the other two tokens
        const float a = dq[k][g][j], b = dq[k][g][2 + j];
        const float snd = lo_lane ? a : b, own = lo_lane ? b : a;
        y[g] = own + dpp<kRowRor8>(snd);
      }
      float x = fmaf(f16_bits_to_f32(kpo[k][j][1] >> 16), L.qs[1], st.hm[j]);
      x = fmaf(f16_bits_to_f32(kpo[k][j][0] >> 16), L.qs[0], x);
      x = fmaf(f16_bits_to_f32(kpo[k][j][1]), y[1], x);
      lg[k][j] = fmaf(f16_bits_to_f32(kpo[k][j][0]), y[0], x);
    }
  if (!has1 || (pp + 2) * kPage > i_hi) {   // wave-uniform: only the last pair can hold missing tokens
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool page_ok = k == 0 || has1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool ok = page_ok && (pp + k) * kPage + 4 * L.r + 2 * L.limb + j < i_hi;
        lg[k][j] = ok ? lg[k][j] : -INFINITY;
        vpo[k][j][0] = ok ? vpo[k][j][0] : 0u;
        vpo[k][j][1] = ok ? vpo[k][j][1] : 0u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // slots at or past the sequence length were never written: s = z = 0 there
        const bool ok = page_ok && (pp + k) * kPage + 4 * L.r + i < i_hi;
        vp[k][i][0] = ok ? vp[k][i][0] : 0u;
        vp[k][i][1] = ok ? vp[k][i][1] : 0u;
      }
    }
  }
  // ---- online softmax of the head (its 8 lanes hold the pair's 32 tokens); rescale only
  // when the maximum grows by more than tau ----
  float pm = fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[1][0], lg[1][1]));
  if (__any(first || pm > L.tau)) {
    pm = rows_max(fmaxf(pm, dpp<kRowRor8>(pm)));   // finite: every pair has a valid token
    const float dm = first || pm > L.tau ? pm : 0.f;
    const float al = first ? 0.f : fast_exp2(-dm);   // the state is still zero: 0, not 2^-dm (may overflow)
    st.m += dm;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st.hm[j] -= dm;
      lg[0][j] -= dm;
      lg[1][j] -= dm;
      st.lsum[j] *= al;
      st.zs[0][j] *= al;
      st.zs[1][j] *= al;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] *= al;
  }
  // ---- probabilities: own tokens here, the other two from lane n ^ 8 ----
  float pa[2][4];   // [page][i]: c_i p of token 4r + i
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float p0 = fast_exp2(lg[0][j]), p1 = fast_exp2(lg[1][j]);
    st.lsum[j] += p0 + p1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const half2v z0 = __builtin_bit_cast(half2v, vpo[0][j][g]), z1 = __builtin_bit_cast(half2v, vpo[1][j][g]);
      st.zs[g][j] = fmaf(p0, (float)z0[1], fmaf(p1, (float)z1[1], st.zs[g][j]));
    }
    const float q0 = dpp<kRowRor8>(p0), q1 = dpp<kRowRor8>(p1);
    pa[0][j] = lo_lane ? q0 : p0;
    pa[1][j] = lo_lane ? q1 : p1;
    pa[0][2 + j] = lo_lane ? p0 : q0;
    pa[1][2 + j] = lo_lane ? p1 : q1;
  }
  // ---- value weights: dword i of group g = limb `limb` of c_i p s_g of token 4r + i in
  // page 0 (low half) and page 1 (high half) ----
  uint32_t w[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = pa[0][i], p1 = pa[1][i];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const half2v sz0 = __builtin_bit_cast(half2v, vp[0][i][g]), sz1 = __builtin_bit_cast(half2v, vp[1][i][g]);
      const float ps0 = fmaf(p0, (float)sz0[0], 0.f), ps1 = fmaf(p1, (float)sz1[0], 0.f);
      // hi-limb lanes: fp16(ps) rounded toward zero.  lo-limb lanes: ps less ps with its low 13
      // mantissa bits cleared (exact), i.e. less the hi lane's fp16 -- the same value wherever ps
      // is in fp16's normal range; below it the two differ by under 2^-24
      const float t0 = ps0 - __uint_as_float(__float_as_uint(ps0) & L.lmask13);
      const float t1 = ps1 - __uint_as_float(__float_as_uint(ps1) & L.lmask13);
      w[g][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(t0, t1));
    }
  }
  const half8 bw[2] = {half8_of(w[0][0], w[0][1], w[0][2], w[0][3]), half8_of(w[1][0], w[1][1], w[1][2], w[1][3])};
  // ---- values: A = the masked subnormal codes of channels 16t + row, B = the weights ----
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t x = __builtin_amdgcn_perm(vw[1][t], vw[0][t], L.perm_sel);
    const half8 av = half8_of(x & L.vm.m[0], x & L.vm.m[1], x & L.vm.m[2], x & L.vm.m[3]);
    st.acc[t] = mfma16(av, bw[t >> 2], st.acc[t]);
  }
}

// INT2 history pages [first, end), two pages (32 tokens) per step; wave w
// takes the pairs starting at first + 2w, + 8, ...  The G query heads are
// handled in quads (NQ = ceil(G / 4)); lane l: n = l % 16, r = l / 16, and
// for the logit MFMA column n = 4 hh + a: head 4 quad + hh, a = g' + 2 limb.
//
// Logits, per page and quad: D[token][column] = sum over the channels of
//   group g' of (base + code) * limb(q')  -- four MFMAs (one per 32-channel
//   slice; a column's B fragment is zero on the other group's slices), the
//   accumulator started at -sum base * limb(q').  A = codes: lane holds token
//   n's code words as unpack16 pairs.  D lands as lane (column n, tokens
//   4r + i).  Two quad exchanges then finish each logit: limbs (lane ^ 2),
//   after which the lane keeps tokens 4r + 2 limb (+1) and applies that
//   group's scale and zero-point term, and groups (lane ^ 1), after which lane
//   (r, hh, a) holds the logit of token 4r + a of head hh: one value per lane.
// Values, per page pair and quad: acc[(hh, j)][channel] += A[(hh, j)][k] *
//   B[k][channel] with k running over the 32 tokens of the pair; row (hh, j)
//   only carries the tokens 4r + j (A dword j holds the fp16 weights of that
//   token in both pages, the other dwords are zero), so each lane's own
//   (token, head) weights feed the MFMA without any exchange; the four rows of
//   a head are summed at the end.  B = channel-major code words of channel
//   16t + n, byte r of each page, masked in place: the code of token 4r + d
//   sits at bits 2d, 2d + 1 of an fp16 half, i.e. it is the subnormal
//   code 2^(2d - 24), taken exactly by the MFMA.  Token 4r + d's weights are
//   c_d p s_g with c_d = 2^(3 - 2d), so every product is 2^-21 p s_g code and
//   no term needs cancelling (all are >= 0).  c_d rides on p itself: the
//   logit of token 4r + d carries log2 c_d (half on each group term), so the
//   lane's shares of l and of the zero-point sums carry c_d too and are
//   divided by it once at the end, where the accumulators are scaled by 2^21.
//   The zero-point term sum p z_g is a per-head scalar.
template <int G, bool kOne>
__device__ void int2_item(const DecodeArgs& a, int b, int h, int split, int first, int end, int i_hi,
                          SplitSmem& sm) {
  constexpr int NQ = (G + 3) / 4;
  constexpr bool kCols = G > 4;   // (head, limb) columns; quads of heads otherwise
  i_hi = __builtin_amdgcn_readfirstlane(i_hi);   // block-uniform: keeps the tail test a scalar branch
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, r = lane >> 4;
  const int hh = n >> 2, a4 = n & 3, gp = a4 & 1, limb = a4 >> 1;
  const int hc = n & 7, climb = n >> 3;   // column layout: head and limb of column n

  // The wave's pages: j -> first + 8 (j / 2) + 2 wave + (j % 2).
  const int base0 = first + 2 * wave;
  int n_w = 0;
  if (base0 < end) n_w = 2 * ((end - base0 + 7) / 8) - ((end - base0 - 1) % 8 == 0 ? 1 : 0);
  auto page_of = [&](int j) { return base0 + 8 * (j >> 1) + (j & 1); };
  constexpr int kIdRegs = kMaxPagesPerSplit / 4 / 64;
  static_assert(kIdRegs == 2, "page offsets in two registers");
  // Every prologue load is issued before any is used, from addresses that are always valid
  // (selects come after), so the block waits one memory latency before its first page DMA:
  // the physical page ids of the wave's pages (lane l: page j = l + 64 k), the q rows and
  // the U_K columns of the block's query rotation.
  int32_t pid_raw[kIdRegs];
  {
    const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) {
      const int j = lane + 64 * k;
      pid_raw[k] = ptab[n_w > 0 ? page_of(min(j, n_w - 1)) : first];
    }
  }
  // zs[g]: per-head zero-point sum of group g's channels, sum over tokens of p z_g; m:
  // running reference maximum of the head's logits, which are formed relative to it
  std::conditional_t<kCols, ColLane, Int2Lane<NQ>> ln;
  std::conditional_t<kCols, ColState, Int2State<NQ>> st;
  if constexpr (kCols) {
    col_lane_init<kOne>(ln, lane, a.resc_thr);
    col_state_init(st, climb);
  } else {
    int2_lane_init<NQ, kOne>(ln, lane, a.resc_thr);
    int2_state_init(st);
  }
  // ---- page blocks stream through a per-wave LDS ring (direct global->LDS loads) ----
  // this lane's bytes of a page block: 16 at 16 lane, then 4 at 1024 + 4 lane (a 1152-byte
  // block's last 128 bytes are read twice, the copy landing past it in the 1280-byte slot)
  const uint32_t off16 = 16 * lane, off4 = 1024 + 4 * (kOne ? (lane & 31) : lane);
  auto issue = [&](const uint32_t (&unit_reg)[kIdRegs], int j, int slot) {   // 2 DMA instructions per page
    const uint32_t u = __builtin_amdgcn_readlane(j < 64 ? unit_reg[0] : unit_reg[1], j & 63);   // wave-uniform
    const uint8_t* row = a.pages + ((uint64_t)u << 7);
    const uint32_t dst = (uint32_t)(uintptr_t)&sm.ring[wave][slot][0];
    dma_page_to_lds(row, off16, off4, dst, dst + 1024);
  };
  // the wave's page blocks as offsets from `pages` in 128-byte units (page id x H x 10 +
  // h x 10: a block is 10 units, 9 with one 128-channel group), held in VGPRs: lane l
  // keeps page j = l + 64 k.  32 bits suffice while the pool is below 512 GiB.
  constexpr uint32_t kUnits = (kOne ? kBlockBytes128 : kBlockBytes) / 128;
  auto unit_offsets = [&](uint32_t (&unit_reg)[kIdRegs]) {
    const uint32_t per_page = (uint32_t)a.H * kUnits, head_units = (uint32_t)h * kUnits;
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) unit_reg[k] = (uint32_t)pid_raw[k] * per_page + head_units;
  };
  // A pair without its second page reads that page's slot anyway and weights it with p = 0;
  // the slot then holds an earlier page of this wave or, before the ring's first turn, the
  // zeros written here, so the value scales it multiplies stay finite.
  static_assert(kRing == 8, "one 16-byte store per lane covers the V parameters of all eight slots");
  auto zero_vparams = [&](bool lower, bool upper) {
    if ((lane >= 32) ? upper : lower)
      *reinterpret_cast<uint4*>(&sm.ring[wave][lane >> 3][(kOne ? kVParams128 : kVParams) + 16 * (lane & 7)]) =
          make_uint4(0, 0, 0, 0);
    wave_lds_sync();   // before any page lands in these slots
  };
  uint32_t unit_reg[kIdRegs];
  if (a.qrot_inline) {
    // ---- the block rotates its own G queries while its first four pages per wave load:
    // scratch in slots 4..7 of the rings of waves 0 (y), 1 (limbs) and 2 (offset sums),
    // which are cleared and filled once every wave holds its fragments ----
    QRotIn qin;
    qrot_load(a, b, h, qin);
    // consume them all here: no wait for them may land after the first page DMA, where it
    // would also wait for every DMA in flight
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) asm volatile("" : "+v"(pid_raw[k]));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      asm volatile("" : "+v"(qin.bq[ks]));
#pragma unroll
      for (int t = 0; t < 2; ++t) asm volatile("" : "+v"(qin.bu[t][ks]));
    }
    unit_offsets(unit_reg);
    zero_vparams(true, false);
    for (int j = 0; j < 4 && j < n_w; ++j) issue(unit_reg, j, j);
    static_assert(sizeof(float) * kMaxGqa * kHeadDim <= 4 * kBlockBytes &&
                      2 * sizeof(uint16_t) * kMaxGqa * kHeadDim <= 4 * kBlockBytes,
                  "rotation scratch fits four ring slots");
    uint8_t* limbs = &sm.ring[1][4][0];
    uint8_t* sums = &sm.ring[2][4][0];
    const QRotLds qv{reinterpret_cast<float(*)[kHeadDim]>(&sm.ring[0][4][0]),
                     reinterpret_cast<uint16_t(*)[kHeadDim]>(limbs),
                     reinterpret_cast<uint16_t(*)[kHeadDim]>(limbs + sizeof(uint16_t) * kMaxGqa * kHeadDim),
                     reinterpret_cast<float(*)[2][2]>(sums),
                     reinterpret_cast<float(*)[2]>(sums + sizeof(float) * kMaxGqa * 4)};
    qrot_product(a, qin, qv);
    block_lds_barrier();
    qrot_finish(a, qv);
    block_lds_barrier();
    if constexpr (kCols) {
      // B fragments of column n: limb climb of head hc, both groups; zero beyond G
      const bool ok = hc < G;
      const int hs = ok ? hc : 0;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const uint4 f = make_uint4(qrot_frag_dword(qv, hs, g, kh, climb, r, 0), qrot_frag_dword(qv, hs, g, kh, climb, r, 1),
                                     qrot_frag_dword(qv, hs, g, kh, climb, r, 2), qrot_frag_dword(qv, hs, g, kh, climb, r, 3));
          ln.qb[g][kh] = half8_of(ok ? f : make_uint4(0, 0, 0, 0));
        }
        ln.cinit[g] = ok ? qv.negc[hs][g][climb] : 0.f;
        ln.qs[g] = ok ? qv.qsum[hs][g] : 0.f;
      }
    } else {
      // B fragments of column n: head 4 qd + hh, group gp, limb; zero on the other group
      // and beyond G
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        const int head = 4 * qd + hh;
        const bool ok = head < G;
        const int hs = ok ? head : 0;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const uint4 f = make_uint4(qrot_frag_dword(qv, hs, gp, kh, limb, r, 0), qrot_frag_dword(qv, hs, gp, kh, limb, r, 1),
                                     qrot_frag_dword(qv, hs, gp, kh, limb, r, 2), qrot_frag_dword(qv, hs, gp, kh, limb, r, 3));
#pragma unroll
          for (int g = 0; g < 2; ++g) ln.qb[qd][g][kh] = half8_of(ok && g == gp ? f : make_uint4(0, 0, 0, 0));
        }
        ln.cinit[qd] = ok ? qv.negc[hs][gp][limb] : 0.f;
        ln.qs[qd] = ok ? qv.qsum[hs][gp] : 0.f;
      }
    }
    block_lds_barrier();   // every wave holds its fragments: slots 4..7 are free
    zero_vparams(false, true);
    for (int j = 4; j < kRing - 2 && j < n_w; ++j) issue(unit_reg, j, j);
  } else if constexpr (kCols) {
    // ---- the q' fragments of column n from the stored record (limb climb of head hc, both
    // groups; zero beyond G), loaded with the page ids ----
    const bool ok = hc < G;
    const QrotRecord* rec = a.qrot + ((size_t)b * a.Hq + h * G + (ok ? hc : 0));
    uint4 qraw[2][2];
    float craw[2], sraw[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) qraw[g][kh] = *reinterpret_cast<const uint4*>(&rec->frag[g][kh][climb][r][0]);
      craw[g] = rec->negc[g][climb];
      sraw[g] = rec->qsum[g];
    }
    // consume them all here: no wait for them may land inside the page loop
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) asm volatile("" : "+v"(pid_raw[k]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        asm volatile("" : "+v"(qraw[g][kh].x), "+v"(qraw[g][kh].y), "+v"(qraw[g][kh].z), "+v"(qraw[g][kh].w));
        ln.qb[g][kh] = half8_of(ok ? qraw[g][kh] : make_uint4(0, 0, 0, 0));
      }
      asm volatile("" : "+v"(craw[g]), "+v"(sraw[g]));
      ln.cinit[g] = ok ? craw[g] : 0.f;
      ln.qs[g] = ok ? sraw[g] : 0.f;
    }
    unit_offsets(unit_reg);
    zero_vparams(true, true);
    for (int j = 0; j < kRing - 2 && j < n_w; ++j) issue(unit_reg, j, j);
  } else {
    // ---- the q' fragments of column n from the stored records (head 4 qd + hh, group gp,
    // limb; zero beyond G), loaded with the page ids ----
    uint4 qraw[NQ][2][2];
    float craw[NQ], sraw[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const int head = 4 * qd + hh;
      const QrotRecord* rec = a.qrot + ((size_t)b * a.Hq + h * G + (head < G ? head : 0));
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) qraw[qd][g][kh] = *reinterpret_cast<const uint4*>(&rec->frag[g][kh][limb][r][0]);
      craw[qd] = rec->negc[gp][limb];
      sraw[qd] = rec->qsum[gp];
    }
    // consume them all here: no wait for them may land inside the page loop, where it would
    // also wait for every page DMA in flight
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) asm volatile("" : "+v"(pid_raw[k]));
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          asm volatile("" : "+v"(qraw[qd][g][kh].x), "+v"(qraw[qd][g][kh].y), "+v"(qraw[qd][g][kh].z),
                       "+v"(qraw[qd][g][kh].w));
      asm volatile("" : "+v"(craw[qd]), "+v"(sraw[qd]));
    }
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const bool ok = 4 * qd + hh < G;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          ln.qb[qd][g][kh] = half8_of(ok && g == gp ? qraw[qd][g][kh] : make_uint4(0, 0, 0, 0));
      ln.cinit[qd] = ok ? craw[qd] : 0.f;
      ln.qs[qd] = ok ? sraw[qd] : 0.f;
    }
    unit_offsets(unit_reg);
    zero_vparams(true, true);
    for (int j = 0; j < kRing - 2 && j < n_w; ++j) issue(unit_reg, j, j);
  }

  // unrolled over one turn of the ring, so every slot offset is an immediate
  for (int j0 = 0; j0 < n_w; j0 += kRing)
#pragma unroll
  for (int u = 0; u < kRing / 2; ++u) {
    const int j = j0 + 2 * u;
    if (j >= n_w) break;   // wave-uniform
    const int pp = page_of(j);
    const bool has1 = j + 1 < n_w;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // earlier reads of the slots being refilled
    if (j + kRing - 2 < n_w) issue(unit_reg, j + kRing - 2, (2 * u + kRing - 2) % kRing);
    if (j + kRing - 1 < n_w) issue(unit_reg, j + kRing - 1, (2 * u + kRing - 1) % kRing);
    if (j + kRing - 1 < n_w) {
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");   // pages j, j+1 landed: 2*(kRing-2) still in flight
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (kCols)
      col_pair<kOne>(st, ln, &sm.ring[wave][2 * u][0], &sm.ring[wave][2 * u + 1][0], has1, pp, i_hi, j == 0);
    else
      int2_pair<NQ, kOne>(st, ln, &sm.ring[wave][2 * u][0], &sm.ring[wave][2 * u + 1][0], has1, pp, i_hi, j == 0);
  }

  // ---- finish the wave: its result goes to its own ring (all of its page loads have landed) ----
  WaveResult& res = wave_result(sm, wave);
  if constexpr (kCols) {
    // per-head totals over the head's 8 lanes (4 rows x the two limb lanes, each holding the
    // shares of its own tokens, which carry c; the accumulators 2^-21 and one limb each)
    float L_h = 0.f, Z0 = 0.f, Z1 = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float ic = __builtin_amdgcn_ldexpf(1.f, 4 * climb + 2 * j - 3);
      L_h = fmaf(st.lsum[j], ic, L_h);
      Z0 = fmaf(st.zs[0][j], ic, Z0);
      Z1 = fmaf(st.zs[1][j], ic, Z1);
    }
    L_h = rows_sum(L_h + dpp<kRowRor8>(L_h));
    Z0 = rows_sum(Z0 + dpp<kRowRor8>(Z0));
    Z1 = rows_sum(Z1 + dpp<kRowRor8>(Z1));
    float o[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] = st.acc[t][i] + dpp<kRowRor8>(st.acc[t][i]);
    if (climb == 0 && hc < G) {
      if (r == 0) {
        res.m[hc] = n_w > 0 ? st.m : -INFINITY;   // a wave without pages contributes nothing
        res.l[hc] = L_h;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float z = t < 4 ? Z0 : Z1;
        *reinterpret_cast<float4*>(&res.acc[hc][16 * t + 4 * r]) =
            make_float4(fmaf(o[t][0], 0x1p21f, z), fmaf(o[t][1], 0x1p21f, z), fmaf(o[t][2], 0x1p21f, z),
                        fmaf(o[t][3], 0x1p21f, z));
      }
    }
  } else {
  #pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      // per-head totals over the 16 lanes of head hh (quad, then rows)
      // (the lane's shares carry its c; the accumulators 2^-21)
      const float ic = inv_c();
      float L_h = st.lsum[qd] * ic, Z0 = st.zs[qd][0] * ic, Z1 = st.zs[qd][1] * ic;
      L_h = rows_sum(quad_sum(L_h));
      Z0 = rows_sum(quad_sum(Z0));
      Z1 = rows_sum(quad_sum(Z1));
      const int head = 4 * qd + hh;
      if (r == 0 && a4 == 0 && head < G) {
        res.m[head] = n_w > 0 ? st.m[qd] : -INFINITY;   // a wave without pages contributes nothing
        res.l[head] = L_h;
      }
      // accumulator rows of this lane: head 4 qd + r, subsets j = 0..3
      const float z0 = __shfl(Z0, 4 * r), z1 = __shfl(Z1, 4 * r);
      const int row_head = 4 * qd + r;
      if (row_head < G) {
  #pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float s = (st.acc[qd][t][0] + st.acc[qd][t][1]) + (st.acc[qd][t][2] + st.acc[qd][t][3]);
          res.acc[row_head][16 * t + n] = fmaf(s, 0x1p21f, t < 4 ? z0 : z1);
        }
      }
    }
  }
  merge_waves_and_store<G>(a, b, h, a.n_bsplit + split, sm);
}

// ---------------------------------------------------------------------------
// Many queries over one range of INT2 pages: pages [first, first + np) of one KV
// head (physical ids in the page-table row ptab) are read once per block into an
// LDS ring of R page slots shared by the four waves, and every wave applies them
// to its own 4 NQ query heads.  Query head e (of n_e) is head h G + e % G of row
// t0 + e / G; the block takes e_block .. e_block + 16 NQ - 1 and wave w the
// heads e_block + 4 NQ w + 4 qd + hh.  Page j is loaded by wave j % 4: before
// a pair is read each wave waits for its own loads of it and the block
// synchronises, which also frees the slots of the pair before for new loads.
// Each (row, head) gets one record, index rec.  Used by extend (rows = chunk
// tokens over the prefix) and by cascade decode (rows = sequences sharing the
// range's pages).
// ---------------------------------------------------------------------------
template <int R>
__device__ __forceinline__ void mq_wait_own_pair(bool all_issued) {
  // of this wave's later loads, (R - 4) / 4 pages (two instructions each) lie among
  // j + 2 .. j + R - 3 once all of those are issued
  static_assert(R == 8 || R == 16, "ring of 8 or 16 slots");
  if (all_issued) {
    if constexpr (R == 8) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <int G, int NQ, int R, bool kOne>
__device__ void mq_int2_range(const DecodeArgs& a, const int32_t* ptab, int h, int first, int np, int i_hi,
                              int t0, int n_e, int e_block, int rec, uint8_t (*ring)[kBlockBytes]) {
  static_assert(R % 4 == 0 && R * 8 <= 256, "whole rounds of the four waves; one thread per V-parameter line");
  i_hi = __builtin_amdgcn_readfirstlane(i_hi);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, r = lane >> 4, hh = n >> 2;
  const int e_wave = e_block + 4 * NQ * wave;
  Int2Lane<NQ> ln;
  int2_lane_init<NQ, kOne>(ln, lane, a.resc_thr);
  // the block offsets (128-byte units) of the pages this wave loads, j = wave + 4 m: lane l
  // holds m = l + 64 k
  constexpr int kIdRegs = kMaxPagesPerSplit / 4 / 64;
  static_assert(kIdRegs == 2, "page offsets in two registers");
  uint32_t unit_reg[kIdRegs];
  {
    constexpr uint32_t kUnits = (kOne ? kBlockBytes128 : kBlockBytes) / 128;
    const uint32_t per_page = (uint32_t)a.H * kUnits, head_units = (uint32_t)h * kUnits;
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k)
      unit_reg[k] = (uint32_t)ptab[first + min(wave + 4 * (lane + 64 * k), np - 1)] * per_page + head_units;
    uint4 qraw[NQ][2][2];
    float craw[NQ], sraw[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const int e_q = e_wave + 4 * qd + hh;
      const bool ok = e_q < n_e;
      const int row = t0 + (ok ? e_q / G : 0), hq = h * G + (ok ? e_q % G : 0);
      const QrotRecord* qr = a.qrot + ((size_t)row * a.Hq + hq);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) qraw[qd][g][kh] = *reinterpret_cast<const uint4*>(&qr->frag[g][kh][ln.limb][r][0]);
      craw[qd] = qr->negc[ln.gp][ln.limb];
      sraw[qd] = qr->qsum[ln.gp];
    }
    // consumed here, before any page load: no wait for them lands in the page loop
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) asm volatile("" : "+v"(unit_reg[k]));
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const bool ok = e_wave + 4 * qd + hh < n_e;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          asm volatile("" : "+v"(qraw[qd][g][kh].x), "+v"(qraw[qd][g][kh].y), "+v"(qraw[qd][g][kh].z),
                       "+v"(qraw[qd][g][kh].w));
          ln.qb[qd][g][kh] = half8_of(ok && g == ln.gp ? qraw[qd][g][kh] : make_uint4(0, 0, 0, 0));
        }
      asm volatile("" : "+v"(craw[qd]), "+v"(sraw[qd]));
      ln.cinit[qd] = ok ? craw[qd] : 0.f;
      ln.qs[qd] = ok ? sraw[qd] : 0.f;
    }
  }
  Int2State<NQ> st;
  int2_state_init(st);
  auto issue = [&](int j) {   // page j of the range (first + j) into slot j % R, by wave j % 4
    if ((j & 3) != wave) return;
    const int m = j >> 2;
    const uint32_t u = __builtin_amdgcn_readlane(m < 64 ? unit_reg[0] : unit_reg[1], m & 63);
    const uint8_t* blk = a.pages + ((uint64_t)u << 7);
    const uint32_t dst = (uint32_t)(uintptr_t)&ring[j % R][0];
    dma_page_to_lds(blk, 16 * lane, 1024 + 4 * (kOne ? (lane & 31) : lane), dst, dst + 1024);
  };
  // the V parameters of every slot start at zero (a missing second page of the last pair is
  // read anyway and weighted 0; its scales must be finite)
  if (threadIdx.x < R * 8)
    *reinterpret_cast<uint4*>(&ring[threadIdx.x >> 3][(kOne ? kVParams128 : kVParams) + 16 * (threadIdx.x & 7)]) =
        make_uint4(0, 0, 0, 0);
  block_lds_barrier();
  for (int j = 0; j < R - 2 && j < np; ++j) issue(j);
  for (int j = 0; j < np; j += 2) {
    mq_wait_own_pair<R>(j + R - 3 < np);
    block_lds_barrier();   // pages j, j + 1 visible to every wave; slots of pair j - 2 no longer read
    if (j + R - 2 < np) issue(j + R - 2);
    if (j + R - 1 < np) issue(j + R - 1);
    int2_pair<NQ, kOne>(st, ln, &ring[j % R][0], &ring[(j + 1) % R][0], j + 1 < np, first + j, i_hi, j == 0);
  }
  // ---- one record per (row, query head) ----
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    // (the lane's shares carry its c; the accumulators 2^-21)
    const float ic = inv_c();
    const float L_h = rows_sum(quad_sum(st.lsum[qd] * ic));
    const float Z0 = rows_sum(quad_sum(st.zs[qd][0] * ic)), Z1 = rows_sum(quad_sum(st.zs[qd][1] * ic));
    const int e_q = e_wave + 4 * qd + hh;
    if (r == 0 && ln.a4 == 0 && e_q < n_e)
      a.part_ml[((size_t)(t0 + e_q / G) * a.Hq + h * G + e_q % G) * a.n_total + rec] = make_float2(st.m[qd], L_h);
    // accumulator rows of this lane: head 4 qd + r of the wave
    const float z0 = __shfl(Z0, 4 * r), z1 = __shfl(Z1, 4 * r);
    const int e_r = e_wave + 4 * qd + r;
    if (e_r < n_e) {
      float* dst = a.part + (((size_t)(t0 + e_r / G) * a.Hq + h * G + e_r % G) * a.n_total + rec) * kHeadDim;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float sum = (st.acc[qd][t][0] + st.acc[qd][t][1]) + (st.acc[qd][t][2] + st.acc[qd][t][3]);
        dst[16 * t + n] = fmaf(sum, 0x1p21f, t < 4 ? z0 : z1);
      }
    }
  }
}

// Many queries over one range of INT2 pages, flash style (chunked prefill): 16 query
// vectors per wave (64 per block) against every page of the range, read once into an LDS
// ring shared by the four waves (page j loaded by wave j % 4).  With queries in the MFMA's
// column dimension a page's codes are unpacked once for 16 queries (the decode layout puts
// (head, group, limb) there and serves 4 heads).  Lane l: n = l % 16 is the lane's query
// (column), r = l / 16 its row group.
//   logits, per page: D_g[token][query] = sum over group g's channels of (base + code) * q'
//     with both limbs of q' accumulated into one D_g (4 MFMAs per group, started at minus
//     the base sums); lane (n, r) gets tokens 4r .. 4r + 3 of query n and forms
//     s_0 D_0 + s_1 D_1 + z_0 sum q'_0 + z_1 sum q'_1 for each.
//   values, per page pair: O^T[channel][query] += V^T[channel][k] W^T[k][query] with the
//     decode's k order (k-slots 8r .. 8r + 7 = tokens 4r .. 4r + 3 of both pages), so B is
//     the lane's own weights W = c_i p s_g (hi and lo limbs as two MFMAs) and A the masked
//     subnormal value codes; tiles 0-3 (group 0 channels) take s_0, tiles 4-7 s_1.
//   c_i = 2^(3 - 2i) for token 4r + i enters through the logit (log2 c_i added); the
//     lane's l and zero-point sums are kept per i and divided by c_i once at the end.
constexpr int kFlashRing = 8;
constexpr int kExtTile = 64;   // query vectors per block (16 per wave)

template <int G, bool kOne>
__device__ void flash_int2_range(const DecodeArgs& a, const int32_t* ptab, int h, int first, int np, int i_hi,
                                 int t0, int n_e, int e_block, int rec, uint8_t (*ring)[kBlockBytes]) {
  constexpr int R = kFlashRing;
  static_assert(R % 4 == 0 && R * 8 <= 256, "whole rounds of the four waves; one thread per V-parameter line");
  i_hi = __builtin_amdgcn_readfirstlane(i_hi);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, r = lane >> 4;
  const int e_q = e_block + 16 * wave + n;   // this lane's query vector
  const bool q_ok = e_q < n_e;
  constexpr int kIdRegs = kMaxPagesPerSplit / 4 / 64;
  static_assert(kIdRegs == 2, "page offsets in two registers");
  uint32_t unit_reg[kIdRegs];
  half8 qb[2][2][2];   // [group][half][limb]: q' of channels 32 (2g + kh) + 8r .. + 8
  float init[2], qs[2];
  {
    constexpr uint32_t kUnits = (kOne ? kBlockBytes128 : kBlockBytes) / 128;
    const uint32_t per_page = (uint32_t)a.H * kUnits, head_units = (uint32_t)h * kUnits;
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k)
      unit_reg[k] = (uint32_t)ptab[first + min(wave + 4 * (lane + 64 * k), np - 1)] * per_page + head_units;
    const int row = t0 + (q_ok ? e_q / G : 0), hq = h * G + (q_ok ? e_q % G : 0);
    const QrotRecord* qr = a.qrot + ((size_t)row * a.Hq + hq);
    uint4 qraw[2][2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int limb = 0; limb < 2; ++limb) qraw[g][kh][limb] = *reinterpret_cast<const uint4*>(&qr->frag[g][kh][limb][r][0]);
    float nc[2][2], qsr[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      nc[g][0] = qr->negc[g][0];
      nc[g][1] = qr->negc[g][1];
      qsr[g] = qr->qsum[g];
    }
    // consumed here, before any page load: no wait for them lands in the page loop
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k) asm volatile("" : "+v"(unit_reg[k]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int limb = 0; limb < 2; ++limb) {
          asm volatile("" : "+v"(qraw[g][kh][limb].x), "+v"(qraw[g][kh][limb].y), "+v"(qraw[g][kh][limb].z),
                       "+v"(qraw[g][kh][limb].w));
          qb[g][kh][limb] = half8_of(q_ok ? qraw[g][kh][limb] : make_uint4(0, 0, 0, 0));
        }
      asm volatile("" : "+v"(nc[g][0]), "+v"(nc[g][1]), "+v"(qsr[g]));
      init[g] = q_ok ? nc[g][0] + nc[g][1] : 0.f;
      qs[g] = q_ok ? qsr[g] : 0.f;
    }
  }
  const PairConsts pk;
  const ValueMasks<true> vm;
  const uint32_t perm_sel = (uint32_t)r | (0x0Cu << 8) | ((4u + r) << 16) | (0x0Cu << 24);
  const int off_kc = kKCodes + 32 * n + 4 * r;   // token n: code word r of group 0 (+16: group 1)
  const int off_vw = kVCodes + 4 * n;            // value code word of channel 16t + n at + 64t
  // running state: m (reference maximum), hmi[i] = log2 c_i - m, per-i shares of l and of
  // the zero-point sums, the value accumulators (tile t: channels 16t + 4r + i of query n)
  float m = 0.f, hmi[4], lsum[4], zs[2][4];
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hmi[i] = 3.f - 2.f * i;
    lsum[i] = zs[0][i] = zs[1][i] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int j) {   // page j of the range (first + j) into slot j % R, by wave j % 4
    if ((j & 3) != wave) return;
    const int mm = j >> 2;
    const uint32_t u = __builtin_amdgcn_readlane(mm < 64 ? unit_reg[0] : unit_reg[1], mm & 63);
    const uint8_t* blk = a.pages + ((uint64_t)u << 7);
    const uint32_t dst = (uint32_t)(uintptr_t)&ring[j % R][0];
    dma_page_to_lds(blk, 16 * lane, 1024 + 4 * (kOne ? (lane & 31) : lane), dst, dst + 1024);
  };
  // the V parameters of every slot start at zero (a missing second page of the last pair is
  // read anyway and weighted 0; its scales must be finite)
  if (threadIdx.x < R * 8)
    *reinterpret_cast<uint4*>(&ring[threadIdx.x >> 3][(kOne ? kVParams128 : kVParams) + 16 * (threadIdx.x & 7)]) =
        make_uint4(0, 0, 0, 0);
  block_lds_barrier();
  for (int j = 0; j < R - 2 && j < np; ++j) issue(j);
  for (int j = 0; j < np; j += 2) {
    mq_wait_own_pair<R>(j + R - 3 < np);
    block_lds_barrier();   // pages j, j + 1 visible to every wave; slots of pair j - 2 no longer read
    if (j + R - 2 < np) issue(j + R - 2);
    if (j + R - 1 < np) issue(j + R - 1);
    const uint8_t* blk[2] = {&ring[j % R][0], &ring[(j + 1) % R][0]};
    const bool has1 = j + 1 < np;
    const int pp = first + j;
    // ---- logits of both pages: lane (n, r) holds tokens 4r + i of query n ----
    float lg[2][4];
    uint2 vpar[2][4];   // value (s0, z0), (s1, z1) of token 4r + i
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint8_t* bk = blk[k];
      uint32_t e0[8], e1[8];
      unpack16(*reinterpret_cast<const uint32_t*>(bk + off_kc), e0, pk);
      unpack16(*reinterpret_cast<const uint32_t*>(bk + off_kc + 16), e1, pk);
      const half8 a00 = half8_of(e0[0], e0[1], e0[2], e0[3]), a01 = half8_of(e0[4], e0[5], e0[6], e0[7]);
      const half8 a10 = half8_of(e1[0], e1[1], e1[2], e1[3]), a11 = half8_of(e1[4], e1[5], e1[6], e1[7]);
      f32x4 d0 = f32x4{init[0], init[0], init[0], init[0]}, d1 = f32x4{init[1], init[1], init[1], init[1]};
      d0 = mfma16(a00, qb[0][0][0], d0);
      d1 = mfma16(a10, qb[1][0][0], d1);
      d0 = mfma16(a00, qb[0][0][1], d0);
      d1 = mfma16(a10, qb[1][0][1], d1);
      d0 = mfma16(a01, qb[0][1][0], d0);
      d1 = mfma16(a11, qb[1][1][0], d1);
      d0 = mfma16(a01, qb[0][1][1], d0);
      d1 = mfma16(a11, qb[1][1][1], d1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * r + i;
        uint32_t k0, k1;   // (s, z) of groups 0 and 1
        if constexpr (kOne) {
          k0 = k1 = *reinterpret_cast<const uint32_t*>(bk + kKParams + 4 * t);
          vpar[k][i].x = vpar[k][i].y = *reinterpret_cast<const uint32_t*>(bk + kVParams128 + 4 * t);
        } else {
          const uint2 kk = *reinterpret_cast<const uint2*>(bk + kKParams + 8 * t);
          k0 = kk.x;
          k1 = kk.y;
          vpar[k][i] = *reinterpret_cast<const uint2*>(bk + kVParams + 8 * t);
        }
        float x = fmaf(f16_bits_to_f32(k1 >> 16), qs[1], hmi[i]);
        x = fmaf(f16_bits_to_f32(k0 >> 16), qs[0], x);
        x = fmaf(f16_bits_to_f32(k1), d1[i], x);
        lg[k][i] = fmaf(f16_bits_to_f32(k0), d0[i], x);
      }
    }
    if (!has1 || (pp + 2) * kPage > i_hi) {   // wave-uniform: only the last pair can hold missing tokens
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (k == 0 || has1) && (pp + k) * kPage + 4 * r + i < i_hi;
          lg[k][i] = ok ? lg[k][i] : -INFINITY;
          vpar[k][i] = ok ? vpar[k][i] : make_uint2(0u, 0u);   // slots never written may hold anything
        }
    }
    // ---- online softmax of query n (its 4 lanes hold the page's 16 tokens); rescale only
    // when the maximum grows by more than tau ----
    float pm = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    if (__any(j == 0 || pm > a.resc_thr)) {
      pm = rows_max(pm);   // finite: every pair has a valid token
      const float dm = j == 0 || pm > a.resc_thr ? pm : 0.f;
      const float al = j == 0 ? 0.f : fast_exp2(-dm);   // the state is still zero: 0, not 2^-dm (may overflow)
      m += dm;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hmi[i] -= dm;
        lg[0][i] -= dm;
        lg[1][i] -= dm;
        lsum[i] *= al;
        zs[0][i] *= al;
        zs[1][i] *= al;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= al;
    }
    // ---- weights W_g = c_i p s_g as fp16 hi + lo of both pages (dword i: page 0, page 1) ----
    uint32_t whi[2][4], wlo[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(lg[0][i]), p1 = fast_exp2(lg[1][i]);
      lsum[i] += p0 + p1;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t v0 = g ? vpar[0][i].y : vpar[0][i].x, v1 = g ? vpar[1][i].y : vpar[1][i].x;
        const half2v sz0 = __builtin_bit_cast(half2v, v0), sz1 = __builtin_bit_cast(half2v, v1);
        zs[g][i] = fmaf(p0, (float)sz0[1], fmaf(p1, (float)sz1[1], zs[g][i]));
        const float ps0 = fmaf(p0, (float)sz0[0], 0.f), ps1 = fmaf(p1, (float)sz1[0], 0.f);
        const half2v hi2 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(ps0, ps1));
        const half2v lo2 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(fmaf(p0, (float)sz0[0], -(float)hi2[0]),
                                                                                fmaf(p1, (float)sz1[0], -(float)hi2[1])));
        whi[g][i] = __builtin_bit_cast(uint32_t, hi2);
        wlo[g][i] = __builtin_bit_cast(uint32_t, lo2);
      }
    }
    const half8 bhi[2] = {half8_of(whi[0][0], whi[0][1], whi[0][2], whi[0][3]),
                          half8_of(whi[1][0], whi[1][1], whi[1][2], whi[1][3])};
    const half8 blo[2] = {half8_of(wlo[0][0], wlo[0][1], wlo[0][2], wlo[0][3]),
                          half8_of(wlo[1][0], wlo[1][1], wlo[1][2], wlo[1][3])};
    // ---- values ----
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t x = __builtin_amdgcn_perm(*reinterpret_cast<const uint32_t*>(blk[1] + off_vw + 64 * t),
                                               *reinterpret_cast<const uint32_t*>(blk[0] + off_vw + 64 * t), perm_sel);
      const half8 av = half8_of(x & vm.m[0], x & vm.m[1], x & vm.m[2], x & vm.m[3]);
      acc[t] = mfma16(av, bhi[t >> 2], acc[t]);
      acc[t] = mfma16(av, blo[t >> 2], acc[t]);
    }
  }
  // ---- one record per query vector: (m, l) and acc = 2^21 O + the zero-point sum of the
  // channel's group; the lane's shares divided by c_i, summed over the query's 4 lanes ----
  float L = 0.f, Z[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ic = __builtin_amdgcn_ldexpf(1.f, 2 * i - 3);
    L = fmaf(lsum[i], ic, L);
    Z[0] = fmaf(zs[0][i], ic, Z[0]);
    Z[1] = fmaf(zs[1][i], ic, Z[1]);
  }
  L = rows_sum(L);
  Z[0] = rows_sum(Z[0]);
  Z[1] = rows_sum(Z[1]);
  if (q_ok) {
    const size_t rr = ((size_t)(t0 + e_q / G) * a.Hq + h * G + e_q % G) * a.n_total + rec;
    if (r == 0) a.part_ml[rr] = make_float2(m, L);
    float* dst = a.part + rr * kHeadDim;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float z = Z[t >> 2];
      *reinterpret_cast<float4*>(dst + 16 * t + 4 * r) =
          make_float4(fmaf(acc[t][0], 0x1p21f, z), fmaf(acc[t][1], 0x1p21f, z), fmaf(acc[t][2], 0x1p21f, z),
                      fmaf(acc[t][3], 0x1p21f, z));
    }
  }
}

// Cascade block w (< n_cas): shared range k of group g, KV head h, query tile qt, with the
// pages of the group's first member's table row.  5..8 query heads per KV head: tiles of
// 64 query vectors in the MFMA columns (the flash layout, which fits the 3 waves per SIMD
// of that split kernel); up to 4: 16 query heads in quads (which fit its 4 waves per SIMD).
template <int G, bool kOne>
__device__ void cascade_block(const DecodeArgs& a, int w, SplitSmem& sm) {
  constexpr int NQ = (G + 3) / 4;
  constexpr bool kFlash = G > 4;
  const int qt = w % a.n_cqt;
  w /= a.n_cqt;
  const int k = w % a.n_sh;
  w /= a.n_sh;
  const int h = w % a.H, g = w / a.H;
  int m0, members, shared;
  cascade_group(a, g, m0, members, shared);
  const int first = a.sink / kPage + k * a.P;
  const int end = min(first + a.P, a.sink / kPage + shared);
  const int e_block = (kFlash ? kExtTile : 16 * NQ) * qt;
  if (first >= end || e_block >= members * G) return;   // block-uniform
  static_assert(sizeof(sm.ring) >= 16 * kBlockBytes, "a 16-slot ring inside the split kernel's LDS");
  const int32_t* ptab = a.page_table + (size_t)m0 * a.max_pages;
  uint8_t(*ring)[kBlockBytes] = reinterpret_cast<uint8_t(*)[kBlockBytes]>(&sm.ring[0][0][0]);
  const int i_hi = (a.sink / kPage + shared) * kPage, rec = a.n_bsplit + a.n_split + k;
  if constexpr (kFlash)
    flash_int2_range<G, kOne>(a, ptab, h, first, end - first, i_hi, m0, members * G, e_block, rec, ring);
  else
    mq_int2_range<G, NQ, 16, kOne>(a, ptab, h, first, end - first, i_hi, m0, members * G, e_block, rec, ring);
}

template <int G, bool kOne>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3))) void split_kernel(DecodeArgs a) {
  __shared__ SplitSmem sm;
  // 1D grid: every (sequence, KV head)'s INT2 ranges first, then all BF16 chunks, which are
  // short and fill the block slots the last INT2 ranges leave idle (measured 1.7% faster
  // than a (sequence, KV head)-major order at 28 x 100K)
  if ((int)blockIdx.x < a.n_cas) {   // cascade decode: shared prefix ranges come first
    cascade_block<G, kOne>(a, blockIdx.x, sm);
    return;
  }
  const int nbh = a.B * a.H, w = blockIdx.x - a.n_cas, n_int2 = nbh * a.n_split;
  const int bh = w < n_int2 ? w / a.n_split : (w - n_int2) / a.n_bsplit;
  const int item = w < n_int2 ? a.n_bsplit + (w - bh * a.n_split) : (w - n_int2) - bh * a.n_bsplit;
  const int b = bh / a.H, h = bh - b * a.H;
  const int L = clamp_len(a.seq_lens[b], a.max_pages);
  if (item < a.n_bsplit) {
    if (item * a.bchunk >= bf16_token_count(L, a.sink, a.recent)) return;
    bf16_item<G>(a, b, h, item, L, sm);
  } else {
    const int split = item - a.n_bsplit;
    const int i_hi = int2_end(L, a.sink, a.recent);
    const int shared = a.cas_eff ? a.cas_eff[b] : 0;   // pages a cascade block reads for this sequence
    const int first = a.sink / kPage + shared + split * a.P;
    const int end = min(first + a.P, (i_hi + kPage - 1) / kPage);
    if (i_hi <= a.sink || first >= end) return;
    int2_item<G, kOne>(a, b, h, split, first, end, i_hi, sm);
  }
}

// ---------------------------------------------------------------------------
// reduce: one 256-thread block per (sequence, KV head, group of GB query
// heads).  The (m, l) of every used record are staged in LDS and each head's
// maximum taken first, so the merge needs no running rescale; wave w then
// requests every record u = w (mod 4) of the GB heads at once (lane l:
// channels 2l, 2l + 1) and sums them with weights 2^(m_u - M).  The four
// waves' sums meet in LDS; wave g finishes head g: acc_rot P H by an in-wave
// Walsh-Hadamard transform, split into three bf16 limbs (hi + mid + lo carry
// the fp32 value).  (acc_rot P H) U_V^T runs on v_mfma_f32_16x16x32_bf16: A
// rows = (head, limb), B = rows of U_V read straight from global memory (row c
// of U_V is column c of U_V^T, contiguous), so each wave produces 32 output
// channels of all GB heads; plain (BF16-region) sum added, divided by l, bf16.
// ---------------------------------------------------------------------------
constexpr int kRedMaxRec = kMaxItems;   // records per (sequence, query head) the reduce accepts

template <int GB>
struct ReduceSmem {
  float2 ml[GB][kRedMaxRec];                 // (m, l) of every used record
  float part_rot[4][GB][kHeadDim];           // per-wave sums
  float part_pl[4][GB][kHeadDim];
  float part_l[4][GB];
  float y[4][kHeadDim];                      // per-wave scratch of the bit reversal
  __attribute__((aligned(16))) uint16_t ya[16][kHeadDim + 8];   // A operand: row 4 g + limb (bf16)
  float plain[GB][kHeadDim];
  float lsum[GB];
};

template <int G, int GB>
__global__ __launch_bounds__(256) void reduce_kernel(DecodeArgs a) {
  static_assert(G % GB == 0 && GB <= 4, "whole head groups of at most four heads per block");
  __shared__ ReduceSmem<GB> sm;
  const int bhg = blockIdx.x, bh = bhg / (G / GB), gq = bhg % (G / GB), b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int head0 = h * G + gq * GB;   // first query head of this block
  const int L = clamp_len(scalar_load_i32(a.seq_lens, b), a.max_pages);
  // B fragments of the final product, requested first: wave w makes output channels
  // 32 w .. 32 w + 31 (column tiles nt = 2 w + t); lane (n, kg) holds U_V[16 nt + n][32 ks + 8 kg, + 8)
  bf16x8 ub[2][4];
  {
    const uint16_t* U = a.u_v + (size_t)h * kHeadDim * kHeadDim;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        ub[t][ks] = *reinterpret_cast<const bf16x8*>(U + (32 * wave + 16 * t + n) * kHeadDim + 32 * ks + 8 * kg);
  }
  // The records are requested once the sequence length is known (a scalar load issued first,
  // short next to a record's latency), so a short sequence reads only its used records:
  // requesting a full-length sequence's records before the length arrived cost the ragged
  // 64 x [4K, 128K] batch 25 us of reduce against 20 us, and saved nothing at 28 x 100K
  constexpr int kBatch = GB == 1 ? 32 : 8;   // records per head requested at once by a wave
  const float* head_base[GB];
#pragma unroll
  for (int g = 0; g < GB; ++g) head_base[g] = a.part + ((size_t)b * a.Hq + head0 + g) * a.n_total * kHeadDim;
  float2 v[GB][kBatch];
  if (L == 0 && !a.ext) {
    for (int e = tid; e < GB * kHeadDim; e += 256) a.out[((size_t)b * a.Hq + head0) * kHeadDim + e] = 0;
    return;
  }
  const int n_b = a.ext ? 1 : (bf16_token_count(L, a.sink, a.recent) + a.bchunk - 1) / a.bchunk;
  const int i_hi = int2_end(L, a.sink, a.recent);
  const int int2_pages = i_hi > a.sink ? (i_hi + kPage - 1) / kPage - a.sink / kPage : 0;
  const int shared = a.cas_eff ? a.cas_eff[b] : 0;   // of which read by cascade blocks
  const int n_i = (int2_pages - shared + a.P - 1) / a.P;
  const int n_bi = n_b + n_i;
  const int n_used = n_bi + (shared + a.P - 1) / a.P;
  // used records: [0, n_b) BF16, [n_bsplit, n_bsplit + n_i) the sequence's own INT2 ranges,
  // then from n_bsplit + n_split the shared ranges
  auto idx_of = [&](int u) { return u < n_b ? u : u < n_bi ? a.n_bsplit + (u - n_b) : a.n_bsplit + a.n_split + (u - n_bi); };
  auto rec_of = [&](int g, int u) { return ((size_t)b * a.Hq + head0 + g) * a.n_total + idx_of(u); };
  auto load_batch = [&](int u0, float2 (&vb)[GB][kBatch]) {
#pragma unroll
    for (int g = 0; g < GB; ++g)
#pragma unroll
      for (int d = 0; d < kBatch; ++d) {
        const int u = u0 + 4 * d;
        const int idx = idx_of(u);
        vb[g][d] = u < n_used ? *reinterpret_cast<const float2*>(head_base[g] + (idx * kHeadDim + 2 * lane))
                              : make_float2(0.f, 0.f);
      }
  };
  {
    // (m, l) of every record into LDS; the first 256 are requested before this wave's records,
    // so the wait for them leaves the record loads in flight
    const bool ml0_ok = tid < GB * n_used;
    const int g0 = ml0_ok ? tid / n_used : 0, u0_ = ml0_ok ? tid - g0 * n_used : 0;
    const float2 ml0 = a.part_ml[rec_of(g0, u0_)];
    load_batch(wave, v);
    if (ml0_ok) sm.ml[g0][u0_] = ml0;
  }
  for (int e = tid + 256; e < GB * n_used; e += 256) {   // more than 256 records: long sequences
    const int g = e / n_used, u = e - g * n_used;
    sm.ml[g][u] = a.part_ml[rec_of(g, u)];
  }
  __syncthreads();
  float M[GB];
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    float m = -INFINITY;
    for (int u = lane; u < n_used; u += 64) m = fmaxf(m, sm.ml[g][u].x);
    M[g] = wave_max_xor(m, 1, 32);   // finite: every used BF16 item has a token
  }
  float rot[GB][2], pl[GB][2], lw[GB];
#pragma unroll
  for (int g = 0; g < GB; ++g) rot[g][0] = rot[g][1] = pl[g][0] = pl[g][1] = lw[g] = 0.f;
  for (int u0 = wave; u0 < n_used; u0 += 4 * kBatch) {
    if (u0 != wave) load_batch(u0, v);   // more records than one batch (long sequences)
#pragma unroll
    for (int g = 0; g < GB; ++g)
#pragma unroll
      for (int d = 0; d < kBatch; ++d) {
        const int u = u0 + 4 * d;
        if (u < n_used) {   // wave-uniform
          const float2 ml = sm.ml[g][u];
          const float e = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M[g]);
          lw[g] = fmaf(e, ml.y, lw[g]);
          if (u < n_b) {
            pl[g][0] = fmaf(e, v[g][d].x, pl[g][0]);
            pl[g][1] = fmaf(e, v[g][d].y, pl[g][1]);
          } else {
            rot[g][0] = fmaf(e, v[g][d].x, rot[g][0]);
            rot[g][1] = fmaf(e, v[g][d].y, rot[g][1]);
          }
        }
      }
  }
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    *reinterpret_cast<float2*>(&sm.part_rot[wave][g][2 * lane]) = make_float2(rot[g][0], rot[g][1]);
    *reinterpret_cast<float2*>(&sm.part_pl[wave][g][2 * lane]) = make_float2(pl[g][0], pl[g][1]);
    if (lane == 0) sm.part_l[wave][g] = lw[g];
  }
  __syncthreads();
  // ---- wave g: head g's sums, bit reversal, Walsh-Hadamard, bf16 limbs ----
  if (wave < GB) {
    const int g = wave;
    float r0 = 0.f, r1 = 0.f, p0 = 0.f, p1 = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 rr = *reinterpret_cast<const float2*>(&sm.part_rot[w][g][2 * lane]);
      const float2 pp = *reinterpret_cast<const float2*>(&sm.part_pl[w][g][2 * lane]);
      r0 += rr.x;
      r1 += rr.y;
      p0 += pp.x;
      p1 += pp.y;
      l += sm.part_l[w][g];
    }
    *reinterpret_cast<float2*>(&sm.plain[g][2 * lane]) = make_float2(p0, p1);
    if (lane == 0) sm.lsum[g] = l;
    // acc_rot P: z-space channel br(c) takes post-rotation channel c
    sm.y[g][bitrev7(2 * lane)] = r0;
    sm.y[g][bitrev7(2 * lane + 1)] = r1;
    wave_lds_sync();
    float y0 = sm.y[g][2 * lane], y1 = sm.y[g][2 * lane + 1];
    {   // Walsh-Hadamard: index bit 0 in registers, bits 1..6 = lane bits 0..5
      const float t0 = y0 + y1, t1 = y0 - y1;
      y0 = t0;
      y1 = t1;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float sgn = (lane & m) ? -1.f : 1.f;   // upper partner: partner - own
      y0 = fmaf(sgn, y0, lane_xor(y0, m));
      y1 = fmaf(sgn, y1, lane_xor(y1, m));
    }
    // three bf16 limbs of each value: rows 4 g + limb of the A operand
    const float ys[2] = {y0, y1};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t hi = f32_to_bf16_bits(ys[k]);
      const float r1v = ys[k] - bf16_bits_to_f32(hi);
      const uint32_t mid = f32_to_bf16_bits(r1v);
      const uint32_t lo = f32_to_bf16_bits(r1v - bf16_bits_to_f32(mid));
      sm.ya[4 * g][2 * lane + k] = (uint16_t)hi;
      sm.ya[4 * g + 1][2 * lane + k] = (uint16_t)mid;
      sm.ya[4 * g + 2][2 * lane + k] = (uint16_t)lo;
      sm.ya[4 * g + 3][2 * lane + k] = 0;
    }
  } else if (wave < 4) {
    for (int r = 4 * GB; r < 16; ++r) {   // rows of heads this block does not have
      sm.ya[r][2 * lane] = 0;
      sm.ya[r][2 * lane + 1] = 0;
    }
  }
  __syncthreads();
  // ---- (acc_rot P H) U_V^T: lane (n, kg) ends with rows 4 kg .. 4 kg + 3 = head kg's limbs ----
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sm.ya[n][32 * ks + 8 * kg]);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ub[t][ks], d, 0, 0, 0);
    }
    const int c = 32 * wave + 16 * t + n;
    if (kg < GB) {
      const float o = (d[0] + d[1]) + d[2];
      const float res = (sm.plain[kg][c] + o * 0.08838834764831845f) / sm.lsum[kg];
      a.out[((size_t)b * a.Hq + head0 + kg) * kHeadDim + c] = (uint16_t)f32_to_bf16_bits(res);
    }
  }
}

// ---------------------------------------------------------------------------
// extend (chunked prefill): the queries of a chunk attend to the cached
// prefix as stored and causally to the chunk's own BF16 keys.  Rows are chunk
// tokens (global index t); each (row, query head) gets one BF16 record (index
// 0: sink rows, ring rows and chunk keys) and one record per INT2 range of the
// prefix (indices 1 ..), merged by reduce_kernel in extend mode.
// ---------------------------------------------------------------------------
struct ExtArgs {
  DecodeArgs d;                 // qrot / part / part_ml over rows = chunk tokens; seq_lens -> row_len
  const uint16_t *k_new, *v_new;   // bf16 [T][H][128]
  const int32_t *cu, *prefix_lens;
  int32_t* row_len;             // [T]: prefix length of the row's sequence (written by the BF16 kernel)
  int32_t n_seq, n_tok, max_chunk;
  int32_t n_qt;                 // tiles of kExtTile query vectors per (sequence, KV head)
};

// Sequence b's chunk: tokens t0 .. t0 + chunk - 1, clamped to [0, n_tok) and to at most
// max_chunk tokens (the grids cover no more), so inconsistent offsets cannot send a write
// past the output.
__device__ __forceinline__ void chunk_of(const ExtArgs& e, int b, int& t0, int& chunk) {
  t0 = min(max(scalar_load_i32(e.cu, b), 0), e.n_tok);
  chunk = min(min(scalar_load_i32(e.cu, b + 1) - t0, e.max_chunk), e.n_tok - t0);
  chunk = max(chunk, 0);
}

constexpr int kMqRing = 8;   // pages per block ring of the multi-query INT2 kernels
static_assert(kFlashRing == kMqRing, "one ring type");

struct __attribute__((aligned(16))) MqSmem {
  uint8_t ring[kMqRing][kBlockBytes];
};

// INT2 prefix pages of one range of one (sequence, KV head), read once per block for 64 query
// vectors of the sequence's chunk (query vector e = chunk position * G + head in the group),
// 16 per wave with the queries in the MFMA's column dimension.
template <int G, bool kOne>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void ext_int2_kernel(ExtArgs e) {
  __shared__ MqSmem sm;
  const DecodeArgs& a = e.d;
  int job = blockIdx.x;
  const int qt = job % e.n_qt;
  job /= e.n_qt;
  const int split = job % a.n_split;
  job /= a.n_split;
  const int h = job % a.H, b = job / a.H;
  int t0, chunk;
  chunk_of(e, b, t0, chunk);
  const int L = clamp_len(scalar_load_i32(e.prefix_lens, b), a.max_pages);
  const int i_hi = int2_end(L, a.sink, a.recent);
  const int first = a.sink / kPage + split * a.P;
  const int end = min(first + a.P, (i_hi + kPage - 1) / kPage);
  const int e_block = kExtTile * qt;
  if (i_hi <= a.sink || first >= end || e_block >= chunk * G) return;   // block-uniform
  flash_int2_range<G, kOne>(a, a.page_table + (size_t)b * a.max_pages, h, first, end - first, i_hi, t0, chunk * G,
                            e_block, 1 + split, sm.ring);
}

// BF16 keys of a chunk query: the prefix's sink rows [0, min(sink, L)), its ring rows
// [max(sink, L - recent), L) as stored, and the chunk's keys 0..i from the input (causal).
// Flash layout on MFMA: block (sequence, KV head, tile of kExtTile query vectors), 16 query
// vectors per wave in the MFMA columns (query vector e = chunk position * G + head), 16 keys
// per round:
//   logits: D[key][query] = K[key] . q (4 v_mfma_f32_16x16x32_bf16, A = the key rows straight
//     from global memory, B = the queries' bf16 rows); lane (n, r) gets keys 4r .. 4r + 3 of
//     query n and masks those past the query's causal end;
//   values: O^T[channel][query] += V^T[channel][key] P^T[key][query]
//     (v_mfma_f32_16x16x16_bf16, B = the lane's own probabilities as bf16 hi + lo limbs, A =
//     the round's V rows gathered from an LDS copy), so each lane's rows are its own query's
//     channels 16t + 4r .. 4r + 3 and a rescale needs no exchange.
// The next round's key and value rows are requested before this round's math.
constexpr int kExtVRow = kHeadDim + 8;   // bf16 per LDS row of the value copy (padded)

struct __attribute__((aligned(16))) ExtB16Smem {
  uint16_t v[4][16][kExtVRow];
};

__device__ __forceinline__ uint32_t bf16_hi_pair(float a, float b) {   // truncated bf16 of a (lo), b (hi)
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

template <int G>
__global__ __launch_bounds__(256) void ext_bf16_kernel(ExtArgs e) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  __shared__ ExtB16Smem sm;
  const DecodeArgs& a = e.d;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, r = lane >> 4;
  int job = blockIdx.x;
  const int qt = job % e.n_qt;
  job /= e.n_qt;
  const int h = job % a.H, b = job / a.H;
  int t0, chunk;
  chunk_of(e, b, t0, chunk);
  const int L = clamp_len(scalar_load_i32(e.prefix_lens, b), a.max_pages);
  const int n_e = chunk * G;
  const int e_wave = kExtTile * qt + 16 * wave;
  if (e_wave >= n_e) return;   // wave-uniform; nothing below synchronises the block
  const int e_q = e_wave + n;
  const bool q_ok = e_q < n_e;
  const int i_q = q_ok ? e_q / G : 0, g_q = q_ok ? e_q % G : 0;
  if (h == 0 && r == 0 && q_ok && g_q == 0) e.row_len[t0 + i_q] = L;
  const int ns = min(a.sink, L);
  const int r_lo = L > a.sink ? max(a.sink, L - a.recent) : L;
  const int nr = L - r_lo;
  const int ring0 = a.recent > 0 ? r_lo % a.recent : 0;
  const int nk_q = ns + nr + i_q + 1;   // keys of this lane's query (a padding column: 1 + ...)
  const int nk = __builtin_amdgcn_readfirstlane(ns + nr + (min(e_wave + 15, n_e - 1) / G) + 1);   // wave's keys
  const size_t head_row = (size_t)b * a.H + h;
  auto key_row = [&](int j, const uint16_t* sink_buf, const uint16_t* ring_buf, const uint16_t* chunk_buf) {
    if (j < ns) return sink_buf + (head_row * a.sink + j) * kHeadDim;
    if (j < ns + nr) {
      int rr = ring0 + (j - ns);
      rr = rr >= a.recent ? rr - a.recent : rr;
      return ring_buf + (head_row * a.recent + rr) * kHeadDim;
    }
    return chunk_buf + ((size_t)(t0 + j - ns - nr) * a.H + h) * kHeadDim;
  };
  // this lane's query as B fragments (channels 32 ks + 8 r ..)
  bf16x8 qf[4];
  {
    const uint16_t* qrow = a.q + ((size_t)(t0 + i_q) * a.Hq + h * G + g_q) * kHeadDim + 8 * r;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  struct RoundIn {
    uint4 k[4];   // key row jbase + n, channels 32 ks + 8 r ..
    uint4 v[4];   // value row jbase + lane / 4, channels 32 (lane % 4) ..
  };
  auto load_round = [&](int jbase, RoundIn& in) {
    const uint16_t* krow = key_row(min(jbase + n, nk - 1), a.k_sink, a.k_ring, e.k_new) + 8 * r;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) in.k[ks] = *reinterpret_cast<const uint4*>(krow + 32 * ks);
    const uint16_t* vrow = key_row(min(jbase + (lane >> 2), nk - 1), a.v_sink, a.v_ring, e.v_new) + 32 * (lane & 3);
#pragma unroll
    for (int x = 0; x < 4; ++x) in.v[x] = *reinterpret_cast<const uint4*>(vrow + 8 * x);
  };
  float m = 0.f, lsum = 0.f;   // m: reference maximum (set by the first round)
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t(*vs)[kExtVRow] = sm.v[wave];
  RoundIn nxt;
  load_round(0, nxt);
  for (int jbase = 0; jbase < nk; jbase += 16) {
    const RoundIn cur = nxt;
    if (jbase + 16 < nk) load_round(jbase + 16, nxt);
    // the round's value rows into this wave's LDS copy (the previous round's reads of it
    // were issued before these writes, and LDS serves one wave's operations in order)
#pragma unroll
    for (int x = 0; x < 4; ++x) *reinterpret_cast<uint4*>(&vs[lane >> 2][32 * (lane & 3) + 8 * x]) = cur.v[x];
    // ---- logits of keys jbase + 4r + i for query n ----
    f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[ks]), qf[ks], d, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jbase + 4 * r + i;
      x[i] = j < (q_ok ? nk_q : 1) ? fmaf(d[i], a.sl2e, -m) : -INFINITY;
    }
    // ---- online softmax of query n; rescale only when the maximum grows by more than 8 ----
    float pm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__any(jbase == 0 || pm > 8.f)) {
      pm = rows_max(pm);   // finite: key 0 is valid for every query
      const float dm = jbase == 0 || pm > 8.f ? pm : 0.f;
      const float al = jbase == 0 ? 0.f : fast_exp2(-dm);   // the state is still zero: 0, not 2^-dm (may overflow)
      m += dm;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] -= dm;
      lsum *= al;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= al;
    }
    float p[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i]);
      lo[i] = p[i] - __uint_as_float(__float_as_uint(p[i]) & 0xFFFF0000u);
    }
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    // B fragment: k = keys 4r .. 4r + 3 of query n, as truncated bf16 hi and lo limbs
    const short4v bhi = __builtin_bit_cast(short4v, make_uint2(bf16_hi_pair(p[0], p[1]), bf16_hi_pair(p[2], p[3])));
    const short4v blo = __builtin_bit_cast(short4v, make_uint2(bf16_hi_pair(lo[0], lo[1]), bf16_hi_pair(lo[2], lo[3])));
    wave_lds_sync();   // the value rows are in LDS
    // ---- values: A row = channel 16t + n, k = keys 4r .. 4r + 3 ----
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = 16 * t + n;
      const uint32_t w0 = (uint32_t)vs[4 * r][c] | ((uint32_t)vs[4 * r + 1][c] << 16);
      const uint32_t w1 = (uint32_t)vs[4 * r + 2][c] | ((uint32_t)vs[4 * r + 3][c] << 16);
      const short4v av = __builtin_bit_cast(short4v, make_uint2(w0, w1));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bhi, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, blo, acc[t], 0, 0, 0);
    }
  }
  // ---- record 0 of each query vector: (m, l) and the unnormalised sum ----
  const float lq = rows_sum(lsum);
  if (q_ok) {
    const size_t rec = ((size_t)(t0 + i_q) * a.Hq + h * G + g_q) * a.n_total;   // record 0: the BF16 keys
    if (r == 0) a.part_ml[rec] = make_float2(m, lq);
    float* dst = a.part + rec * kHeadDim;
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<float4*>(dst + 16 * t + 4 * r) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
}

// query heads per reduce block: one when few (sequence, KV head) pairs would leave most CUs
// idle, else two for G = 4 and 8 (measured against four: 326.7 vs 328.2 us per call at
// 28 x 100K, 856 vs 861 us on the ragged 64 x [4K, 128K] batch), else the largest divisor of
// G that is at most four
template <int G>
constexpr int reduce_group() {
  return G == 4 || G == 8 ? 2 : G <= 4 ? G : G % 4 == 0 ? 4 : G % 3 == 0 ? 3 : G % 2 == 0 ? 2 : 1;
}

template <int G>
void launch_split(const DecodeArgs& a, int B, hipStream_t stream) {
  const dim3 grid(a.n_cas + (a.n_split + a.n_bsplit) * a.H * B);
  if (a.one_group)
    hipLaunchKernelGGL((split_kernel<G, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((split_kernel<G, false>), grid, dim3(256), 0, stream, a);
  constexpr int GB = reduce_group<G>();
  if (GB > 1 && B * a.H < kFewPairs)
    hipLaunchKernelGGL((reduce_kernel<G, 1>), dim3(B * a.H * G), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<G, GB>), dim3(B * a.H * (G / GB)), dim3(256), 0, stream, a);
}

}  // namespace

DecodePlan make_decode_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t recent,
                            int32_t batch, int32_t max_pages) {
  DecodePlan p{};
  const long long int2_pages = max(0, max_pages - sink / kPage);
  const long long bh = (long long)batch * num_kv_heads;
  p.n_bsplit = (sink + recent + kBf16Chunk - 1) / kBf16Chunk;
  // Items per (sequence, KV head): m ranges of ~400 pages (measured on MI355X at
  // 28 x 100K tokens: 16 to 20 items per (sequence, KV head) are within 0.7% of
  // each other, 13 items -- three rounds of block slots -- is 2.5% and 41 items 5%
  // slower), but at least enough items for half the resident block slots (2 per CU
  // for G <= 4, 1 above, 256 CUs).  Measured with 1 and 2 sequences of 100K tokens
  // (8 KV heads): filling every slot made ranges of ~50 pages whose records cost the
  // reduce more than the extra blocks saved (45 against 51 us per call at batch 1,
  // 53 against 59 at batch 2).
  const long long slots = (num_q_heads / num_kv_heads <= 4 ? 2 : 1) * 256;
  const long long max_m = kMaxItems - p.n_bsplit;
  long long best_m = 0;
  if (int2_pages > 0 && bh > 0) {
    best_m = max((int2_pages + 399) / 400, (slots + bh - 1) / bh);
    best_m = min(best_m, min(max_m, (int2_pages + 15) / 16));   // at least 16 pages per item
    best_m = max(best_m, (int2_pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit);
  }
  long long per = best_m > 0 ? (int2_pages + best_m - 1) / best_m : kPage;
  per = (per + 3) / 4 * 4;   // whole rounds of the 4 waves' page pairs
  if (per > kMaxPagesPerSplit) per = kMaxPagesPerSplit;
  p.pages_per_split = (int)per;
  p.n_split = int2_pages > 0 ? (int)((int2_pages + per - 1) / per) : 0;
  p.bf16_chunk = kBf16Chunk;
  // Few (sequence, KV head) pairs (a batch of one or two at 8 KV heads): the INT2 ranges are
  // short, and a 320-token BF16 item, walked in five dependent rounds of loads, would
  // finish last.  64-token items, one round each, as long as the records still fit.
  if (bh > 0 && bh < kFewPairs) {
    const int nb64 = (sink + recent + kBf16ChunkFew - 1) / kBf16ChunkFew;
    if (p.n_split + nb64 <= kMaxItems) {
      p.n_bsplit = nb64;
      p.bf16_chunk = kBf16ChunkFew;
    }
  }
  p.n_total = p.n_split + p.n_bsplit;
  const size_t qrot = (size_t)batch * num_q_heads * kQrotBytes;
  p.qrot_off = 0;
  p.part_off = (qrot + 511) / 512 * 512;   // records on 128-byte line boundaries
  const size_t n_rec = (size_t)batch * num_q_heads * p.n_total;
  p.ml_off = p.part_off + n_rec * kHeadDim * sizeof(float);
  p.eff_off = p.bytes = p.ml_off + n_rec * sizeof(float2);
  return p;
}

DecodePlan make_cascade_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t recent,
                             int32_t batch, int32_t max_pages, int32_t max_shared_pages) {
  DecodePlan p = make_decode_plan(num_kv_heads, num_q_heads, sink, recent, batch, max_pages);
  const int int2_pages = max(0, max_pages - sink / kPage);
  const int shared = min(max(max_shared_pages, 0), int2_pages);
  p.n_sh = shared > 0 ? (shared + p.pages_per_split - 1) / p.pages_per_split : 0;
  p.n_total += p.n_sh;
  if (p.n_total > kMaxItems) {
    p.bytes = 0;
    return p;
  }
  const size_t n_rec = (size_t)batch * num_q_heads * p.n_total;
  p.ml_off = p.part_off + n_rec * kHeadDim * sizeof(float);
  p.eff_off = (p.ml_off + n_rec * sizeof(float2) + 255) / 256 * 256;
  p.bytes = p.eff_off + (size_t)batch * sizeof(int32_t);
  return p;
}

namespace {
DecodeArgs make_decode_args(const DecodeLaunch& L) {
  DecodeArgs a{};
  a.pages = L.pages;
  a.k_sink = L.k_sink;
  a.v_sink = L.v_sink;
  a.k_ring = L.k_ring;
  a.v_ring = L.v_ring;
  a.u_k = L.u_k;
  a.u_v = L.u_v;
  a.q = L.q;
  a.page_table = L.page_table;
  a.seq_lens = L.seq_lens;
  a.out = L.out;
  a.qrot = reinterpret_cast<QrotRecord*>(L.workspace + L.plan.qrot_off);
  a.part = reinterpret_cast<float*>(L.workspace + L.plan.part_off);
  a.part_ml = reinterpret_cast<float2*>(L.workspace + L.plan.ml_off);
  a.sl2e = L.sm_scale * 1.4426950408889634f;
  {
    // W = fp16(p s) must stay below fp16's maximum: a value scale is at most
    // fp16((max - min) / 3) <= 2 clip_v / 3 (+ rounding), so p <= 2^tau with
    // 2^tau * s_max < 65000; tau in [2, 8]
    const double s_max = 2.0 * L.clip_v / 3.0 * (1.0 + 1.0 / 1024);
    int tau = (int)std::floor(std::log2(65000.0 / s_max));
    a.resc_thr = (float)(tau < 2 ? 2 : tau > 8 ? 8 : tau);
  }
  a.H = L.num_kv_heads;
  a.Hq = L.num_q_heads;
  a.G = L.num_q_heads / L.num_kv_heads;
  a.B = L.batch;
  a.max_pages = L.max_pages;
  a.sink = L.sink;
  a.recent = L.recent;
  a.P = L.plan.pages_per_split;
  a.n_split = L.plan.n_split;
  a.n_bsplit = L.plan.n_bsplit;
  a.n_total = L.plan.n_total;
  a.bchunk = L.plan.bf16_chunk;
  a.one_group = L.group == 128;
  if (L.n_groups > 0 && L.plan.n_sh > 0) {   // cascade decode
    constexpr int kHeadsPerTile = 16;          // per NQ: a block's 4 waves x 4 NQ query heads
    const int nq = (a.G + 3) / 4;
    const int tile = a.G > 4 ? kExtTile : kHeadsPerTile * nq;   // query vectors per cascade block
    a.cu_groups = L.cu_groups;
    a.group_pages = L.group_pages;
    a.cas_eff = reinterpret_cast<int32_t*>(L.workspace + L.plan.eff_off);
    a.n_groups = L.n_groups;
    a.max_group = L.max_group;
    a.n_sh = L.plan.n_sh;
    a.n_cqt = (L.max_group * a.G + tile - 1) / tile;
    a.n_cas = L.n_groups * a.H * a.n_sh * a.n_cqt;
  }
  return a;
}

int launch_split_reduce(const DecodeArgs& a, int B, hipStream_t stream) {
  switch (a.G) {
    case 1: launch_split<1>(a, B, stream); break;
    case 2: launch_split<2>(a, B, stream); break;
    case 3: launch_split<3>(a, B, stream); break;
    case 4: launch_split<4>(a, B, stream); break;
    case 5: launch_split<5>(a, B, stream); break;
    case 6: launch_split<6>(a, B, stream); break;
    case 7: launch_split<7>(a, B, stream); break;
    case 8: launch_split<8>(a, B, stream); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
}  // namespace

int launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  if (L.batch == 0) return 0;
  DecodeArgs a = make_decode_args(L);
  // With few (sequence, KV head) pairs the GPU idles through a separate rotation launch,
  // so the split kernel's INT2 items rotate their own queries while their first pages
  // load (measured at 1 x 100K: 32.5 against 34.4 us per call); with many, that per-block
  // prologue costs more than the launch (366.6 against 356.7 us at 28 x 100K).  Cascade
  // blocks serve the query heads of many sequences and always read stored records.
  a.qrot_inline = (long long)L.batch * L.num_kv_heads < kFewPairs && a.n_cas == 0;
  if (!a.qrot_inline)
    hipLaunchKernelGGL(rotate_q_kernel, dim3(L.batch * L.num_kv_heads), dim3(kSideThreads), 0, stream, a);
  return launch_split_reduce(a, L.batch, stream);
}

ExtendPlan make_extend_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t num_tokens,
                            int32_t max_pages, int32_t max_chunk) {
  ExtendPlan p{};
  const long long int2_pages = max(0, max_pages - sink / kPage);
  // ranges of about 400 pages (at most 512, whole page pairs)
  long long n_split = int2_pages > 0 ? max(1LL, (int2_pages + 399) / 400) : 0;
  long long per = n_split > 0 ? (int2_pages + n_split - 1) / n_split : 2;
  per = (per + 1) / 2 * 2;
  if (per > kMaxPagesPerSplit) per = kMaxPagesPerSplit;
  p.pages_per_split = (int)per;
  p.n_split = int2_pages > 0 ? (int)((int2_pages + per - 1) / per) : 0;
  p.n_total = 1 + p.n_split;
  p.n_qt = (int)(((long long)max_chunk * (num_q_heads / num_kv_heads) + kExtTile - 1) / kExtTile);
  const size_t rows = (size_t)num_tokens * num_q_heads;
  p.qrot_off = 0;
  p.part_off = (rows * kQrotBytes + 511) / 512 * 512;
  p.ml_off = p.part_off + rows * p.n_total * kHeadDim * sizeof(float);
  p.len_off = (p.ml_off + rows * p.n_total * sizeof(float2) + 255) / 256 * 256;
  p.bytes = p.len_off + (size_t)num_tokens * sizeof(int32_t);
  return p;
}

namespace {
template <int G>
void launch_extend_g(const ExtArgs& e, hipStream_t stream) {
  const DecodeArgs& a = e.d;
  if (a.n_split > 0) {
    const dim3 grid(e.n_seq * a.H * a.n_split * e.n_qt);
    if (a.one_group)
      hipLaunchKernelGGL((ext_int2_kernel<G, true>), grid, dim3(256), 0, stream, e);
    else
      hipLaunchKernelGGL((ext_int2_kernel<G, false>), grid, dim3(256), 0, stream, e);
  }
  hipLaunchKernelGGL(ext_bf16_kernel<G>, dim3(e.n_seq * a.H * e.n_qt), dim3(256), 0, stream, e);
  constexpr int GB = reduce_group<G>();
  hipLaunchKernelGGL((reduce_kernel<G, GB>), dim3(e.n_tok * a.H * (G / GB)), dim3(256), 0, stream, a);
}
}  // namespace

int launch_extend(const ExtendLaunch& X, hipStream_t stream) {
  if (X.num_tokens == 0) return 0;
  DecodeLaunch D{};
  D.pages = X.pages;
  D.k_sink = X.k_sink;
  D.v_sink = X.v_sink;
  D.k_ring = X.k_ring;
  D.v_ring = X.v_ring;
  D.u_k = X.u_k;
  D.u_v = X.u_v;
  D.q = X.q;
  D.page_table = X.page_table;
  D.seq_lens = reinterpret_cast<const int32_t*>(X.workspace + X.plan.len_off);   // row prefix lengths
  D.out = X.out;
  D.workspace = X.workspace;
  D.sm_scale = X.sm_scale;
  D.clip_v = X.clip_v;
  D.num_kv_heads = X.num_kv_heads;
  D.num_q_heads = X.num_q_heads;
  D.max_pages = X.max_pages;
  D.batch = X.num_tokens;
  D.sink = X.sink;
  D.recent = X.recent;
  D.group = X.group;
  D.plan.pages_per_split = X.plan.pages_per_split;
  D.plan.n_split = X.plan.n_split;
  D.plan.n_bsplit = 1;
  D.plan.n_total = X.plan.n_total;
  D.plan.bf16_chunk = kBf16Chunk;
  D.plan.qrot_off = X.plan.qrot_off;
  D.plan.part_off = X.plan.part_off;
  D.plan.ml_off = X.plan.ml_off;
  ExtArgs e{};
  e.d = make_decode_args(D);
  e.d.ext = 1;
  e.k_new = X.k;
  e.v_new = X.v;
  e.cu = X.cu_seqlens;
  e.prefix_lens = X.prefix_lens;
  e.row_len = reinterpret_cast<int32_t*>(X.workspace + X.plan.len_off);
  e.n_seq = X.batch;
  e.n_tok = X.num_tokens;
  e.max_chunk = X.max_chunk;
  e.n_qt = X.plan.n_qt;
  // rows = chunk tokens: the rotation of every chunk query, then the INT2 ranges, the BF16 keys
  // and the merge (which reads row_len, written by the BF16 kernel)
  hipLaunchKernelGGL(rotate_q_kernel, dim3(X.num_tokens * X.num_kv_heads), dim3(kSideThreads), 0, stream, e.d);
  switch (e.d.G) {
    case 1: launch_extend_g<1>(e, stream); break;
    case 2: launch_extend_g<2>(e, stream); break;
    case 3: launch_extend_g<3>(e, stream); break;
    case 4: launch_extend_g<4>(e, stream); break;
    case 5: launch_extend_g<5>(e, stream); break;
    case 6: launch_extend_g<6>(e, stream); break;
    case 7: launch_extend_g<7>(e, stream); break;
    case 8: launch_extend_g<8>(e, stream); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_decode_step(const KvWriteLaunch& W, const DecodeLaunch& D, hipStream_t stream) {
  if (launch_kv_write(W, stream)) return 1;
  return launch_decode(D, stream);
}

}  // namespace oscar
