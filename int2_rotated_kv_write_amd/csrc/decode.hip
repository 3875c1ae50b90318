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
// sum_i p_i v_hat_i = (sum_i p_i v_hat'_i) R_V^T.  Three launches:
//   rotate_q  q' = q U_K H P (times sm_scale*log2 e) once per (sequence, head)
//   split     split-K over the pages: BF16 chunks with the plain q, INT2 page
//             ranges with q' on the packed codes; online softmax in base 2
//   reduce    log-sum-exp merge, acc_rot R_V^T = ((acc_rot P) H) U_V^T, bf16 out
#include "common.h"
#include "kernels.h"

namespace oscar {

namespace {

// Rotated query of one (sequence, query head), as 16-bit fixed point:
// q'_c = alpha * Q_c with Q_c = rne(q'_c / alpha) in [-32767, 32767] and
// alpha = max|q'| / 32767; Q_c = 256 * hi_c + lo_c with hi_c a signed byte and
// lo_c an unsigned byte.  For chunk q (post-rotation channels 32q .. 32q+31 =
// code words d = 2q, 2q+1), limb[16q + 4w + j] (w = 0, 1) packs the hi bytes
// of channels 16d + j, +4, +8, +12 (byte b holds channel 16d + 4b + j) and
// limb[16q + 8 + 4w + j] the lo bytes, matching the byte vectors
// (word >> 2j) & 0x03030303 of code word d.
struct QrotRecord {
  uint32_t limb[64];
  float alpha;
  float qsum[4];   // sum_c q'_c over each chunk (fp32)
  float pad[11];
};
static_assert(sizeof(QrotRecord) == kQrotBytes, "record size");

struct DecodeArgs {
  const uint8_t* pages;
  const uint16_t *k_sink, *v_sink, *k_ring, *v_ring, *u_k, *u_v, *q;
  const int32_t *page_table, *seq_lens;
  uint16_t* out;
  QrotRecord* qrot;
  float* part;
  float sl2e;   // sm_scale * log2(e)
  int32_t H, Hq, G, max_pages, sink, recent, P, n_split, n_bsplit, n_total;
};

__device__ __forceinline__ int bf16_token_count(int L, int sink, int recent) {
  if (L <= sink) return L;
  return sink + (L - max(sink, L - recent));
}
__device__ __forceinline__ int int2_end(int L, int sink, int recent) {   // INT2 tokens [sink, end)
  return L <= sink ? sink : max(sink, L - recent);
}

// ---------------------------------------------------------------------------
// rotate_q: one block per (sequence, KV head); two query heads at a time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rotate_q_kernel(DecodeArgs a) {
  __shared__ float y[2][kHeadDim];
  __shared__ float qs[2][kHeadDim];
  __shared__ int32_t qi[2][kHeadDim];
  __shared__ float amax[2][4];
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x, hl = tid >> 7, j = tid & 127;
  const uint16_t* U = a.u_k + (size_t)h * kHeadDim * kHeadDim;
  for (int h0 = 0; h0 < a.G; h0 += 2) {
    const int hh = h0 + hl;
    const bool act = hh < a.G;
    const int hq = h * a.G + hh;
    if (act) {
      const uint16_t* qv = a.q + ((size_t)b * a.Hq + hq) * kHeadDim;
      float acc = 0.f;
      for (int i = 0; i < kHeadDim; ++i)
        acc = fmaf(bf16_bits_to_f32(qv[i]), bf16_bits_to_f32(U[i * kHeadDim + j]), acc);
      y[hl][j] = acc;
    }
    __syncthreads();
    for (int s = 1; s < kHeadDim; s <<= 1) {
      if (act && j < 64) {
        const int lo = ((j & ~(s - 1)) << 1) | (j & (s - 1)), hi = lo | s;
        const float x0 = y[hl][lo], x1 = y[hl][hi];
        y[hl][lo] = x0 + x1;
        y[hl][hi] = x0 - x1;
      }
      __syncthreads();
    }
    float w = 0.f;
    if (act) {
      w = y[hl][bitrev7(j)] * 0.08838834764831845f * a.sl2e;   // (z P)_j = z_br(j)
      qs[hl][j] = w;
    }
    // max |q'| over the 128 channels of this head: 2 waves per head
    float mx = wave_max_xor(fabsf(w), 1, 32);
    if ((tid & 63) == 0) amax[hl][(tid >> 6) & 1] = mx;
    __syncthreads();
    const float qmax = fmaxf(amax[hl][0], amax[hl][1]);
    const float alpha = qmax > 0.f ? qmax / 32767.0f : 1.0f;
    if (act) qi[hl][j] = (int32_t)fminf(fmaxf(__builtin_rintf(w / alpha), -32767.f), 32767.f);
    __syncthreads();
    if (act) {
      QrotRecord* rec = a.qrot + ((size_t)b * a.Hq + hq);
      if (j < 64) {
        // j = 16 q + 8 lohi + 4 w + jj  ->  word d = 2q + w, byte b: channel 16d + 4b + jj
        const int qq = j >> 4, lohi = (j >> 3) & 1, w2 = (j >> 2) & 1, jj = j & 3, d = 2 * qq + w2;
        uint32_t packed = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int Q = qi[hl][16 * d + 4 * bb + jj];
          const uint32_t byte = lohi ? (uint32_t)(Q & 0xFF) : (uint32_t)((Q >> 8) & 0xFF);
          packed |= byte << (8 * bb);
        }
        rec->limb[j] = packed;
      } else if (j < 68) {
        const int ch = j - 64;
        float sum = 0.f;
        for (int c = 32 * ch; c < 32 * ch + 32; ++c) sum += qs[hl][c];
        rec->qsum[ch] = sum;
      } else if (j == 68) {
        rec->alpha = alpha;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// split: block (item, KV head, sequence), 4 waves.
// ---------------------------------------------------------------------------
constexpr int kMaxPagesPerSplit = 128;

struct __attribute__((aligned(16))) SplitSmem {
  int32_t pid[kMaxPagesPerSplit];    // physical page ids of the item's page range
  uint32_t w[4][kMaxGqa][2][8];      // fp16 pairs of p*s per (wave, head, group, pair)
  float p[4][kMaxGqa][16];           // BF16 items: probabilities per token
  float m[4][kMaxGqa];
  float l[4][kMaxGqa];
  float acc[4][kMaxGqa][kHeadDim];
};

template <int G>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs& a, int b, int h, int item,
                                                      SplitSmem& sm) {
  __syncthreads();
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o >> 7, c = o & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.m[w][hh]);
    float val = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = sm.m[w][hh] == -INFINITY ? 0.f : exp2f(sm.m[w][hh] - M);
      val += e * sm.acc[w][hh][c];
      lsum += e * sm.l[w][hh];
    }
    float* rec = a.part + ((size_t)(b * a.Hq + h * G + hh) * a.n_total + item) * kPartFloats;
    rec[4 + c] = val;
    if (c == 0) {
      rec[0] = M;
      rec[1] = lsum;
    }
  }
}

// BF16 sink + recent tokens, 64 per item, 16 per wave; plain (unrotated) q.
template <int G>
__device__ void bf16_item(const DecodeArgs& a, int b, int h, int chunk, int L, SplitSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane >> 2, q = lane & 3;
  const int nsink = min(a.sink, L);
  const int r_lo = L > a.sink ? max(a.sink, L - a.recent) : L;
  const int nb = bf16_token_count(L, a.sink, a.recent);
  const int jbase = chunk * kBf16Chunk + 16 * wave;
  const size_t head_row = (size_t)b * a.H + h;

  auto row_offset = [&](int jj) -> size_t {   // element offset of BF16 token jj's row
    if (jj < nsink) return (head_row * a.sink + jj) * kHeadDim;
    const int p = r_lo + (jj - nsink);
    return (head_row * a.recent + (p % a.recent)) * kHeadDim;
  };
  auto kbuf = [&](int jj) { return jj < nsink ? a.k_sink : a.k_ring; };
  auto vbuf = [&](int jj) { return jj < nsink ? a.v_sink : a.v_ring; };

  const int j = jbase + t;
  const bool valid = j < nb;
  float lg[G];
  {
    uint4 kd[4] = {};
    if (valid) {
      const uint16_t* krow = kbuf(j) + row_offset(j) + 32 * q;
#pragma unroll
      for (int x = 0; x < 4; ++x) kd[x] = reinterpret_cast<const uint4*>(krow)[x];
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint16_t* qv = a.q + ((size_t)b * a.Hq + h * G + hh) * kHeadDim + 32 * q;
      float d = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint4 qd = reinterpret_cast<const uint4*>(qv)[x];
        d = dot2_bf16(qd.x, kd[x].x, d);
        d = dot2_bf16(qd.y, kd[x].y, d);
        d = dot2_bf16(qd.z, kd[x].z, d);
        d = dot2_bf16(qd.w, kd[x].w, d);
      }
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      lg[hh] = valid ? d * a.sl2e : -INFINITY;
    }
  }
  float m[G], lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = wave_max_xor(lg[hh], 4, 32);
    const float p = (valid && m[hh] != -INFINITY) ? exp2f(lg[hh] - m[hh]) : 0.f;
    lsum[hh] = wave_sum_xor(p, 4, 32);
    if (q == 0) sm.p[wave][hh][t] = p;
  }
  wave_lds_sync();
  float acc[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) acc[hh][0] = acc[hh][1] = 0.f;
  for (int tt = 0; tt < 16; ++tt) {
    const int jj = jbase + tt;
    if (jj >= nb) break;   // wave-uniform
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(vbuf(jj) + row_offset(jj) + 2 * lane);
    const float v0 = bf16_bits_to_f32(vv & 0xFFFFu), v1 = bf16_bits_to_f32(vv >> 16);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = sm.p[wave][hh][tt];
      acc[hh][0] = fmaf(p, v0, acc[hh][0]);
      acc[hh][1] = fmaf(p, v1, acc[hh][1]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      sm.m[wave][hh] = m[hh];
      sm.l[wave][hh] = lsum[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.acc[wave][hh][2 * lane] = acc[hh][0];
    sm.acc[wave][hh][2 * lane + 1] = acc[hh][1];
  }
  merge_waves_and_store<G>(a, b, h, chunk, sm);
}

// INT2 history pages [first, end): wave w takes pages first + w, + 4, ...
// K stage: lane = (token t = l/4, chunk q = l%4) -> 32 channels, logits by
//          fp16 dot2 of q' with (base + code) pairs; 4-lane reduction.
// V stage: lane = channels 2l, 2l+1 -> their channel-major code words hold all
//          16 tokens; fp16 dot2 of (p*s) pairs with (base + code) pairs.
template <int G>
__device__ void int2_item(const DecodeArgs& a, int b, int h, int split, int first, int end, int i_hi,
                          SplitSmem& sm) {
  constexpr int NJ = (G + 3) / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane >> 2, q = lane & 3;
  const int gv = lane >> 5;                       // group of channels 2l, 2l+1
  const int tpair = pair_of_k(t & 7), thalf = t >> 3;
  const float tbase = (float)pair_base(tpair);

  uint32_t qhi[G][8], qlo[G][8];
  float alpha_q[G], qsum[G];
  const QrotRecord* qr = a.qrot + ((size_t)b * a.Hq + h * G);
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint4* src = reinterpret_cast<const uint4*>(&qr[hh].limb[16 * q]);
    const uint4 h0 = src[0], h1 = src[1], l0 = src[2], l1 = src[3];
    qhi[hh][0] = h0.x; qhi[hh][1] = h0.y; qhi[hh][2] = h0.z; qhi[hh][3] = h0.w;
    qhi[hh][4] = h1.x; qhi[hh][5] = h1.y; qhi[hh][6] = h1.z; qhi[hh][7] = h1.w;
    qlo[hh][0] = l0.x; qlo[hh][1] = l0.y; qlo[hh][2] = l0.z; qlo[hh][3] = l0.w;
    qlo[hh][4] = l1.x; qlo[hh][5] = l1.y; qlo[hh][6] = l1.z; qlo[hh][7] = l1.w;
    alpha_q[hh] = qr[hh].alpha;
    qsum[hh] = qr[hh].qsum[q];
  }

  float m[G], lp[G], acc[G][2];
  float zacc[NJ][2], oacc[NJ][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    lp[hh] = 0.f;
    acc[hh][0] = acc[hh][1] = 0.f;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) zacc[jj][0] = zacc[jj][1] = oacc[jj][0] = oacc[jj][1] = 0.f;

  // physical page ids of this item, once per block
  {
    const int32_t* ptab = a.page_table + (size_t)b * a.max_pages + first;
    for (int i = threadIdx.x; i < end - first; i += 256) sm.pid[i] = ptab[i];
    __syncthreads();
  }
  uint16_t* wl = reinterpret_cast<uint16_t*>(&sm.w[wave][0][0][0]);
  const size_t head_off = (size_t)h * kBlockBytes;
  const size_t page_stride = (size_t)a.H * kBlockBytes;

  struct PageRegs {
    uint2 kc, vc, vp;
    uint32_t kp;
  };
  auto load_page = [&](int pg) {
    const uint8_t* blk = a.pages + (size_t)sm.pid[pg - first] * page_stride + head_off;
    PageRegs r;
    r.kc = *reinterpret_cast<const uint2*>(blk + kKCodes + 32 * t + 8 * q);
    r.kp = *reinterpret_cast<const uint32_t*>(blk + kKParams + 8 * t + 4 * (q >> 1));
    r.vc = *reinterpret_cast<const uint2*>(blk + kVCodes + 8 * lane);
    r.vp = *reinterpret_cast<const uint2*>(blk + kVParams + 8 * t);
    return r;
  };

  int pg = first + wave;
  PageRegs cur = {}, nxt = {};
  if (pg < end) cur = load_page(pg);
  for (; pg < end; pg += 4) {
    if (pg + 4 < end) nxt = load_page(pg + 4);   // keep the next page in flight
    const uint2 kc = cur.kc, vc = cur.vc, vp = cur.vp;
    const uint32_t kp = cur.kp;

    // ---- logits (base-2 units): exact integer dot of Q with the codes ----
    uint32_t bv[8];   // byte vectors: bv[4w + j] holds channels 16(2q+w) + 4b + j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bv[j] = (kc.x >> (2 * j)) & 0x03030303u;
      bv[4 + j] = (kc.y >> (2 * j)) & 0x03030303u;
    }
    const float ks = f16_bits_to_f32(kp), kz = f16_bits_to_f32(kp >> 16);
    const bool tok_ok = pg * 16 + t < i_hi;
    float lg[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      int dh = 0, dl = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        dh = __builtin_amdgcn_sdot4((int)qhi[hh][k], (int)bv[k], dh, false);
        dl = (int)__builtin_amdgcn_udot4(qlo[hh][k], bv[k], (uint32_t)dl, false);
      }
      const float d = (float)(dh * 256 + dl) * alpha_q[hh];
      const float x = quad_sum(fmaf(ks, d, kz * qsum[hh]));
      lg[hh] = tok_ok ? x : -INFINITY;
    }

    // ---- online softmax (exact running max; the page's first token is valid) ----
    float alpha[G], pr[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mn = fmaxf(m[hh], tok_max(lg[hh]));
      alpha[hh] = fast_exp2(m[hh] - mn);
      pr[hh] = tok_ok ? fast_exp2(lg[hh] - mn) : 0.f;
      m[hh] = mn;
      lp[hh] = fmaf(lp[hh], alpha[hh], pr[hh]);
    }

    // ---- weights p*s (fp16) for the V stage ----
    const float vs0 = f16_bits_to_f32(vp.x), vz0 = f16_bits_to_f32(vp.x >> 16);
    const float vs1 = f16_bits_to_f32(vp.y), vz1 = f16_bits_to_f32(vp.y >> 16);
    wave_lds_sync();
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int hh = q + 4 * jj;
      if (hh < G) {
        float prh = 0.f, al = 1.f;
#pragma unroll
        for (int x = 0; x < G; ++x)
          if (x == hh) {
            prh = pr[x];
            al = alpha[x];
          }
        const uint32_t w0 = f32_to_f16_bits(prh * vs0), w1 = f32_to_f16_bits(prh * vs1);
        wl[((hh * 2 + 0) * 8 + tpair) * 2 + thalf] = (uint16_t)w0;
        wl[((hh * 2 + 1) * 8 + tpair) * 2 + thalf] = (uint16_t)w1;
        zacc[jj][0] = fmaf(zacc[jj][0], al, prh * vz0);
        zacc[jj][1] = fmaf(zacc[jj][1], al, prh * vz1);
        oacc[jj][0] = fmaf(oacc[jj][0], al, tbase * f16_bits_to_f32(w0));
        oacc[jj][1] = fmaf(oacc[jj][1], al, tbase * f16_bits_to_f32(w1));
      }
    }
    wave_lds_sync();

    // ---- V accumulation on the channel-major code words ----
    uint32_t e0[8], e1[8];
    unpack16(vc.x, e0);
    unpack16(vc.y, e1);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4* wr = reinterpret_cast<const uint4*>(&sm.w[wave][hh][gv][0]);
      const uint4 wa = wr[0], wb = wr[1];
      const uint32_t W[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      float a0 = acc[hh][0] * alpha[hh], a1 = acc[hh][1] * alpha[hh];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a0 = dot2_f16(W[i], e0[i], a0);
        a1 = dot2_f16(W[i], e1[i], a1);
      }
      acc[hh][0] = a0;
      acc[hh][1] = a1;
    }
    cur = nxt;
  }

  // ---- finish the wave: l, and acc += sum(p z) - sum(base * p s) ----
  float lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) lsum[hh] = tok_sum(lp[hh]);
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int g = 0; g < 2; ++g) zacc[jj][g] = tok_sum(zacc[jj][g] - oacc[jj][g]);
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float d0 = __shfl(zacc[hh / 4][0], hh % 4);
    const float d1 = __shfl(zacc[hh / 4][1], hh % 4);
    const float d = gv ? d1 : d0;
    acc[hh][0] += d;
    acc[hh][1] += d;
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      sm.m[wave][hh] = m[hh];
      sm.l[wave][hh] = lsum[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.acc[wave][hh][2 * lane] = acc[hh][0];
    sm.acc[wave][hh][2 * lane + 1] = acc[hh][1];
  }
  merge_waves_and_store<G>(a, b, h, a.n_bsplit + split, sm);
}

template <int G>
__global__ __launch_bounds__(256) void split_kernel(DecodeArgs a) {
  __shared__ SplitSmem sm;
  const int item = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  if (item < a.n_bsplit) {
    if (item * kBf16Chunk >= bf16_token_count(L, a.sink, a.recent)) return;
    bf16_item<G>(a, b, h, item, L, sm);
  } else {
    const int split = item - a.n_bsplit;
    const int i_hi = int2_end(L, a.sink, a.recent);
    const int first = a.sink / kPage + split * a.P;
    const int end = min(first + a.P, (i_hi + kPage - 1) / kPage);
    if (i_hi <= a.sink || first >= end) return;
    int2_item<G>(a, b, h, split, first, end, i_hi, sm);
  }
}

// ---------------------------------------------------------------------------
// reduce: one block per (sequence, KV head); two query heads at a time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_kernel(DecodeArgs a) {
  __shared__ float y[2][kHeadDim];
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x, hl = tid >> 7, c = tid & 127;
  const int L = a.seq_lens[b];
  const int n_b = (bf16_token_count(L, a.sink, a.recent) + kBf16Chunk - 1) / kBf16Chunk;
  const int i_hi = int2_end(L, a.sink, a.recent);
  const int int2_pages = i_hi > a.sink ? (i_hi + kPage - 1) / kPage - a.sink / kPage : 0;
  const int n_i = (int2_pages + a.P - 1) / a.P;
  const uint16_t* UV = a.u_v + (size_t)h * kHeadDim * kHeadDim;
  for (int h0 = 0; h0 < a.G; h0 += 2) {
    const int hh = h0 + hl;
    const bool act = hh < a.G;
    const int hq = h * a.G + hh;
    float plain = 0.f, rot = 0.f, lsum = 0.f;
    if (act && L > 0) {
      const float* base = a.part + (size_t)(b * a.Hq + hq) * a.n_total * kPartFloats;
      float M = -INFINITY;
      for (int s = 0; s < n_b; ++s) M = fmaxf(M, base[(size_t)s * kPartFloats]);
      for (int s = 0; s < n_i; ++s) M = fmaxf(M, base[(size_t)(a.n_bsplit + s) * kPartFloats]);
      for (int s = 0; s < n_b; ++s) {
        const float* r = base + (size_t)s * kPartFloats;
        const float e = r[0] == -INFINITY ? 0.f : exp2f(r[0] - M);
        lsum += e * r[1];
        plain += e * r[4 + c];
      }
      for (int s = 0; s < n_i; ++s) {
        const float* r = base + (size_t)(a.n_bsplit + s) * kPartFloats;
        const float e = r[0] == -INFINITY ? 0.f : exp2f(r[0] - M);
        lsum += e * r[1];
        rot += e * r[4 + c];
      }
    }
    // acc_rot P: z-space channel br(c) takes post-rotation channel c
    y[hl][bitrev7(c)] = rot;
    __syncthreads();
    for (int s = 1; s < kHeadDim; s <<= 1) {
      if (c < 64) {
        const int lo = ((c & ~(s - 1)) << 1) | (c & (s - 1)), hi = lo | s;
        const float x0 = y[hl][lo], x1 = y[hl][hi];
        y[hl][lo] = x0 + x1;
        y[hl][hi] = x0 - x1;
      }
      __syncthreads();
    }
    if (act) {
      float o = 0.f;
      const uint16_t* urow = UV + (size_t)c * kHeadDim;   // (y U^T)_c = sum_j y_j U[c][j]
      for (int jb = 0; jb < kHeadDim; jb += 8) {
        const uint4 u8 = *reinterpret_cast<const uint4*>(urow + jb);
        const uint32_t uu[4] = {u8.x, u8.y, u8.z, u8.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o = fmaf(y[hl][jb + 2 * k], bf16_bits_to_f32(uu[k] & 0xFFFFu), o);
          o = fmaf(y[hl][jb + 2 * k + 1], bf16_bits_to_f32(uu[k] >> 16), o);
        }
      }
      const float res = L > 0 ? (plain + o * 0.08838834764831845f) / lsum : 0.f;
      a.out[((size_t)b * a.Hq + hq) * kHeadDim + c] = (uint16_t)f32_to_bf16_bits(res);
    }
    __syncthreads();
  }
}

template <int G>
void launch_split(const DecodeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(split_kernel<G>, dim3(a.n_total, a.H, B), dim3(256), 0, stream, a);
}

}  // namespace

DecodePlan make_decode_plan(int32_t num_kv_heads, int32_t num_q_heads, int32_t sink, int32_t recent,
                            int32_t batch, int32_t max_pages) {
  DecodePlan p{};
  const int int2_pages = max(0, max_pages - sink / kPage);
  const long long page_heads = (long long)int2_pages * batch * num_kv_heads;
  long long per = (page_heads + 2047) / 2048;   // aim for ~2048 INT2 items
  per = per < 32 ? 32 : per > 128 ? 128 : per;
  p.pages_per_split = (int)((per + 3) / 4 * 4);
  p.n_split = int2_pages > 0 ? (int2_pages + p.pages_per_split - 1) / p.pages_per_split : 0;
  p.n_bsplit = (sink + recent + kBf16Chunk - 1) / kBf16Chunk;
  p.n_total = p.n_split + p.n_bsplit;
  const size_t qrot = (size_t)batch * num_q_heads * kQrotBytes;
  p.qrot_off = 0;
  p.part_off = (qrot + 255) / 256 * 256;
  p.bytes = p.part_off + (size_t)batch * num_q_heads * p.n_total * kPartFloats * sizeof(float);
  return p;
}

int launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  if (L.batch == 0) return 0;
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
  a.sl2e = L.sm_scale * 1.4426950408889634f;
  a.H = L.num_kv_heads;
  a.Hq = L.num_q_heads;
  a.G = L.num_q_heads / L.num_kv_heads;
  a.max_pages = L.max_pages;
  a.sink = L.sink;
  a.recent = L.recent;
  a.P = L.plan.pages_per_split;
  a.n_split = L.plan.n_split;
  a.n_bsplit = L.plan.n_bsplit;
  a.n_total = L.plan.n_total;
  const int BH = L.batch * L.num_kv_heads;
  hipLaunchKernelGGL(rotate_q_kernel, dim3(BH), dim3(256), 0, stream, a);
  switch (a.G) {
    case 1: launch_split<1>(a, L.batch, stream); break;
    case 2: launch_split<2>(a, L.batch, stream); break;
    case 3: launch_split<3>(a, L.batch, stream); break;
    case 4: launch_split<4>(a, L.batch, stream); break;
    case 5: launch_split<5>(a, L.batch, stream); break;
    case 6: launch_split<6>(a, L.batch, stream); break;
    case 7: launch_split<7>(a, L.batch, stream); break;
    case 8: launch_split<8>(a, L.batch, stream); break;
    default: return 1;
  }
  hipLaunchKernelGGL(reduce_kernel, dim3(BH), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace oscar
