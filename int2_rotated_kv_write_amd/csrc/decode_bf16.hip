// bf16_decode_attn: one decode step of attention over a plain BF16 paged KV
// cache, at the same shapes and on the same harness as the INT2 decode.
//
// This is the comparison point the pages measure OSCAR against: their decode
// speedups at 100K context are stated relative to a BF16 KV cache (Italian
// page, section "Velocita di decodifica"; Spanish summary, section 4).  Here it
// is a kernel of its own so that the INT2 path's gain can be measured on the
// same MI355X, per layer, with no serving stack around either.
//
// Page block: one 8192-byte block per (physical page, KV head):
//   [   0, 4096)  K, token-major: slot t, channel c at bf16 element 128 t + c
//   [4096, 8192)  V, channel-major: channel c, slot t at element 2048 + 16 c + t
// V is stored channel-major (as in the INT2 block) so that one lane's 8-byte
// read is 4 consecutive tokens of one channel: exactly a B fragment of the
// value MFMA.
//
// Two launches:
//   split   one block per (sequence, KV head, page range); each wave streams
//           every 4th page of the range straight into registers (two pages in
//           flight), logits on v_mfma_f32_16x16x32_bf16 (the G query heads of
//           the KV head are the MFMA columns), online softmax in base 2,
//           p V on v_mfma_f32_16x16x16_bf16 with p as bf16 hi + lo limbs
//   reduce  log-sum-exp merge of the ranges, bf16 out
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace oscar {

namespace {

constexpr int kB16Block = 8192;
constexpr int kB16VOff = 4096;
constexpr int kB16MaxPages = 512;   // pages per range (a wave keeps its page ids in 2 VGPRs)
constexpr int kB16Reduce = 32;
constexpr int kB16Ahead = 3;     // pages in flight per wave while one is processed

typedef short short4v __attribute__((ext_vector_type(4)));

struct B16Args {
  const uint8_t* pages;
  const uint16_t* q;
  const int32_t *page_table, *seq_lens;
  uint16_t* out;
  float* part;       // acc[128] per (sequence, query head, range)
  float2* part_ml;   // (m, l) per (sequence, query head, range); m in log2 units
  float sl2e;        // sm_scale * log2(e)
  int32_t H, Hq, G, B, max_pages, P, n_split;
};

// One page's fragments in one lane: lane (qq = lane / 16, t = lane % 16)
//   k[ks]  K of token t, channels 32 ks + 8 qq .. + 8      (A of the logit MFMA)
//   v[ct]  V of channel 16 ct + t, tokens 4 qq .. 4 qq + 3 (B of the value MFMA)
struct B16Page {
  uint4 k[4];
  uint2 v[8];
};

// non-temporal: the pages are read once per call and would displace the records from the caches
__device__ __forceinline__ void load_b16_page(B16Page& f, const uint8_t* blk, uint32_t koff, uint32_t voff) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) f.k[ks] = load_nt(reinterpret_cast<const uint4*>(blk + koff + 64 * ks));
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) f.v[ct] = load_nt(reinterpret_cast<const uint2*>(blk + voff + 512 * ct));
}

// high bf16 halves of two floats packed in one word (truncation)
__device__ __forceinline__ uint32_t hi_halves(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

__device__ __forceinline__ float trunc_bf16(float x) { return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }

struct __attribute__((aligned(16))) B16Smem {
  float acc[4][kMaxGqa][kHeadDim];
  float2 ml[4][kMaxGqa];
};

__global__ __launch_bounds__(256) void b16_split_kernel(B16Args a) {
  __shared__ B16Smem sm;
  const int w_blk = blockIdx.x;
  const int bh = w_blk / a.n_split, split = w_blk - bh * a.n_split;
  const int b = bh / a.H, h = bh - b * a.H;
  const int L = clamp_len(a.seq_lens[b], a.max_pages);
  const int n_pages = (L + kPage - 1) / kPage;
  const int first = split * a.P;
  const int end = min(first + a.P, n_pages);
  if (first >= end) return;   // block-uniform: the reduce skips ranges past the sequence

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, qq = lane >> 4;
  const int G = a.G;

  // q fragments: column n = query head h G + n (zero beyond G), channels 32 ks + 8 qq .. + 8
  bf16x8 qf[4];
  {
    const bool ok = n < G;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.Hq + h * G + (ok ? n : 0)) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = qp[4 * ks + qq];
      u = ok ? u : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // this wave's pages: j -> first + wave + 4 j
  const int base0 = first + wave;
  const int n_w = base0 < end ? (end - base0 + 3) / 4 : 0;
  int32_t pid_reg[2];
  {
    const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = lane + 64 * k;
      pid_reg[k] = j < n_w ? ptab[base0 + 4 * j] : 0;
    }
  }
  auto blk_of = [&](int j) {   // wave-uniform j < n_w
    const int v = (j >> 6) ? pid_reg[1] : pid_reg[0];
    const int pid = __builtin_amdgcn_readlane(v, j & 63);
    return a.pages + ((size_t)pid * a.H + h) * kB16Block;
  };
  const uint32_t koff = 256 * n + 16 * qq;
  const uint32_t voff = kB16VOff + 32 * n + 8 * qq;

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kTau = 8.f;   // rescale only when the max grows by more than this (p <= 2^8)

  auto process = [&](B16Page& f, int j) {
    f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.k[ks]), qf[ks], d, 0, 0, 0);
    // lane (qq, n): logits of tokens 4 qq + i, head n
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = d[i] * a.sl2e;
    const int page = base0 + 4 * j;
    if ((page + 1) * kPage > L) {   // wave-uniform: the sequence's last, partial page
      const int nv = L - page * kPage;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = 4 * qq + i < nv ? s[i] : -INFINITY;
      // slots past the end may hold anything: zero their values so that p = 0 stays 0
      const uint32_t m0 = (4 * qq < nv ? 0xFFFFu : 0u) | (4 * qq + 1 < nv ? 0xFFFF0000u : 0u);
      const uint32_t m1 = (4 * qq + 2 < nv ? 0xFFFFu : 0u) | (4 * qq + 3 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f.v[ct].x &= m0;
        f.v[ct].y &= m1;
      }
    }
    float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    pm = swap32(swap16(pm, true), true);   // max over the head's 16 tokens (lanes n + 16 r)
    const bool up = pm > m + kTau;
    if (__any(up)) {
      const float mn = up ? pm : m;
      const float al = fast_exp2(m - mn);   // m = -inf on the first page: 0
      m = mn;
      lsum *= al;
      // accumulator rows of this lane are heads 4 qq + r
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(al, 4 * qq + r);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ct][r] *= ar[r];
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    // A fragment of the value MFMA: row = head n, k = tokens 4 qq .. + 3 -- this lane's own p.
    // hi = p truncated to bf16, lo = the remainder truncated: p to about 2^-14 relative.
    float lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = p[i] - trunc_bf16(p[i]);
    const short4v ahi = __builtin_bit_cast(short4v, make_uint2(hi_halves(p[0], p[1]), hi_halves(p[2], p[3])));
    const short4v alo = __builtin_bit_cast(short4v, make_uint2(hi_halves(lo[0], lo[1]), hi_halves(lo[2], lo[3])));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const short4v bv = __builtin_bit_cast(short4v, f.v[ct]);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bv, acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bv, acc[ct], 0, 0, 0);
    }
  };

  // kB16Ahead pages in flight while one is processed; unrolled over the
  // buffers so each stays in fixed registers.  The prefetch is unconditional
  // (past the wave's last page it reloads that page):
  // with a conditional one the compiler's wait before each page became
  // vmcnt(0), which also waited for the pages behind it.
  constexpr int NB = kB16Ahead + 1;
  B16Page buf[NB];
  if (n_w > 0) {
#pragma unroll
    for (int u = 0; u < kB16Ahead; ++u) load_b16_page(buf[u], blk_of(min(u, n_w - 1)), koff, voff);
  }
  for (int j0 = 0; j0 < n_w; j0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u;
      if (j >= n_w) break;
      load_b16_page(buf[(u + kB16Ahead) % NB], blk_of(min(j + kB16Ahead, n_w - 1)), koff, voff);
      process(buf[u], j);
    }
  }

  // ---- merge the four waves of the block, store one partial record per head ----
  const float lt = swap32(swap16(lsum, false), false);
  if (qq == 0 && n < G) sm.ml[wave][n] = make_float2(n_w > 0 ? m : -INFINITY, lt);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int head = 4 * qq + r;
    if (head < G) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) sm.acc[wave][head][16 * ct + n] = acc[ct][r];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int head = idx >> 7, c = idx & (kHeadDim - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.ml[w][head].x);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 ml = sm.ml[w][head];
      const float e = ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - M);
      l = fmaf(e, ml.y, l);
      o = fmaf(e, sm.acc[w][head][c], o);
    }
    const size_t rec = ((size_t)b * a.Hq + h * G + head) * a.n_split + split;
    a.part[rec * kHeadDim + c] = o;
    if (c == 0) a.part_ml[rec] = make_float2(M, l);
  }
}

// one block of 128 threads per (sequence, query head); thread c owns channel c
__global__ __launch_bounds__(kHeadDim) void b16_reduce_kernel(B16Args a) {
  const int bhq = blockIdx.x, b = bhq / a.Hq, c = threadIdx.x;
  uint16_t* out = a.out + (size_t)bhq * kHeadDim;
  const int L = clamp_len(a.seq_lens[b], a.max_pages);
  if (L <= 0) {
    out[c] = 0;
    return;
  }
  const int n_used = ((L + kPage - 1) / kPage + a.P - 1) / a.P;
  const size_t rec0 = (size_t)bhq * a.n_split;
  float M = -INFINITY, l = 0.f, o = 0.f;
  for (int u0 = 0; u0 < n_used; u0 += kB16Reduce) {
    float mu[kB16Reduce], lu[kB16Reduce], vu[kB16Reduce];
#pragma unroll
    for (int d = 0; d < kB16Reduce; ++d) {
      const int u = u0 + d;
      const bool ok = u < n_used;
      const size_t rec = rec0 + (ok ? u : 0);
      const float2 ml = ok ? a.part_ml[rec] : make_float2(-INFINITY, 0.f);
      mu[d] = ml.x;
      lu[d] = ml.y;
      vu[d] = ok ? a.part[rec * kHeadDim + c] : 0.f;
    }
    float bm = M;
#pragma unroll
    for (int d = 0; d < kB16Reduce; ++d) bm = fmaxf(bm, mu[d]);
    const float sc = M == -INFINITY ? 0.f : exp2f(M - bm);
    l *= sc;
    o *= sc;
    M = bm;
#pragma unroll
    for (int d = 0; d < kB16Reduce; ++d) {
      const float e = mu[d] == -INFINITY ? 0.f : exp2f(mu[d] - M);
      l = fmaf(e, lu[d], l);
      o = fmaf(e, vu[d], o);
    }
  }
  out[c] = (uint16_t)f32_to_bf16_bits(o / l);
}

}  // namespace

B16Plan make_bf16_decode_plan(int32_t num_kv_heads, int32_t batch, int32_t max_pages, int32_t num_q_heads) {
  B16Plan p{};
  const long long bh = (long long)batch * num_kv_heads;
  // ranges of ~400 pages, at least enough ranges to give each of the ~3 resident
  // block slots per CU (256 CUs) work, at least 16 pages per range
  long long m = 0;
  if (bh > 0) {
    m = max((long long)(max_pages + 399) / 400, (3 * 256 + bh - 1) / bh);
    m = min(m, (long long)(max_pages + 15) / 16);
    m = max(m, (long long)(max_pages + kB16MaxPages - 1) / kB16MaxPages);
    m = max(m, 1LL);
  }
  long long per = m > 0 ? (max_pages + m - 1) / m : 4;
  per = (per + 3) / 4 * 4;   // whole rounds of the 4 waves
  if (per > kB16MaxPages) per = kB16MaxPages;
  p.pages_per_split = (int)per;
  p.n_split = (int)((max_pages + per - 1) / per);
  const size_t n_rec = (size_t)batch * num_q_heads * p.n_split;
  p.part_off = 0;
  p.ml_off = n_rec * kHeadDim * sizeof(float);
  p.bytes = p.ml_off + n_rec * sizeof(float2);
  return p;
}

int launch_bf16_decode(const B16Launch& L, hipStream_t stream) {
  if (L.batch == 0) return 0;
  B16Args a{};
  a.pages = L.pages;
  a.q = L.q;
  a.page_table = L.page_table;
  a.seq_lens = L.seq_lens;
  a.out = L.out;
  a.part = reinterpret_cast<float*>(L.workspace + L.plan.part_off);
  a.part_ml = reinterpret_cast<float2*>(L.workspace + L.plan.ml_off);
  a.sl2e = L.sm_scale * 1.4426950408889634f;
  a.H = L.num_kv_heads;
  a.Hq = L.num_q_heads;
  a.G = L.num_q_heads / L.num_kv_heads;
  a.B = L.batch;
  a.max_pages = L.max_pages;
  a.P = L.plan.pages_per_split;
  a.n_split = L.plan.n_split;
  hipLaunchKernelGGL(b16_split_kernel, dim3(L.batch * L.num_kv_heads * a.n_split), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(b16_reduce_kernel, dim3(L.batch * L.num_q_heads), dim3(kHeadDim), 0, stream, a);
  return hipGetLastError() != hipSuccess;
}

}  // namespace oscar

// ---------------------------------------------------------------------------
// Read-bandwidth probe: streams `bytes` (a multiple of 16) once with 16-byte
// loads, 8 per thread in flight, grid-stride, and stores one xor-word per
// thread.  Its duration gives the HBM read rate a plain stream reaches on the
// device, the practical ceiling next to the 8 TB/s specification.
// ---------------------------------------------------------------------------
namespace oscar {
namespace {
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * kProbeUnroll;
  for (size_t i = (size_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; i < n16; i += stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = i + 256 * u < n16 ? p[i + 256 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}
}  // namespace

int launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<const uint4*>(buf),
                     bytes / 16, sink);
  return hipGetLastError() != hipSuccess;
}
}  // namespace oscar
