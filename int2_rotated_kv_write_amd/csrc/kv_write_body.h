// The block-level body of the kv_write kernel, shared by the kv_write launch
// and the first launch of a decode step (which also carries the query
// rotation): rotate (x U on MFMA, then Walsh-Hadamard and bit reversal), clip,
// quantize to INT2 and pack new K/V tokens into the paged cache.
//
// Method: the Italian page "OSCAR: Come Together AI Comprime la KV Cache a
// 2-bit per LLM", sections "I tre fattori della rotazione" (R = U H_Had P_br)
// and "Architettura del Sistema di Serving e Layout di Memoria" (each token is
// rotated, clipped and quantized at write time; sink and recent tokens stay
// BF16); the Spanish summary "Resumen Tecnico: OSCAR ...", section 2.2 B.
#pragma once

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace oscar {
namespace {

// U^T row stride in LDS (288 B): the fragment reads count no LDS bank conflicts on gfx950
// (SQ_LDS_BANK_CONFLICT 0; at 272 B, 4 conflict cycles per 16-byte fragment read)
constexpr int kUtRow = kHeadDim + 16;
constexpr float kInvSqrt128 = 0.08838834764831845f;

// LDS row of channel j in the V transposition buffer: channel bits 3, 4 (the lane's
// quarter when the codes are written) go to row bits 0, 1 and bits 1, 2 to row bits 2, 3,
// so both the byte writes (4 quarters x 16 tokens) and the 16-byte row reads (16
// consecutive channels) fall in distinct LDS banks.
__device__ __forceinline__ int vrow(int j) {
  return ((j >> 3) & 3) | (((j >> 1) & 3) << 2) | ((j & 1) << 4) | (j & 0x60);
}

struct KvWriteArgs {
  const uint16_t* x[2];
  const uint16_t* u[2];
  float clip[2];
  uint16_t* sink[2];
  uint16_t* ring[2];
  uint8_t* pages;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* page_table;
  const int32_t* lens_after;
  int32_t num_tokens, num_heads, max_pages, sink_len, recent, num_tiles;
  int32_t kind_of_z[2];
  // page block format: 64-channel groups (1280 B, fp16 s0 z0 s1 z1 per slot) or one
  // 128-channel group per token (1152 B, fp16 s z per slot)
  int32_t one_group, block_bytes, params_off[2], param_bytes;
};

struct KvWriteSmem {
  __attribute__((aligned(16))) uint16_t ut[kHeadDim * kUtRow];    // U^T, rows padded
  __attribute__((aligned(16))) uint8_t vbytes[4][kHeadDim][16];  // V transposition
};

// Block (bx of gdx along the tile groups, KV head hy, half zi of the present K/V halves).
__device__ __forceinline__ void kv_write_block(const KvWriteArgs& a, KvWriteSmem& sm, int bx, int gdx, int hy,
                                               int zi) {

  uint16_t* ut = sm.ut;
  auto& vbytes = sm.vbytes;

  const int kind = a.kind_of_z[zi];
  const int h = hy;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15;   // token within the tile (MFMA N index)
  const int q = lane >> 4;   // channel quarter: channels 16mt + 4q + r

  const uint16_t* X = a.x[kind];
  // Per-tile inputs, loaded one tile ahead so their latency overlaps the previous tile's
  // math (the first tile's before U^T is staged).  Every load reads a valid token (tokens
  // past the end read the last one), so none needs a branch.  The loads that depend on a
  // tile's indices (its page id, its sequence's length after the call) are issued at the
  // start of the tile, before the next tile's prefetch, so waiting for them leaves the
  // prefetch in flight.
  struct TileIn {
    uint4 x[4];   // x[t][h][32ks + 8q .. +7]
    int b, p;
    bool valid;
  };
  auto load_tile = [&](int tg, TileIn& in) {   // tile 4 tg + wave
    const int t = (tg * 4 + wave) * 16 + n;
    in.valid = t < a.num_tokens;
    const int tc = in.valid ? t : a.num_tokens - 1;
    in.b = a.seq_idx[tc];
    in.p = a.pos[tc];
    const uint16_t* xrow = X + ((size_t)tc * a.num_heads + h) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) in.x[ks] = *reinterpret_cast<const uint4*>(xrow + 32 * ks + 8 * q);
  };
  const int n_groups = (a.num_tiles + 3) / 4;   // groups of four 16-token tiles, one per wave
  TileIn nxt;
  load_tile(bx, nxt);

  // ---- stage U^T: ut[j][i] = U[i][j]; consecutive threads take consecutive rows i,
  // so each LDS store instruction writes consecutive halfwords ----
  const uint16_t* U = a.u[kind] + (size_t)h * kHeadDim * kHeadDim;
  {
    constexpr int kPer = kHeadDim * kHeadDim / 8 / 256;
    uint4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + 256 * k, i = e & (kHeadDim - 1), jb = e >> 7;
      v[k] = reinterpret_cast<const uint4*>(U + i * kHeadDim)[jb];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + 256 * k, i = e & (kHeadDim - 1), j0 = (e >> 7) * 8;
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        ut[(j0 + 2 * q2) * kUtRow + i] = (uint16_t)(w[q2] & 0xFFFFu);
        ut[(j0 + 2 * q2 + 1) * kUtRow + i] = (uint16_t)(w[q2] >> 16);
      }
    }
  }
  __syncthreads();

  // A fragment (mt, ks): rows = output channel 16mt + n', cols = input channels
  // 32ks + 8q' .. +7 (the same k mapping as the B fragment below), read from LDS for
  // every tile: holding all 32 in registers would cost 128 VGPRs and a third of the
  // waves per SIMD.
  auto afrag = [&](int mt, int ks) {
    return *reinterpret_cast<const bf16x8*>(&ut[(16 * mt + n) * kUtRow + 32 * ks + 8 * q]);
  };

  // post-rotation channel j = bitrev7(c) of register i in this lane after the
  // Walsh-Hadamard without swaps back: c = r + 4 (lane bit 5 + 2 (i bit 3)) + 16 (i bit 2 +
  // 2 (lane bit 4) + 4 (i bit 4)), r = i & 3
  auto vj = [&](int i) {
    return 64 * (i & 1) + 32 * ((i >> 1) & 1) + 16 * (q >> 1) + 8 * ((i >> 3) & 1) + 4 * ((i >> 2) & 1) + 2 * (q & 1) +
           ((i >> 4) & 1);
  };
  const float clip_s = a.clip[kind] * 11.313708498984761f;   // clip threshold before the 1/sqrt(128)
  uint16_t* sink_buf = a.sink[kind];
  uint16_t* ring_buf = a.ring[kind];
  const int params_off = a.params_off[kind];
  const bool one_group = a.one_group;


  // The block walks tile groups bx, bx + gdx, ...: U^T is staged once per block.  Two tile
  // buffers alternate (the loop below is unrolled twice), so the tile being processed is
  // never copied out of the registers its loads landed in while the next tile's loads fly.
  int tg = bx;
  auto step = [&](const TileIn& cur, TileIn& nxt_buf) {
    if (tg >= n_groups || tg * 4 + wave >= a.num_tiles) return false;   // wave-uniform
    const bool valid = cur.valid;
    const int b = cur.b, p = cur.p;
    const bool is_int2 = valid && p >= a.sink_len;
    const int32_t pid = a.page_table[(size_t)b * a.max_pages + max(0, min(p >> 4, a.max_pages - 1))];
    const int L_after = a.lens_after[b];
    asm volatile("" ::: "memory");   // keep those two loads ahead of the prefetch
    if (tg + gdx < n_groups) load_tile(tg + gdx, nxt_buf);
    bf16x8 bfrag[4];
    uint4 xraw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      xraw[ks] = cur.x[ks];
      bfrag[ks] = __builtin_bit_cast(bf16x8, xraw[ks]);
    }

    // ---- y^T = U^T x^T ----
    float v[32];   // v[4*mt + r] = channel 16mt + 4q + r of token n
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag(mt, ks), bfrag[ks], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * mt + r] = acc[r];
    }

    // ---- Walsh-Hadamard over the 128 channels (Sylvester order) ----
    // in-register bits: index bits 0,1 (channel bits 0,1) and 2,3,4 (channel bits 4,5,6)
#pragma unroll
    for (int s = 1; s < 32; s <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & s) continue;
        const float x0 = v[i], x1 = v[i | s];
        v[i] = x0 + x1;
        v[i | s] = x0 - x1;
      }
    }
    // cross-lane bits: channel bit 2 = lane bit 4, channel bit 3 = lane bit 5.  Registers
    // x = v[i], y = v[i ^ 8] go through a permlane swap, which leaves in each lane the
    // (bit-clear, bit-set) partner values of one of them; sum and difference are the
    // butterfly outputs, kept where the swap leaves them: after both stages register bit 3
    // holds channel bit 3, lane bit 5 channel bit 2 and lane bit 4 channel bit 5 (vj above).
    // The codes are placed by that map (V through LDS, K by halfwords merged across the
    // lane pair), so no swap puts a result back.
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & 8) continue;
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i | 8]), false, false);
      const float a0 = __uint_as_float(r[0]), b0 = __uint_as_float(r[1]);
      v[i] = a0 + b0;
      v[i | 8] = a0 - b0;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & 8) continue;
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i | 8]), false, false);
      const float a0 = __uint_as_float(r[0]), b0 = __uint_as_float(r[1]);
      v[i] = a0 + b0;
      v[i | 8] = a0 - b0;
    }

    // ---- clip, group min/max (v holds the rotation times sqrt(128): the 1/sqrt(128)
    // goes into the clip threshold, the group parameters and the code scale below) ----
    // channel c = 16mt + 4q + r goes to post-rotation index j = bitrev7(c),
    // whose group j/64 is bit 0 of c, i.e. r & 1.  Clipping is monotone, so the group's
    // clipped min/max are the clipped min/max of the raw values; the values themselves are
    // clipped through their codes below.
    float mn[2] = {INFINITY, INFINITY}, mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      mn[i & 1] = fminf(mn[i & 1], v[i]);
      mx[i & 1] = fmaxf(mx[i & 1], v[i]);
    }
    // across the four quarters through the LDS crossbar (ds_bpermute): this kernel is bound
    // by its vector-ALU issue, and permlane swaps here measured 2-4% slower
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      mn[g] = fminf(mn[g], __shfl_xor(mn[g], 16));
      mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 16));
      mn[g] = __builtin_amdgcn_fmed3f(fminf(mn[g], __shfl_xor(mn[g], 32)), -clip_s, clip_s);
      mx[g] = __builtin_amdgcn_fmed3f(fmaxf(mx[g], __shfl_xor(mx[g], 32)), -clip_s, clip_s);
    }
    if (one_group) {   // one 128-channel group: both halves share its range
      mn[0] = mn[1] = fminf(mn[0], mn[1]);
      mx[0] = mx[1] = fmaxf(mx[0], mx[1]);
    }
    uint32_t sbits[2], zbits[2];
    float sf[2], zf[2], inv[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      sbits[g] = f32_to_f16_bits((mx[g] - mn[g]) * (kInvSqrt128 / 3.0f));
      zbits[g] = f32_to_f16_bits(mn[g] * kInvSqrt128);   // = the smallest scaled value, rounded once
      sf[g] = f16_bits_to_f32(sbits[g]);
      zf[g] = f16_bits_to_f32(zbits[g]);
      inv[g] = sf[g] > 0.f ? __builtin_amdgcn_rcpf(sf[g]) : 0.f;
      zf[g] = -zf[g] * inv[g];          // t = w * inv - z * inv with w = v / sqrt(128)
      inv[g] = inv[g] * kInvSqrt128;
    }
    // t(v) = fma(v, inv, zf) is non-decreasing in v, so the code of the clipped value,
    // clamp(t(clip(v)), 0, 3), is t(v) clamped to [clamp(t(-c), 0, 3), clamp(t(c), 0, 3)]:
    // one med3 per value, bit for bit the same (also where fp16 rounding put z beyond c)
    float lo[2], hi[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      lo[g] = __builtin_amdgcn_fmed3f(fmaf(-clip_s, inv[g], zf[g]), 0.f, 3.f);
      hi[g] = __builtin_amdgcn_fmed3f(fmaf(clip_s, inv[g], zf[g]), 0.f, 3.f);
    }
    float tq[32];   // (w - z) / s clamped to [0, 3]; rounded to the code where it is stored
#pragma unroll
    for (int i = 0; i < 32; ++i) tq[i] = __builtin_amdgcn_fmed3f(fmaf(v[i], inv[i & 1], zf[i & 1]), lo[i & 1], hi[i & 1]);

    // ---- store INT2 ----
    // whole aligned page written by this tile?
    const int b0 = __shfl(b, 0), p0 = __shfl(p, 0);
    const bool full_page = __all(is_int2 && b == b0 && p == p0 + n && (p0 & 15) == 0);
    uint8_t* blk = a.pages + ((size_t)pid * a.num_heads + h) * a.block_bytes;   // used only if is_int2
    const int slot = p & 15;
    if (kind == 0) {
      // K, token-major: channel j = vj(i) is code j % 8 = 4 i2 + 2 (q & 1) + i4 of halfword
      // j / 8 = 8 i0 + 4 i1 + 2 (q >> 1) + i3 (i_k = bit k of i).  A lane holds four codes of
      // each of eight halfwords, the lane 16 apart (the other q & 1) the other four: each
      // lane sums its codes into halfwords (code * 4^position: exact in fp32), pairs them
      // into the dwords of halfwords (2m, 2m + 1), and one permlane swap per two dwords
      // gives each lane of the pair both halves of one of them.
      float w4[4];   // 4^position of code (i2, i4) = k >> 1, k & 1 in this lane
#pragma unroll
      for (int k = 0; k < 4; ++k) w4[k] = (float)(1u << (2 * (4 * (k >> 1) + 2 * (q & 1) + (k & 1))));
      float hf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // [i0 + 2 i1 + 4 i3]
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int u = (i & 3) | (((i >> 3) & 1) << 2), k = (((i >> 2) & 1) << 1) | ((i >> 4) & 1);
        hf[u] = fmaf(__builtin_rintf(tq[i]), w4[k], hf[u]);
      }
      uint32_t d[4];   // [m = i0 + 2 i1]: halfwords with i3 = 0 (low) and 1 (high)
#pragma unroll
      for (int m = 0; m < 4; ++m) d[m] = (uint32_t)hf[m] | ((uint32_t)hf[m + 4] << 16);
      // lane bit 4 clear: dwords m = 0, 2 of the pair; set: m = 1, 3
      const auto s01 = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
      const auto s23 = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
      if (is_int2) {
        // dword m at byte 2 (8 i0 + 4 i1 + 2 (q >> 1)) of the token's codes, i0 = q & 1
        uint8_t* row = blk + kKCodes + 32 * slot + 16 * (q & 1) + 4 * (q >> 1);
        *reinterpret_cast<uint32_t*>(row) = s01[0] | s01[1];
        *reinterpret_cast<uint32_t*>(row + 8) = s23[0] | s23[1];
      }
    } else if (full_page) {
      // V, channel-major, whole page: transpose through LDS, write whole words.  The code
      // byte is the low byte of tq + 2^23 (adding 2^23 rounds to the nearest integer, ties
      // to even, exactly like rint).
      {
        float c23 = 8388608.0f;   // held in a register: a literal operand costs a slower issue
        asm volatile("" : "+v"(c23));
        // token n's byte at 4 (n % 4) + n / 4 of the row: dword d then holds tokens d, d + 4,
        // d + 8, d + 12 in bytes 0..3, and shifting it left by 2 d puts each token t's code at
        // bits 2 t of the page word
        const int vpos = ((n & 3) << 2) | (n >> 2);
#pragma unroll
        for (int i = 0; i < 32; ++i) vbytes[wave][vrow(vj(i))][vpos] = (uint8_t)__float_as_uint(tq[i] + c23);
      }
      wave_lds_sync();
      // every lane of the tile holds the same page: lane 0's id
      const uint8_t* page_blk = a.pages + ((size_t)__shfl(pid, 0) * a.num_heads + h) * a.block_bytes;
      uint32_t words[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 by = *reinterpret_cast<const uint4*>(&vbytes[wave][vrow(2 * lane + c)][0]);
        words[c] = by.x | (by.y << 2) | (by.z << 4) | (by.w << 6);   // codes are 0..3: no carries
      }
      *reinterpret_cast<uint2*>(const_cast<uint8_t*>(page_blk) + kVCodes + 8 * lane) = make_uint2(words[0], words[1]);
      wave_lds_sync();
    } else if (is_int2) {
      // V, partial page: merge this slot's two bits into each word atomically.
      uint32_t* words = reinterpret_cast<uint32_t*>(blk + kVCodes);
      const uint32_t clear = ~(3u << (2 * slot));
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int j = vj(i);
        const uint32_t code = (uint32_t)__builtin_rintf(tq[i]);
        atomicAnd(&words[j], clear);
        if (code) atomicOr(&words[j], code << (2 * slot));
      }
    }
    if (is_int2 && q == 0) {
      const uint32_t lo = sbits[0] | (zbits[0] << 16), hi = sbits[1] | (zbits[1] << 16);
      if (one_group)
        *reinterpret_cast<uint32_t*>(blk + params_off + 4 * slot) = lo;
      else
        *reinterpret_cast<uint2*>(blk + params_off + 8 * slot) = make_uint2(lo, hi);
    }

    // ---- bf16 copies (sink rows, recent ring), last: the sequence length they need was
    // requested at the start of the tile ----
    if (valid) {
      if (p < a.sink_len) {
        uint16_t* row = sink_buf + (((size_t)b * a.num_heads + h) * a.sink_len + p) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4*>(row + 32 * ks + 8 * q) = xraw[ks];
      }
      if (p >= max(a.sink_len, L_after - a.recent)) {
        uint16_t* row = ring_buf + (((size_t)b * a.num_heads + h) * a.recent + (p % a.recent)) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4*>(row + 32 * ks + 8 * q) = xraw[ks];
      }
    }
    tg += gdx;
    return true;
  };
  TileIn nxt2;
  while (step(nxt, nxt2) && step(nxt2, nxt)) {
  }
}

// Kernel arguments and grid of one kv_write launch: (blocks per (KV head, K/V),
// KV heads, present halves).  Blocks per slice: enough for three resident blocks
// per CU over the whole grid (LDS and registers allow three), never more than
// there are tile groups.  Returns false when there is nothing to write.
inline bool kv_write_setup(const KvWriteLaunch& L, int cus, KvWriteArgs& a, dim3& grid) {
  a = KvWriteArgs{};
  int nz = 0;
  const uint16_t* xs[2] = {L.k, L.v};
  for (int kind = 0; kind < 2; ++kind) {
    a.x[kind] = xs[kind];
    if (xs[kind]) a.kind_of_z[nz++] = kind;
  }
  if (nz == 0 || L.num_tokens == 0) return false;
  a.u[0] = L.u_k;
  a.u[1] = L.u_v;
  a.clip[0] = L.clip_k;
  a.clip[1] = L.clip_v;
  a.sink[0] = L.k_sink;
  a.sink[1] = L.v_sink;
  a.ring[0] = L.k_ring;
  a.ring[1] = L.v_ring;
  a.pages = L.pages;
  a.seq_idx = L.seq_idx;
  a.pos = L.pos;
  a.page_table = L.page_table;
  a.lens_after = L.seq_lens_after;
  a.num_tokens = L.num_tokens;
  a.num_heads = L.num_kv_heads;
  a.max_pages = L.max_pages;
  a.sink_len = L.sink;
  a.recent = L.recent;
  a.num_tiles = (L.num_tokens + 15) / 16;
  const PageFormat f = page_format(L.group);
  a.one_group = L.group == 128;
  a.block_bytes = f.block_bytes;
  a.params_off[0] = f.k_params;
  a.params_off[1] = f.v_params;
  a.param_bytes = f.param_bytes;
  const int n_groups = (a.num_tiles + 3) / 4;
  const int per_slice = std::max(1, (3 * cus + L.num_kv_heads * nz - 1) / (L.num_kv_heads * nz));
  grid = dim3(std::min(n_groups, per_slice), L.num_kv_heads, nz);
  return true;
}

}  // namespace
}  // namespace oscar
