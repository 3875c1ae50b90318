// Device helpers shared by the OSCAR gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kBlockBytes = 1280;   // one page block per (physical page, KV head), 64-channel groups
constexpr int kKCodes = 0;          // K codes, token-major [16][32 B]
constexpr int kVCodes = 512;        // V codes, channel-major [128] uint32, slot t at bits 2t
constexpr int kKParams = 1024;      // [16] x {fp16 s0, z0, s1, z1}
constexpr int kVParams = 1152;
// One 128-channel group per token (2.25 bits per element): the same codes, then
// [16] x {fp16 s, z} for K at 1024 and for V at 1088; 1152 bytes per block.
constexpr int kBlockBytes128 = 1152;
constexpr int kVParams128 = 1088;

struct PageFormat {
  int block_bytes, k_params, v_params, param_bytes;
};
__host__ __device__ constexpr PageFormat page_format(int group) {
  return group == 128 ? PageFormat{kBlockBytes128, kKParams, kVParams128, 4}
                      : PageFormat{kBlockBytes, kKParams, kVParams, 8};
}
constexpr int kMaxGqa = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;   // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
}

// fp32 <- sum of two fp16 products plus c (v_dot2_f32_f16).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

// fp32 <- sum of two bf16 products plus c (v_dot2_f32_bf16); bf16 x bf16 is exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2v, a), __builtin_bit_cast(short2v, b), c,
                                         false);
}

// ---------------------------------------------------------------------------
// Code-pair unpacking.
//
// A 32-bit word holds 16 two-bit codes, code k at bits 2k.  unpack16 turns it
// into 8 fp16 pairs without any integer->float conversion: a code placed in
// fraction bits 4-5 of an fp16 whose exponent is 2^6 reads as 64 + code, in
// bits 6-7 under 2^4 as 16 + code, in bits 8-9 under 2^2 as 4 + code.  The
// word itself, the word >> 6 and the word << 6 each expose codes at those
// three positions of both halves, so 8 pairs cost two shifts and eight
// and-or operations.  Pair i holds codes (k_i, k_i + 8) from the low and
// high halves of the word, with the constant kPairBase[i] added to both.
// Consumers subtract sum(base * weight).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int pair_k(int i) {   // k of pair i
  return i == 0 ? 2 : i == 1 ? 3 : i == 2 ? 4 : i == 3 ? 5 : i == 4 ? 6 : i == 5 ? 7 : i == 6 ? 0 : 1;
}
__host__ __device__ constexpr int pair_base(int i) {
  return (i == 0 || i == 3) ? 64 : (i == 2 || i == 5 || i == 7) ? 4 : 16;
}
__host__ __device__ constexpr int pair_of_k(int k) {  // inverse of pair_k (k in 0..7)
  return k == 2 ? 0 : k == 3 ? 1 : k == 4 ? 2 : k == 5 ? 3 : k == 6 ? 4 : k == 7 ? 5 : k == 0 ? 6 : 7;
}

// Masks in SGPRs, bases in VGPRs, so that (x & m) | b is one v_and_or_b32
// (on gfx9 a VOP3 instruction takes no literal and at most one SGPR).
struct PairConsts {
  uint32_t m64, b64, m16, b16, m4, b4;
  __device__ __forceinline__ PairConsts()
      : m64(0x00300030u), b64(0x54005400u), m16(0x00C000C0u), b16(0x4C004C00u), m4(0x03000300u),
        b4(0x44004400u) {
    asm volatile("" : "+s"(m64), "+s"(m16), "+s"(m4));
    asm volatile("" : "+v"(b64), "+v"(b16), "+v"(b4));
  }
};

// Non-temporal (streaming) loads of data read once per call: they bypass cache
// allocation so the data that is reused stays resident.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
  return make_uint2(v[0], v[1]);
}

// Masks of the value codes: dword d keeps bits 2d, 2d + 1 of each 16-bit half, which as
// an fp16 is the subnormal code * 2^(2d - 24).  In VGPRs (kVgpr) the masking v_and_b32 issues
// at the full rate (measured ~2.5 against ~4.7 cycles per wave64 instruction with an SGPR
// operand); in SGPRs the four registers are saved where VGPRs are the tighter limit.
template <bool kVgpr>
struct ValueMasks {
  uint32_t m[4];
  __device__ __forceinline__ ValueMasks() : m{0x00030003u, 0x000C000Cu, 0x00300030u, 0x00C000C0u} {
    if constexpr (kVgpr)
      asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]));
    else
      asm volatile("" : "+s"(m[0]), "+s"(m[1]), "+s"(m[2]), "+s"(m[3]));
  }
};

__device__ __forceinline__ void unpack16(uint32_t x, uint32_t e[8], const PairConsts& k) {
  const uint32_t r6 = x >> 6, l6 = x << 6;
  e[0] = (x & k.m64) | k.b64;    // k = 2
  e[1] = (x & k.m16) | k.b16;    // k = 3
  e[2] = (x & k.m4) | k.b4;      // k = 4
  e[3] = (r6 & k.m64) | k.b64;   // k = 5
  e[4] = (r6 & k.m16) | k.b16;   // k = 6
  e[5] = (r6 & k.m4) | k.b4;     // k = 7
  e[6] = (l6 & k.m16) | k.b16;   // k = 0
  e[7] = (l6 & k.m4) | k.b4;     // k = 1
}

// 7-bit / 3-bit index reversal.
__host__ __device__ constexpr int bitrev3(int x) { return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1); }
__host__ __device__ constexpr int bitrev7(int x) {
  return ((x & 1) << 6) | ((x & 2) << 4) | ((x & 4) << 2) | (x & 8) | ((x >> 2) & 4) | ((x >> 4) & 2) |
         ((x >> 6) & 1);
}


// ---------------------------------------------------------------------------
// Cross-lane reductions without LDS traffic: DPP inside a 16-lane row, the
// gfx950 permlane swaps across rows.  "tok" reductions combine the lanes that
// share lane%4 (stride 4), "quad" ones the 4 lanes of a quad.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kQuadRot1 = 0x39;   // quad_perm [1, 2, 3, 0]: lane i of a quad reads lane (i + 1) % 4
constexpr int kRowRor12 = 0x12C;   // row_ror:n: lane l of a row reads lane (l - n) % 16

// The value held by lane ^ m, m one of 1, 2, 4, 8, 16, 32 (a constant once inlined), from the
// vector ALU alone: DPP inside a row, permlane swaps across rows.  Every lane of the wave must
// be active.
__device__ __forceinline__ float lane_xor(float x, int m) {
  const int lane = threadIdx.x & 63;
  switch (m) {
    case 1: return dpp<kQuadXor1>(x);
    case 2: return dpp<kQuadXor2>(x);
    case 4: {
      const float up = dpp<kRowRor4>(x), down = dpp<kRowRor12>(x);   // lanes l - 4, l + 4
      return (lane & 4) ? up : down;
    }
    case 8: return dpp<kRowRor8>(x);
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
  }
}
// butterfly reductions over lane bits from .. to (powers of two): every lane gets the result
__device__ __forceinline__ float wave_sum_xor(float v, int from, int to) {
#pragma unroll
  for (int m = from; m <= to; m <<= 1) v += lane_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max_xor(float v, int from, int to) {
#pragma unroll
  for (int m = from; m <= to; m <<= 1) v = fmaxf(v, lane_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_min_xor(float v, int from, int to) {
#pragma unroll
  for (int m = from; m <= to; m <<= 1) v = fminf(v, lane_xor(v, m));
  return v;
}

__device__ __forceinline__ float swap16(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float swap32(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadXor1>(x);
  return x + dpp<kQuadXor2>(x);
}
// reduce over the 16 lanes with the same lane%4 (all four rows, stride 4)
__device__ __forceinline__ float tok_max(float x) {
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  return swap32(swap16(x, true), true);
}
__device__ __forceinline__ float tok_sum(float x) {
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  return swap32(swap16(x, false), false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform int32 read through the scalar cache (constant address space), for arrays
// the kernel never writes: counted by lgkmcnt, so waiting for it does not also wait for
// the vector loads issued before it.
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p, size_t i) {
  typedef __attribute__((address_space(4))) const int32_t* cptr;
  return ((cptr)(p))[i];
}

// A sequence length as the kernels use it: clamped to [0, the tokens a page table row of
// max_pages pages holds], so a length outside the documented range cannot send a read
// past the row or past the records a plan provides.
__device__ __forceinline__ int clamp_len(int L, int max_pages) { return min(max(L, 0), kPage * max_pages); }

// Make this wave's earlier LDS writes visible to its own other lanes: wait for the wave's
// LDS operations only (a workgroup-scope fence would also wait for every global load in
// flight, draining any prefetch), and keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Block barrier for LDS data only: this wave's LDS operations complete, then s_barrier.
// Unlike __syncthreads it does not wait for global loads in flight (a workgroup-scope fence
// would), so a prefetch into registers or LDS keeps streaming across it.  Data a wave loaded
// into LDS by DMA is visible to the others once that wave has waited for it (vmcnt) before
// the barrier.
__device__ __forceinline__ void block_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace oscar
