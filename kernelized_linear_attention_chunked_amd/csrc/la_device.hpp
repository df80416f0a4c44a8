// Device helpers shared by the liblinattn kernels (gfx950 / CDNA4 only).
//
// Conventions used by every kernel:
//  * a workgroup is 256 threads = 4 wavefronts of 64 lanes;
//  * lane l of a wave is split as lr = l % 16 (row/column inside a 16x16 MFMA
//    tile) and lg = l / 16 (one of the four lane groups that share the
//    contraction index);
//  * MFMA tiles are 16x16 with fp32 accumulators.  For an accumulator the lane
//    holds column lr and rows 4*lg + q (q = 0..3).  An A operand lane supplies
//    row lr, a B operand lane supplies column lr, and both supply the same set
//    of contraction indices for their lane group; which indices a lane group
//    carries is free as long as A and B agree, which is how the kernels avoid
//    transposes (see each contraction's comment);
//  * bf16 data are handled as raw 16-bit patterns; conversions round to
//    nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));  // 4 bf16 (16x16x16 MFMA operand)

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kChunk = 64;     // tokens per chunk of the chunk-parallel kernels

enum FeatureMap { kEluPlusOne = 0, kReluEps = 1 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two values rounded to bf16 in one word (one v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// phi of the Keras proposal, section "Feature maps": elu(x)+1 with slope 1, or
// relu(x)+eps.  Evaluated in fp32 (the accumulator type).
// elu(x)+1 is taken as max(x + 1, exp(-|x|)): exp(x) >= 1 + x for every x, and
// for x > 0 exp(-x) < 1 < 1 + x, so the maximum is exp(x) for x <= 0 and x + 1
// otherwise, in four instructions (the -|.| is an input modifier of v_exp_f32)
// instead of a compare and a select on top.
template <int FM>
__device__ __forceinline__ float phi(float x, float eps) {
  if constexpr (FM == kEluPlusOne) {
    return fmaxf(x + 1.f, __builtin_amdgcn_exp2f(-fabsf(x * 1.44269504088896340736f)));
  } else {
    return fmaxf(x, 0.f) + eps;
  }
}

// The lane index of the calling thread, passed through an empty asm: values
// derived from it (swizzled LDS addresses, row offsets) are then formed where
// they are used instead of being hoisted out of a loop and held in registers,
// or spilled, across all of it.
__device__ __forceinline__ int opaque_lane(int tid) {
  int x = tid & 63;
  asm volatile("" : "+v"(x));
  return x;
}

// ---------------------------------------------------------------------------
// LDS layouts shared by the chunk kernels.  gfx950 LDS has 64 banks of 4 bytes;
// a 16-byte read serves the 8-lane blocks {0,3}, {1,2}, {4,7}, {5,6} of a
// wavefront together (16 lanes, 256 bytes per cycle), while writes and
// narrower reads go 32 banks wide (measured with SQ_LDS_BANK_CONFLICT).  Tiles
// are rows of 16-byte blocks whose block index is XORed by a function of the
// row, chosen against that model so that the operand reads are conflict-free
// and the transposed writes two-way at most:
//   V^T  [d][token], 128-byte rows : g(r) = ((r >> 1) & 7) ^ ((r >> 4) & 3)
//   K    [token][d], rows of D + one block : 4*bit3(t) ^ 5*bit4(t)
//   Q, S^T [row][d], rows of D + one block : bit3(r)
__device__ __forceinline__ int vt_swz(int r) { return ((r >> 1) & 7) ^ ((r >> 4) & 3); }
__device__ __forceinline__ int kn_swz(int t) { return (4 * ((t >> 3) & 1)) ^ (5 * ((t >> 4) & 1)); }
__device__ __forceinline__ int sq_swz(int r) { return (r >> 3) & 1; }

// Block swizzles of the unpadded 16-bit phi(K) rows (ksw) and phi(Q) / S^T rows
// (qsw), CB 16-byte blocks per row.  Chosen by a search over XOR functions of
// the row bits against a model of the gfx950 LDS banks, for the permuted-row
// and column reads of phi(K), the row reads and 8-byte writes of S^T and
// phi(Q), and the staging writes; the padded rows they replace had measured
// bank-conflict stalls on the S^T and phi(K) operand reads (about 7 and 4% of
// the causal prefill's cycles).
template <int CB>
__device__ __forceinline__ int ksw(int t) {
  if constexpr (CB == 16) return (t & 3) | (((t >> 3) & 3) << 2);
  else if constexpr (CB == 8) return ((t >> 1) & 1) | (((t >> 3) & 3) << 1);
  else return (t >> 3) & 3;
}
template <int CB>
__device__ __forceinline__ int qsw(int r) {
  if constexpr (CB == 16) return r & 15;
  else if constexpr (CB == 8) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// ---------------------------------------------------------------------------
// Operand traits.  A "vector" is 16 bytes of one row in memory: 8 bf16 or 4
// fp32 values.  One vector-step contracts KB = 4 * VEC indices: lane group lg
// carries indices [KB*m + VEC*lg, KB*m + VEC*lg + VEC).  For bf16 that is one
// v_mfma_f32_16x16x32_bf16; for fp32 four v_mfma_f32_16x16x4_f32 (element e of
// the vector in the e-th instruction).
template <typename DT>
struct Op;

template <>
struct Op<uint16_t> {
  static constexpr int VEC = 8;
  static constexpr int KB = 32;
  static constexpr int ESZ = 2;
  __device__ __forceinline__ static void mma(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4_t pack(const float (&f)[8]) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
  }
};

template <>
struct Op<float> {
  static constexpr int VEC = 4;
  static constexpr int KB = 16;
  static constexpr int ESZ = 4;
  __device__ __forceinline__ static void mma(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                 0, 0, 0);
  }
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4_t pack(const float (&f)[4]) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
};

// ---------------------------------------------------------------------------
// I/O element types.  q, k, v, the decay and the outputs are bf16, fp16 or fp32
// in memory; the MFMA operands are bf16 for both 16-bit types (an fp16 operand
// would overflow on the running sums S and Z of long sequences) and fp32 for
// fp32.  Io<IT> decodes 16-byte vectors of the I/O type to fp32, encodes fp32
// results back, and converts a raw 16-byte vector to operand words.
typedef _Float16 f16_t;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <typename IT>
struct Io;

template <>
struct Io<uint16_t> {  // bf16
  using DT = uint16_t;
  __device__ __forceinline__ static float to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
  __device__ __forceinline__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4_t to_operand(const u32x4_t& v) { return v; }
};

template <>
struct Io<f16_t> {  // fp16, fed to bf16 operands
  using DT = uint16_t;
  __device__ __forceinline__ static float to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(f16_t, (uint16_t)bits16);
  }
  __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
  }
  // (the word is copied out of the vector before the bit cast: a bit cast
  // applied to a vector element expression read element 0 whatever the index)
  __device__ __forceinline__ static f32x2_t word_to_f32x2(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
  }
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      const f32x2_t x = word_to_f32x2(w);
      f[2 * i] = x[0];
      f[2 * i + 1] = x[1];
    }
  }
  __device__ __forceinline__ static u32x4_t to_operand(const u32x4_t& v) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      const f32x2_t x = word_to_f32x2(w);
      r[i] = pack_bf16x2(x[0], x[1]);
    }
    return r;
  }
};

template <>
struct Io<float> {
  using DT = float;
  __device__ __forceinline__ static float to_f32(uint32_t bits) { return __uint_as_float(bits); }
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4_t to_operand(const u32x4_t& v) { return v; }
};

// 16x16x32 product of raw fp16 operands (8 values per lane, same lane layout
// as the bf16 form), fp32 accumulation: the products are exact.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void mma_f16(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                               acc, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ void st16(void* p, const u32x4_t& v) { *(u32x4_t*)p = v; }

// Store four consecutive fp32 results as the output dtype.
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  *(u32x2_t*)p = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4_t v = {a, b, c, d};
  *(f32x4_t*)p = v;
}
__device__ __forceinline__ void store4(f16_t* p, float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = Io<f16_t>::pack2(a, b);
  v[1] = Io<f16_t>::pack2(c, d);
  *(u32x2_t*)p = v;
}

}  // namespace la
