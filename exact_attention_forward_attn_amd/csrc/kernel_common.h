// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace attn {
namespace dev {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;

struct TrueT {
  static constexpr bool value = true;
};
struct FalseT {
  static constexpr bool value = false;
};
template <int I>
struct Int {
  static constexpr int value = I;
};
template <bool B>
struct Bool {
  typedef FalseT type;
};
template <>
struct Bool<true> {
  typedef TrueT type;
};

// s_waitcnt with only the vector-memory counter constrained (<= N in flight).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt vmcnt(n) for a run-time n in [0, 15] (the immediate is chosen by
// a uniform branch).
__device__ __forceinline__ void wait_vmcnt_upto15(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}
// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Combine x across lanes l and l+32. v_permlane32_swap with both operands
// equal to x returns, per lane, the pair {x of lanes 0-31, x of lanes 32-63}
// of its column, i.e. {x[l], x[l+32]} for l < 32 and {x[l-32], x[l]} above;
// a symmetric op over the pair is the cross-half reduction.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v_exp_f32 (2^x) without range reduction; outputs below 2^-126 flush to 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup id -> (query block, batch*head). Causal grids go longest first
// (the last query blocks see the most keys); non-causal grids are renumbered
// so that each of the 8 XCDs (which receive workgroup ids round-robin) gets
// a contiguous range, keeping one head's query blocks on one L2.
__device__ __forceinline__ void decode_block(int w, int n_mblk, int BH, bool causal, int& mblk, int& bh) {
  if (causal) {
    mblk = n_mblk - 1 - w / BH;
    bh = w % BH;
  } else {
    const int nblk = n_mblk * BH;
    const int per = nblk / 8, rem = nblk % 8;
    const int x = w % 8, kk = w / 8;
    const int L = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + kk;
    mblk = L % n_mblk;
    bh = L / n_mblk;
  }
}

// The same mapping with the two sizes as launch-time division constants
// (scalar multiply-high instead of the float-reciprocal division sequence).
__device__ __forceinline__ void decode_block(uint32_t w, const FastDiv& n_mblk, const FastDiv& BH, bool causal, int& mblk,
                                             int& bh) {
  uint32_t q, r;
  if (causal) {
    fdivmod(w, BH, q, r);
    mblk = (int)(n_mblk.d - 1 - q);
    bh = (int)r;
  } else {
    const uint32_t nblk = n_mblk.d * BH.d;
    const uint32_t per = nblk >> 3, rem = nblk & 7;
    const uint32_t x = w & 7, kk = w >> 3;
    const uint32_t L = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + kk;
    fdivmod(L, n_mblk, q, r);
    mblk = (int)r;
    bh = (int)q;
  }
}

// XOR swizzle of the 16-byte chunk index of LDS row r, for rows of ROWB bytes
// that are read 32 rows x one chunk per instruction: 16 consecutive rows land
// on 16 different bank groups.
template <int ROWB>
__device__ __forceinline__ int swz_rows(int r) {
  static_assert(ROWB == 64 || ROWB == 128 || ROWB >= 256, "row size");
  return ROWB >= 256 ? (r & 15) : ROWB == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}

// Lambdas of the kernels are always inlined (their captures must stay in
// registers).
#define ATTN_INLINE __attribute__((always_inline))

// Empty asm that takes x in VGPRs and may change it: the computation of x
// cannot move past this point, which keeps work inside its pipeline step.
template <typename X>
__device__ __forceinline__ void pin(X& x) {
  asm volatile("" : "+v"(x));
}

// Compile-time loop: f(Int<u>) for u = B .. E-1.
template <int B, int E>
struct For {
  template <typename F>
  static __device__ __forceinline__ void run(F&& f) {
    if constexpr (B < E) {
      f(Int<B>{});
      For<B + 1, E>::run(f);
    }
  }
};

// ---- 16-bit element traits, tile geometry and swizzles (16-bit kernels) ----

template <typename T>
struct Elt;

template <>
struct Elt<__bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 tr_read(const LDS_AS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS v4*)p);
  }
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  // two floats rounded (to nearest even) to one packed 16-bit pair
  static __device__ __forceinline__ v2 cvt2(float a, float b) {
    const float __attribute__((ext_vector_type(2))) f = {a, b};
    return __builtin_convertvector(f, v2);
  }
  // acc + x.x + x.y, summed in float32 (v_dot2 against (1, 1))
  static __device__ __forceinline__ float dot2(v2 x, float acc) {
    const v2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // the two halves of a packed pair widened exactly to float32: a bf16 is
  // the top 16 bits of the float32 with the same value (one shift, one and)
  static __device__ __forceinline__ float lo(v2 x) { return __uint_as_float(__builtin_bit_cast(uint32_t, x) << 16); }
  static __device__ __forceinline__ float hi(v2 x) {
    return __uint_as_float(__builtin_bit_cast(uint32_t, x) & 0xFFFF0000u);
  }
};

template <>
struct Elt<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  static __device__ __forceinline__ v4 tr_read(const LDS_AS char* p) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS raw4*)p));
  }
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ v2 cvt2(float a, float b) {
    const float __attribute__((ext_vector_type(2))) f = {a, b};
    return __builtin_convertvector(f, v2);
  }
  static __device__ __forceinline__ float dot2(v2 x, float acc) {
    const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, one, acc, false);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // the two halves of a packed pair widened exactly to float32
  static __device__ __forceinline__ float lo(v2 x) { return (float)x[0]; }
  static __device__ __forceinline__ float hi(v2 x) { return (float)x[1]; }
};

// Geometry of the K/V tiles in LDS for head dimension D.
template <int D, int KB>
struct Geo {
  static constexpr int BN = 32 * KB;                // keys per KV tile
  static constexpr int ROWB = D * 2;                // bytes per key row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;            // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;            // K tile then V tile
  static constexpr int SEGS = TILE / 1024;          // 1 KiB copy segments per tile
  static constexpr int RPS = 1024 / ROWB;           // rows per segment
  static constexpr int SEG_PER_WAVE = SEGS / 4;
  static_assert(SEGS % 4 == 0, "tile must split evenly over 4 waves");
};

// XOR swizzles of the 16-byte chunk index of LDS row r. K rows are read 32
// rows x one chunk at a time (A operand of S^T); V rows are read through the
// transposing load, 4 rows x 4 chunks per 16 lanes.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return swz_rows<2 * D>(r);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

}  // namespace dev
}  // namespace attn
