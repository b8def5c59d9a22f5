// FP8 (OCP e4m3) attention forward on gfx950: the quantisation pre-pass and
// the forward kernel.
//
// Pre-pass ("FlashAttention-3 on Hopper", sections 6.3 and 6.4; "FlashAttention-3
// paper review", FP8 section): incoherent processing replaces each row x of Q
// and K by x M with M = H D / sqrt(d) (H Sylvester-ordered +-1 Hadamard, D a
// seeded +-1 diagonal), computed as a fast Walsh-Hadamard transform; then
// every (b, h, 128-row) block (or the whole tensor) gets one float32 scale,
// the smallest power of two >= amax / 448, and its elements are rounded to
// e4m3. V is quantised without
// the transform. All arithmetic is float32 in a fixed order (butterfly
// stages h = 1, 2, ..., d/2; one multiply by +-1/sqrt(d); IEEE division by
// the scale; round-to-nearest-even with saturation at 448) so that the codes
// are reproducible bit for bit.
//
// Forward ("FlashAttention-3 on Hopper", sections 6.3 and 6.5; "03 · FA3：Hopper
// 上的异步化与 overlap", section 4): same structure as the 16-bit kernel -- S^T =
// K Q^T so a lane owns one query, online softmax, O^T += V^T P^T -- with the
// 32x32x64 f8f6f4 MFMA. The descales fold into per-tile scalars: the score
// scale of tile (i, j) is alpha*log2(e)*dq_i*dk_j, and the running max is
// kept in those scaled (base-2) units. P is formed as 2^(s - m + kOff8)
// against a reference m that may trail the true max by up to kTau8, so the
// largest probability is at most 2^(kOff8 + kTau8) < 448, inside e4m3's range
// (the pages' Max_offset, section 6.5), rounded to e4m3 and fed to the PV product straight from the score
// registers. Every 128-row block scale is a power of two, and the PV product
// applies the V tile's scale as the E8M0 scale of its operand, so O~ is in
// true units and the epilogue only divides by l (with one scale per tensor,
// O~ is in units of that dv and the epilogue multiplies by it).
// The V^T operand comes from the row-major V tile through ds_read_b64_tr_b8,
// the byte-granular transposing LDS read (the pages transpose V inside the
// kernel through registers; gfx950 does it in the load).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "attn_internal.h"
#include "kernel_common.h"

namespace attn {
namespace fp8 {

using namespace attn::dev;

// ============================================================================
// Quantisation pre-pass
// ============================================================================

struct PrepKernelArgs {
  const __bf16* x;
  uint8_t* x8;
  float* descale;
  int B, H, N;
  int nblk;        // ceil(N / 128)
  float inv_sqrt_d;
  uint64_t seed;
};

__device__ __forceinline__ uint64_t splitmix64(uint64_t s) {
  // first output of a SplitMix64 generator whose state is s
  uint64_t z = s + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Round-to-nearest-even e4m3 codes of (a, b, c, d) after saturation, packed
// little-endian in one 32-bit word. The first conversion writes the low half
// and keeps the high half of its third operand, which the second one then
// overwrites: any word serves there, and a's own bits need no extra register.
__device__ __forceinline__ uint32_t pack_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float sat448(float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.f), 448.f); }

// Block scale: the smallest power of two >= amax / 448 (IEEE float division),
// at least 2^-126; 1 when amax is 0. A power of two divides exactly, and its
// exponent field is the E8M0 scale of the scaled MFMA. The per-tensor scale
// stays amax / 448: it is one number, which the forward applies at the end.
__device__ __forceinline__ float block_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const uint32_t b = __float_as_uint(amax / 448.0f);
  return __uint_as_float((b & 0x7F800000u) + ((b & 0x007FFFFFu) ? 0x00800000u : 0u));
}

// Value of lane (lane ^ LM) for LM < 16, through the DPP lane moves inside a
// row of 16 lanes (no LDS round trip): xor 1 and 2 are quad permutations,
// xor 8 is a rotation of the row by 8, and xor 4 takes the rotation by 12 or
// by 4 depending on the lane's bit 2. li is the lane's index within its
// (16-aligned) group. Wider partners go through the LDS permute.
template <int LM>
__device__ __forceinline__ float lane_xor(float v, int li) {
  const int x = __float_as_int(v);
  if constexpr (LM == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  } else if constexpr (LM == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  } else if constexpr (LM == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true));  // row_ror 8
  } else if constexpr (LM == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x12C, 0xF, 0xF, true);  // row_ror 12: lane + 4
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, true);  // row_ror 4: lane - 4
    return __int_as_float((li & 4) ? dn : up);
  } else {
    return __shfl_xor(v, LM);
  }
}

// MODE 0: per-block scales (block_rows = 128), writes codes and descales.
// MODE 1: per-tensor amax pass (atomic max of the float bits into descale[0]).
// MODE 2: per-tensor quantisation with amax read from descale[0].
// One workgroup handles the 128 rows of one (b, h, block); a row of D values
// is spread over D/8 lanes, 8 values per lane.
template <int D, bool HAD, int MODE>
__global__ __launch_bounds__(256) void prep_kernel(PrepKernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int LSTAGES = LPR == 8 ? 3 : LPR == 16 ? 4 : 5;  // log2(LPR)
  static_assert((1 << LSTAGES) == LPR, "lanes per row");
  constexpr int RPI = 256 / LPR;        // rows per iteration of the workgroup
  constexpr int ITER = 128 / RPI;
  __shared__ float red[4];

  const int blk = blockIdx.x % a.nblk;
  const int bh = blockIdx.x / a.nblk;
  const int b = bh / a.H, h = bh % a.H;
  const int li = threadIdx.x % LPR;     // lane within its row
  const int rsub = threadIdx.x / LPR;   // row within an iteration
  const int64_t rs = (int64_t)a.H * D;  // elements between rows

  float sgn[8];
  if (HAD) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t z = splitmix64(a.seed + (uint64_t)(8 * li + j));
      sgn[j] = (z >> 63) ? -a.inv_sqrt_d : a.inv_sqrt_d;
    }
  }

  // buffer resources over this (b, h)'s rows: rows past N read as zero
  // (which leaves the block amax unchanged) and their stores are dropped,
  // so no lane takes a branch around its loads
  const int64_t head0 = ((int64_t)b * a.N * a.H + h) * D;
  const uint32_t span = (uint32_t)((int64_t)(a.N - 1) * rs + D);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + head0, span * 2);
  const __amdgpu_buffer_rsrc_t rx8 = make_rsrc(a.x8 + head0, span);
  float y[ITER][8];
  float amax = 0.f;
  u32x4 raw[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const uint32_t n = (uint32_t)(blk * 128 + it * RPI + rsub);
    raw[it] = __builtin_amdgcn_raw_buffer_load_b128(rx, (n * (uint32_t)rs + 8 * li) * 2, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    bf16x8 xv = __builtin_bit_cast(bf16x8, raw[it]);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[it][j] = (float)xv[j];
    if (HAD) {
      // butterfly stages h = 1, 2, 4 inside the lane, then 8 .. D/2 across lanes
#pragma unroll
      for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((j & hs) == 0) {
            const float u = y[it][j], w = y[it][j + hs];
            y[it][j] = u + w;
            y[it][j + hs] = u - w;
          }
      }
      // lane stages: the partner is lane li ^ lm; the lower lane of the pair
      // keeps own + other, the upper one other - own (one FMA with a +-1)
      For<0, LSTAGES>::run([&](auto st_tag) ATTN_INLINE {
        constexpr int lm = 1 << decltype(st_tag)::value;
        const float sg = (li & lm) ? -1.f : 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float own = y[it][j];
          y[it][j] = __builtin_fmaf(sg, own, lane_xor<lm>(own, li));
        }
      });
#pragma unroll
      for (int j = 0; j < 8; ++j) y[it][j] *= sgn[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[it][j]));
  }

  if (MODE == 0 || MODE == 1) {
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  }
  if (MODE == 1) {
    if (threadIdx.x == 0) atomicMax((unsigned*)a.descale, __float_as_uint(amax));
    return;
  }
  if (MODE == 2) amax = __uint_as_float(*(const volatile unsigned*)a.descale);
  const float scale = MODE == 0 ? block_scale(amax) : (amax > 0.f ? amax / 448.0f : 1.0f);
  if (MODE == 0 && threadIdx.x == 0) a.descale[(int64_t)bh * a.nblk + blk] = scale;
  // A block scale is a power of two, so multiplying by its (exact)
  // reciprocal rounds exactly like the division; the per-tensor scale
  // amax / 448 is not, and is divided by.
  const float inv = 1.0f / scale;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const uint32_t n = (uint32_t)(blk * 128 + it * RPI + rsub);
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = sat448(MODE == 0 ? y[it][j] * inv : y[it][j] / scale);
    u32x2 w;
    w[0] = pack_e4m3(q[0], q[1], q[2], q[3]);
    w[1] = pack_e4m3(q[4], q[5], q[6], q[7]);
    // non-temporal: the codes are read by a later launch, not from this L2
    __builtin_amdgcn_raw_buffer_store_b64(w, rx8, n * (uint32_t)rs + 8 * li, 0, 2);
  }
#endif
}

__global__ void fill_u32_kernel(unsigned* p, unsigned v) { *p = v; }

__global__ void finalize_tensor_scale_kernel(float* descale) {
  const float amax = __uint_as_float(*(const unsigned*)descale);
  descale[0] = amax > 0.f ? amax / 448.0f : 1.0f;
}

template <int D, bool HAD>
int launch_prep(const PrepArgs& p, hipStream_t st) {
  PrepKernelArgs a;
  a.x = (const __bf16*)p.x;
  a.x8 = (uint8_t*)p.x8;
  a.descale = p.descale;
  a.B = p.B; a.H = p.H; a.N = p.N;
  a.nblk = (p.N + 127) / 128;
  a.inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  a.seed = p.seed;
  const int grid = a.nblk * p.B * p.H;
  if (p.block_rows == 128) {
    hipLaunchKernelGGL((prep_kernel<D, HAD, 0>), dim3(grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, st, (unsigned*)p.descale, 0u);
    hipLaunchKernelGGL((prep_kernel<D, HAD, 1>), dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL((prep_kernel<D, HAD, 2>), dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL(finalize_tensor_scale_kernel, dim3(1), dim3(1), 0, st, p.descale);
  }
  return (int)hipGetLastError();
}

// ============================================================================
// Forward
// ============================================================================

template <int D>
struct Geo8 {
  static constexpr int BN = 64;             // keys per KV tile (two 32-key blocks)
  static constexpr int ROWB = D;            // bytes per key row (e4m3)
  static constexpr int CPR = D / 16;        // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;
  static constexpr int STAGE = 2 * TILE;
  static constexpr int SEGS = TILE / 1024;
  static constexpr int RPS = 1024 / ROWB;
  static constexpr int SEG_PER_WAVE = SEGS / 4;
  static_assert(SEGS % 4 == 0, "tile must split evenly over 4 waves");
};

// Swizzle for the V rows read by the byte-transposing load: each read covers
// 16 rows x 32 bytes per wave.
template <int ROWB>
__device__ __forceinline__ int swz_v8(int r) {
  return ROWB >= 256 ? 2 * (r & 7) : ROWB == 128 ? 2 * ((r >> 1) & 3) : 2 * ((r >> 2) & 1);
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with A scaled by 2^(ea - 127) (E8M0, bias 127) and B by 1.
__device__ __forceinline__ f32x16 mfma8_scale_a(i32x8 a, i32x8 b, f32x16 c, int ea) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, 127);
}

struct Fwd8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  __bf16* o;
  float* lse;
  const float* dq;
  const float* dk;
  const float* dv;
  int B, H, N;
  int Hkv;        // key/value heads; query head h reads head h / (H / Hkv)
  int n_mblk;
  int nsb;        // descale blocks per (b, head): ceil(N/128), or 0 for per-tensor
  float c;        // alpha * log2(e)
  // division constants of n_mblk, B * H, H and H / Hkv
  FastDiv fd_mblk, fd_bh, fd_h, fd_g;
};

// Exponent offset (the pages' Max_offset) and rescale threshold of the lazy
// path, in base-2 units: a score at most kTau8 above the reference gives
// p <= 2^(kOff8 + kTau8) = 2^8.8 < 448, the e4m3 maximum. The pages shift by
// 8 against the exact running max; with a lazy reference the same bound can
// be split as 8 + 0.8, 5 + 3.8 or 4 + 4.8. A larger tau re-does fewer tiles
// (with 8 + 0.8 about 30% of tiles were computed twice; the re-done tile's
// maximum then gets p = 2^kOff8 exactly, which keeps peaked rows accurate),
// and P still reaches up to 2^8.8.
constexpr float kOff8 = 4.0f;
constexpr float kTau8 = 4.8f;
static_assert(kOff8 + kTau8 <= 8.807f, "p must stay below the e4m3 maximum 448");
// The common path tests the rule on the lane's float32 sum of its tile's p
// (computed anyway for l): every p is at most that sum, so a sum of at most
// 2^(kOff8 + kTau8) keeps every p inside e4m3 without a max tree. The tile
// maximum is then needed only on the rare path.
constexpr float kPsum8 = 445.0f;  // <= 2^8.8
static_assert(kPsum8 <= 448.0f, "p must stay below the e4m3 maximum 448");

// Waves per SIMD each kernel is compiled for (its register budget).
template <int D>
constexpr int kWaves8 = D == 256 ? 1 : 2;

// Software pipeline of one wave, as in the 16-bit kernel (tile i = i-th KV
// tile of 64 keys in processing order):
//
//   block i:  S_{i+2}^T = K_{i+2} Q^T  (MFMA, K = 64 dims per step)
//             O^T += V_i^T P_i^T       (MFMA, K = 64 keys per step)
//             P_{i+1} from S_{i+1}     (VALU, in the MFMA shadow)
//
// Descales. The score scale of tile (i, j) is ct = alpha*log2(e)*dq_i*dk_j and
// the running max m is kept in those scaled base-2 units; P = 2^(s ct - m +
// kOff8). The V block scales are powers of two, and the PV product applies
// the tile's as the E8M0 scale of its V^T operand, so O~ stays in true units
// and never needs the dv_prev/dv_cur rescale of the pages' design
// ("FlashAttention-3 on Hopper", section 6.3: the descale folded into the O
// rescale). l sums p in float32 (the pages' row sum), so O = O~ / l.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves8<D>, kWaves8<D>)))
void fwd8_kernel(Fwd8Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Geo8<D> G;
  constexpr int BN = G::BN;
  constexpr int BM = 128;
  constexpr int KC = D / 64;     // k-steps of QK^T (64 dims each)
  constexpr int DB = D / 32;

  __shared__ __attribute__((aligned(1024))) char kbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[G::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  int mblk, bh;
  decode_block((uint32_t)blockIdx.x, a.fd_mblk, a.fd_bh, CAUSAL, mblk, bh);
  const int b = (int)fdiv((uint32_t)bh, a.fd_h);
  const int hh = bh - b * a.H;
  const int N = a.N;
  const int q0 = mblk * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const uint32_t RS = (uint32_t)a.H * D;
  const int64_t head_off = ((int64_t)b * N * a.H + hh) * D;
  const uint32_t span = (uint32_t)(N - 1) * RS + D;
  // grouped heads ("FlashAttention-3 on Hopper", section 5.6.1): the
  // key/value head of query head hh, and its row stride
  const int hk = (int)fdiv((uint32_t)hh, a.fd_g);
  const uint32_t RSK = (uint32_t)a.Hkv * D;
  const int64_t kv_off = ((int64_t)b * N * a.Hkv + hk) * D;
  const uint32_t span_kv = (uint32_t)(N - 1) * RSK + D;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + head_off, span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_off, span_kv);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_off, span_kv);

  // descales of this head: one per 128-row block, or one per tensor
  const int nsb = a.nsb;
  const int64_t sb0 = nsb ? (int64_t)bh * nsb : 0;
  const int64_t sbk0 = nsb ? ((int64_t)b * a.Hkv + hk) * nsb : 0;
  const uint32_t nsb_bytes = (uint32_t)(nsb ? nsb : 1) * 4;
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc(a.dk + sbk0, nsb_bytes);
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc(a.dv + sbk0, nsb_bytes);
  auto sblk = [&](int row) ATTN_INLINE { return nsb ? row / 128 : 0; };

  // Q^T operands: dims 64kc + 32*h32 .. +31 of query row qi
  i32x8 qreg[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const uint32_t off = (uint32_t)qi * RS + 64 * kc + 32 * h32;
    u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    qreg[kc] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // the wave's 32 rows sit in one 128-row scale block
  const float cq = a.c * a.dq[sb0 + sblk(min(qw, N - 1))];

  uint32_t kg[G::SEG_PER_WAVE], vg[G::SEG_PER_WAVE];
#pragma unroll
  for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
    const int seg = wave + 4 * t;
    const int r = seg * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    kg[t] = (uint32_t)r * RSK + (uint32_t)((pc ^ swz_rows<G::ROWB>(r)) << 4);
    vg[t] = (uint32_t)r * RSK + (uint32_t)((pc ^ swz_v8<G::ROWB>(r)) << 4);
  }
  // K operand: row kb*32 + l32, chunks 4kc + 2*h32 + u
  int kofs[KC][2];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      kofs[kc][u] = l32 * G::ROWB + (((4 * kc + 2 * h32 + u) ^ swz_rows<G::ROWB>(l32)) << 4);
  // V^T operand (byte-transposing loads): group g = lane/16 -> (h = g/2, dh = g%2);
  // piece p = lane%16 -> key row 8*(t/4) + 4h + t%4 (t = p/2), dims db*32 + 16dh + 8*(p%2)
  int vofs[DB];
  {
    const int p = lane & 15, dh = (lane >> 4) & 1, t = p >> 1;
    const int r0 = 8 * (t >> 2) + 4 * h32 + (t & 3);
    const int sw = swz_v8<G::ROWB>(r0);
#pragma unroll
    for (int db = 0; db < DB; ++db) vofs[db] = r0 * G::ROWB + (((2 * db + dh) ^ sw) << 4) + 8 * (p & 1);
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // m_run: the reference (scaled base-2 units); l_run: float32 sum of p;
  // ev: the E8M0 exponent of the V scale of the tile whose P sits in slot X
  float m_run = -__builtin_inff(), l_run = 0.f;
  int ev[2] = {127, 127};

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;
  // masked tiles form a prefix of the descending order (as in the 16-bit kernel)
  int jm = N >= BN ? (N - BN) / BN + 1 : 0;
  if (CAUSAL) {
    const int x = qw - BN + 1;
    jm = min(jm, x >= 0 ? x / BN + 1 : 0);
  }
  const int n_masked = max(0, nt - jm);

  auto kslot = [&](auto j) ATTN_INLINE -> char* { return (decltype(j)::value & 1) ? kbuf1 : kbuf0; };
  auto vslot = [&](auto j) ATTN_INLINE -> char* { return (decltype(j)::value & 1) ? vbuf1 : vbuf0; };
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, bool is_k, char* dst, int i) ATTN_INLINE {
    const uint32_t base = (uint32_t)((nt - 1 - i) * BN) * RSK;
#pragma unroll
    for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
      const uint32_t voff = (is_k ? kg[t] : vg[t]) + base;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (wave + 4 * t) * 1024), 16, voff, 0, 0, 0);
    }
  };
  auto barrier = [&]() ATTN_INLINE {
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 s[2][2];    // S^T of two tiles (tile parity) x two 32-key blocks
  i32x8 p8[2];       // P of two tiles as e4m3 bytes (the K = 64 B operand)
  float dkt[2], dvt[2];  // descales of two tiles (tile parity)
  // descales of tile i into slot X (vector loads: they complete with the
  // tile copies, under the same vmcnt wait)
  auto load_desc = [&](auto x_tag, int i) ATTN_INLINE {
    constexpr int X = decltype(x_tag)::value & 1;
    const uint32_t off = (uint32_t)sblk((nt - 1 - i) * BN) * 4;
    dkt[X] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdk, off, 0, 0));
    dvt[X] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdv, off, 0, 0));
  };

  auto qk = [&](auto sb_tag, const char* kt) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
#pragma unroll
    for (int t = 0; t < KC * 2; ++t) {
      const int kc = t / 2, kb = t % 2;
      const u32x4 lo = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][0]);
      const u32x4 hi = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][1]);
      const i32x8 ka = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      s[SB][kb] = mfma8(ka, qreg[kc], kc == 0 ? f32x16{} : s[SB][kb]);
    }
  };
  // Keys at lane offset o >= lim are masked (at or past N, or right of the
  // diagonal). The sign of o - lim selects the score or -inf: no compare
  // mask per element is kept live.
  auto apply_mask = [&](auto sb_tag, int kv0) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    const int tn = N - kv0 - 4 * h32;
    const int lim = CAUSAL ? min(tn, qi - kv0 - 4 * h32 + 1) : tn;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = kb * 32 + 8 * (r >> 2) + (r & 3);
        const int vis = (o - lim) >> 31;  // all ones iff o < lim
        s[SB][kb][r] = __int_as_float((__float_as_int(s[SB][kb][r]) & vis) | (int)(0xff800000u & ~(uint32_t)vis));
      }
  };

  // ---- online softmax of one tile (32 scores per lane) -----------------------
  // Conditional rescale ("FlashAttention v1-v4", FA4 section): p is computed
  // against the current reference and the rule is checked on the lane sums
  // (kPsum8); a tile that breaks it (always the first) is redone after its
  // block against its maximum, and O~ and l are multiplied by
  // rho = 2^(m_old - m_new).
  constexpr int NV = 32;
  float fv[NV];
  float r32p[2], r32v;
  float ct, ot;  // per-tile score scale and exponent offset
  uint32_t pw[8];
  bool need = false;

  struct Sched {
    int M;
    constexpr int span() const { return M > 3 ? M - 2 : 1; }
    constexpr int f(int e) const { return (e * span()) / NV; }
    constexpr int last() const { return f(NV - 1) + 3; }
  };

  // per-tile scalars for the tile with descale slot X
  auto tile_scalars = [&](auto x_tag) ATTN_INLINE {
    constexpr int X = decltype(x_tag)::value & 1;
    ct = cq * dkt[X];
    // exponent offset: Max_offset minus the reference
    ot = (m_run == -__builtin_inff() ? 0.f : -m_run) + kOff8;
  };

  auto sm_step = [&](auto sb_tag, auto k_tag, auto m_tag, auto check_tag) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    constexpr int K = decltype(k_tag)::value;
    constexpr Sched S{decltype(m_tag)::value};
    constexpr bool CHECK = decltype(check_tag)::value;  // the redo pass does not re-test
    For<0, NV>::run([&](auto e_tag) ATTN_INLINE {
      constexpr int e = decltype(e_tag)::value;
      constexpr int f = S.f(e);
      if constexpr (f == K) {
        fv[e] = __builtin_fmaf(s[SB][e / 16][e % 16], ct, ot);
        pin(fv[e]);
      }
      if constexpr (f + 1 == K) {
        fv[e] = exp2_fast(fv[e]);
        pin(fv[e]);
      }
      if constexpr (f + 2 == K) {
        r32p[e % 2] = e < 2 ? fv[e] : r32p[e % 2] + fv[e];
        pin(r32p[e % 2]);
        if constexpr (e % 4 == 3) {
          pw[e / 4] = pack_e4m3(fv[e - 3], fv[e - 2], fv[e - 1], fv[e]);
          pin(pw[e / 4]);
        }
      }
    });
    if constexpr (K == S.last()) {
      r32v = r32p[0] + r32p[1];
      if constexpr (CHECK)
        need = __builtin_amdgcn_ballot_w64(!(r32v <= kPsum8) || m_run == -__builtin_inff()) != 0;
      i32x8 w;
#pragma unroll
      for (int g = 0; g < 8; ++g) w[g] = (int)pw[g];
      p8[SB] = w;
    }
  };
  // After the block that added tile j-1 to O~: the rare reference update for
  // tile j, and tile j's V exponent taken while its descale slot still holds
  // it (the slot is reloaded for tile j+2 before tile j's PV product).
  auto finish_tile = [&](auto sb_tag) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    float f = 1.f;
    if (need) {
      float mx = s[SB][0][0];
#pragma unroll
      for (int e = 1; e < NV; ++e) mx = __builtin_fmaxf(mx, s[SB][e / 16][e % 16]);
      const float mt = halves_max(mx) * ct;
      const float m_new = __builtin_fmaxf(m_run, mt);
      f = (m_new == -__builtin_inff()) ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      ot = (m_new == -__builtin_inff() ? 0.f : -m_new) + kOff8;
      constexpr Sched S1{1};
      For<0, S1.last() + 1>::run([&](auto k) ATTN_INLINE { sm_step(Int<SB>{}, k, Int<1>{}, FalseT{}); });
      l_run *= f;
    }
    if (need) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= f;
    }
    ev[SB] = nsb ? (int)((__float_as_uint(dvt[SB]) >> 23) & 0xFFu) : 127;
    l_run += r32v;
  };

  auto block = [&](auto j_tag, auto qk_tag, auto sm_tag) ATTN_INLINE {
    constexpr int J = decltype(j_tag)::value;
    constexpr int SN = J ^ 1;
    constexpr bool DO_QK = decltype(qk_tag)::value;
    constexpr bool DO_SM = decltype(sm_tag)::value;
    constexpr int MQK = DO_QK ? KC * 2 : 0;
    constexpr int M = MQK + DB;
    constexpr Sched S{M};
    constexpr int STEPS = DO_SM ? (S.last() + 1 > M ? S.last() + 1 : M) : M;
    const LDS_AS char* vt = (const LDS_AS char*)vslot(Int<J>{});
    const char* kt = kslot(Int<J>{});
    auto load_op = [&](auto m_tag) ATTN_INLINE -> i32x8 {
      constexpr int m = decltype(m_tag)::value;
      if constexpr (m < MQK) {
        constexpr int kc = m / 2, kb = m % 2;
        const u32x4 lo = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][0]);
        const u32x4 hi = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][1]);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        constexpr int db = m - MQK;
        i32x8 va;
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) {
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(vt + vofs[db] + 16 * rd * G::ROWB));
          va[2 * rd] = w[0];
          va[2 * rd + 1] = w[1];
        }
        return va;
      }
    };
    auto mfma_op = [&](auto m_tag, i32x8 op) ATTN_INLINE {
      constexpr int m = decltype(m_tag)::value;
      if constexpr (m < MQK) {
        constexpr int kc = m / 2, kb = m % 2;
        s[J][kb] = mfma8(op, qreg[kc], kc == 0 ? f32x16{} : s[J][kb]);
      } else {
        oacc[m - MQK] = mfma8_scale_a(op, p8[J], oacc[m - MQK], ev[J]);
      }
    };
    if constexpr (DO_SM) tile_scalars(Int<SN>{});
    i32x8 ring[2];
    For<0, (2 < M ? 2 : M)>::run([&](auto m) ATTN_INLINE { ring[decltype(m)::value % 2] = load_op(m); });
    For<0, STEPS>::run([&](auto k_tag) ATTN_INLINE {
      constexpr int k = decltype(k_tag)::value;
      if constexpr (k < M) {
        mfma_op(k_tag, ring[k % 2]);
        if constexpr (k + 2 < M) ring[k % 2] = load_op(Int<k + 2>{});
      }
      if constexpr (DO_SM) sm_step(Int<SN>{}, k_tag, Int<M>{}, TrueT{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (DO_SM) finish_tile(Int<SN>{});
    if constexpr (!DO_QK && !DO_SM) {
      // The kernel's last PV products: the tails merge here, and the register
      // copies of the merge read O~ right behind the 16-pass e4m3 MFMA. The
      // compiler spaces that read 19 wait states from the MFMA, and its last
      // result registers then come back stale (passes + 4 = 20 is the spacing
      // it keeps for the 8-pass 16-bit MFMA), so the drain is padded here.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: K_0, K_1, V_0 and the descales of tiles 0, 1; S_0, S_1; P_0
  issue(rk, true, kbuf0, 0);
  if (nt > 1) issue(rk, true, kbuf1, 1);
  issue(rv, false, vbuf0, 0);
  load_desc(Int<0>{}, 0);
  if (nt > 1) load_desc(Int<1>{}, 1);
  wait_vmcnt<0>();
  barrier();
  qk(Int<0>{}, kbuf0);
  if (nt > 1) qk(Int<1>{}, kbuf1);
  barrier();
  if (nt > 2) issue(rk, true, kbuf0, 2);
  if (n_masked > 0) apply_mask(Int<0>{}, (nt - 1) * BN);
  if (n_masked > 1) apply_mask(Int<1>{}, (nt - 2) * BN);
  {
    // The first tile always sets the reference (it starts at -inf): the row
    // maximum first, then P in one pass; O~ and l are still zero.
    tile_scalars(Int<0>{});
    float mx = s[0][0][0];
#pragma unroll
    for (int e = 1; e < NV; ++e) mx = __builtin_fmaxf(mx, s[0][e / 16][e % 16]);
    m_run = halves_max(mx) * ct;
    ot = (m_run == -__builtin_inff() ? 0.f : -m_run) + kOff8;
    constexpr Sched S1{1};
    For<0, S1.last() + 1>::run([&](auto k) ATTN_INLINE { sm_step(Int<0>{}, k, Int<1>{}, FalseT{}); });
    ev[0] = nsb ? (int)((__float_as_uint(dvt[0]) >> 23) & 0xFFu) : 127;
    l_run = r32v;
  }

  auto iteration = [&](int i, auto j_tag, auto qk_tag, auto sm_tag) ATTN_INLINE {
    constexpr int J = decltype(j_tag)::value;
    wait_vmcnt<0>();
    barrier();
    if (i + 1 < nt) issue(rv, false, vslot(Int<J + 1>{}), i + 1);
    if (i + 3 < nt) issue(rk, true, kslot(Int<J + 1>{}), i + 3);
    if (i + 2 < nt) load_desc(Int<J>{}, i + 2);
    block(j_tag, qk_tag, sm_tag);
    if (decltype(qk_tag)::value && i + 2 < n_masked) apply_mask(Int<J>{}, (nt - 3 - i) * BN);
  };
  int i = 0;
  for (; i + 3 < nt; i += 2) {
    iteration(i, Int<0>{}, TrueT{}, TrueT{});
    iteration(i + 1, Int<1>{}, TrueT{}, TrueT{});
  }
  if (i + 2 < nt) {
    iteration(i, Int<0>{}, TrueT{}, TrueT{});
    iteration(i + 1, Int<1>{}, FalseT{}, TrueT{});
    iteration(i + 2, Int<0>{}, FalseT{}, FalseT{});
  } else if (i + 1 < nt) {
    iteration(i, Int<0>{}, FalseT{}, TrueT{});
    iteration(i + 1, Int<1>{}, FalseT{}, FalseT{});
  } else {
    iteration(i, Int<0>{}, FalseT{}, FalseT{});
  }

  // finalize: O = O~ / l (per tensor: O~ dv / l), LSE = (m + log2 l - kOff8) ln 2
  const float lt = halves_sum(l_run);
  const bool ok = lt > 0.f;
  const float inv = ok ? (nsb ? 1.f : dvt[0]) / lt : 0.f;
  if (qi < N && h32 == 0) {
    const float lse = ok ? (m_run + __builtin_amdgcn_logf(lt) - kOff8) * kLn2 : -__builtin_inff();
    a.lse[(int64_t)bh * N + qi] = lse;
  }
  // O through LDS, as in the 16-bit kernel: each wave's 32 x D bf16 tile is
  // written to the K/V slots (free after the barrier) as [32 rows][D] with
  // the 16-byte chunk index XOR the row, and read back row-wise, so each
  // store instruction writes 64 / (D / 8) whole rows instead of 16 bytes
  // into each of 32 rows.
  {
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per store instruction
    constexpr int OW = 32 * D * 2;
    static_assert(4 * OW <= 4 * G::TILE && G::TILE % OW == 0, "the K/V slots hold the workgroup's O tile");
    barrier();
    const int byte = wave * OW, slot = byte / G::TILE, within = byte - slot * G::TILE;
    char* ow = (slot == 0 ? kbuf0 : slot == 1 ? kbuf1 : slot == 2 ? vbuf0 : vbuf1) + within;
    // O is written once (not read again by this launch): non-temporal, as a
    // buffer store over this head's rows (the host keeps them under 2^31 B)
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + head_off, span * 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = oacc[db][4 * g + e] * inv;
        const bf16x4 ov = __builtin_convertvector(f, bf16x4);
        *(u32x2*)(ow + l32 * (2 * D) + (((4 * db + g) ^ (l32 & (CPR - 1))) << 4) + 8 * h32) =
            __builtin_bit_cast(u32x2, ov);
      }
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = it * RPI + lane / CPR, cc = lane % CPR;
      const u32x4 val = *(const u32x4*)(ow + r * (2 * D) + ((cc ^ (r & (CPR - 1))) << 4));
      const int qr = qw + r;
      if (qr < N) __builtin_amdgcn_raw_buffer_store_b128(val, ro, ((uint32_t)qr * RS + 8 * cc) * 2, 0, 2);
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool CAUSAL>
int launch_fwd(const FwdArgs& f, hipStream_t st) {
  constexpr int BM = 128;
  Fwd8Args a;
  a.q = (const uint8_t*)f.q; a.k = (const uint8_t*)f.k; a.v = (const uint8_t*)f.v;
  a.o = (__bf16*)f.o; a.lse = f.lse;
  a.dq = f.dq; a.dk = f.dk; a.dv = f.dv;
  a.B = f.B; a.H = f.H; a.N = f.N;
  a.Hkv = f.Hkv > 0 ? f.Hkv : f.H;
  a.n_mblk = (f.N + BM - 1) / BM;
  a.nsb = f.block_rows ? (f.N + f.block_rows - 1) / f.block_rows : 0;
  a.c = f.scale_log2;
  a.fd_mblk = make_fastdiv(a.n_mblk);
  a.fd_bh = make_fastdiv(f.B * f.H);
  a.fd_h = make_fastdiv(f.H);
  a.fd_g = make_fastdiv(f.H / a.Hkv);
  const int grid = a.n_mblk * f.B * f.H;
  hipLaunchKernelGGL((fwd8_kernel<D, CAUSAL>), dim3(grid), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

template <int D>
int dispatch_fwd(const FwdArgs& f, hipStream_t st) {
  return f.causal ? launch_fwd<D, true>(f, st) : launch_fwd<D, false>(f, st);
}

}  // namespace fp8

int launch_fwd_fp8(const FwdArgs& f, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (f.d) {
    case 64: return fp8::dispatch_fwd<64>(f, st);
    case 128: return fp8::dispatch_fwd<128>(f, st);
    case 256: return fp8::dispatch_fwd<256>(f, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_fp8_prepare(const PrepArgs& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (p.d) {
    case 64: return p.hadamard ? fp8::launch_prep<64, true>(p, st) : fp8::launch_prep<64, false>(p, st);
    case 128: return p.hadamard ? fp8::launch_prep<128, true>(p, st) : fp8::launch_prep<128, false>(p, st);
    case 256: return p.hadamard ? fp8::launch_prep<256, true>(p, st) : fp8::launch_prep<256, false>(p, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
