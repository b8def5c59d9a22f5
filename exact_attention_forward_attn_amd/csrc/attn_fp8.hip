// FP8 (OCP e4m3) attention forward on gfx950: the quantisation pre-pass and
// the forward kernel.
//
// Pre-pass ("FlashAttention-3 on Hopper", sections 6.3 and 6.4; "FlashAttention-3
// paper review", FP8 section): incoherent processing replaces each row x of Q
// and K by x M with M = H D / sqrt(d) (H Sylvester-ordered +-1 Hadamard, D a
// seeded +-1 diagonal), computed as a fast Walsh-Hadamard transform; then
// every (b, h, 128-row) block (or the whole tensor) gets one float32 scale
// amax / 448 and its elements are rounded to e4m3. V is quantised without
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
// kept in those scaled (base-2) units. P is formed as 2^(s - m + 8)
// (Max_offset = 8 puts the largest probability at 256, inside e4m3's range),
// rounded to e4m3 and fed to the PV product straight from the score
// registers. O~ is kept in units of the current tile's dv: when the tile's dv
// differs from the previous one the rescale factor includes dv_prev/dv_cur,
// and the epilogue multiplies by the last dv and divides by l.
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
// little-endian in one 32-bit word.
__device__ __forceinline__ uint32_t pack_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float sat448(float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.f), 448.f); }

// MODE 0: per-block scales (block_rows = 128), writes codes and descales.
// MODE 1: per-tensor amax pass (atomic max of the float bits into descale[0]).
// MODE 2: per-tensor quantisation with amax read from descale[0].
// One workgroup handles the 128 rows of one (b, h, block); a row of D values
// is spread over D/8 lanes, 8 values per lane.
template <int D, bool HAD, int MODE>
__global__ __launch_bounds__(256) void prep_kernel(PrepKernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int LPR = D / 8;            // lanes per row
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

  float y[ITER][8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int n = blk * 128 + it * RPI + rsub;
    const bool valid = n < a.N;
    const __bf16* src = a.x + ((int64_t)b * a.N + (valid ? n : 0)) * rs + (int64_t)h * D + 8 * li;
    u32x4 raw = valid ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
    bf16x8 xv = __builtin_bit_cast(bf16x8, raw);
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
#pragma unroll
      for (int hs = 8; hs < D; hs <<= 1) {
        const int lm = hs / 8;
        const bool lower = (li & lm) == 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float own = y[it][j];
          const float oth = __shfl_xor(own, lm);
          y[it][j] = lower ? own + oth : oth - own;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) y[it][j] *= sgn[j];
    }
    if (valid) {
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[it][j]));
    }
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
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  if (MODE == 0 && threadIdx.x == 0) a.descale[(int64_t)bh * a.nblk + blk] = scale;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int n = blk * 128 + it * RPI + rsub;
    if (n < a.N) {
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = sat448(y[it][j] / scale);
      u32x2 w;
      w[0] = pack_e4m3(q[0], q[1], q[2], q[3]);
      w[1] = pack_e4m3(q[4], q[5], q[6], q[7]);
      *(u32x2*)(a.x8 + ((int64_t)b * a.N + n) * rs + (int64_t)h * D + 8 * li) = w;
    }
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
  int n_mblk;
  int nsb;        // descale blocks per (b, h): ceil(N/128), or 0 for per-tensor
  float c;        // alpha * log2(e)
};

#ifndef ATTN8_SB_K
#define ATTN8_SB_K 2
#endif

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd8_kernel(Fwd8Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Geo8<D> G;
  constexpr int BN = G::BN;
  constexpr int WQ = 32 * QB;
  constexpr int BM = 4 * WQ;
  constexpr int KC = D / 64;     // k-steps of QK^T (64 dims each)
  constexpr int DB = D / 32;
  static_assert(WQ <= 128 && 128 % WQ == 0, "a wave's rows must sit in one 128-row scale block");

  __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const int BH = a.B * a.H;
  int mblk, bh;
  decode_block(blockIdx.x, a.n_mblk, BH, CAUSAL, mblk, bh);
  const int b = bh / a.H;
  const int hh = bh % a.H;
  const int N = a.N;
  const int q0 = mblk * BM;
  const int qw = q0 + wave * WQ;
  const uint32_t RS = (uint32_t)a.H * D;
  const int64_t head_off = ((int64_t)b * N * a.H + hh) * D;
  const uint32_t span = (uint32_t)(N - 1) * RS + D;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + head_off, span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + head_off, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + head_off, span);

  // descales of this head: index j of the 128-row block, or 0 per tensor
  const float* dqh = a.dq + (a.nsb ? (int64_t)bh * a.nsb : 0);
  const float* dkh = a.dk + (a.nsb ? (int64_t)bh * a.nsb : 0);
  const float* dvh = a.dv + (a.nsb ? (int64_t)bh * a.nsb : 0);
  auto sblk = [&](int row) { return a.nsb ? row / 128 : 0; };

  // Q^T operands: dims 64kc + 32*h32 .. +31 of query row qw + 32qb + l32
  i32x8 qreg[QB][KC];
  float cq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t row = (uint32_t)(qw + qb * 32 + l32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint32_t off = row * RS + 64 * kc + 32 * h32;
      u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
      qreg[qb][kc] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int qrow = min(qw + qb * 32, N - 1);
    cq[qb] = a.c * dqh[sblk(qrow)];
  }

  uint32_t kg[G::SEG_PER_WAVE], vg[G::SEG_PER_WAVE];
#pragma unroll
  for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
    const int seg = wave + 4 * t;
    const int r = seg * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    kg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz_rows<G::ROWB>(r)) << 4);
    vg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz_v8<G::ROWB>(r)) << 4);
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

  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }
  float dv_prev = 1.f;
  bool first = true;

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;

  auto issue_tile = [&](int kv0, int st) {
    const uint32_t base = (uint32_t)kv0 * RS;
#pragma unroll
    for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
      const int seg = wave + 4 * t;
      char* kdst = smem + st * G::STAGE + seg * 1024;
      char* vdst = smem + st * G::STAGE + G::TILE + seg * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)kdst, 16, base + kg[t], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS_AS void*)vdst, 16, base + vg[t], 0, 0, 0);
    }
  };

  auto process = [&](const char* kt, const LDS_AS char* vt, int kv0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc % ATTN8_SB_K == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 lo = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][0]);
        const u32x4 hi = *(const u32x4*)(kt + kb * 32 * G::ROWB + kofs[kc][1]);
        const i32x8 ka = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma8(ka, qreg[qb][kc], s[kb][qb]);
      }
    }
    if (MASKED) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            if (key >= N || (CAUSAL && key > qi)) s[kb][qb][r] = -__builtin_inff();
          }
      }
    }
    const float dk_t = dkh[sblk(kv0)];
    const float dv_t = dvh[sblk(kv0)];
    const float dv_ratio = first ? 1.f : dv_prev / dv_t;
    i32x8 p8[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float ct = cq[qb] * dk_t;
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      mx = halves_max(mx) * ct;
      const float m_new = __builtin_fmaxf(m_run[qb], mx);
      const float ref = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float rho = exp2_fast(m_run[qb] - ref);
      m_run[qb] = m_new;
      const float off = 8.0f - ref;  // Max_offset: the row maximum maps to 2^8
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(__builtin_fmaf(s[kb][qb][r], ct, off));
          s[kb][qb][r] = p;
          rs += p;
        }
      l_run[qb] = l_run[qb] * rho + rs;
      const float f = rho * dv_ratio;
      if (__builtin_amdgcn_ballot_w64(f != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= f;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          p8[qb][4 * kb + g] = (int)pack_e4m3(s[kb][qb][4 * g], s[kb][qb][4 * g + 1], s[kb][qb][4 * g + 2],
                                              s[kb][qb][4 * g + 3]);
    }
    dv_prev = dv_t;
    first = false;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db % 2 == 0) __builtin_amdgcn_sched_barrier(0);
      i32x8 va;
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) {
        const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(vt + vofs[db] + 16 * rd * G::ROWB));
        va[2 * rd] = w[0];
        va[2 * rd + 1] = w[1];
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma8(va, p8[qb], oacc[qb][db]);
    }
  };

  if (nt > 0) issue_tile((nt - 1) * BN, 0);
  for (int it = 0; it < nt; ++it) {
    const int kv0 = (nt - 1 - it) * BN;
    const int st = it & 1;
    if (it + 1 < nt) {
      issue_tile(kv0 - BN, st ^ 1);
      wait_vmcnt<2 * G::SEG_PER_WAVE>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    const bool skip = (CAUSAL && kv0 > qw + WQ - 1) || qw >= N;
    if (!skip) {
      const char* kt = smem + st * G::STAGE;
      const LDS_AS char* vt = (const LDS_AS char*)(smem + st * G::STAGE + G::TILE);
      const bool masked = (kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > qw);
      if (masked)
        process(kt, vt, kv0, TrueT{});
      else
        process(kt, vt, kv0, FalseT{});
    }
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
  }

  // finalize: O = O~ * dv_last / l, LSE = (m + log2 l - 8) ln 2
  __bf16* obase = a.o + head_off;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const bool ok = lt > 0.f;
    const float inv = ok ? dv_prev / lt : 0.f;
    const int qi = qw + qb * 32 + l32;
    if (qi < N) {
      if (h32 == 0) {
        const float lse = ok ? (m_run[qb] + __builtin_amdgcn_logf(lt) - 8.0f) * kLn2 : -__builtin_inff();
        a.lse[(int64_t)bh * N + qi] = lse;
      }
      __bf16* orow = obase + (int64_t)qi * a.H * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = oacc[qb][db][4 * g + e] * inv;
          bf16x4 ov = __builtin_convertvector(f, bf16x4);
          *(u32x2*)(orow + db * 32 + 8 * g + 4 * h32) = __builtin_bit_cast(u32x2, ov);
        }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

#ifndef ATTN8_D64_QB
#define ATTN8_D64_QB 2
#endif
#ifndef ATTN8_D128_QB
#define ATTN8_D128_QB 1
#endif
#ifndef ATTN8_D256_QB
#define ATTN8_D256_QB 1
#endif

template <int D, bool CAUSAL>
int launch_fwd(const FwdArgs& f, hipStream_t st) {
  constexpr int QB = D == 64 ? ATTN8_D64_QB : D == 128 ? ATTN8_D128_QB : ATTN8_D256_QB;
  constexpr int BM = 128 * QB;
  Fwd8Args a;
  a.q = (const uint8_t*)f.q; a.k = (const uint8_t*)f.k; a.v = (const uint8_t*)f.v;
  a.o = (__bf16*)f.o; a.lse = f.lse;
  a.dq = f.dq; a.dk = f.dk; a.dv = f.dv;
  a.B = f.B; a.H = f.H; a.N = f.N;
  a.n_mblk = (f.N + BM - 1) / BM;
  a.nsb = f.block_rows ? (f.N + f.block_rows - 1) / f.block_rows : 0;
  a.c = f.scale_log2;
  const int grid = a.n_mblk * f.B * f.H;
  hipLaunchKernelGGL((fwd8_kernel<D, QB, CAUSAL>), dim3(grid), dim3(256), 0, st, a);
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
