// Exact attention forward for 16-bit inputs on gfx950 (MI355X).
//
// What is computed (pages on FlashAttention-3): for every (batch, head),
// O = softmax(alpha Q K^T) V and LSE = log-sum-exp of the scaled scores
// ("FlashAttention-3 paper review", problem background; "FlashAttention-3 on
// Hopper", section 3.1). The N x N scores never leave the chip: a workgroup
// owns a block of query rows and streams K/V tiles through LDS, keeping the
// online state (running max m, running sum l, unnormalised output O~) per row
// ("FlashAttention-3 on Hopper", sections 3.2, 4.1, 4.2, 4.6).
//
// gfx950 design
// -------------
// * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 MFMA:
//   K (32 keys x 16 dims) is the A operand read from LDS, Q^T is the B
//   operand kept in VGPRs for the whole KV loop. In the S^T accumulator a
//   lane owns one query (its column) and 16 of the 32 keys, so a row max is
//   15 lane-local max ops plus one v_permlane32_swap, and the softmax state
//   (m, l) of a query lives in a single lane.
// * P never moves: the same registers, converted to 16-bit, are exactly the
//   B operand of O^T += V^T P^T (the contraction over keys may use any key
//   order as long as both operands agree; we use the accumulator's). Each
//   lane's O^T accumulators belong to its query, so the per-row rescale by
//   rho is a per-lane scalar multiply. (The pages keep P in registers as the
//   RS operand of the second GEMM; section 4.5, 5.8.)
// * V^T operands come straight from the row-major V tile through
//   ds_read_b64_tr_b16 (the transpose is done by the LDS read; the pages use
//   a transposed shared-memory view for 16-bit V, section 6.2).
// * K and V tiles are copied global -> LDS with buffer_load ... lds (no VGPR
//   round trip), double buffered; the buffer resource clamps reads past the
//   last key to zero (the role TMA zero-fill plays on the pages, section 4.7).
//   LDS rows are XOR-swizzled at 16-byte granularity so the MFMA operand
//   reads spread over the banks.
// * Each wave owns 32*QB query rows (split-Q, "FlashAttention-3 on Hopper",
//   section 3.4.3); a workgroup is 4 waves (one per SIMD) sharing the K/V
//   tiles. KV tiles are visited in descending order so the tail / diagonal
//   tiles that need masking come first and the steady state runs without
//   mask code (section 4.7, the split loop).
// * Work order: non-causal grids are remapped so that all query blocks of a
//   head land on one XCD (its L2 serves the K/V re-reads); causal grids go
//   longest-first (LPT) over the query blocks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kernel_common.h"

namespace attn {
namespace fwd16 {

using namespace attn::dev;

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

#ifndef ATTN_SB_K
#define ATTN_SB_K 4
#endif
#ifndef ATTN_SB_V
#define ATTN_SB_V 2
#endif

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;
  int n_mblk;     // ceil(N / BM)
  float c;        // alpha * log2(e)
};

template <int D, int QB, int KB, bool CAUSAL, typename T>
__global__ __launch_bounds__(256) void fwd_kernel(KernelArgs a) {
  // The body is device code only; the host pass just needs the launch stub
  // (instantiating the body there makes clang drop the stub silently).
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef typename E::v4 v4;
  typedef Geo<D, KB> G;
  constexpr int BN = G::BN;
  constexpr int WQ = 32 * QB;         // query rows per wave
  constexpr int BM = 4 * WQ;          // query rows per workgroup
  constexpr int KC = D / 16;          // k-steps of the QK^T product
  constexpr int KCL = KC < 8 ? KC : 8;
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DBL = DB < 4 ? DB : 4;

  __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;

  // ---- work decomposition -------------------------------------------------
  const int BH = a.B * a.H;
  int mblk, bh;
  decode_block(blockIdx.x, a.n_mblk, BH, CAUSAL, mblk, bh);
  const int b = bh / a.H;
  const int hh = bh % a.H;
  const int N = a.N;
  const int q0 = mblk * BM;
  const int qw = q0 + wave * WQ;              // first query row of this wave
  const uint32_t RS = (uint32_t)a.H * D * 2;  // bytes between consecutive rows
  const int64_t head_off = ((int64_t)b * N * a.H + hh) * D;  // elements
  const uint32_t span = (uint32_t)(N - 1) * RS + D * 2;       // valid bytes of this head

  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const T*)a.q + head_off, span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T*)a.k + head_off, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T*)a.v + head_off, span);

  // ---- Q^T operands (B operand of S^T = K Q^T), resident in VGPRs ----------
  v8 qreg[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t row = (uint32_t)(qw + qb * 32 + l32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rq, row * RS + (16 * kc + 8 * h32) * 2, 0, 0);
      qreg[qb][kc] = __builtin_bit_cast(v8, raw);
    }
  }

  // ---- per-lane LDS offsets -------------------------------------------------
  // global -> LDS copy: segment seg, lane i covers row seg*RPS + i/CPR, chunk i%CPR
  uint32_t kg[G::SEG_PER_WAVE], vg[G::SEG_PER_WAVE];
#pragma unroll
  for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
    const int seg = wave + 4 * t;
    const int r = seg * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    kg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz_k<D>(r)) << 4);
    vg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz_v<D>(r)) << 4);
  }
  // K operand reads: row kb*32 + l32, logical chunk 2kc + h32
  int kofs[KCL];
#pragma unroll
  for (int i = 0; i < KCL; ++i) kofs[i] = l32 * G::ROWB + (((2 * i + h32) ^ swz_k<D>(l32)) << 4);
  // V^T operand reads (transposing loads): 16-lane group g = lane/16,
  // piece p = lane%16 points at row 4*h32 + p/4, dims db*32 + 16*(g%2) + 4*(p%4)
  int vofs[DBL];
  {
    const int p = lane & 15, dh = (lane >> 4) & 1;
    const int r0 = 4 * h32 + (p >> 2);
    const int sw = swz_v<D>(r0);
#pragma unroll
    for (int i = 0; i < DBL; ++i)
      vofs[i] = r0 * G::ROWB + (((4 * i + 2 * dh + ((p & 3) >> 1)) ^ sw) << 4) + 8 * (p & 1);
  }

  // ---- online softmax state -------------------------------------------------
  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }
  const float c = a.c;

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

  // One KV tile: S^T, (mask), online softmax, O^T += V^T P^T.
  auto process = [&](const char* kt, const LDS_AS char* vt, int kv0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc % ATTN_SB_K == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const v8 ka = *(const v8*)(kt + kb * 32 * G::ROWB + (kc / 8) * 256 + kofs[kc % 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(ka, qreg[qb][kc], s[kb][qb]);
      }
    }
    if (MASKED) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            const bool bad = key >= N || (CAUSAL && key > qi);
            if (bad) s[kb][qb][r] = -__builtin_inff();
          }
      }
    }
    typename E::v8 pk[KB][QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      mx = halves_max(mx);
      const float m_new = __builtin_fmaxf(m_run[qb], mx);
      const float ms = (m_new == -__builtin_inff()) ? 0.f : m_new * c;
      const float rho = exp2_fast(m_run[qb] * c - ms);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(__builtin_fmaf(s[kb][qb][r], c, -ms));
          s[kb][qb][r] = p;
          rs += p;
        }
      l_run[qb] = l_run[qb] * rho + rs;
      // the rescale is skipped when no row of the wave changed its maximum
      if (__builtin_amdgcn_ballot_w64(rho != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= rho;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f32x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = s[kb][qb][8 * ks + e];
          pk[kb][qb][ks] = __builtin_convertvector(f, typename E::v8);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db % ATTN_SB_V == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const LDS_AS char* pv = vt + (kb * 32 + 16 * ks) * G::ROWB + (db / 4) * 256 + vofs[db % 4];
          const v4 lo = E::tr_read(pv);
          const v4 hi = E::tr_read(pv + 8 * G::ROWB);
          const v8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(va, pk[kb][qb][ks], oacc[qb][db]);
        }
    }
  };

  if (nt > 0) issue_tile((nt - 1) * BN, 0);
  for (int it = 0; it < nt; ++it) {
    const int j = nt - 1 - it;
    const int kv0 = j * BN;
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
    // every LDS read of this stage must have landed before any wave refills it
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
  }

  // ---- finalize and epilogue ------------------------------------------------
  T* obase = (T*)a.o + head_off;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const bool ok = lt > 0.f;  // false for 0 and NaN
    const float inv = ok ? 1.0f / lt : 0.f;
    const int qi = qw + qb * 32 + l32;
    if (qi < N) {
      if (h32 == 0) {
        const float lse = ok ? (m_run[qb] * c + __builtin_amdgcn_logf(lt)) * kLn2 : -__builtin_inff();
        a.lse[(int64_t)bh * N + qi] = lse;
      }
      T* orow = obase + (int64_t)qi * a.H * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typedef T t4 __attribute__((ext_vector_type(4)));
          float __attribute__((ext_vector_type(4))) f;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = oacc[qb][db][4 * g + e] * inv;
          t4 ov = __builtin_convertvector(f, t4);
          *(u32x2*)(orow + db * 32 + 8 * g + 4 * h32) = __builtin_bit_cast(u32x2, ov);
        }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, int QB, int KB, bool CAUSAL, typename T>
int launch(const FwdArgs& f, hipStream_t st) {
  constexpr int BM = 128 * QB;
  KernelArgs a;
  a.q = f.q; a.k = f.k; a.v = f.v; a.o = f.o; a.lse = f.lse;
  a.B = f.B; a.H = f.H; a.N = f.N;
  a.n_mblk = (f.N + BM - 1) / BM;
  a.c = f.scale_log2;
  const int grid = a.n_mblk * f.B * f.H;
  hipLaunchKernelGGL((fwd_kernel<D, QB, KB, CAUSAL, T>), dim3(grid), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

// Tile configuration per head dimension: QB = 32-row query blocks per wave,
// KB = 32-key blocks per KV tile.
#ifndef ATTN_D64_QB
#define ATTN_D64_QB 2
#endif
#ifndef ATTN_D64_KB
#define ATTN_D64_KB 2
#endif
#ifndef ATTN_D128_QB
#define ATTN_D128_QB 1
#endif
#ifndef ATTN_D128_KB
#define ATTN_D128_KB 2
#endif
#ifndef ATTN_D256_QB
#define ATTN_D256_QB 1
#endif
#ifndef ATTN_D256_KB
#define ATTN_D256_KB 1
#endif

template <int D, typename T>
int dispatch_d(const FwdArgs& f, hipStream_t st) {
  constexpr int QB = D == 64 ? ATTN_D64_QB : D == 128 ? ATTN_D128_QB : ATTN_D256_QB;
  constexpr int KB = D == 64 ? ATTN_D64_KB : D == 128 ? ATTN_D128_KB : ATTN_D256_KB;
  return f.causal ? launch<D, QB, KB, true, T>(f, st) : launch<D, QB, KB, false, T>(f, st);
}

template <typename T>
int dispatch(const FwdArgs& f, hipStream_t st) {
  switch (f.d) {
    case 64: return dispatch_d<64, T>(f, st);
    case 128: return dispatch_d<128, T>(f, st);
    case 256: return dispatch_d<256, T>(f, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace fwd16

int launch_fwd_16(const FwdArgs& f, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return f.dtype == 0 ? fwd16::dispatch<__bf16>(f, st) : fwd16::dispatch<_Float16>(f, st);
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace attn
