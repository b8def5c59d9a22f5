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
  // acc + sum of the eight 16-bit values (v_dot2 against (1, 1), fp32 sum)
  static __device__ __forceinline__ float sum8(v8 x, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    struct P4 { b2 p[4]; };
    const P4 pr = __builtin_bit_cast(P4, x);
    const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(pr.p[i], one, acc, false);
    return acc;
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
  static __device__ __forceinline__ float sum8(v8 x, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    struct P4 { h2 p[4]; };
    const P4 pr = __builtin_bit_cast(P4, x);
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(pr.p[i], one, acc, false);
    return acc;
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

#ifndef ATTN_STAGES
#define ATTN_STAGES 2
#endif
#ifndef ATTN_LDS_PAD
#define ATTN_LDS_PAD 0
#endif
#ifndef ATTN_SETPRIO
#define ATTN_SETPRIO 0
#endif
#ifndef ATTN_LAZY_RESCALE
#define ATTN_LAZY_RESCALE 1
#endif
// rescale threshold of the lazy path, in base-2 exponent units
constexpr float kTau = 8.0f;
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

template <int D, int QB, int KB, bool CAUSAL, bool PP, typename T>
__global__ __launch_bounds__(PP ? 512 : 256) void fwd_kernel(KernelArgs a) {
  // The body is device code only; the host pass just needs the launch stub
  // (instantiating the body there makes clang drop the stub silently).
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef typename E::v4 v4;
  typedef Geo<D, KB> G;
  constexpr int BN = G::BN;
  constexpr int WQ = 32 * QB;         // query rows per wave
  constexpr int WAVES = PP ? 8 : 4;   // ping-pong: two groups of four waves
  constexpr int BM = WAVES * WQ;      // query rows per workgroup
  constexpr int KC = D / 16;          // k-steps of the QK^T product
  constexpr int KCL = KC < 8 ? KC : 8;
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DBL = DB < 4 ? DB : 4;

  // NS K slots and NS V slots, each its own object: slot choice is a
  // compile-time constant below (the loop is unrolled by NS), so the
  // compiler can see that a copy into one slot never aliases reads of
  // another and need not serialise them.
  constexpr int NS = ATTN_STAGES;
  static_assert(NS == 2 || NS == 3, "2 or 3 LDS stages");
  __shared__ __attribute__((aligned(1024))) char kbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf2[NS > 2 ? G::TILE : 1];
  __shared__ __attribute__((aligned(1024))) char vbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf2[NS > 2 ? G::TILE : 1];
#if ATTN_LDS_PAD
  // extra LDS only to cap the number of resident workgroups per CU
  __shared__ char ldspad[ATTN_LDS_PAD];
  if (threadIdx.x == 1u << 30) ldspad[0] = 0;
#endif

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;
  // Group 0 (waves 0-3) issues every K/V copy; with ping-pong, group 1
  // (waves 4-7) runs one phase behind it.
  const int grp = PP ? (wave >> 2) : 0;
  const int lw = wave & 3;     // wave index within its group (copy segments)

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
  // global -> LDS copy: segment seg = lw + 4t, lane i covers row seg*RPS + i/CPR,
  // chunk i%CPR. The swizzles depend on the row modulo 16 (K) or 4 (V); a step
  // of t moves the row by 4*RPS, which keeps both except for K rows of 512
  // bytes (RPS = 2), where the parity of t matters. So one per-lane base
  // (two for that K case) plus a uniform per-segment stride covers all t.
  constexpr int KGP = (G::RPS * 4) % 16 == 0 ? 1 : 2;
  uint32_t kg[KGP], vg0;
#pragma unroll
  for (int t = 0; t < KGP; ++t) {
    const int r = (lw + 4 * t) * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    kg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz_k<D>(r)) << 4) - (uint32_t)t * 4 * G::RPS * RS;
  }
  {
    const int r = lw * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    vg0 = (uint32_t)r * RS + (uint32_t)((pc ^ swz_v<D>(r)) << 4);
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
  // m_run: running max (the exponent reference); l_run: sum of the rounded P
  // that entered P V (normalises O); l_lse: float32 sum of P (gives LSE)
  float m_run[QB], l_run[QB], l_lse[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.f;
    l_lse[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }
  const float c = a.c;

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;
  // Processing order i = 0 .. nt-1 visits KV tile j = nt-1-i (descending).
  // The tiles this wave must mask (tail past N, keys right of its diagonal)
  // form a prefix of that order: tile j is masked iff j >= jm.
  int jm = N >= BN ? (N - BN) / BN + 1 : 0;
  if (CAUSAL) {
    const int x = qw - BN + 1;
    jm = min(jm, x >= 0 ? x / BN + 1 : 0);
  }
  const int n_masked = max(0, nt - jm);

  // LDS ring of NS stages; K runs one tile ahead of V. While tile i's V and
  // tile i+1's K are read, tile i+NS-1's V and tile i+NS's K load. Tile j
  // lives in slot j % NS (slot indices are compile-time constants).
  auto kslot = [&](auto j) -> char* {
    constexpr int J = decltype(j)::value % NS;
    return J == 0 ? kbuf0 : J == 1 ? kbuf1 : kbuf2;
  };
  auto vslot = [&](auto j) -> char* {
    constexpr int J = decltype(j)::value % NS;
    return J == 0 ? vbuf0 : J == 1 ? vbuf1 : vbuf2;
  };
  // Copy tile i (in processing order) of K or V into dst. The row offset of
  // segment t is the per-lane base plus a uniform stride; the base goes
  // through an empty asm so the compiler cannot hoist one VGPR per
  // (slot, segment) out of the loop.
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, bool is_k, char* dst, int i) {
    const uint32_t base = (uint32_t)((nt - 1 - i) * BN) * RS;
    uint32_t g0 = is_k ? kg[0] : vg0;
    uint32_t g1 = is_k ? kg[KGP - 1] : vg0;
    asm volatile("" : "+v"(g0), "+v"(g1));
#pragma unroll
    for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
      const uint32_t voff = ((t & 1) ? g1 : g0) + (base + (uint32_t)t * 4 * G::RPS * RS);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (lw + 4 * t) * 1024), 16, voff, 0, 0, 0);
    }
  };
  // Workgroup barrier at a phase boundary. Every LDS read of this wave has
  // landed first (the compiler may otherwise sink the barrier above a pending
  // ds_read), and no work crosses it in either direction.
  auto barrier = [&]() {
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Start of a tile's MFMA phase: the copies group 0 issued two phases ago
  // have landed (its own wait, then the barrier publishes them).
  // Before iteration i (tile i's V, tile i+1's K): the copies issued after
  // those two -- by the NS-2 iterations before i -- may stay in flight.
  auto sync_tile = [&](int i) {
    if (grp == 0) {
      int later = 0;
#pragma unroll
      for (int t = 1; t <= NS - 2; ++t) later += (i + t < nt) + (i + t + 1 < nt);
      wait_vmcnt_upto15(later * G::SEG_PER_WAVE);
    }
    barrier();
  };
  auto phase_barrier = [&]() {
    if (PP) barrier();
  };

  f32x16 s[KB][QB];
  v8 pk[KB][QB][2];

  // S^T = K Q^T for one tile (QK only: the prologue)
  auto qk = [&](const char* kt) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int t = 0; t < KC * KB; ++t) {
      const int kc = t / KB, kb = t % KB;
      const v8 ka = *(const v8*)(kt + kb * 32 * G::ROWB + (kc / 8) * 256 + kofs[kc % 8]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(ka, qreg[qb][kc], s[kb][qb]);
    }
  };

  // The MFMA phase of one iteration: O^T += V^T P^T for the current tile,
  // interleaved with S^T = K Q^T for the next one (the pages' intra-warpgroup
  // overlap: GEMM1 of tile i and GEMM0 of tile i+1 are independent).
  auto mfma_phase = [&](const LDS_AS char* vt, const char* kt, auto do_qk_tag) {
    constexpr bool DO_QK = decltype(do_qk_tag)::value;
    if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T first (P dies), then S^T = K Q^T (S is born): the two
    // never need registers at the same time
    constexpr int STEPS = DB * KB * 2;  // == KC * KB
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      if (t % ATTN_SB_V == 0) __builtin_amdgcn_sched_barrier(0);
      const int db = t / (2 * KB), kb = (t / 2) % KB, ks = t % 2;
      const LDS_AS char* pv = vt + (kb * 32 + 16 * ks) * G::ROWB + (db / 4) * 256 + vofs[db % 4];
      const v4 lo = E::tr_read(pv);
      const v4 hi = E::tr_read(pv + 8 * G::ROWB);
      const v8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(va, pk[kb][qb][ks], oacc[qb][db]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (DO_QK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KC * KB; ++t) {
        if (t % ATTN_SB_K == 0) __builtin_amdgcn_sched_barrier(0);
        const int kc = t / KB, kb = t % KB;
        const v8 ka = *(const v8*)(kt + kb * 32 * G::ROWB + (kc / 8) * 256 + kofs[kc % 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(ka, qreg[qb][kc], s[kb][qb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of the scores in s (tile starting at key kv0): running
  // max, P = 2^(s c - m c) packed to 16 bits in pk, l, and the O rescale.
  // Scores of keys past N or right of the diagonal become -inf (only the
  // tiles of the masked prefix call this).
  auto apply_mask = [&](int kv0) {
    // key offset within the tile = 4*h32 + o with o a compile-time constant,
    // so compare o against per-lane thresholds (no per-element index vectors)
    const int tn = N - kv0 - 4 * h32;  // o >= tn: key at or past N
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int tc = qw + qb * 32 + l32 - kv0 - 4 * h32;  // o > tc: key right of the diagonal
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = kb * 32 + 8 * (r >> 2) + (r & 3);
          if (o >= tn || (CAUSAL && o > tc)) s[kb][qb][r] = -__builtin_inff();
        }
    }
  };

  auto softmax = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      mx = halves_max(mx);
#if ATTN_LAZY_RESCALE
      // Conditional rescale ("FlashAttention v1-v4", FA4 section): m_run is
      // the reference the exponents are taken against. It only moves when
      // some row's maximum exceeds it by more than kTau base-2 units, so
      // p <= 2^kTau, and O~ and l are rescaled only then. O = O~/l and
      // LSE = m c + log2 l are unchanged in exact arithmetic.
      const float mref = m_run[qb];
      if (__builtin_amdgcn_ballot_w64((mx - mref) * c > kTau) != 0) {
        const float m_new = __builtin_fmaxf(mref, mx);
        const float rho = (m_new == -__builtin_inff()) ? 1.f : exp2_fast((mref - m_new) * c);
        m_run[qb] = m_new;
        l_run[qb] *= rho;
        l_lse[qb] *= rho;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= rho;
      }
      const float ms = (m_run[qb] == -__builtin_inff()) ? 0.f : m_run[qb] * c;
#else
      const float m_new = __builtin_fmaxf(m_run[qb], mx);
      const float ms = (m_new == -__builtin_inff()) ? 0.f : m_new * c;
      const float rho = exp2_fast(m_run[qb] * c - ms);
      m_run[qb] = m_new;
      l_run[qb] *= rho;
      l_lse[qb] *= rho;
#endif
      // P = 2^(s c - m c), rounded to 16 bits in place: these registers are
      // the B operand of the next P V product. l sums the rounded values, so
      // O~/l is an exact convex combination of the weights the product used.
      float rs = 0.f, rs32 = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f32x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            f[e] = exp2_fast(__builtin_fmaf(s[kb][qb][8 * ks + e], c, -ms));
            rs32 += f[e];
          }
          pk[kb][qb][ks] = __builtin_convertvector(f, v8);
          rs = E::sum8(pk[kb][qb][ks], rs);
        }
      l_run[qb] += rs;
      l_lse[qb] += rs32;
#if !ATTN_LAZY_RESCALE
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[qb][db] *= rho;
#endif
    }
  };

  // Ping-pong: group 1 takes one extra barrier first so its phases trail
  // group 0's by one; group 0 takes one extra at the end to match the count.
  if (PP && grp == 1) barrier();

  // prologue: K_0, V_0, K_1, then V_t, K_{t+1} for t < NS-1; S and P of tile 0
  if (grp == 0) {
    issue(rk, true, kslot(Int<0>{}), 0);
    issue(rv, false, vslot(Int<0>{}), 0);
    if (nt > 1) issue(rk, true, kslot(Int<1>{}), 1);
    if (NS > 2) {
      if (nt > 1) issue(rv, false, vslot(Int<1>{}), 1);
      if (nt > 2) issue(rk, true, kslot(Int<2>{}), 2);
    }
    wait_vmcnt<0>();
  }
  barrier();
  qk(kslot(Int<0>{}));
  phase_barrier();
  if (n_masked > 0) apply_mask((nt - 1) * BN);
  softmax();

  // steady state: iteration i (slot phase J = i % NS) consumes V_i and
  // K_{i+1}, loads V_{i+NS-1} and K_{i+NS}
  auto iteration = [&](int i, auto jtag) {
    constexpr int J = decltype(jtag)::value;
    sync_tile(i);  // V_i, K_{i+1} landed; every wave is done with V_{i-1}, K_i
    if (grp == 0) {
      if (i + NS - 1 < nt) issue(rv, false, vslot(Int<J + NS - 1>{}), i + NS - 1);
      if (i + NS < nt) issue(rk, true, kslot(Int<J + NS>{}), i + NS);
    }
    mfma_phase((const LDS_AS char*)vslot(Int<J>{}), kslot(Int<J + 1>{}), TrueT{});
    phase_barrier();
    if (i + 1 < n_masked) apply_mask((nt - 2 - i) * BN);
    softmax();
  };
  // unrolled by NS (the trip count is uniform over the workgroup), which
  // makes every slot index a compile-time constant
  int i = 0;
  for (; i + NS - 1 < nt - 1; i += NS) {
    iteration(i, Int<0>{});
    iteration(i + 1, Int<1>{});
    if (NS > 2) iteration(i + 2, Int<2>{});
  }
  if (i < nt - 1) iteration(i, Int<0>{});
  if (NS > 2 && i + 1 < nt - 1) iteration(i + 1, Int<1>{});
  // drain: the last tile's P V
  sync_tile(nt - 1);
  switch ((nt - 1) % NS) {
    case 0: mfma_phase((const LDS_AS char*)vslot(Int<0>{}), nullptr, FalseT{}); break;
    case 1: mfma_phase((const LDS_AS char*)vslot(Int<1>{}), nullptr, FalseT{}); break;
    default: mfma_phase((const LDS_AS char*)vslot(Int<2>{}), nullptr, FalseT{}); break;
  }
  if (PP && grp == 0) barrier();

  // ---- finalize and epilogue ------------------------------------------------
  T* obase = (T*)a.o + head_off;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const float ll = halves_sum(l_lse[qb]);
    const bool ok = lt > 0.f;  // false for 0 and NaN
    const float inv = ok ? 1.0f / lt : 0.f;
    const int qi = qw + qb * 32 + l32;
    if (qi < N) {
      if (h32 == 0) {
        const float lse = ok ? (m_run[qb] * c + __builtin_amdgcn_logf(ll)) * kLn2 : -__builtin_inff();
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

template <int D, int QB, int KB, bool CAUSAL, bool PP, typename T>
int launch(const FwdArgs& f, hipStream_t st) {
  constexpr int BM = (PP ? 256 : 128) * QB;
  KernelArgs a;
  a.q = f.q; a.k = f.k; a.v = f.v; a.o = f.o; a.lse = f.lse;
  a.B = f.B; a.H = f.H; a.N = f.N;
  a.n_mblk = (f.N + BM - 1) / BM;
  a.c = f.scale_log2;
  const int grid = a.n_mblk * f.B * f.H;
  hipLaunchKernelGGL((fwd_kernel<D, QB, KB, CAUSAL, PP, T>), dim3(grid), dim3(PP ? 512 : 256), 0, st, a);
  return (int)hipGetLastError();
}

// Tile configuration per head dimension: QB = 32-row query blocks per wave,
// KB = 32-key blocks per KV tile.
#ifndef ATTN_D64_QB
#define ATTN_D64_QB 1
#endif
#ifndef ATTN_D64_KB
#define ATTN_D64_KB 2
#endif
#ifndef ATTN_D128_QB
#define ATTN_D128_QB 1
#endif
#ifndef ATTN_D128_KB
#define ATTN_D128_KB 1
#endif
#ifndef ATTN_D64_PP
#define ATTN_D64_PP 0
#endif
#ifndef ATTN_D128_PP
#define ATTN_D128_PP 0
#endif
#ifndef ATTN_D256_PP
#define ATTN_D256_PP 0
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
  constexpr bool PP = D == 64 ? ATTN_D64_PP : D == 128 ? ATTN_D128_PP : ATTN_D256_PP;
  return f.causal ? launch<D, QB, KB, true, PP, T>(f, st) : launch<D, QB, KB, false, PP, T>(f, st);
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
