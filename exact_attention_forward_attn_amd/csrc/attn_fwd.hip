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

#include <mutex>

#include "attn_internal.h"
#include "kernel_common.h"

// The static split-KV workspace of attn_fwd_ex_noalloc: kStaticWorkspaceBytes
// of device memory per GPU, for callers that cannot allocate. In host code
// `scratch` names a host-side stand-in, never the device memory: host code
// uses only the address hipGetSymbolAddress returns for it on each device.
static __device__ __align__(256) float scratch[attn::kStaticWorkspaceBytes / 4];

namespace attn {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

namespace fwd16 {

using namespace attn::dev;

#ifndef ATTN_DS_LEAD
#define ATTN_DS_LEAD 2
#endif
// rescale threshold of the lazy path, in base-2 exponent units
constexpr float kTau = 8.0f;
constexpr float kPmax = 256.0f;  // 2^kTau
static_assert(kPmax == (float)(1 << (int)kTau), "kPmax must be 2^kTau");

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* opart;       // split partials (null unless nsplit > 1)
  float* lpart;
  const int* cu_q;    // packed batches: row offsets, else null
  const int* cu_k;
  int Hq, Hkv, g;     // query heads, key/value heads, g = Hq / Hkv
  int Nq, Nk;         // rows per batch entry (maxima for packed batches)
  int total_q, total_k;
  int hu;             // head units per batch entry: Hkv if packed, else Hq
  int pack;
  int n_mblk;         // query blocks per (batch entry, head unit)
  int o_nt;           // store O with the non-temporal hint
  int nunit;          // B * hu
  int nsplit, split_len;
  int win_l, win_r;   // window widths (masked kernels; wide = unbounded)
  float c;            // alpha * log2(e)
  // division constants of n_mblk, nunit * nsplit, nsplit, hu and g
  FastDiv fd_mblk, fd_bh, fd_split, fd_hu, fd_g;
};

// Waves per SIMD each kernel is compiled for (its register budget). At
// d = 64 with 32-key tiles a wave needs about 150 VGPRs, so three fit (168
// each): the third wave hides latency where the softmax's VALU work per MFMA
// is highest.
#ifndef ATTN_D128_WAVES
#define ATTN_D128_WAVES 2
#endif
#ifndef ATTN_D64_WAVES
#define ATTN_D64_WAVES 3
#endif
template <int D>
constexpr int kWavesPerEU = D == 256 ? 1 : D == 128 ? ATTN_D128_WAVES : ATTN_D64_WAVES;

// Software pipeline of one wave (tile i = i-th KV tile in processing order):
//
//   block i:  S_{i+2}^T = K_{i+2} Q^T  (MFMA)
//             O^T += V_i^T P_i^T       (MFMA)
//             P_{i+1} from S_{i+1}     (VALU, in the MFMA shadow)
//
// The three parts are independent, so the VALU work of the softmax issues
// while the matrix core runs the two products (the pages overlap the softmax
// of one block with the GEMMs of others, "FlashAttention-3 on Hopper",
// sections 3.4.2 and 4.5). S and P are double-buffered in registers by tile
// parity.
//
// LDS holds two K and two V tiles. K runs two tiles ahead of V: block i
// reads V_i and K_{i+2} while V_{i+1} and K_{i+3} are copied in.
template <int D, int KB, int NW, bool CAUSAL, typename T>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D>, kWavesPerEU<D>)))
void fwd_kernel(KernelArgs a) {
  // The body is device code only; the host pass just needs the launch stub
  // (instantiating the body there makes clang drop the stub silently).
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef typename E::v4 v4;
  typedef typename E::v2 v2;
  typedef Geo<D, KB> G;
  constexpr int BN = G::BN;
  constexpr int BM = 32 * NW;         // query rows per workgroup (32 per wave)
  constexpr int SPW = G::SEGS / NW;   // 1 KiB copy segments per wave and tile
  static_assert(G::SEGS % NW == 0, "a tile must split evenly over the waves");
  constexpr int KC = D / 16;          // k-steps of the QK^T product
  constexpr int KCL = KC < 8 ? KC : 8;
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DBL = DB < 4 ? DB : 4;

  // Each slot is its own object and every slot index below is a compile-time
  // constant (the loop is unrolled by two), so the compiler can see that a
  // copy into one slot never aliases reads of another and need not serialise
  // them.
  __shared__ __attribute__((aligned(1024))) char kbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[G::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;

  // ---- work decomposition -------------------------------------------------
  // workgroup -> (query block, head unit, key range). A head unit is one
  // query head, or with packing one key/value head and its g query heads,
  // whose rows interleave: tile row r is query r / g of head r % g of the
  // group (the KV head of query head h is floor(h / g), "FlashAttention-3 on
  // Hopper", section 5.6.1).
  int mblk, rest;
  decode_block((uint32_t)blockIdx.x, a.fd_mblk, a.fd_bh, CAUSAL, mblk, rest);
  const int unit = (int)fdiv((uint32_t)rest, a.fd_split);
  const int split = rest - unit * a.nsplit;
  const int b = (int)fdiv((uint32_t)unit, a.fd_hu);
  const int hu = unit - b * a.hu;
  // x / g for the non-negative row and head indices below
  auto gdiv = [&](int x) ATTN_INLINE { return (int)fdiv((uint32_t)x, a.fd_g); };
  const int grp = a.g;
  const bool pack = a.pack != 0;
  // rows of this batch entry in q/o and k/v; offsets of packed batches are
  // clamped into the tensors, so malformed offsets never address outside
  int q_row0, len_q, k_row0, len_k;
  if (a.cu_q) {
    q_row0 = min(max(a.cu_q[b], 0), a.total_q);
    len_q = min(min(max(a.cu_q[b + 1], q_row0), a.total_q) - q_row0, a.Nq);
    k_row0 = min(max(a.cu_k[b], 0), a.total_k);
    len_k = min(min(max(a.cu_k[b + 1], k_row0), a.total_k) - k_row0, a.Nk);
  } else {
    q_row0 = b * a.Nq; len_q = a.Nq;
    k_row0 = b * a.Nk; len_k = a.Nk;
  }
  const int rows = pack ? len_q * grp : len_q;  // tile rows of this unit
  const int q0 = mblk * BM;
  if (q0 >= rows) return;  // past a short sequence (uniform over the workgroup)
  const int qw = q0 + wave * 32;              // first tile row of this wave
  const int qi = qw + l32;                    // this lane's tile row
  const int n_i = pack ? gdiv(qi) : qi;       // its query index
  const int hq_i = pack ? hu * grp + (qi - n_i * grp) : hu;  // its query head
  const int hk = pack ? hu : gdiv(hu);
  const int off = len_k - len_q;              // causal offset (bottom-right)
  const uint32_t RSQ = (uint32_t)a.Hq * D * 2;   // bytes between query rows
  const uint32_t RSK = (uint32_t)a.Hkv * D * 2;  // bytes between key rows
  const int hq0 = pack ? hu * grp : hu;       // first query head of the unit
  const int64_t q_off = ((int64_t)q_row0 * a.Hq + hq0) * D;  // elements
  const int64_t k_off = ((int64_t)k_row0 * a.Hkv + hk) * D;
  const uint32_t qspan = (uint32_t)(len_q - 1) * RSQ + (uint32_t)(pack ? grp : 1) * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const T*)a.q + q_off, qspan);
  const uint32_t kspan = len_k > 0 ? (uint32_t)(len_k - 1) * RSK + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T*)a.k + k_off, kspan);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T*)a.v + k_off, kspan);

  // ---- Q^T operands (B operand of S^T = K Q^T), resident in VGPRs ----------
  // (rows past the unit's end read as zero through the buffer range check)
  const uint32_t qofs = (uint32_t)n_i * RSQ + (uint32_t)(hq_i - hq0) * D * 2;
  v8 qreg[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rq, qofs + (16 * kc + 8 * h32) * 2, 0, 0);
    qreg[kc] = __builtin_bit_cast(v8, raw);
  }

  // last key of this lane's row, less the lane's key offset in a tile
  const int diag = n_i + off + a.win_r - 4 * h32;

  // ---- per-lane LDS offsets -------------------------------------------------
  // global -> LDS copy: segment seg = wave + NW t, lane i covers row seg*RPS +
  // i/CPR, chunk i%CPR. The swizzles depend on the row modulo 16 (K) or 4 (V);
  // a step of t moves the row by 4*RPS, which keeps both except for K rows of
  // 512 bytes (RPS = 2), where the parity of t matters. So one per-lane base
  // (two for that K case) plus a uniform per-segment stride covers all t.
  // In general a step of t moves the row by RPS*NW, so K needs one base per
  // residue of t modulo 16 / gcd(RPS*NW, 16).
  constexpr int KSTEP = (G::RPS * NW) % 16;
  constexpr int KGP = KSTEP == 0 ? 1 : KSTEP % 8 == 0 ? 2 : KSTEP % 4 == 0 ? 4 : 16;
  static_assert((G::RPS * NW) % 4 == 0, "the V swizzle must repeat with the segment step");
  uint32_t kg[KGP], vg0;
#pragma unroll
  for (int t = 0; t < KGP; ++t) {
    const int r = (wave + NW * t) * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    kg[t] = (uint32_t)r * RSK + (uint32_t)((pc ^ swz_k<D>(r)) << 4) - (uint32_t)t * NW * G::RPS * RSK;
  }
  {
    const int r = wave * G::RPS + lane / G::CPR;
    const int pc = lane % G::CPR;
    vg0 = (uint32_t)r * RSK + (uint32_t)((pc ^ swz_v<D>(r)) << 4);
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
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  const float c = a.c;
  // m_run: the exponent reference (a running max); msc = m_run * c (0 while
  // m_run = -inf).
  // lsum: the sum of the rounded P that entered P V (it normalises O),
  // accumulated by the matrix core with the 16x16x32 MFMA, one per 16-key P
  // operand. That MFMA reads a lane's 8 P values as contraction rows
  // 8 (l / 16) .. + 7 of column l % 16, so column n gathers lanes n, n + 16,
  // n + 32, n + 48: queries n (lanes n, n + 32, row groups 0 and 2) and
  // n + 16 (lanes n + 16, n + 48, groups 1 and 3). The A operand `sel`
  // picks, for output rows m with m % 8 < 4, groups 0 and 2, and for the
  // others groups 1 and 3. Lane l receives rows 4 (l / 16) .. + 3 of
  // column l % 16, and that row choice lands exactly on its own query
  // l % 32: every register of lsum holds the lane's query sum, and the
  // lane's rho rescales it. l_lse: float32 sum of the unrounded P (gives
  // LSE), this lane's half of its query's keys.
  float m_run = -__builtin_inff(), msc = 0.f;
  f32x4 lsum = {};
  float l_lse = 0.f;
  v8 sel;
  {
    // lane l holds row m = l % 16 of A over contraction group l / 16
    const T one = (T)((((lane >> 2) ^ (lane >> 4)) & 1) == 0 ? 1.0f : 0.0f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }

  // Keys of this workgroup: its key range [kb0, kb1), cut to the keys some
  // query of the workgroup sees. In the masked instantiation query n sees
  // key j iff n + off - win_l <= j <= n + off + win_r: causal is win_r = 0
  // with an unbounded left side (bottom-right alignment, "FlashAttention-3
  // on Hopper", section 4.7, which also names the left boundary of local
  // attention).
  const int kb0 = split * a.split_len;
  const int kb1 = min(len_k, kb0 + a.split_len);
  int kv_end = kb1, kbase = kb0;
  if (CAUSAL) {
    const int n_first = pack ? gdiv(q0) : q0;
    const int n_last = min(len_q - 1, pack ? gdiv(q0 + BM - 1) : q0 + BM - 1);
    kv_end = min(kv_end, n_last + off + a.win_r + 1);
    const int lo = n_first + off - a.win_l;  // first key the workgroup sees
    if (lo > kb0) kbase = kb0 + (min(lo, kb1) - kb0) / BN * BN;
  }
  const int nt = kv_end > kbase ? (kv_end - kbase + BN - 1) / BN : 0;
  // Processing order i = 0 .. nt-1 visits KV tile j = nt-1-i (descending;
  // tile j starts at key kbase + j*BN). The tiles this wave must mask on the
  // right (keys at or past kb1, keys right of its diagonal) form a prefix of
  // that order: tile j is masked iff j >= jm. Tiles holding keys left of a
  // row's window form a suffix: processing index i >= left_from.
  int jm = kb1 - kbase >= BN ? (kb1 - kbase - BN) / BN + 1 : 0;
  int left_from = nt;
  if (CAUSAL) {
    const int x = (pack ? gdiv(qw) : qw) + off + a.win_r - kbase - BN + 1;
    jm = min(jm, x >= 0 ? x / BN + 1 : 0);
    const int lw = (pack ? gdiv(qw + 31) : qw + 31) + off - a.win_l;  // the wave's last left bound
    if (lw > kbase) left_from = max(0, nt - (lw - kbase + BN - 1) / BN);
  }
  const int n_masked = max(0, nt - jm);
  const int wsum = a.win_l + a.win_r;

  // Tile i (processing order) lives in slot i % 2.
  auto kslot = [&](auto j) ATTN_INLINE -> char* { return (decltype(j)::value & 1) ? kbuf1 : kbuf0; };
  auto vslot = [&](auto j) ATTN_INLINE -> char* { return (decltype(j)::value & 1) ? vbuf1 : vbuf0; };
  // Copy tile i (in processing order) of K or V into dst. The row offset of
  // segment t is the per-lane base plus a uniform stride. (All of it goes in
  // the VGPR offset: the buffer range check, which zero-fills rows past N,
  // does not cover the scalar offset.)
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, bool is_k, char* dst, int i) ATTN_INLINE {
    const uint32_t base = (uint32_t)(kbase + (nt - 1 - i) * BN) * RSK;
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      const uint32_t voff = (is_k ? kg[t % KGP] : vg0) + (base + (uint32_t)t * NW * G::RPS * RSK);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (wave + NW * t) * 1024), 16, voff, 0, 0, 0);
    }
  };
  // Workgroup barrier. Every LDS read of this wave has landed first (the
  // compiler may otherwise sink the barrier above a pending ds_read), and no
  // work crosses it in either direction.
  auto barrier = [&]() ATTN_INLINE {
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 s[2][KB];   // S^T of two tiles (index: tile parity)
  v8 pk[2][KB][2];   // P of two tiles, 16-bit, as MFMA B operands

  // S^T = K Q^T of one tile into s[SB] (prologue only)
  auto qk = [&](auto sb_tag, const char* kt) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
#pragma unroll
    for (int t = 0; t < KC * KB; ++t) {
      const int kc = t / KB, kb = t % KB;
      const v8 ka = *(const v8*)(kt + kb * 32 * G::ROWB + (kc / 8) * 256 + kofs[kc % 8]);
      s[SB][kb] = E::mfma(ka, qreg[kc], kc == 0 ? f32x16{} : s[SB][kb]);
    }
  };

  // Scores of keys at or past kb1, right of the diagonal or left of the
  // window become -inf (only the tiles of the masked prefix and suffix call
  // this). kv0: first key of the tile.
  auto apply_mask = [&](auto sb_tag, int kv0) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    // key offset within the tile = 4*h32 + o with o a compile-time constant,
    // so compare o against per-lane thresholds (no per-element index vectors)
    const int tn = kb1 - kv0 - 4 * h32;        // o >= tn: key at or past kb1
    const int tc = diag - kv0;                 // o > tc: key right of the window
    const int tl = tc - wsum;                  // o < tl: key left of the window
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = kb * 32 + 8 * (r >> 2) + (r & 3);
        if (o >= tn || (CAUSAL && (o > tc || o < tl))) s[SB][kb][r] = -__builtin_inff();
      }
  };

  // ---- online softmax of one tile -------------------------------------------
  // Conditional rescale ("FlashAttention v1-v4", FA4 section): the exponent
  // reference m_run moves only when some row's maximum exceeds it by more
  // than kTau base-2 units, so every p = 2^(s c - m_run c) <= 2^kTau. A tile
  // therefore nearly always keeps the current reference, and P is computed
  // against it right away; a tile that breaks the rule (the first one always
  // does) is redone after its
  // block against the new reference, and O~ and l are multiplied by
  // rho = 2^((m_old - m_new) c). O = O~/l and LSE = m c + log2 l are
  // unchanged in exact arithmetic. The check needs no max: every p is at
  // most the lane's float32 sum of its tile, so a sum <= 2^kTau proves the
  // rule held (a reference still at -inf always takes the update, which sets
  // it to the row maximum). O~ is normalised by the sum of the
  // rounded p that entered P V (lsum), so O is an exact convex
  // combination of the weights the product used; l_lse is the float32 sum
  // (gives LSE).
  //
  // The work is cut into single VALU instructions placed on the steps of a
  // block (one MFMA each) so that no instruction waits on the one just
  // before it: score e has its fma at step f(e), its exp at f(e)+1, its
  // float32 add and 16-bit pack at f(e)+2. The sum uses two independent
  // partials. (The sum of the rounded p is left to the matrix core: adding
  // the rounded pairs on the VALU costs as much as the products it saves,
  // and a v_dot2 next to an MFMA in flight waits for that MFMA to finish.)
  constexpr int NV = 16 * KB;  // scores per lane in a tile
  float fv[NV];
  float r32p[2], r32v;
  v2 pp[NV / 2];
  bool need = false;

  // The step schedule of a block of M MFMA steps.
  struct Sched {
    int M;
    constexpr int span() const { return M > 4 ? M - 2 : 1; }
    constexpr int f(int e) const { return (e * span()) / NV; }
    constexpr int last() const { return f(NV - 1) + 3; }
  };

  // VALU work of step k (on the M-step schedule) for the tile in s[SB].
  // WITH_CHECK adds the check of the reference rule.
  auto sm_step = [&](auto sb_tag, auto k_tag, auto m_tag, auto check_tag) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    constexpr int K = decltype(k_tag)::value;
    constexpr Sched S{decltype(m_tag)::value};
    constexpr bool WITH_CHECK = decltype(check_tag)::value;
    For<0, NV>::run([&](auto e_tag) ATTN_INLINE {
      constexpr int e = decltype(e_tag)::value;
      constexpr int f = S.f(e);
      if constexpr (f == K) {
        fv[e] = __builtin_fmaf(s[SB][e / 16][e % 16], c, -msc);
        pin(fv[e]);
      }
      if constexpr (f + 1 == K) {
        fv[e] = exp2_fast(fv[e]);
        pin(fv[e]);
      }
      if constexpr (f + 2 == K) {
        r32p[e % 2] = e < 2 ? fv[e] : r32p[e % 2] + fv[e];
        pin(r32p[e % 2]);
        if constexpr (e % 2 == 1) {
          pp[e / 2] = E::cvt2(fv[e - 1], fv[e]);
          pin(pp[e / 2]);
        }
      }
    });
    if constexpr (K == S.last()) {
      r32v = r32p[0] + r32p[1];
      // !(x <= y) also catches a NaN sum
      if constexpr (WITH_CHECK) need = __builtin_amdgcn_ballot_w64(!(r32v <= kPmax) || m_run == -__builtin_inff()) != 0;
      // the packed pairs become the B operands of the tile's P V product
#pragma unroll
      for (int g = 0; g < 2 * KB; ++g) {
        struct P4 { v2 p[4]; };
        const P4 t = {{pp[4 * g], pp[4 * g + 1], pp[4 * g + 2], pp[4 * g + 3]}};
        pk[SB][g / 2][g % 2] = __builtin_bit_cast(v8, t);
      }
    }
  };
  // Close a tile's softmax after its block: the rare reference update (P
  // redone against the new reference, O~ and l rescaled), then l.
  auto finish_tile = [&](auto sb_tag) ATTN_INLINE {
    constexpr int SB = decltype(sb_tag)::value;
    if (need) {
      float mx = s[SB][0][0];
#pragma unroll
      for (int e = 1; e < NV; ++e) mx = __builtin_fmaxf(mx, s[SB][e / 16][e % 16]);
      const float m_new = __builtin_fmaxf(m_run, halves_max(mx));
      const float rho = (m_new == -__builtin_inff()) ? 1.f : exp2_fast((m_run - m_new) * c);
      m_run = m_new;
      msc = (m_new == -__builtin_inff()) ? 0.f : m_new * c;
      constexpr Sched S1{1};
      For<0, S1.last() + 1>::run([&](auto k) ATTN_INLINE { sm_step(Int<SB>{}, k, Int<1>{}, FalseT{}); });
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= rho;
      lsum *= rho;
      l_lse *= rho;
    }
    l_lse += r32v;
  };

  // Block i of the pipeline (J = i % 2): S_{i+2}^T = K_{i+2} Q^T into s[J]
  // (the buffer S_i came from) and O^T += V_i^T P_i^T, one MFMA per step;
  // each step also issues the LDS reads of the MFMA DS_LEAD steps later and
  // its share of the softmax of S_{i+1}. Fences between the steps keep that
  // order (the compiler would otherwise cluster the VALU work).
  auto block = [&](auto j_tag, auto qk_tag, auto sm_tag) ATTN_INLINE {
    constexpr int J = decltype(j_tag)::value;
    constexpr int SN = J ^ 1;
    constexpr bool DO_QK = decltype(qk_tag)::value;
    constexpr bool DO_SM = decltype(sm_tag)::value;
    constexpr int MPV = DB * KB * 2 + 2 * KB;  // P V, then ones^T P^T
    constexpr int MQK = DO_QK ? KC * KB : 0;
    constexpr int M = MPV + MQK;
    constexpr Sched S{M};
    constexpr int STEPS = DO_SM ? (S.last() + 1 > M ? S.last() + 1 : M) : M;
    constexpr int LEAD = ATTN_DS_LEAD;
    const LDS_AS char* vt = (const LDS_AS char*)vslot(Int<J>{});
    const char* kt = kslot(Int<J>{});
    // MFMA m: QK step (kc, kb) first, then PV step (db, kb, ks), then the
    // row sums (kb, ks)
    auto load_op = [&](auto m_tag) ATTN_INLINE -> v8 {
      constexpr int m = decltype(m_tag)::value;
      if constexpr (m < MQK) {
        constexpr int kc = m / KB, kb = m % KB;
        return *(const v8*)(kt + kb * 32 * G::ROWB + (kc / 8) * 256 + kofs[kc % 8]);
      } else if constexpr (m - MQK >= DB * KB * 2) {
        return sel;
      } else {
        constexpr int t = m - MQK;
        constexpr int db = t / (2 * KB), kb = (t / 2) % KB, ks = t % 2;
        const LDS_AS char* p = vt + (kb * 32 + 16 * ks) * G::ROWB + (db / 4) * 256 + vofs[db % 4];
        const v4 lo = E::tr_read(p);
        const v4 hi = E::tr_read(p + 8 * G::ROWB);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    auto mfma_op = [&](auto m_tag, v8 op) ATTN_INLINE {
      constexpr int m = decltype(m_tag)::value;
      if constexpr (m < MQK) {
        constexpr int kc = m / KB, kb = m % KB;
        s[J][kb] = E::mfma(op, qreg[kc], kc == 0 ? f32x16{} : s[J][kb]);
      } else {
        constexpr int t = m - MQK;
        constexpr int db = t / (2 * KB), kb = (t / 2) % KB, ks = t % 2;
        if constexpr (t < DB * KB * 2) {
          oacc[db] = E::mfma(op, pk[J][kb][ks], oacc[db]);
        } else {
          constexpr int u = t - DB * KB * 2;
          lsum = E::mfma16(op, pk[J][u / 2][u % 2], lsum);
        }
      }
    };
    v8 ring[LEAD];
    For<0, (LEAD < M ? LEAD : M)>::run([&](auto m) ATTN_INLINE { ring[decltype(m)::value % LEAD] = load_op(m); });
    For<0, STEPS>::run([&](auto k_tag) ATTN_INLINE {
      constexpr int k = decltype(k_tag)::value;
      if constexpr (k < M) {
        mfma_op(k_tag, ring[k % LEAD]);
        if constexpr (k + LEAD < M) ring[k % LEAD] = load_op(Int<k + LEAD>{});
      }
      if constexpr (DO_SM) sm_step(Int<SN>{}, k_tag, Int<M>{}, TrueT{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (DO_SM) finish_tile(Int<SN>{});
  };

  // A workgroup with no visible key (causal with N_q > N_k, an empty key
  // range or sequence) skips to the epilogue, which then writes O = 0 and
  // LSE = -inf. nt is uniform over the workgroup, so every barrier inside is
  // reached by all of its waves or by none.
  if (nt > 0) {
  // prologue: K_0, K_1, V_0; S_0, S_1; P_0; then K_2 into K_0's slot
  issue(rk, true, kbuf0, 0);
  if (nt > 1) issue(rk, true, kbuf1, 1);
  issue(rv, false, vbuf0, 0);
  wait_vmcnt<0>();
  barrier();
  qk(Int<0>{}, kbuf0);
  if (nt > 1) qk(Int<1>{}, kbuf1);
  barrier();  // every wave has read K_0
  if (nt > 2) issue(rk, true, kbuf0, 2);
  if (n_masked > 0 || left_from == 0) apply_mask(Int<0>{}, kbase + (nt - 1) * BN);
  if (nt > 1 && (n_masked > 1 || left_from <= 1)) apply_mask(Int<1>{}, kbase + (nt - 2) * BN);
  {
    // The first tile always moves the reference (it starts at -inf), so it
    // takes the row maximum directly and P in one pass; O~ and the sums are
    // still zero, so nothing is rescaled.
    float mx = s[0][0][0];
#pragma unroll
    for (int e = 1; e < NV; ++e) mx = __builtin_fmaxf(mx, s[0][e / 16][e % 16]);
    m_run = halves_max(mx);
    msc = (m_run == -__builtin_inff()) ? 0.f : m_run * c;
    constexpr Sched S1{1};
    For<0, S1.last() + 1>::run([&](auto k) ATTN_INLINE { sm_step(Int<0>{}, k, Int<1>{}, FalseT{}); });
    l_lse = r32v;
  }

  // iteration i: V_i and K_{i+2} have landed (copied during iteration i-1)
  // and every wave is past block i-1, so the slots of V_{i-1} and K_{i+1}
  // take V_{i+1} and K_{i+3}.
  auto iteration = [&](int i, auto j_tag, auto qk_tag, auto sm_tag) ATTN_INLINE {
    constexpr int J = decltype(j_tag)::value;
    wait_vmcnt<0>();
    barrier();
    if (i + 1 < nt) issue(rv, false, vslot(Int<J + 1>{}), i + 1);
    if (i + 3 < nt) issue(rk, true, kslot(Int<J + 1>{}), i + 3);
    block(j_tag, qk_tag, sm_tag);
    if (decltype(qk_tag)::value && (i + 2 < n_masked || i + 2 >= left_from))
      apply_mask(Int<J>{}, kbase + (nt - 3 - i) * BN);
  };
  // unrolled by two (the trip count is uniform over the workgroup), which
  // makes every slot and buffer index a compile-time constant
  int i = 0;
  for (; i + 3 < nt; i += 2) {
    iteration(i, Int<0>{}, TrueT{}, TrueT{});
    iteration(i + 1, Int<1>{}, TrueT{}, TrueT{});
  }
  // i is even here and nt - i is 1, 2 or 3
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
  }  // nt > 0

  // ---- finalize and epilogue ------------------------------------------------
  const float lt = lsum[0];
  const float ll = halves_sum(l_lse);
  const bool ok = lt > 0.f;  // false for 0 and NaN
  const float inv = ok ? 1.0f / lt : 0.f;
  // The row indices are recomputed from a fresh read of the lane id (asm
  // volatile, so the compiler cannot reuse the prologue's values), which
  // frees their registers during the loop.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int qi_e = qw + (lane_e & 31);
  const int ne = pack ? gdiv(qi_e) : qi_e;
  const int hq_e = pack ? hu * grp + (qi_e - ne * grp) : hu;
  if (qi_e < rows) {
    const float lse = ok ? (m_run * c + __builtin_amdgcn_logf(ll)) * kLn2 : -__builtin_inff();
    const int64_t qrow = (int64_t)q_row0 + ne;  // row in q / o
    typedef float f4 __attribute__((ext_vector_type(4)));
    if (a.nsplit > 1) {
      // normalised state of this key range, float32 (merged by the combine
      // kernel)
      const int64_t pr = ((int64_t)split * a.total_q + qrow) * a.Hq + hq_e;
      if (h32 == 0) a.lpart[pr] = lse;
      float* orow = a.opart + pr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = oacc[db][4 * q4 + e] * inv;
          *(f4*)(orow + db * 32 + 8 * q4 + 4 * h32) = f;
        }
    } else {
      if (h32 == 0) {
        // LSE is [B, Hq, Nq] for dense inputs and [Hq, total_q] for packed
        // batches
        const int64_t li = a.cu_q ? (int64_t)hq_e * a.total_q + qrow : ((int64_t)b * a.Hq + hq_e) * a.Nq + ne;
        a.lse[li] = lse;
      }
    }
  }
  if (a.nsplit <= 1) {
    // O goes out through LDS: the accumulator gives a lane 4 consecutive
    // dims of its row at a 32-byte stride, so stored directly each
    // instruction would write 16 bytes into each of 32 rows. Written to LDS
    // as [32 rows][D] (16-byte chunk index XOR the row, so the 32 rows of a
    // write land on different banks) and read back row-wise, every store
    // instruction writes 64 / (D / 8) whole rows. The wave's 32 x D area is
    // carved from the K/V slots, free once every wave has passed its last
    // block (the barrier; a workgroup that saw no key has issued no copy).
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per store instruction
    constexpr int OW = 32 * D * 2;  // bytes of one wave's area
    constexpr bool IN_SLOTS = NW * OW <= 4 * G::TILE && G::TILE % OW == 0;
    // (eight-wave workgroups at d = 128 need more than the slots hold)
    __shared__ __attribute__((aligned(1024))) char oextra[IN_SLOTS ? 16 : NW * OW];
    char* ow;
    if constexpr (IN_SLOTS) {
      barrier();
      // the slots are four separate objects: wave w's area starts at byte
      // w * OW of the sequence kbuf0, kbuf1, vbuf0, vbuf1
      const int byte = wave * OW, slot = byte / G::TILE, within = byte - slot * G::TILE;
      ow = (slot == 0 ? kbuf0 : slot == 1 ? kbuf1 : slot == 2 ? vbuf0 : vbuf1) + within;
    } else {
      ow = oextra + wave * OW;
    }
    const int rl = lane_e & 31, hl = lane_e >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        typedef T t4 __attribute__((ext_vector_type(4)));
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = oacc[db][4 * q4 + e] * inv;
        const t4 ov = __builtin_convertvector(f, t4);
        *(u32x2*)(ow + rl * (2 * D) + (((4 * db + q4) ^ (rl & (CPR - 1))) << 4) + 8 * hl) = __builtin_bit_cast(u32x2, ov);
      }
    // this unit's O rows, laid out like its Q rows (the non-temporal path)
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const T*)a.o + q_off, qspan);
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = it * RPI + lane_e / CPR, cc = lane_e % CPR;
      const u32x4 val = *(const u32x4*)(ow + r * (2 * D) + ((cc ^ (r & (CPR - 1))) << 4));
      const int qr = qw + r;
      if (qr < rows) {
        const int nr = pack ? gdiv(qr) : qr;
        const int hr = pack ? hu * grp + (qr - nr * grp) : hu;
        if (a.o_nt) {
          // a buffer store, whose cache policy is an immediate (a plain
          // store with the hint would be merged with the other branch)
          const uint32_t ob = (uint32_t)nr * RSQ + (uint32_t)(hr - hq0) * (D * 2) + 16u * cc;
          __builtin_amdgcn_raw_buffer_store_b128(val, ro, ob, 0, 2);
        } else {
          *(u32x4*)((T*)a.o + (((int64_t)q_row0 + nr) * a.Hq + hr) * D + 8 * cc) = val;
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---- split-KV combine -------------------------------------------------------
// Merges the normalised states (O_s, LSE_s) that the key ranges of one
// (query row, query head) left in the workspace: LSE = ln sum_s e^(LSE_s),
// O = sum_s e^(LSE_s - LSE) O_s. This is the block-combine rule of
// "FlashAttention-3 on Hopper", section 3.2.1, in the units O = O~ / l and
// LSE = m + ln l; the pages name a separate combine kernel for split-KV
// (chapter 10). One wave per (row, head); lane l owns dims D/64 * l ...
struct CombineArgs {
  const float* opart;  // [nsplit, npairs, D]
  const float* lpart;  // [nsplit, npairs]
  void* o;             // [total_q, Hq, D] (pair = row * Hq + head)
  float* lse;
  int npairs;          // total_q * Hq
  int nsplit;
  int Hq, Nq, total_q;
  int varlen;          // LSE layout: [Hq, total_q] if set, else [B, Hq, Nq]
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int D, typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int PER = D / 64;
  typedef float fv __attribute__((ext_vector_type(PER)));
  typedef T tv __attribute__((ext_vector_type(PER)));
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.npairs) return;
  float mx = -__builtin_inff();
  for (int s = lane; s < a.nsplit; s += 64) mx = __builtin_fmaxf(mx, a.lpart[(int64_t)s * a.npairs + pair]);
  mx = wave_max(mx);
  const bool ok = mx > -__builtin_inff();  // some range saw a key
  float sum = 0.f;
  if (ok)
    for (int s = lane; s < a.nsplit; s += 64)
      sum += exp2_fast((a.lpart[(int64_t)s * a.npairs + pair] - mx) * kLog2e);  // -inf -> 0
  sum = wave_sum(sum);  // >= 1: the maximal range contributes e^0
  const float lse = ok ? mx + __builtin_amdgcn_logf(sum) * kLn2 : -__builtin_inff();
  fv acc = {};
  if (ok) {
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t sp = (int64_t)s * a.npairs + pair;
      const float w = exp2_fast((a.lpart[sp] - lse) * kLog2e);
      if (w == 0.f) continue;  // empty range (uniform over the wave)
      acc += w * *(const fv*)(a.opart + sp * D + PER * lane);
    }
  }
  *(tv*)((T*)a.o + (int64_t)pair * D + PER * lane) = __builtin_convertvector(acc, tv);
  if (lane == 0) {
    const int row = pair / a.Hq, h = pair - row * a.Hq;
    const int64_t li = a.varlen ? (int64_t)h * a.total_q + row
                                : ((int64_t)(row / a.Nq) * a.Hq + h) * a.Nq + row % a.Nq;
    a.lse[li] = lse;
  }
}

template <int D, int KB, int NW, bool CAUSAL, typename T>
int launch(const FwdArgs& f, hipStream_t st) {
  constexpr int BM = 32 * NW;
  KernelArgs a;
  a.q = f.q; a.k = f.k; a.v = f.v; a.o = f.o; a.lse = f.lse;
  a.opart = f.opart; a.lpart = f.lpart;
  a.cu_q = f.cu_q; a.cu_k = f.cu_k;
  a.Hq = f.H; a.Hkv = f.Hkv; a.g = f.H / f.Hkv;
  a.Nq = f.N; a.Nk = f.Nk;
  a.total_q = f.total_q; a.total_k = f.total_k;
  a.pack = (f.pack && a.g > 1) ? 1 : 0;
  a.hu = a.pack ? f.Hkv : f.H;
  const int rows = a.pack ? f.N * a.g : f.N;
  a.n_mblk = (rows + BM - 1) / BM;
  // O is written once and not read again by this launch. For long
  // sequences the non-temporal hint keeps it from displacing, in L2, the K/V
  // tiles that a head's query blocks share (L2 fetches at d = 128, N = 8192:
  // 1.29x -> 1.18x the Q/K/V bytes, same speed); for short ones the plain
  // store measured as fast or faster, with cold inputs in particular.
  a.o_nt = f.N >= 2048 ? 1 : 0;
  a.nunit = f.B * a.hu;
  a.nsplit = f.nsplit > 1 ? f.nsplit : 1;
  a.split_len = f.nsplit > 1 ? f.split_len : 0x7fffffff;
  a.win_l = f.win_l;
  a.win_r = f.win_r;
  a.c = f.scale_log2;
  a.fd_mblk = make_fastdiv(a.n_mblk);
  a.fd_bh = make_fastdiv(a.nunit * a.nsplit);
  a.fd_split = make_fastdiv(a.nsplit);
  a.fd_hu = make_fastdiv(a.hu);
  a.fd_g = make_fastdiv(a.g);
  const int grid = a.n_mblk * a.nunit * a.nsplit;
  hipLaunchKernelGGL((fwd_kernel<D, KB, NW, CAUSAL, T>), dim3(grid), dim3(64 * NW), 0, st, a);
  return (int)hipGetLastError();
}

template <int D, typename T>
int launch_combine(const FwdArgs& f, hipStream_t st) {
  CombineArgs cb;
  cb.opart = f.opart; cb.lpart = f.lpart; cb.o = f.o; cb.lse = f.lse;
  cb.npairs = f.total_q * f.H;
  cb.nsplit = f.nsplit;
  cb.Hq = f.H; cb.Nq = f.N; cb.total_q = f.total_q;
  cb.varlen = f.cu_q != nullptr;
  hipLaunchKernelGGL((combine_kernel<D, T>), dim3((cb.npairs + 3) / 4), dim3(256), 0, st, cb);
  return (int)hipGetLastError();
}

// KV tile size per head dimension, in 32-key blocks.
#ifndef ATTN_D64_KB
#define ATTN_D64_KB 1
#endif
#ifndef ATTN_D128_KB
#define ATTN_D128_KB 1
#endif
#ifndef ATTN_D256_KB
#define ATTN_D256_KB 1
#endif
// Waves per workgroup (32 query rows each), non-causal and causal grids.
#ifndef ATTN_D64_NW
#define ATTN_D64_NW 4
#endif
#ifndef ATTN_D128_NW
#define ATTN_D128_NW 4
#endif
#ifndef ATTN_D64_NW_CAUSAL
#define ATTN_D64_NW_CAUSAL 4
#endif
#ifndef ATTN_D128_NW_CAUSAL
#define ATTN_D128_NW_CAUSAL 4
#endif

template <int D, typename T>
int dispatch_d(const FwdArgs& f, hipStream_t st) {
  constexpr int KB = D == 64 ? ATTN_D64_KB : D == 128 ? ATTN_D128_KB : ATTN_D256_KB;
  // one wave per SIMD at d = 256: a workgroup has at most 4 waves
  constexpr int NW = D == 64 ? ATTN_D64_NW : D == 128 ? ATTN_D128_NW : 4;
  constexpr int NWC = D == 64 ? ATTN_D64_NW_CAUSAL : D == 128 ? ATTN_D128_NW_CAUSAL : 4;
  return f.causal ? launch<D, KB, NWC, true, T>(f, st) : launch<D, KB, NW, false, T>(f, st);
}

template <typename T>
int dispatch(const FwdArgs& f, hipStream_t st, bool combine) {
  switch (f.d) {
    case 64: return combine ? launch_combine<64, T>(f, st) : dispatch_d<64, T>(f, st);
    case 128: return combine ? launch_combine<128, T>(f, st) : dispatch_d<128, T>(f, st);
    case 256: return combine ? launch_combine<256, T>(f, st) : dispatch_d<256, T>(f, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace fwd16

// Sequences with at most kDecodeRows query rows per key/value head (query
// rows times g) and d <= 128 go to the decode kernel, the others to the
// tiled kernel; with several key ranges the combine kernel follows either.
int launch_fwd_16(const FwdArgs& f, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool bf = f.dtype == 0;
  int err;
  if (uses_decode_kernel(f.N, f.H, f.Hkv, f.d))
    err = launch_decode_16(f, stream);
  else
    err = bf ? fwd16::dispatch<__bf16>(f, st, false) : fwd16::dispatch<_Float16>(f, st, false);
  if (err || f.nsplit <= 1) return err;
  return bf ? fwd16::dispatch<__bf16>(f, st, true) : fwd16::dispatch<_Float16>(f, st, true);
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace attn
