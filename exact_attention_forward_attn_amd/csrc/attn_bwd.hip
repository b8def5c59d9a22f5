// Exact attention backward for 16-bit inputs on gfx950 (MI355X).
//
// What is computed ("FlashAttention-3 on Hopper", chapter 7, section 7.1):
// for S = alpha Q K^T, P = softmax(S), O = P V and an upstream gradient dO,
//   D_i = rowsum(dO_i o O_i)                   (section 7.1.2)
//   P   = 2^(S log2(e) - LSE_i log2(e))        (section 7.1.3: no running max)
//   dV  = P^T dO,   dP = dO V^T,   dS = P o (dP - D)
//   dQ  = alpha dS K,   dK = alpha dS^T Q      (alpha applied once, at the end,
//                                               section 7.1.5)
//
// Three kernels:
// * pre_kernel: D (HBM-bound, one 16-byte load per operand and lane).
// * dkdv_kernel: KV-parallel (section 7.2): a workgroup owns 128 keys (32 per
//   wave) of one head and loops over 32-query tiles of Q and dO staged in
//   LDS; dK^T and dV^T stay in registers. With the wave's keys as the B
//   operand, S = Q K^T and dP = dO V^T come out with a lane owning one key
//   column, so the converted P and dS registers are directly the B operands
//   of dV^T += dO^T P and dK^T += Q^T dS, whose A operands come from the Q and
//   dO tiles through the transposing LDS read (the contraction runs over the
//   queries in the accumulator's row order, as the forward's P V does over
//   keys).
// * dq_kernel: query-parallel, the forward's structure without the online
//   softmax: S^T = K Q^T and dP^T = V dO^T with a lane owning one query, then
//   dQ^T += K^T dS^T. This is the pages' "second kernel that recomputes the
//   intermediates" option for the dQ reduction (section 7.2.3): it costs two
//   extra products per tile but needs no atomics or fp32 dQ buffer and is
//   deterministic.
// Causal masking follows section 7.2.2: a key block only meets query rows at
// or below its first key, so the query loop of dkdv_kernel starts there.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kernel_common.h"

namespace attn {
namespace bwd16 {

using namespace attn::dev;

[[maybe_unused]] constexpr float kLog2e = 1.4426950408889634f;  // device code only

// ---- D = rowsum(dO o O) ------------------------------------------------------
// rows in memory order r = row*H + h with row = b*N + n (dense) or the packed
// row (varlen); D_i is stored like LSE: delta[(b*H + h)*N + n], or
// delta[h*total + row] for packed batches (total > 0)
template <int D, typename T>
__global__ __launch_bounds__(256) void pre_kernel(const T* o, const T* dout, float* delta, int B, int H, int N,
                                                  int total) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int LPR = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;   // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int li = threadIdx.x % LPR;
  const int64_t nrows = total > 0 ? (int64_t)total * H : (int64_t)B * N * H;
  float acc = 0.f;
  if (row < nrows) {
    typedef T t8 __attribute__((ext_vector_type(8)));
    const t8 x = __builtin_bit_cast(t8, *(const u32x4*)(o + row * D + 8 * li));
    const t8 y = __builtin_bit_cast(t8, *(const u32x4*)(dout + row * D + 8 * li));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && li == 0) {
    const int64_t h = row % H, bn = row / H;
    if (total > 0) {
      delta[h * total + bn] = acc;
    } else {
      const int64_t n = bn % N, b = bn / N;
      delta[(b * H + h) * N + n] = acc;
    }
  }
#endif
}

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, g;  // query heads, key/value heads, g = Hq / Hkv
  int Nq, Nk;         // query and key rows per batch entry
  int n_kblk;         // ceil(Nk / 128): dK/dV workgroups per (b, KV head)
  int n_qblk;         // ceil(Nq / 128): dQ workgroups per (b, query head)
  const int* cu_q;    // packed batches: row offsets (Nq, Nk are then maxima)
  const int* cu_k;
  int total_q, total_k;
  int win_l, win_r;   // masked kernels: query n sees key j iff
                      // n + off - win_l <= j <= n + off + win_r
  float c;            // alpha * log2(e)
  float alpha;
};

// Rows of batch entry b in q/o and k/v: dense strides or clamped packed
// offsets (malformed offsets never address outside the tensors).
__device__ __forceinline__ void seq_extent(const KernelArgs& a, int b, int& q_row0, int& len_q, int& k_row0,
                                           int& len_k) {
  if (a.cu_q) {
    q_row0 = min(max(a.cu_q[b], 0), a.total_q);
    len_q = min(min(max(a.cu_q[b + 1], q_row0), a.total_q) - q_row0, a.Nq);
    k_row0 = min(max(a.cu_k[b], 0), a.total_k);
    len_k = min(min(max(a.cu_k[b + 1], k_row0), a.total_k) - k_row0, a.Nk);
  } else {
    q_row0 = b * a.Nq; len_q = a.Nq;
    k_row0 = b * a.Nk; len_k = a.Nk;
  }
}

// LDS reads in flight ahead of the MFMAs of the pipelined dK/dV step
#ifndef ATTN_BWD_RING
#define ATTN_BWD_RING 4
#endif

// waves per SIMD each kernel is compiled for (its register budget): dK/dV
// keeps K, V, dK^T and dV^T in registers. At d = 64 both kernels fit three
// waves (168 VGPRs each) without spilling.
template <int D>
constexpr int kWavesDkdv = D == 64 ? 3 : 1;
// dK/dV kernels that run the software-pipelined loop (those at one wave per
// SIMD, which have the registers for a second tile's S and dP)
template <int D>
constexpr bool kPipeDkdv = D == 128;
template <int D>
constexpr int kWavesDq = D == 256 ? 1 : D == 128 ? 2 : 3;

// XOR swizzle of the 16-byte chunk index of row r of a backward tile. The
// tiles are read two ways. Row-wise (ds_read_b128, the A operand of S or
// dP), 16 lanes read 16 consecutive rows at one logical chunk, so those rows
// must land on 16 different 16-byte bank groups. Transposed
// (ds_read_b64_tr_b16, the A operand of dV, dK or dQ), 32 lanes read 4
// consecutive rows (4h..4h+3) of an aligned 4-chunk quad, so the 4 rows must
// land in different quads of the 256-byte bank line. A plain r & 15 XOR only
// permutes chunks inside a quad, which put all 4 rows of a transposed read
// on the same banks. At d >= 128 (a row spans whole lines) the low two row
// bits move the quad and the next two bits permute inside it. At d = 64 two
// rows share a line, so the row parity already separates them; row bit 1
// moves the quad and row bits 2-3 permute inside it. Both are bijections
// over 16 consecutive rows and have period 16, which the copy offsets assume.
template <int D>
__device__ __forceinline__ int swz_b(int r) {
  return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// Per-lane LDS offsets shared by both kernels for 32-row tiles stored with the
// swz_b swizzle (they are read row-wise as MFMA A operands and, for the
// transposed operands, through ds_read_b64_tr_b16).
template <int D, bool SWB = true>
struct TileOffsets {
  typedef Geo<D, 1> G;
  static __device__ __forceinline__ int swz(int r) { return SWB ? swz_b<D>(r) : swz_k<D>(r); }
  static constexpr int KC = D / 16;
  static constexpr int KCL = KC < 8 ? KC : 8;
  static constexpr int DB = D / 32;
  static constexpr int DBL = DB < 4 ? DB : 4;
  static constexpr int KGP = (G::RPS * 4) % 16 == 0 ? 1 : 2;
  uint32_t cg[KGP];     // global -> LDS copy: per-lane byte offset of segment t
  int rofs[KCL];        // row reads: row l32, logical chunk 2kc + h32
  int tlo[DBL], thi[DBL];  // transposing reads: rows r0 and r0 + 8
  __device__ __forceinline__ void init(int lane, int wave, uint32_t RS) {
    const int h32 = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int t = 0; t < KGP; ++t) {
      const int r = (wave + 4 * t) * G::RPS + lane / G::CPR;
      const int pc = lane % G::CPR;
      cg[t] = (uint32_t)r * RS + (uint32_t)((pc ^ swz(r)) << 4) - (uint32_t)t * 4 * G::RPS * RS;
    }
#pragma unroll
    for (int i = 0; i < KCL; ++i) rofs[i] = l32 * G::ROWB + (((2 * i + h32) ^ swz(l32)) << 4);
    // 16-lane group g = lane/16, piece p = lane%16: row 4*h32 + p/4 (+8 for the
    // second read), dims db*32 + 16*(g%2) + 4*(p%4)
    const int p = lane & 15, dh = (lane >> 4) & 1;
    const int r0 = 4 * h32 + (p >> 2);
#pragma unroll
    for (int i = 0; i < DBL; ++i) {
      const int ch = 4 * i + 2 * dh + ((p & 3) >> 1);
      tlo[i] = r0 * G::ROWB + ((ch ^ swz(r0)) << 4) + 8 * (p & 1);
      thi[i] = (r0 + 8) * G::ROWB + ((ch ^ swz(r0 + 8)) << 4) + 8 * (p & 1);
    }
  }
};

// Copy 32 rows starting at row0 of one head into an LDS tile (swz_b
// swizzle); extra is a byte offset added to every row (the head within a
// group of heads that share the buffer resource).
template <int D, bool SWB>
__device__ __forceinline__ void copy_tile(const TileOffsets<D, SWB>& to, const __amdgpu_buffer_rsrc_t& rs, char* dst,
                                          int wave, int row0, uint32_t RS, uint32_t extra = 0) {
  typedef Geo<D, 1> G;
  const uint32_t base = (uint32_t)row0 * RS + extra;
#pragma unroll
  for (int t = 0; t < G::SEG_PER_WAVE; ++t) {
    const uint32_t voff = to.cg[(t & 1) % TileOffsets<D, SWB>::KGP] + (base + (uint32_t)t * 4 * G::RPS * RS);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (wave + 4 * t) * 1024), 16, voff, 0, 0, 0);
  }
}

// A operand of row-read tile rows (32 rows x 16 dims, step kc)
template <int D, typename T, bool SWB>
__device__ __forceinline__ typename Elt<T>::v8 row_op(const TileOffsets<D, SWB>& to, const char* tile, int kc) {
  return *(const typename Elt<T>::v8*)(tile + (kc / 8) * 256 + to.rofs[kc % 8]);
}
// A operand of the transposed tile: 32 dims (block db) x 16 rows (chunk ks)
template <int D, typename T, bool SWB>
__device__ __forceinline__ typename Elt<T>::v8 tr_op(const TileOffsets<D, SWB>& to, const char* tile, int db, int ks) {
  typedef Elt<T> E;
  const LDS_AS char* base = (const LDS_AS char*)tile + 16 * ks * Geo<D, 1>::ROWB + (db / 4) * 256;
  const typename E::v4 lo = E::tr_read(base + to.tlo[db % 4]);
  const typename E::v4 hi = E::tr_read(base + to.thi[db % 4]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void barrier_all() {
  wait_lgkmcnt0();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// B operand registers of a row of one head: dims 16kc + 8*h32 .. +7
template <int D, typename T>
__device__ __forceinline__ void load_row_operand(const __amdgpu_buffer_rsrc_t& rs, uint32_t row, uint32_t RS, int h32,
                                                 typename Elt<T>::v8 (&reg)[D / 16]) {
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rs, row * RS + (16 * kc + 8 * h32) * 2, 0, 0);
    reg[kc] = __builtin_bit_cast(typename Elt<T>::v8, raw);
  }
}

// Store an accumulator of dims x rows (lane = row l32) as row `row` of one
// head, scaled by f.
template <int D, typename T>
__device__ __forceinline__ void store_rows(T* head, int row, uint32_t RS_elems, int h32, const f32x16 (&acc)[D / 32],
                                           float f) {
  T* rp = head + (int64_t)row * RS_elems;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef T t4 __attribute__((ext_vector_type(4)));
      float __attribute__((ext_vector_type(4))) x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g + e] * f;
      t4 ov = __builtin_convertvector(x, t4);
      *(u32x2*)(rp + db * 32 + 8 * g + 4 * h32) = __builtin_bit_cast(u32x2, ov);
    }
}

// Two 16-bit B operands (rows 0-7 and 8-15 of the accumulator) from 16 floats.
template <typename T>
__device__ __forceinline__ void pack16(const float (&x)[16], typename Elt<T>::v8 (&out)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = x[8 * ks + e];
    out[ks] = __builtin_convertvector(f, typename Elt<T>::v8);
  }
}

// ---- dK, dV: KV-parallel ---------------------------------------------------------
// PARTS selects the outputs: 3 = dK and dV in one pass; at d = 256 their
// accumulators, K and V do not fit one wave's registers, so the kernel runs
// twice, 1 = dV (needs K for S), then 2 = dK (needs K and V), recomputing S.
template <int D, bool CAUSAL, typename T, int PARTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesDkdv<D>, kWavesDkdv<D>)))
void dkdv_kernel(KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool DO_K = (PARTS & 2) != 0;
  constexpr bool DO_V = (PARTS & 1) != 0;
  constexpr bool PIPE = kPipeDkdv<D> && PARTS == 3;
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef Geo<D, 1> G;
  typedef TileOffsets<D> TO;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;

  __shared__ __attribute__((aligned(1024))) char qbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char qbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char qbuf2[PIPE ? G::TILE : 16];
  __shared__ __attribute__((aligned(1024))) char obuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char obuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char obuf2[PIPE ? G::TILE : 16];
  // LSE (floats 0..63) and D (64..127) of each slot's 32 query rows, copied
  // by DMA with the tile (rows r and r + 32 hold the same value); every lane
  // of a half-wave reads the same 16 rows back
  __shared__ __attribute__((aligned(16))) float rows0[128];
  __shared__ __attribute__((aligned(16))) float rows1[128];
  __shared__ __attribute__((aligned(16))) float rows2[PIPE ? 128 : 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;

  // key blocks of one key/value head: causal grids go from the first block
  // (the longest query range) to the last. With grouped heads the g query
  // heads that read this key/value head all contribute to its dK and dV
  // ("FlashAttention-3 on Hopper", section 8.8); the workgroup loops over
  // their query tiles itself, so the sum needs no atomics.
  const int BH = a.B * a.Hkv;
  int kblk, bh;
  decode_block(blockIdx.x, a.n_kblk, BH, CAUSAL, kblk, bh);
  if (CAUSAL) kblk = a.n_kblk - 1 - kblk;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int grp = a.g;
  int q_row0, Nq, k_row0, Nk;             // this batch entry's rows and lengths
  seq_extent(a, b, q_row0, Nq, k_row0, Nk);
  const int k0 = kblk * 128;
  if (k0 >= Nk) return;                   // past a short key sequence (uniform)
  const int off = Nk - Nq;                // causal offset (bottom-right)
  const int key = k0 + 32 * wave + l32;   // this lane's key (column of S)
  const uint32_t RSQ = (uint32_t)a.Hq * D * 2, RSK = (uint32_t)a.Hkv * D * 2;
  const int64_t k_off = ((int64_t)k_row0 * a.Hkv + hk) * D;
  const int64_t q_off = ((int64_t)q_row0 * a.Hq + (int64_t)hk * grp) * D;  // first head of the group
  const uint32_t kspan = (uint32_t)(Nk - 1) * RSK + D * 2;
  const uint32_t qspan = Nq > 0 ? (uint32_t)(Nq - 1) * RSQ + (uint32_t)grp * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const T*)a.q + q_off, qspan);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T*)a.k + k_off, kspan);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T*)a.v + k_off, kspan);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((const T*)a.dout + q_off, qspan);
  // LSE and D of the group's heads, head j at l_off + j * l_hs: [B, Hq, Nq]
  // for dense inputs, [Hq, total_q] for packed batches
  const int64_t l_off = a.cu_q ? (int64_t)hk * grp * a.total_q + q_row0 : ((int64_t)b * a.Hq + (int64_t)hk * grp) * a.Nq;
  const uint32_t l_hs = a.cu_q ? (uint32_t)a.total_q : (uint32_t)a.Nq;
  const uint32_t lspan = Nq > 0 ? ((uint32_t)(grp - 1) * l_hs + (uint32_t)Nq) * 4 : 0;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + l_off, lspan);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.delta + l_off, lspan);

  v8 kreg[KC], vreg[DO_K ? KC : 1];
  load_row_operand<D, T>(rk, (uint32_t)key, RSK, h32, kreg);
  if constexpr (DO_K) load_row_operand<D, T>(rv, (uint32_t)key, RSK, h32, vreg);
  TO to;
  to.init(lane, wave, RSQ);

  f32x16 dkt[DO_K ? DB : 1], dvt[DO_V ? DB : 1];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    if constexpr (DO_K) dkt[db] = f32x16{};
    if constexpr (DO_V) dvt[db] = f32x16{};
  }
  const float c = a.c;

  // query tiles of one head: in the masked instantiation query n sees key k
  // iff n + off - win_l <= k <= n + off + win_r, so only the tiles of rows
  // k0 - off - win_r .. k0 + 127 - off + win_l meet these keys; the loop runs
  // over (head of the group, tile) pairs u = j * nt_h + (t - t0)
  const int nqt = (Nq + 31) / 32;
  int t0 = 0, t1 = nqt;
  if (CAUSAL) {
    t0 = min(nqt, max(0, k0 - off - a.win_r) / 32);
    const int hi = k0 + 127 - off + a.win_l;
    t1 = hi < 0 ? 0 : min(nqt, hi / 32 + 1);
  }
  const int nt_h = max(0, t1 - t0);
  const int nu = grp * nt_h;
  auto tile_of = [&](int u, int& q0t, int& j) ATTN_INLINE {
    j = u / nt_h;
    q0t = 32 * (t0 + u - j * nt_h);
  };

  // Band test of score r of a lane (row q0t + 4*h32 + 8*(r>>2) + (r&3), the
  // lane's key): the row sees the key iff 0 <= key - row - off + win_l <=
  // win_l + win_r, one unsigned compare against a per-tile base. Rows past
  // Nq need no test: their Q and dO rows read as zero (and LSE, D as 0), so
  // p = 1 and dS = 0 add nothing; keys past Nk only reach their own dK/dV
  // rows, which are not stored. Nor do rows with LSE = -inf: such a row sees
  // no key, so the band test is false for every key of a masked call, and
  // an unmasked call with keys has no such row.
  const uint32_t wspan = (uint32_t)(a.win_l + a.win_r);
  auto band_base = [&](int q0t) ATTN_INLINE { return key - q0t - 4 * h32 - off + a.win_l; };
  auto in_band = [&](int kb, int r) ATTN_INLINE {
    return (uint32_t)(kb - (8 * (r >> 2) + (r & 3))) <= wspan;
  };

  auto compute = [&](const char* qt, const char* ot, int q0t, const f32x4 (&l2)[4], const f32x4 (&dl)[4]) ATTN_INLINE {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) s = E::mfma(row_op<D, T>(to, qt, kc), kreg[kc], s);
    if constexpr (DO_K) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) dp = E::mfma(row_op<D, T>(to, ot, kc), vreg[kc], dp);
    }
    float pv[16], dsv[16];
    const int kb = band_base(q0t);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = !CAUSAL || in_band(kb, r);
      const float lse = l2[r >> 2][r & 3];
      const float p = ok ? exp2_fast(__builtin_fmaf(s[r], c, -lse * kLog2e)) : 0.f;
      pv[r] = p;
      if constexpr (DO_K) dsv[r] = p * (dp[r] - dl[r >> 2][r & 3]);
    }
    v8 pk[2], dk8[2];
    if constexpr (DO_V) pack16<T>(pv, pk);
    if constexpr (DO_K) pack16<T>(dsv, dk8);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (DO_V) dvt[db] = E::mfma(tr_op<D, T>(to, ot, db, ks), pk[ks], dvt[db]);
        if constexpr (DO_K) dkt[db] = E::mfma(tr_op<D, T>(to, qt, db, ks), dk8[ks], dkt[db]);
      }
  };

  // copy tile u (Q and dO rows of its head, and their LSE and D) into a slot;
  // rows past Nq read as 0 (harmless: their Q and dO rows are zero too)
  auto copy_u = [&](int u, char* qd, char* od, float* rd_) ATTN_INLINE {
    int q0t, j;
    tile_of(u, q0t, j);
    copy_tile<D>(to, rq, qd, wave, q0t, RSQ, (uint32_t)j * D * 2);
    copy_tile<D>(to, ro, od, wave, q0t, RSQ, (uint32_t)j * D * 2);
    const int row = q0t + l32;
    const uint32_t lo = row < Nq ? ((uint32_t)j * l_hs + (uint32_t)row) * 4 : 0xffffffffu;
    if (wave == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LDS_AS void*)rd_, 4, lo, 0, 0, 0);
    if (wave == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (LDS_AS void*)(rd_ + 64), 4, lo, 0, 0, 0);
  };
  // LSE and D of rows 8g + 4*h32 + 0..3 of the tile in a slot
  auto read_rows = [&](const float* rw, f32x4 (&l2)[4], f32x4 (&dl)[4]) ATTN_INLINE {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l2[g] = *(const f32x4*)(rw + 8 * g + 4 * h32);
      dl[g] = *(const f32x4*)(rw + 64 + 8 * g + 4 * h32);
    }
  };

  if constexpr (!PIPE) {
    if (nu > 0) {
      copy_u(0, qbuf0, obuf0, rows0);
      wait_vmcnt<0>();
      barrier_all();
    }
    // slot of tile u is u % 2; the loop is unrolled by two so that both
    // slots are compile-time objects
    auto step = [&](int u, auto j_tag) ATTN_INLINE {
      constexpr int J = decltype(j_tag)::value;
      char* qcur = J ? qbuf1 : qbuf0;
      char* ocur = J ? obuf1 : obuf0;
      char* qnxt = J ? qbuf0 : qbuf1;
      char* onxt = J ? obuf0 : obuf1;
      if (u + 1 < nu) copy_u(u + 1, qnxt, onxt, J ? rows0 : rows1);
      f32x4 l2c[4], dlc[4];
      read_rows(J ? rows1 : rows0, l2c, dlc);
      int q0t, j;
      tile_of(u, q0t, j);
      compute(qcur, ocur, q0t, l2c, dlc);
      wait_vmcnt<0>();
      barrier_all();
    };
    int u = 0;
    for (; u + 1 < nu; u += 2) {
      step(u, Int<0>{});
      step(u + 1, Int<1>{});
    }
    if (u < nu) step(u, Int<0>{});
  } else {
    // Software pipeline (one wave per SIMD, so no other wave fills the
    // gaps): step u runs the S and dP products of tile u+1 interleaved with
    // the VALU work of tile u (p and dS), then the dV and dK products of tile
    // u. Q/dO tiles rotate through three LDS slots: step u reads tiles u
    // (transposed) and u+1 (rows) while tile u+2 is copied in.
    f32x16 sc = f32x16{}, dpc = f32x16{};
    auto slot_r = [&](auto j) ATTN_INLINE -> float* {
      constexpr int J = decltype(j)::value % 3;
      return J == 0 ? rows0 : J == 1 ? rows1 : rows2;
    };
    auto slot_q = [&](auto j) ATTN_INLINE -> char* {
      constexpr int J = decltype(j)::value % 3;
      return J == 0 ? qbuf0 : J == 1 ? qbuf1 : qbuf2;
    };
    auto slot_o = [&](auto j) ATTN_INLINE -> char* {
      constexpr int J = decltype(j)::value % 3;
      return J == 0 ? obuf0 : J == 1 ? obuf1 : obuf2;
    };
    if (nu > 0) {
      copy_u(0, qbuf0, obuf0, rows0);
      if (nu > 1) copy_u(1, qbuf1, obuf1, rows1);
      wait_vmcnt<0>();
      barrier_all();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) sc = E::mfma(row_op<D, T>(to, qbuf0, kc), kreg[kc], sc);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) dpc = E::mfma(row_op<D, T>(to, obuf0, kc), vreg[kc], dpc);
    }
    constexpr int NM = 2 * KC;  // S and dP MFMAs of one tile
    auto pstep = [&](int u, auto j_tag, auto next_tag) ATTN_INLINE {
      constexpr int J = decltype(j_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;  // tile u+1 exists
      const char* qn = slot_q(Int<J + 1>{});
      const char* on = slot_o(Int<J + 1>{});
      if (u + 2 < nu) copy_u(u + 2, slot_q(Int<J + 2>{}), slot_o(Int<J + 2>{}), slot_r(Int<J + 2>{}));
      // LSE and D of this tile's rows, from its slot
      f32x4 l2c[4], dlc[4];
      read_rows(slot_r(Int<J>{}), l2c, dlc);
      f32x16 sn = f32x16{}, dpn = f32x16{};
      float pv[16], dsv[16], xv[16], dd[16];
      // -LSE log2(e) of the tile's rows (the exponent's addend)
      f32x4 nl[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) nl[g] = l2c[g] * -kLog2e;
      int q0t, jcur;
      tile_of(u, q0t, jcur);
      const int kb = band_base(q0t);
      // operand ring: the LDS read of MFMA m + RL is issued at step m
      constexpr int RL = ATTN_BWD_RING;
      v8 ring[RL];
      auto opnd = [&](auto m_tag) ATTN_INLINE -> v8 {
        constexpr int m = decltype(m_tag)::value;
        return m < KC ? row_op<D, T>(to, qn, m) : row_op<D, T>(to, on, m - KC);
      };
      if constexpr (NEXT) For<0, (RL < NM ? RL : NM)>::run([&](auto m) ATTN_INLINE { ring[decltype(m)::value] = opnd(m); });
      For<0, NM>::run([&](auto m_tag) ATTN_INLINE {
        constexpr int m = decltype(m_tag)::value;
        if constexpr (NEXT) {
          if constexpr (m < KC)
            sn = E::mfma(ring[m % RL], kreg[m], sn);
          else
            dpn = E::mfma(ring[m % RL], vreg[m - KC], dpn);
          if constexpr (m + RL < NM) ring[m % RL] = opnd(Int<m + RL>{});
        }
        // p and dS of score r, skewed over three steps so that no VALU
        // instruction waits on the one before it: the exponent and dP - D
        // at step f(r), the exp at f(r) + 1, the mask and dS at f(r) + 2
        For<0, 16>::run([&](auto r_tag) ATTN_INLINE {
          constexpr int r = decltype(r_tag)::value;
          constexpr int f = (r * (NM - 2)) / 16;
          if constexpr (f == m) {
            xv[r] = __builtin_fmaf(sc[r], c, nl[r >> 2][r & 3]);
            pin(xv[r]);
            dd[r] = dpc[r] - dlc[r >> 2][r & 3];
            pin(dd[r]);
          }
          if constexpr (f + 1 == m) {
            xv[r] = exp2_fast(xv[r]);
            pin(xv[r]);
          }
          if constexpr (f + 2 == m) {
            // unmasked: the LSE = -inf select never fires (no row is without
            // keys), but without it the register allocation of this
            // instantiation spills
            const bool ok = CAUSAL ? in_band(kb, r) : l2c[r >> 2][r & 3] != -__builtin_inff();
            const float p = ok ? xv[r] : 0.f;
            pv[r] = p;
            dsv[r] = p * dd[r];
            pin(dsv[r]);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      // dV^T and dK^T products of tile u, alternating (each accumulator is
      // reused every other MFMA); their transposed operands come through a
      // ring of R2 reads issued ahead, the first ones before P and dS are
      // packed
      const char* qc = slot_q(Int<J>{});
      const char* oc = slot_o(Int<J>{});
      constexpr int R2 = ATTN_BWD_RING;
      constexpr int NM2 = 4 * DB;
      auto opnd2 = [&](auto m_tag) ATTN_INLINE -> v8 {
        constexpr int m = decltype(m_tag)::value;
        return tr_op<D, T>(to, (m & 1) ? qc : oc, m / 4, (m / 2) % 2);
      };
      v8 ring2[R2];
      For<0, (R2 < NM2 ? R2 : NM2)>::run([&](auto m) ATTN_INLINE { ring2[decltype(m)::value] = opnd2(m); });
      v8 pk[2], dk8[2];
      pack16<T>(pv, pk);
      pack16<T>(dsv, dk8);
      __builtin_amdgcn_sched_barrier(0);
      For<0, NM2>::run([&](auto m_tag) ATTN_INLINE {
        constexpr int m = decltype(m_tag)::value;
        constexpr int db = m / 4, ks = (m / 2) % 2;
        if constexpr (m & 1)
          dkt[db] = E::mfma(ring2[m % R2], dk8[ks], dkt[db]);
        else
          dvt[db] = E::mfma(ring2[m % R2], pk[ks], dvt[db]);
        if constexpr (m + R2 < NM2) ring2[m % R2] = opnd2(Int<m + R2>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      wait_vmcnt<0>();
      barrier_all();
      sc = sn;
      dpc = dpn;
    };
    // unrolled by three so every slot is a compile-time object
    int u = 0;
    for (; u + 3 < nu; u += 3) {
      pstep(u, Int<0>{}, TrueT{});
      pstep(u + 1, Int<1>{}, TrueT{});
      pstep(u + 2, Int<2>{}, TrueT{});
    }
    // 0 to 3 tiles left (the last one without a next tile)
    if (u + 2 < nu) {
      pstep(u, Int<0>{}, TrueT{});
      pstep(u + 1, Int<1>{}, TrueT{});
      pstep(u + 2, Int<2>{}, FalseT{});
    } else if (u + 1 < nu) {
      pstep(u, Int<0>{}, TrueT{});
      pstep(u + 1, Int<1>{}, FalseT{});
    } else if (u < nu) {
      pstep(u, Int<0>{}, FalseT{});
    }
  }

  if (key < Nk) {
    if constexpr (DO_K) store_rows<D, T>((T*)a.dk + k_off, key, (uint32_t)a.Hkv * D, h32, dkt, a.alpha);
    if constexpr (DO_V) store_rows<D, T>((T*)a.dv + k_off, key, (uint32_t)a.Hkv * D, h32, dvt, 1.0f);
  }
#endif
}

// ---- dQ: query-parallel ----------------------------------------------------------
template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesDq<D>, kWavesDq<D>)))
void dq_kernel(KernelArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef Geo<D, 1> G;
  typedef TileOffsets<D> TO;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;

  __shared__ __attribute__((aligned(1024))) char kbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[G::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;

  const int BH = a.B * a.Hq;
  int mblk, bh;
  decode_block(blockIdx.x, a.n_qblk, BH, CAUSAL, mblk, bh);
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int hk = hq / a.g;                // the key/value head this head reads
  int q_row0, Nq, k_row0, Nk;             // this batch entry's rows and lengths
  seq_extent(a, b, q_row0, Nq, k_row0, Nk);
  const int q0 = mblk * 128;
  if (q0 >= Nq) return;                   // past a short query sequence (uniform)
  const int off = Nk - Nq;                // causal offset (bottom-right)
  const int qi = q0 + 32 * wave + l32;    // this lane's query (column of S^T)
  const uint32_t RSQ = (uint32_t)a.Hq * D * 2, RSK = (uint32_t)a.Hkv * D * 2;
  const int64_t q_off = ((int64_t)q_row0 * a.Hq + hq) * D;
  const int64_t k_off = ((int64_t)k_row0 * a.Hkv + hk) * D;
  const uint32_t qspan = (uint32_t)(Nq - 1) * RSQ + D * 2;
  const uint32_t kspan = Nk > 0 ? (uint32_t)(Nk - 1) * RSK + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const T*)a.q + q_off, qspan);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T*)a.k + k_off, kspan);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T*)a.v + k_off, kspan);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((const T*)a.dout + q_off, qspan);

  v8 qreg[KC], oreg[KC];
  load_row_operand<D, T>(rq, (uint32_t)qi, RSQ, h32, qreg);
  load_row_operand<D, T>(ro, (uint32_t)qi, RSQ, h32, oreg);
  TO to;
  to.init(lane, wave, RSK);
  const int64_t li = a.cu_q ? (int64_t)hq * a.total_q + q_row0 + qi : (int64_t)bh * a.Nq + qi;
  const float lse = qi < Nq ? a.lse[li] : -__builtin_inff();
  const float dl = qi < Nq ? a.delta[li] : 0.f;
  const bool live = lse != -__builtin_inff();
  // a row past Nq or with LSE = -inf gets l2 = +inf: p = 2^(s c - inf) = 0
  const float l2 = live ? lse * kLog2e : __builtin_inff();

  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = f32x16{};
  const float c = a.c;

  // keys some row of the block sees (masked: from q0 + off - win_l to
  // q0 + 127 + off + win_r), in tiles starting at tile tk0
  int kv_lo = 0, kv_end = Nk;
  if (CAUSAL) {
    kv_lo = min(Nk, max(0, q0 + off - a.win_l));
    kv_end = min(Nk, q0 + 128 + off + a.win_r);
  }
  const int tk0 = kv_lo / 32;
  const int nkt = kv_end > 32 * tk0 ? (kv_end - 32 * tk0 + 31) / 32 : 0;

  // MASK: the tile holds keys past Nk or outside some row's band; without
  // it every key of the tile is seen by every row of the wave
  auto compute = [&](const char* kt, const char* vt, int kv0, auto mask_tag) ATTN_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    // keys this lane's row sees, relative to the lane's first key of the tile
    // (kv0 + 4*h32); a row past Nq or with LSE = -inf sees none
    int lo = 0;
    uint32_t span = 0;
    if constexpr (MASK) {
      const int base = kv0 + 4 * h32;
      lo = CAUSAL ? qi + off - a.win_l - base : -base;
      const int hi = min(Nk - 1, CAUSAL ? qi + off + a.win_r : Nk) - base;
      span = (uint32_t)(hi - lo);
      if (!live || hi < lo) {
        lo = 1 << 30;
        span = 0;
      }
    }
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) s = E::mfma(row_op<D, T>(to, kt, kc), qreg[kc], s);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) dp = E::mfma(row_op<D, T>(to, vt, kc), oreg[kc], dp);
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // key kv0 + 4*h32 + cr, cr = 8*(r>>2) + (r&3), is seen iff cr - lo
      // lies in [0, span] (unsigned); the span also stops at Nk, since a
      // zero-filled key row past Nk could make p overflow
      const int cr = 8 * (r >> 2) + (r & 3);
      const bool ok = !MASK || (uint32_t)(cr - lo) <= span;
      const float p = ok ? exp2_fast(__builtin_fmaf(s[r], c, -l2)) : 0.f;
      dsv[r] = p * (dp[r] - dl);
    }
    v8 dk8[2];
    pack16<T>(dsv, dk8);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dqt[db] = E::mfma(tr_op<D, T>(to, kt, db, ks), dk8[ks], dqt[db]);
  };

  if (nkt > 0) {
    copy_tile<D>(to, rk, kbuf0, wave, 32 * tk0, RSK);
    copy_tile<D>(to, rv, vbuf0, wave, 32 * tk0, RSK);
    wait_vmcnt<0>();
    barrier_all();
  }
  auto step = [&](int t, auto j_tag) ATTN_INLINE {
    constexpr int J = decltype(j_tag)::value;
    char* kcur = J ? kbuf1 : kbuf0;
    char* vcur = J ? vbuf1 : vbuf0;
    char* knxt = J ? kbuf0 : kbuf1;
    char* vnxt = J ? vbuf0 : vbuf1;
    if (t + 1 < nkt) {
      copy_tile<D>(to, rk, knxt, wave, 32 * (tk0 + t + 1), RSK);
      copy_tile<D>(to, rv, vnxt, wave, 32 * (tk0 + t + 1), RSK);
    }
    const int kv0 = 32 * (tk0 + t);
    const int qw0 = q0 + 32 * wave;  // the wave's first query row
    const bool full = kv0 + 32 <= Nk && (!CAUSAL || (kv0 + 31 <= qw0 + off + a.win_r &&
                                                     kv0 >= qw0 + 31 + off - a.win_l));
    if (full)
      compute(kcur, vcur, kv0, FalseT{});
    else
      compute(kcur, vcur, kv0, TrueT{});
    wait_vmcnt<0>();
    barrier_all();
  };
  int t = 0;
  for (; t + 1 < nkt; t += 2) {
    step(t, Int<0>{});
    step(t + 1, Int<1>{});
  }
  if (t < nkt) step(t, Int<0>{});

  if (qi < Nq) store_rows<D, T>((T*)a.dq + q_off, qi, (uint32_t)a.Hq * D, h32, dqt, a.alpha);
#endif
}

template <int D, typename T>
int launch_d(const BwdArgs& f, hipStream_t st) {
  const int64_t qrows = (f.cu_q ? (int64_t)f.total_q : (int64_t)f.B * f.N) * f.H;
  if (qrows > 0) {
    constexpr int RPB = 256 / (D / 8);
    const int grid = (int)((qrows + RPB - 1) / RPB);
    hipLaunchKernelGGL((pre_kernel<D, T>), dim3(grid), dim3(256), 0, st, (const T*)f.o, (const T*)f.dout, f.delta,
                       f.B, f.H, f.N, f.cu_q ? f.total_q : 0);
  }
  KernelArgs a;
  a.q = f.q; a.k = f.k; a.v = f.v; a.dout = f.dout; a.lse = f.lse; a.delta = f.delta;
  a.dq = f.dq; a.dk = f.dk; a.dv = f.dv;
  a.B = f.B; a.Hq = f.H; a.Hkv = f.Hkv; a.g = f.H / f.Hkv;
  a.Nq = f.N; a.Nk = f.Nk;
  a.n_kblk = (f.Nk + 127) / 128;
  a.n_qblk = (f.N + 127) / 128;
  a.cu_q = f.cu_q; a.cu_k = f.cu_k;
  a.total_q = f.total_q; a.total_k = f.total_k;
  a.win_l = f.win_l; a.win_r = f.win_r;
  a.c = f.scale_log2;
  a.alpha = f.alpha;
  const int kgrid = a.n_kblk * f.B * f.Hkv;
  const int qgrid = a.n_qblk * f.B * f.H;
  if (f.causal) {
    if (kgrid > 0) {
      if constexpr (D == 256) {
        hipLaunchKernelGGL((dkdv_kernel<D, true, T, 1>), dim3(kgrid), dim3(256), 0, st, a);
        hipLaunchKernelGGL((dkdv_kernel<D, true, T, 2>), dim3(kgrid), dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((dkdv_kernel<D, true, T, 3>), dim3(kgrid), dim3(256), 0, st, a);
      }
    }
    if (qgrid > 0) hipLaunchKernelGGL((dq_kernel<D, true, T>), dim3(qgrid), dim3(256), 0, st, a);
  } else {
    if (kgrid > 0) {
      if constexpr (D == 256) {
        hipLaunchKernelGGL((dkdv_kernel<D, false, T, 1>), dim3(kgrid), dim3(256), 0, st, a);
        hipLaunchKernelGGL((dkdv_kernel<D, false, T, 2>), dim3(kgrid), dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((dkdv_kernel<D, false, T, 3>), dim3(kgrid), dim3(256), 0, st, a);
      }
    }
    if (qgrid > 0) hipLaunchKernelGGL((dq_kernel<D, false, T>), dim3(qgrid), dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

template <typename T>
int dispatch(const BwdArgs& f, hipStream_t st) {
  switch (f.d) {
    case 64: return launch_d<64, T>(f, st);
    case 128: return launch_d<128, T>(f, st);
    case 256: return launch_d<256, T>(f, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace bwd16

int launch_bwd_16(const BwdArgs& f, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return f.dtype == 0 ? bwd16::dispatch<__bf16>(f, st) : bwd16::dispatch<_Float16>(f, st);
}

}  // namespace attn
