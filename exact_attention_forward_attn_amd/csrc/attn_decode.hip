// Attention forward for few query rows per key/value head (decode), 16-bit
// inputs, gfx950.
//
// Same result as the main forward kernel (O = softmax(alpha Q K^T) V and
// LSE per row, "FlashAttention-3 on Hopper", sections 3.1-3.2, 4.6-4.7), for
// the case the pages single out as a different workload: one or a few query
// rows against a long key/value cache, where the query tiles cannot fill the
// machine and the run is bound by reading K and V once from HBM (the pages
// point to split-KV and the combine of per-range states for it: section
// 3.2.1 and chapter 10).
//
// gfx950 design
// -------------
// * A workgroup owns one key/value head of one sequence, one key range
//   (split), and all query rows that read that head: the g query heads of
//   the group times the sequence's query rows, at most 16 rows, packed
//   query-major / head-minor. Scores are S^T = K Q^T with the 16x16x32 MFMA
//   (a lane owns one query row and 4 keys of each 16-key block), and
//   O^T += V^T P^T with the same MFMA; P stays in the registers the scores
//   came from (the contraction over keys uses the accumulator's key order on
//   both operands).
// * Bytes in flight, not arithmetic, set the speed. Each wave streams its own
//   32-key tiles (tiles w, w + NW, w + 2 NW, ... of the range), two at a
//   time: K straight into registers (its MFMA operand layout is row-major,
//   16 bytes of one key per lane), V global -> LDS with buffer_load ... lds
//   into a private two-stage ring (the transposing LDS read gives V^T). The
//   loop has no workgroup barrier: a wave only waits for its own copies.
//   A workgroup of 4 waves takes 32 KiB (d = 64) or 64 KiB (d = 128) of LDS,
//   so two to four share a compute unit with up to 256 KiB of K and V in
//   flight. (At d = 256 two tiles would need 64 memory instructions in
//   flight per wave, past what the wave's counter tracks; that head
//   dimension stays on the tiled kernel.)
// * Each wave keeps an exact online softmax state (running max, sum, O~) over
//   its tiles; at the end the waves' states are merged through LDS with the
//   block-combine rule and written as the final O and LSE, or, with several
//   key ranges, as this range's normalised state for the combine kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kernel_common.h"

namespace attn {
namespace dec16 {

using namespace attn::dev;

struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* opart;
  float* lpart;
  const int* cu_q;
  const int* cu_k;
  int Hq, Hkv, g;
  int Nq, Nk;
  int total_q, total_k;
  int nsplit, split_len;
  int win_l, win_r;  // window widths (masked kernels; wide = unbounded)
  float c;           // alpha * log2(e)
};

template <int D>
struct DGeo {
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int BN = 32;                 // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per key row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;        // one V tile
  static constexpr int RING = NW * TILE;        // one ring stage, all waves
  static constexpr int LDS = 2 * RING;
  static constexpr int INSTR = TILE / 1024;     // 1 KiB copies per V tile
  static constexpr int RPI = 1024 / ROWB;       // rows per copy
  static constexpr int KLOADS = 2 * (D / 32);   // 16-byte K loads per lane per tile
  static constexpr int PER_TILE = KLOADS + INSTR;  // vector memory ops per tile
  static_assert(LDS <= 64 * 1024, "two workgroups per compute unit");
  static_assert(NW * 16 * D * 4 <= RING && 2 * NW * 16 * 4 <= RING, "merge area must fit in the ring");
  // two tiles and the Q loads in flight must fit the 6-bit vmcnt counter
  static_assert(2 * PER_TILE + D / 32 <= 63, "vmcnt range");
};

// XOR swizzle of the 16-byte chunk index of LDS row r of a V tile: the
// transposing reads (4 rows x 2 chunks per 16 lanes) spread over the banks.
template <int D>
__device__ __forceinline__ int swz_val(int r) {
  return D == 64 ? (((r >> 1) & 3) << 1) : ((r & 7) << 1);
}

template <typename T>
struct Mfma16;
template <>
struct Mfma16<__bf16> {
  static __device__ __forceinline__ f32x4 run(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma16<_Float16> {
  static __device__ __forceinline__ f32x4 run(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(DGeo<D>::NW * 64) void decode_kernel(Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef DGeo<D> G;
  typedef Elt<T> E;
  typedef typename E::v8 v8;
  typedef typename E::v4 v4;
  constexpr int NW = G::NW;
  constexpr int KC = D / 32;  // k-steps of S^T = K Q^T
  constexpr int DB = D / 16;  // 16-dim blocks of O^T
  // The two ring stages are separate objects and every stage index below is
  // a compile-time constant, so the compiler sees that a copy into one stage
  // never aliases reads of the other and does not wait for it.
  __shared__ __attribute__((aligned(1024))) char ring0[G::RING];
  __shared__ __attribute__((aligned(1024))) char ring1[G::RING];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;  // this lane's query row (tile row)
  const int grp = lane >> 4;  // which 4 keys of a 16-key block / 8 dims of a k-step

  // ---- work: (batch entry, key/value head, key range) ------------------------
  const int unit = blockIdx.x / a.nsplit;
  const int split = blockIdx.x - unit * a.nsplit;
  const int b = unit / a.Hkv;
  const int hk = unit - b * a.Hkv;
  const int g = a.g;
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
  const int rows = len_q * g;  // <= 16 (host dispatch rule)
  if (rows <= 0) return;       // uniform
  const int off = len_k - len_q;
  const uint32_t RSQ = (uint32_t)a.Hq * D * 2;
  const uint32_t RSK = (uint32_t)a.Hkv * D * 2;
  const int64_t q_off = ((int64_t)q_row0 * a.Hq + (int64_t)hk * g) * D;
  const int64_t k_off = ((int64_t)k_row0 * a.Hkv + hk) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const T*)a.q + q_off, (uint32_t)(len_q - 1) * RSQ + (uint32_t)g * D * 2);
  const uint32_t kspan = len_k > 0 ? (uint32_t)(len_k - 1) * RSK + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T*)a.k + k_off, kspan);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T*)a.v + k_off, kspan);

  // Q^T operands: lane holds row l16, dims 32 kc + 8 grp + 0..7 (zero past
  // the unit's rows through the buffer range check)
  const int n_r = l16 / g;  // query index of this lane's row
  v8 qreg[KC];
  {
    const uint32_t qo = (uint32_t)n_r * RSQ + (uint32_t)(l16 - n_r * g) * D * 2 + grp * 16;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qreg[kc] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, qo + kc * 64, 0, 0));
  }

  // ---- key range and this wave's tiles ---------------------------------------
  const int kb0 = split * a.split_len;
  const int kb1 = min(len_k, kb0 + a.split_len);
  // (the right bound never shortens the range: with bottom-right alignment
  // the last query row of a sequence sees every key up to len_k - 1 + win_r)
  // masked instantiation: query n sees key j iff
  // n + off - win_l <= j <= n + off + win_r; tiles left of the first row's
  // window are skipped (t0)
  const int nt = kb1 > kb0 ? (kb1 - kb0 + G::BN - 1) / G::BN : 0;
  int t0 = 0;
  if (CAUSAL) {
    const int lo = off - a.win_l;  // first key of row 0's window
    if (lo > kb0) t0 = min((lo - kb0) / G::BN, nt);
  }
  const int cnt = nt - t0 > wave ? (nt - t0 - wave + NW - 1) / NW : 0;
  auto stage = [&](auto st_tag) ATTN_INLINE -> char* {
    return (decltype(st_tag)::value ? ring1 : ring0) + wave * G::TILE;
  };

  // ---- online softmax state of this wave (exact rescale every tile) ----------
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
  float m_run = -__builtin_inff();  // scaled (base-2) units
  float l_run = 0.f;                // this lane's partial sum
  const float c = a.c;

  // K operands of two tiles (by parity of the wave's tile index): lane holds
  // key 16 kb + l16, dims 32 kc + 8 grp + 0..7 (zero past the sequence)
  v8 kreg[2][2 * KC];
  // Tile i of this wave (key tile wave + NW i) into buffer ST: K loads, then
  // the V copies; copy ii moves V rows ii*RPI ..: lane x writes the 16 bytes
  // at LDS offset 16 x of the copy, i.e. row ii*RPI + x/CPR, stored chunk
  // x%CPR, which holds logical chunk (x%CPR) ^ swizzle(row).
  auto issue = [&](auto st_tag, int i) ATTN_INLINE {
    constexpr int ST = decltype(st_tag)::value;
    const int kv0 = kb0 + (t0 + wave + NW * i) * G::BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kreg[ST][kb * KC + kc] = __builtin_bit_cast(
            v8, __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)(kv0 + 16 * kb + l16) * RSK + (uint32_t)(64 * kc + 16 * grp), 0, 0));
    char* dst = stage(st_tag);
#pragma unroll
    for (int ii = 0; ii < G::INSTR; ++ii) {
      const int r = ii * G::RPI + lane / G::CPR;
      const int pc = lane % G::CPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (LDS_AS void*)(dst + ii * 1024), 16,
          (uint32_t)(kv0 + r) * RSK + (uint32_t)((pc ^ swz_val<D>(r)) << 4), 0, 0, 0);
    }
  };

  auto step = [&](auto st_tag, int i) ATTN_INLINE {
    constexpr int ST = decltype(st_tag)::value;
    // tile i's V copy has landed (tile i+1's may be in flight); the compiler
    // adds the waits for the K and Q registers itself
    if (i + 1 < cnt)
      wait_vmcnt<G::PER_TILE>();
    else
      wait_vmcnt<0>();
    const LDS_AS char* vt = (const LDS_AS char*)stage(st_tag);
    const int kv0 = kb0 + (t0 + wave + NW * i) * G::BN;

    // S^T for keys kv0 + 16 kb + 4 grp + e (e = 0..3), row l16
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) s[kb] = Mfma16<T>::run(kreg[ST][kb * KC + kc], qreg[kc], s[kb]);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e / 4][e % 4] * c;
    // keys at or past kb1, and (masked) outside the row's window; rows
    // 0 .. len_q-1 bound which tiles can need it
    if (kv0 + G::BN > kb1 ||
        (CAUSAL && (kv0 + G::BN - 1 > off + a.win_r || kv0 < len_q - 1 + off - a.win_l))) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kv0 + 16 * (e / 4) + 4 * grp + (e % 4);
        if (key >= kb1 || (CAUSAL && (key > n_r + off + a.win_r || key < n_r + off - a.win_l)))
          x[e] = -__builtin_inff();
      }
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = __builtin_fmaxf(mx, x[e]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = __builtin_fmaxf(m_run, mx);
    const float msub = m_new == -__builtin_inff() ? 0.f : m_new;
    const float rho = exp2_fast(m_run - msub);  // 0 while m_run = -inf
    m_run = m_new;
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2_fast(x[e] - msub);  // -inf -> 0
      ps += p[e];
    }
    l_run = l_run * rho + ps;
    v8 pk;
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[e] = (T)p[e];
    // O^T += V^T P^T: slot 8 grp + e of the contraction is key
    // 16 (e / 4) + 4 grp + e % 4, so the 16 lanes of group grp read the
    // 4 x 16 blocks at rows 4 grp and 16 + 4 grp through the transposing load
    const int tr_row = 4 * grp + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = 2 * db + ((l16 & 3) >> 1);
      const int bo = 8 * (l16 & 1);
      // (rows r and r + 16 share the swizzle; the second offset goes through
      // readfirstlane, without which the compiler loses track of which LDS
      // object the read touches and waits for every copy in flight)
      const int o1 = tr_row * G::ROWB + ((ch ^ swz_val<D>(tr_row)) << 4) + bo;
      const v4 lo = E::tr_read(vt + o1);
      const v4 hi = E::tr_read(vt + __builtin_amdgcn_readfirstlane(16 * G::ROWB) + o1);
      oacc[db] = Mfma16<T>::run(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk, oacc[db] * rho);
    }
    if (i + 2 < cnt) {
      wait_lgkmcnt0();  // this V stage's reads have returned before it is refilled
      issue(st_tag, i + 2);
    }
  };

  if (cnt > 0) issue(Int<0>{}, 0);
  if (cnt > 1) issue(Int<1>{}, 1);
  // unrolled by two so the K buffer and ring stage indices are constants
  for (int i = 0; i < cnt; i += 2) {
    step(Int<0>{}, i);
    if (i + 1 < cnt) step(Int<1>{}, i + 1);
  }

  // ---- merge the waves' states (block-combine rule) ---------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // every wave is done with its ring: reuse it for the merge
  float* ost = (float*)ring0;                // [NW][16 rows][D]
  float* mst = (float*)ring1;                // [NW][16]
  float* lst = mst + NW * 16;                // [NW][16]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) ost[(wave * 16 + l16) * D + 16 * db + 4 * grp + e] = oacc[db][e];
  if (grp == 0) {
    mst[wave * 16 + l16] = m_run;
    lst[wave * 16 + l16] = l_run;
  }
  __syncthreads();
  constexpr int TPR = NW * 4;    // threads per row
  constexpr int DPT = D / TPR;   // dims per thread
  const int t = threadIdx.x;
  const int r = t / TPR;
  const int d0 = (t % TPR) * DPT;
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < NW; ++w) M = __builtin_fmaxf(M, mst[w * 16 + r]);
  const float Msub = M == -__builtin_inff() ? 0.f : M;
  float wgt[NW], L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wgt[w] = exp2_fast(mst[w * 16 + r] - Msub);
    L += wgt[w] * lst[w * 16 + r];
  }
  const bool ok = L > 0.f;
  const float inv = ok ? 1.0f / L : 0.f;
  const float lse = ok ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -__builtin_inff();
  float outv[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += wgt[w] * ost[(w * 16 + r) * D + d0 + e];
    outv[e] = acc * inv;
  }
  if (r < rows) {
    const int n = r / g;
    const int hq = hk * g + (r - n * g);
    const int64_t qrow = (int64_t)q_row0 + n;
    if (a.nsplit > 1) {
      const int64_t pr = ((int64_t)split * a.total_q + qrow) * a.Hq + hq;
      if (t % TPR == 0) a.lpart[pr] = lse;
      float* dst = a.opart + pr * D + d0;
#pragma unroll
      for (int e = 0; e < DPT; e += 4) *(f32x4*)(dst + e) = f32x4{outv[e], outv[e + 1], outv[e + 2], outv[e + 3]};
    } else {
      if (t % TPR == 0) {
        const int64_t li = a.cu_q ? (int64_t)hq * a.total_q + qrow : ((int64_t)b * a.Hq + hq) * a.Nq + n;
        a.lse[li] = lse;
      }
      T* dst = (T*)a.o + (qrow * a.Hq + hq) * D + d0;
      typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int e = 0; e < DPT; e += 4) {
        const f32x4 f = {outv[e], outv[e + 1], outv[e + 2], outv[e + 3]};
        *(u32x2*)(dst + e) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, t4));
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool CAUSAL, typename T>
int launch(const FwdArgs& f, hipStream_t st) {
  Args a;
  a.q = f.q; a.k = f.k; a.v = f.v; a.o = f.o; a.lse = f.lse;
  a.opart = f.opart; a.lpart = f.lpart;
  a.cu_q = f.cu_q; a.cu_k = f.cu_k;
  a.Hq = f.H; a.Hkv = f.Hkv; a.g = f.H / f.Hkv;
  a.Nq = f.N; a.Nk = f.Nk;
  a.total_q = f.total_q; a.total_k = f.total_k;
  a.nsplit = f.nsplit > 1 ? f.nsplit : 1;
  a.split_len = f.nsplit > 1 ? f.split_len : 0x7fffffff;
  a.win_l = f.win_l;
  a.win_r = f.win_r;
  a.c = f.scale_log2;
  const int grid = f.B * f.Hkv * a.nsplit;
  hipLaunchKernelGGL((decode_kernel<D, CAUSAL, T>), dim3(grid), dim3(DGeo<D>::NW * 64), 0, st, a);
  return (int)hipGetLastError();
}

template <typename T>
int dispatch(const FwdArgs& f, hipStream_t st) {
  switch (f.d) {
    case 64: return f.causal ? launch<64, true, T>(f, st) : launch<64, false, T>(f, st);
    case 128: return f.causal ? launch<128, true, T>(f, st) : launch<128, false, T>(f, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace dec16

int launch_decode_16(const FwdArgs& f, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return f.dtype == 0 ? dec16::dispatch<__bf16>(f, st) : dec16::dispatch<_Float16>(f, st);
}

}  // namespace attn
