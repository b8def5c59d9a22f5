// Internal interface between the C ABI front end (attn_api.cpp) and the HIP
// kernels. Not installed; the public ABI is include/attn.h.
#pragma once

#include <stdint.h>

namespace attn {

// Arguments of one attention forward launch, already validated on the host.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* dq;  // FP8 descales (null for 16-bit inputs)
  const float* dk;
  const float* dv;
  int B, H, N, d;  // H: query heads; N: query rows per batch entry (the
                   // maximum over the sequences for packed batches)
  int causal;
  int dtype;       // 0 bf16, 1 f16 (16-bit path)
  int block_rows;  // FP8: 128 or 0 (per tensor)
  float scale_log2;  // alpha * log2(e), clamped to >= 1e-30
  // 16-bit path only (the FP8 path requires Hkv = H, Nk = N, no packing,
  // one split):
  int Hkv;           // key/value heads (H % Hkv == 0)
  int Nk;            // key rows per batch entry (maximum for packed batches)
  const int* cu_q;   // packed batches: B + 1 row offsets (device), else null
  const int* cu_k;
  int total_q;       // rows of q and o (B * N for dense inputs)
  int total_k;       // rows of k and v
  int pack;          // query heads of one key/value head share a tile
  int win_l, win_r;  // masked path (causal = 1): query n sees key j iff
                     // n + off - win_l <= j <= n + off + win_r, off = Nk - Nq
                     // (widths >= 0; "unbounded" is passed as Nq + Nk + 1)
  int nsplit;        // key ranges (1: no split)
  int split_len;     // keys per range, a multiple of 64
  float* opart;      // nsplit > 1: [nsplit, total_q, H, d] float32 partial O
  float* lpart;      //             [nsplit, total_q, H] float32 partial LSE
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int B, H, N, d;    // H: query heads, N: query rows per batch entry
  int Hkv, Nk;       // key/value heads (H % Hkv == 0), key rows
  const int* cu_q;   // packed batches: B + 1 row offsets (N, Nk are maxima)
  const int* cu_k;
  int total_q, total_k;
  int win_l, win_r;  // masked path (causal = 1), as in FwdArgs
  int causal;
  int dtype;
  float alpha;       // alpha, clamped to >= 1e-30 / log2(e)
  float scale_log2;  // alpha * log2(e), clamped to >= 1e-30
};

struct PrepArgs {
  const void* x;
  void* x8;
  float* descale;
  int B, H, N, d;
  int block_rows;
  int hadamard;
  uint64_t seed;
};

// Query rows per key/value head (N_q * H / Hkv) up to which the 16-bit
// forward runs the decode kernel (d = 64 and 128).
constexpr int kDecodeRows = 16;
inline bool uses_decode_kernel(int Nq, int Hq, int Hkv, int d) {
  return d <= 128 && (int64_t)Nq * (Hq / Hkv) <= kDecodeRows;
}

// Bytes of the static split-KV workspace each GPU holds for
// attn_fwd_ex_noalloc (a file-scope device array, resident from the first
// call on a device until the process ends).
constexpr int64_t kStaticWorkspaceBytes = int64_t(16) << 20;

// Device address of the current device's static workspace, looked up once
// per device (hipGetSymbolAddress; allocates nothing). Returns 0 or a
// hipError_t value.
int static_workspace(void** ptr);

// Each returns 0 on success or a hipError_t value.
int launch_fwd_16(const FwdArgs& a, void* stream);
int launch_decode_16(const FwdArgs& a, void* stream);
int launch_fwd_fp8(const FwdArgs& a, void* stream);
int launch_fp8_prepare(const PrepArgs& a, void* stream);
int launch_bwd_16(const BwdArgs& a, void* stream);
const char* hip_error_name(int err);

}  // namespace attn
