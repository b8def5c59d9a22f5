// C ABI front end of libattn.so (declared in include/attn.h).
//
// Every entry point validates its arguments on the host, before anything is
// launched, and reports failures through a negative status plus a
// thread-local message (attn_last_error). No exception crosses the ABI and
// nothing is printed. The kernels live in the .hip translation units; this
// file has no HIP dependency so its checks can be exercised without a GPU.

#include "attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "attn_internal.h"

static_assert(attn::kStaticWorkspaceBytes == ATTN_STATIC_WORKSPACE_BYTES, "header and library disagree");

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Shape checks shared by the forward entry points. Returns ATTN_OK, a
// negative status, or 1 for "valid but empty" (nothing to do).
int check_shape(int B, int H, int N, int d, int elem_bytes) {
  if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_INVALID_ARG, "B, H, N must be >= 0 (got %d, %d, %d)", B, H, N);
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d is not supported (64, 128 or 256)", d);
  if (B == 0 || H == 0 || N == 0) return 1;
  // the kernels address one head with 32-bit byte offsets (up to a tile
  // past its last row) and index rows and LSE entries with 32-bit integers
  const int64_t head_span = ((int64_t)N + 128) * H * d * elem_bytes;
  if (head_span >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "N*H*d too large for one batch entry (%lld bytes >= 2^31)",
                (long long)head_span);
  if ((int64_t)B * H * N >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "B*H*N too large (>= 2^31)");
  return ATTN_OK;
}

int check_fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int N, int d, int causal, float alpha, int elem_bytes) {
  const int s = check_shape(B, H, N, d, elem_bytes);
  if (s != ATTN_OK) return s;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(alpha) || alpha < 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "alpha must be finite and >= 0 (got %g)", (double)alpha);
  const void* ptrs[5] = {q, k, v, o, lse};
  const char* names[5] = {"q", "k", "v", "o", "lse"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  const int64_t in_bytes = (int64_t)B * N * H * d * elem_bytes;
  const int64_t out_bytes = (int64_t)B * N * H * d * 2;
  const int64_t lse_bytes = (int64_t)B * H * N * 4;
  const void* ins[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, out_bytes, ins[i], in_bytes)) return fail(ATTN_ERR_INVALID_ARG, "o overlaps %s", names[i]);
    if (overlaps(lse, lse_bytes, ins[i], in_bytes)) return fail(ATTN_ERR_INVALID_ARG, "lse overlaps %s", names[i]);
  }
  if (overlaps(o, out_bytes, lse, lse_bytes)) return fail(ATTN_ERR_INVALID_ARG, "o overlaps lse");
  return ATTN_OK;
}

float scale_log2(float alpha) {
  // alpha * log2(e); a zero scale is replaced by 1e-30, which gives the same
  // float32 result (every exponent rounds to 2^0) and keeps the running max
  // arithmetic free of 0 * inf.
  const float c = alpha * 1.4426950408889634f;
  return c < 1e-30f ? 1e-30f : c;
}

int hip_status(int err, const char* what) {
  if (err == 0) return ok();
  return fail(ATTN_ERR_HIP, "%s: HIP error %d (%s)", what, err, attn::hip_error_name(err));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             int causal, float alpha, int dtype, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported (0 = bf16, 1 = f16)", dtype);
  const int s = check_fwd_common(q, k, v, o, lse, B, H, N, d, causal, alpha, 2);
  if (s == 1) return ok();
  if (s != ATTN_OK) return s;
  attn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.causal = causal;
  a.dtype = dtype;
  a.scale_log2 = scale_log2(alpha);
  a.Hkv = H; a.Nk = N;
  a.total_q = a.total_k = B * N;
  a.win_l = 2 * N + 1;  // unbounded left
  a.win_r = 0;          // causal (used only when causal = 1)
  a.nsplit = 1;
  return hip_status(attn::launch_fwd_16(a, stream), "attn_fwd launch");
}

int64_t attn_splitkv_workspace_bytes(int num_splits, int total_q, int Hq, int d) {
  if (num_splits <= 1 || total_q <= 0 || Hq <= 0 || d <= 0) return 0;
  return (int64_t)num_splits * total_q * Hq * (d + 1) * 4;
}

int attn_pack_gqa_heuristic(int Hq, int Hkv, int Nq) {
  if (Hkv <= 0 || Hq <= Hkv || Hq % Hkv != 0 || Nq <= 0) return 0;
  const int64_t g = Hq / Hkv;
  // pack when it takes fewer 128-row query tiles
  return ((int64_t)Nq * g + 127) / 128 < g * (((int64_t)Nq + 127) / 128) ? 1 : 0;
}

int attn_num_splits_heuristic(int B, int Hq, int Hkv, int Nq, int Nk, int d, int pack_gqa, int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Nq <= 0 || Nk <= 0 || num_cus <= 0) return 1;
  const int64_t g = Hq / Hkv;
  int64_t blocks, target, min_keys;
  if (attn::uses_decode_kernel(Nq, Hq, Hkv, d)) {
    // decode kernel: one workgroup per (sequence, KV head, range); about one
    // per compute unit, each range long enough to amortise its start-up
    blocks = (int64_t)B * Hkv;
    target = num_cus;
    min_keys = 512;
  } else {
    const bool pack = pack_gqa < 0 ? attn_pack_gqa_heuristic(Hq, Hkv, Nq) != 0 : (pack_gqa != 0 && g > 1);
    const int64_t rows = pack ? (int64_t)Nq * g : Nq;
    blocks = (rows + 127) / 128 * B * (pack ? Hkv : Hq);
    target = (int64_t)num_cus * (d == 256 ? 1 : 2);  // resident workgroups
    min_keys = 256;
  }
  if (blocks >= target) return 1;
  int64_t s = (target + blocks - 1) / blocks;
  const int64_t by_keys = ((int64_t)Nk + min_keys - 1) / min_keys;
  if (s > by_keys) s = by_keys;
  if (s > 128) s = 128;
  return s < 1 ? 1 : (int)s;
}

}  // extern "C"

namespace {

// attn_fwd_ex, with the split-KV workspace either the caller's
// (use_static = false) or the library's static device array (use_static =
// true: attn_fwd_ex_noalloc, which passes no workspace).
int fwd_ex_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                int Nq, int Nk, int d, const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q,
                int total_k, int causal, int window_left, int window_right, float alpha, int dtype,
                int pack_gqa, int num_splits, float* workspace, int64_t workspace_bytes, bool use_static,
                const char* what, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported (0 = bf16, 1 = f16)", dtype);
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_ERR_INVALID_ARG, "B, Hq, Hkv, Nq, Nk must be >= 0 (got %d, %d, %d, %d, %d)", B, Hq, Hkv,
                Nq, Nk);
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d is not supported (64, 128 or 256)", d);
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID_ARG, "Hq = %d must be a positive multiple of Hkv = %d", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (window_left < -1 || window_right < -1)
    return fail(ATTN_ERR_INVALID_ARG, "window widths must be >= -1 (got %d, %d)", window_left, window_right);
  if (!std::isfinite(alpha) || alpha < 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "alpha must be finite and >= 0 (got %g)", (double)alpha);
  if (pack_gqa < -1 || pack_gqa > 1) return fail(ATTN_ERR_INVALID_ARG, "pack_gqa must be -1, 0 or 1");
  if (num_splits < 1) return fail(ATTN_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", num_splits);
  const bool varlen = cu_seqlens_q != nullptr || cu_seqlens_k != nullptr;
  if (varlen && (!cu_seqlens_q || !cu_seqlens_k))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must both be given or both be null");
  if (varlen && (total_q < 0 || total_k < 0))
    return fail(ATTN_ERR_INVALID_ARG, "total_q, total_k must be >= 0 (got %d, %d)", total_q, total_k);
  if (!varlen) {
    if ((int64_t)B * Nq >= (int64_t(1) << 31) || (int64_t)B * Nk >= (int64_t(1) << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "B*Nq or B*Nk too large (>= 2^31)");
    total_q = B * Nq;
    total_k = B * Nk;
  }
  if (B == 0 || Hq == 0 || Nq == 0 || total_q == 0) return ok();
  // kernels address one sequence of one head with 32-bit byte offsets (up to
  // a tile past its end) and index rows, LSE entries and tiles with 32-bit
  // integers
  if (((int64_t)Nq + 128) * Hq * d * 2 >= (int64_t(1) << 31) || ((int64_t)Nk + 128) * Hkv * d * 2 >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "sequence too long for the number of heads (N*H*d*2 near 2^31)");
  if ((int64_t)total_q * Hq >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "total_q*Hq too large (>= 2^31)");
  const int g = Hq / Hkv;
  const int pack = pack_gqa < 0 ? attn_pack_gqa_heuristic(Hq, Hkv, Nq) : (pack_gqa && g > 1 ? 1 : 0);
  // effective key ranges: a multiple of 64 keys each, none empty
  int split_len = 0, nsplit = 1;
  if (num_splits > 1 && Nk > 0) {
    const int64_t per = ((int64_t)Nk + num_splits - 1) / num_splits;
    split_len = (int)((per + 63) / 64 * 64);
    nsplit = (int)(((int64_t)Nk + split_len - 1) / split_len);
  }
  const int64_t rows = pack ? (int64_t)Nq * g : Nq;
  const int64_t grid = (rows + 127) / 128 * B * (pack ? Hkv : Hq) * nsplit;
  if (grid >= (int64_t(1) << 31)) return fail(ATTN_ERR_UNSUPPORTED, "too many workgroups (>= 2^31)");
  const void* ptrs[5] = {q, k, v, o, lse};
  const char* names[5] = {"q", "k", "v", "o", "lse"};
  for (int i = 0; i < 5; ++i) {
    // k and v hold no rows when no sequence has keys (every row then gets
    // O = 0, LSE = -inf) and may be null
    if ((i == 1 || i == 2) && total_k == 0) continue;
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  if (varlen && ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens are not 4-byte aligned");
  const int64_t qb = (int64_t)total_q * Hq * d * 2, kb = (int64_t)total_k * Hkv * d * 2;
  const int64_t lb = (int64_t)total_q * Hq * 4;
  const int64_t ws_need = nsplit > 1 ? attn_splitkv_workspace_bytes(nsplit, total_q, Hq, d) : 0;
  if (use_static) {
    if (ws_need > attn::kStaticWorkspaceBytes)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "%d key ranges need %lld bytes of split-KV workspace, more than the %lld-byte static "
                  "workspace of %s (use fewer splits, or attn_fwd_ex with a caller workspace)",
                  nsplit, (long long)ws_need, (long long)attn::kStaticWorkspaceBytes, what);
    workspace = nullptr;
    workspace_bytes = 0;
    if (ws_need > 0) {
      void* p = nullptr;
      const int e = attn::static_workspace(&p);
      if (e != 0) return hip_status(e, "static workspace lookup");
      workspace = static_cast<float*>(p);
      workspace_bytes = attn::kStaticWorkspaceBytes;
    }
  }
  const void* in[3] = {q, k, v};
  const int64_t in_b[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, qb, in[i], in_b[i])) return fail(ATTN_ERR_INVALID_ARG, "o overlaps %s", names[i]);
    if (overlaps(lse, lb, in[i], in_b[i])) return fail(ATTN_ERR_INVALID_ARG, "lse overlaps %s", names[i]);
  }
  if (overlaps(o, qb, lse, lb)) return fail(ATTN_ERR_INVALID_ARG, "o overlaps lse");
  if (ws_need > 0) {
    if (!workspace) return fail(ATTN_ERR_INVALID_ARG, "workspace is null but %d key ranges need %lld bytes", nsplit,
                                (long long)ws_need);
    if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < ws_need)
      return fail(ATTN_ERR_INVALID_ARG, "workspace has %lld bytes, %d key ranges need %lld", (long long)workspace_bytes,
                  nsplit, (long long)ws_need);
    const void* all[5] = {q, k, v, o, lse};
    const int64_t all_b[5] = {qb, kb, kb, qb, lb};
    for (int i = 0; i < 5; ++i)
      if (overlaps(workspace, ws_need, all[i], all_b[i]))
        return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps %s", names[i]);
  }
  attn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = Hq; a.N = Nq; a.d = d;
  // the masked kernels take the window; causal is its right width 0, and an
  // unbounded side is any width past the sequence (Nq + Nk + 1)
  const int wide = Nq + Nk + 1;
  a.win_l = window_left < 0 ? wide : (window_left < wide ? window_left : wide);
  a.win_r = window_right < 0 ? wide : (window_right < wide ? window_right : wide);
  if (causal) a.win_r = 0;
  a.causal = (causal || window_left >= 0 || window_right >= 0) ? 1 : 0;
  a.dtype = dtype;
  a.scale_log2 = scale_log2(alpha);
  a.Hkv = Hkv; a.Nk = Nk;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.total_q = total_q; a.total_k = total_k;
  a.pack = pack;
  a.nsplit = nsplit;
  a.split_len = split_len;
  if (nsplit > 1) {
    a.opart = workspace;
    a.lpart = workspace + (int64_t)nsplit * total_q * Hq * d;
  }
  return hip_status(attn::launch_fwd_16(a, stream), what);
}

}  // namespace

extern "C" {

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                int Nq, int Nk, int d, const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q,
                int total_k, int causal, int window_left, int window_right, float alpha, int dtype,
                int pack_gqa, int num_splits, float* workspace, int64_t workspace_bytes, void* stream) {
  return fwd_ex_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k, causal,
                     window_left, window_right, alpha, dtype, pack_gqa, num_splits, workspace, workspace_bytes,
                     false, "attn_fwd_ex", stream);
}

int attn_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                        int Nq, int Nk, int d, const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q,
                        int total_k, int causal, int window_left, int window_right, float alpha, int dtype,
                        int pack_gqa, int num_splits, void* stream) {
  return fwd_ex_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k, causal,
                     window_left, window_right, alpha, dtype, pack_gqa, num_splits, nullptr, 0, true,
                     "attn_fwd_ex_noalloc", stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float alpha,
             int dtype, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported (0 = bf16, 1 = f16)", dtype);
  const int s = check_shape(B, H, N, d, 2);
  if (s == 1) return ok();
  if (s != ATTN_OK) return s;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(alpha) || alpha < 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "alpha must be finite and >= 0 (got %g)", (double)alpha);
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
  const char* names[10] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  const int64_t tb = (int64_t)B * N * H * d * 2;
  const int64_t rb = (int64_t)B * H * N * 4;
  const int64_t bytes[10] = {tb, tb, tb, tb, tb, rb, tb, tb, tb, rb};
  // outputs (dq, dk, dv, delta) must not overlap each other or any input
  for (int i = 6; i < 10; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != i && overlaps(ptrs[i], bytes[i], ptrs[j], bytes[j]))
        return fail(ATTN_ERR_INVALID_ARG, "%s overlaps %s", names[i], names[j]);
  attn::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = delta;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.Hkv = H; a.Nk = N;
  a.win_l = 2 * N + 1;  // unbounded left
  a.win_r = 0;          // causal (used only when causal = 1)
  a.causal = causal;
  a.dtype = dtype;
  a.scale_log2 = scale_log2(alpha);
  a.alpha = a.scale_log2 / 1.4426950408889634f;
  return hip_status(attn::launch_bwd_16(a, stream), "attn_bwd launch");
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                const int* cu_seqlens_q, const int* cu_seqlens_k, int total_q, int total_k, int causal,
                int window_left, int window_right, float alpha, int dtype, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported (0 = bf16, 1 = f16)", dtype);
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_ERR_INVALID_ARG, "B, Hq, Hkv, Nq, Nk must be >= 0 (got %d, %d, %d, %d, %d)", B, Hq, Hkv,
                Nq, Nk);
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d is not supported (64, 128 or 256)", d);
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID_ARG, "Hq = %d must be a positive multiple of Hkv = %d", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (window_left < -1 || window_right < -1)
    return fail(ATTN_ERR_INVALID_ARG, "window widths must be >= -1 (got %d, %d)", window_left, window_right);
  if (!std::isfinite(alpha) || alpha < 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "alpha must be finite and >= 0 (got %g)", (double)alpha);
  const bool varlen = cu_seqlens_q != nullptr || cu_seqlens_k != nullptr;
  if (varlen && (!cu_seqlens_q || !cu_seqlens_k))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must both be given or both be null");
  if (varlen && (total_q < 0 || total_k < 0))
    return fail(ATTN_ERR_INVALID_ARG, "total_q, total_k must be >= 0 (got %d, %d)", total_q, total_k);
  if (!varlen) {
    if ((int64_t)B * Nq >= (int64_t(1) << 31) || (int64_t)B * Nk >= (int64_t(1) << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "B*Nq or B*Nk too large (>= 2^31)");
    total_q = B * Nq;
    total_k = B * Nk;
  }
  if (B == 0 || Hq == 0 || (total_q == 0 && total_k == 0)) return ok();
  if (((int64_t)Nq + 128) * Hq * d * 2 >= (int64_t(1) << 31) || ((int64_t)Nk + 128) * Hkv * d * 2 >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "sequence too long for the number of heads (N*H*d*2 near 2^31)");
  if ((int64_t)total_q * Hq >= (int64_t(1) << 31) || (int64_t)total_k * Hkv >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "total rows * heads too large (>= 2^31)");
  if (varlen && ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens are not 4-byte aligned");
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
  const char* names[10] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta"};
  const int64_t qb = (int64_t)total_q * Hq * d * 2, kb = (int64_t)total_k * Hkv * d * 2;
  const int64_t rb = (int64_t)total_q * Hq * 4;
  const int64_t bytes[10] = {qb, kb, kb, qb, qb, rb, qb, kb, kb, rb};
  // operands of size zero (no query or no key rows) may be null
  for (int i = 0; i < 10; ++i) {
    if (bytes[i] == 0) continue;
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  for (int i = 6; i < 10; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != i && overlaps(ptrs[i], bytes[i], ptrs[j], bytes[j]))
        return fail(ATTN_ERR_INVALID_ARG, "%s overlaps %s", names[i], names[j]);
  attn::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = delta;
  a.B = B; a.H = Hq; a.N = Nq; a.d = d;
  a.Hkv = Hkv; a.Nk = Nk;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.total_q = total_q; a.total_k = total_k;
  // same window convention as attn_fwd_ex: causal is a right width of 0 and
  // an unbounded side is any width past the sequence
  const int wide = Nq + Nk + 1;
  a.win_l = window_left < 0 ? wide : (window_left < wide ? window_left : wide);
  a.win_r = window_right < 0 ? wide : (window_right < wide ? window_right : wide);
  if (causal) a.win_r = 0;
  a.causal = (causal || window_left >= 0 || window_right >= 0) ? 1 : 0;
  a.dtype = dtype;
  a.scale_log2 = scale_log2(alpha);
  a.alpha = a.scale_log2 / 1.4426950408889634f;
  return hip_status(attn::launch_bwd_16(a, stream), "attn_bwd_ex launch");
}

int attn_fp8_prepare(const void* x, void* x8, float* descale, int B, int H, int N, int d, int block_rows,
                     int hadamard, uint64_t hadamard_seed, void* stream) {
  const int s = check_shape(B, H, N, d, 2);
  if (s == 1) return ok();
  if (s != ATTN_OK) return s;
  if (block_rows != 0 && block_rows != 128)
    return fail(ATTN_ERR_INVALID_ARG, "block_rows must be 0 or 128 (got %d)", block_rows);
  if (hadamard != 0 && hadamard != 1) return fail(ATTN_ERR_INVALID_ARG, "hadamard must be 0 or 1");
  const void* ptrs[3] = {x, x8, descale};
  const char* names[3] = {"x", "x8", "descale"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  const int64_t n = (int64_t)B * N * H * d;
  const int64_t dbytes = block_rows ? (int64_t)B * H * ((N + block_rows - 1) / block_rows) * 4 : 4;
  if (overlaps(x8, n, x, 2 * n)) return fail(ATTN_ERR_INVALID_ARG, "x8 overlaps x");
  if (overlaps(descale, dbytes, x, 2 * n)) return fail(ATTN_ERR_INVALID_ARG, "descale overlaps x");
  if (overlaps(descale, dbytes, x8, n)) return fail(ATTN_ERR_INVALID_ARG, "descale overlaps x8");
  attn::PrepArgs a{};
  a.x = x; a.x8 = x8; a.descale = descale;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.block_rows = block_rows;
  a.hadamard = hadamard;
  a.seed = hadamard_seed;
  return hip_status(attn::launch_fp8_prepare(a, stream), "attn_fp8_prepare launch");
}

int attn_fwd_fp8_ex(const void* q8, const void* k8, const void* v8, void* o, float* lse, int B, int Hq, int Hkv,
                    int N, int d, int causal, float alpha, const float* descale_q, const float* descale_k,
                    const float* descale_v, int block_rows, uint64_t hadamard_seed, void* stream) {
  // The seed only names the transform q8 and k8 were prepared with: the
  // product (Q M)(K M)^T equals Q K^T for the orthogonal M, so the forward
  // never applies M, and nothing in the codes records which M was used.
  (void)hadamard_seed;
  // the head grouping is checked before the empty-problem return, as in
  // attn_fwd_ex
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID_ARG, "Hq = %d must be a positive multiple of Hkv = %d", Hq, Hkv);
  const int s = check_shape(B, Hq, N, d, 1);
  if (s == 1) return ok();
  if (s != ATTN_OK) return s;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(alpha) || alpha < 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "alpha must be finite and >= 0 (got %g)", (double)alpha);
  if (block_rows != 0 && block_rows != 128)
    return fail(ATTN_ERR_INVALID_ARG, "block_rows must be 0 or 128 (got %d)", block_rows);
  const void* ptrs[5] = {q8, k8, v8, o, lse};
  const char* names[5] = {"q", "k", "v", "o", "lse"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", names[i]);
    if (!aligned16(ptrs[i])) return fail(ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  const float* ds[3] = {descale_q, descale_k, descale_v};
  const char* dnames[3] = {"descale_q", "descale_k", "descale_v"};
  for (int i = 0; i < 3; ++i)
    if (!ds[i]) return fail(ATTN_ERR_INVALID_ARG, "%s is null", dnames[i]);
  const int64_t q_bytes = (int64_t)B * N * Hq * d;
  const int64_t kv_bytes = (int64_t)B * N * Hkv * d;
  const int64_t out_bytes = (int64_t)B * N * Hq * d * 2;
  const int64_t lse_bytes = (int64_t)B * Hq * N * 4;
  const void* ins[3] = {q8, k8, v8};
  const int64_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, out_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_INVALID_ARG, "o overlaps %s", names[i]);
    if (overlaps(lse, lse_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_INVALID_ARG, "lse overlaps %s", names[i]);
  }
  if (overlaps(o, out_bytes, lse, lse_bytes)) return fail(ATTN_ERR_INVALID_ARG, "o overlaps lse");
  // the kernel writes o and lse while it reads the descales
  const int64_t nsb = block_rows ? ((int64_t)N + block_rows - 1) / block_rows : 0;
  const int64_t ds_bytes[3] = {block_rows ? (int64_t)B * Hq * nsb * 4 : 4, block_rows ? (int64_t)B * Hkv * nsb * 4 : 4,
                               block_rows ? (int64_t)B * Hkv * nsb * 4 : 4};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, out_bytes, ds[i], ds_bytes[i])) return fail(ATTN_ERR_INVALID_ARG, "o overlaps %s", dnames[i]);
    if (overlaps(lse, lse_bytes, ds[i], ds_bytes[i]))
      return fail(ATTN_ERR_INVALID_ARG, "lse overlaps %s", dnames[i]);
  }
  attn::FwdArgs a{};
  a.q = q8; a.k = k8; a.v = v8; a.o = o; a.lse = lse;
  a.dq = descale_q; a.dk = descale_k; a.dv = descale_v;
  a.B = B; a.H = Hq; a.N = N; a.d = d;
  a.Hkv = Hkv;
  a.causal = causal;
  a.block_rows = block_rows;
  a.scale_log2 = scale_log2(alpha);
  return hip_status(attn::launch_fwd_fp8(a, stream), "attn_fwd_fp8 launch");
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse, int B, int H, int N,
                 int d, int causal, float alpha, const float* descale_q, const float* descale_k,
                 const float* descale_v, int block_rows, uint64_t hadamard_seed, void* stream) {
  return attn_fwd_fp8_ex(q8, k8, v8, o, lse, B, H, H, N, d, causal, alpha, descale_q, descale_k, descale_v,
                         block_rows, hadamard_seed, stream);
}

const char* attn_last_error(void) { return g_err.c_str(); }

#ifndef ATTN_BUILD_INFO
#define ATTN_BUILD_INFO "unknown build"
#endif
const char* attn_version(void) { return "attn-gfx950 0.2 (" ATTN_BUILD_INFO ")"; }

}  // extern "C"
