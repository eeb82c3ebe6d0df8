// C ABI of libflashattn.so: argument validation, kernel dispatch, status codes.
// The operation, layouts, ownership and error conventions are documented in
// include/flash_attn.h.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "flash_attn.h"
#include "fa_launch.hpp"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point. Element offsets are computed in
// 64-bit inside the kernels; grid sizes and per-head row indices are 32-bit.
int check_shape(int B, int Hq, int Hkv, int N, int d, int causal) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  const long long rows = (long long)B * Hq * N;
  if (rows * (long long)d > ((long long)1 << 40)) return FA_ERR_SHAPE;
  const long long nqb = (N + 127) / 128;
  if (nqb * (long long)Hq * B > 0x7fffffffLL) return FA_ERR_SHAPE;
  if ((long long)N * d > 0x7fffffffLL) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_scale(float scale) {
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
  return FA_OK;
}

int check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return FA_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!aligned16(ptrs[i])) return FA_ERR_ALIGN;
  return FA_OK;
}

int fwd_common(bool f32, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse};
  int st = check_ptrs(ptrs, 5);
  if (st == FA_OK) st = check_shape(B, Hq, Hkv, N, d, causal);
  if (st == FA_OK) st = check_scale(scale);
  if (st != FA_OK) return st;
  const float c = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = f32 ? fa::fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, c, causal, s)
                           : fa::fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, c, causal, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Arguments of the bf16 backward; the workspace holds D then l2.
fa::BwdKvArgs bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, const int* cu_q, const int* cu_k,
                       void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int max_nq, int max_nk,
                       long long rows, float scale) {
  fa::BwdKvArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = static_cast<float*>(workspace);
  a.l2 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + fa::bwd_ws_l2_offset(rows));
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.max_nq = max_nq;
  a.max_nk = max_nk;
  a.compact = (cu_q != nullptr && B <= 256) ? 1 : 0;
  a.rows = rows;
  a.c = scale * kLog2e;
  a.scale = scale;
  return a;
}

int check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (workspace == nullptr) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  return FA_OK;
}

int bwd_common(bool f32, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  int st = check_ptrs(ptrs, 9);
  if (st == FA_OK) st = check_shape(B, Hq, Hkv, N, d, causal);
  if (st == FA_OK) st = check_scale(scale);
  if (st == FA_OK) st = check_workspace(workspace, workspace_bytes, flash_attn_bwd_workspace_bytes(B, Hq, Hkv, N, d));
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (f32) {
    e = fa::bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv, N, d, scale,
                    scale * kLog2e, causal, s);
  } else {
    const fa::BwdKvArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, workspace, B, Hq, Hkv, N, N,
                                     N, N, (long long)B * Hq * N, scale);
    e = fa::bwd_bf16(a, d, causal, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Shape checks of the general forward and backward: positive sizes, Hq a
// multiple of Hkv, supported d, element offsets within 2^40, grids within
// int32 (the backward's key blocks are 64 keys at the smallest).
int check_kv_shape(int B, int Hq, int Hkv, int Nq, int Nk, int max_nq, int max_nk, int d, int causal,
                   bool varlen) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Nq <= 0 || Nk <= 0 || max_nq <= 0 || max_nk <= 0)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  const long long rows = varlen ? (long long)Hq * Nq : (long long)B * Hq * Nq;
  const long long krows = varlen ? (long long)Hkv * Nk : (long long)B * Hkv * Nk;
  if (rows * d > ((long long)1 << 40) || krows * d > ((long long)1 << 40)) return FA_ERR_SHAPE;
  if (((long long)max_nk + 63) / 64 * Hkv * B > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (((long long)max_nq + 31) / 32 * Hq * B > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (Hkv > 65535 || B > 65535) return FA_ERR_SHAPE;
  return FA_OK;
}

int bwd_kv_common(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, const int* cu_q, const int* cu_k, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int max_nq, int max_nk, int d,
                  float scale, int causal, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  int st = check_ptrs(ptrs, 9);
  if (st == FA_OK) st = check_kv_shape(B, Hq, Hkv, Nq, Nk, max_nq, max_nk, d, causal, cu_q != nullptr);
  if (st == FA_OK) st = check_scale(scale);
  const long long rows = cu_q ? (long long)Hq * Nq : (long long)B * Hq * Nq;
  if (st == FA_OK) st = check_workspace(workspace, workspace_bytes, fa::bwd_ws_bytes(rows));
  if (st != FA_OK) return st;
  const fa::BwdKvArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, cu_q, cu_k, workspace, B, Hq, Hkv, Nq, Nk,
                                   max_nq, max_nk, rows, scale);
  const hipError_t e = fa::bwd_bf16(a, d, causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}


// Split count for the general forward: one unless the (batch, K/V head, row
// block) workgroups are too few to fill the chip; then enough splits for about
// four workgroups per compute unit (eight for one-wave decoding workgroups,
// whose work is streaming K and V), each split at least 256 keys. At d = 256
// one four-wave workgroup fills a compute unit's LDS: a grid of 256 of them
// already fills the chip, and the four-wave target halves.
int kv_splits_auto(int B, int Hq, int Hkv, int max_nq, int max_nk, int d) {
  const long long G = Hq / Hkv;
  const long long rows = (long long)max_nq * G;
  const long long bm = rows <= 32 ? 32 : 128;
  const long long wgs = (long long)B * Hkv * ((rows + bm - 1) / bm);
  const long long target = (rows <= 32 ? 8 : (d == 256 ? 2 : 4)) * 256;
  if (wgs >= target / 2 || max_nk <= 512) return 1;
  long long s = (target + wgs - 1) / wgs;
  s = s < (max_nk + 255) / 256 ? s : (max_nk + 255) / 256;
  s = s < 256 ? s : 256;
  return (int)(s < 1 ? 1 : s);
}

size_t kv_workspace(long long rows, int d, int splits) {
  if (splits <= 1) return 0;
  const size_t po = (size_t)splits * rows * d * 4;
  const size_t pl = (size_t)splits * rows * 4;
  return ((po + 255) & ~(size_t)255) + ((pl + 255) & ~(size_t)255);
}

// Static scratch of flash_attn_fwd_kv_noalloc: the split partials live in
// this file-scope device array instead of a caller's workspace. Each device
// the library runs on holds its own copy until the process ends. In host code
// `scratch` is only a stand-in for the symbol, never a device address: the
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and kept in g_scratch_ptr, and only that pointer reaches kernels.
static __device__ __align__(256) uint8_t scratch[FLASH_ATTN_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[64];

// Device address of `scratch` on the current device (looked up on the first
// call per device; concurrent first calls store the same address).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

// use_scratch: the split partials go to the static scratch (no workspace
// argument); num_splits = 0 then picks the library's count capped so that the
// partials fit, and an explicit count whose partials do not fit is refused.
int kv_common(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_q, const int* cu_k,
              int B, int Hq, int Hkv, int Nq, int Nk, int max_nq, int max_nk, int d, float scale, int causal,
              int num_splits, void* workspace, size_t workspace_bytes, void* stream, bool use_scratch = false) {
  const void* ptrs[] = {q, k, v, o, lse};
  int st = check_ptrs(ptrs, 5);
  if (st != FA_OK) return st;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Nq <= 0 || Nk <= 0 || max_nq <= 0 || max_nk <= 0)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (num_splits < 0) return FA_ERR_SHAPE;
  const long long rows = cu_q ? (long long)Hq * Nq : (long long)B * Hq * Nq;
  const long long krows = cu_q ? (long long)Hkv * Nk : (long long)B * Hkv * Nk;
  if (rows * d > ((long long)1 << 40) || krows * d > ((long long)1 << 40)) return FA_ERR_SHAPE;
  const long long G = Hq / Hkv;
  const long long nrb = ((long long)max_nq * G + 31) / 32;
  const long long hb = (long long)Hkv * B;
  if ((long long)max_nq * G > 0x7fffffffLL || nrb * 256 > 0x7fffffffLL || hb > 0x7fffffffLL) return FA_ERR_SHAPE;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  int splits = num_splits == 0 ? kv_splits_auto(B, Hq, Hkv, max_nq, max_nk, d) : num_splits;
  if (splits < 1 || splits > 256) return FA_ERR_SHAPE;
  // Workgroups (32-row blocks at the smallest) within the 65536 x 65535 grid;
  // variable-length batches of up to 256 sequences take the compact grid.
  const bool compact = cu_q != nullptr && B <= 256;
  const long long items = compact ? ((long long)Nq * G + 31) / 32 + B : nrb * B;
  if (items * splits * Hkv > 65536LL * 65535) return FA_ERR_SHAPE;
  if (use_scratch && splits > 1) {
    if (num_splits == 0)
      while (splits > 1 && kv_workspace(rows, d, splits) > (size_t)FLASH_ATTN_SCRATCH_BYTES) --splits;
    if (kv_workspace(rows, d, splits) > (size_t)FLASH_ATTN_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    if (splits > 1) {
      st = scratch_ptr(&workspace);
      if (st != FA_OK) return st;
      workspace_bytes = FLASH_ATTN_SCRATCH_BYTES;
    }
  }
  if (splits > 1) {
    if (workspace == nullptr) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if (workspace_bytes < kv_workspace(rows, d, splits)) return FA_ERR_WORKSPACE;
  }
  fa::KvArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.max_nq = max_nq;
  a.max_nk = max_nk;
  a.num_splits = splits;
  a.compact = compact ? 1 : 0;
  a.split_keys = (((max_nk + splits - 1) / splits) + 63) / 64 * 64;
  a.rows = rows;
  a.c = scale * kLog2e;
  if (splits > 1) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + (((size_t)splits * rows * d * 4 + 255) & ~(size_t)255));
  }
  const hipError_t e = fa::fwd_kv_bf16(a, d, causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  return fwd_common(false, q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream);
}

int flash_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  return fwd_common(true, q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream);
}

size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (check_shape(B, Hq, Hkv, N, d, 0) != FA_OK) return 0;
  // D (fp32 per query row), then lse * log2(e) (fp32 per query row) from the
  // next 256-byte boundary.
  return fa::bwd_ws_bytes((long long)B * Hq * N);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  return bwd_common(false, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d, scale,
                    causal, stream);
}

int flash_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                       const float* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream) {
  return bwd_common(true, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d, scale,
                    causal, stream);
}

size_t flash_attn_bwd_kv_workspace_bytes(long long rows, int d) {
  if (rows <= 0 || (d != 64 && d != 128 && d != 256)) return 0;
  return fa::bwd_ws_bytes(rows);
}

int flash_attn_bwd_kv(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, float scale, int causal, void* stream) {
  return bwd_kv_common(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, workspace, workspace_bytes, B, Hq, Hkv,
                       Nq, Nk, Nq, Nk, d, scale, causal, stream);
}

int flash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                          const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                          int Tq, int Tk, int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                          void* stream) {
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return FA_ERR_NULL;
  return bwd_kv_common(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, workspace, workspace_bytes, B,
                       Hq, Hkv, Tq, Tk, max_seqlen_q, max_seqlen_k, d, scale, causal, stream);
}

int flash_attn_fwd_kv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Nq <= 0 || Nk <= 0) return 0;
  if (d != 64 && d != 128 && d != 256) return 0;
  return kv_splits_auto(B, Hq, Hkv, Nq, Nk, d);
}

size_t flash_attn_fwd_kv_workspace_bytes(long long rows, int d, int num_splits) {
  if (rows <= 0 || (d != 64 && d != 128 && d != 256) || num_splits < 1 || num_splits > 256) return 0;
  return kv_workspace(rows, d, num_splits);
}

int flash_attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return kv_common(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, Nq, Nk, d, scale, causal, num_splits,
                   workspace, workspace_bytes, stream);
}

int flash_attn_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                              int num_splits, void* stream) {
  return kv_common(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, Nq, Nk, d, scale, causal, num_splits,
                   nullptr, 0, stream, true);
}

int flash_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                          int Tq, int Tk, int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return FA_ERR_NULL;
  return kv_common(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Tq, Tk, max_seqlen_q, max_seqlen_k, d,
                   scale, causal, num_splits, workspace, workspace_bytes, stream);
}

size_t flash_attn_naive_workspace_bytes(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  const size_t pairs = (size_t)B * Hq * N * N;
  return ((pairs * 4 + 255) & ~(size_t)255) + ((pairs * 2 + 255) & ~(size_t)255);
}

int flash_attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse};
  int st = check_ptrs(ptrs, 5);
  if (st == FA_OK) st = check_shape(B, Hq, Hkv, N, d, causal);
  if (st == FA_OK && (long long)B * Hq * N > 0x7fffffffLL) st = FA_ERR_SHAPE;
  if (st == FA_OK) st = check_scale(scale);
  if (st != FA_OK) return st;
  if (workspace == nullptr) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (workspace_bytes < flash_attn_naive_workspace_bytes(B, Hq, N)) return FA_ERR_WORKSPACE;
  const size_t pairs = (size_t)B * Hq * N * N;
  float* s = static_cast<float*>(workspace);
  uint16_t* p = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + ((pairs * 4 + 255) & ~(size_t)255));
  const hipError_t e = fa::naive_bf16(q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, scale, causal,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* flash_attn_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN";
    case FA_ERR_SCALE: return "FA_ERR_SCALE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH";
    default: return "FA_UNKNOWN";
  }
}

}  // extern "C"
