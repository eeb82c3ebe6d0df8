// Host-side launchers of the attention kernels (one per storage type).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs;

// Arguments of the general forward (see fa_fwd_kv_bf16.hpp).
struct KvArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;    // [num_splits][rows][D] fp32, when num_splits > 1
  float* part_lse;  // [num_splits][rows]
  const int* cu_q;  // variable-length offsets [B+1] (device), or null
  const int* cu_k;
  int B, Hq, Hkv;
  int Nq, Nk;          // uniform: lengths; variable length: totals Tq, Tk
  int max_nq, max_nk;  // largest sequence lengths (grid sizing)
  int num_splits, split_keys;  // keys per split: a multiple of 64
  int compact;                 // variable length: grid of the sequences' row blocks only (B <= 256)
  long long rows;              // number of (batch, head, query) rows
  float c;                     // scale * log2(e)
};

// Arguments of the bf16 backward (square, rectangular and variable-length
// problems; see fa_bwd_bf16.hpp).
struct BwdKvArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;      // workspace: D_i = dO_i . O_i, one per query row
  float* l2;        // workspace: lse_i * log2(e), one per query row
  const int* cu_q;  // variable-length offsets [B+1] (device), or null
  const int* cu_k;
  int B, Hq, Hkv;
  int Nq, Nk;          // uniform: lengths; variable length: totals Tq, Tk
  int max_nq, max_nk;  // largest sequence lengths (grid sizing)
  int compact;         // variable length: grids of the sequences' blocks only (B <= 256)
  long long rows;      // query rows: B*Hq*Nq, or Hq*Tq
  float c;             // scale * log2(e)
  float scale;
};

// Forward: picks the kernel instance for (d, causal) and launches it on stream.
hipError_t fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream);
hipError_t fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream);

// General forward (rectangular, variable length, split keys; bf16): the
// kernel for (d, rows per K/V head, causal), then the combine when split.
hipError_t fwd_kv_bf16(const KvArgs& a, int d, int causal, hipStream_t stream);

// Three-pass materialising baseline (bf16): S (fp32) and P (bf16) of every
// (query, key) pair go through the caller's workspace s and p.
hipError_t naive_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* s, uint16_t* p,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal, hipStream_t stream);

// Backward (bf16): D and l2 into the workspace, then the dK/dV and dQ
// kernels, all on stream. Square problems are the case Nq = Nk.
hipError_t bwd_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream);

// Bytes of the backward workspace for `rows` query rows: D and l2 (fp32
// each), the second from a 256-byte boundary.
inline size_t bwd_ws_l2_offset(long long rows) { return ((size_t)rows * 4 + 255) & ~(size_t)255; }
inline size_t bwd_ws_bytes(long long rows) { return 2 * bwd_ws_l2_offset(rows); }

// Backward, fp32 check mode (square): D = rowsum(dO * O) into dsum, then the
// dK/dV and dQ kernels, all on stream.
hipError_t bwd_f32(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* dsum,
                   int B, int Hq, int Hkv, int N, int d, float scale, float c, int causal, hipStream_t stream);

}  // namespace fa
