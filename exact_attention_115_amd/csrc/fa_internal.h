// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"
#include "fa_philox.h"

namespace fa {

// Problem description after validation (all sizes positive, d in {64, 128}).
struct Problem {
  int B, Hq, Hkv, Nq, Nkv, d;
  int G;             // Hq / Hkv
  float scale;       // > 0
  int causal;        // 0 / 1
  fa_dtype dt;
};

struct FwdPtrs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* ws;          // decode split state, else unused
};

// Paged K/V for decode: the page pools take the places of k and v in
// FwdPtrs ([num_pages, Hkv, page_size, d]); Problem::Nkv = max_pages *
// page_size.
struct PagedPtrs {
  const int* page_table;  // [B, max_pages] physical page of each logical page
  const int* seq_lens;    // [B] keys of each sequence
  int page_size, max_pages, num_pages;
};

// FP8 forward: E4M3 codes for q, k, v with per-tensor descale factors
// (real value = code value * descale); o is bf16.
struct Fp8Ptrs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float descale_q, descale_k, descale_v;
};

struct BwdPtrs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* nd;         // [B, Hq, Nq] float32 -D, in the workspace
  float* lneg;       // [B, Hq, Nq] float32 -LSE / scale (-inf: no key), in the workspace
  float* dk_part;    // [gsplit, B, Hkv, Nkv, d] float32 partial sums, or NULL
  float* dv_part;    //   (present only when the head group is split)
  const DropParams* drop;  // dropout parameters, or NULL for none
};

// Decode (N_q == 1) split-KV geometry, shared by the workspace size and the
// launcher so both always agree.
struct DecodeSplit {
  int splits;        // key-range splits per (b, kv head)
  int keys_per_split;
};
DecodeSplit decode_split(const Problem& p);
size_t decode_workspace_bytes(const Problem& p);
size_t bwd_workspace_bytes(const Problem& p);
// Number of workgroups that share the query heads of one key block in the
// backward (1 unless there are too few key blocks to fill the GPU); always a
// divisor of G.
int bwd_group_split(const Problem& p);

// fa_bwd with a workspace the library provides: validates every argument
// as fa_bwd does (the workspace aside), then calls get_ws(bytes needed,
// &ptr), which returns FA_OK and a device pointer or an error status, and
// runs the three backward stages on that workspace. get_ws is called only
// after the arguments passed the host-side checks.
typedef int (*LibraryWorkspace)(size_t bytes, void** ws);
int bwd_with_library_workspace(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dO, void* dq, void* dk, void* dv,
                               int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
                               int causal, fa_dtype dt, hipStream_t stream, LibraryWorkspace get_ws);

// Launchers: each enqueues its kernel(s) on `stream` and returns the
// hipError_t of the launch.
hipError_t launch_fwd_f32(const Problem& p, const FwdPtrs& t, hipStream_t stream);
// drop: dropout parameters, or null for none.
hipError_t launch_fwd_mfma(const Problem& p, const FwdPtrs& t, hipStream_t stream,
                           const DropParams* drop = nullptr);
hipError_t launch_decode(const Problem& p, const FwdPtrs& t, hipStream_t stream);
hipError_t launch_fwd_fp8(const Problem& p, const Fp8Ptrs& t, hipStream_t stream);
hipError_t launch_decode_paged(const Problem& p, const FwdPtrs& t, const PagedPtrs& pg,
                               hipStream_t stream);
hipError_t launch_dropout_mask(uint8_t* keep, int B, int Hq, int Nq, int Nkv, const DropParams& dp,
                               hipStream_t stream);
// Backward stages, in order: dQ and the row terms (fa_bwd_dq.hip); dK, dV
// per key block; the sum of split dK, dV partials (no-op unless split).
hipError_t launch_bwd_dq_rows(const Problem& p, const BwdPtrs& t, hipStream_t stream);
hipError_t launch_bwd_main(const Problem& p, const BwdPtrs& t, hipStream_t stream);
hipError_t launch_bwd_reduce(const Problem& p, const BwdPtrs& t, hipStream_t stream);

}  // namespace fa
