// C-ABI entry points of libfa.so: argument checks (pure host code, run before
// any HIP call), workspace sizing and kernel selection. See include/fa.h for
// the contract of each call.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kVersion = 100;  // 0.1.0

size_t elem_bytes(fa_dtype dt) { return dt == FA_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == FA_F32 || dt == FA_F16 || dt == FA_BF16; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Whether the product of non-negative factors is below `limit` (> 0). It
// multiplies factor by factor and stops before a partial product could pass
// the limit, so sizes near INT_MAX in every argument cannot overflow it.
bool product_below(std::initializer_list<long long> factors, long long limit) {
  for (long long f : factors)
    if (f == 0) return true;
  long long p = 1;
  for (long long f : factors) {
    if (p > (limit - 1) / f) return false;
    p *= f;
  }
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + bytes};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Shape checks shared by every entry point. Returns FA_OK, or an error, and
// sets *empty when there is nothing to compute.
int check_shape(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int dt, bool* empty) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nkv < 0 || d < 0) return FA_ERR_SHAPE;
  if (!valid_dtype(dt)) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hkv == 0) {
    if (Hq != 0) return FA_ERR_SHAPE;
  } else if (Hq % Hkv != 0) {
    return FA_ERR_SHAPE;
  }
  // Element counts must fit the kernels' 64-bit offsets and 32-bit grids.
  const long long big = 1LL << 31;
  if (!product_below({B, Hq, ((long long)Nq + 127) / 128}, big)) return FA_ERR_UNSUPPORTED;
  if (!product_below({B, Hq, Nq}, big) || !product_below({B, Hkv, Nkv}, big))
    return FA_ERR_UNSUPPORTED;
  // One head's K (or V) is addressed with 32-bit byte offsets.
  if ((long long)Nkv * d * 4 >= big) return FA_ERR_UNSUPPORTED;
  *empty = (B == 0 || Hq == 0 || Nq == 0);
  return FA_OK;
}

Problem make_problem(int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale, int causal,
                     fa_dtype dt) {
  Problem p;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nkv = Nkv; p.d = d;
  p.G = Hkv > 0 ? Hq / Hkv : 1;
  p.scale = scale; p.causal = causal; p.dt = dt;
  return p;
}

int check_scale(float scale, int causal) {
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_SCALE;
  return FA_OK;
}

bool is_decode(const Problem& p) { return p.Nq == 1 && p.dt != FA_F32; }

int to_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

int check_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
              size_t ws_bytes, int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
              int causal, int dt, bool* empty, Problem* prob) {
  int st = check_shape(B, Hq, Hkv, Nq, Nkv, d, dt, empty);
  if (st != FA_OK) return st;
  st = check_scale(scale, causal);
  if (st != FA_OK) return st;
  if (*empty) return FA_OK;
  *prob = make_problem(B, Hq, Hkv, Nq, Nkv, d, scale, causal, (fa_dtype)dt);
  const size_t e = elem_bytes((fa_dtype)dt);
  const size_t qb = (size_t)B * Hq * Nq * d * e;
  const size_t kb = (size_t)B * Hkv * Nkv * d * e;
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  if (!q || !o || !lse) return FA_ERR_NULLPTR;
  if (kb > 0 && (!k || !v)) return FA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 16)) return FA_ERR_ALIGNMENT;
  if (kb > 0 && (!aligned(k, 16) || !aligned(v, 16))) return FA_ERR_ALIGNMENT;
  const size_t need = is_decode(*prob) ? decode_workspace_bytes(*prob) : 0;
  if (need > 0) {
    if (!ws) return FA_ERR_NULLPTR;
    if (!aligned(ws, 256)) return FA_ERR_ALIGNMENT;
    if (ws_bytes < need) return FA_ERR_WORKSPACE;
  }
  const Range in[3] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range out[3] = {range_of(o, qb), range_of(lse, lb), range_of(ws, need)};
  for (const Range& a : out) {
    for (const Range& b : in)
      if (overlap(a, b)) return FA_ERR_OVERLAP;
  }
  if (overlap(out[0], out[1]) || overlap(out[0], out[2]) || overlap(out[1], out[2]))
    return FA_ERR_OVERLAP;
  return FA_OK;
}

// check_ws = false: the library supplies the workspace itself (it is then
// neither checked nor part of the overlap checks).
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, int B,
              int Hq, int Hkv, int Nq, int Nkv, int d, float scale, int causal, int dt,
              bool* empty, Problem* prob, bool check_ws = true) {
  int st = check_shape(B, Hq, Hkv, Nq, Nkv, d, dt, empty);
  if (st != FA_OK) return st;
  if (dt == FA_F32) return FA_ERR_UNSUPPORTED;
  st = check_scale(scale, causal);
  if (st != FA_OK) return st;
  *prob = make_problem(B, Hq, Hkv, Nq, Nkv, d, scale, causal, (fa_dtype)dt);
  const size_t e = elem_bytes((fa_dtype)dt);
  const size_t qb = (size_t)B * Hq * Nq * d * e;
  const size_t kb = (size_t)B * Hkv * Nkv * d * e;
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  // dk, dv must still be cleared when there are no queries, so an empty query
  // side is not "empty" for the backward unless the key side is empty too.
  if (kb == 0 && qb == 0) {
    *empty = true;
    return FA_OK;
  }
  *empty = false;
  if (qb > 0 && (!q || !o || !lse || !dO || !dq)) return FA_ERR_NULLPTR;
  if (kb > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULLPTR;
  const void* al[9] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : al)
    if (p && !aligned(p, 16)) return FA_ERR_ALIGNMENT;
  const size_t need = check_ws ? bwd_workspace_bytes(*prob) : 0;
  if (need > 0) {
    if (!ws) return FA_ERR_NULLPTR;
    if (!aligned(ws, 256)) return FA_ERR_ALIGNMENT;
    if (ws_bytes < need) return FA_ERR_WORKSPACE;
  }
  const Range in[6] = {range_of(q, qb), range_of(k, kb), range_of(v, kb),
                       range_of(o, qb), range_of(lse, lb), range_of(dO, qb)};
  const Range out[4] = {range_of(dq, qb), range_of(dk, kb), range_of(dv, kb),
                        range_of(ws, need)};
  for (const Range& a : out)
    for (const Range& b : in)
      if (overlap(a, b)) return FA_ERR_OVERLAP;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_OVERLAP;
  return FA_OK;
}

BwdPtrs bwd_ptrs(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv, void* ws) {
  BwdPtrs t;
  t.q = q; t.k = k; t.v = v; t.o = o; t.lse = lse; t.dO = dO;
  t.dq = dq; t.dk = dk; t.dv = dv;
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  const size_t del = align_up(rows * sizeof(float), 256);
  char* base = static_cast<char*>(ws);
  t.nd = reinterpret_cast<float*>(base);
  t.lneg = base ? reinterpret_cast<float*>(base + del) : nullptr;
  t.dk_part = t.dv_part = nullptr;
  t.drop = nullptr;
  const int gs = bwd_group_split(p);
  if (gs > 1 && base) {
    const size_t part = align_up((size_t)gs * p.B * p.Hkv * p.Nkv * p.d * sizeof(float), 256);
    t.dk_part = reinterpret_cast<float*>(base + 2 * del);
    t.dv_part = reinterpret_cast<float*>(base + 2 * del + part);
  }
  return t;
}

// Dropout parameters from the probability: theta = min(255, floor(256 p + 1/2)),
// rscale = 256 / (256 - theta). p must be finite and in [0, 1).
int drop_params(float p, uint64_t seed, uint64_t offset, DropParams* out) {
  if (!(p >= 0.0f && p < 1.0f)) return FA_ERR_SCALE;  // also rejects NaN
  double t = floor(256.0 * (double)p + 0.5);
  if (t > 255.0) t = 255.0;
  out->seed = seed;
  out->offset = offset;
  out->theta = (uint32_t)t;
  out->rscale = (float)(256.0 / (256.0 - t));
  return FA_OK;
}

int run_bwd_stage(int stage, const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  switch (stage) {
    case 0: return to_status(launch_bwd_dq_rows(p, t, stream));
    case 1: return to_status(launch_bwd_main(p, t, stream));
    case 2: return to_status(launch_bwd_reduce(p, t, stream));
    default: return FA_ERR_UNSUPPORTED;
  }
}

}  // namespace

DecodeSplit decode_split(const Problem& p) {
  // One workgroup per CU (its LDS holds a private 64-key K tile and V tile
  // for each of its four waves, each refilled as soon as it has been read):
  // split the key range so that about 256 workgroups cover all (b, kv head,
  // query-head group) units, with at least two tiles per split.
  const long long units = (long long)p.B * p.Hkv * ((p.G + 31) / 32);
  const int tiles = (p.Nkv + 63) / 64;
  long long want = units > 0 ? (256 + units - 1) / units : 1;
  long long max_splits = (tiles + 1) / 2;
  if (max_splits < 1) max_splits = 1;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int tiles_per_split = (int)((tiles + want - 1) / want);
  if (tiles_per_split < 1) tiles_per_split = 1;
  DecodeSplit s;
  s.keys_per_split = tiles_per_split * 64;
  s.splits = p.Nkv > 0 ? (p.Nkv + s.keys_per_split - 1) / s.keys_per_split : 1;
  return s;
}

size_t decode_workspace_bytes(const Problem& p) {
  const DecodeSplit s = decode_split(p);
  const size_t rows = (size_t)p.B * p.Hq * s.splits;
  return align_up(rows * p.d * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

int bwd_group_split(const Problem& p) {
  // Aim for at least ~512 workgroups; split the G query heads of a key block
  // across workgroups (each sums its share of dK, dV) when there are fewer.
  const long long blocks = (long long)((p.Nkv + 127) / 128) * p.B * p.Hkv;
  if (blocks <= 0 || p.G <= 1 || blocks >= 512) return 1;
  int want = (int)((512 + blocks - 1) / blocks);
  int best = 1;
  for (int s = 1; s <= p.G; ++s)
    if (p.G % s == 0 && s <= want) best = s;
  return best;
}

size_t bwd_workspace_bytes(const Problem& p) {
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  const size_t kv = (size_t)p.B * p.Hkv * p.Nkv * p.d;
  if (rows == 0 && kv == 0) return 0;
  size_t bytes = 2 * align_up(rows * sizeof(float), 256);
  const int gs = bwd_group_split(p);
  if (gs > 1) bytes += 2 * align_up((size_t)gs * kv * sizeof(float), 256);
  return bytes;
}

int bwd_with_library_workspace(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dO, void* dq, void* dk, void* dv,
                               int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
                               int causal, fa_dtype dt, hipStream_t stream, LibraryWorkspace get_ws) {
  bool empty = false;
  Problem p;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, nullptr, 0, B, Hq, Hkv, Nq, Nkv, d, scale,
                     causal, dt, &empty, &p, /*check_ws=*/false);
  if (st != FA_OK || empty) return st;
  void* ws = nullptr;
  st = get_ws(bwd_workspace_bytes(p), &ws);
  if (st != FA_OK) return st;
  const BwdPtrs t = bwd_ptrs(p, q, k, v, o, lse, dO, dq, dk, dv, ws);
  for (int stage = 0; stage < 3; ++stage) {
    st = run_bwd_stage(stage, p, t, stream);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

}  // namespace fa

using namespace fa;

// Paged decode: the shape of the equivalent contiguous decode (N_q = 1,
// N_kv = max_pages * page_size) plus the page geometry.
static int check_paged_shape(int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                      int dt, bool* empty) {
  if (num_pages < 0 || page_size < 0 || max_pages < 0) return FA_ERR_SHAPE;
  if (dt != FA_F16 && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (page_size == 0 || page_size % 64 != 0) return FA_ERR_UNSUPPORTED;
  if (max_pages == 0 || num_pages == 0) return FA_ERR_SHAPE;
  const long long nkv = (long long)max_pages * page_size;
  if (nkv >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  int st = check_shape(B, Hq, Hkv, 1, (int)nkv, d, dt, empty);
  if (st != FA_OK) return st;
  // One page of one kv head is addressed with 32-bit byte offsets; pages with
  // 64-bit ones.
  if (!product_below({num_pages, Hkv, page_size}, 1LL << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

static int check_paged(const void* q, const void* kp, const void* vp, const int* table, const int* lens,
                void* o, float* lse, void* ws, size_t ws_bytes, int B, int Hq, int Hkv,
                int num_pages, int page_size, int max_pages, int d, float scale, int dt,
                bool* empty, Problem* prob) {
  int st = check_paged_shape(B, Hq, Hkv, num_pages, page_size, max_pages, d, dt, empty);
  if (st != FA_OK) return st;
  st = check_scale(scale, 0);
  if (st != FA_OK) return st;
  if (*empty) return FA_OK;
  *prob = make_problem(B, Hq, Hkv, 1, max_pages * page_size, d, scale, 0, (fa_dtype)dt);
  const size_t e = elem_bytes((fa_dtype)dt);
  const size_t qb = (size_t)B * Hq * d * e;
  const size_t pb = (size_t)num_pages * Hkv * page_size * d * e;
  const size_t tb = (size_t)B * max_pages * sizeof(int);
  const size_t nb = (size_t)B * sizeof(int);
  const size_t lb = (size_t)B * Hq * sizeof(float);
  if (!q || !kp || !vp || !table || !lens || !o || !lse || !ws) return FA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(kp, 16) || !aligned(vp, 16) || !aligned(o, 16) ||
      !aligned(lse, 16) || !aligned(table, 4) || !aligned(lens, 4))
    return FA_ERR_ALIGNMENT;
  const size_t need = decode_workspace_bytes(*prob);
  if (!aligned(ws, 256)) return FA_ERR_ALIGNMENT;
  if (ws_bytes < need) return FA_ERR_WORKSPACE;
  const Range in[5] = {range_of(q, qb), range_of(kp, pb), range_of(vp, pb), range_of(table, tb),
                       range_of(lens, nb)};
  const Range out[3] = {range_of(o, qb), range_of(lse, lb), range_of(ws, need)};
  for (const Range& a : out) {
    for (const Range& b : in)
      if (overlap(a, b)) return FA_ERR_OVERLAP;
  }
  if (overlap(out[0], out[1]) || overlap(out[0], out[2]) || overlap(out[1], out[2]))
    return FA_ERR_OVERLAP;
  return FA_OK;
}

extern "C" {

size_t fa_fwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int d, fa_dtype dt) {
  bool empty = false;
  if (check_shape(B, Hq, Hkv, Nq, Nkv, d, dt, &empty) != FA_OK || empty) return 0;
  Problem p = make_problem(B, Hq, Hkv, Nq, Nkv, d, 1.0f, 0, dt);
  return is_decode(p) ? decode_workspace_bytes(p) : 0;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int d, fa_dtype dt) {
  bool empty = false;
  if (check_shape(B, Hq, Hkv, Nq, Nkv, d, dt, &empty) != FA_OK || empty) return 0;
  if (dt == FA_F32) return 0;
  Problem p = make_problem(B, Hq, Hkv, Nq, Nkv, d, 1.0f, 0, dt);
  return bwd_workspace_bytes(p);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
           size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
           int causal, fa_dtype dt, hipStream_t stream) {
  bool empty = false;
  Problem p;
  int st = check_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nkv, d, scale,
                     causal, dt, &empty, &p);
  if (st != FA_OK || empty) return st;
  FwdPtrs t{q, k, v, o, lse, workspace};
  if (dt == FA_F32) return to_status(launch_fwd_f32(p, t, stream));
  if (is_decode(p)) return to_status(launch_decode(p, t, stream));
  return to_status(launch_fwd_mfma(p, t, stream));
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                 float scale, int causal, fa_dtype dt, hipStream_t stream) {
  if (stage < 0 || stage > 2) return FA_ERR_UNSUPPORTED;
  bool empty = false;
  Problem p;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                     Nkv, d, scale, causal, dt, &empty, &p);
  if (st != FA_OK || empty) return st;
  return run_bwd_stage(stage, p, bwd_ptrs(p, q, k, v, o, lse, dO, dq, dk, dv, workspace), stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale, int causal, fa_dtype dt,
           hipStream_t stream) {
  bool empty = false;
  Problem p;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                     Nkv, d, scale, causal, dt, &empty, &p);
  if (st != FA_OK || empty) return st;
  const BwdPtrs t = bwd_ptrs(p, q, k, v, o, lse, dO, dq, dk, dv, workspace);
  for (int stage = 0; stage < 3; ++stage) {
    st = run_bwd_stage(stage, p, t, stream);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nkv,
                   int d, float scale, int causal, float dropout_p, uint64_t seed, uint64_t offset,
                   fa_dtype dt, hipStream_t stream) {
  bool empty = false;
  Problem p;
  int st = check_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nkv, d, scale,
                     causal, dt, &empty, &p);
  if (st != FA_OK) return st;
  if (dt == FA_F32) return FA_ERR_UNSUPPORTED;
  DropParams dp;
  st = drop_params(dropout_p, seed, offset, &dp);
  if (st != FA_OK || empty) return st;
  FwdPtrs t{q, k, v, o, lse, workspace};
  // Every query length, one row included, takes the tiled kernel.
  return to_status(launch_fwd_mfma(p, t, stream, &dp));
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                   float scale, int causal, float dropout_p, uint64_t seed, uint64_t offset,
                   fa_dtype dt, hipStream_t stream) {
  bool empty = false;
  Problem p;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                     Nkv, d, scale, causal, dt, &empty, &p);
  if (st != FA_OK) return st;
  DropParams dp;
  st = drop_params(dropout_p, seed, offset, &dp);
  if (st != FA_OK || empty) return st;
  BwdPtrs t = bwd_ptrs(p, q, k, v, o, lse, dO, dq, dk, dv, workspace);
  t.drop = &dp;
  for (int stage = 0; stage < 3; ++stage) {
    st = run_bwd_stage(stage, p, t, stream);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nkv, int d, float scale, int causal, float descale_q,
               float descale_k, float descale_v, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, Nq, Nkv, d, FA_BF16, &empty);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  st = check_scale(scale, causal);
  if (st != FA_OK) return st;
  const float ds[3] = {descale_q, descale_k, descale_v};
  for (float x : ds)
    if (!(x > 0.0f) || !isfinite(x)) return FA_ERR_SCALE;
  if (empty) return FA_OK;
  Problem p = make_problem(B, Hq, Hkv, Nq, Nkv, d, scale, causal, FA_BF16);
  const size_t qb = (size_t)B * Hq * Nq * d;   // one byte per element
  const size_t kb = (size_t)B * Hkv * Nkv * d;
  const size_t ob = 2 * qb;                    // bf16 output
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  if (!q || !o || !lse) return FA_ERR_NULLPTR;
  if (kb > 0 && (!k || !v)) return FA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 16)) return FA_ERR_ALIGNMENT;
  if (kb > 0 && (!aligned(k, 16) || !aligned(v, 16))) return FA_ERR_ALIGNMENT;
  const Range in[3] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range out[2] = {range_of(o, ob), range_of(lse, lb)};
  for (const Range& a : out)
    for (const Range& b : in)
      if (overlap(a, b)) return FA_ERR_OVERLAP;
  if (overlap(out[0], out[1])) return FA_ERR_OVERLAP;
  Fp8Ptrs t{q, k, v, o, lse, descale_q, descale_k, descale_v};
  return to_status(launch_fwd_fp8(p, t, stream));
}

int fa_dropout_mask(unsigned char* keep, int B, int Hq, int Nq, int Nkv, float dropout_p,
                    uint64_t seed, uint64_t offset, hipStream_t stream) {
  if (B < 0 || Hq < 0 || Nq < 0 || Nkv < 0) return FA_ERR_SHAPE;
  DropParams dp;
  int st = drop_params(dropout_p, seed, offset, &dp);
  if (st != FA_OK) return st;
  if (B == 0 || Hq == 0 || Nq == 0 || Nkv == 0) return FA_OK;
  if ((long long)B * Hq >= (1LL << 31) || (double)B * Hq * Nq * Nkv >= 4.0e18)
    return FA_ERR_UNSUPPORTED;
  if (!keep) return FA_ERR_NULLPTR;
  return to_status(launch_dropout_mask(keep, B, Hq, Nq, Nkv, dp, stream));
}

size_t fa_fwd_paged_workspace_size(int B, int Hq, int Hkv, int page_size, int max_pages, int d,
                                   fa_dtype dt) {
  bool empty = false;
  if (check_paged_shape(B, Hq, Hkv, 1, page_size, max_pages, d, dt, &empty) != FA_OK || empty)
    return 0;
  Problem p = make_problem(B, Hq, Hkv, 1, max_pages * page_size, d, 1.0f, 0, dt);
  return decode_workspace_bytes(p);
}

int fa_fwd_paged(const void* q, const void* k_pages, const void* v_pages, const int* page_table,
                 const int* seq_lens, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, int B, int Hq, int Hkv, int num_pages, int page_size,
                 int max_pages, int d, float scale, fa_dtype dt, hipStream_t stream) {
  bool empty = false;
  Problem p;
  int st = check_paged(q, k_pages, v_pages, page_table, seq_lens, o, lse, workspace,
                       workspace_bytes, B, Hq, Hkv, num_pages, page_size, max_pages, d, scale, dt,
                       &empty, &p);
  if (st != FA_OK || empty) return st;
  FwdPtrs t{q, k_pages, v_pages, o, lse, workspace};
  PagedPtrs pg{page_table, seq_lens, page_size, max_pages, num_pages};
  return to_status(launch_decode_paged(p, t, pg, stream));
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (negative size, Hkv == 0 or Hq not a multiple of Hkv)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype, pass or stage";
    case FA_ERR_ALIGNMENT: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case FA_ERR_WORKSPACE: return "workspace smaller than the size the library asks for";
    case FA_ERR_SCALE: return "scale must be finite and > 0, causal must be 0 or 1";
    case FA_ERR_HIP: return "the HIP runtime reported an error at kernel launch";
    case FA_ERR_OVERLAP: return "an output buffer overlaps an input or another output";
    case FA_ERR_SCRATCH:
      return "the problem needs more workspace than the library's static scratch buffer holds";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
